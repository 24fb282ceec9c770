"""Build and run the C ABI's argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer on the host (no GPU): kvc_api.hip and the driver
tests/abi_sanitize_main.cpp are compiled with the sanitizers on their host code only, and
linked with the library's other (unsanitised) objects from agent_kv_cache_kvc_amd/_build."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "agent_kv_cache_kvc_amd", "csrc")
OBJ = os.path.join(ROOT, "agent_kv_cache_kvc_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
OTHER = ["kvc_correct.o", "kvc_correct_general.o", "kvc_fit.o", "kvc_rank.o", "kvc_metrics.o",
         "kvc_anchor_pool.o", "kvc_warm.o"]


def build_and_run() -> str:
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = os.path.join(OBJ, "kvc_api_san.o")
    drv = os.path.join(OBJ, "abi_sanitize_main.o")
    exe = os.path.join(OBJ, "abi_sanitize")
    base = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    subprocess.run(base + SAN + inc + ["-c", os.path.join(CSRC, "kvc_api.hip"), "-o", api],
                   check=True, capture_output=True)
    subprocess.run([HIPCC, "-O1", "-std=c++17", "-x", "c++"] + SAN + inc +
                   ["-c", os.path.join(HERE, "abi_sanitize_main.cpp"), "-o", drv],
                   check=True, capture_output=True)
    objs = [os.path.join(OBJ, o) for o in OTHER]
    # host link (the objects carry their device code): clang++ with the sanitizer runtimes
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin",
                         "clang++")
    subprocess.run([clang, "-fsanitize=address,undefined", drv, api] + objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    return res.stdout + res.stderr + f"\nexit {res.returncode}\n"
