"""Build libkvc.so for gfx950 in-tree with hipcc (no JIT cache, no torch extension).

Each HIP source is compiled to its own object in parallel (every translation unit carries
its own device code object), then the objects are linked into one shared library.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvc.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["kvc_api.hip", "kvc_correct.hip", "kvc_correct_general.hip", "kvc_fit.hip",
           "kvc_rank.hip", "kvc_metrics.hip",
           "kvc_anchor_pool.hip", "kvc_warm.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
_NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if _NOISE not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into agent_kv_cache_kvc_amd/libkvc.so; returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs, cmds = [], []
    for s in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
