"""The C-ABI library: it loads, exports every symbol the header declares, and rejects bad
arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import agent_kv_cache_kvc_amd as kvc
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kvc.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", src)))


def test_header_symbols_are_exported():
    lib = kvc.lib()
    names = _declared()
    assert "kvc_correct" in names and "kvc_fit_anchor" in names and "kvc_correct_chain" in names
    for n in names:
        assert hasattr(lib, n), n


def test_binding_covers_the_abi():
    for n in ("pool_descriptor", "correct", "correct_chain", "fit_anchor"):
        assert callable(getattr(kvc, n))
    assert set(kvc._SIGS) == set(_declared())


def test_version_and_empty_error():
    assert kvc.lib().kvc_version().startswith(b"kvc")


def _correct(**kw):
    args = dict(K=FAKE, V=FAKE, L=2, H=2, T=64, d=128, dtype=0, desc=FAKE, U=FAKE, W=FAKE, A=4,
                r=32, tau=0.3, q_in=None, K_fb=None, V_fb=None, K_out=FAKE, V_out=FAKE,
                mask=FAKE, score=None, w=None, qn=None, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    st = kvc.lib().kvc_correct(*args.values())
    return st, kvc.lib().kvc_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=None), 1, "K is NULL"),
    (dict(V=FAKE + 4), 1, "aligned"),
    (dict(T=-1), 1, "negative"),
    (dict(d=96), 2, "d=96"),
    (dict(d=0), 1, "positive"),
    (dict(dtype=7), 1, "dtype"),
    (dict(A=0), 1, "A=0"),
    (dict(A=17), 2, "A*r=544"),
    (dict(r=0), 1, "r=0"),
    (dict(r=65), 2, "A*r=260"),
    (dict(A=8, r=48), 2, "A*r=384"),
    (dict(A=257, r=1), 2, "A*r=257"),
    (dict(d=64, A=1, r=65), 1, "exceeds d=64"),
    (dict(A=1, r=129), 1, "exceeds d=128"),
    (dict(K_fb=FAKE), 1, "both"),
    (dict(mask=None), 1, "mask_out"),
    (dict(ws=None), 4, "workspace"),
    (dict(ws=FAKE, ws_bytes=16), 4, "workspace"),
    (dict(ws=FAKE + 16, ws_bytes=1 << 30), 4, "aligned"),
    (dict(L=70000, H=1), 2, "segments"),
])
def test_correct_rejects_bad_arguments(kw, status, msg):
    st, err = _correct(**kw)
    assert st == status, err
    assert msg in err


def test_empty_cache_is_a_no_op():
    # L*H == 0: nothing to do, no pointer is needed and no HIP call is made
    st, err = _correct(L=0, K=None, V=None, U=None, W=None, desc=None, K_out=None, V_out=None,
                       mask=None)
    # desc/W/mask are still required pointers only when there are segments
    assert st == 0, err


def test_fit_rejects_bad_arguments():
    lib = kvc.lib()
    base = dict(delta=FAKE, M=4, T=64, d=128, dtype=0, r=32, energy=0.9, U=FAKE, W=FAKE,
                k=FAKE, eig=None, ws=None, nb=0, st=None)
    for kw, status in [(dict(r=0), 1), (dict(r=129), 1), (dict(energy=0.0), 1),
                       (dict(energy=1.5), 1), (dict(energy=float("nan")), 1), (dict(d=32), 2),
                       (dict(delta=None), 1), (dict(M=-1), 1), (dict(), 4),
                       (dict(U=FAKE + 8), 1)]:
        a = dict(base)
        a.update(kw)
        assert lib.kvc_fit_anchor(*a.values()) == status, (kw, lib.kvc_last_error())
    a = dict(base, M=0, delta=None, U=None, W=None, k=None)
    assert lib.kvc_fit_anchor(*a.values()) == 0


def test_chain_rejects_bad_arguments():
    lib = kvc.lib()
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE + 256)
    st = lib.kvc_correct_chain(FAKE, FAKE, 1, 1, 64, 128, 0, 0, arr, arr, arr, 4, 32, 0.3, None,
                               None, arr, arr, arr, None, None, 0, None)
    assert st == 1 and b"n_edges" in lib.kvc_last_error()
    st = lib.kvc_correct_chain(FAKE, FAKE, 1, 1, 64, 128, 0, 2, None, arr, arr, 4, 32, 0.3, None,
                               None, arr, arr, arr, None, None, 0, None)
    assert st == 1
    # an edge whose output aliases its source
    outs = (ctypes.c_void_p * 2)(FAKE, FAKE + 4096)
    st = lib.kvc_correct_chain(FAKE, FAKE, 1, 1, 64, 128, 0, 2, arr, arr, arr, 4, 32, 0.3, None,
                               None, outs, outs, arr, None, FAKE, 1 << 30, None)
    assert st == 1 and b"source" in lib.kvc_last_error()


def test_workspace_sizes_are_monotone():
    a = kvc.correct_workspace_bytes(32, 8, 2048, 128, 4, 32)
    b = kvc.correct_workspace_bytes(32, 8, 8192, 128, 4, 32)
    assert 0 < a < b
    assert kvc.fit_workspace_bytes(512, 8192, 128, 32) >= kvc.fit_workspace_bytes(512, 2048, 128, 32) > 0
    assert kvc.fit_workspace_bytes(1, 8192, 128, 32) > kvc.fit_workspace_bytes(1, 128, 128, 32) > 0


def test_streaming_fit_rejects_bad_arguments():
    lib = kvc.lib()
    # kvc_gram_accumulate(delta, M, T, d, dtype, G, ws, ws_bytes, stream)
    base = dict(delta=FAKE, M=4, T=64, d=128, dtype=0, G=FAKE, ws=None, nb=0, st=None)
    for kw, status in [(dict(d=32), 2), (dict(dtype=5), 1), (dict(M=-1), 1), (dict(T=-1), 1),
                       (dict(delta=None), 1), (dict(G=FAKE + 4), 1), (dict(), 4)]:
        a = dict(base)
        a.update(kw)
        assert lib.kvc_gram_accumulate(*a.values()) == status, (kw, lib.kvc_last_error())
    assert lib.kvc_gram_accumulate(*dict(base, T=0, delta=None, G=None).values()) == 0
    # kvc_fit_from_gram(G, M, d, r, energy, W, k, eig, stream)
    base = dict(G=FAKE, M=4, d=128, r=32, energy=0.9, W=FAKE, k=FAKE, eig=None, st=None)
    for kw, status in [(dict(r=0), 1), (dict(r=129), 1), (dict(energy=2.0), 1), (dict(d=96), 2),
                       (dict(G=None), 1), (dict(W=None), 1), (dict(k=FAKE + 2), 1)]:
        a = dict(base)
        a.update(kw)
        assert lib.kvc_fit_from_gram(*a.values()) == status, (kw, lib.kvc_last_error())
    assert lib.kvc_fit_from_gram(*dict(base, M=0, G=None, W=None, k=None).values()) == 0
    # kvc_refit_warm(G, M, d, r, energy, W_prev, W_out, k, warm, stream)
    base = dict(G=FAKE, M=4, d=128, r=32, energy=0.9, Wp=FAKE, W=FAKE, k=FAKE, warm=None,
                st=None)
    for kw, status in [(dict(r=0), 1), (dict(r=129), 1), (dict(energy=0.0), 1), (dict(d=96), 2),
                       (dict(G=None), 1), (dict(Wp=None), 1), (dict(W=None), 1),
                       (dict(k=None), 1), (dict(warm=FAKE + 2), 1), (dict(G=FAKE + 4), 1)]:
        a = dict(base)
        a.update(kw)
        assert lib.kvc_refit_warm(*a.values()) == status, (kw, lib.kvc_last_error())
    assert lib.kvc_refit_warm(*dict(base, M=0, G=None, Wp=None, W=None, k=None).values()) == 0
    # kvc_project(delta, M, T, d, dtype, W, r, U, ws, ws_bytes, stream)
    base = dict(delta=FAKE, M=4, T=64, d=128, dtype=0, W=FAKE, r=32, U=FAKE, ws=None, nb=0,
                st=None)
    for kw, status in [(dict(r=0), 1), (dict(d=64, r=65), 1), (dict(U=None), 1),
                       (dict(W=FAKE + 4), 1), (dict(dtype=7), 1)]:
        a = dict(base)
        a.update(kw)
        assert lib.kvc_project(*a.values()) == status, (kw, lib.kvc_last_error())
    assert lib.kvc_project_workspace_bytes(4, 128, 32, 1) == 0  # W is split in the kernel
    assert lib.kvc_project_workspace_bytes(4, 128, 32, 0) == 0
    assert lib.kvc_gram_workspace_bytes(512, 8192, 128) > lib.kvc_gram_workspace_bytes(1, 128, 128) > 0


def test_fanout_rejects_bad_arguments():
    lib = kvc.lib()
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE + (1 << 24))
    big = 1 << 30
    # kvc_correct_fanout(K, V, L, H, T, d, dtype, n, desc, U, W, A, r, tau, K_fb, V_fb,
    #                    K_out, V_out, mask, score, ws, ws_bytes, stream)
    st = lib.kvc_correct_fanout(FAKE, FAKE, 1, 1, 64, 128, 0, 0, arr, arr, arr, 4, 32, 0.3,
                                None, None, arr, arr, arr, None, None, 0, None)
    assert st == 1 and b"n_agents" in lib.kvc_last_error()
    st = lib.kvc_correct_fanout(FAKE, FAKE, 1, 1, 64, 128, 0, 2, arr, None, arr, 4, 32, 0.3,
                                None, None, arr, arr, arr, None, None, 0, None)
    assert st == 1 and b"arrays" in lib.kvc_last_error()
    # an agent's output on top of the shared reference
    K, V = 1 << 28, 1 << 29
    outk = (ctypes.c_void_p * 2)(K + 4096, 1 << 30)
    outv = (ctypes.c_void_p * 2)(1 << 31, 1 << 32)
    st = lib.kvc_correct_fanout(K, V, 1, 1, 64, 128, 0, 2, arr, arr, arr, 4, 32, 0.3, None,
                                None, outk, outv, arr, None, FAKE, big, None)
    assert st == 1 and b"reference" in lib.kvc_last_error()
    # two agents writing the same cache
    outk = (ctypes.c_void_p * 2)(1 << 30, 1 << 30)
    st = lib.kvc_correct_fanout(K, V, 1, 1, 64, 128, 0, 2, arr, arr, arr, 4, 32, 0.3, None,
                                None, outk, outv, arr, None, FAKE, big, None)
    assert st == 1 and b"overlap" in lib.kvc_last_error()
    # the per-agent checks of kvc_correct apply, with the agent named
    st = lib.kvc_correct_fanout(K, V, 1, 1, 64, 128, 0, 2, arr, arr, arr, 17, 32, 0.3, None,
                                None, outv, outk, arr, None, FAKE, big, None)
    assert st == 2 and b"agent 0" in lib.kvc_last_error()
    assert lib.kvc_fanout_workspace_bytes(32, 8, 2048, 128, 4, 32) == \
        kvc.correct_workspace_bytes(32, 8, 2048, 128, 4, 32)


def test_error_measures_reject_bad_arguments():
    lib = kvc.lib()
    # kvc_segment_error(X, ref, L, H, T, d, dtype, out, ws, ws_bytes, stream)
    base = dict(X=FAKE, R=FAKE, L=2, H=2, T=300, d=128, dtype=0, out=FAKE, ws=None, nb=0,
                st=None)
    for kw, status in [(dict(d=96), 2), (dict(dtype=3), 1), (dict(T=-2), 1), (dict(X=None), 1),
                       (dict(R=FAKE + 2), 1), (dict(out=FAKE + 4), 1), (dict(), 4),
                       (dict(ws=FAKE + 64, nb=1 << 20), 4)]:
        a = dict(base)
        a.update(kw)
        assert lib.kvc_segment_error(*a.values()) == status, (kw, lib.kvc_last_error())
    assert lib.kvc_segment_error(*dict(base, L=0, X=None, R=None, out=None).values()) == 0
    # two partials per segment and 256-token chunk
    assert lib.kvc_segment_error_workspace_bytes(2, 2, 300, 128) == 2 * 4 * 2 * 8
    # kvc_rank_error_curve(eig, M, n, curve, stream)
    assert lib.kvc_rank_error_curve(FAKE, 4, 0, FAKE, None) == 1
    assert lib.kvc_rank_error_curve(FAKE, 4, 257, FAKE, None) == 2
    assert lib.kvc_rank_error_curve(None, 4, 8, FAKE, None) == 1
    assert lib.kvc_rank_error_curve(FAKE, 4, 8, FAKE + 2, None) == 1
    assert lib.kvc_rank_error_curve(None, 0, 8, None, None) == 0


def test_anchor_pool_rejects_bad_arguments():
    lib = kvc.lib()
    big = 1 << 30
    # kvc_correct_pooled(K, V, L, H, T, d, dtype, desc, U, W, count, Vc, A, r, tau, q_in,
    #                    K_fb, V_fb, K_out, V_out, mask, score, w, slot, ws, ws_bytes, stream)
    base = dict(K=FAKE, V=FAKE, L=2, H=2, T=64, d=128, dtype=0, desc=FAKE, U=FAKE, W=FAKE,
                count=FAKE, Vc=10, A=4, r=32, tau=0.3, q_in=None, K_fb=None, V_fb=None,
                K_out=FAKE, V_out=FAKE, mask=FAKE, score=None, w=None, slot=None, ws=FAKE,
                nb=big, st=None)
    for kw, status, msg in [(dict(Vc=0), 1, "Vc=0"), (dict(Vc=33), 2, "Vc=33"),
                            (dict(A=5, Vc=4), 1, "capacity"), (dict(count=None), 1, "count"),
                            (dict(count=FAKE + 2), 1, "count"), (dict(A=17, Vc=20), 2, "A*r=544"),
                            (dict(slot=FAKE + 1), 1, "slot_out"), (dict(ws=None), 4, "work")]:
        a = dict(base)
        a.update(kw)
        assert lib.kvc_correct_pooled(*a.values()) == status, (kw, lib.kvc_last_error())
        assert msg in lib.kvc_last_error().decode()
    assert lib.kvc_correct_pooled(*dict(base, L=0).values()) == 0
    # kvc_anchor_pool_insert(mask, U_new, W_new, q, L, H, T, d, dtype, Vc, r, U_pool, W_pool,
    #                        desc_pool, count, head, stream)
    base = dict(mask=FAKE, U=FAKE, W=FAKE, q=FAKE, L=2, H=2, T=64, d=128, dtype=0, Vc=4, r=32,
                Up=FAKE, Wp=FAKE, dp=FAKE, count=FAKE, head=FAKE, st=None)
    for kw, status in [(dict(Vc=0), 1), (dict(Vc=40), 2), (dict(r=0), 1), (dict(r=129), 1),
                       (dict(d=48), 2), (dict(mask=None), 1), (dict(head=None), 1),
                       (dict(q=FAKE + 2), 1), (dict(U=None), 1)]:
        a = dict(base)
        a.update(kw)
        assert lib.kvc_anchor_pool_insert(*a.values()) == status, (kw, lib.kvc_last_error())
    assert lib.kvc_anchor_pool_insert(*dict(base, L=0).values()) == 0  # no segment: no-op


def test_noalloc_refuses_oversize_shapes_before_any_hip_call():
    lib = kvc.lib()
    # 32 x 8 x 8192 x 128, A = 4: about 33 MiB of workspace, more than the 16 MiB array
    st = lib.kvc_correct_noalloc(FAKE, FAKE, 32, 8, 8192, 128, 0, FAKE, FAKE, FAKE, 4, 32,
                                 ctypes.c_float(0.3), None, None, None, FAKE, FAKE, FAKE, None,
                                 None, None, None)
    assert st == 2 and "scratch" in lib.kvc_last_error().decode()
    st = lib.kvc_correct_noalloc(FAKE, FAKE, 2, 2, 64, 96, 0, FAKE, FAKE, FAKE, 4, 32,
                                 ctypes.c_float(0.3), None, None, None, FAKE, FAKE, FAKE, None,
                                 None, None, None)
    assert st == 2 and "d=96" in lib.kvc_last_error().decode()


def test_validation_paths_under_address_and_undefined_behaviour_sanitizers():
    """kvc_api.hip's host code built with ASan and UBSan, driven through every entry point's
    rejection paths (tests/abi_sanitize_main.cpp): no sanitizer report, every status right."""
    import shutil

    sanitize_abi = pytest.importorskip("sanitize_abi")

    if shutil.which(sanitize_abi.HIPCC) is None and not os.path.exists(sanitize_abi.HIPCC):
        pytest.skip("hipcc not available")
    if not all(os.path.exists(os.path.join(sanitize_abi.OBJ, o)) for o in sanitize_abi.OTHER):
        pytest.skip("library objects not built")
    out = sanitize_abi.build_and_run()
    assert "abi-sanitize ok" in out and "exit 0" in out, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
