"""Python binding of libkvc, the gfx950 HIP library for KVCMAS's online KV-cache correction.

Argument marshalling only: torch tensors supply device memory and the current stream;
every step of the computation runs in the library's HIP kernels.  The library is loaded
from this directory (built by ``agent_kv_cache_kvc_amd/build.py``); when it is missing
every call raises -- there is no fallback implementation.

Entry points (same names as the C ABI in include/kvc.h):
    pool_descriptor(K, V)                               -> q
    correct(K, V, desc, U, W, tau, ...)                 -> CorrectResult
    correct_chain(K0, V0, edges, tau)                   -> list[CorrectResult]
    correct_fanout(K, V, agents, tau)                   -> list[CorrectResult]
    rank_descriptor(K, V, rC) / correct_rank(...)       (matching on rank-rC representations)
    AnchorPool.empty(...) / correct_pooled / anchor_pool_insert   (online anchor pool)
    fit_anchor(delta, r=32, energy=0.9)                 -> FitResult
    gram_accumulate / fit_from_gram / project           (streaming fit)
    segment_error(X, ref)                               -> float64 [L, H, 2]
    rank_error_curve(eig)                               -> float32 [M, n + 1]
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "KvcError",
    "CorrectResult",
    "FitResult",
    "lib",
    "lib_path",
    "pool_descriptor",
    "correct",
    "correct_chain",
    "correct_fanout",
    "rank_descriptor",
    "correct_rank",
    "AnchorPool",
    "correct_pooled",
    "anchor_pool_insert",
    "fit_anchor",
    "correct_workspace_bytes",
    "chain_workspace_bytes",
    "fit_workspace_bytes",
    "gram_accumulate",
    "fit_from_gram",
    "refit_warm",
    "project",
    "segment_error",
    "rank_error_curve",
    "KVC_BF16",
    "KVC_F32",
]

KVC_BF16 = 0
KVC_F32 = 1
_STATUS = {0: "KVC_OK", 1: "KVC_ERR_ARG", 2: "KVC_ERR_UNSUPPORTED", 3: "KVC_ERR_HIP",
           4: "KVC_ERR_WORKSPACE"}

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libkvc.so")


class KvcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_SIGS = {
    "kvc_version": (ctypes.c_char_p, []),
    "kvc_last_error": (ctypes.c_char_p, []),
    "kvc_pool_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "kvc_pool_descriptor": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "kvc_correct_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "kvc_correct": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, ctypes.c_float,
                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kvc_correct_noalloc": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i,
                                 ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp]),
    "kvc_rank_descriptor_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "kvc_rank_descriptor": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "kvc_correct_rank": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _i, _i,
                              ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kvc_chain_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "kvc_correct_chain": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i,
                               ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kvc_fanout_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "kvc_correct_fanout": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i,
                                ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kvc_correct_pooled_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "kvc_correct_pooled": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _i,
                                ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _sz, _vp]),
    "kvc_anchor_pool_insert": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                    _vp, _vp, _vp, _vp]),
    "kvc_segment_error_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "kvc_segment_error": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "kvc_rank_error_curve": (_i, [_vp, _i, _i, _vp, _vp]),
    "kvc_fit_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "kvc_fit_anchor": (_i, [_vp, _i, _i, _i, _i, _i, ctypes.c_double, _vp, _vp, _vp, _vp, _vp,
                            _sz, _vp]),
    "kvc_gram_workspace_bytes": (_sz, [_i, _i, _i]),
    "kvc_gram_accumulate": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "kvc_fit_from_gram": (_i, [_vp, _i, _i, _i, ctypes.c_double, _vp, _vp, _vp, _vp]),
    "kvc_refit_warm": (_i, [_vp, _i, _i, _i, ctypes.c_double, _vp, _vp, _vp, _vp, _vp]),
    "kvc_project_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "kvc_project": (_i, [_vp, _i, _i, _i, _i, _vp, _i, _vp, _vp, _sz, _vp]),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libkvc.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is missing: build it with agent_kv_cache_kvc_amd/build.py")
        h = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = h
    return _LIB


def _check(status: int) -> None:
    if status != 0:
        raise KvcError(status, lib().kvc_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    if t.dtype == torch.float32:
        return KVC_F32
    raise TypeError(f"cache dtype must be bfloat16 or float32, got {t.dtype}")


def _need(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _ws(workspace: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    """The caller's workspace after checking it (device, contiguity; the library checks its
    size and alignment), or a new one of ``nbytes``."""
    if workspace is None:
        return _workspace(nbytes, device)
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace


def _ws_bytes(ws: torch.Tensor) -> int:
    return ws.numel() * ws.element_size()


def correct_workspace_bytes(L, H, T, d, A, r) -> int:
    return int(lib().kvc_correct_workspace_bytes(L, H, T, d, A, r))


def chain_workspace_bytes(L, H, T, d, A, r) -> int:
    return int(lib().kvc_chain_workspace_bytes(L, H, T, d, A, r))


def fit_workspace_bytes(M, T, d, r) -> int:
    return int(lib().kvc_fit_workspace_bytes(M, T, d, r))


def pool_descriptor(K: torch.Tensor, V: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q[l, h] = [mean_t K[l, h] ; mean_t V[l, h]] (float32) for K, V of shape [L, H, T, d]."""
    L, H, T, d = K.shape
    dev = K.device
    dt = _dtype_code(K)
    _need(V, "V", K.shape, K.dtype, dev)
    _need(K, "K", K.shape, K.dtype, dev)
    q = out if out is not None else torch.empty(L, H, 2 * d, dtype=torch.float32, device=dev)
    _need(q, "q_out", (L, H, 2 * d), torch.float32, dev)
    nb = int(lib().kvc_pool_workspace_bytes(L, H, T, d))
    ws = _ws(workspace, nb, dev)
    _check(lib().kvc_pool_descriptor(_ptr(K), _ptr(V), L, H, T, d, dt, _ptr(q), _ptr(ws),
                                     _ws_bytes(ws), _stream(dev)))
    return q


@dataclasses.dataclass
class CorrectResult:
    K: torch.Tensor
    V: torch.Tensor
    mask: torch.Tensor  # uint8 [L, H], 1 = fall back to dense prefill
    score: Optional[torch.Tensor] = None  # float32 [L, H]
    w: Optional[torch.Tensor] = None  # float32 [L, H, A]
    q_next: Optional[torch.Tensor] = None  # float32 [L, H, 2d]
    slots: Optional[torch.Tensor] = None  # int32 [L, H, A], pool slots (correct_pooled)


def correct(K: torch.Tensor, V: torch.Tensor, desc: torch.Tensor, U: torch.Tensor,
            W: torch.Tensor, tau: float, *, q_in: Optional[torch.Tensor] = None,
            K_fb: Optional[torch.Tensor] = None, V_fb: Optional[torch.Tensor] = None,
            K_out: Optional[torch.Tensor] = None, V_out: Optional[torch.Tensor] = None,
            want_score: bool = True, want_w: bool = True, want_q_next: bool = False,
            workspace: Optional[torch.Tensor] = None) -> CorrectResult:
    """Correct a reused cache with its segments' anchors (see kvc_correct in include/kvc.h).

    K, V: [L, H, T, d]; desc: [L, H, A, 2d] float32; U: [2, L, H, A, T, r];
    W: [2, L, H, A, r, d] (cache dtype).  Pass K_out=K, V_out=V to correct in place.
    """
    L, H, T, d = K.shape
    dev = K.device
    dt = _dtype_code(K)
    A = desc.shape[2]
    r = U.shape[-1]
    _need(K, "K", (L, H, T, d), K.dtype, dev)
    _need(V, "V", (L, H, T, d), K.dtype, dev)
    _need(desc, "desc", (L, H, A, 2 * d), torch.float32, dev)
    _need(U, "U", (2, L, H, A, T, r), K.dtype, dev)
    _need(W, "W", (2, L, H, A, r, d), K.dtype, dev)
    if q_in is not None:
        _need(q_in, "q_in", (L, H, 2 * d), torch.float32, dev)
    for name, t in (("K_fb", K_fb), ("V_fb", V_fb)):
        if t is not None:
            _need(t, name, (L, H, T, d), K.dtype, dev)
    Ko = K_out if K_out is not None else torch.empty_like(K)
    Vo = V_out if V_out is not None else torch.empty_like(V)
    _need(Ko, "K_out", (L, H, T, d), K.dtype, dev)
    _need(Vo, "V_out", (L, H, T, d), K.dtype, dev)
    mask = torch.empty(L, H, dtype=torch.uint8, device=dev)
    score = torch.empty(L, H, dtype=torch.float32, device=dev) if want_score else None
    w = torch.empty(L, H, A, dtype=torch.float32, device=dev) if want_w else None
    qn = torch.empty(L, H, 2 * d, dtype=torch.float32, device=dev) if want_q_next else None
    ws = _ws(workspace, correct_workspace_bytes(L, H, T, d, A, r), dev)
    _check(lib().kvc_correct(_ptr(K), _ptr(V), L, H, T, d, dt, _ptr(desc), _ptr(U), _ptr(W), A,
                             r, float(tau), _ptr(q_in), _ptr(K_fb), _ptr(V_fb), _ptr(Ko),
                             _ptr(Vo), _ptr(mask), _ptr(score), _ptr(w), _ptr(qn), _ptr(ws),
                             _ws_bytes(ws), _stream(dev)))
    return CorrectResult(Ko, Vo, mask, score, w, qn)


def rank_descriptor(K: torch.Tensor, V: torch.Tensor, rC: int = 32, *,
                    workspace: Optional[torch.Tensor] = None):
    """Rank-rC representation of every segment of a cache [L, H, T, d]: (F float32
    [2, L, H, rC, d], k_eff int32 [2, L, H]) -- see kvc_rank_descriptor in include/kvc.h."""
    L, H, T, d = K.shape
    dev = K.device
    dt = _dtype_code(K)
    _need(K, "K", (L, H, T, d), K.dtype, dev)
    _need(V, "V", (L, H, T, d), K.dtype, dev)
    F = torch.empty(2, L, H, rC, d, dtype=torch.float32, device=dev)
    k = torch.empty(2, L, H, dtype=torch.int32, device=dev)
    ws = _ws(workspace, lib().kvc_rank_descriptor_workspace_bytes(L, H, T, d, rC), dev)
    _check(lib().kvc_rank_descriptor(_ptr(K), _ptr(V), L, H, T, d, dt, int(rC), _ptr(F), _ptr(k),
                                     _ptr(ws), _ws_bytes(ws), _stream(dev)))
    return F, k


def correct_rank(K: torch.Tensor, V: torch.Tensor, Fq: torch.Tensor, Fa: torch.Tensor,
                 U: torch.Tensor, W: torch.Tensor, tau: float, *,
                 K_fb: Optional[torch.Tensor] = None, V_fb: Optional[torch.Tensor] = None,
                 K_out: Optional[torch.Tensor] = None, V_out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> CorrectResult:
    """kvc_correct with the anchors matched on rank-rC representations (see kvc_correct_rank in
    include/kvc.h).  Fq: [2, L, H, rC, d]; Fa: [2, L, H, A, rC, d] float32."""
    L, H, T, d = K.shape
    dev = K.device
    dt = _dtype_code(K)
    A, rC = Fa.shape[3], Fa.shape[4]
    r = U.shape[-1]
    _need(K, "K", (L, H, T, d), K.dtype, dev)
    _need(V, "V", (L, H, T, d), K.dtype, dev)
    _need(Fq, "Fq", (2, L, H, rC, d), torch.float32, dev)
    _need(Fa, "Fa", (2, L, H, A, rC, d), torch.float32, dev)
    _need(U, "U", (2, L, H, A, T, r), K.dtype, dev)
    _need(W, "W", (2, L, H, A, r, d), K.dtype, dev)
    for name, t in (("K_fb", K_fb), ("V_fb", V_fb)):
        if t is not None:
            _need(t, name, (L, H, T, d), K.dtype, dev)
    Ko = K_out if K_out is not None else torch.empty_like(K)
    Vo = V_out if V_out is not None else torch.empty_like(V)
    _need(Ko, "K_out", (L, H, T, d), K.dtype, dev)
    _need(Vo, "V_out", (L, H, T, d), K.dtype, dev)
    mask = torch.empty(L, H, dtype=torch.uint8, device=dev)
    score = torch.empty(L, H, dtype=torch.float32, device=dev)
    w = torch.empty(L, H, A, dtype=torch.float32, device=dev)
    ws = _ws(workspace, correct_workspace_bytes(L, H, T, d, A, r), dev)
    _check(lib().kvc_correct_rank(_ptr(K), _ptr(V), L, H, T, d, dt, _ptr(Fq), _ptr(Fa), int(rC),
                                  _ptr(U), _ptr(W), A, r, float(tau), _ptr(K_fb), _ptr(V_fb),
                                  _ptr(Ko), _ptr(Vo), _ptr(mask), _ptr(score), _ptr(w), _ptr(ws),
                                  _ws_bytes(ws), _stream(dev)))
    return CorrectResult(Ko, Vo, mask, score, w)


def _ptr_array(ts: Sequence[Optional[torch.Tensor]]):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if t is None else t.data_ptr()
    return arr


def correct_chain(K0: torch.Tensor, V0: torch.Tensor, edges: Sequence[dict], tau: float, *,
                  outputs: Optional[Sequence[tuple]] = None,
                  workspace: Optional[torch.Tensor] = None) -> list:
    """Chained correction A0 -> A1 -> ... (see kvc_correct_chain in include/kvc.h).

    ``edges``: one dict per edge with desc, U, W and optionally K_fb, V_fb.  ``outputs``:
    optional preallocated (K_out, V_out) per edge.  Returns one CorrectResult per edge.
    """
    L, H, T, d = K0.shape
    dev = K0.device
    dt = _dtype_code(K0)
    n = len(edges)
    if n < 1:
        raise ValueError("need at least one edge")
    A = edges[0]["desc"].shape[2]
    r = edges[0]["U"].shape[-1]
    _need(K0, "K0", (L, H, T, d), K0.dtype, dev)
    _need(V0, "V0", (L, H, T, d), K0.dtype, dev)
    if outputs is not None and len(outputs) != n:
        raise ValueError(f"outputs holds {len(outputs)} pairs for {n} edges")
    res = []
    for e, ed in enumerate(edges):
        _need(ed["desc"], f"desc[{e}]", (L, H, A, 2 * d), torch.float32, dev)
        _need(ed["U"], f"U[{e}]", (2, L, H, A, T, r), K0.dtype, dev)
        _need(ed["W"], f"W[{e}]", (2, L, H, A, r, d), K0.dtype, dev)
        for name in ("K_fb", "V_fb"):
            if ed.get(name) is not None:
                _need(ed[name], f"{name}[{e}]", K0.shape, K0.dtype, dev)
        if outputs is not None:
            Ko, Vo = outputs[e]
            _need(Ko, f"K_out[{e}]", (L, H, T, d), K0.dtype, dev)
            _need(Vo, f"V_out[{e}]", (L, H, T, d), K0.dtype, dev)
        else:
            Ko, Vo = torch.empty_like(K0), torch.empty_like(V0)
        res.append(CorrectResult(Ko, Vo, torch.empty(L, H, dtype=torch.uint8, device=dev),
                                 torch.empty(L, H, dtype=torch.float32, device=dev)))
    has_fb = [ed.get("K_fb") is not None for ed in edges]
    ws = _ws(workspace, int(lib().kvc_chain_workspace_bytes(L, H, T, d, A, r)), dev)
    _check(lib().kvc_correct_chain(
        _ptr(K0), _ptr(V0), L, H, T, d, dt, n,
        _ptr_array([ed["desc"] for ed in edges]), _ptr_array([ed["U"] for ed in edges]),
        _ptr_array([ed["W"] for ed in edges]), A, r, float(tau),
        _ptr_array([ed.get("K_fb") for ed in edges]) if any(has_fb) else None,
        _ptr_array([ed.get("V_fb") for ed in edges]) if any(has_fb) else None,
        _ptr_array([x.K for x in res]), _ptr_array([x.V for x in res]),
        _ptr_array([x.mask for x in res]), _ptr_array([x.score for x in res]),
        _ptr(ws), _ws_bytes(ws), _stream(dev)))
    return res


def correct_fanout(K: torch.Tensor, V: torch.Tensor, agents: Sequence[dict], tau: float, *,
                   outputs: Optional[Sequence[tuple]] = None,
                   workspace: Optional[torch.Tensor] = None) -> list:
    """Non-chained correction of one reference cache toward several agents (see
    kvc_correct_fanout in include/kvc.h).  ``agents``: one dict per agent with desc, U, W
    and optionally K_fb, V_fb.  Returns one CorrectResult per agent."""
    L, H, T, d = K.shape
    dev = K.device
    dt = _dtype_code(K)
    n = len(agents)
    if n < 1:
        raise ValueError("need at least one agent")
    A = agents[0]["desc"].shape[2]
    r = agents[0]["U"].shape[-1]
    _need(K, "K", (L, H, T, d), K.dtype, dev)
    _need(V, "V", (L, H, T, d), K.dtype, dev)
    if outputs is not None and len(outputs) != n:
        raise ValueError(f"outputs holds {len(outputs)} pairs for {n} agents")
    res = []
    for j, ag in enumerate(agents):
        _need(ag["desc"], f"desc[{j}]", (L, H, A, 2 * d), torch.float32, dev)
        _need(ag["U"], f"U[{j}]", (2, L, H, A, T, r), K.dtype, dev)
        _need(ag["W"], f"W[{j}]", (2, L, H, A, r, d), K.dtype, dev)
        for name in ("K_fb", "V_fb"):
            if ag.get(name) is not None:
                _need(ag[name], f"{name}[{j}]", K.shape, K.dtype, dev)
        if outputs is not None:
            Ko, Vo = outputs[j]
            _need(Ko, f"K_out[{j}]", (L, H, T, d), K.dtype, dev)
            _need(Vo, f"V_out[{j}]", (L, H, T, d), K.dtype, dev)
        else:
            Ko, Vo = torch.empty_like(K), torch.empty_like(V)
        res.append(CorrectResult(Ko, Vo, torch.empty(L, H, dtype=torch.uint8, device=dev),
                                 torch.empty(L, H, dtype=torch.float32, device=dev)))
    has_fb = any(ag.get("K_fb") is not None for ag in agents)
    ws = _ws(workspace, int(lib().kvc_fanout_workspace_bytes(L, H, T, d, A, r)), dev)
    _check(lib().kvc_correct_fanout(
        _ptr(K), _ptr(V), L, H, T, d, dt, n,
        _ptr_array([ag["desc"] for ag in agents]), _ptr_array([ag["U"] for ag in agents]),
        _ptr_array([ag["W"] for ag in agents]), A, r, float(tau),
        _ptr_array([ag.get("K_fb") for ag in agents]) if has_fb else None,
        _ptr_array([ag.get("V_fb") for ag in agents]) if has_fb else None,
        _ptr_array([x.K for x in res]), _ptr_array([x.V for x in res]),
        _ptr_array([x.mask for x in res]), _ptr_array([x.score for x in res]),
        _ptr(ws), _ws_bytes(ws), _stream(dev)))
    return res


@dataclasses.dataclass
class AnchorPool:
    """Device storage of the online anchor pools of all segments (see kvc_correct_pooled and
    kvc_anchor_pool_insert in include/kvc.h): Vc slots per segment."""
    desc: torch.Tensor  # float32 [L, H, Vc, 2d]
    U: torch.Tensor  # cache dtype [2, L, H, Vc, T, r]
    W: torch.Tensor  # cache dtype [2, L, H, Vc, r, d]
    count: torch.Tensor  # int32 [L, H], valid slots
    head: torch.Tensor  # int32 [L, H], next slot to write

    @staticmethod
    def empty(L, H, T, d, Vc, r, dtype=torch.bfloat16, device="cuda") -> "AnchorPool":
        z = dict(device=device)
        return AnchorPool(torch.zeros(L, H, Vc, 2 * d, dtype=torch.float32, **z),
                          torch.zeros(2, L, H, Vc, T, r, dtype=dtype, **z),
                          torch.zeros(2, L, H, Vc, r, d, dtype=dtype, **z),
                          torch.zeros(L, H, dtype=torch.int32, **z),
                          torch.zeros(L, H, dtype=torch.int32, **z))

    @property
    def Vc(self) -> int:
        return self.desc.shape[2]


def correct_pooled(K: torch.Tensor, V: torch.Tensor, pool: AnchorPool, A: int, tau: float, *,
                   q_in: Optional[torch.Tensor] = None, K_fb: Optional[torch.Tensor] = None,
                   V_fb: Optional[torch.Tensor] = None, K_out: Optional[torch.Tensor] = None,
                   V_out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> CorrectResult:
    """Correct a reused cache from each segment's online anchor pool (top-A slots by cosine;
    see kvc_correct_pooled in include/kvc.h).  The result's ``w`` holds the selected
    anchors' weights; ``slots`` (int32 [L, H, A]) their pool slots."""
    L, H, T, d = K.shape
    dev = K.device
    dt = _dtype_code(K)
    Vc = pool.Vc
    r = pool.U.shape[-1]
    _need(K, "K", (L, H, T, d), K.dtype, dev)
    _need(V, "V", (L, H, T, d), K.dtype, dev)
    _need(pool.desc, "desc_pool", (L, H, Vc, 2 * d), torch.float32, dev)
    _need(pool.U, "U_pool", (2, L, H, Vc, T, r), K.dtype, dev)
    _need(pool.W, "W_pool", (2, L, H, Vc, r, d), K.dtype, dev)
    _need(pool.count, "count", (L, H), torch.int32, dev)
    if q_in is not None:
        _need(q_in, "q_in", (L, H, 2 * d), torch.float32, dev)
    for name, t in (("K_fb", K_fb), ("V_fb", V_fb)):
        if t is not None:
            _need(t, name, (L, H, T, d), K.dtype, dev)
    Ko = K_out if K_out is not None else torch.empty_like(K)
    Vo = V_out if V_out is not None else torch.empty_like(V)
    _need(Ko, "K_out", (L, H, T, d), K.dtype, dev)
    _need(Vo, "V_out", (L, H, T, d), K.dtype, dev)
    mask = torch.empty(L, H, dtype=torch.uint8, device=dev)
    score = torch.empty(L, H, dtype=torch.float32, device=dev)
    w = torch.empty(L, H, A, dtype=torch.float32, device=dev)
    slots = torch.empty(L, H, A, dtype=torch.int32, device=dev)
    ws = _ws(workspace, lib().kvc_correct_pooled_workspace_bytes(L, H, T, d, A, r), dev)
    _check(lib().kvc_correct_pooled(_ptr(K), _ptr(V), L, H, T, d, dt, _ptr(pool.desc),
                                    _ptr(pool.U), _ptr(pool.W), _ptr(pool.count), Vc, int(A), r,
                                    float(tau), _ptr(q_in), _ptr(K_fb), _ptr(V_fb), _ptr(Ko),
                                    _ptr(Vo), _ptr(mask), _ptr(score), _ptr(w), _ptr(slots),
                                    _ptr(ws), _ws_bytes(ws), _stream(dev)))
    return CorrectResult(Ko, Vo, mask, score, w, slots=slots)


def anchor_pool_insert(pool: AnchorPool, mask: torch.Tensor, U_new: torch.Tensor,
                       W_new: torch.Tensor, q: torch.Tensor) -> AnchorPool:
    """Insert new anchors (fit factors U_new float32 [2, L, H, T, r] or [2LH, T, r], W_new
    float32 [2, L, H, r, d] or [2LH, r, d]) with descriptors q [L, H, 2d] into the pools of
    the segments whose mask is set, first in first out (see kvc_anchor_pool_insert)."""
    _, L, H, Vc, T, r = pool.U.shape
    d = pool.W.shape[-1]
    dev = pool.U.device
    dt = _dtype_code(pool.U)
    U_new = U_new.reshape(2, L, H, T, r)
    W_new = W_new.reshape(2, L, H, r, d)
    _need(mask, "mask", (L, H), torch.uint8, dev)
    _need(U_new, "U_new", (2, L, H, T, r), torch.float32, dev)
    _need(W_new, "W_new", (2, L, H, r, d), torch.float32, dev)
    _need(q, "q", (L, H, 2 * d), torch.float32, dev)
    _need(pool.head, "head", (L, H), torch.int32, dev)
    _check(lib().kvc_anchor_pool_insert(_ptr(mask), _ptr(U_new), _ptr(W_new), _ptr(q), L, H, T,
                                        d, dt, Vc, r, _ptr(pool.U), _ptr(pool.W),
                                        _ptr(pool.desc), _ptr(pool.count), _ptr(pool.head),
                                        _stream(dev)))
    return pool


def segment_error(X: torch.Tensor, ref: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per segment [sum (X - ref)^2, sum ref^2] (float64 [L, H, 2]) for caches [L, H, T, d]
    (see kvc_segment_error in include/kvc.h)."""
    L, H, T, d = X.shape
    dev = X.device
    dt = _dtype_code(X)
    _need(X, "X", (L, H, T, d), X.dtype, dev)
    _need(ref, "ref", (L, H, T, d), X.dtype, dev)
    o = out if out is not None else torch.empty(L, H, 2, dtype=torch.float64, device=dev)
    _need(o, "out", (L, H, 2), torch.float64, dev)
    ws = _ws(workspace, lib().kvc_segment_error_workspace_bytes(L, H, T, d), dev)
    _check(lib().kvc_segment_error(_ptr(X), _ptr(ref), L, H, T, d, dt, _ptr(o), _ptr(ws),
                                   _ws_bytes(ws), _stream(dev)))
    return o


def rank_error_curve(eig: torch.Tensor) -> torch.Tensor:
    """Relative error of the best rank-k approximation, k = 0..n, from descending eigenvalues
    eig float32 [M, n] -> float32 [M, n + 1] (see kvc_rank_error_curve in include/kvc.h)."""
    M, n = eig.shape
    dev = eig.device
    _need(eig, "eig", (M, n), torch.float32, dev)
    c = torch.empty(M, n + 1, dtype=torch.float32, device=dev)
    _check(lib().kvc_rank_error_curve(_ptr(eig), M, n, _ptr(c), _stream(dev)))
    return c


@dataclasses.dataclass
class FitResult:
    U: Optional[torch.Tensor]  # float32 [M, T, r] (None from fit_from_gram)
    W: torch.Tensor  # float32 [M, r, d]
    k_eff: torch.Tensor  # int32 [M]
    eig: Optional[torch.Tensor] = None  # float32 [M, d], descending


def fit_anchor(delta: torch.Tensor, r: int = 32, energy: float = 0.9, *, want_eig: bool = True,
               workspace: Optional[torch.Tensor] = None) -> FitResult:
    """Rank-r anchor of delta [M, T, d] (see kvc_fit_anchor in include/kvc.h)."""
    M, T, d = delta.shape
    dev = delta.device
    dt = _dtype_code(delta)
    _need(delta, "delta", (M, T, d), delta.dtype, dev)
    U = torch.empty(M, T, r, dtype=torch.float32, device=dev)
    W = torch.empty(M, r, d, dtype=torch.float32, device=dev)
    k = torch.empty(M, dtype=torch.int32, device=dev)
    eig = torch.empty(M, d, dtype=torch.float32, device=dev) if want_eig else None
    ws = _ws(workspace, fit_workspace_bytes(M, T, d, r), dev)
    _check(lib().kvc_fit_anchor(_ptr(delta), M, T, d, dt, int(r), float(energy), _ptr(U),
                                _ptr(W), _ptr(k), _ptr(eig), _ptr(ws), _ws_bytes(ws), _stream(dev)))
    return FitResult(U, W, k, eig)


def gram_accumulate(delta: torch.Tensor, G: Optional[torch.Tensor] = None, *,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """G += delta^T delta for a block of rows delta [M, T, d]; G float64 [M, d, d] (a new zero
    G when None).  See kvc_gram_accumulate in include/kvc.h."""
    M, T, d = delta.shape
    dev = delta.device
    dt = _dtype_code(delta)
    _need(delta, "delta", (M, T, d), delta.dtype, dev)
    if G is None:
        G = torch.zeros(M, d, d, dtype=torch.float64, device=dev)
    _need(G, "G", (M, d, d), torch.float64, dev)
    ws = _ws(workspace, lib().kvc_gram_workspace_bytes(M, T, d), dev)
    _check(lib().kvc_gram_accumulate(_ptr(delta), M, T, d, dt, _ptr(G), _ptr(ws), _ws_bytes(ws),
                                     _stream(dev)))
    return G


def fit_from_gram(G: torch.Tensor, r: int = 32, energy: float = 0.9, *,
                  want_eig: bool = True) -> FitResult:
    """W, k_eff (and eigenvalues) from an accumulated Gram matrix G float64 [M, d, d]; U is
    None (see project).  See kvc_fit_from_gram in include/kvc.h."""
    M, d, _ = G.shape
    dev = G.device
    _need(G, "G", (M, d, d), torch.float64, dev)
    W = torch.empty(M, r, d, dtype=torch.float32, device=dev)
    k = torch.empty(M, dtype=torch.int32, device=dev)
    eig = torch.empty(M, d, dtype=torch.float32, device=dev) if want_eig else None
    _check(lib().kvc_fit_from_gram(_ptr(G), M, d, int(r), float(energy), _ptr(W), _ptr(k),
                                   _ptr(eig), _stream(dev)))
    return FitResult(None, W, k, eig)


def refit_warm(G: torch.Tensor, W_prev: torch.Tensor, energy: float = 0.9, *,
               W_out: Optional[torch.Tensor] = None, want_warm: bool = True):
    """Refit from an accumulated G [M, d, d] float64 starting from the previous W_prev
    [M, r, d] float32 (kvc_refit_warm in include/kvc.h).  Returns (FitResult with W and
    k_eff, warm [M] int32 or None: 1 where the warm result was kept).  W_out may be W_prev
    itself (in-place update)."""
    M, d, _ = G.shape
    r = W_prev.shape[1]
    dev = G.device
    _need(G, "G", (M, d, d), torch.float64, dev)
    _need(W_prev, "W_prev", (M, r, d), torch.float32, dev)
    if W_out is None:
        W_out = torch.empty(M, r, d, dtype=torch.float32, device=dev)
    _need(W_out, "W_out", (M, r, d), torch.float32, dev)
    k = torch.empty(M, dtype=torch.int32, device=dev)
    warm = torch.empty(M, dtype=torch.int32, device=dev) if want_warm else None
    _check(lib().kvc_refit_warm(_ptr(G), M, d, int(r), float(energy), _ptr(W_prev), _ptr(W_out),
                                _ptr(k), _ptr(warm), _stream(dev)))
    return FitResult(None, W_out, k, None), warm


def project(delta: torch.Tensor, W: torch.Tensor, *,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """U = delta W^T for delta [M, T, d] and W float32 [M, r, d].  See kvc_project."""
    M, T, d = delta.shape
    r = W.shape[1]
    dev = delta.device
    dt = _dtype_code(delta)
    _need(delta, "delta", (M, T, d), delta.dtype, dev)
    _need(W, "W", (M, r, d), torch.float32, dev)
    U = torch.empty(M, T, r, dtype=torch.float32, device=dev)
    need = lib().kvc_project_workspace_bytes(M, d, r, dt)
    ws = _ws(workspace, need, dev) if (need or workspace is not None) else None
    _check(lib().kvc_project(_ptr(delta), M, T, d, dt, _ptr(W), r, _ptr(U), _ptr(ws),
                             0 if ws is None else _ws_bytes(ws), _stream(dev)))
    return U
