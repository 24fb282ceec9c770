"""Shared pieces of the GPU parity tests: inputs on the device, oracle references on the host,
and the comparison bars.

Bars (floating point): relative Frobenius error <= 1e-3 and max-abs error <= 1e-2 * max|ref|
against the oracle rounded to the cache dtype; the fallback mask and the effective rank
must match exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

REL_FROB = 1e-3
MAX_ABS = 1e-2


def dev() -> torch.device:
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def pool_all(K: torch.Tensor, V: torch.Tensor) -> np.ndarray:
    """Oracle pooled descriptors of every segment, converted layer by layer (host memory)."""
    L, H, T, d = K.shape
    q = np.empty((L, H, 2 * d))
    for l in range(L):
        q[l] = oracle.pool(synth.to_f64(K[l]), synth.to_f64(V[l]))
    return q


def check_close(name: str, got: np.ndarray, ref: np.ndarray, rel=REL_FROB, mabs=MAX_ABS) -> float:
    err = oracle.rel_frobenius(got, ref)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    worst = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    say(f"  {name}: rel-Frobenius {err:.3e} (bar {rel:.0e}), max-abs {worst:.3e} "
        f"= {worst / m if m > 0 else 0.0:.3e} x max|ref| (bar {mabs:.0e})")
    assert err <= rel, f"{name}: relative Frobenius error {err:.3e} > {rel:.0e}"
    assert worst <= mabs * m + 1e-30, f"{name}: max-abs error {worst:.3e} > {mabs:.0e} * {m:.3e}"
    return err


def correct_inputs(case: synth.Case, device, edge: int = 0, q=None):
    """(desc on device, q used for it) for one edge whose source is the case's edge source."""
    if q is None:
        if edge == 0:
            q = pool_all(case.K0, case.V0)
        else:
            q = pool_all(case.edges[edge - 1].exact_K, case.edges[edge - 1].exact_V)
    desc = synth.build_descriptors(case, edge, q)
    return desc.to(device), q


def oracle_correct_segments(case, desc, segs, tau, K=None, V=None, edge=0, K_fb=None, V_fb=None):
    """Oracle correction of the listed (l, h) segments only, stacked as [n, 1, ...]."""
    cfg = case.cfg
    K = case.K0 if K is None else K
    V = case.V0 if V is None else V
    ed = case.edges[edge]
    ls = torch.tensor([s[0] for s in segs])
    hs = torch.tensor([s[1] for s in segs])

    def pick(t):
        return synth.to_f64(t[ls.to(t.device), hs.to(t.device)])[:, None]

    def pick_f(t):  # factors [2, L, H, ...]
        return synth.to_f64(t[:, ls.to(t.device), hs.to(t.device)])[:, :, None]

    return oracle.correct(pick(K), pick(V), pick(desc), pick_f(ed.U), pick_f(ed.W), tau,
                          cfg.dtype, K_fb=None if K_fb is None else pick(K_fb),
                          V_fb=None if V_fb is None else pick(V_fb))


def sample_segments(L, H, mask: np.ndarray, n: int, seed: int = 0):
    """Up to n segments: masked and unmasked ones both represented, first and last included."""
    rng = np.random.default_rng(seed)
    allsegs = [(l, h) for l in range(L) for h in range(H)]
    fall = [s for s in allsegs if mask[s]]
    keep = [s for s in allsegs if not mask[s]]
    pick = {allsegs[0], allsegs[-1]}
    for pool_, k in ((fall, max(1, n // 4)), (keep, n)):
        if pool_:
            idx = rng.choice(len(pool_), size=min(k, len(pool_)), replace=False)
            pick.update(pool_[i] for i in idx)
    return sorted(pick)[: max(n, 2)]


def check_fit(name, got_U, got_W, got_k, got_eig, ref, r, delta):
    """Fit parity of a set of matrices against the oracle's truncated SVD.

    Always: effective rank exact; eigenvalues within 2e-5 * lambda_0 (and top ones within
    1e-3 relative); the truncation error ||delta - U W||^2 equal to the oracle's tail energy
    within 1e-4 of ||delta||^2 (Eckart-Young: every correct truncation has it).  When the
    rank-r subspace is unique (gap lambda_{r-1} - lambda_r > 1e-3 lambda_0): U W within the
    1e-3 bar.  When every kept eigenvalue is separated (gaps > 1e-4 lambda_0): W and U
    themselves (canonical signs on both sides) within the bar.
    """
    M = got_k.shape[0]
    np.testing.assert_array_equal(got_k, ref["k_eff"], err_msg=f"{name}: effective rank")
    for m in range(M):
        lam = ref["eig"][m]
        l0 = lam[0]
        if l0 == 0:
            assert np.all(got_U[m] == 0), f"{name}[{m}]: zero delta must give U = 0"
            continue
        np.testing.assert_allclose(got_eig[m], lam, rtol=0, atol=2e-5 * l0,
                                   err_msg=f"{name}[{m}]: eigenvalues")
        big = lam[:r] >= 1e-3 * l0
        np.testing.assert_allclose(got_eig[m][:r][big], lam[:r][big], rtol=1e-3,
                                   err_msg=f"{name}[{m}]: top eigenvalues")
        total = float(np.sum(delta[m] ** 2))
        tail_g = float(np.sum((delta[m] - got_U[m] @ got_W[m]) ** 2))
        tail_o = float(np.sum(lam[r:]))
        assert abs(tail_g - tail_o) <= 1e-4 * total, \
            f"{name}[{m}]: truncation energy {tail_g / total:.6e} vs {tail_o / total:.6e}"
        if r < lam.shape[0] and (lam[r - 1] - lam[r]) <= 1e-3 * l0:
            continue
        e = oracle.rel_frobenius(got_U[m] @ got_W[m], ref["U"][m] @ ref["W"][m])
        assert e <= REL_FROB, f"{name}[{m}]: U W relative error {e:.3e}"
        gaps = -np.diff(lam[: min(r + 1, lam.shape[0])])
        if np.all(gaps > 1e-4 * l0) and lam[r - 1] > 1e-4 * l0:
            e = oracle.rel_frobenius(got_W[m], ref["W"][m])
            assert e <= REL_FROB, f"{name}[{m}]: W relative error {e:.3e}"
            e = oracle.rel_frobenius(got_U[m], ref["U"][m])
            assert e <= REL_FROB, f"{name}[{m}]: U relative error {e:.3e}"


def energy_margin(eig: np.ndarray, energy: float = 0.9) -> np.ndarray:
    """Distance of the cumulative energy fractions at k_eff - 1 and k_eff from the threshold."""
    lam = np.clip(eig, 0, None)
    tot = lam.sum(-1, keepdims=True)
    frac = np.cumsum(lam, -1) / np.where(tot > 0, tot, 1)
    return np.min(np.abs(frac - energy), axis=-1)


def check_every_segment(name: str, got_K, got_V, ref_layer, L: int, mask=None) -> None:
    """Corrected caches of every segment against the oracle, one layer at a time.
    ref_layer(l) returns the oracle's result for layer l (a dict with K_out, V_out, mask of
    shape [1, H, ...]); got_K, got_V are the library's [L, H, T, d] outputs; mask (if given)
    is the expected [L, H] decision.  The bars apply to the whole tensors; the worst segment's
    relative error is printed as well."""
    acc = {x: [0.0, 0.0, 0.0, 0.0] for x in ("K", "V")}  # err^2, ref^2, max|diff|, max|ref|
    worst = (0.0, None)
    for l in range(L):
        ref = ref_layer(l)
        if mask is not None:
            np.testing.assert_array_equal(ref["mask"][0], mask[l], err_msg=f"{name} layer {l}")
        for x, got_t in (("K", got_K), ("V", got_V)):
            got = synth.to_f64(got_t[l:l + 1])
            want = ref[f"{x}_out"]
            diff = got - want
            a = acc[x]
            a[0] += float(np.sum(diff ** 2))
            a[1] += float(np.sum(want ** 2))
            a[2] = max(a[2], float(np.max(np.abs(diff))) if diff.size else 0.0)
            a[3] = max(a[3], float(np.max(np.abs(want))) if want.size else 0.0)
            seg = np.sqrt(np.sum(diff ** 2, axis=(-2, -1)) /
                          np.maximum(np.sum(want ** 2, axis=(-2, -1)), 1e-300))
            h = int(np.argmax(seg[0]))
            if seg[0, h] > worst[0]:
                worst = (float(seg[0, h]), (x, l, h))
    for x in ("K", "V"):
        e2, r2, da, ra = acc[x]
        rel = float(np.sqrt(e2 / r2)) if r2 > 0 else 0.0
        say(f"  {name} {x}' every segment: rel-Frobenius {rel:.3e} (bar {REL_FROB:.0e}), "
            f"max-abs {da:.3e} = {da / ra if ra > 0 else 0.0:.3e} x max|ref| (bar {MAX_ABS:.0e})")
        assert rel <= REL_FROB, f"{name} {x}': relative Frobenius error {rel:.3e}"
        assert da <= MAX_ABS * ra + 1e-30, f"{name} {x}': max-abs error {da:.3e}"
    say(f"  {name} worst segment {worst[1]}: rel-Frobenius {worst[0]:.3e}")
