"""GPU parity of the anchor fit (kvc_fit_anchor: Gram, eigensolver, effective rank, projection)
against the fp64 oracle's truncated SVD, through the C ABI."""
import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import oracle
import synth
from gpu_helpers import check_fit, dev, energy_margin, say

pytestmark = pytest.mark.gpu


# Effective ranks are compared on every matrix.  The library decides k_eff in float64 from
# float64 Gram sums whenever its fast path cannot certify the decision, and the oracle takes it
# from a float64 SVD; both resolve the cumulative energy fraction to about 1e-13, so only a
# matrix whose fraction lies within TIE of the threshold could legitimately differ (none of the
# inputs here comes near it; the count is printed).
TIE = 1e-11


def _fit_and_check(name, delta_host: torch.Tensor, r, energy=0.9, idx=None, tie_band=TIE):
    d = dev()
    out = kvc.fit_anchor(delta_host.to(d), r=r, energy=energy)
    torch.cuda.synchronize()
    idx = list(range(delta_host.shape[0])) if idx is None else idx
    dh = synth.to_f64(delta_host[idx])
    ref = oracle.fit_anchor(dh, r, energy)
    margin = energy_margin(ref["eig"], energy)
    ok = margin > tie_band
    got_k = out.k_eff.cpu().numpy()[idx]
    say(f"  {name}: {len(idx)} matrices, min energy margin {margin.min():.2e}, "
        f"{int((margin < 1e-4).sum())} within 1e-4 of the threshold, "
        f"{int((~ok).sum())} within {tie_band:.0e}")
    assert ok.all(), "a matrix sits on the threshold within float64 resolution"
    sel = np.nonzero(ok)[0]
    sub = {k: v[sel] for k, v in ref.items()}
    check_fit(name, out.U.cpu().numpy()[idx][sel].astype(np.float64),
              out.W.cpu().numpy()[idx][sel].astype(np.float64), got_k[sel],
              out.eig.cpu().numpy()[idx][sel].astype(np.float64), sub, r, dh[sel])
    return out, ref


def test_tiny_fit_planted_closed_form():
    case = synth.generate("tiny")
    delta = synth.fit_input(case)
    out, ref = _fit_and_check("tiny", delta, 8)
    # planted rho = 0.8, r = 8: the top-5 energy is 0.918 >= 0.9 > 0.856 (top-4)
    assert out.k_eff.cpu().tolist() == [5, 5]


@pytest.mark.parametrize("dtype,d,T,r,M", [
    ("bf16", 128, 700, 32, 6),
    ("bf16", 128, 129, 1, 3),
    ("bf16", 64, 1000, 16, 4),
    ("bf16", 128, 16, 32, 2),     # T < d: rank-deficient Gram
    ("bf16", 128, 3000, 64, 3),
    ("bf16", 128, 2048, 128, 2),
    ("f32", 64, 300, 8, 3),
    ("f32", 128, 517, 40, 2),
])
def test_fit_small_shapes(dtype, d, T, r, M):
    say(f"[fit] {dtype} d={d} T={T} r={r} M={M}")
    g = torch.Generator().manual_seed(T * 7 + r)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # planted geometric spectrum (decay 0.85) of rank min(T, d) plus noise
    k = min(T, d)
    out = torch.empty(M, T, d, dtype=tdt)
    for m in range(M):
        P, _ = torch.linalg.qr(torch.randn(T, k, generator=g, dtype=torch.float64))
        Q, _ = torch.linalg.qr(torch.randn(d, k, generator=g, dtype=torch.float64))
        s = 5.0 * 0.85 ** torch.arange(k, dtype=torch.float64)
        x = (P * s) @ Q.T + 1e-3 * torch.randn(T, d, generator=g, dtype=torch.float64)
        out[m] = x.to(tdt)
    _fit_and_check(f"small-{dtype}-{d}-{T}-{r}", out, r)


def test_fit_exact_low_rank_and_zero():
    g = torch.Generator().manual_seed(3)
    T, d, r = 500, 128, 32
    P, _ = torch.linalg.qr(torch.randn(T, 5, generator=g, dtype=torch.float64))
    Q, _ = torch.linalg.qr(torch.randn(d, 5, generator=g, dtype=torch.float64))
    x = ((P * torch.tensor([4.0, 3.0, 2.0, 1.0, 0.5], dtype=torch.float64)) @ Q.T)
    delta = torch.stack([x.float(), torch.zeros(T, d)])
    out = kvc.fit_anchor(delta.to(dev()), r=r)
    torch.cuda.synchronize()
    U, W = out.U.cpu().double(), out.W.cpu().double()
    rec = (U[0] @ W[0]).numpy()
    assert oracle.rel_frobenius(rec, x.float().double().numpy()) < 1e-4
    assert out.k_eff.cpu().tolist()[1] == 0
    assert float(U[1].abs().sum()) == 0.0
    ref = oracle.fit_anchor(delta[:1].double().numpy(), r)
    assert out.k_eff.cpu().tolist()[0] == int(ref["k_eff"][0])
    # rows of W are orthonormal
    np.testing.assert_allclose((W[0] @ W[0].T).numpy(), np.eye(r), atol=1e-5)


def test_fit_deterministic():
    g = torch.Generator().manual_seed(4)
    delta = torch.randn(4, 1500, 128, generator=g).to(torch.bfloat16).to(dev())
    a = kvc.fit_anchor(delta, r=32)
    b = kvc.fit_anchor(delta, r=32)
    torch.cuda.synchronize()
    assert torch.equal(a.U, b.U) and torch.equal(a.W, b.W) and torch.equal(a.k_eff, b.k_eff)


def _full_fit(cfg, n_samples=None, edge=0):
    """Full-size fit of a workload's delta: the effective rank of every matrix equals the
    planted closed form (11); U, W, eigenvalues and k_eff against the oracle's SVD on every
    matrix (n_samples None, in chunks of 64) or on a sample."""
    say(f"[fit-full] {cfg.name} M={2 * cfg.L * cfg.H} T={cfg.T}")
    d = dev()
    case = synth.generate(cfg, d)
    delta = synth.fit_input(case, edge)
    del case
    torch.cuda.empty_cache()
    M = delta.shape[0]
    out = kvc.fit_anchor(delta, r=cfg.r)
    torch.cuda.synchronize()
    k = out.k_eff.cpu().numpy()
    # planted decay 0.9 with r = 32 has the closed-form effective rank 11 (energy 0.9026
    # at 11, 0.8795 at 10); every matrix shows it
    assert np.all(k == 11), np.unique(k, return_counts=True)
    if n_samples is None:
        chunks = [list(range(c, min(M, c + 64))) for c in range(0, M, 64)]
    else:
        rng = np.random.default_rng(0)
        chunks = [sorted(set([0, M - 1] + rng.choice(M, n_samples, replace=False).tolist()))]
    margin_min = np.inf
    for idx in chunks:
        dh = synth.to_f64(delta[idx])
        ref = oracle.fit_anchor(dh, cfg.r)
        margin_min = min(margin_min, float(energy_margin(ref["eig"], 0.9).min()))
        check_fit(cfg.name, out.U[idx].cpu().double().numpy(), out.W[idx].cpu().double().numpy(),
                  k[idx], out.eig[idx].cpu().double().numpy(), ref, cfg.r, dh)
    n = sum(len(c) for c in chunks)
    say(f"  {n} of {M} matrices match the oracle (U, W, eigenvalues, k_eff); min energy margin "
        f"{margin_min:.2e}")
    del delta, out
    torch.cuda.empty_cache()


def test_llama8b_t8192_fit_full_size():
    _full_fit(synth.CONFIGS["llama8b_t8192_fit"])


def test_vl_t9216_fit_full_size():
    _full_fit(synth.CONFIGS["vl_t9216"])


def test_chain_t32768_fit_full_size():
    _full_fit(synth.CONFIGS["chain_t32768"].replace(n_edges=1), 30)


@pytest.mark.parametrize("d,T,r,M,flat", [
    (128, 700, 32, 4, False),   # effective rank within the r largest
    (128, 600, 4, 3, True),     # flat spectrum: effective rank far above r
    (64, 900, 16, 3, False),
    (64, 500, 2, 2, True),
])
def test_fit_without_eigenvalues_matches(d, T, r, M, flat):
    """Without eigenvalue output only the r largest are bracketed unless the effective rank
    needs more; U, W and k_eff must not depend on that."""
    say(f"[fit] want_eig False vs True: d={d} T={T} r={r} M={M} flat={flat}")
    g = torch.Generator().manual_seed(T + r)
    if flat:
        x = torch.randn(M, T, d, generator=g, dtype=torch.float64)
    else:
        k = min(T, d)
        x = torch.empty(M, T, d, dtype=torch.float64)
        for m in range(M):
            P, _ = torch.linalg.qr(torch.randn(T, k, generator=g, dtype=torch.float64))
            Q, _ = torch.linalg.qr(torch.randn(d, k, generator=g, dtype=torch.float64))
            x[m] = (P * (4.0 * 0.8 ** torch.arange(k, dtype=torch.float64))) @ Q.T
    delta = x.to(torch.bfloat16).to(dev())
    a = kvc.fit_anchor(delta, r=r, want_eig=True)
    b = kvc.fit_anchor(delta, r=r, want_eig=False)
    torch.cuda.synchronize()
    assert b.eig is None
    assert torch.equal(a.U, b.U) and torch.equal(a.W, b.W) and torch.equal(a.k_eff, b.k_eff)
    dh = synth.to_f64(delta.cpu())
    ref = oracle.fit_anchor(dh, r)
    assert np.all(energy_margin(ref["eig"], 0.9) > TIE)
    np.testing.assert_array_equal(b.k_eff.cpu().numpy(), ref["k_eff"])
    if flat:
        assert np.all(ref["k_eff"] > r)


def test_base_cache_rank_representation():
    """The fit kernels applied to a cache itself (its rank-r representation and effective
    rank, as the listing's Fig. 2 reports for model caches): K and V of every segment."""
    base = synth.CONFIGS["llama8b_t2048"]
    cfg = base.replace(name="base_rank", L=2, H=2, T=600, seed=77)
    case = synth.generate(cfg)
    x = torch.stack([case.K0, case.V0]).reshape(2 * cfg.L * cfg.H, cfg.T, cfg.d)
    _fit_and_check("base-cache", x, cfg.r)


def test_base_cache_rank_full_size_every_matrix():
    """Flat spectra at full size: K and V of all 256 segments of the 8B cache at T = 2048 (512
    matrices, effective rank near 78, far above r = 32).  Every effective rank must equal the
    oracle's; most matrices sit within 1e-4 of the 0.9 threshold at some rank, which is where
    the fast path hands its decision to the float64 path."""
    cfg = synth.CONFIGS["llama8b_t2048"]
    say(f"[fit-base] {cfg.name}: K and V of {cfg.L * cfg.H} segments, T={cfg.T}, r={cfg.r}")
    case = synth.generate(cfg, dev())
    x = torch.stack([case.K0, case.V0]).reshape(2 * cfg.L * cfg.H, cfg.T, cfg.d)
    del case
    out = kvc.fit_anchor(x, r=cfg.r, want_eig=True)
    torch.cuda.synchronize()
    k = out.k_eff.cpu().numpy()
    xh = x.cpu()
    del x
    torch.cuda.empty_cache()
    ref_k = np.empty_like(k)
    margins = np.empty(k.shape[0])
    for i0 in range(0, k.shape[0], 64):
        ref = oracle.fit_anchor(synth.to_f64(xh[i0:i0 + 64]), cfg.r)
        ref_k[i0:i0 + 64] = ref["k_eff"]
        lam = np.clip(ref["eig"], 0, None)
        frac = np.cumsum(lam, -1) / lam.sum(-1, keepdims=True)
        kk = ref["k_eff"]
        rows = np.arange(lam.shape[0])
        margins[i0:i0 + 64] = np.minimum(0.9 - frac[rows, kk - 2], frac[rows, kk - 1] - 0.9)
    say(f"  k_eff {int(ref_k.min())}..{int(ref_k.max())}; margin at the decision: min "
        f"{margins.min():.2e}, {int((margins < 1e-4).sum())} below 1e-4, "
        f"{int((margins < 1e-6).sum())} below 1e-6")
    assert np.all(margins > TIE)
    np.testing.assert_array_equal(k, ref_k)


@pytest.mark.parametrize("side", [-1, 1])
@pytest.mark.parametrize("dtype,r", [("bf16", 32), ("f32", 8), ("bf16", 40)])
def test_effective_rank_at_a_near_tie(side, dtype, r):
    """The energy threshold placed 1e-10 (relative) above or below the oracle's cumulative
    energy fraction at rank 5: far inside the fast path's error bound, so the float64 path
    decides, and it must land on the oracle's side of the tie (rank 5 or 6)."""
    g = torch.Generator().manual_seed(55 + r)
    M, T, d = 3, 900, 128
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.empty(M, T, d, dtype=tdt)
    for m in range(M):
        P, _ = torch.linalg.qr(torch.randn(T, d, generator=g, dtype=torch.float64))
        Q, _ = torch.linalg.qr(torch.randn(d, d, generator=g, dtype=torch.float64))
        x[m] = ((P * (3.0 * 0.8 ** torch.arange(d, dtype=torch.float64))) @ Q.T).to(tdt)
    dh = synth.to_f64(x)
    lam = np.clip(oracle.fit_anchor(dh, r)["eig"], 0, None)
    frac5 = np.cumsum(lam, -1)[:, 4] / lam.sum(-1)
    for m in range(M):
        energy = float(frac5[m] * (1.0 + side * 1e-10))
        ref = oracle.fit_anchor(dh[m:m + 1], r, energy)
        want = 5 if side < 0 else 6
        assert int(ref["k_eff"][0]) == want
        out = kvc.fit_anchor(x[m:m + 1].to(dev()), r=r, energy=energy)
        G = torch.from_numpy(oracle.gram(dh[m:m + 1])).to(dev())
        fg = kvc.fit_from_gram(G, r=r, energy=energy)
        torch.cuda.synchronize()
        say(f"  [{dtype} r={r}] matrix {m}: energy {energy!r} -> oracle {want}, fit "
            f"{int(out.k_eff[0])}, from G {int(fg.k_eff[0])}")
        assert int(out.k_eff[0]) == want
        assert int(fg.k_eff[0]) == int(oracle.fit_from_gram(G.cpu().numpy(), r, energy)["k_eff"][0])
