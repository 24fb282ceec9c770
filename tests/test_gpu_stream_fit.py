"""GPU parity of the streaming fit (kvc_gram_accumulate, kvc_fit_from_gram, kvc_project)
against the fp64 oracle and against the one-call fit, through the C ABI."""
import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import oracle
import synth
from gpu_helpers import check_fit, dev, energy_margin, say

pytestmark = pytest.mark.gpu


def _planted_delta(M, T, d, dtype, seed, decay=0.85):
    g = torch.Generator().manual_seed(seed)
    k = min(T, d)
    out = torch.empty(M, T, d, dtype=torch.float64)
    for m in range(M):
        P, _ = torch.linalg.qr(torch.randn(T, k, generator=g, dtype=torch.float64))
        Q, _ = torch.linalg.qr(torch.randn(d, k, generator=g, dtype=torch.float64))
        s = 5.0 * decay ** torch.arange(k, dtype=torch.float64)
        out[m] = (P * s) @ Q.T + 1e-3 * torch.randn(T, d, generator=g, dtype=torch.float64)
    return out.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


@pytest.mark.parametrize("dtype,d,T,r,M", [
    ("bf16", 128, 700, 32, 4),
    ("f32", 64, 300, 8, 3),
    ("bf16", 64, 1000, 16, 2),
])
def test_one_block_from_zero_equals_the_one_call_fit(dtype, d, T, r, M):
    """G accumulated once onto zero is the G of kvc_fit_anchor, so W, k_eff, the eigenvalues
    and U = delta W^T agree bit for bit."""
    say(f"[stream] one block {dtype} d={d} T={T} r={r} M={M}")
    delta = _planted_delta(M, T, d, dtype, 10 + T).to(dev())
    G = kvc.gram_accumulate(delta)
    a = kvc.fit_from_gram(G, r=r)
    U = kvc.project(delta, a.W)
    b = kvc.fit_anchor(delta, r=r)
    torch.cuda.synchronize()
    assert torch.equal(a.W, b.W) and torch.equal(a.k_eff, b.k_eff) and torch.equal(a.eig, b.eig)
    assert torch.equal(U, b.U)


def test_gram_matches_the_oracle():
    delta = _planted_delta(3, 900, 128, "bf16", 7).to(dev())
    G = kvc.gram_accumulate(delta)
    G = kvc.gram_accumulate(delta[:, :5].contiguous(), G)  # a second block
    torch.cuda.synchronize()
    dh = synth.to_f64(delta.cpu())
    ref = oracle.gram(dh) + oracle.gram(dh[:, :5])
    got = G.cpu().numpy()
    np.testing.assert_array_equal(got, np.swapaxes(got, 1, 2))
    assert oracle.rel_frobenius(got, ref) < 1e-6


@pytest.mark.parametrize("dtype,d,T,M", [
    ("bf16", 128, 40000, 1),  # 313 splits of 128 rows
    ("f32", 64, 20000, 2),    # 79 splits of 256 rows
])
def test_gram_fold_over_many_splits(dtype, d, T, M):
    """Few matrices and many rows: the fold sums hundreds of split partials per element.
    Onto zero it equals the one-call fit's G (same W, k_eff and eigenvalues, bit for bit);
    onto a non-zero G it matches the oracle's float64 sum and stays symmetric."""
    say(f"[stream] many splits {dtype} d={d} T={T} M={M}")
    delta = _planted_delta(M, T, d, dtype, 17 + M).to(dev())
    G = kvc.gram_accumulate(delta)
    a = kvc.fit_from_gram(G, r=16)
    b = kvc.fit_anchor(delta, r=16)
    torch.cuda.synchronize()
    assert torch.equal(a.W, b.W) and torch.equal(a.k_eff, b.k_eff) and torch.equal(a.eig, b.eig)
    head = delta[:, : T // 3].contiguous()
    G2 = kvc.gram_accumulate(delta[:, T // 3:].contiguous(), kvc.gram_accumulate(head))
    torch.cuda.synchronize()
    dh = synth.to_f64(delta.cpu())
    ref = oracle.gram(dh)
    trace = np.trace(ref, axis1=1, axis2=2)
    bar = gram_gamma(dtype, 256)  # |E|_F <= gamma trace (splits of at most 256 rows)
    for name, got in (("one block", G.cpu().numpy()), ("two blocks", G2.cpu().numpy())):
        np.testing.assert_array_equal(got, np.swapaxes(got, 1, 2))
        e = np.linalg.norm(got - ref, axis=(1, 2)) / trace
        say(f"  {name}: |G - G_oracle|_F / trace worst {e.max():.3e} (bar {bar:.1e}), "
            f"rel-Frobenius {oracle.rel_frobenius(got, ref):.3e}")
        assert np.all(e <= bar)


@pytest.mark.parametrize("dtype,d,T,r,M", [
    ("bf16", 128, 1, 1, 2),
    ("bf16", 128, 700, 33, 3),
    ("bf16", 64, 37, 5, 4),
    ("bf16", 128, 513, 100, 2),
    ("f32", 128, 260, 64, 2),
    ("f32", 64, 129, 17, 3),
])
def test_projection_matches_the_oracle(dtype, d, T, r, M):
    """U = delta W^T for any float32 W (not only orthonormal rows), any r <= d and ragged T:
    the bf16 path splits W into bf16 halves in the kernel (rows >= r read as zero)."""
    say(f"[stream] projection {dtype} d={d} T={T} r={r} M={M}")
    g = torch.Generator().manual_seed(1000 + T + r)
    delta = torch.randn(M, T, d, generator=g, dtype=torch.float64)
    W = torch.randn(M, r, d, generator=g, dtype=torch.float64).float()
    delta = delta.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    U = kvc.project(delta.to(dev()), W.to(dev()))
    torch.cuda.synchronize()
    want = oracle.project(synth.to_f64(delta), W.double().numpy())
    got = U.cpu().double().numpy()
    e = oracle.rel_frobenius(got, want)
    mx = np.abs(got - want).max() / np.abs(want).max()
    say(f"  U rel-Frobenius {e:.3e}, max |diff| / max |U| {mx:.3e} (bar 1e-4)")
    assert e <= 1e-4 and mx <= 1e-4


def gram_gamma(dtype, rows):
    """Error bound of an accumulated Gram per unit of trace for blocks of at most `rows` rows:
    (steps + 2) float32 roundings of a split's sum, doubled (steps: rows / 16 MFMA steps for
    bf16, one rounded product per row for fp32)."""
    steps = rows / 16.0 if dtype == "bf16" else float(rows)
    return 2.0 * (steps + 2.0) * 2.0 ** -24


def test_fit_from_gram_is_exact_for_the_given_gram():
    """G computed on the host (float64 delta^T delta) and handed to the library: k_eff must equal
    the oracle's symmetric eigen-decomposition of the same G on every matrix, flat spectra
    included (the fast path passes close decisions to the float64 path)."""
    g = torch.Generator().manual_seed(808)
    M, T, d = 16, 400, 128
    dh = torch.randn(M, T, d, generator=g, dtype=torch.float64).numpy()
    dh[: M // 2] *= np.linspace(0.2, 3.0, d)  # half of them with a sloped spectrum
    G = oracle.gram(dh)
    for r in (32, 48):
        fit = kvc.fit_from_gram(torch.from_numpy(G).to(dev()), r=r)
        torch.cuda.synchronize()
        ref = oracle.fit_from_gram(G, r)
        margin = energy_margin(ref["eig"], 0.9)
        say(f"  r={r}: min energy margin {margin.min():.2e}, {int((margin < 1e-4).sum())} below 1e-4")
        assert np.all(margin > 1e-11)
        np.testing.assert_array_equal(fit.k_eff.cpu().numpy(), ref["k_eff"])


@pytest.mark.parametrize("dtype,d,blocks,r,M", [
    ("bf16", 128, (300, 1, 517, 64), 32, 3),
    ("f32", 128, (100, 400), 40, 2),      # r > 32: the Jacobi route
    ("bf16", 64, (16, 16, 600), 8, 2),
])
def test_streamed_blocks_match_the_oracle(dtype, d, blocks, r, M):
    """Rows appended block by block: the refit from the accumulated G is the fit of all rows,
    and U of the last block alone is its projection on the new W."""
    say(f"[stream] blocks {blocks} {dtype} d={d} r={r} M={M}")
    T = sum(blocks)
    delta = _planted_delta(M, T, d, dtype, 100 + T + r)
    dd = delta.to(dev())
    G = None
    t0 = 0
    for b in blocks:
        G = kvc.gram_accumulate(dd[:, t0:t0 + b].contiguous(), G)
        t0 += b
    fit = kvc.fit_from_gram(G, r=r)
    U_all = kvc.project(dd, fit.W)
    last = dd[:, T - blocks[-1]:].contiguous()
    U_last = kvc.project(last, fit.W)
    torch.cuda.synchronize()
    dh = synth.to_f64(delta)
    ref = oracle.fit_anchor(dh, r)
    # k_eff from G is exact for the G it is given; the accumulated G differs from delta^T delta
    # by at most gamma * trace in Frobenius norm, which moves the energy fraction at rank k by
    # at most (sqrt(k) + 1) * gamma
    band = (np.sqrt(d) + 1.0) * gram_gamma(dtype, max(blocks))
    margin = energy_margin(ref["eig"], 0.9)
    say(f"  min energy margin {margin.min():.2e} (band {band:.1e})")
    ok = margin > band
    assert ok.all()
    sel = np.nonzero(ok)[0]
    sub = {k: v[sel] for k, v in ref.items()}
    check_fit(f"stream-{dtype}-{d}-{r}", U_all.cpu().double().numpy()[sel],
              fit.W.cpu().double().numpy()[sel], fit.k_eff.cpu().numpy()[sel],
              fit.eig.cpu().double().numpy()[sel], sub, r, dh[sel])
    # the last block's U is its own projection (same kernel, rows independent)
    np.testing.assert_array_equal(U_last.cpu().numpy(), U_all[:, T - blocks[-1]:].cpu().numpy())
    want = oracle.project(synth.to_f64(last.cpu()), fit.W.cpu().double().numpy())
    assert oracle.rel_frobenius(U_last.cpu().double().numpy(), want) < 1e-5


def test_llama8b_t8192_streamed_in_four_blocks():
    """The 8B delta at T = 8192 appended in four blocks of 2048 rows: the refit from the
    accumulated G against the oracle's SVD of all rows (k_eff on every matrix, U = delta W^T,
    W and eigenvalues on a sample of 32 matrices), and the same rank-32 subspace as the
    one-call fit on every matrix."""
    cfg = synth.CONFIGS["llama8b_t8192_fit"]
    say(f"[stream] {cfg.name} in 4 blocks of {cfg.T // 4}")
    case = synth.generate(cfg, dev())
    delta = synth.fit_input(case)
    del case
    torch.cuda.empty_cache()
    M, T, d = delta.shape
    ws = torch.empty(kvc.lib().kvc_gram_workspace_bytes(M, T // 4, d), dtype=torch.uint8,
                     device=dev())
    G = None
    for i in range(4):
        G = kvc.gram_accumulate(delta[:, i * T // 4:(i + 1) * T // 4].contiguous(), G,
                                workspace=ws)
    fit = kvc.fit_from_gram(G, r=cfg.r)
    U = kvc.project(delta, fit.W)
    one = kvc.fit_anchor(delta, r=cfg.r, want_eig=False)
    torch.cuda.synchronize()
    assert torch.all(fit.k_eff == 11)
    # the same rank-32 subspace as the one-call fit: W W^T agree
    P1 = fit.W.double().transpose(1, 2) @ fit.W.double()
    P2 = one.W.double().transpose(1, 2) @ one.W.double()
    err = ((P1 - P2).norm(dim=(1, 2)) / P2.norm(dim=(1, 2))).max().item()
    say(f"  W^T W against the one-call fit: max relative difference {err:.2e}")
    assert err < 1e-3, err
    rng = np.random.default_rng(5)
    idx = sorted(set([0, M - 1] + rng.choice(M, 30, replace=False).tolist()))
    dh = synth.to_f64(delta[idx])
    ref = oracle.fit_anchor(dh, cfg.r)
    check_fit(f"stream-{cfg.name}", U[idx].cpu().double().numpy(),
              fit.W[idx].cpu().double().numpy(), fit.k_eff[idx].cpu().numpy(),
              fit.eig[idx].cpu().double().numpy(), ref, cfg.r, dh)
    say(f"  {len(idx)} sampled matrices match the oracle's SVD of all rows")
