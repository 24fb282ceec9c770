"""GPU parity of the warm-started refit (kvc_refit_warm) against the fp64 oracle's
eigen-decomposition of the same G, through the C ABI: the effective rank exact on every
matrix, W within the bars where the eigenvalue gaps determine it, the matrices the warm path
leaves open solved by the full path (bit for bit the kvc_fit_from_gram result)."""
import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import oracle
import synth
from gpu_helpers import REL_FROB, dev, energy_margin, say
from test_gpu_stream_fit import _planted_delta

pytestmark = pytest.mark.gpu


def _check_against_oracle(name, G, W, k, r, energy=0.9):
    """k_eff on every matrix; W where the top-r gaps are resolved; the rank-r projector where
    only the subspace is unique."""
    Gh = G.cpu().numpy()
    ref = oracle.fit_from_gram(Gh, r, energy)
    got_k = k.cpu().numpy()
    margin = energy_margin(ref["eig"], energy)
    say(f"  {name}: min energy margin {margin.min():.2e}")
    assert np.all(margin > 1e-11)
    np.testing.assert_array_equal(got_k, ref["k_eff"], err_msg=f"{name}: effective rank")
    Wg = W.cpu().double().numpy()
    worst_w = worst_p = 0.0
    n_w = n_p = 0
    for m in range(Gh.shape[0]):
        lam = ref["eig"][m]
        l0 = lam[0]
        if l0 <= 0:
            continue
        if r < lam.shape[0] and lam[r - 1] - lam[r] <= 1e-3 * l0:
            continue
        P_g = Wg[m].T @ Wg[m]
        P_o = ref["W"][m].T @ ref["W"][m]
        e = oracle.rel_frobenius(P_g, P_o)
        worst_p = max(worst_p, e)
        n_p += 1
        assert e <= REL_FROB, f"{name}[{m}]: projector error {e:.3e}"
        gaps = -np.diff(lam[: min(r + 1, lam.shape[0])])
        if np.all(gaps > 1e-4 * l0) and lam[r - 1] > 1e-4 * l0:
            e = oracle.rel_frobenius(Wg[m], ref["W"][m])
            worst_w = max(worst_w, e)
            n_w += 1
            assert e <= REL_FROB, f"{name}[{m}]: W relative error {e:.3e}"
    say(f"  {name}: W rel-Frobenius worst {worst_w:.3e} over {n_w} matrices, projector worst "
        f"{worst_p:.3e} over {n_p} (bar {REL_FROB:.0e})")


@pytest.mark.parametrize("dtype,d,t_old,t_new,r,M", [
    ("bf16", 128, 1500, 500, 32, 6),
    ("bf16", 128, 900, 60, 16, 4),
    ("f32", 64, 400, 200, 8, 4),
    ("bf16", 64, 700, 300, 32, 3),
    ("f32", 128, 600, 50, 5, 3),
])
def test_refit_after_appended_rows_matches_the_oracle(dtype, d, t_old, t_new, r, M):
    say(f"[warm] {dtype} d={d} {t_old}+{t_new} rows r={r} M={M}")
    delta = _planted_delta(M, t_old + t_new, d, dtype, 31 + d + r + t_new).to(dev())
    G = kvc.gram_accumulate(delta[:, :t_old].contiguous())
    W_old = kvc.fit_from_gram(G, r=r, want_eig=False).W
    G = kvc.gram_accumulate(delta[:, t_old:].contiguous(), G)
    fit, warm = kvc.refit_warm(G, W_old)
    torch.cuda.synchronize()
    say(f"  warm kept on {int(warm.sum())} of {M}")
    _check_against_oracle(f"warm-{dtype}-{d}-{r}", G, fit.W, fit.k_eff, r)
    # the same G through the full path: the same effective ranks
    full = kvc.fit_from_gram(G, r=r, want_eig=False)
    torch.cuda.synchronize()
    assert torch.equal(full.k_eff, fit.k_eff)


def test_llama8b_t8192_appended_block_every_matrix():
    """The 8B delta at T = 8192: the anchor of the first 6144 rows refit after the last 2048
    rows are appended (M = 512).  k_eff on every matrix and W on every matrix whose gaps
    resolve it, against the oracle; the warm result is kept on (nearly) every matrix."""
    cfg = synth.CONFIGS["llama8b_t8192_fit"]
    say(f"[warm] {cfg.name}: 6144 + 2048 rows")
    case = synth.generate(cfg, dev())
    delta = synth.fit_input(case)
    del case
    torch.cuda.empty_cache()
    M, T, d = delta.shape
    G = kvc.gram_accumulate(delta[:, :6144].contiguous())
    W_old = kvc.fit_from_gram(G, r=cfg.r, want_eig=False).W
    G = kvc.gram_accumulate(delta[:, 6144:].contiguous(), G)
    fit, warm = kvc.refit_warm(G, W_old)
    torch.cuda.synchronize()
    kept = int(warm.sum())
    say(f"  warm kept on {kept} of {M}")
    _check_against_oracle("warm-llama8b", G, fit.W, fit.k_eff, cfg.r)
    assert kept >= 0.9 * M
    del delta, G


def _sweep_cases(n):
    """Seeded random configurations: dtype, d, rows before and after the append, r, energy,
    spectral decay of the planted delta."""
    rng = np.random.default_rng(2026)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        out.append(("bf16" if rng.random() < 0.6 else "f32", d, int(rng.integers(200, 1500)),
                    int(rng.integers(20, 600)), int(rng.integers(1, 33)),
                    float(rng.choice([0.5, 0.8, 0.9, 0.99])), float(rng.choice([0.8, 0.9, 0.95])),
                    100 + i))
    return out


@pytest.mark.parametrize("dtype,d,t_old,t_new,r,energy,decay,seed", _sweep_cases(12))
def test_random_configurations_match_the_oracle(dtype, d, t_old, t_new, r, energy, decay, seed):
    """A seeded sweep over shapes, ranks, energies and spectra: k_eff exact on every matrix
    (the warm certificate or the full path, whichever decided it), W within the bars, and the
    matrices the warm path left open equal to the full path bit for bit."""
    M = 4
    say(f"[warm] sweep {dtype} d={d} {t_old}+{t_new} rows r={r} energy={energy} decay={decay}")
    delta = _planted_delta(M, t_old + t_new, d, dtype, seed, decay).to(dev())
    G = kvc.gram_accumulate(delta[:, :t_old].contiguous())
    W_old = kvc.fit_from_gram(G, r=r, energy=energy, want_eig=False).W
    G = kvc.gram_accumulate(delta[:, t_old:].contiguous(), G)
    fit, warm = kvc.refit_warm(G, W_old, energy)
    full = kvc.fit_from_gram(G, r=r, energy=energy, want_eig=False)
    torch.cuda.synchronize()
    w = warm.cpu().numpy()
    say(f"  warm kept on {int(w.sum())} of {M}")
    _check_against_oracle(f"sweep-{seed}", G, fit.W, fit.k_eff, r, energy)
    assert torch.equal(full.k_eff, fit.k_eff)
    for m in range(M):
        if w[m] == 0:
            assert torch.equal(fit.W[m], full.W[m]), f"sweep-{seed}[{m}]: W differs from the full path"


def _flat_gram(M, T, d, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, T, d, generator=g, dtype=torch.float64)
    return torch.einsum("mtd,mte->mde", x, x)


@pytest.mark.parametrize("case", ["zero", "flat", "random_start", "r_above_32"])
def test_matrices_left_open_take_the_full_path(case):
    """Cases the warm path must leave to the full solve (or may not finish itself): the
    outputs equal the kvc_fit_from_gram ones bit for bit where the full path ran, and the
    oracle's effective rank everywhere."""
    say(f"[warm] open case {case}")
    M, d, r = 4, 128, 32
    if case == "zero":
        G = torch.zeros(M, d, d, dtype=torch.float64)
    elif case == "flat":
        G = _flat_gram(M, 3000, d, 5)
    elif case == "random_start":
        delta = _planted_delta(M, 2000, d, "f32", 77).double()
        G = torch.einsum("mtd,mte->mde", delta, delta)
    else:
        r = 40
        delta = _planted_delta(M, 2000, d, "f32", 78).double()
        G = torch.einsum("mtd,mte->mde", delta, delta)
    G = G.to(dev())
    gen = torch.Generator().manual_seed(9)
    W_prev = torch.linalg.qr(torch.randn(M, d, r, generator=gen, dtype=torch.float64))[0]
    W_prev = W_prev.transpose(1, 2).contiguous().float().to(dev())
    fit, warm = kvc.refit_warm(G, W_prev)
    full = kvc.fit_from_gram(G, r=r, want_eig=False)
    torch.cuda.synchronize()
    w = warm.cpu().numpy()
    say(f"  warm kept on {int(w.sum())} of {M}")
    if case in ("zero", "flat", "r_above_32"):
        assert w.sum() == 0
    for m in range(M):
        if w[m] == 0:
            assert torch.equal(fit.W[m], full.W[m]), f"{case}[{m}]: W differs from the full path"
    np.testing.assert_array_equal(fit.k_eff.cpu().numpy(), full.k_eff.cpu().numpy())
    _check_against_oracle(f"open-{case}", G, fit.W, fit.k_eff, r)


def test_in_place_and_repeatable():
    """W_out may be W_prev itself; two calls give the same bits."""
    M, d, r = 8, 128, 32
    delta = _planted_delta(M, 1200, d, "bf16", 91).to(dev())
    G = kvc.gram_accumulate(delta[:, :1000].contiguous())
    W = kvc.fit_from_gram(G, r=r, want_eig=False).W
    G = kvc.gram_accumulate(delta[:, 1000:].contiguous(), G)
    a, wa = kvc.refit_warm(G, W)
    b, wb = kvc.refit_warm(G, W)
    W2 = W.clone()
    c, wc = kvc.refit_warm(G, W2, W_out=W2)
    torch.cuda.synchronize()
    assert torch.equal(a.W, b.W) and torch.equal(a.k_eff, b.k_eff) and torch.equal(wa, wb)
    assert torch.equal(c.W, a.W) and torch.equal(c.k_eff, a.k_eff) and torch.equal(wc, wa)
    assert c.W.data_ptr() == W2.data_ptr()
