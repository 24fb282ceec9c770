"""GPU parity of the matching on rank-r_C cache representations (kvc_rank_descriptor,
kvc_correct_rank) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import oracle
import synth
from gpu_helpers import check_close, dev, say

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-4  # |score - tau| below this: float32 (kernel) and float64 (oracle) may differ


def _gram_of(F):
    """Truncated second-moment matrices F^T F of factors [..., rC, d] (sign- and rotation-free)."""
    F = np.asarray(F, dtype=np.float64)
    return np.einsum("...ki,...kj->...ij", F, F)


@pytest.mark.parametrize("dtype,d,T,rC", [("bf16", 128, 300, 32), ("bf16", 64, 500, 8),
                                          ("f32", 128, 200, 16), ("bf16", 128, 260, 48)])
def test_rank_descriptor_matches_the_oracle(dtype, d, T, rC):
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=2, H=3, T=T, d=d, dtype=dtype, seed=90 + rC)
    say(f"[rank-desc] {dtype} d={d} T={T} rC={rC}")
    case = synth.generate(cfg)
    F, k = kvc.rank_descriptor(case.K0.to(dev()), case.V0.to(dev()), rC)
    torch.cuda.synchronize()
    ref = oracle.rank_descriptor(synth.to_f64(case.K0), synth.to_f64(case.V0), rC)
    np.testing.assert_array_equal(k.cpu().numpy(), ref["k_eff"])
    Fg = F.cpu().double().numpy()
    check_close("F^T F", _gram_of(Fg), _gram_of(ref["F"]))
    # rows: sqrt(lambda_i) v_i with orthogonal directions (F F^T diagonal, descending)
    FF = np.einsum("...id,...jd->...ij", Fg, Fg)
    diag = np.diagonal(FF, axis1=-2, axis2=-1)
    off = FF - np.einsum("...i,ij->...ij", diag, np.eye(rC))
    assert np.max(np.abs(off)) <= 1e-4 * np.max(diag)
    np.testing.assert_allclose(diag, np.diagonal(np.einsum("...id,...jd->...ij", ref["F"], ref["F"]),
                                                 axis1=-2, axis2=-1), rtol=1e-3, atol=1e-6 * diag.max())


def _anchor_factors(Fq, A, rng):
    """Anchor representations near the query's: Fq plus a Gaussian of relative size
    base * 2^a, with a per-segment base drawn log-uniformly from [0.1, 3] (so the segments'
    best scores spread over a wide range)."""
    Fa = np.empty(Fq.shape[:3] + (A,) + Fq.shape[3:])
    base = np.exp(rng.uniform(np.log(0.1), np.log(3.0), size=Fq.shape[1:3]))
    scale = np.sqrt(np.mean(Fq ** 2, axis=(-1, -2), keepdims=True))
    for a in range(A):
        eps = (base * 2.0 ** a)[None, :, :, None, None]
        Fa[:, :, :, a] = Fq + eps * scale * rng.standard_normal(Fq.shape)
    return Fa.astype(np.float32).astype(np.float64)


def _pick_tau(best):
    """A threshold in the widest gap between the segments' best scores (middle of the range)."""
    b = np.sort(best.ravel())
    lo, hi = len(b) // 5, len(b) - len(b) // 5
    gaps = b[lo + 1:hi] - b[lo:hi - 1]
    i = int(np.argmax(gaps)) + lo
    return float(0.5 * (b[i] + b[i + 1]))


@pytest.mark.parametrize("dtype,d,T,A,r,rC", [("bf16", 128, 400, 4, 32, 32),
                                              ("f32", 64, 300, 3, 8, 8),
                                              ("bf16", 128, 250, 2, 128, 16),
                                              ("bf16", 128, 300, 2, 32, 100),  # 4 x 4 tiles, ragged
                                              ("f32", 64, 200, 5, 16, 40)])    # 2 x 2 tiles, ragged
def test_correct_rank_matches_the_oracle(dtype, d, T, A, r, rC):
    """The same query representation (the oracle's, in float32) handed to both sides: masks
    exact, scores and weights to float32 accuracy, caches within the bars."""
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=3, H=4, T=T, d=d, dtype=dtype, A=A, r=r,
                                                 seed=120 + A + rC)
    say(f"[rank-correct] {dtype} d={d} T={T} A={A} r={r} rC={rC}")
    case = synth.generate(cfg)
    rng = np.random.default_rng(7 + rC)
    K, V = synth.to_f64(case.K0), synth.to_f64(case.V0)
    Fq = oracle.rank_descriptor(K, V, rC)["F"].astype(np.float32).astype(np.float64)
    Fa = _anchor_factors(Fq, A, rng)
    s = oracle.rank_scores(Fq, Fa)
    tau = _pick_tau(s.max(-1))
    ed = case.edges[0]
    ref = oracle.correct_rank(K, V, Fq, Fa, synth.to_f64(ed.U), synth.to_f64(ed.W), tau, cfg.dtype,
                              K_fb=synth.to_f64(ed.exact_K), V_fb=synth.to_f64(ed.exact_V))
    g = dev()
    t32 = lambda x: torch.from_numpy(x.astype(np.float32)).to(g)  # noqa: E731
    res = kvc.correct_rank(case.K0.to(g), case.V0.to(g), t32(Fq), t32(Fa), ed.U.to(g), ed.W.to(g),
                           tau, K_fb=ed.exact_K.to(g), V_fb=ed.exact_V.to(g))
    torch.cuda.synchronize()
    margin = np.abs(ref["score"] - tau)
    say(f"  tau {tau:.4f}, min |score - tau| {margin.min():.2e}, fallback {int(ref['mask'].sum())}")
    assert margin.min() > NEAR_TIE
    np.testing.assert_array_equal(res.mask.cpu().numpy(), ref["mask"])
    np.testing.assert_allclose(res.score.cpu().numpy(), ref["score"], atol=1e-5)
    np.testing.assert_allclose(res.w.cpu().numpy(), ref["w"], rtol=1e-4, atol=1e-6)
    check_close("K'", synth.to_f64(res.K), ref["K_out"])
    check_close("V'", synth.to_f64(res.V), ref["V_out"])
    assert 0 < int(ref["mask"].sum()) < ref["mask"].size


def test_rank_matching_full_size_8b():
    """The 8B shape (32 x 8 segments, T = 2048, r_C = 32): the library's own representation of
    the cache, then the rank-matched correction; every mask against the oracle's decision from
    the oracle's representation, caches on sampled segments."""
    cfg = synth.CONFIGS["llama8b_t2048"]
    rC = 32
    say(f"[rank-full] {cfg.name} rC={rC}")
    g = dev()
    case = synth.generate(cfg, g)
    F, k = kvc.rank_descriptor(case.K0, case.V0, rC)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    # the oracle's representation of every segment (float64 SVD), layer by layer
    Fq = np.empty((2, cfg.L, cfg.H, rC, cfg.d))
    kref = np.empty((2, cfg.L, cfg.H), dtype=np.int32)
    for l in range(cfg.L):
        o = oracle.rank_descriptor(synth.to_f64(case.K0[l:l + 1]), synth.to_f64(case.V0[l:l + 1]), rC)
        Fq[:, l] = o["F"][:, 0]
        kref[:, l] = o["k_eff"][:, 0]
    np.testing.assert_array_equal(k.cpu().numpy(), kref)
    check_close("F^T F (all segments)", _gram_of(F.cpu().double().numpy()), _gram_of(Fq))
    Fa = _anchor_factors(Fq, cfg.A, rng)
    s = oracle.rank_scores(Fq, Fa)
    tau = _pick_tau(s.max(-1))
    ed = case.edges[0]
    res = kvc.correct_rank(case.K0, case.V0, F, torch.from_numpy(Fa.astype(np.float32)).to(g),
                           ed.U, ed.W, tau, K_fb=ed.exact_K, V_fb=ed.exact_V)
    torch.cuda.synchronize()
    score = s.max(-1)
    m_ref = (~(score >= tau)).astype(np.uint8)
    margin = np.abs(score - tau)
    tie = margin < NEAR_TIE
    say(f"  tau {tau:.4f}, min |score - tau| {margin.min():.2e}, {int(tie.sum())} near-tie(s), "
        f"fallback {int(m_ref.sum())} of {m_ref.size}")
    got = res.mask.cpu().numpy()
    np.testing.assert_array_equal(got[~tie], m_ref[~tie])
    np.testing.assert_allclose(res.score.cpu().numpy(), score, atol=2e-5)
    allsegs = [(l, h) for l in range(cfg.L) for h in range(cfg.H)]
    pick = [allsegs[i] for i in rng.choice(len(allsegs), size=12, replace=False)]
    for l, h in pick:
        if tie[l, h]:
            continue
        sub = oracle.correct_rank(synth.to_f64(case.K0[l, h])[None, None],
                                  synth.to_f64(case.V0[l, h])[None, None],
                                  Fq[:, l, h][:, None, None], Fa[:, l, h][:, None, None],
                                  synth.to_f64(ed.U[:, l, h])[:, None, None],
                                  synth.to_f64(ed.W[:, l, h])[:, None, None], tau, cfg.dtype,
                                  K_fb=synth.to_f64(ed.exact_K[l, h])[None, None],
                                  V_fb=synth.to_f64(ed.exact_V[l, h])[None, None])
        check_close(f"K'({l},{h})", synth.to_f64(res.K[l, h]), sub["K_out"][0, 0])
        check_close(f"V'({l},{h})", synth.to_f64(res.V[l, h]), sub["V_out"][0, 0])
