"""GPU parity of the non-chained correction (kvc_correct_fanout) and of the error measures of
the studies (kvc_segment_error: Fig. 3's per-layer / per-agent error; kvc_rank_error_curve:
Fig. 7(b)'s error against the retained rank) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import oracle
import synth
from gpu_helpers import check_close, check_every_segment, dev, pool_all, say

pytestmark = pytest.mark.gpu


def _fanout_inputs(cfg, with_fb):
    case = synth.generate_fanout(cfg)
    q = oracle.pool(synth.to_f64(case.K0), synth.to_f64(case.V0))
    d = dev()
    ag_o, ag_g = [], []
    for j, ed in enumerate(case.edges):
        desc = synth.build_descriptors(case, j, q)
        fb = with_fb and j % 2 == 1
        ag_o.append({"desc": synth.to_f64(desc), "U": synth.to_f64(ed.U), "W": synth.to_f64(ed.W),
                     "K_fb": synth.to_f64(ed.exact_K) if fb else None,
                     "V_fb": synth.to_f64(ed.exact_V) if fb else None})
        ag_g.append({"desc": desc.to(d), "U": ed.U.to(d), "W": ed.W.to(d),
                     "K_fb": ed.exact_K.to(d) if fb else None,
                     "V_fb": ed.exact_V.to(d) if fb else None})
    return case, ag_o, ag_g


@pytest.mark.parametrize("dtype,d,T,A,r", [("bf16", 128, 600, 4, 32), ("bf16", 64, 1000, 3, 16),
                                           ("f32", 128, 300, 2, 8), ("bf16", 128, 300, 2, 128),
                                           ("f32", 128, 200, 4, 32)])
def test_fanout_matches_the_oracle(dtype, d, T, A, r):
    cfg = synth.CONFIGS["chain_t32768"].replace(L=2, H=3, T=T, d=d, dtype=dtype, A=A, r=r,
                                                seed=41, fallback_prob=0.35, outliers=2)
    say(f"[fanout] {dtype} d={d} T={T} A={A} r={r} agents={cfg.n_edges}")
    case, ag_o, ag_g = _fanout_inputs(cfg, with_fb=True)
    refs = oracle.fanout(synth.to_f64(case.K0), synth.to_f64(case.V0), ag_o, cfg.tau, cfg.dtype)
    K, V = case.K0.to(dev()), case.V0.to(dev())
    Kc, Vc = K.clone(), V.clone()
    res = kvc.correct_fanout(K, V, ag_g, cfg.tau)
    torch.cuda.synchronize()
    assert torch.equal(K, Kc) and torch.equal(V, Vc)  # the reference is read only
    n_fall = 0
    for j, (g, ref) in enumerate(zip(res, refs)):
        np.testing.assert_array_equal(g.mask.cpu().numpy(), ref["mask"], err_msg=f"agent {j}")
        n_fall += int(ref["mask"].sum())
        check_close(f"K'[{j}]", synth.to_f64(g.K), ref["K_out"])
        check_close(f"V'[{j}]", synth.to_f64(g.V), ref["V_out"])
        fin = np.isfinite(ref["score"])
        np.testing.assert_allclose(g.score.cpu().numpy()[fin], ref["score"][fin], atol=2e-6)
        # a fallback segment is the agent's fallback cache (or the reference) bit for bit
        fb_k = ag_g[j]["K_fb"] if ag_g[j]["K_fb"] is not None else K
        m = torch.from_numpy(ref["mask"].astype(bool)).to(dev())
        assert torch.equal(g.K[m], fb_k[m])
    assert n_fall > 0


@pytest.mark.parametrize("n_agents,A,r,dtype", [(4, 4, 32, "bf16"), (9, 3, 16, "bf16"),
                                                (2, 2, 8, "f32")])
def test_fanout_equals_one_correction_per_agent_bit_for_bit(n_agents, A, r, dtype):
    """Each agent's output, mask and score equal a kvc_correct call on the same inputs: every
    agent is matched from the reference's chunk sums, and the multi-target correction (up to
    8 agents per launch; 9 agents take two launches) does each agent's arithmetic exactly as
    the single-target kernel."""
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=4, H=4, T=1300, seed=42 + n_agents,
                                                 n_edges=n_agents, fallback_prob=0.3, A=A, r=r,
                                                 dtype=dtype)
    say(f"[fanout-vs-correct] L={cfg.L} H={cfg.H} T={cfg.T} agents={cfg.n_edges}")
    case, _, ag_g = _fanout_inputs(cfg, with_fb=True)
    K, V = case.K0.to(dev()), case.V0.to(dev())
    res = kvc.correct_fanout(K, V, ag_g, cfg.tau)
    one = [kvc.correct(K, V, a["desc"], a["U"], a["W"], cfg.tau, K_fb=a["K_fb"], V_fb=a["V_fb"])
           for a in ag_g]
    torch.cuda.synchronize()
    for j, (a, b) in enumerate(zip(res, one)):
        assert torch.equal(a.mask, b.mask), f"agent {j} mask"
        assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V), f"agent {j} outputs"
        assert torch.equal(a.score, b.score), f"agent {j} score"


def test_fanout_full_size_every_segment():
    """Three agents on the 8B shape at T = 2048 (the launch configuration of the benchmark's
    non-chained leg at a shorter context): every mask, and every segment of every agent's
    output against the oracle."""
    cfg = synth.CONFIGS["llama8b_t2048"].replace(n_edges=3, seed=43)
    say(f"[fanout-full] L={cfg.L} H={cfg.H} T={cfg.T} agents={cfg.n_edges}")
    d = dev()
    case = synth.generate_fanout(cfg, d)
    q = pool_all(case.K0, case.V0)
    ag = [{"desc": synth.build_descriptors(case, j, q), "U": ed.U, "W": ed.W,
           "K_fb": ed.exact_K, "V_fb": ed.exact_V} for j, ed in enumerate(case.edges)]
    res = kvc.correct_fanout(case.K0, case.V0, ag, cfg.tau)
    torch.cuda.synchronize()
    for j, g in enumerate(res):
        s = oracle.cosine_scores(q, synth.to_f64(ag[j]["desc"]))
        _, m = oracle.reliability(s, cfg.tau)
        np.testing.assert_array_equal(g.mask.cpu().numpy(), m, err_msg=f"agent {j}")
        a = ag[j]
        check_every_segment(f"agent {j}", g.K, g.V, lambda l, a=a: oracle.correct(
            synth.to_f64(case.K0[l:l + 1]), synth.to_f64(case.V0[l:l + 1]),
            synth.to_f64(a["desc"][l:l + 1]), synth.to_f64(a["U"][:, l:l + 1]),
            synth.to_f64(a["W"][:, l:l + 1]), cfg.tau, cfg.dtype,
            K_fb=synth.to_f64(a["K_fb"][l:l + 1]), V_fb=synth.to_f64(a["V_fb"][l:l + 1])),
            cfg.L, m)


@pytest.mark.parametrize("dtype,d,T", [("bf16", 128, 300), ("bf16", 64, 257), ("f32", 128, 511),
                                       ("f32", 64, 1), ("bf16", 128, 0)])
def test_segment_error_matches_the_oracle(dtype, d, T):
    say(f"[segment-error] {dtype} d={d} T={T}")
    g = torch.Generator().manual_seed(T + d)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    L, H = 3, 5
    ref = torch.randn(L, H, T, d, generator=g).to(tdt)
    X = (ref.float() + 0.1 * torch.randn(L, H, T, d, generator=g)).to(tdt)
    X[1, 2] = ref[1, 2]  # an exact segment
    if T > 0:
        X[2, 4, 0, 0] = 1e30 if dtype == "f32" else 3e38  # a large entry stays finite in float64
    out = kvc.segment_error(X.to(dev()), ref.to(dev()))
    torch.cuda.synchronize()
    e, r = oracle.segment_error(synth.to_f64(X), synth.to_f64(ref))
    got = out.cpu().numpy()
    np.testing.assert_allclose(got[..., 0], e, rtol=1e-12, atol=0)
    np.testing.assert_allclose(got[..., 1], r, rtol=1e-12, atol=0)
    assert got[1, 2, 0] == 0.0


def test_segment_error_full_size_per_layer_and_agent():
    """The 8B shape at T = 2048: per-segment sums against the oracle, then Fig. 3's per-layer
    and whole-cache errors assembled from them."""
    cfg = synth.CONFIGS["llama8b_t2048"]
    say(f"[segment-error-full] L={cfg.L} H={cfg.H} T={cfg.T}")
    case = synth.generate(cfg, dev())
    ed = case.edges[0]
    out = kvc.segment_error(case.K0, ed.exact_K)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    e = np.empty((cfg.L, cfg.H))
    r = np.empty((cfg.L, cfg.H))
    for l in range(cfg.L):
        e[l], r[l] = oracle.segment_error(synth.to_f64(case.K0[l]), synth.to_f64(ed.exact_K[l]))
    np.testing.assert_allclose(got[..., 0], e, rtol=1e-12)
    np.testing.assert_allclose(got[..., 1], r, rtol=1e-12)
    np.testing.assert_allclose(oracle.layer_error(got[..., 0], got[..., 1]),
                               oracle.layer_error(e, r), rtol=1e-12)
    whole = oracle.rel_frobenius(synth.to_f64(case.K0), synth.to_f64(ed.exact_K))
    assert abs(np.sqrt(got[..., 0].sum() / got[..., 1].sum()) - whole) <= 1e-12 * whole


def test_rank_error_curve_matches_the_oracle():
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=2, H=4, T=700, seed=44)
    say(f"[rank-error-curve] M={2 * cfg.L * cfg.H} T={cfg.T}")
    case = synth.generate(cfg)
    delta = synth.fit_input(case)
    fit = kvc.fit_anchor(delta.to(dev()), r=cfg.r)
    curve = kvc.rank_error_curve(fit.eig)
    # a zero spectrum, an unsorted-free descending one with negative round-off, one entry
    extra = torch.tensor([[0.0] * 4, [9.0, 4.0, 1.0, -1e-7]], device=dev())
    c2 = kvc.rank_error_curve(extra)
    one = kvc.rank_error_curve(torch.tensor([[2.5]], device=dev()))
    torch.cuda.synchronize()
    eig = fit.eig.cpu().numpy().astype(np.float64)
    # same eigenvalues in: the curve within float32 output rounding
    np.testing.assert_allclose(curve.cpu().numpy(), oracle.rank_error_curve(eig), rtol=2e-7,
                               atol=1e-7)
    np.testing.assert_allclose(c2.cpu().numpy(), oracle.rank_error_curve(
        extra.cpu().numpy().astype(np.float64)), rtol=2e-7, atol=0)
    np.testing.assert_array_equal(one.cpu().numpy(), [[1.0, 0.0]])
    # against the oracle's own SVD of delta: the fit's eigenvalue bar (each within 2e-5 of the
    # largest) bounds the squared curve's error by d * 2e-5 * lambda_0 / total
    ref = oracle.fit_anchor(synth.to_f64(delta), cfg.r)
    want = oracle.rank_error_curve(ref["eig"])
    lam = ref["eig"]
    bound = cfg.d * 2e-5 * lam[:, :1] / lam.sum(-1, keepdims=True) + 1e-7
    c = curve.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(c ** 2 - want ** 2) <= bound)
    say(f"  curve at k = 1, 8, 11, 32: {np.round(c[0, [1, 8, 11, 32]], 5).tolist()}")
