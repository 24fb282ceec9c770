"""GPU parity of pooling, matching and correction (kvc_pool_descriptor, kvc_correct) against
the fp64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import oracle
import synth
from gpu_helpers import check_close, check_every_segment, correct_inputs, dev, say

pytestmark = pytest.mark.gpu


def _run_full(cfg, seed_note="", K_fb=False, tau=None, device_gen="cpu"):
    tau = cfg.tau if tau is None else tau
    say(f"[correct] {cfg.name} L={cfg.L} H={cfg.H} T={cfg.T} d={cfg.d} A={cfg.A} r={cfg.r} "
        f"{cfg.dtype} tau={tau} {seed_note}")
    case = synth.generate(cfg, device_gen)
    d = dev()
    desc, q = correct_inputs(case, "cpu")
    ed = case.edges[0]
    fbK = ed.exact_K if K_fb else None
    fbV = ed.exact_V if K_fb else None
    ref = oracle.correct(synth.to_f64(case.K0), synth.to_f64(case.V0), synth.to_f64(desc),
                         synth.to_f64(ed.U), synth.to_f64(ed.W), tau, cfg.dtype,
                         K_fb=None if fbK is None else synth.to_f64(fbK),
                         V_fb=None if fbV is None else synth.to_f64(fbV))
    out = kvc.correct(case.K0.to(d), case.V0.to(d), desc.to(d), ed.U.to(d), ed.W.to(d), tau,
                      K_fb=None if fbK is None else fbK.to(d),
                      V_fb=None if fbV is None else fbV.to(d), want_q_next=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.mask.cpu().numpy(), ref["mask"])
    check_close("K'", synth.to_f64(out.K), ref["K_out"])
    check_close("V'", synth.to_f64(out.V), ref["V_out"])
    fin = np.isfinite(ref["score"])
    np.testing.assert_allclose(out.score.cpu().numpy()[fin], ref["score"][fin], atol=2e-6)
    keep = ref["mask"] == 0
    np.testing.assert_allclose(out.w.cpu().numpy()[keep], ref["w"][keep], rtol=1e-5, atol=1e-6)
    qn = oracle.pool(synth.to_f64(out.K), synth.to_f64(out.V))
    np.testing.assert_allclose(out.q_next.cpu().numpy(), qn, rtol=1e-5, atol=1e-6)
    return case, out, ref


def test_tiny_config():
    case, out, ref = _run_full(synth.CONFIGS["tiny"])
    assert out.mask.item() == 0  # cos(q, q - noise) ~ 0.76 > tau = 0.3
    # the correction moves the cache towards the exact one
    e0 = oracle.rel_frobenius(synth.to_f64(case.K0), synth.to_f64(case.edges[0].exact_K))
    e1 = oracle.rel_frobenius(synth.to_f64(out.K), synth.to_f64(case.edges[0].exact_K))
    assert e1 < e0


SMALL = [
    # (dtype, d, T, A, r)
    ("bf16", 128, 700, 4, 32),
    ("bf16", 128, 1, 4, 32),
    ("bf16", 128, 31, 1, 1),
    ("bf16", 64, 1537, 3, 16),
    ("bf16", 128, 513, 5, 40),
    ("bf16", 64, 129, 2, 64),
    ("bf16", 128, 260, 16, 16),
    ("bf16", 128, 96, 2, 7),
    ("bf16", 128, 700, 6, 32),   # compact LDS layout (6 and 8 anchors of rank 32)
    ("bf16", 128, 333, 8, 32),
    ("f32", 64, 256, 2, 8),
    ("f32", 128, 777, 3, 12),
    ("f32", 128, 64, 1, 64),
    ("f32", 64, 333, 8, 5),
    # general correction: every shape with r <= d and A * r <= 256 outside the specialised
    # kernel's budget (one contraction over the concatenated rank index)
    ("bf16", 128, 700, 2, 128),   # r = d
    ("f32", 128, 300, 4, 32),
    ("bf16", 64, 500, 4, 64),     # r = d = 64, A * r = 256
    ("bf16", 128, 333, 256, 1),   # 256 anchors of rank 1
    ("bf16", 128, 200, 20, 12),   # A > 16, r not a multiple of 8
    ("f32", 64, 129, 3, 64),
    ("f32", 128, 257, 1, 128),
    ("bf16", 128, 96, 9, 28),
    ("f32", 64, 70, 17, 15),
]


@pytest.mark.parametrize("dtype,d,T,A,r", SMALL)
def test_small_shapes(dtype, d, T, A, r):
    base = synth.CONFIGS["llama8b_t2048"]
    cfg = base.replace(name=f"small_{dtype}_{d}_{T}_{A}_{r}", L=2, H=3, T=T, d=d, A=A, r=r,
                       dtype=dtype, seed=1000 + T + A + r, fallback_prob=0.3)
    _run_full(cfg)


@pytest.mark.parametrize("L,H,T", [(1, 13, 2048), (3, 3, 1500), (5, 7, 300)])
def test_segment_counts_not_a_multiple_of_the_grid(L, H, T):
    """Segment counts that leave the persistent grid's work uneven (prime segment counts,
    fewer items than workgroups) must not change any result."""
    base = synth.CONFIGS["llama8b_t2048"]
    cfg = base.replace(name=f"queues_{L}x{H}_{T}", L=L, H=H, T=T, seed=2000 + L * H + T,
                       fallback_prob=0.3)
    _run_full(cfg)


def test_fallback_sources_are_copied_bit_exact():
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=3, H=2, T=700, seed=77, fallback_prob=0.5)
    case, out, ref = _run_full(cfg, K_fb=True)
    m = out.mask.cpu().numpy().astype(bool)
    assert m.any() and (~m).any()
    got = out.K.cpu()[torch.from_numpy(m)]
    want = case.edges[0].exact_K[torch.from_numpy(m)]
    assert torch.equal(got, want)


def test_threshold_extremes_and_zero_factors():
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=2, H=2, T=300, seed=5)
    case = synth.generate(cfg)
    d = dev()
    desc, _ = correct_inputs(case, "cpu")
    ed = case.edges[0]
    K, V = case.K0.to(d), case.V0.to(d)
    # tau = +inf: everything falls back, outputs are the sources bit for bit
    out = kvc.correct(K, V, desc.to(d), ed.U.to(d), ed.W.to(d), math.inf)
    torch.cuda.synchronize()
    assert int(out.mask.sum()) == 4
    assert torch.equal(out.K, K) and torch.equal(out.V, V)
    # zero factors with tau = -inf: nothing falls back and the correction is the identity
    Z = torch.zeros_like(ed.U).to(d)
    out = kvc.correct(K, V, desc.to(d), Z, ed.W.to(d), -math.inf)
    torch.cuda.synchronize()
    assert int(out.mask.sum()) == 0
    assert torch.equal(out.K, K) and torch.equal(out.V, V)
    # NaN descriptor -> NaN score -> fall back even at tau = -inf
    dn = desc.clone()
    dn[0, 1, 2, 5] = float("nan")
    out = kvc.correct(K, V, dn.to(d), ed.U.to(d), ed.W.to(d), -math.inf)
    torch.cuda.synchronize()
    assert out.mask.cpu().tolist() == [[0, 1], [0, 0]]
    assert math.isnan(out.score[0, 1].item())


@pytest.mark.parametrize("A", [4, 6])
def test_in_place_and_precomputed_query(A):
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=2, H=4, T=1000, seed=9 + A, A=A)
    case = synth.generate(cfg)
    d = dev()
    desc, q = correct_inputs(case, "cpu")
    ed = case.edges[0]
    ref = kvc.correct(case.K0.to(d), case.V0.to(d), desc.to(d), ed.U.to(d), ed.W.to(d), cfg.tau)
    qg = kvc.pool_descriptor(case.K0.to(d), case.V0.to(d))
    torch.cuda.synchronize()
    np.testing.assert_allclose(qg.cpu().numpy(), q, rtol=1e-5, atol=1e-6)
    K, V = case.K0.to(d), case.V0.to(d)
    out = kvc.correct(K, V, desc.to(d), ed.U.to(d), ed.W.to(d), cfg.tau, q_in=qg, K_out=K,
                      V_out=V)
    torch.cuda.synchronize()
    assert out.K.data_ptr() == K.data_ptr()
    assert torch.equal(out.mask, ref.mask)
    assert torch.equal(K, ref.K) and torch.equal(V, ref.V)


def test_deterministic_and_empty():
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=2, H=2, T=900, seed=11)
    case = synth.generate(cfg)
    d = dev()
    desc, _ = correct_inputs(case, "cpu")
    ed = case.edges[0]
    args = (case.K0.to(d), case.V0.to(d), desc.to(d), ed.U.to(d), ed.W.to(d), cfg.tau)
    a = kvc.correct(*args, want_q_next=True)
    b = kvc.correct(*args, want_q_next=True)
    torch.cuda.synchronize()
    assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V) and torch.equal(a.q_next, b.q_next)
    assert torch.equal(a.score, b.score)
    # no segments: a no-op
    e = torch.empty(0, 2, 16, 128, dtype=torch.bfloat16, device=d)
    out = kvc.correct(e, e, torch.empty(0, 2, 4, 256, device=d),
                      torch.empty(2, 0, 2, 4, 16, 32, dtype=torch.bfloat16, device=d),
                      torch.empty(2, 0, 2, 4, 32, 128, dtype=torch.bfloat16, device=d), 0.3)
    assert out.K.numel() == 0
    # no tokens: the pooled query is 0, every score is 0
    e = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device=d)
    out = kvc.correct(e, e, torch.randn(1, 2, 4, 256, device=d),
                      torch.empty(2, 1, 2, 4, 0, 32, dtype=torch.bfloat16, device=d),
                      torch.randn(2, 1, 2, 4, 32, 128, device=d).to(torch.bfloat16), 0.3,
                      want_q_next=True)
    torch.cuda.synchronize()
    assert out.mask.cpu().tolist() == [[1, 1]] and float(out.score.abs().sum()) == 0.0
    assert float(out.q_next.abs().sum()) == 0.0


def _run_every_segment(cfg):
    """Full-size workload generated on the GPU: mask and score of every segment against the
    oracle's matching, and the corrected K', V' of every segment against the oracle's
    correction, one layer at a time."""
    say(f"[correct-full] {cfg.name} L={cfg.L} H={cfg.H} T={cfg.T} A={cfg.A} r={cfg.r}")
    d = dev()
    case = synth.generate(cfg, d)
    desc, q = correct_inputs(case, d)
    ed = case.edges[0]
    out = kvc.correct(case.K0, case.V0, desc, ed.U, ed.W, cfg.tau)
    torch.cuda.synchronize()
    s = oracle.cosine_scores(q, synth.to_f64(desc))
    score, mask = oracle.reliability(s, cfg.tau)
    np.testing.assert_array_equal(out.mask.cpu().numpy(), mask)
    np.testing.assert_allclose(out.score.cpu().numpy(), score, atol=2e-6)
    say(f"  reuse ratio {1.0 - mask.mean():.3f}")
    check_every_segment(cfg.name, out.K, out.V, lambda l: oracle.correct(
        synth.to_f64(case.K0[l:l + 1]), synth.to_f64(case.V0[l:l + 1]),
        synth.to_f64(desc[l:l + 1]), synth.to_f64(ed.U[:, l:l + 1]),
        synth.to_f64(ed.W[:, l:l + 1]), cfg.tau, cfg.dtype), cfg.L, mask)
    del case, out
    torch.cuda.empty_cache()


def test_llama8b_t2048_full_size():
    _run_every_segment(synth.CONFIGS["llama8b_t2048"])


def test_llama8b_t8192_full_size():
    _run_every_segment(synth.CONFIGS["llama8b_t8192_fit"])


def test_vl_t9216_full_size():
    _run_every_segment(synth.CONFIGS["vl_t9216"])


def test_three_tilings_of_one_correction_agree():
    """The same correction through three kernels: A = 2 anchors of rank 32 (the compile-time
    variant), the same factors zero-padded to rank 40 (the runtime-shaped specialised kernel:
    other k-steps, other accumulation groups) and to rank 80 (the general kernel: one
    contraction over the concatenated rank index).  Zero factor columns add exact zeros, so the
    three results differ only by float32 accumulation order (and the general kernel's hi + lo
    split of the weighted factor), which flips a last bf16 place now and then: every pair
    within 2e-4 relative Frobenius (each within the bars of the oracle); masks and weights
    identical."""
    base = synth.CONFIGS["llama8b_t2048"]
    cfg = base.replace(name="tilings", L=3, H=2, T=777, A=2, r=32, seed=313, fallback_prob=0.3)
    say(f"[tilings] {cfg.L}x{cfg.H}x{cfg.T} A=2, r = 32 / 40 / 80")
    case = synth.generate(cfg, "cpu")
    d = dev()
    desc, _ = correct_inputs(case, d)
    ed = case.edges[0]
    K, V = case.K0.to(d), case.V0.to(d)
    outs = []
    for rr in (32, 40, 80):
        U = torch.zeros(2, cfg.L, cfg.H, 2, cfg.T, rr, dtype=torch.bfloat16)
        W = torch.zeros(2, cfg.L, cfg.H, 2, rr, cfg.d, dtype=torch.bfloat16)
        U[..., :32] = ed.U
        W[..., :32, :] = ed.W
        outs.append(kvc.correct(K, V, desc, U.to(d), W.to(d), cfg.tau))
    torch.cuda.synchronize()
    ref = oracle.correct(synth.to_f64(case.K0), synth.to_f64(case.V0), synth.to_f64(desc),
                         synth.to_f64(ed.U), synth.to_f64(ed.W), cfg.tau, cfg.dtype)
    for i, o in enumerate(outs):
        assert torch.equal(o.mask, outs[0].mask) and torch.equal(o.w, outs[0].w)
        np.testing.assert_array_equal(o.mask.cpu().numpy(), ref["mask"])
        check_close(f"K' tiling {i}", synth.to_f64(o.K), ref["K_out"])
        for j in range(i):
            e = oracle.rel_frobenius(synth.to_f64(o.K), synth.to_f64(outs[j].K))
            say(f"  tilings {j} vs {i}: K' relative difference {e:.2e}")
            assert e <= 2e-4
