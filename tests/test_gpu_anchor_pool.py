"""GPU parity of the online anchor pool (kvc_correct_pooled, kvc_anchor_pool_insert) against
the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import oracle
import synth
from gpu_helpers import check_close, check_every_segment, dev, pool_all, say

pytestmark = pytest.mark.gpu


def _device_pool(p, desc, d):
    return kvc.AnchorPool(desc.to(d), p["U"].to(d), p["W"].to(d), p["count"].to(d),
                          torch.zeros_like(p["count"]).to(d))


def _host_pool(p, desc):
    return {"desc": synth.to_f64(desc), "U": synth.to_f64(p["U"]), "W": synth.to_f64(p["W"]),
            "count": p["count"].cpu().numpy()}


@pytest.mark.parametrize("dtype,dd,T,Vc,A,r", [("bf16", 128, 600, 6, 4, 32),
                                               ("bf16", 64, 333, 10, 3, 16),
                                               ("f32", 128, 257, 5, 2, 8),
                                               ("bf16", 128, 300, 20, 4, 32),
                                               ("bf16", 128, 200, 32, 16, 16),
                                               ("bf16", 64, 100, 1, 1, 8),
                                               ("bf16", 128, 150, 24, 20, 12),  # general
                                               ("f32", 128, 120, 8, 4, 32)])    # general
def test_pooled_correction_matches_the_oracle(dtype, dd, T, Vc, A, r):
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=2, H=4, T=T, d=dd, dtype=dtype, A=A, r=r,
                                                 seed=51 + Vc, fallback_prob=0.25)
    say(f"[pooled] {dtype} d={dd} T={T} Vc={Vc} A={A} r={r}")
    case = synth.generate(cfg)
    p = synth.generate_pool(cfg, Vc)
    p["count"][0, 0] = 0  # an empty pool
    p["count"][1, 1] = A - 1 if A > 1 else 1  # fewer valid slots than A
    p["count"][1, 2] = Vc  # a full pool
    q = oracle.pool(synth.to_f64(case.K0), synth.to_f64(case.V0))
    desc = synth.pool_descriptors(p, q)
    ed = case.edges[0]
    ref = oracle.correct_pooled(synth.to_f64(case.K0), synth.to_f64(case.V0), _host_pool(p, desc),
                                A, cfg.tau, cfg.dtype, K_fb=synth.to_f64(ed.exact_K),
                                V_fb=synth.to_f64(ed.exact_V))
    d = dev()
    res = kvc.correct_pooled(case.K0.to(d), case.V0.to(d), _device_pool(p, desc, d), A, cfg.tau,
                             K_fb=ed.exact_K.to(d), V_fb=ed.exact_V.to(d))
    torch.cuda.synchronize()
    mask = res.mask.cpu().numpy()
    np.testing.assert_array_equal(mask, ref["mask"])
    cnt = p["count"].numpy()
    sl = res.slots.cpu().numpy()
    for l in range(cfg.L):
        for h in range(cfg.H):
            n = min(A, int(cnt[l, h]))
            np.testing.assert_array_equal(sl[l, h, :n], ref["slots"][l, h, :n],
                                          err_msg=f"slots of ({l},{h})")
    np.testing.assert_allclose(res.w.cpu().numpy(), ref["w"], rtol=0, atol=2e-6)
    check_close("K'", synth.to_f64(res.K), ref["K_out"])
    check_close("V'", synth.to_f64(res.V), ref["V_out"])
    assert mask[0, 0] == 1  # the empty pool falls back
    say(f"  fallback {int(mask.sum())} of {mask.size}; counts {cnt.ravel().tolist()}")


def test_full_pool_in_score_order_equals_kvc_correct_bit_for_bit():
    """A full pool of A slots whose scores fall with the slot index selects slots 0..A-1 in
    order, so the pooled path computes exactly what kvc_correct computes from the same q."""
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=3, H=4, T=700, seed=61)
    say("[pooled-vs-correct]")
    case = synth.generate(cfg)
    p = synth.generate_pool(cfg, cfg.A, full=True)
    p["cos"] = torch.sort(p["cos"], dim=-1, descending=True).values
    d = dev()
    K, V = case.K0.to(d), case.V0.to(d)
    q = kvc.pool_descriptor(K, V)
    torch.cuda.synchronize()
    desc = synth.pool_descriptors(p, q.double().cpu()).to(d)
    pool = _device_pool(p, desc, d)
    a = kvc.correct_pooled(K, V, pool, cfg.A, cfg.tau, q_in=q)
    b = kvc.correct(K, V, desc, pool.U, pool.W, cfg.tau, q_in=q)
    c = kvc.correct_pooled(K, V, pool, cfg.A, cfg.tau)  # pooled here: the same q bits
    torch.cuda.synchronize()
    for x in (a, c):
        assert torch.equal(x.mask, b.mask)
        assert torch.equal(x.w, b.w)
        assert torch.equal(x.K, b.K) and torch.equal(x.V, b.V)
        assert torch.equal(x.slots.cpu(), torch.arange(cfg.A, dtype=torch.int32).expand(
            cfg.L, cfg.H, cfg.A))


def test_insert_matches_the_oracle():
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=2, H=3, T=200, seed=62)
    say("[pool-insert]")
    L, H, T, dd, r, Vc = cfg.L, cfg.H, cfg.T, cfg.d, cfg.r, 3
    d = dev()
    pool = kvc.AnchorPool.empty(L, H, T, dd, Vc, r, torch.bfloat16, d)
    st = {"desc": np.zeros((L, H, Vc, 2 * dd)), "U": np.zeros((2, L, H, Vc, T, r)),
          "W": np.zeros((2, L, H, Vc, r, dd)), "count": np.zeros((L, H), dtype=np.int64),
          "head": np.zeros((L, H), dtype=np.int64)}
    g = torch.Generator().manual_seed(5)
    for i in range(5):
        mask = (torch.rand(L, H, generator=g) < 0.6).to(torch.uint8)
        U = torch.randn(2, L, H, T, r, generator=g)
        W = torch.randn(2, L, H, r, dd, generator=g)
        qv = torch.randn(L, H, 2 * dd, generator=g)
        kvc.anchor_pool_insert(pool, mask.to(d), U.to(d), W.to(d), qv.to(d))
        st = oracle.pool_insert(st, mask.numpy(), U.double().numpy(), W.double().numpy(),
                                qv.double().numpy(), "bf16")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(synth.to_f64(pool.U), st["U"])
    np.testing.assert_array_equal(synth.to_f64(pool.W), st["W"])
    np.testing.assert_array_equal(synth.to_f64(pool.desc), st["desc"])
    np.testing.assert_array_equal(pool.count.cpu().numpy(), st["count"])
    np.testing.assert_array_equal(pool.head.cpu().numpy(), st["head"])
    assert st["count"].max() == Vc  # some pool wrapped around


def test_online_loop_fallback_fit_insert_then_reuse():
    """Empty pools fall back; the fit of exact - reused, inserted with the reused cache's
    descriptor, makes the next request reuse every segment and land near the exact cache;
    the second pass matches the oracle run on the device's pool state."""
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=2, H=4, T=1024, seed=63)
    say("[online-loop]")
    d = dev()
    case = synth.generate(cfg, d)
    ed = case.edges[0]
    pool = kvc.AnchorPool.empty(cfg.L, cfg.H, cfg.T, cfg.d, 4, cfg.r, torch.bfloat16, d)
    first = kvc.correct_pooled(case.K0, case.V0, pool, 2, cfg.tau, K_fb=ed.exact_K,
                               V_fb=ed.exact_V)
    assert torch.all(first.mask == 1)
    assert torch.equal(first.K, ed.exact_K)  # fallback: the dense-prefill stand-in
    fit = kvc.fit_anchor(synth.fit_input(case), r=cfg.r)
    q = kvc.pool_descriptor(case.K0, case.V0)
    kvc.anchor_pool_insert(pool, first.mask, fit.U, fit.W, q)
    second = kvc.correct_pooled(case.K0, case.V0, pool, 2, cfg.tau, K_fb=ed.exact_K,
                                V_fb=ed.exact_V)
    torch.cuda.synchronize()
    assert torch.all(second.mask == 0)
    assert torch.all(pool.count == 1)
    np.testing.assert_allclose(second.score.cpu().numpy(), 1.0, atol=1e-5)
    err = oracle.rel_frobenius(synth.to_f64(second.K), synth.to_f64(ed.exact_K))
    base = oracle.rel_frobenius(synth.to_f64(case.K0), synth.to_f64(ed.exact_K))
    say(f"  error vs exact: reused {base:.3e}, corrected {err:.3e}")
    assert err < 0.05 * base
    hp = {"desc": synth.to_f64(pool.desc), "U": synth.to_f64(pool.U), "W": synth.to_f64(pool.W),
          "count": pool.count.cpu().numpy()}
    ref = oracle.correct_pooled(synth.to_f64(case.K0), synth.to_f64(case.V0), hp, 2, cfg.tau,
                                cfg.dtype)
    np.testing.assert_array_equal(second.mask.cpu().numpy(), ref["mask"])
    check_close("K'", synth.to_f64(second.K), ref["K_out"])
    check_close("V'", synth.to_f64(second.V), ref["V_out"])


def test_pooled_full_size_every_segment():
    """The 8B shape at T = 2048 with pools of 10 slots (the listing's main setting) and A = 4:
    every mask and selection exactly, and every segment's output against the oracle."""
    cfg = synth.CONFIGS["llama8b_t2048"]
    Vc = 10
    say(f"[pooled-full] Vc={Vc} A={cfg.A}")
    d = dev()
    case = synth.generate(cfg, d)
    p = synth.generate_pool(cfg, Vc, d, full=True)
    q = pool_all(case.K0, case.V0)
    desc = synth.pool_descriptors(p, q)
    pool = kvc.AnchorPool(desc, p["U"], p["W"], p["count"], torch.zeros_like(p["count"]))
    res = kvc.correct_pooled(case.K0, case.V0, pool, cfg.A, cfg.tau)
    torch.cuda.synchronize()
    s = oracle.cosine_scores(q, synth.to_f64(desc))
    slots, w, score = oracle.select_anchors(s, p["count"].cpu().numpy(), cfg.A)
    m = (~(score >= cfg.tau)).astype(np.uint8)
    np.testing.assert_array_equal(res.mask.cpu().numpy(), m)
    np.testing.assert_array_equal(res.slots.cpu().numpy(), slots)
    count = p["count"].cpu().numpy()

    def ref_layer(l):
        hp = {"desc": synth.to_f64(desc[l:l + 1]), "U": synth.to_f64(p["U"][:, l:l + 1]),
              "W": synth.to_f64(p["W"][:, l:l + 1]), "count": count[l:l + 1]}
        return oracle.correct_pooled(synth.to_f64(case.K0[l:l + 1]),
                                     synth.to_f64(case.V0[l:l + 1]), hp, cfg.A, cfg.tau,
                                     cfg.dtype)

    check_every_segment(f"pooled Vc={Vc}", res.K, res.V, ref_layer, cfg.L, m)
