"""The synthetic workload generator: determinism, planted spectra, guard bands."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_generate_is_deterministic():
    a = synth.generate("tiny")
    b = synth.generate("tiny")
    assert torch.equal(a.K0, b.K0) and torch.equal(a.edges[0].U, b.edges[0].U)
    assert torch.equal(a.edges[0].exact_V, b.edges[0].exact_V)


def test_tiny_planted_factors_and_spectrum():
    c = synth.generate("tiny")
    cfg = c.cfg
    ed = c.edges[0]
    assert c.K0.dtype == torch.float32 and ed.U.shape == (2, 1, 1, 2, 256, 8)
    W0 = ed.W[0, 0, 0, 0].double()
    np.testing.assert_allclose((W0 @ W0.T).numpy(), np.eye(8), atol=1e-6)
    base = math.sqrt(float((c.K0.double() ** 2).sum()))
    want = cfg.scale0 * cfg.decay ** np.arange(cfg.r) * base
    np.testing.assert_allclose(ed.sigma[0, 0, 0].numpy(), want, rtol=1e-12)
    U0 = ed.U[0, 0, 0, 0].double()
    np.testing.assert_allclose(torch.linalg.vector_norm(U0, dim=0).numpy(), want, rtol=1e-6)
    # the delta the fit sees has the planted spectrum (up to the 1e-4 noise)
    delta = synth.to_f64(synth.fit_input(c))
    sv = np.linalg.svd(delta[0], compute_uv=False)
    np.testing.assert_allclose(sv[:8], want, rtol=2e-3)


def test_descriptor_targets_and_guard_band():
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=3, H=4, T=64)
    c = synth.generate(cfg)
    q = oracle.pool(synth.to_f64(c.K0), synth.to_f64(c.V0))
    desc = synth.build_descriptors(c, 0, q).double().numpy()
    s = oracle.cosine_scores(q, desc)
    tgt = c.edges[0].cos_target.numpy()
    np.testing.assert_allclose(s, tgt, atol=2e-6)  # float32 storage of the descriptors
    score = s.max(-1)
    assert np.all(np.abs(score - cfg.tau) >= cfg.guard - 1e-5)


def test_fit_input_is_exact_minus_reused():
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=1, H=2, T=32)
    c = synth.generate(cfg)
    d = synth.fit_input(c)
    assert d.shape == (4, 32, 128) and d.dtype == torch.bfloat16
    want = (c.edges[0].exact_K.double() - c.K0.double()).to(torch.bfloat16).reshape(2, 32, 128)
    assert torch.equal(d[:2], want)


def test_vl_visual_rows_have_twice_the_variance():
    cfg = synth.CONFIGS["vl_t9216"].replace(L=1, H=1, T=9216)
    c = synth.generate(cfg)
    k = c.K0[0, 0].float()
    v_vis = float(k[1024:8024].var())
    v_txt = float(torch.cat([k[:1024], k[8024:]]).var())
    assert v_vis / v_txt == pytest.approx(2.0, rel=0.05)


def test_chain_exact_caches_follow_each_other():
    cfg = synth.CONFIGS["chain_t32768"].replace(L=1, H=1, T=64)
    c = synth.generate(cfg)
    assert len(c.edges) == 3
    for e in range(3):
        d = synth.fit_input(c, e).double()
        assert float(d.abs().sum()) > 0
