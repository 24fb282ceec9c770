"""Pins of the oracle's storage rounding, pooling, cosine, softmax and reliability steps.

Every expected value comes from a hand-worked fixture (tests/golden), a brute-force loop,
a library routine on a special case, or an invariant -- never from the oracle itself.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from conftest import GOLDEN


def _ev(expr):
    return float(eval(expr, {"sqrt": math.sqrt, "exp": math.exp, "e": math.e, "float": float}))


# ---------------------------------------------------------------- bf16 rounding


def test_bf16_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "bf16_rne.json")))["cases"]
    xs = np.array([_ev(c["x"]) for c in cases])
    want = np.array([_ev(c["want"]) for c in cases])
    got = oracle.round_to_bf16(xs)
    for c, g, w in zip(cases, got, want):
        assert (g == w and math.copysign(1, g) == math.copysign(1, w)) or (np.isnan(g) and np.isnan(w)), c
    assert np.isnan(oracle.round_to_bf16(np.array([np.nan])))[0]


def test_bf16_matches_library_on_float32_values():
    # Special case that reduces to a library routine: values exactly representable in
    # float32 are rounded by torch's float32 -> bfloat16 conversion (nearest, ties to even).
    g = torch.Generator().manual_seed(7)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 8)
    lib = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(x.to(torch.float64).numpy())
    np.testing.assert_array_equal(got, lib)
    # ties of every kind: low 16 bits exactly 0x8000
    bits = (torch.randint(0, 2 ** 15, (50000,), generator=g, dtype=torch.int64) << 16) | 0x8000
    bits = bits | (torch.randint(0, 2, (50000,), generator=g) << 31)
    xt = torch.from_numpy(bits.numpy().astype(np.uint32).view(np.float32).copy())
    xt = xt[torch.isfinite(xt)]
    np.testing.assert_array_equal(oracle.round_to_bf16(xt.double().numpy()),
                                  xt.to(torch.bfloat16).double().numpy())


def test_f32_rounding_is_numpy_cast():
    x = np.array([1 + 2 ** -30, 0.1, -3.5])
    np.testing.assert_array_equal(oracle.round_to_dtype(x, "f32"), x.astype(np.float32).astype(np.float64))
    with pytest.raises(ValueError):
        oracle.round_to_dtype(x, "fp8")


# ---------------------------------------------------------------- pooling


def test_pool_constant_rows_return_the_row():
    row_k = np.array([1.5, -2.0, 3.25])
    row_v = np.array([0.0, 7.0, -1.0])
    K = np.tile(row_k, (2, 3, 17, 1))
    V = np.tile(row_v, (2, 3, 17, 1))
    q = oracle.pool(K, V)
    assert q.shape == (2, 3, 6)
    np.testing.assert_array_equal(q[1, 2], np.concatenate([row_k, row_v]))


def test_pool_brute_force_loops():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((2, 2, 5, 3))
    V = rng.standard_normal((2, 2, 5, 3))
    q = oracle.pool(K, V)
    for l in range(2):
        for h in range(2):
            for c in range(3):
                sk = 0.0
                sv = 0.0
                for t in range(5):
                    sk += K[l, h, t, c]
                    sv += V[l, h, t, c]
                assert q[l, h, c] == pytest.approx(sk / 5, rel=1e-15, abs=1e-15)
                assert q[l, h, 3 + c] == pytest.approx(sv / 5, rel=1e-15, abs=1e-15)


def test_pool_empty_segment_is_zero():
    q = oracle.pool(np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 0, 4)))
    np.testing.assert_array_equal(q, np.zeros((1, 1, 8)))


# ---------------------------------------------------------------- cosine / softmax / mask


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "matching_hand.json")))["cases"])
def test_matching_hand_cases(case):
    q = np.array(case["q"], dtype=np.float64)
    desc = np.array(case["desc"], dtype=np.float64)
    s = oracle.cosine_scores(q, desc)
    np.testing.assert_allclose(s, [_ev(c) for c in case["cos"]], rtol=1e-14, atol=1e-15)
    w = oracle.softmax_weights(s)
    np.testing.assert_allclose(w, [_ev(c) for c in case["w"]], rtol=1e-14, atol=1e-15)
    for tau, want in case["tau_mask"]:
        score, mask = oracle.reliability(s, tau)
        assert score == pytest.approx(_ev(case["score"]), abs=1e-15)
        assert int(mask) == want, (tau, score)


def test_cosine_invariances():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 16))
    desc = rng.standard_normal((4, 5, 16))
    s = oracle.cosine_scores(q, desc)
    assert np.all(np.abs(s) <= 1 + 1e-15)
    # positive scaling of either side leaves the score unchanged
    np.testing.assert_allclose(oracle.cosine_scores(3.5 * q, desc * 0.01), s, rtol=1e-13, atol=1e-15)
    # negation flips the sign
    np.testing.assert_allclose(oracle.cosine_scores(-q, desc), -s, rtol=1e-13, atol=1e-15)
    # self-similarity is 1
    np.testing.assert_allclose(oracle.cosine_scores(q, q[:, None, :]), 1.0, rtol=1e-14)
    # NaN propagates to the score and falls back
    qn = q.copy()
    qn[0, 0] = np.nan
    sn = oracle.cosine_scores(qn, desc)
    assert np.all(np.isnan(sn[0])) and np.all(np.isfinite(sn[1:]))
    _, mask = oracle.reliability(sn, -np.inf)
    assert mask[0] == 1 and np.all(mask[1:] == 0)


def test_softmax_invariances():
    rng = np.random.default_rng(5)
    s = rng.uniform(-1, 1, (6, 4))
    w = oracle.softmax_weights(s)
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=1e-15)
    assert np.all(w > 0)
    np.testing.assert_allclose(oracle.softmax_weights(s + 0.37), w, rtol=1e-14)
    perm = [2, 0, 3, 1]
    np.testing.assert_allclose(oracle.softmax_weights(s[:, perm]), w[:, perm], rtol=1e-15)
    # ordering is preserved and the ratio of two weights is exp of the score gap
    np.testing.assert_allclose(w[:, 0] / w[:, 1], np.exp(s[:, 0] - s[:, 1]), rtol=1e-13)


def test_reliability_threshold_edges():
    s = np.array([[0.3, 0.1], [0.29, -1.0], [np.nan, 0.9]])
    score, mask = oracle.reliability(s, 0.3)
    # score == tau reuses; below falls back; NaN falls back
    assert list(mask) == [0, 1, 1]
    assert list(oracle.reliability(s, np.inf)[1]) == [1, 1, 1]
    assert list(oracle.reliability(s, -np.inf)[1]) == [0, 0, 1]
    # strict "<" on the float64 values: one float64 ulp below tau falls back, tau itself and
    # one ulp above reuse (no rounding of either side)
    for tau in (0.32, 0.6, 0.3, -0.2, 1.0):
        below, above = np.nextafter(tau, -np.inf), np.nextafter(tau, np.inf)
        assert oracle.reliability(np.array([below]), tau)[1] == 1
        assert oracle.reliability(np.array([tau]), tau)[1] == 0
        assert oracle.reliability(np.array([above]), tau)[1] == 0
    # a score between float32(tau) and tau falls back, although score and tau would round
    # to the same float32 value
    t32 = float(np.float32(0.32))
    mid = 0.5 * (0.32 + t32)
    assert t32 < mid < 0.32 and float(np.float32(mid)) == t32
    assert oracle.reliability(np.array([mid]), 0.32)[1] == 1
    # the score is the best cosine, whatever the other anchors hold; -inf never reuses
    assert oracle.reliability(np.array([[-np.inf, 0.5]]), 0.5)[1][0] == 0
    assert oracle.reliability(np.array([[-np.inf]]), -1e300)[1][0] == 1
