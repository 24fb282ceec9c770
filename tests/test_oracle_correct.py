"""Pins of the oracle's correction and chaining (hand-worked case, brute force, invariants)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def _brute_correct(K, V, desc, U, W, tau, K_fb=None, V_fb=None):
    """Pure-Python loops over one segment per (l, h): pool, cosine, softmax, max, weighted sum."""
    L, H, T, d = K.shape
    A = desc.shape[2]
    r = U.shape[-1]
    outK = np.zeros_like(K)
    outV = np.zeros_like(V)
    masks = np.zeros((L, H), dtype=np.uint8)
    for l in range(L):
        for h in range(H):
            q = []
            for c in range(d):
                q.append(sum(K[l, h, t, c] for t in range(T)) / T)
            for c in range(d):
                q.append(sum(V[l, h, t, c] for t in range(T)) / T)
            nq = math.sqrt(sum(v * v for v in q))
            s = []
            for a in range(A):
                dv = desc[l, h, a]
                nd = math.sqrt(sum(v * v for v in dv))
                s.append(0.0 if nq * nd == 0 else sum(x * y for x, y in zip(q, dv)) / (nq * nd))
            m = max(s)
            ex = [math.exp(v - m) for v in s]
            w = [v / sum(ex) for v in ex]
            fall = not (m >= tau)  # NaN compares false: falls back
            masks[l, h] = fall
            for x, (X, Xfb, out) in enumerate(((K, K_fb, outK), (V, V_fb, outV))):
                for t in range(T):
                    for c in range(d):
                        if fall:
                            out[l, h, t, c] = X[l, h, t, c] if Xfb is None else Xfb[l, h, t, c]
                            continue
                        acc = X[l, h, t, c]
                        for a in range(A):
                            acc += w[a] * sum(U[x, l, h, a, t, k] * W[x, l, h, a, k, c] for k in range(r))
                        out[l, h, t, c] = acc
    return outK, outV, masks


def _ev(expr, **kw):
    env = {"sqrt": math.sqrt, "exp": math.exp, "e": math.e}
    env.update(kw)
    return float(eval(expr, env))


def test_correct_hand_case():
    g = json.load(open(os.path.join(GOLDEN, "correct_hand.json")))
    K = np.array(g["K"], dtype=np.float64)[None, None]
    V = np.array(g["V"], dtype=np.float64)[None, None]
    desc = np.array(g["desc"], dtype=np.float64)[None, None]
    U = np.stack([np.array(g["UK"]), np.array(g["UV"])])[:, None, None].astype(np.float64)
    W = np.stack([np.array(g["WK"]), np.array(g["WV"])])[:, None, None].astype(np.float64)
    out = oracle.correct(K, V, desc, U, W, g["tau_reuse"], "f32")
    w0, w1 = (_ev(x) for x in g["w"])
    np.testing.assert_allclose(out["q"][0, 0], g["q"], rtol=0, atol=0)
    np.testing.assert_allclose(out["w"][0, 0], [w0, w1], rtol=1e-15)
    wantK = np.array([[_ev(x, w0=w0, w1=w1) for x in row] for row in g["K_out"]])
    wantV = np.array([[_ev(x, w0=w0, w1=w1) for x in row] for row in g["V_out"]])
    np.testing.assert_allclose(out["K_exact"][0, 0], wantK, rtol=1e-15)
    np.testing.assert_allclose(out["V_exact"][0, 0], wantV, rtol=1e-15, atol=1e-16)
    np.testing.assert_array_equal(out["K_out"][0, 0], wantK.astype(np.float32).astype(np.float64))
    assert out["mask"][0, 0] == 0
    fb = oracle.correct(K, V, desc, U, W, g["tau_fallback"], "f32", K_fb=K + 100, V_fb=None)
    assert fb["mask"][0, 0] == 1
    np.testing.assert_array_equal(fb["K_out"], K + 100)
    np.testing.assert_array_equal(fb["V_out"], V)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_correct_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    L, H, T, d, A, r = 2, 2, 5, 3, 3, 2
    K = rng.standard_normal((L, H, T, d))
    V = rng.standard_normal((L, H, T, d))
    desc = rng.standard_normal((L, H, A, 2 * d))
    U = rng.standard_normal((2, L, H, A, T, r))
    W = rng.standard_normal((2, L, H, A, r, d))
    K_fb = rng.standard_normal((L, H, T, d))
    tau = 0.1
    out = oracle.correct(K, V, desc, U, W, tau, "f32", K_fb=K_fb)
    bK, bV, bm = _brute_correct(K, V, desc, U, W, tau, K_fb=K_fb)
    np.testing.assert_array_equal(out["mask"], bm)
    np.testing.assert_allclose(out["K_exact"], bK, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out["V_exact"], bV, rtol=1e-13, atol=1e-13)


def test_zero_factors_are_identity_bit_exact():
    rng = np.random.default_rng(4)
    K = oracle.round_to_bf16(rng.standard_normal((2, 3, 7, 4)))
    V = oracle.round_to_bf16(rng.standard_normal((2, 3, 7, 4)))
    desc = rng.standard_normal((2, 3, 2, 8))
    U = np.zeros((2, 2, 3, 2, 7, 5))
    W = rng.standard_normal((2, 2, 3, 2, 5, 4))
    out = oracle.correct(K, V, desc, U, W, -np.inf, "bf16")
    assert np.all(out["mask"] == 0)
    np.testing.assert_array_equal(out["K_out"], K)
    np.testing.assert_array_equal(out["V_out"], V)
    out = oracle.correct(K, V, desc, W[..., :1, :1].repeat(7, -2).repeat(5, -1), W, np.inf, "bf16")
    assert np.all(out["mask"] == 1)
    np.testing.assert_array_equal(out["K_out"], K)


def test_anchor_permutation_invariance():
    rng = np.random.default_rng(8)
    K = rng.standard_normal((1, 2, 6, 4))
    V = rng.standard_normal((1, 2, 6, 4))
    desc = rng.standard_normal((1, 2, 4, 8))
    U = rng.standard_normal((2, 1, 2, 4, 6, 3))
    W = rng.standard_normal((2, 1, 2, 4, 3, 4))
    perm = [3, 1, 0, 2]
    a = oracle.correct(K, V, desc, U, W, -1.0, "f32")
    b = oracle.correct(K, V, desc[:, :, perm], U[:, :, :, perm], W[:, :, :, perm], -1.0, "f32")
    np.testing.assert_allclose(b["K_exact"], a["K_exact"], rtol=1e-13)
    np.testing.assert_allclose(b["w"], a["w"][..., perm], rtol=1e-14)


def test_single_exact_anchor_recovers_exact_cache():
    # One anchor whose factors are the planted delta: w = 1 and X' = X + delta exactly.
    rng = np.random.default_rng(9)
    T, d, r = 12, 6, 3
    K = rng.standard_normal((1, 1, T, d))
    V = rng.standard_normal((1, 1, T, d))
    U = rng.standard_normal((2, 1, 1, 1, T, r))
    W = rng.standard_normal((2, 1, 1, 1, r, d))
    EK = K + U[0, 0, 0, 0] @ W[0, 0, 0, 0]
    EV = V + U[1, 0, 0, 0] @ W[1, 0, 0, 0]
    desc = rng.standard_normal((1, 1, 1, 2 * d))
    out = oracle.correct(K, V, desc, U, W, -np.inf, "f32")
    assert out["w"][0, 0, 0] == 1.0
    np.testing.assert_allclose(out["K_exact"], EK, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out["V_exact"], EV, rtol=1e-14, atol=1e-14)


def test_precomputed_query_is_used():
    rng = np.random.default_rng(10)
    K = rng.standard_normal((1, 1, 4, 2))
    V = rng.standard_normal((1, 1, 4, 2))
    desc = np.array([[[[1.0, 0, 0, 0], [0, 1.0, 0, 0]]]])
    U = rng.standard_normal((2, 1, 1, 2, 4, 1))
    W = rng.standard_normal((2, 1, 1, 2, 1, 2))
    q = np.array([[[0.0, 5.0, 0, 0]]])
    out = oracle.correct(K, V, desc, U, W, 0.5, "f32", q=q)
    np.testing.assert_allclose(out["s"][0, 0], [0.0, 1.0])


def test_chain_first_source_is_exact_and_edges_compose():
    rng = np.random.default_rng(12)
    L, H, T, d, A, r = 1, 2, 5, 3, 2, 2
    K0 = oracle.round_to_bf16(rng.standard_normal((L, H, T, d)))
    V0 = oracle.round_to_bf16(rng.standard_normal((L, H, T, d)))
    edges = []
    for _ in range(3):
        edges.append({
            "desc": rng.standard_normal((L, H, A, 2 * d)),
            "U": oracle.round_to_bf16(rng.standard_normal((2, L, H, A, T, r))),
            "W": oracle.round_to_bf16(rng.standard_normal((2, L, H, A, r, d))),
            "K_fb": oracle.round_to_bf16(rng.standard_normal((L, H, T, d))),
            "V_fb": oracle.round_to_bf16(rng.standard_normal((L, H, T, d))),
        })
    res = oracle.chain(K0, V0, edges, 0.0, "bf16")
    np.testing.assert_array_equal(res[0]["K_src"], K0)
    np.testing.assert_array_equal(res[0]["V_src"], V0)
    srcK, srcV = K0, V0
    for ed, out in zip(edges, res):
        one = oracle.correct(srcK, srcV, ed["desc"], ed["U"], ed["W"], 0.0, "bf16",
                             K_fb=ed["K_fb"], V_fb=ed["V_fb"])
        np.testing.assert_array_equal(out["K_out"], one["K_out"])
        np.testing.assert_array_equal(out["mask"], one["mask"])
        # every stored output is a bf16 value
        np.testing.assert_array_equal(oracle.round_to_bf16(out["K_out"]), out["K_out"])
        srcK, srcV = one["K_out"], one["V_out"]


def test_rel_frobenius_definition():
    ref = np.array([[3.0, 0.0], [0.0, 4.0]])
    x = np.array([[3.0, 1.0], [0.0, 4.0]])
    assert oracle.rel_frobenius(x, ref) == pytest.approx(1.0 / 5.0, rel=1e-15)
    assert oracle.rel_frobenius(ref, ref) == 0.0
