"""Property tests of the oracle over random small shapes (hypothesis): its two routes to the
anchor fit (Gram + symmetric eigen-decomposition, and the SVD of delta) agree, and the
matching, correction and rounding keep the invariants their definitions imply."""
import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True)


@st.composite
def deltas(draw):
    M = draw(st.integers(1, 3))
    T = draw(st.integers(1, 24))
    d = draw(st.integers(1, 10))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    kind = draw(st.sampled_from(["gauss", "lowrank", "decay", "zero_rows"]))
    x = rng.standard_normal((M, T, d))
    if kind == "lowrank":
        k = draw(st.integers(1, min(T, d)))
        x = rng.standard_normal((M, T, k)) @ rng.standard_normal((M, k, d))
    elif kind == "decay":
        x = x * (0.6 ** np.arange(d))
    elif kind == "zero_rows":
        x[:, : T // 2] = 0.0
    r = draw(st.integers(1, d))
    energy = draw(st.sampled_from([0.5, 0.9, 0.99, 1.0]))
    return x, r, energy


@SETTINGS
@given(deltas())
def test_gram_route_equals_svd_route(case):
    x, r, energy = case
    a = oracle.fit_anchor(x, r, energy)
    b = oracle.fit_from_gram(oracle.gram(x), r, energy)
    lam = a["eig"]
    scale = np.maximum(lam[:, :1], 1e-300)
    np.testing.assert_allclose(b["eig"], lam, rtol=0, atol=1e-9 * scale.max())
    # k_eff agrees unless the energy fraction sits on the threshold within rounding
    tot = lam.sum(-1, keepdims=True)
    frac = np.cumsum(lam, -1) / np.where(tot > 0, tot, 1)
    clear = np.min(np.abs(frac - energy), axis=-1) > 1e-9
    np.testing.assert_array_equal(a["k_eff"][clear], b["k_eff"][clear])
    # the rank-r subspace agrees where it is unique (a clear gap after the r-th eigenvalue)
    for m in range(x.shape[0]):
        d = lam.shape[1]
        gap = lam[m, r - 1] - (lam[m, r] if r < d else 0.0)
        if gap > 1e-6 * max(lam[m, 0], 1e-300) and lam[m, r - 1] > 1e-9 * max(lam[m, 0], 1e-300):
            Pa = a["W"][m].T @ a["W"][m]
            Pb = b["W"][m].T @ b["W"][m]
            np.testing.assert_allclose(Pa, Pb, atol=1e-6)


@SETTINGS
@given(deltas())
def test_truncation_error_is_the_tail_energy(case):
    x, r, _ = case
    a = oracle.fit_anchor(x, r)
    for m in range(x.shape[0]):
        tail = float(np.sum(a["eig"][m, r:]))
        err = float(np.sum((x[m] - a["U"][m] @ a["W"][m]) ** 2))
        total = float(np.sum(x[m] ** 2))
        assert abs(err - tail) <= 1e-9 * max(total, 1e-300)


@st.composite
def caches(draw):
    L = draw(st.integers(1, 2))
    H = draw(st.integers(1, 2))
    T = draw(st.integers(1, 12))
    d = draw(st.integers(1, 6))
    A = draw(st.integers(1, 4))
    r = draw(st.integers(1, d))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    K, V = rng.standard_normal((L, H, T, d)), rng.standard_normal((L, H, T, d))
    desc = rng.standard_normal((L, H, A, 2 * d))
    U = rng.standard_normal((2, L, H, A, T, r))
    W = rng.standard_normal((2, L, H, A, r, d))
    tau = draw(st.floats(-1.0, 1.0))
    return K, V, desc, U, W, tau


@SETTINGS
@given(caches())
def test_correction_invariants(case):
    K, V, desc, U, W, tau = case
    out = oracle.correct(K, V, desc, U, W, tau, "f32")
    np.testing.assert_allclose(out["w"].sum(-1), 1.0, rtol=1e-12)
    assert np.all((out["s"] >= -1 - 1e-12) & (out["s"] <= 1 + 1e-12))
    # zero factors: the stored cache is the source (every segment, either decision)
    z = oracle.correct(K, V, desc, 0 * U, 0 * W, tau, "f32")
    np.testing.assert_array_equal(z["K_out"], oracle.round_to_dtype(K, "f32"))
    # anchors permuted: weights permuted, corrected cache unchanged
    perm = np.arange(desc.shape[2])[::-1]
    p = oracle.correct(K, V, desc[:, :, perm], U[:, :, :, perm], W[:, :, :, perm], tau, "f32")
    np.testing.assert_allclose(p["w"], out["w"][..., perm], rtol=1e-12)
    np.testing.assert_allclose(p["K_exact"], out["K_exact"], rtol=1e-11, atol=1e-11)
    # tokens permuted: the pooled descriptor, hence the decision, is unchanged
    tp = np.arange(K.shape[2])[::-1]
    np.testing.assert_allclose(oracle.pool(K[:, :, tp], V[:, :, tp]), out["q"], rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_array_equal(out["mask"], (~(out["score"] >= tau)).astype(np.uint8))


@SETTINGS
@given(caches(), st.integers(1, 4))
def test_rank_scores_properties(case, rC):
    K, V, _, _, _, _ = case
    rC = min(rC, K.shape[-1])
    F = oracle.rank_descriptor(K, V, rC)["F"]
    G = oracle.rank_descriptor(K[:, :, ::-1], 2.0 * V, rC)["F"]
    s_fg = oracle.rank_scores(F, G[:, :, :, None])[..., 0]
    s_gf = oracle.rank_scores(G, F[:, :, :, None])[..., 0]
    np.testing.assert_allclose(s_fg, s_gf, rtol=1e-12, atol=1e-15)  # symmetric
    assert np.all((s_fg >= -1e-12) & (s_fg <= 1 + 1e-12))
    np.testing.assert_allclose(oracle.rank_scores(F, F[:, :, :, None])[..., 0][
        np.any(F != 0, axis=(0, 3, 4))], 1.0, rtol=1e-12)


@SETTINGS
@given(st.lists(st.floats(-1e30, 1e30, allow_nan=False), min_size=1, max_size=50))
def test_bf16_rounding_is_idempotent_and_monotone(xs):
    x = np.sort(np.array(xs, dtype=np.float64))
    y = oracle.round_to_bf16(x)
    np.testing.assert_array_equal(oracle.round_to_bf16(y), y)
    assert np.all(np.diff(y) >= 0)
    # half a unit in the last of 8 significant bits, or half the subnormal spacing 2^-133
    fin = np.isfinite(y)
    assert np.all(np.abs(y[fin] - x[fin]) <= np.maximum(2.0 ** -8 * np.abs(x[fin]), 2.0 ** -134))
