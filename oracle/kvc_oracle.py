"""fp64 CPU oracle of KVCMAS's online KV-cache correction and its rank-r anchor fit.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this module; the HIP library never calls it and shares no
code, table or constant with it.

Source: "KVCMAS: Efficient KV cache Correction for Shared Context in Multi-Agent Systems"
(arXiv:2609.34060), as shown on the thelatestinai listing (captions of Figs. 1, 2, 3, 7, 13
and Tables 3, 6, 13) and the metraipolis abstract.  The pages describe the method in prose
only; every formula below is the plainest reading of that prose, and each function says
which.

Conventions
* Caches K, V: [L, H, T, d] (layer, kv-head, token, channel); one (l, h) is a segment.
* Descriptors: [L, H, A, 2d]; anchor factors U: [2, L, H, A, T, r], W: [2, L, H, A, r, d]
  (index 0 = K, 1 = V).  Fit input delta: [M, T, d].
* All arithmetic is float64.  Cache values given in bf16 / fp32 are widened exactly.
  Outputs stored in the cache dtype are rounded ONCE from the float64 value.

Parity pins: every function is checked in ``tests/test_oracle_*.py`` against closed forms,
hand-worked fixtures (``tests/golden``), brute force on tiny inputs and invariants.  The
reading of the method itself (mean-pooled descriptor, cosine, softmax with temperature 1,
max-cosine reliability) is not pinned by any number on the pages: parity with the
authors' own implementation is unpinned; parity of the GPU path with this oracle is.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------------------


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and float32's exponent
    range: normal numbers down to 2^-126, subnormals in steps of 2^-133, overflow to inf
    at (2 - 2^-8) * 2^127 and above.  The rounding is done directly from float64, so a
    value is rounded exactly once.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    v = x[fin]
    _, e = np.frexp(v)  # |v| = m * 2^e with m in [0.5, 1)
    # quantum of the 8-bit significand at this binade; below 2^-126 the spacing is fixed
    q_exp = np.maximum(e - 8, -133)
    scaled = np.ldexp(v, -q_exp)  # exact: power-of-two scaling
    y = np.ldexp(np.rint(scaled), q_exp)  # np.rint rounds half to even
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, v), y)
    out[fin] = y
    return out


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Store float64 values in the cache dtype ("bf16" or "f32") once, back as float64."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------------------
# matching: descriptor, cosine, softmax, reliability
# --------------------------------------------------------------------------------------


def pool(K, V) -> np.ndarray:
    """Pooled descriptor of a cache segment: q = [mean_t K ; mean_t V], shape [..., 2d].

    Fig. 1(b): the current cache representation is matched against the segment's
    online anchors.  Reading: the representation is the token mean of the segment's
    keys followed by the token mean of its values.  An empty segment (T = 0) pools to 0.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    T = K.shape[-2]
    if T == 0:
        return np.zeros(K.shape[:-2] + (2 * K.shape[-1],), dtype=np.float64)
    return np.concatenate([K.sum(axis=-2) / T, V.sum(axis=-2) / T], axis=-1)


def cosine_scores(q, desc) -> np.ndarray:
    """s_a = <q, desc_a> / (||q|| ||desc_a||), and 0 when either norm is 0. Shape [..., A].

    Fig. 1(b): similarity between the current representation and each online anchor.
    Reading: cosine similarity; a zero vector has no direction and scores 0; a NaN in
    either vector gives a NaN score (which then falls back, see ``reliability``).
    """
    q = np.asarray(q, dtype=np.float64)
    desc = np.asarray(desc, dtype=np.float64)
    dots = np.einsum("...k,...ak->...a", q, desc)
    qq = np.einsum("...k,...k->...", q, q)[..., None]
    dd = np.einsum("...ak,...ak->...a", desc, desc)
    # ||q|| ||d|| as one square root of the product of the squared norms (one rounding fewer
    # than a product of two roots: parallel vectors with exact squared norms give exactly 1)
    den = np.sqrt(qq * dd)
    with np.errstate(invalid="ignore", divide="ignore"):
        s = np.where(den == 0, 0.0, dots / np.where(den == 0, 1.0, den))
    return s


def softmax_weights(s) -> np.ndarray:
    """w_a = exp(s_a - max s) / sum_b exp(s_b - max s) over the anchors (last axis).

    Fig. 1(b): anchor corrections are combined with similarity-based weights.
    Reading: a softmax of the cosines with temperature 1 over all A anchors.
    """
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def reliability(s, tau):
    """score = max_a s_a; fallback mask = score < tau, or score not a number.

    Fig. 1(a): a shared segment's cache is reused when its correction is reliable and
    falls back to dense prefill otherwise; Table 3 gives one threshold tau per workload.
    Reading: the reliability score is the best anchor cosine and the comparison is
    strict (score == tau reuses, score < tau falls back); a NaN score compares false
    and falls back.  Score and tau are compared as float64 values, tau as passed.
    """
    s = np.asarray(s, dtype=np.float64)
    score = np.max(s, axis=-1)  # NaN propagates
    mask = ~(score >= np.float64(tau))
    return score, mask.astype(np.uint8)


# --------------------------------------------------------------------------------------
# correction
# --------------------------------------------------------------------------------------


def _apply(K, V, s, U, W, tau, dtype, K_fb, V_fb) -> dict:
    """Weights, decision and correction from given anchor scores s [L, H, A] (see ``correct``)."""
    w = softmax_weights(s)
    score, mask = reliability(s, tau)
    outs = []
    for x, (X, X_fb) in enumerate(((K, K_fb), (V, V_fb))):
        delta = np.zeros_like(X)
        for a in range(U.shape[3]):
            delta += w[..., a, None, None] * np.matmul(U[x, :, :, a], W[x, :, :, a])
        corrected = X + delta
        keep = X if X_fb is None else np.asarray(X_fb, dtype=np.float64)
        exact = np.where(mask[..., None, None].astype(bool), keep, corrected)
        outs.append(exact)
    return {
        "K_exact": outs[0],
        "V_exact": outs[1],
        "K_out": round_to_dtype(outs[0], dtype),
        "V_out": round_to_dtype(outs[1], dtype),
        "s": s,
        "w": w,
        "score": score,
        "mask": mask,
    }


def correct(K, V, desc, U, W, tau, dtype, K_fb=None, V_fb=None, q=None) -> dict:
    """Correct a reused cache with the similarity-weighted sum of the anchors' low-rank deltas.

    For every segment (l, h) and X in {K, V}:
        X' = X + sum_a w_a U^X_a W^X_a        if the segment is reliable,
        X' = X_fb (dense-prefill stand-in) or X   if it falls back,
    then X' is stored once in ``dtype``.  The weights w are shared by K and V.

    Figs. 1(a) and 1(b); the abstract (cross-agent deviations kept as compact low-rank
    states).  Inputs: K, V [L, H, T, d]; desc [L, H, A, 2d]; U [2, L, H, A, T, r];
    W [2, L, H, A, r, d]; optional fallback caches and a precomputed pooled query q.
    Returns float64 arrays: K_out, V_out (stored values), K_exact, V_exact (before
    storage rounding), and q, s, w, score, mask.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if q is None:
        q = pool(K, V)
    q = np.asarray(q, dtype=np.float64)
    out = _apply(K, V, cosine_scores(q, desc), U, W, tau, dtype, K_fb, V_fb)
    out["q"] = q
    return out


# --------------------------------------------------------------------------------------
# matching on the rank-r_C representation of the cache
# --------------------------------------------------------------------------------------


def rank_descriptor(K, V, rC: int) -> dict:
    """Rank-r_C representation of every cache segment (Fig. 13: base-cache rank r_C, 32 by
    default; Fig. 2: effective rank of the base cache).  Reading: for X in {K, V} the segment
    is represented by its rank-r_C truncated second-moment matrix G_r = sum_{i <= r_C}
    sigma_i^2 v_i v_i^T (sigma_i, v_i: singular values and right singular vectors of the
    T x d matrix X), stored as the factor F = diag(sigma_1..r_C) V_r^T (r_C x d), so that
    G_r = F^T F; each row's largest-magnitude entry is positive (the sign does not enter
    any similarity).  Returns F [2, L, H, rC, d] (index 0 = K) and the cache's effective rank
    k_eff [2, L, H] at 90% energy (``effective_rank``)."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, H, T, d = K.shape
    F = np.zeros((2, L, H, rC, d))
    lam = np.zeros((2, L, H, d))
    for x, X in enumerate((K, V)):
        for l in range(L):
            for h in range(H):
                if T == 0:
                    continue
                _, sv, vt = np.linalg.svd(X[l, h], full_matrices=False)
                k = sv.shape[0]
                lam[x, l, h, :k] = sv * sv
                rr = min(rC, k)
                F[x, l, h, :rr] = sv[:rr, None] * _canonical_rows(vt[:rr])
    return {"F": F, "k_eff": effective_rank(lam), "eig": lam}


def rank_scores(Fq, Fa) -> np.ndarray:
    """Similarity of rank-r_C representations: the cosine of the truncated second-moment
    matrices of K and V taken together as one vector,
        s_a = (<Gq_K, Ga_K> + <Gq_V, Ga_V>) / (||(Gq_K, Gq_V)|| ||(Ga_K, Ga_V)||),
    with Frobenius inner products <G, G'> = ||F F'^T||_F^2 (G = F^T F) and 0 when either norm
    is 0.  Sign flips and rotations of the factor rows leave it unchanged.  Reading of the
    listing's Fig. 1(b) matching on the cache representation of Fig. 13 (r_C).
    Fq: [2, L, H, rC, d]; Fa: [2, L, H, A, rC, d] -> s [L, H, A]."""
    Fq = np.asarray(Fq, dtype=np.float64)
    Fa = np.asarray(Fa, dtype=np.float64)
    A = Fa.shape[3]
    L, H = Fq.shape[1], Fq.shape[2]
    s = np.zeros((L, H, A))
    for l in range(L):
        for h in range(H):
            nq = sum(np.sum((Fq[x, l, h] @ Fq[x, l, h].T) ** 2) for x in range(2))
            for a in range(A):
                na = sum(np.sum((Fa[x, l, h, a] @ Fa[x, l, h, a].T) ** 2) for x in range(2))
                dot = sum(np.sum((Fq[x, l, h] @ Fa[x, l, h, a].T) ** 2) for x in range(2))
                den = np.sqrt(nq * na)
                s[l, h, a] = 0.0 if den == 0 else dot / den
    return s


def correct_rank(K, V, Fq, Fa, U, W, tau, dtype, K_fb=None, V_fb=None) -> dict:
    """``correct`` with the anchors matched on rank-r_C representations (``rank_scores``)
    instead of the mean-pooled descriptor: softmax weights, reliability and correction as
    in ``correct``."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return _apply(K, V, rank_scores(Fq, Fa), U, W, tau, dtype, K_fb, V_fb)


def chain(K0, V0, edges, tau, dtype) -> list:
    """Chained correction along a workflow A0 -> A1 -> ... (Fig. 1(c), Fig. 3(b)).

    Agent A0's cache is exact and is the first edge's source, untouched.  Edge i
    corrects its source and stores the result in ``dtype``; that stored cache is the
    source of edge i+1, with no separate reference prefill.  ``edges`` is a list of
    dicts with keys desc, U, W and optionally K_fb, V_fb (agent i+1's dense-prefill
    cache, used where the segment falls back) and q (a precomputed pooled query).
    Returns the per-edge outputs of ``correct``; each also carries its source.
    """
    srcK = np.asarray(K0, dtype=np.float64)
    srcV = np.asarray(V0, dtype=np.float64)
    res = []
    for ed in edges:
        out = correct(srcK, srcV, ed["desc"], ed["U"], ed["W"], tau, dtype,
                      K_fb=ed.get("K_fb"), V_fb=ed.get("V_fb"), q=ed.get("q"))
        out["K_src"], out["V_src"] = srcK, srcV
        res.append(out)
        srcK, srcV = out["K_out"], out["V_out"]
    return res


def fanout(K, V, targets, tau, dtype) -> list:
    """Non-chained correction: every agent corrects the same context-free reference cache.

    Fig. 3 and Fig. 6 / Table 9 of the listing compare chained correction (the source is the
    preceding agent's cache) with non-chained correction, whose source is a context-free
    reference cache of the shared context.  Reading: agent j's cache is that reference
    corrected with agent j's own anchors, exactly as in ``correct``; the reference itself
    is never modified, and every agent matches the same pooled descriptor.  ``targets`` is
    a list of dicts with keys desc, U, W and optionally K_fb, V_fb.  Returns the per-agent
    outputs of ``correct``.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    return [correct(K, V, t["desc"], t["U"], t["W"], tau, dtype,
                    K_fb=t.get("K_fb"), V_fb=t.get("V_fb")) for t in targets]


# --------------------------------------------------------------------------------------
# online anchor pool
# --------------------------------------------------------------------------------------


def select_anchors(s, count, A: int):
    """Top-A anchors of a segment's pool by cosine, for pools holding ``count`` valid slots.

    Table 13 of the listing varies the capacity V of the online anchor pool (V = 10 in the
    main setting).  Reading: the segment's current representation is scored against every
    valid slot (``cosine_scores``); the A best slots (ties to the lower slot; a NaN score
    ranks below every number) are combined with softmax weights over their scores; the
    reliability score is the best valid score.  With fewer than A valid slots the unused
    positions carry weight 0 and repeat the best slot.  An empty pool has score -inf, so the
    segment falls back.  s: [..., V]; count: [...] int.  Returns (slots int [..., A],
    w [..., A], score [...]).
    """
    s = np.asarray(s, dtype=np.float64)
    count = np.asarray(count)
    lead = s.shape[:-1]
    flat = s.reshape(-1, s.shape[-1])
    cnt = count.reshape(-1)
    slots = np.zeros((flat.shape[0], A), dtype=np.int64)
    w = np.zeros((flat.shape[0], A))
    score = np.full(flat.shape[0], -np.inf)
    for i, row in enumerate(flat):
        n = int(cnt[i])
        if n <= 0:
            continue
        # rank by score descending, NaN last, ties by slot index (a stable sort)
        key = np.where(np.isnan(row[:n]), np.inf, -row[:n])
        order = np.argsort(key, kind="stable")
        take = order[: min(A, n)]
        slots[i, : len(take)] = take
        slots[i, len(take):] = take[0]
        sel = row[take]
        w[i, : len(take)] = softmax_weights(sel)
        score[i] = np.nan if np.isnan(row[:n]).any() else np.max(row[:n])
    return slots.reshape(lead + (A,)), w.reshape(lead + (A,)), score.reshape(lead)


def correct_pooled(K, V, anchor_pool: dict, A: int, tau, dtype, K_fb=None, V_fb=None) -> dict:
    """Correction of a reused cache from each segment's online anchor pool.

    ``anchor_pool``: desc [L, H, V, 2d], U [2, L, H, V, T, r], W [2, L, H, V, r, d], count [L, H].
    Every segment is matched against its valid slots (``select_anchors``) and corrected with
    the weighted sum of its selected anchors' low-rank deltas, or falls back, as in
    ``correct``; the result is stored once in ``dtype``.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    U = np.asarray(anchor_pool["U"], dtype=np.float64)
    W = np.asarray(anchor_pool["W"], dtype=np.float64)
    q = pool(K, V)
    s = cosine_scores(q, anchor_pool["desc"])
    slots, w, score = select_anchors(s, anchor_pool["count"], A)
    mask = (~(score >= np.float64(tau))).astype(np.uint8)
    L, H = K.shape[:2]
    outs = []
    for x, (X, X_fb) in enumerate(((K, K_fb), (V, V_fb))):
        out = np.array(X, copy=True)
        for l in range(L):
            for h in range(H):
                if mask[l, h]:
                    if X_fb is not None:
                        out[l, h] = np.asarray(X_fb, dtype=np.float64)[l, h]
                    continue
                delta = np.zeros_like(X[l, h])
                for a in range(A):
                    j = slots[l, h, a]
                    delta += w[l, h, a] * (U[x, l, h, j] @ W[x, l, h, j])
                out[l, h] = X[l, h] + delta
        outs.append(out)
    return {"K_exact": outs[0], "V_exact": outs[1],
            "K_out": round_to_dtype(outs[0], dtype), "V_out": round_to_dtype(outs[1], dtype),
            "q": q, "s": s, "slots": slots, "w": w, "score": score, "mask": mask}


def pool_insert(pool_state: dict, mask, U_new, W_new, q, dtype) -> dict:
    """Insert a new online anchor into the pool of every segment where ``mask`` is set.

    After a fallback the dense prefill yields the exact cache, so the deviation of the
    reused cache is observed and becomes a new anchor of that shared segment.  Reading
    (the pages give no insertion or eviction rule): the anchor's factors are the rank-r fit
    of delta = exact - reused (``fit_anchor``), stored once in the cache ``dtype``; its
    descriptor is the pooled descriptor q of the reused cache; it goes to the slot after the
    last one written (first-in first-out), replacing the oldest anchor once the pool holds
    V.  pool_state: desc [L,H,V,2d], U [2,L,H,V,T,r], W [2,L,H,V,r,d], count [L,H],
    head [L,H] (next slot).  U_new [2,L,H,T,r], W_new [2,L,H,r,d], q [L,H,2d].
    Returns a new state; the input is not modified.
    """
    st = {k: np.array(v, copy=True) for k, v in pool_state.items()}
    Vc = st["desc"].shape[2]
    mask = np.asarray(mask)
    L, H = mask.shape
    for l in range(L):
        for h in range(H):
            if not mask[l, h]:
                continue
            j = int(st["head"][l, h])
            st["U"][:, l, h, j] = round_to_dtype(np.asarray(U_new)[:, l, h], dtype)
            st["W"][:, l, h, j] = round_to_dtype(np.asarray(W_new)[:, l, h], dtype)
            st["desc"][l, h, j] = round_to_dtype(np.asarray(q)[l, h], "f32")  # float32 pool
            st["head"][l, h] = (j + 1) % Vc
            st["count"][l, h] = min(int(st["count"][l, h]) + 1, Vc)
    return st


# --------------------------------------------------------------------------------------
# anchor fit
# --------------------------------------------------------------------------------------


def effective_rank(lam, energy: float = 0.9) -> np.ndarray:
    """Smallest k >= 1 whose top-k eigenvalues hold at least ``energy`` of the total.

    Figs. 2 and 7(a): effective rank is the minimum rank that retains 90% of the
    singular-value energy.  Reading: energy of singular value sigma_i is sigma_i^2 = lambda_i
    (eigenvalue of delta^T delta), summed over all of them; values are sorted descending and
    negative round-off is clamped to 0; a zero matrix has effective rank 0.  The running
    sum and the comparison are float64.  ``lam``: [..., n]; returns int32 [...].
    """
    lam = np.asarray(lam, dtype=np.float64)
    lam = np.clip(-np.sort(-lam, axis=-1), 0.0, None)
    flat = lam.reshape(-1, lam.shape[-1])
    out = np.zeros(flat.shape[0], dtype=np.int32)
    for i, row in enumerate(flat):
        total = 0.0
        for v in row:
            total += v
        if total == 0.0:
            continue
        need = energy * total
        run = 0.0
        for k, v in enumerate(row, start=1):
            run += v
            if run >= need:
                out[i] = k
                break
        else:
            out[i] = row.shape[0]
    return out.reshape(lam.shape[:-1])


def _canonical_rows(Wr: np.ndarray) -> np.ndarray:
    """Flip each row so that its largest-magnitude entry (first one on ties) is positive."""
    Wr = np.array(Wr, copy=True)
    for i in range(Wr.shape[0]):
        j = int(np.argmax(np.abs(Wr[i])))
        if Wr[i, j] < 0:
            Wr[i] = -Wr[i]
    return Wr


def fit_anchor(delta, r: int, energy: float = 0.9) -> dict:
    """Rank-r anchor of a cache delta: the truncated SVD written out.

    delta = exact - reused (one [T, d] matrix per (K|V, layer, head)).  The compact
    low-rank state of the abstract is read as the best rank-r approximation of delta
    (Eckart-Young), with r = r_delta = 32 by default (Fig. 13 caption); its eigenvalues
    lambda_i = sigma_i^2 give the effective rank (Figs. 2, 7).  Factors:
        W = top-r right singular vectors as rows (orthonormal), each row's
            largest-magnitude entry made positive;
        U = delta W^T, so U W is the truncation and U's columns carry sigma.
    delta: [M, T, d].  Returns U [M, T, r], W [M, r, d], k_eff int32 [M],
    eig [M, d] (descending, zero-padded when T < d).
    """
    delta = np.asarray(delta, dtype=np.float64)
    M, T, d = delta.shape
    U = np.zeros((M, T, r))
    W = np.zeros((M, r, d))
    eig = np.zeros((M, d))
    for m in range(M):
        if T == 0:
            continue
        _, sv, vt = np.linalg.svd(delta[m], full_matrices=False)
        k = sv.shape[0]
        eig[m, :k] = sv * sv
        rr = min(r, k)
        W[m, :rr] = _canonical_rows(vt[:rr])
        U[m] = delta[m] @ W[m].T
    return {"U": U, "W": W, "k_eff": effective_rank(eig, energy), "eig": eig}


def gram(delta) -> np.ndarray:
    """G = delta^T delta per matrix, float64: the Gram matrix whose eigen-decomposition gives
    the anchor (lambda_i = sigma_i^2).  Rows appended to delta add their own Gram matrix:
    gram(concat(D1, D2)) = gram(D1) + gram(D2), which is what lets the fit follow a
    growing shared context (abstract: dynamically changing context; Figs. 10-11).
    delta: [M, T, d] -> [M, d, d]."""
    delta = np.asarray(delta, dtype=np.float64)
    return np.einsum("mti,mtj->mij", delta, delta)


def fit_from_gram(G, r: int, energy: float = 0.9) -> dict:
    """The anchor's W, effective rank and eigenvalues from an accumulated Gram matrix:
    the symmetric eigen-decomposition of G written out (eigenvalues descending, negative
    round-off clamped to 0; W = the top-r eigenvectors as rows, each row's
    largest-magnitude entry positive; k_eff as in effective_rank).  G: [M, d, d]."""
    G = np.asarray(G, dtype=np.float64)
    M, d, _ = G.shape
    W = np.zeros((M, r, d))
    eig = np.zeros((M, d))
    for m in range(M):
        lam, vec = np.linalg.eigh(0.5 * (G[m] + G[m].T))
        order = np.argsort(-lam, kind="stable")
        eig[m] = np.clip(lam[order], 0.0, None)
        W[m] = _canonical_rows(vec[:, order[:r]].T)
    return {"W": W, "k_eff": effective_rank(eig, energy), "eig": eig}


def project(delta, W) -> np.ndarray:
    """U = delta W^T for any block of rows: the anchor's row factor.  delta [M, T, d],
    W [M, r, d] -> [M, T, r]."""
    delta = np.asarray(delta, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return np.einsum("mtd,mrd->mtr", delta, W)


# --------------------------------------------------------------------------------------
# metrics
# --------------------------------------------------------------------------------------


def rel_frobenius(x, ref) -> float:
    """||x - ref||_F / ||ref||_F: the error normalised by the target (Fig. 3 caption)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def segment_error(X, ref):
    """Per-segment sums of the Fig. 3 error: (sum (X - ref)^2, sum ref^2) over the tokens and
    channels of every (layer, kv-head) segment, float64.  X, ref: [L, H, T, d] ->
    two [L, H] arrays.  Fig. 3 normalises the reconstruction error by the Frobenius norm of
    the target (the exact cache from full prefill); per-layer (Fig. 3(a)) and per-agent
    (Fig. 3(b)) errors are square roots of ratios of sums of these."""
    X = np.asarray(X, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = X - ref
    return (diff * diff).sum(axis=(-2, -1)), (ref * ref).sum(axis=(-2, -1))


def layer_error(err_sq, ref_sq) -> np.ndarray:
    """Relative error of every layer, sqrt(sum_h err / sum_h ref) (Fig. 3(a)); inputs [L, H]."""
    num = np.asarray(err_sq, dtype=np.float64).sum(axis=-1)
    den = np.asarray(ref_sq, dtype=np.float64).sum(axis=-1)
    return np.sqrt(num / np.where(den > 0, den, 1.0))


def rank_error_curve(eig) -> np.ndarray:
    """Relative reconstruction error of the best rank-k approximation for k = 0..n (Fig. 7(b):
    the error as the retained rank grows).  By Eckart-Young the rank-k truncation of delta
    leaves exactly the singular values past k, so the error normalised by ||delta||_F is
    sqrt(sum_{i > k} lambda_i / sum_i lambda_i) with lambda = sigma^2 sorted descending and
    negative round-off clamped to 0; a zero matrix gives 0 at every k.
    eig: [..., n] -> [..., n + 1]."""
    lam = np.asarray(eig, dtype=np.float64)
    lam = np.clip(-np.sort(-lam, axis=-1), 0.0, None)
    n = lam.shape[-1]
    flat = lam.reshape(-1, n)
    out = np.zeros((flat.shape[0], n + 1))
    for i, row in enumerate(flat):
        total = 0.0
        for v in row:
            total += v
        if total == 0.0:
            continue
        tail = 0.0  # sum_{i >= k} lambda_i, added from the smallest eigenvalue up
        for k in range(n, -1, -1):
            if k < n:
                tail += row[k]
            out[i, k] = np.sqrt(tail / total)
    return out.reshape(lam.shape[:-1] + (n + 1,))
