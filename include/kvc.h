/*
 * kvc.h -- C ABI of the MI355X (gfx950) library for KVCMAS's online KV-cache correction.
 *
 * Method: "KVCMAS: Efficient KV cache Correction for Shared Context in Multi-Agent
 * Systems" (arXiv:2609.34060).  Fig. 1 of the thelatestinai listing: a shared-context
 * (PH) segment's cache, reused from the preceding agent, is matched against the segment's
 * online anchors; their low-rank corrections are combined with similarity-based weights;
 * an unreliable segment falls back to dense prefill; the corrected cache becomes the next
 * workflow edge's reference (chaining).  Figs. 2 and 7 define the effective rank at 90% of
 * the singular-value energy; Fig. 13 sets the delta rank (default 32).
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers (HIP global memory), dense, row-major,
 *    with the shapes given below.  The caller owns every buffer, including the workspace;
 *    the library allocates nothing and keeps no state between calls.
 *  - Caches K, V (and fallbacks, outputs): [L, H, T, d] = (layer, kv-head, token,
 *    channel).  One (l, h) pair is a segment; S = L*H.
 *  - dtype: KVC_BF16 (bfloat16) or KVC_F32 (float32) for caches, anchor factors and the
 *    fit input.  Descriptors, weights and fit outputs are float32.
 *  - d must be 64 or 128.  Sizes are int; every element count must fit in 2^62.
 *  - Pointers to caches, factors and float outputs must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work
 *    on it and return; results are valid once the stream has been synchronised.
 *  - Arguments are validated before any HIP call: a bad argument returns KVC_ERR_ARG
 *    (or KVC_ERR_UNSUPPORTED, KVC_ERR_WORKSPACE) and enqueues nothing.  A failing HIP
 *    launch returns KVC_ERR_HIP.  kvc_last_error() then describes the failure.
 *  - Calls that overlap in time on different streams must not share a workspace.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KVC_BF16 = 0, KVC_F32 = 1 } kvc_dtype;

typedef enum {
    KVC_OK = 0,
    KVC_ERR_ARG = 1,         /* null / misaligned pointer, negative size, bad shape    */
    KVC_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement           */
    KVC_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed             */
    KVC_ERR_WORKSPACE = 4    /* workspace pointer null or smaller than required        */
} kvc_status;

/* Library version string, static storage. */
const char* kvc_version(void);

/* Message for the last non-OK status returned on the calling thread (thread-local,
 * valid until that thread's next call); "" if none. */
const char* kvc_last_error(void);


/* ---------------------------------------------------------------------------------------
 * Pooled descriptor (Fig. 1(b): the current cache representation that is matched
 * against the online anchors).  Read here as the token mean of K followed by the token
 * mean of V:  q[l,h,0:d] = (1/T) sum_t K[l,h,t,:],  q[l,h,d:2d] = (1/T) sum_t V[l,h,t,:].
 * T = 0 gives q = 0.  Summation is float32 in a fixed order (deterministic).
 *   K, V   : [L,H,T,d] dtype, read only
 *   q_out  : [L,H,2d] float32, written
 *   ws     : workspace of at least kvc_pool_workspace_bytes(L,H,T,d) bytes
 * ------------------------------------------------------------------------------------- */
size_t kvc_pool_workspace_bytes(int L, int H, int T, int d);
kvc_status kvc_pool_descriptor(const void* K, const void* V, int L, int H, int T, int d,
                               int dtype, float* q_out, void* ws, size_t ws_bytes,
                               void* stream);

/* ---------------------------------------------------------------------------------------
 * Correction of a reused shared-context cache (Figs. 1(a), 1(b); the abstract's compact
 * low-rank states).  Per segment (l,h), with q the pooled descriptor of (K, V):
 *   s_a   = cos(q, desc[l,h,a])  (0 if either vector is zero)          a = 0..A-1
 *   w     = softmax(s)           (temperature 1)
 *   score = max_a s_a;  fallback = !(score >= tau)   (float32 compare; NaN falls back)
 *   reliable segment:  X' = X + sum_a w_a U[x,l,h,a] W[x,l,h,a]   for X in {K, V}
 *                      (x = 0 for K, 1 for V; products accumulated in float32 and the
 *                      sum stored once in dtype, round-to-nearest-even)
 *   fallback segment:  X' = X_fb (dense-prefill stand-in) if given, else X, bit exact;
 *                      U and W are not read.
 *   K, V        : [L,H,T,d] dtype                      (source cache, read only)
 *   desc        : [L,H,A,2d] float32                   (anchor descriptors)
 *   U           : [2,L,H,A,T,r] dtype                  (left factors, index 0 = K)
 *   W           : [2,L,H,A,r,d] dtype                  (right factors)
 *   A, r        : 1 <= A, 1 <= r <= d, A * r <= 256 (shapes outside the specialised
 *                 kernel's budget -- bf16: A <= 16, r <= 64, A * ceil(r/16)*16 <= 256; fp32:
 *                 A * ceil(r/8)*8 <= 64 -- run as a separate pooling, matching and general
 *                 correction pass; results meet the same bars)
 *   tau         : reliability threshold (+inf: every segment falls back; -inf: none)
 *   q_in        : [L,H,2d] float32 or NULL: a precomputed pooled descriptor of (K, V);
 *                 when NULL a pooling pass computes it first (bit-identical to the q that
 *                 kvc_pool_descriptor returns); then one matching and one correction launch
 *   K_fb, V_fb  : [L,H,T,d] dtype or NULL (both or neither)
 *   K_out, V_out: [L,H,T,d] dtype, written; may equal K / V (in place); must not
 *                 otherwise overlap any input
 *   mask_out    : [L,H] uint8, 1 = fall back, 0 = corrected, written
 *   score_out   : [L,H] float32 or NULL;  w_out: [L,H,A] float32 or NULL
 *   q_next_out  : [L,H,2d] float32 or NULL: pooled descriptor of (K_out, V_out)
 *   ws          : at least kvc_correct_workspace_bytes(L,H,T,d,A,r) bytes
 * ------------------------------------------------------------------------------------- */
size_t kvc_correct_workspace_bytes(int L, int H, int T, int d, int A, int r);
kvc_status kvc_correct(const void* K, const void* V, int L, int H, int T, int d, int dtype,
                       const float* desc, const void* U, const void* W, int A, int r,
                       float tau, const float* q_in, const void* K_fb, const void* V_fb,
                       void* K_out, void* V_out, uint8_t* mask_out, float* score_out,
                       float* w_out, float* q_next_out, void* ws, size_t ws_bytes,
                       void* stream);

/* ---------------------------------------------------------------------------------------
 * kvc_correct for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments, computation and
 * outputs as kvc_correct, except that the workspace is a library-owned device array of
 * KVC_SCRATCH_BYTES (16 MiB) instead of a caller-provided one.  The call allocates nothing.
 *   - Limit: shapes whose kvc_correct_workspace_bytes(L,H,T,d,A,r) exceeds KVC_SCRATCH_BYTES
 *     return KVC_ERR_UNSUPPORTED before any HIP call (e.g. 32 x 8 x 2048 x 128 with A = 4
 *     needs about 8.7 MiB and fits; the same cache at T = 8192 does not).
 *   - Each device has its own array, kept until the process ends; its address is looked up
 *     on the first call made with that device current.
 *   - Every call on a device shares that device's array and its contents from the last
 *     call (the kernels re-initialise everything they read).  Calls that overlap on one
 *     device (two streams, or two host threads, without ordering between them) race on it:
 *     the caller must order them.
 * ------------------------------------------------------------------------------------- */
#define KVC_SCRATCH_BYTES (16u << 20)
kvc_status kvc_correct_noalloc(const void* K, const void* V, int L, int H, int T, int d,
                               int dtype, const float* desc, const void* U, const void* W, int A,
                               int r, float tau, const float* q_in, const void* K_fb,
                               const void* V_fb, void* K_out, void* V_out, uint8_t* mask_out,
                               float* score_out, float* w_out, float* q_next_out,
                               void* stream);

/* ---------------------------------------------------------------------------------------
 * Rank-rC representation of a cache (Fig. 13: the base cache is kept at rank r_C, 32 by
 * default; Fig. 2: the effective rank of the base cache).  Per segment and for X in {K, V}:
 * the rank-rC truncation of X^T X, stored as F = diag(sigma_1..rC) V_rC^T (the top rC right
 * singular vectors of X scaled by the singular values; each row's largest-magnitude entry
 * positive), computed with kvc_fit_anchor's Gram and eigensolver kernels.
 *   K, V      : [L,H,T,d] dtype
 *   rC        : 1 <= rC <= d
 *   F_out     : [2,L,H,rC,d] float32 (index 0 = K), written
 *   k_eff_out : [2,L,H] int32 or NULL: the effective rank at 90% energy (exact, as for
 *               kvc_fit_anchor)
 *   ws        : at least kvc_rank_descriptor_workspace_bytes(L,H,T,d,rC) bytes
 * ------------------------------------------------------------------------------------- */
size_t kvc_rank_descriptor_workspace_bytes(int L, int H, int T, int d, int rC);
kvc_status kvc_rank_descriptor(const void* K, const void* V, int L, int H, int T, int d,
                               int dtype, int rC, float* F_out, int32_t* k_eff_out, void* ws,
                               size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * kvc_correct with the anchors matched on rank-rC representations instead of the mean-pooled
 * descriptor (Fig. 1(b) matching of the cache representation; Fig. 13 rank r_C):
 *   s_a = (<Gq_K, Ga_K> + <Gq_V, Ga_V>) / (||(Gq_K, Gq_V)|| ||(Ga_K, Ga_V)||)
 * with G = F^T F and <G, G'> = ||F F'^T||_F^2 (0 when either norm is 0): the cosine of the
 * truncated second-moment matrices, independent of the signs and rotations of the factor
 * rows.  Softmax weights, score, fallback and correction as in kvc_correct.
 *   Fq : [2,L,H,rC,d] float32, the source cache's representation (kvc_rank_descriptor)
 *   Fa : [2,L,H,A,rC,d] float32, the anchors' representations
 *   other arguments and the workspace (kvc_correct_workspace_bytes) as for kvc_correct
 * ------------------------------------------------------------------------------------- */
kvc_status kvc_correct_rank(const void* K, const void* V, int L, int H, int T, int d, int dtype,
                            const float* Fq, const float* Fa, int rC, const void* U,
                            const void* W, int A, int r, float tau, const void* K_fb,
                            const void* V_fb, void* K_out, void* V_out, uint8_t* mask_out,
                            float* score_out, float* w_out, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------------------
 * Chained correction along a workflow A0 -> A1 -> ... (Fig. 1(c); Fig. 3(b): A0's cache
 * is exact).  Edge e corrects its source with its own anchors; the stored result is the
 * source of edge e+1; edge 0's source is (K0, V0), which is not modified.  The pooled
 * descriptor of every edge >= 1 is taken from the previous edge's output pass, so each
 * source is read from memory once.
 *   n_edges >= 1.  Every array below is a HOST array of n_edges DEVICE pointers, laid
 *   out as for kvc_correct: desc[e], U[e], W[e], K_out[e], V_out[e], mask_out[e]
 *   required; K_fb / V_fb (the array itself or an entry, both or neither per edge) and
 *   score_out may be NULL.  K_out[e] must not overlap K_out[e-1] or the edge's inputs.
 *   ws: at least kvc_chain_workspace_bytes(L,H,T,d,A,r) bytes.
 * ------------------------------------------------------------------------------------- */
size_t kvc_chain_workspace_bytes(int L, int H, int T, int d, int A, int r);
kvc_status kvc_correct_chain(const void* K0, const void* V0, int L, int H, int T, int d,
                             int dtype, int n_edges, const float* const* desc,
                             const void* const* U, const void* const* W, int A, int r,
                             float tau, const void* const* K_fb, const void* const* V_fb,
                             void* const* K_out, void* const* V_out,
                             uint8_t* const* mask_out, float* const* score_out, void* ws,
                             size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Non-chained correction (Fig. 3 and Fig. 6 / Table 9 of the listing: each agent corrects a
 * context-free reference cache of the shared context instead of the preceding agent's
 * cache).  One reference (K, V), n_agents targets: agent j's output is exactly what
 * kvc_correct(K, V, desc[j], U[j], W[j], ...) stores, and its mask, score and weights are
 * the same.  The reference is pooled once (every agent is matched against the same pooled
 * descriptor, bit for bit); then one correction launch per group of up to 8 agents reads
 * each tile of the reference once and corrects it for every agent of the group (a single
 * agent is exactly kvc_correct; anchor shapes outside the specialised kernel are corrected
 * agent by agent).  The same call serves one agent whose cache feeds several successors on a
 * workflow graph.
 *   n_agents >= 1.  desc, U, W, K_out, V_out, mask_out: HOST arrays of n_agents DEVICE
 *   pointers laid out as for kvc_correct; K_fb / V_fb (the array or an entry, both or
 *   neither per agent) and score_out may be NULL.  No output may overlap the reference or
 *   another output (KVC_ERR_ARG).  (K, V) are read only.
 *   ws: at least kvc_fanout_workspace_bytes(L,H,T,d,A,r) bytes.
 * ------------------------------------------------------------------------------------- */
size_t kvc_fanout_workspace_bytes(int L, int H, int T, int d, int A, int r);
kvc_status kvc_correct_fanout(const void* K, const void* V, int L, int H, int T, int d,
                              int dtype, int n_agents, const float* const* desc,
                              const void* const* U, const void* const* W, int A, int r,
                              float tau, const void* const* K_fb, const void* const* V_fb,
                              void* const* K_out, void* const* V_out,
                              uint8_t* const* mask_out, float* const* score_out, void* ws,
                              size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Online anchor pool (Table 13 of the listing varies the capacity V of each shared segment's
 * pool of online anchors; V = 10 in the main setting).  The pages give no insertion,
 * eviction or selection rule; this library reads them as follows.
 *
 * kvc_correct_pooled: kvc_correct against each segment's pool.  Per segment the first
 * count[l,h] of the Vc slots are valid; each valid slot v is scored s_v = cos(q, desc[v]);
 * the A best valid slots are selected (a NaN ranks last, ties go to the lower slot) and
 * combined with softmax weights over their scores; score = the best valid score (NaN if any
 * valid score is NaN, -inf for an empty pool, which therefore falls back); fallback =
 * !(score >= tau).  With fewer than A valid slots the unused positions repeat the best slot
 * with weight 0 (valid slots must hold finite factors).  Corrected output, fallback and
 * rounding as in kvc_correct.  Pooling, matching and correction run as three launches (the
 * pool is read after the query is known).
 *   desc_pool : [L,H,Vc,2d] float32;  U_pool: [2,L,H,Vc,T,r] dtype;  W_pool: [2,L,H,Vc,r,d]
 *   count     : [L,H] int32, valid slots per segment (clamped to [0, Vc] on the device)
 *   Vc, A     : 1 <= A <= Vc <= 32; A and r as for kvc_correct
 *   q_in      : as for kvc_correct (NULL: pooled here)
 *   w_out     : [L,H,A] float32 or NULL;  slot_out: [L,H,A] int32 or NULL (selected slots)
 *   other arguments as for kvc_correct (no q_next_out)
 *   ws        : at least kvc_correct_pooled_workspace_bytes(L,H,T,d,A,r) bytes
 *
 * kvc_anchor_pool_insert: after a fallback, the dense prefill gives the exact cache, so the
 * deviation delta = exact - reused of that segment is observed; its rank-r fit
 * (kvc_fit_anchor on the [2*L*H, T, d] delta: K matrices, then V) becomes a new anchor.  For
 * every segment with mask[l,h] != 0 the slot head[l,h] receives U_new and W_new (stored in
 * the cache dtype, round to nearest even) and the descriptor q[l,h] (the pooled descriptor
 * of the reused cache, as matched); then head advances by one slot modulo Vc (first in,
 * first out: the oldest anchor is replaced once the pool is full) and count grows up to Vc.
 *   mask  : [L,H] uint8;  U_new: [2,L,H,T,r] float32;  W_new: [2,L,H,r,d] float32
 *   q     : [L,H,2d] float32
 *   U_pool, W_pool, desc_pool: as above, updated in place
 *   count, head: [L,H] int32, updated in place (start both at 0; a head outside [0, Vc)
 *           is treated as 0)
 *   1 <= Vc <= 32, 1 <= r <= d.  No workspace.
 * ------------------------------------------------------------------------------------- */
size_t kvc_correct_pooled_workspace_bytes(int L, int H, int T, int d, int A, int r);
kvc_status kvc_correct_pooled(const void* K, const void* V, int L, int H, int T, int d,
                              int dtype, const float* desc_pool, const void* U_pool,
                              const void* W_pool, const int32_t* count, int Vc, int A, int r,
                              float tau, const float* q_in, const void* K_fb, const void* V_fb,
                              void* K_out, void* V_out, uint8_t* mask_out, float* score_out,
                              float* w_out, int32_t* slot_out, void* ws, size_t ws_bytes,
                              void* stream);
kvc_status kvc_anchor_pool_insert(const uint8_t* mask, const float* U_new, const float* W_new,
                                  const float* q, int L, int H, int T, int d, int dtype, int Vc,
                                  int r, void* U_pool, void* W_pool, float* desc_pool,
                                  int32_t* count, int32_t* head, void* stream);

/* ---------------------------------------------------------------------------------------
 * Error measures of the studies.
 *
 * kvc_segment_error: Fig. 3 of the listing reports the reconstruction error of a cache
 * normalised by the Frobenius norm of the target (the exact cache from full prefill), per
 * layer (a) and per agent (b).  This call returns, per segment, the two sums those ratios
 * are made of:  out[l,h,0] = sum_{t,c} (X - ref)^2,  out[l,h,1] = sum_{t,c} ref^2,  summed
 * in float64 (the differences of the widened inputs are exact) in a fixed order.
 *   X, ref : [L,H,T,d] dtype, read only;  out: [L,H,2] float64 (8-byte aligned), written
 *   ws     : at least kvc_segment_error_workspace_bytes(L,H,T,d) bytes, 256-byte aligned
 *
 * kvc_rank_error_curve: Fig. 7(b) reports the relative reconstruction error as the
 * retained rank grows.  The best rank-k approximation of delta leaves the singular values
 * past k (Eckart-Young), so from the eigenvalues lambda = sigma^2 of delta^T delta:
 *   curve[m,k] = sqrt( sum_{i>=k} lambda[m,i] / sum_i lambda[m,i] ),  k = 0..n,
 * float64 sums (the tail added from the smallest eigenvalue up); negative entries count as
 * 0; a zero total gives 0 at every k.
 *   eig      : [M,n] float32, sorted descending (as kvc_fit_anchor's eig_out); the order
 *              is not checked;  1 <= n <= 256
 *   curve_out: [M,n+1] float32, written
 * ------------------------------------------------------------------------------------- */
size_t kvc_segment_error_workspace_bytes(int L, int H, int T, int d);
kvc_status kvc_segment_error(const void* X, const void* ref, int L, int H, int T, int d,
                             int dtype, double* out, void* ws, size_t ws_bytes, void* stream);
kvc_status kvc_rank_error_curve(const float* eig, int M, int n, float* curve_out, void* stream);

/* ---------------------------------------------------------------------------------------
 * Rank-r anchor fit of a cache delta (delta = exact - reused, one [T,d] matrix per
 * (K|V, layer, head)).  The anchor is the best rank-r approximation U W of delta (the
 * compact low-rank state of the abstract; r = r_delta of Fig. 13), computed as
 *   G = delta^T delta (float32 accumulation of exact bf16 products, fixed order),
 *   G = Q diag(lambda) Q^T, lambda sorted descending: for r <= 32 by Householder
 *     tridiagonalisation (float64), multisection for the eigenvalues (float32) and inverse
 *     iteration for the r vectors (float64); for r > 32 by one-sided Jacobi (float32),
 *   W = first r columns of Q, as rows, each row's largest-|.| entry positive,
 *   U = delta W^T (float32 accumulation),
 * and the effective rank k = min{k >= 1 : sum_{i<k} lambda_i >= energy * total} with
 * total = sum lambda = trace G = ||delta||_F^2 (0 for a zero delta), the running sum and
 * compare in float64 (Figs. 2, 7(a)).  k is exact (the value the exact eigenvalues of
 * delta^T delta give, up to float64 rounding): the fast path keeps its k only when both
 * running sums around the threshold clear a stated bound on its own error (float32 Gram
 * sums, float32 eigenvalue brackets, float64 reduction); otherwise a float64 pass (Gram
 * from delta in float64, Householder, multisection to float64 resolution) decides it.
 *   delta    : [M,T,d] dtype, read only
 *   r        : 1 <= r <= d
 *   energy   : in (0, 1], 0.9 in the pages
 *   U_out    : [M,T,r] float32;  W_out: [M,r,d] float32;  k_eff_out: [M] int32
 *   eig_out  : [M,d] float32 (lambda, descending) or NULL
 *   ws       : at least kvc_fit_workspace_bytes(M,T,d,r) bytes
 * ------------------------------------------------------------------------------------- */
size_t kvc_fit_workspace_bytes(int M, int T, int d, int r);
kvc_status kvc_fit_anchor(const void* delta, int M, int T, int d, int dtype, int r,
                          double energy, float* U_out, float* W_out, int32_t* k_eff_out,
                          float* eig_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Streaming fit for a growing shared context (the dynamically changing context of the
 * abstract; generated tokens accumulating over turns, listing Figs. 10-11): the Gram matrix
 * of a delta is accumulated block by block as rows are appended, and the anchor is refit
 * from it.  With G accumulated over all rows of delta, kvc_fit_from_gram + kvc_project give
 * the same W, k_eff and U as kvc_fit_anchor (bit for bit for r <= 32 when delta was
 * accumulated in one call onto G = 0).
 *
 * kvc_gram_accumulate: G += delta^T delta for a block of rows.
 *   delta   : [M,T,d] dtype, read only (the appended rows; T = 0 leaves G unchanged)
 *   G_inout : [M,d,d] float64, full symmetric, 8-byte aligned; the caller zeroes it first
 *             (products of the inputs are exact, summed in float32 per split of T, the
 *             splits in a fixed order in float64); the upper triangle is read and the sum
 *             written to both triangles (the lower triangle on entry is not read)
 *   ws      : at least kvc_gram_workspace_bytes(M,T,d) bytes, 256-byte aligned
 * kvc_fit_from_gram: eigen-decomposition of G and the factors of kvc_fit_anchor.
 *   G       : [M,d,d] float64 as accumulated; r, energy, W_out, k_eff_out, eig_out as in
 *             kvc_fit_anchor (no workspace)
 * kvc_project: U = delta W^T for any block of rows (e.g. only the appended ones).
 *   W       : [M,r,d] float32 (from kvc_fit_from_gram or kvc_fit_anchor)
 *   U_out   : [M,T,r] float32
 *   ws      : kvc_project_workspace_bytes(M,d,r,dtype) bytes (0 for both dtypes: NULL ok)
 * Errors as for kvc_fit_anchor; nothing is enqueued when validation fails.
 * ------------------------------------------------------------------------------------- */
size_t kvc_gram_workspace_bytes(int M, int T, int d);
kvc_status kvc_gram_accumulate(const void* delta, int M, int T, int d, int dtype,
                               double* G_inout, void* ws, size_t ws_bytes, void* stream);
kvc_status kvc_fit_from_gram(const double* G, int M, int d, int r, double energy, float* W_out,
                             int32_t* k_eff_out, float* eig_out, void* stream);
size_t kvc_project_workspace_bytes(int M, int d, int r, int dtype);
kvc_status kvc_project(const void* delta, int M, int T, int d, int dtype, const float* W, int r,
                       float* U_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Warm-started refit for the growing context (same passages as the streaming fit): after
 * rows were appended and G accumulated, the new anchor is found starting from the previous
 * W instead of from scratch.  Results as kvc_fit_from_gram (W = the top-r eigenvectors of G
 * as rows with the canonical sign, k_eff exact for the given G), found by
 *   Q0 = [W_prev^T, 32 - r fixed directions orthogonal to it], then at most three passes of
 *   Z = G Q (first G Q0), Q = Cholesky-QR(Z), Rayleigh-Ritz on Q^T G Q (float64; 32 columns
 *   in the first pass, 48 in later ones);
 * the Ritz vectors are kept when each residual |G x - rho x| is within 2^-28 of the
 * Gershgorin bound of G and they are orthonormal to 1e-8, and k_eff is kept when the Ritz
 * values prove it (lower bound: Ky Fan; upper bound: the residual and the energy left outside
 * the Ritz block; k_eff <= r).  Every other matrix (no convergence, k_eff not proven or above
 * r, a zero G) is solved by the kvc_fit_from_gram path, so the outputs always meet that
 * contract; r > 32 takes that path for every matrix.  A matrix whose Ritz values cannot reach
 * the energy threshold, or whose residuals shrink too slowly for the passes left, is handed
 * over early.  The call pays off when the r wanted eigenvalues stand apart from the rest;
 * where no matrix converges it costs about 1.7-1.8 times kvc_fit_from_gram.
 *   G         : [M,d,d] float64 (lower triangle read), as for kvc_fit_from_gram
 *   W_prev    : [M,r,d] float32, the previous W (e.g. the last kvc_fit_from_gram or
 *               kvc_refit_warm output for the same r); any values are allowed: a poor start
 *               only sends the matrix to the full solve
 *   W_out     : [M,r,d] float32; may be the same buffer as W_prev (each matrix's W_prev is
 *               read before its W_out is written)
 *   k_eff_out : [M] int32
 *   warm_out  : [M] int32 or NULL: 1 where the warm result was kept, 0 where the full solve ran
 * No workspace.  Errors as for kvc_fit_from_gram.
 * ------------------------------------------------------------------------------------- */
kvc_status kvc_refit_warm(const double* G, int M, int d, int r, double energy,
                          const float* W_prev, float* W_out, int32_t* k_eff_out,
                          int32_t* warm_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
