// Internal definitions shared by the HIP translation units of libkvc (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

// ---------------------------------------------------------------- launch geometry
constexpr int kWave = 64;             // CDNA wavefront width
constexpr int kBlock = 256;           // 4 waves per workgroup everywhere
constexpr int kRowsPerPass = 128;     // tokens of one 32-token tile per wave, 4 waves
constexpr int kMaxA = 16;             // anchors per segment held in registers
constexpr int kMaxAnchorsGeneral = 256;  // A * r <= 256: the general correction's bound
constexpr int kMaxRankC = 128;        // rank of the cache representation (rank matching)
constexpr int kMaxKSlots = 256;       // A * ceil16(r) bound of the LDS-staged factors
constexpr int kMaxR = 64;             // rank bound of the correction kernel
constexpr int kMaxPool = 32;          // slots of an online anchor pool per segment
constexpr int kMaxTargets = 8;        // targets of one multi-target correction launch
constexpr int kJacobiMaxSweeps = 40;  // hard cap: every workgroup leaves the sweep loop
constexpr int kEigMaxR = 32;         // rank bound of the tridiagonal eigensolver route
constexpr int32_t kWarmMiss = INT32_MIN;  // k_eff mark: the warm refit left the matrix open

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Tiles of kRowsPerPass tokens per correction work item (and per pooled chunk): the item's
// share of X held in registers is 64 VGPRs per lane, i.e. 16 KB per wave.
constexpr int item_tiles_for(int row_bytes) {
  return row_bytes <= 128 ? 4 : (row_bytes <= 256 ? 2 : 1);
}
inline int chunk_tokens(int d, int dtype) {
  return kRowsPerPass * item_tiles_for(d * (dtype == KVC_BF16 ? 2 : 4));
}

// chunk sums per segment and per K|V (one all-zero chunk when T = 0)
inline int chunks_of(int T, int d, int dtype) {
  return T > 0 ? ceil_div(T, chunk_tokens(d, dtype)) : 1;
}
// the most chunks any dtype gives (workspace sizes do not depend on the dtype)
inline int max_chunks_of(int T) { return T > 0 ? ceil_div(T, kRowsPerPass) : 1; }

// ---------------------------------------------------------------- correction workspace
struct CorrectLayout {
  int S, T, d, A;
  int max_chunks;     // chunk sums per segment and per K|V, most any dtype needs
  size_t off_pool;    // float [2][S][n_chunks][d]   chunk sums of the source
  size_t off_next;    // float [2][S][n_chunks][d]   chunk sums of the output (pooled next)
  size_t off_w;       // float [S][A]
  size_t off_mask;    // uint8 [S]
  size_t off_ctr;     // int: work counter of the correction pass
  size_t off_slot;    // int [S][A]: pool slots of the selected anchors (pooled correction)
  size_t off_wmt;     // float [kMaxTargets][S][A]: weights of a multi-target launch
  size_t off_mmt;     // uint8 [kMaxTargets][S]: flags of a multi-target launch
  size_t off_q;       // float [S][2d]: pooled descriptors (general correction)
  size_t bytes;
};

inline CorrectLayout correct_layout(int L, int H, int T, int d, int A) {
  CorrectLayout c{};
  c.S = L * H;
  c.T = T;
  c.d = d;
  c.A = A;
  c.max_chunks = max_chunks_of(T);
  const size_t sums = sizeof(float) * 2ull * c.S * c.max_chunks * d;
  size_t o = 0;
  c.off_pool = o;  o = align_up(o + sums, 256);
  c.off_next = o;  o = align_up(o + sums, 256);
  c.off_w = o;     o = align_up(o + sizeof(float) * (size_t)c.S * A, 256);
  c.off_mask = o;  o = align_up(o + (size_t)c.S, 256);
  c.off_ctr = o;   o = align_up(o + sizeof(int), 256);
  c.off_slot = o;  o = align_up(o + sizeof(int) * (size_t)c.S * A, 256);
  c.off_wmt = o;   o = align_up(o + sizeof(float) * (size_t)kMaxTargets * c.S * A, 256);
  c.off_mmt = o;   o = align_up(o + (size_t)kMaxTargets * c.S, 256);
  c.off_q = o;     o = align_up(o + sizeof(float) * 2ull * c.S * d, 256);
  c.bytes = o;
  return c;
}

// Everything one correction launch needs (see launch_correct).
struct CorrectLaunch {
  const void* K;
  const void* V;
  int S, T, d, dtype;
  const void* U;
  const void* W;
  int A, r, rp;
  float* w_ws;              // weights (from launch_score / launch_select)
  const uint8_t* mask_ws;   // fallback flags (from launch_score / launch_select)
  const void* K_fb;
  const void* V_fb;
  void* K_out;
  void* V_out;
  float* next_partials;     // chunk sums of the output, or null
  int* ctr;                 // work counter, reset by launch_score / launch_select
  const int* slot_ws;       // pooled correction: [S][A] slots of Vc per segment, or null
  int Vc;
  int n_t;                  // multi-target correction: 0 (off) or the targets below (w_ws and
  const void* tU[kMaxTargets];  // mask_ws then hold n_t blocks of [S][A] weights / [S] flags)
  const void* tW[kMaxTargets];
  void* tK[kMaxTargets];
  void* tV[kMaxTargets];
  const void* tKfb[kMaxTargets];
  const void* tVfb[kMaxTargets];
};

// ---------------------------------------------------------------- fit workspace
struct FitLayout {
  int M, T, d, r;
  int rpad;         // r rounded up to 32 (rows of the bf16 hi/lo factor copies)
  int slab;         // rows staged per Gram iteration
  int nsplit;       // Gram partials per matrix
  int chunk;        // rows per Gram workgroup (multiple of slab)
  int nblk;         // upper-triangular 32x32 blocks of G
  size_t off_gram;  // double [M][nsplit][nblk][16][64]
  size_t off_whi;   // bf16 [M][rpad][d]
  size_t off_wlo;   // bf16 [M][rpad][d]
  size_t off_sweeps;// int [M]
  size_t bytes;
};

inline FitLayout fit_layout(int M, int T, int d, int r, int target_wgs = 1024) {
  FitLayout f{};
  f.M = M; f.T = T; f.d = d; f.r = r;
  f.rpad = (r + 31) / 32 * 32;
  f.slab = 16384 / d;  // 128 rows at d = 128, 256 at d = 64
  int nb = d / 32;
  f.nblk = nb * (nb + 1) / 2;
  int max_split = T > 0 ? ceil_div(T, f.slab) : 1;
  int want = M > 0 ? ceil_div(target_wgs, M) : 1;
  int ns = want < 1 ? 1 : (want > max_split ? max_split : want);
  int slabs_per = T > 0 ? ceil_div(ceil_div(T, f.slab), ns) : 1;
  f.chunk = slabs_per * f.slab;
  f.nsplit = T > 0 ? ceil_div(T, f.chunk) : 1;
  size_t o = 0;
  f.off_gram = o;   o = align_up(o + sizeof(double) * (size_t)M * f.nsplit * f.nblk * 1024, 256);
  f.off_whi = o;    o = align_up(o + 2ull * M * f.rpad * d, 256);
  f.off_wlo = o;    o = align_up(o + 2ull * M * f.rpad * d, 256);
  f.off_sweeps = o; o = align_up(o + sizeof(int) * (size_t)M, 256);
  f.bytes = o;
  return f;
}

// ---------------------------------------------------------------- launchers (.hip files)
hipError_t launch_pool_partials(const void* K, const void* V, int S, int T, int d, int dtype,
                                float* partials, int n_chunks, hipStream_t st);
hipError_t launch_reduce_pool(const float* partials, int n_chunks, int T, int S, int d,
                              float* q_out, hipStream_t st);
// Matching of every segment from chunk sums (or from q_in when not null); resets *ctr.
hipError_t launch_score(const float* partials, int n_chunks, int T, const float* q_in,
                        const float* desc, int S, int d, int A, float tau, float* w_ws,
                        uint8_t* mask_ws, float* score_out, float* w_out, uint8_t* mask_out,
                        int* ctr, hipStream_t st);
// Online anchor pool: matching of every segment against its pool's valid slots, top-A
// selection (weights and slots into the workspace); resets *ctr.
hipError_t launch_select(const float* partials, int n_chunks, int T, const float* q_in,
                         const float* desc, const int* count, int Vc, int S, int d, int A,
                         float tau, float* w_ws, int* slot_ws, uint8_t* mask_ws,
                         float* score_out, float* w_out, int* slot_out, uint8_t* mask_out,
                         int* ctr, hipStream_t st);
// Pool insertion: the slot after the last one written takes the new anchor (factors stored in
// the cache dtype) of every segment whose mask is set; then head and count advance.
hipError_t launch_pool_insert(const uint8_t* mask, const float* U_new, const float* W_new,
                              const float* q, int S, int T, int d, int dtype, int Vc, int r,
                              void* U_pool, void* W_pool, float* desc_pool, int* count,
                              int* head, hipStream_t st);
// Correction, after launch_score / launch_select (which reset its work counter).
hipError_t launch_correct(const CorrectLaunch& L, hipStream_t st);
// Anchor shapes the specialised correction kernel holds in registers and LDS.
inline bool correct_specialised(int A, int r, int dtype) {
  if (A > kMaxA || r > kMaxR) return false;
  return dtype == KVC_BF16 ? A * ((r + 15) / 16 * 16) <= kMaxKSlots : A * ((r + 7) / 8 * 8) <= 64;
}
// General correction (kvc_correct_general.hip): matching of any number of anchors from q
// [S][2d], then the correction as one contraction over the anchors' concatenated rank index
// (uses K, V, U, W, w_ws, mask_ws, slot_ws / Vc, K_fb, V_fb, K_out, V_out, S, T, d, dtype, A, r).
hipError_t launch_score_general(const float* q, const float* desc, int S, int d, int A,
                                float tau, float* w_ws, uint8_t* mask_ws, float* score_out,
                                float* w_out, uint8_t* mask_out, hipStream_t st);
hipError_t launch_correct_general(const CorrectLaunch& L, hipStream_t st);
// Rank-rC representation of a cache (kvc_fit.hip): F [2][S][rC][d] float32 (K then V),
// effective rank k_eff [2][S] and eigenvalues eig [2][S][d] (descending) through the fit's
// Gram and eigensolver kernels; ws holds fit_layout(2S, T, d, rC).
hipError_t launch_rank_descriptor(const void* K, const void* V, int S, int T, int d, int dtype,
                                  int rC, float* F, int32_t* k_eff, float* eig, char* ws,
                                  hipStream_t st);
// Matching on rank-rC representations (kvc_rank.hip): Fq [2][S][rC][d], Fa [2][S][A][rC][d]
// -> weights, flags and outputs as launch_score; resets *ctr.
hipError_t launch_score_rank(const float* Fq, const float* Fa, int S, int d, int A, int rC,
                             float tau, float* w_ws, uint8_t* mask_ws, float* score_out,
                             float* w_out, uint8_t* mask_out, int* ctr, hipStream_t st);
hipError_t launch_fit(const void* delta, const FitLayout& f, int dtype, double energy,
                      float* U_out, float* W_out, int32_t* k_eff, float* eig, char* ws,
                      hipStream_t st);
// Streaming fit: G += delta^T delta (float64, full symmetric) through the Gram partials of
// the workspace (FitLayout off_gram); eigensolver from a given G; projection U = delta W^T
// (bf16 deltas stage W as bf16 hi/lo in ws: 2 * M * rpad * d * 2 bytes).
hipError_t launch_gram_accumulate(const void* delta, const FitLayout& f, int dtype, double* G,
                                  char* ws, hipStream_t st);
hipError_t launch_fit_from_gram(const double* G, int M, int d, int r, double energy,
                                float* W_out, int32_t* k_eff, float* eig, hipStream_t st);
hipError_t launch_project(const void* delta, int M, int T, int d, int dtype, const float* W,
                          int r, float* U_out, char* ws, hipStream_t st);
// Warm-started refit from a given G and the previous W (kvc_warm.hip: the warm kernel alone,
// marking k_eff = kWarmMiss where it gives up; kvc_fit.hip: the whole refit, the full
// eigensolver finishing the marked matrices).
hipError_t launch_refit_warm_kernel(const double* G, int M, int d, int r, double energy,
                                    const float* W_prev, float* W_out, int32_t* k_eff,
                                    int32_t* warm, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st);
hipError_t launch_refit_warm(const double* G, int M, int d, int r, double energy,
                             const float* W_prev, float* W_out, int32_t* k_eff, int32_t* warm,
                             hipStream_t st);
// Error measures (kvc_metrics.hip): per-segment float64 sums of (X - R)^2 and R^2 through
// chunk partials (2 doubles per segment and 256-token chunk), and the rank-error curve.
int segment_error_chunks(int T);
hipError_t launch_segment_error(const void* X, const void* R, int S, int T, int d, int dtype,
                                double* partials, double* out, hipStream_t st);
hipError_t launch_rank_error_curve(const float* eig, int M, int n, float* curve, hipStream_t st);
int rank_error_curve_max_n();  // eigenvalues per matrix the curve kernel stages
// Streaming Gram workspace: float32 partials [M][nsplit][nblk][16][64].
inline size_t gram_ws_bytes(const FitLayout& f) {
  return align_up(sizeof(float) * (size_t)f.M * f.nsplit * f.nblk * 1024, 256);
}
// The projection splits W into bf16 halves inside its kernel: no workspace for either dtype.
inline size_t project_ws_bytes(int, int, int, int) { return 0; }

}  // namespace kvc
