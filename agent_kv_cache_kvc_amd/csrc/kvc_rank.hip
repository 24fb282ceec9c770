// Matching on the rank-rC representation of a cache segment.
//
// KVCMAS, thelatestinai listing: Fig. 13 keeps the base cache at rank r_C (32 by default) next
// to the delta rank r_delta; Fig. 1(b) matches the current cache representation against the
// segment's online anchors by similarity.  Here a segment is represented, for K and for V, by
// its rank-rC truncated second-moment matrix G = F^T F with F = diag(sigma_1..rC) V_rC^T (the
// sigma-scaled top right singular vectors; kvc_rank_descriptor computes F), and two
// representations are compared by the cosine of (G_K, G_V) as one vector:
//   s = (<Gq_K, Ga_K> + <Gq_V, Ga_V>) / (||(Gq_K, Gq_V)|| ||(Ga_K, Ga_V)||),
//   <G, G'> = ||F F'^T||_F^2   (rC x rC products; no d x d matrix is formed),
// which does not depend on the signs or any rotation of the factor rows.  Then softmax
// weights (temperature 1), score = max s, fallback = !(score >= tau), as for the mean-pooled
// descriptor.
//
//   score_rank_kernel   one 256-thread workgroup per segment: the squared Frobenius norms of
//                       the rC x rC products, 32 channels of both factors staged in LDS at a
//                       time; each thread owns PAIRS (i, j) entries; fixed-order reductions
#include <hip/hip_runtime.h>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kRankChunk = 32;  // channels of the factors staged per step

__device__ __forceinline__ float rank_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ||F1 F2^T||_F^2 for two rC x D row-major factors (float32 sums, fixed order; every thread of
// the workgroup returns the same value)
template <int D, int PAIRS>
__device__ float prod_sq(const float* __restrict__ F1, const float* __restrict__ F2, int rC,
                         float (*t1)[kRankChunk + 1], float (*t2)[kRankChunk + 1], float* red) {
  const int tid = threadIdx.x;
  float acc[PAIRS];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) acc[p] = 0.f;
  for (int c0 = 0; c0 < D; c0 += kRankChunk) {
    __syncthreads();
    for (int e = tid; e < rC * kRankChunk; e += kBlock) {
      const int i = e / kRankChunk, c = e % kRankChunk;
      t1[i][c] = F1[(size_t)i * D + c0 + c];
      t2[i][c] = F2[(size_t)i * D + c0 + c];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      const int pr = tid + kBlock * p;
      if (pr < rC * rC) {
        const int i = pr / rC, j = pr % rC;
        float a = acc[p];
#pragma unroll 8
        for (int c = 0; c < kRankChunk; ++c) a += t1[i][c] * t2[j][c];
        acc[p] = a;
      }
    }
  }
  float sq = 0.f;
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) sq += acc[p] * acc[p];
  sq = rank_wave_sum(sq);
  __syncthreads();
  if (tid % kWave == 0) red[tid / kWave] = sq;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

}  // namespace

// Fq [2][S][rC][D], Fa [2][S][A][rC][D] float32.
template <int D, int PAIRS>
__global__ __launch_bounds__(kBlock) void score_rank_kernel(
    const float* __restrict__ Fq, const float* __restrict__ Fa, int S, int A, int rC, float tau,
    float* __restrict__ w_ws, uint8_t* __restrict__ mask_ws, float* __restrict__ score_out,
    float* __restrict__ w_out, uint8_t* __restrict__ mask_out, int* __restrict__ ctr) {
  __shared__ float t1[kMaxRankC][kRankChunk + 1];
  __shared__ float t2[kMaxRankC][kRankChunk + 1];
  __shared__ float red[kBlock / kWave];
  __shared__ float sc[kMaxAnchorsGeneral];
  const int s = blockIdx.x, tid = threadIdx.x;
  if (s == 0 && tid == 0) *ctr = 0;  // work counter of the correction that follows
  const size_t fsz = (size_t)rC * D;
  const float* qK = Fq + (size_t)s * fsz;
  const float* qV = Fq + ((size_t)S + s) * fsz;
  const float nq = prod_sq<D, PAIRS>(qK, qK, rC, t1, t2, red) +
                   prod_sq<D, PAIRS>(qV, qV, rC, t1, t2, red);
  for (int a = 0; a < A; ++a) {
    const float* aK = Fa + ((size_t)s * A + a) * fsz;
    const float* aV = Fa + (((size_t)S + s) * A + a) * fsz;
    const float na = prod_sq<D, PAIRS>(aK, aK, rC, t1, t2, red) +
                     prod_sq<D, PAIRS>(aV, aV, rC, t1, t2, red);
    const float dq = prod_sq<D, PAIRS>(qK, aK, rC, t1, t2, red) +
                     prod_sq<D, PAIRS>(qV, aV, rC, t1, t2, red);
    const float den = sqrtf(nq) * sqrtf(na);
    if (tid == 0) sc[a] = den == 0.f ? 0.f : dq / den;
  }
  __syncthreads();
  if (tid >= kWave) return;
  // wave 0: score, softmax (the lanes' anchors a = lane + 64 i, joined in a fixed order)
  const int lane = tid;
  float best = -INFINITY;
  bool nan = false;
  for (int a = lane; a < A; a += kWave) {
    best = fmaxf(best, sc[a]);
    nan |= sc[a] != sc[a];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) best = fmaxf(best, __shfl_xor(best, off, 64));
  nan = __any(nan);
  const float score = nan ? __uint_as_float(0x7fc00000u) : best;
  float z = 0.f;
  for (int a = lane; a < A; a += kWave) z += expf(sc[a] - score);
  z = rank_wave_sum(z);
  for (int a = lane; a < A; a += kWave) {
    const float wv = expf(sc[a] - score) / z;
    w_ws[(size_t)s * A + a] = wv;
    if (w_out) w_out[(size_t)s * A + a] = wv;
  }
  if (lane == 0) {
    const uint8_t fall = !(score >= tau);
    mask_ws[s] = fall;
    mask_out[s] = fall;
    if (score_out) score_out[s] = score;
  }
}

hipError_t launch_score_rank(const float* Fq, const float* Fa, int S, int d, int A, int rC,
                             float tau, float* w_ws, uint8_t* mask_ws, float* score_out,
                             float* w_out, uint8_t* mask_out, int* ctr, hipStream_t st) {
  if (S == 0) return hipSuccess;
  const int pairs = (rC * rC + kBlock - 1) / kBlock;  // rC <= 128: at most 64
#define KVC_RANK_LAUNCH(DD, PP)                                                              \
  hipLaunchKernelGGL((score_rank_kernel<DD, PP>), dim3(S), dim3(kBlock), 0, st, Fq, Fa, S, A, \
                     rC, tau, w_ws, mask_ws, score_out, w_out, mask_out, ctr)
  if (d == 128) {
    if (pairs <= 4) KVC_RANK_LAUNCH(128, 4);
    else if (pairs <= 16) KVC_RANK_LAUNCH(128, 16);
    else KVC_RANK_LAUNCH(128, 64);
  } else {
    if (pairs <= 4) KVC_RANK_LAUNCH(64, 4);
    else KVC_RANK_LAUNCH(64, 16);
  }
#undef KVC_RANK_LAUNCH
  return hipGetLastError();
}

}  // namespace kvc
