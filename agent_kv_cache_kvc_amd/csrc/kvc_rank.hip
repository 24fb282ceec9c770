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
//                       the rC x rC products, each 32 x 32 tile of a product one wave's
//                       MFMA (fp32 32x32x2: lane (i, h) feeds row i of both factors over
//                       the h-th half of the channels, so the MFMA steps run through every
//                       channel once); per-wave sums joined in a fixed order
#include <hip/hip_runtime.h>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

__device__ __forceinline__ float rank_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// sum of the squared entries of the 32 x 32 tile (bi, bj) of F1 F2^T, F1 and F2 rC x D
// row-major (rows past rC are zero); every lane of the wave returns the same value
template <int D>
__device__ float tile_sq(const float* __restrict__ F1, const float* __restrict__ F2, int rC,
                         int bi, int bj, int lane) {
  constexpr int HK = D / 2;  // channels per half
  const int i = lane & 31, h = lane >> 5;
  const int r1 = bi * 32 + i, r2 = bj * 32 + i;
  const float4* a = reinterpret_cast<const float4*>(F1 + (size_t)r1 * D + h * HK);
  const float4* b = reinterpret_cast<const float4*>(F2 + (size_t)r2 * D + h * HK);
  const bool va = r1 < rC, vb = r2 < rC;
  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int m = 0; m < HK / 4; ++m) {
    const float4 x = va ? a[m] : float4{0.f, 0.f, 0.f, 0.f};
    const float4 y = vb ? b[m] : float4{0.f, 0.f, 0.f, 0.f};
    acc = mfma_f32(x.x, y.x, acc);
    acc = mfma_f32(x.y, y.y, acc);
    acc = mfma_f32(x.z, y.z, acc);
    acc = mfma_f32(x.w, y.w, acc);
  }
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) sq = fmaf(acc[e], acc[e], sq);
  return rank_wave_sum(sq);
}

}  // namespace

// Fq [2][S][rC][D], Fa [2][S][A][rC][D] float32.  Products per segment: p = 0, 1 the query's
// own K and V products (||q||^2); per anchor a, p = 2 + 4a + {0, 1} its own (||a||^2) and
// p = 2 + 4a + {2, 3} the query's with it (<q, a>).  Work unit u = (p, tile) goes to wave
// u % 4; each wave adds its units' tile sums in increasing u, then the waves are added in
// order.
template <int D>
__global__ __launch_bounds__(kBlock) void score_rank_kernel(
    const float* __restrict__ Fq, const float* __restrict__ Fa, int S, int A, int rC, float tau,
    float* __restrict__ w_ws, uint8_t* __restrict__ mask_ws, float* __restrict__ score_out,
    float* __restrict__ w_out, uint8_t* __restrict__ mask_out, int* __restrict__ ctr) {
  constexpr int NW = kBlock / kWave;
  __shared__ float part[NW][1 + 2 * kMaxAnchorsGeneral];  // [wave][||q||^2, ||a||^2, <q,a>]
  __shared__ float sc[kMaxAnchorsGeneral];
  const int s = blockIdx.x, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  if (s == 0 && tid == 0) *ctr = 0;  // work counter of the correction that follows
  const int nq = 1 + 2 * A;
  for (int e = tid; e < NW * nq; e += kBlock) part[e / nq][e % nq] = 0.f;
  __syncthreads();
  const size_t fsz = (size_t)rC * D;
  const float* qX[2] = {Fq + (size_t)s * fsz, Fq + ((size_t)S + s) * fsz};
  const int nt = (rC + 31) / 32, nt2 = nt * nt;
  const int n_units = (2 + 4 * A) * nt2;
  for (int u = wave; u < n_units; u += NW) {  // uniform per wave
    const int p = u / nt2, t = u - p * nt2;
    const int bi = t / nt, bj = t - bi * nt;
    const float* F1;
    const float* F2;
    int tgt;
    if (p < 2) {
      F1 = F2 = qX[p];
      tgt = 0;
    } else {
      const int a = (p - 2) >> 2, k = (p - 2) & 3, x = k & 1;
      const float* aX = Fa + (((size_t)x * S + s) * A + a) * fsz;
      F1 = k < 2 ? aX : qX[x];
      F2 = aX;
      tgt = k < 2 ? 1 + a : 1 + A + a;
    }
    const float v = tile_sq<D>(F1, F2, rC, bi, bj, lane);
    if (lane == 0) part[wave][tgt] += v;
  }
  __syncthreads();
  for (int a = tid; a < A; a += kBlock) {
    float nqq = 0.f, naa = 0.f, dqa = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      nqq += part[w][0];
      naa += part[w][1 + a];
      dqa += part[w][1 + A + a];
    }
    const float den = sqrtf(nqq) * sqrtf(naa);
    sc[a] = den == 0.f ? 0.f : dqa / den;
  }
  __syncthreads();
  if (tid >= kWave) return;
  // wave 0: score, softmax (the lanes' anchors a = lane + 64 i, joined in a fixed order)
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
  if (d == 128)
    hipLaunchKernelGGL((score_rank_kernel<128>), dim3(S), dim3(kBlock), 0, st, Fq, Fa, S, A, rC,
                       tau, w_ws, mask_ws, score_out, w_out, mask_out, ctr);
  else
    hipLaunchKernelGGL((score_rank_kernel<64>), dim3(S), dim3(kBlock), 0, st, Fq, Fa, S, A, rC,
                       tau, w_ws, mask_ws, score_out, w_out, mask_out, ctr);
  return hipGetLastError();
}

}  // namespace kvc
