// Error measures of the KVCMAS listing's studies, on the device (gfx950).
//
//   segment_error_kernel       per (segment, 256-token chunk): sum (X - ref)^2 and sum ref^2 in
//                              float64 (Fig. 3: reconstruction error normalised by the
//                              Frobenius norm of the exact full-prefill cache)   (HBM stream)
//   segment_error_sum_kernel   chunk partials -> one pair per segment, chunk order
//   rank_error_curve_kernel    relative error of the best rank-k approximation for k = 0..n
//                              from the eigenvalues of delta^T delta (Fig. 7(b))
//
// Every sum runs in a fixed order, so results are deterministic.
#include <hip/hip_runtime.h>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

constexpr int kErrChunk = 256;  // tokens per workgroup of segment_error_kernel
constexpr int kErrUnroll = 4;   // 16-byte loads of each input in flight per thread

template <class E>
__device__ __forceinline__ void add_error(const u32x4& x, const u32x4& r, double& e, double& rr) {
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // two bf16 per 32-bit word; widening is exact and so is the float64 difference
      const double x0 = (double)__uint_as_float(x[j] << 16);
      const double x1 = (double)__uint_as_float(x[j] & 0xffff0000u);
      const double r0 = (double)__uint_as_float(r[j] << 16);
      const double r1 = (double)__uint_as_float(r[j] & 0xffff0000u);
      const double d0 = x0 - r0, d1 = x1 - r1;
      e = fma(d0, d0, e);
      e = fma(d1, d1, e);
      rr = fma(r0, r0, rr);
      rr = fma(r1, r1, rr);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double xv = (double)__uint_as_float(x[j]);
      const double rv = (double)__uint_as_float(r[j]);
      const double dv = xv - rv;
      e = fma(dv, dv, e);
      rr = fma(rv, rv, rr);
    }
  }
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// grid (n_chunks, S); partials[(s * n_chunks + chunk) * 2 + {0, 1}].
template <class E, int D>
__global__ __launch_bounds__(kBlock) void segment_error_kernel(const E* __restrict__ X,
                                                               const E* __restrict__ R, int T,
                                                               int n_chunks,
                                                               double* __restrict__ partials) {
  constexpr int VPR = D * (int)sizeof(E) / 16;  // 16-byte vectors per token row
  const int chunk = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int t0 = chunk * kErrChunk;
  const int t1 = T < t0 + kErrChunk ? T : t0 + kErrChunk;
  const int nvec = (t1 - t0) * VPR;
  const size_t base = ((size_t)s * T + t0) * D;
  const u32x4* xp = reinterpret_cast<const u32x4*>(X + base);
  const u32x4* rp = reinterpret_cast<const u32x4*>(R + base);
  double e = 0.0, rr = 0.0;
  for (int i0 = tid; i0 < nvec; i0 += kBlock * kErrUnroll) {
    u32x4 xa[kErrUnroll], ra[kErrUnroll];
#pragma unroll
    for (int u = 0; u < kErrUnroll; ++u) {
      const int i = i0 + u * kBlock;
      if (i < nvec) {
        xa[u] = __builtin_nontemporal_load(xp + i);
        ra[u] = __builtin_nontemporal_load(rp + i);
      } else {
        xa[u] = u32x4{0u, 0u, 0u, 0u};
        ra[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kErrUnroll; ++u) add_error<E>(xa[u], ra[u], e, rr);
  }
  e = wave_sum_f64(e);
  rr = wave_sum_f64(rr);
  __shared__ double red[2][kBlock / kWave];
  const int wave = tid / kWave, lane = tid % kWave;
  if (lane == 0) {
    red[0][wave] = e;
    red[1][wave] = rr;
  }
  __syncthreads();
  if (tid < 2) {
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) v += red[tid][w];
    partials[((size_t)s * n_chunks + chunk) * 2 + tid] = v;
  }
}

__global__ __launch_bounds__(kBlock) void segment_error_sum_kernel(
    const double* __restrict__ partials, int n_chunks, int S, double* __restrict__ out) {
  const int s = blockIdx.x * kBlock + threadIdx.x;
  if (s >= S) return;
  double e = 0.0, rr = 0.0;
  for (int c = 0; c < n_chunks; ++c) {
    e += partials[((size_t)s * n_chunks + c) * 2];
    rr += partials[((size_t)s * n_chunks + c) * 2 + 1];
  }
  out[(size_t)s * 2] = e;
  out[(size_t)s * 2 + 1] = rr;
}

// One wave per matrix.  eig: [M, n] descending (negative round-off counts as 0);
// curve[k] = sqrt(sum_{i >= k} lambda_i / sum_i lambda_i), the tail added from the smallest
// eigenvalue up and the total from the largest down (float64, in that fixed order: the sums
// are a dependent chain that lane 0 runs out of LDS); a zero total gives 0.  The eigenvalues
// are staged and the curve written with coalesced accesses.
constexpr int kCurveMax = 256;  // eigenvalues per matrix staged in LDS

__global__ __launch_bounds__(kWave) void rank_error_curve_kernel(const float* __restrict__ eig,
                                                                 int n,
                                                                 float* __restrict__ curve) {
  __shared__ double lam[kCurveMax + 1];  // eigenvalues, then the tails
  __shared__ double tot;
  const int m = blockIdx.x, lane = threadIdx.x;
  const float* e = eig + (size_t)m * n;
  float* o = curve + (size_t)m * (n + 1);
  for (int i = lane; i < n; i += kWave) lam[i] = (double)fmaxf(e[i], 0.f);
  __syncthreads();
  if (lane == 0) {  // the two dependent chains of additions, in the fixed order
    double total = 0.0;
    for (int i = 0; i < n; ++i) total += lam[i];
    double tail = 0.0;
    lam[n] = 0.0;
    for (int k = n - 1; k >= 0; --k) {
      tail += lam[k];
      lam[k] = tail;
    }
    tot = total;
  }
  __syncthreads();
  const double total = tot;
  for (int k = lane; k <= n; k += kWave)
    o[k] = total > 0.0 ? (float)sqrt(lam[k] / total) : 0.f;
}

int segment_error_chunks(int T) { return T > 0 ? ceil_div(T, kErrChunk) : 0; }

template <class E, int D>
static hipError_t segment_error_t(const void* X, const void* R, int S, int T, double* partials,
                                  int n_chunks, hipStream_t st) {
  hipLaunchKernelGGL((segment_error_kernel<E, D>), dim3(n_chunks, S), dim3(kBlock), 0, st,
                     static_cast<const E*>(X), static_cast<const E*>(R), T, n_chunks, partials);
  return hipGetLastError();
}

hipError_t launch_segment_error(const void* X, const void* R, int S, int T, int d, int dtype,
                                double* partials, double* out, hipStream_t st) {
  if (S == 0) return hipSuccess;
  const int nc = segment_error_chunks(T);
  if (nc > 0) {
    hipError_t e;
    if (dtype == KVC_BF16)
      e = d == 128 ? segment_error_t<uint16_t, 128>(X, R, S, T, partials, nc, st)
                   : segment_error_t<uint16_t, 64>(X, R, S, T, partials, nc, st);
    else
      e = d == 128 ? segment_error_t<float, 128>(X, R, S, T, partials, nc, st)
                   : segment_error_t<float, 64>(X, R, S, T, partials, nc, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(segment_error_sum_kernel, dim3(ceil_div(S, kBlock)), dim3(kBlock), 0, st,
                     partials, nc, S, out);
  return hipGetLastError();
}

int rank_error_curve_max_n() { return kCurveMax; }

hipError_t launch_rank_error_curve(const float* eig, int M, int n, float* curve, hipStream_t st) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(rank_error_curve_kernel, dim3(M), dim3(kWave), 0, st, eig, n, curve);
  return hipGetLastError();
}

}  // namespace kvc
