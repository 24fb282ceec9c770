// Online anchor pool of the KVCMAS listing (Table 13: pool capacity V), insertion side.
//
//   pool_insert_kernel   copies a new anchor (fp32 fit factors -> cache dtype, round to nearest
//                        even; its descriptor) into the slot `head` of every segment whose
//                        mask is set                                          (HBM stream)
//   pool_advance_kernel  then moves head to the next slot (first in, first out) and counts
//
// Two launches, so every copy reads the head that was current when the call began.
#include <hip/hip_runtime.h>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

constexpr int kInsRows = 128;  // token rows of U per workgroup

__device__ __forceinline__ void put(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void put(float* p, float v) { *p = v; }

// n consecutive values src -> dst in the cache dtype: 8 per thread with 16-byte accesses when
// both ends are 16-byte aligned, element by element otherwise.
template <class E>
__device__ __forceinline__ void convert(E* __restrict__ dst, const float* __restrict__ src, int n,
                                        int tid) {
  const bool vec = (reinterpret_cast<uintptr_t>(dst) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(src) % 16 == 0);
  int done = 0;
  if (vec) {
    const int n8 = n / 8;
    for (int i = tid; i < n8; i += kBlock) {
      const floatx4 a = reinterpret_cast<const floatx4*>(src)[2 * i];
      const floatx4 b = reinterpret_cast<const floatx4*>(src)[2 * i + 1];
      if constexpr (sizeof(E) == 2) {
        u32x4 o;
        o[0] = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
        o[1] = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
        o[2] = (uint32_t)f32_to_bf16(b[0]) | ((uint32_t)f32_to_bf16(b[1]) << 16);
        o[3] = (uint32_t)f32_to_bf16(b[2]) | ((uint32_t)f32_to_bf16(b[3]) << 16);
        reinterpret_cast<u32x4*>(dst)[i] = o;
      } else {
        reinterpret_cast<floatx4*>(dst)[2 * i] = a;
        reinterpret_cast<floatx4*>(dst)[2 * i + 1] = b;
      }
    }
    done = n8 * 8;
  }
  for (int i = done + tid; i < n; i += kBlock) put(dst + i, src[i]);
}

__device__ __forceinline__ int pool_slot(const int* head, int s, int Vc) {
  const int j = head[s];
  return (j >= 0 && j < Vc) ? j : 0;  // the library keeps head in range; never write outside
}

// grid (row blocks of U + 1, 2 (K|V), S); the last row block copies W (and, for K, desc).
template <class E>
__global__ __launch_bounds__(kBlock) void pool_insert_kernel(
    const uint8_t* __restrict__ mask, const float* __restrict__ U_new,
    const float* __restrict__ W_new, const float* __restrict__ q, int S, int T, int d, int Vc,
    int r, E* __restrict__ U_pool, E* __restrict__ W_pool, float* __restrict__ desc_pool,
    const int* __restrict__ head) {
  const int blk = blockIdx.x, x = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
  if (mask[s] == 0) return;
  const int j = pool_slot(head, s, Vc);
  const size_t m = (size_t)x * S + s;  // fit matrix: K matrices, then V
  if (blk < (int)gridDim.x - 1) {
    const int t0 = blk * kInsRows;
    const int rows = T - t0 < kInsRows ? T - t0 : kInsRows;
    const int n = rows * r;
    convert(U_pool + ((m * Vc + j) * T + t0) * r, U_new + (m * T + t0) * r, n, tid);
  } else {
    const int n = r * d;
    convert(W_pool + (m * Vc + j) * n, W_new + m * n, n, tid);
    if (x == 0)
      for (int i = tid; i < 2 * d; i += kBlock)
        desc_pool[((size_t)s * Vc + j) * 2 * d + i] = q[(size_t)s * 2 * d + i];
  }
}

__global__ __launch_bounds__(kBlock) void pool_advance_kernel(const uint8_t* __restrict__ mask,
                                                              int S, int Vc, int* __restrict__ count,
                                                              int* __restrict__ head) {
  const int s = blockIdx.x * kBlock + threadIdx.x;
  if (s >= S || mask[s] == 0) return;
  const int j = pool_slot(head, s, Vc);
  head[s] = j + 1 == Vc ? 0 : j + 1;
  const int c = count[s];
  count[s] = c < 0 ? 1 : (c >= Vc ? Vc : c + 1);
}

hipError_t launch_pool_insert(const uint8_t* mask, const float* U_new, const float* W_new,
                              const float* q, int S, int T, int d, int dtype, int Vc, int r,
                              void* U_pool, void* W_pool, float* desc_pool, int* count,
                              int* head, hipStream_t st) {
  if (S == 0) return hipSuccess;
  const dim3 grid(ceil_div(T, kInsRows) + 1, 2, S);
  if (dtype == KVC_BF16)
    hipLaunchKernelGGL(pool_insert_kernel<uint16_t>, grid, dim3(kBlock), 0, st, mask, U_new,
                       W_new, q, S, T, d, Vc, r, static_cast<uint16_t*>(U_pool),
                       static_cast<uint16_t*>(W_pool), desc_pool, head);
  else
    hipLaunchKernelGGL(pool_insert_kernel<float>, grid, dim3(kBlock), 0, st, mask, U_new, W_new,
                       q, S, T, d, Vc, r, static_cast<float*>(U_pool),
                       static_cast<float*>(W_pool), desc_pool, head);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pool_advance_kernel, dim3(ceil_div(S, kBlock)), dim3(kBlock), 0, st, mask, S,
                     Vc, count, head);
  return hipGetLastError();
}

}  // namespace kvc
