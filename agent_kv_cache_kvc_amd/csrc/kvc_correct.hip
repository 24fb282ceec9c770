// Online correction of a reused shared-context KV cache on gfx950.
//
// KVCMAS, thelatestinai listing, Fig. 1: the reused cache of a shared segment is matched
// against the segment's online anchors (pooled descriptor vs. anchor descriptors, cosine),
// the anchors' low-rank corrections are combined with similarity weights (softmax) and
// added to K and V; a segment whose best match is below tau falls back to dense prefill.
//
// Kernels (all deterministic: fixed-order reductions, no floating-point atomics)
//   pool_partials_kernel  token sums of K and V per 256-token tile          (HBM stream)
//   score_kernel          tile sums -> q, cosines, softmax, score, mask     (one wave/segment)
//   correct_kernel        X' = X + sum_a w_a U_a W_a on MFMA, or copy-through (HBM stream)
//   reduce_pool_kernel    tile sums -> q (the pooling entry point)
#include <hip/hip_runtime.h>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

// ------------------------------------------------------------------------- dtype traits
struct TrBF16 {
  using elem = uint16_t;
  using frag = u32x4;
  static constexpr int VEC = 8;    // elements per 16-byte access
  static constexpr int SLOT = 8;   // consecutive k per lane per MFMA
  static constexpr int MAXF = 16;  // register-resident U fragments per 32-token tile
  static constexpr int RPAD = 16;  // r is padded to a multiple of this
  static constexpr int LPT = 8;    // lanes per 64-channel half row (16 bytes each)
  __device__ static float f(elem e) { return bf16_to_f32(e); }
  __device__ static elem e(float v) { return f32_to_bf16(v); }
  __device__ static floatx16 mma(const frag& a, const frag& b, const floatx16& c) {
    return mfma_bf16(a, b, c);
  }
};

struct TrF32 {
  using elem = float;
  using frag = float;
  static constexpr int VEC = 4;
  static constexpr int SLOT = 1;
  static constexpr int MAXF = 32;
  static constexpr int RPAD = 8;
  static constexpr int LPT = 16;
  __device__ static float f(elem e) { return e; }
  __device__ static elem e(float v) { return v; }
  __device__ static floatx16 mma(const frag& a, const frag& b, const floatx16& c) {
    return mfma_f32(a, b, c);
  }
};

template <class Tr>
__device__ __forceinline__ void load16(const typename Tr::elem* p, float (&v)[Tr::VEC]) {
  u32x4 raw = *reinterpret_cast<const u32x4*>(p);
  if constexpr (Tr::VEC == 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(raw[j] << 16);
      v[2 * j + 1] = __uint_as_float(raw[j] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(raw[j]);
  }
}

// ------------------------------------------------------------------------- pooling
// grid (n_tiles, S, 2); each workgroup sums kPoolRows tokens of one segment's K or V.
template <class Tr, int D>
__global__ __launch_bounds__(kBlock) void pool_partials_kernel(
    const typename Tr::elem* __restrict__ K, const typename Tr::elem* __restrict__ V, int T,
    float* __restrict__ partials, int n_tiles) {
  using elem = typename Tr::elem;
  constexpr int VEC = Tr::VEC;
  constexpr int LPR = D / VEC;       // lanes per token row
  constexpr int RPP = kBlock / LPR;  // rows per pass
  __shared__ float red[RPP][D + 1];
  const int tile = blockIdx.x, s = blockIdx.y, x = blockIdx.z, S = gridDim.y;
  const elem* src = (x == 0 ? K : V) + (size_t)s * T * D;
  const int tid = threadIdx.x;
  const int cg = tid % LPR, rs = tid / LPR;
  float acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = 0.f;
  const int t0 = tile * kPoolRows;
  const int t1 = min(T, t0 + kPoolRows);
#pragma unroll 4
  for (int t = t0 + rs; t < t1; t += RPP) {
    float v[VEC];
    load16<Tr>(src + (size_t)t * D + cg * VEC, v);
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] += v[j];
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) red[rs][cg * VEC + j] = acc[j];
  __syncthreads();
  if (tid < D) {
    float sum = 0.f;
    for (int i = 0; i < RPP; ++i) sum += red[i][tid];
    partials[(((size_t)x * S + s) * n_tiles + tile) * D + tid] = sum;
  }
}

// tile sums -> pooled descriptor, one wave per segment.
template <int D>
__device__ __forceinline__ void pooled_query(const float* __restrict__ partials, int n_tiles,
                                             int T, int s, int S, int lane,
                                             float (&q)[2 * D / kWave]) {
  constexpr int PER = 2 * D / kWave;
  // tile sums are added in tile order; loads are issued 8 tiles at a time
  float sum[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sum[i] = 0.f;
  for (int t0 = 0; t0 < n_tiles; t0 += 8) {
    float v[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = lane + kWave * i;
        const int x = c / D, ch = c % D;
        v[u][i] = (t0 + u < n_tiles)
                      ? partials[(((size_t)x * S + s) * n_tiles + t0 + u) * D + ch]
                      : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (t0 + u < n_tiles) sum[i] += v[u][i];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) q[i] = T > 0 ? sum[i] / (float)T : 0.f;
}

template <int D>
__global__ __launch_bounds__(kWave) void reduce_pool_kernel(const float* __restrict__ partials,
                                                            int n_tiles, int T,
                                                            float* __restrict__ q_out) {
  constexpr int PER = 2 * D / kWave;
  const int s = blockIdx.x, S = gridDim.x, lane = threadIdx.x;
  float q[PER];
  pooled_query<D>(partials, n_tiles, T, s, S, lane, q);
#pragma unroll
  for (int i = 0; i < PER; ++i) q_out[(size_t)s * 2 * D + lane + kWave * i] = q[i];
}

// ------------------------------------------------------------------------- matching
// One wave per segment: q, s_a = cos(q, desc_a), w = softmax(s), score = max s, mask.
template <int D>
__global__ __launch_bounds__(kWave) void score_kernel(
    const float* __restrict__ partials, int n_tiles, int T, const float* __restrict__ q_in,
    const float* __restrict__ desc, int A, float tau, float* __restrict__ w_ws,
    uint8_t* __restrict__ mask_ws, float* __restrict__ q_out, float* __restrict__ score_out,
    float* __restrict__ w_out, uint8_t* __restrict__ mask_out, int* __restrict__ ctr) {
  constexpr int PER = 2 * D / kWave;
  const int s = blockIdx.x, S = gridDim.x, lane = threadIdx.x;
  if (s == 0 && lane == 0) *ctr = 0;  // work counter of the correction pass that follows
  float q[PER];
  if (q_in != nullptr) {
#pragma unroll
    for (int i = 0; i < PER; ++i) q[i] = q_in[(size_t)s * 2 * D + lane + kWave * i];
  } else {
    pooled_query<D>(partials, n_tiles, T, s, S, lane, q);
  }
  float qq = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) qq += q[i] * q[i];
  qq = wave_sum(qq);
  const float nq = sqrtf(qq);
  float sc[kMaxA];
  float best = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int a = 0; a < kMaxA; ++a) {
    sc[a] = 0.f;
    if (a < A) {
      const float* da = desc + ((size_t)s * A + a) * 2 * D;
      float dd = 0.f, dq = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const float v = da[lane + kWave * i];
        dd += v * v;
        dq += v * q[i];
      }
      dd = wave_sum(dd);
      dq = wave_sum(dq);
      const float den = nq * sqrtf(dd);
      const float c = (den == 0.f) ? 0.f : dq / den;
      sc[a] = c;
      nan |= (c != c);
      best = fmaxf(best, c);
    }
  }
  const float score = nan ? __uint_as_float(0x7fc00000u) : best;
  float z = 0.f;
  float ex[kMaxA];
#pragma unroll
  for (int a = 0; a < kMaxA; ++a) {
    ex[a] = 0.f;
    if (a < A) {
      ex[a] = expf(sc[a] - score);
      z += ex[a];
    }
  }
  const uint8_t fall = !(score >= tau);
  if (lane < A) {
    float wv = 0.f;
#pragma unroll
    for (int a = 0; a < kMaxA; ++a)
      if (a == lane) wv = ex[a] / z;
    w_ws[(size_t)s * A + lane] = wv;
    if (w_out) w_out[(size_t)s * A + lane] = wv;
  }
  if (lane == 0) {
    mask_ws[s] = fall;
    if (mask_out) mask_out[s] = fall;
    if (score_out) score_out[s] = score;
  }
  if (q_out) {
#pragma unroll
    for (int i = 0; i < PER; ++i) q_out[(size_t)s * 2 * D + lane + kWave * i] = q[i];
  }
}

// ------------------------------------------------------------------------- correction
// Persistent workgroups (4 waves) take work items (segment, K|V, 512-token chunk) from a
// counter that the score kernel resets.  A wave owns 32 tokens per tile and all d channels.
//
// MFMA: (delta X)^T = W^T U^T per 32-channel block; A operand = W_a^T staged in LDS (rows
// permuted by cmap32), B operand = U_a rows (8 consecutive k per lane, straight from HBM);
// result register i of lane l = (token l % 32, channel 16 (l / 32) + i).  Each anchor's
// product is finished in float32 and scaled by its weight, so w never passes through bf16.
// k layout: r is padded to rp (multiple of 2*SLOT); lane half g covers k in
// [g*rp/2, (g+1)*rp/2), MFMA step ks takes SLOT consecutive k from there.
//
// Memory: X is loaded and X' stored with coalesced 16-byte accesses (lane l of an access
// covers token l / LPT of the group, channels 8 (l % LPT) ... of a 64-channel half row);
// the MFMA result goes through a per-wave LDS tile [32][64 + 4] floats to meet that layout.
// The next tile's U (double-buffered) is requested before the current tile's MFMAs, and
// each half of the next tile's X as soon as the epilogue has consumed that half.
constexpr int kChunk = kCorrRowsPerIter * kCorrIters;  // tokens per work item
constexpr int kStageRow = 68;                          // floats per staged token row

// Inverse of cmap32: channel within a 32-block -> MFMA operand row.  W^T rows are stored in
// LDS in operand-row order, so the 16 lanes of a quarter wave read 16 consecutive rows.
__device__ __forceinline__ int cinv32(int c) {
  return 8 * ((c >> 2) & 3) + 4 * (c >> 4) + (c & 3);
}

// VEC float32 results -> VEC stored elements (bf16: hardware round-to-nearest-even pairs)
template <class Tr>
__device__ __forceinline__ u32x4 pack_out(const float* v) {
  u32x4 o;
  if constexpr (Tr::VEC == 8) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = __builtin_bit_cast(uint32_t,
                                __builtin_convertvector(f2_t{v[2 * j], v[2 * j + 1]}, bf16x2_t));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = __float_as_uint(v[j]);
  }
  return o;
}

template <class Tr>
__device__ __forceinline__ void unpack_in(const u32x4& raw, float* v) {
  if constexpr (Tr::VEC == 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(raw[j] << 16);
      v[2 * j + 1] = __uint_as_float(raw[j] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(raw[j]);
  }
}

template <class Tr, int D, int NF>
struct CorrTile {
  static constexpr int NH = D / 64;        // 64-channel halves
  static constexpr int JN = Tr::LPT / 2;   // coalesced accesses per half per 32 tokens
  u32x4 x[NH][JN];                         // X of the tile in flight (coalesced layout)
  typename Tr::frag u[NF];                 // U fragments of the tile in flight
};

// NA > 0: compile-time anchor count NA and MFMA steps per anchor KSC (r = 2 KSC SLOT);
// NA == 0: runtime A and r with up to NFG register-resident fragments.
template <class Tr, int D, int NA, int KSC, int NFG, bool POOL_OUT>
__global__ __launch_bounds__(kBlock, 2) void correct_kernel(
    const typename Tr::elem* __restrict__ K, const typename Tr::elem* __restrict__ V,
    const typename Tr::elem* __restrict__ U, const typename Tr::elem* __restrict__ W,
    const float* __restrict__ w_all, const uint8_t* __restrict__ mask,
    const typename Tr::elem* __restrict__ K_fb, const typename Tr::elem* __restrict__ V_fb,
    typename Tr::elem* K_out, typename Tr::elem* V_out, float* __restrict__ next_partials,
    int T, int S, int A_rt, int r_rt, int rp_rt, int n_chunks, int n_items,
    int* __restrict__ ctr) {
  using elem = typename Tr::elem;
  using frag = typename Tr::frag;
  constexpr bool FIX = NA > 0;
  constexpr int NF = FIX ? NA * KSC : NFG;
  using Tile = CorrTile<Tr, D, NF>;
  constexpr int VEC = Tr::VEC;
  constexpr int SLOT = Tr::SLOT;
  constexpr int LPT = Tr::LPT;
  constexpr int TPI = kWave / LPT;  // tokens per coalesced access
  constexpr int NH = Tile::NH, JN = Tile::JN;
  constexpr int PADK = 16 / sizeof(elem);

  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ float wsh[kMaxA];
  __shared__ float red[4][D];
  __shared__ int s_item;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 5, ln = lane & 31;
  float* stage = reinterpret_cast<float*>(smem_raw) + wave * 32 * kStageRow;
  elem* wt = reinterpret_cast<elem*>(smem_raw + 4 * 32 * kStageRow * sizeof(float));
  const int A = FIX ? NA : A_rt;
  const int r = FIX ? 2 * KSC * SLOT : r_rt;
  const int rp = FIX ? 2 * KSC * SLOT : rp_rt;
  const int RS = rp + PADK;
  const int half = rp / 2;
  const int KS = FIX ? KSC : half / SLOT;  // MFMA steps per anchor
  const int nfrag = A * KS;
  const bool uvec = FIX || (r % VEC) == 0;
  const int lrow = lane / LPT;               // token within a coalesced access
  const int lcol = VEC * (lane % LPT);       // channel offset within a half row

  for (;;) {
    if (tid == 0) s_item = atomicAdd(ctr, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item >= n_items) break;
    const int chunk = item % n_chunks;
    const int sx = item / n_chunks;
    const int x = sx & 1, s = sx >> 1;
    const size_t seg = (size_t)s * T * D;
    const elem* X = (x == 0 ? K : V) + seg;
    elem* Y = (x == 0 ? K_out : V_out) + seg;
    const elem* Xfb = (x == 0 ? K_fb : V_fb);
    const int tb = chunk * kChunk;

    float qs[POOL_OUT ? NH : 1][VEC];
    if constexpr (POOL_OUT) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) qs[h][e] = 0.f;
    }

    if (mask[s]) {
      // dense-prefill stand-in: copy the fallback cache (or the source) bit for bit
      const elem* src = Xfb ? Xfb + seg : X;
      for (int it = 0; it < kCorrIters; ++it) {
        const int t0 = tb + it * kCorrRowsPerIter + wave * 32;
        if (t0 >= T) break;
        u32x4 v[NH][JN];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            const int tok = t0 + TPI * j + lrow;
            v[h][j] = tok < T ? *reinterpret_cast<const u32x4*>(src + tok * D + 64 * h + lcol)
                              : u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            const int tok = t0 + TPI * j + lrow;
            if (tok < T) {
              *reinterpret_cast<u32x4*>(Y + tok * D + 64 * h + lcol) = v[h][j];
              if constexpr (POOL_OUT) {
                float fv[VEC];
                unpack_in<Tr>(v[h][j], fv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) qs[h][e] += fv[e];
              }
            }
          }
      }
    } else {
      // ---- stage W_a^T of this segment in LDS, rows in MFMA operand order (zero for
      //      k >= r), and the weights
      const elem* Wseg = W + ((size_t)x * S + s) * A * r * D;
      const int chunks = A * r * (D / VEC);
      for (int q = tid; q < chunks; q += kBlock) {
        // k varies fastest across lanes, so the transposed LDS writes are contiguous
        const int k = q % r;
        const int rest = q / r;
        const int c0 = (rest % (D / VEC)) * VEC;
        const int a = rest / (D / VEC);
        elem v[VEC];
        *reinterpret_cast<u32x4*>(v) =
            *reinterpret_cast<const u32x4*>(Wseg + ((size_t)a * r + k) * D + c0);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int c = c0 + j;
          wt[(a * D + (c & ~31) + cinv32(c & 31)) * RS + k] = v[j];
        }
      }
      if (!FIX && rp > r) {
        const int pad = rp - r;
        for (int q = tid; q < A * D * pad; q += kBlock) {
          const int k = r + q % pad;
          const int ac = q / pad;
          wt[ac * RS + k] = Tr::e(0.f);
        }
      }
      if (tid < A) wsh[tid] = w_all[(size_t)s * A + tid];
      __syncthreads();

      const elem* Useg = U + ((size_t)x * S + s) * A * (size_t)T * r;
      const int first = tb + wave * 32;
      const int n_my = first < T ? min(kCorrIters, (T - first + kCorrRowsPerIter - 1) / kCorrRowsPerIter) : 0;

      Tile b;
      frag u2[NF];
      auto load_x = [&](int h, int t0) {
        if (t0 + 32 <= T) {
#pragma unroll
          for (int j = 0; j < JN; ++j)
            b.x[h][j] = *reinterpret_cast<const u32x4*>(X + (t0 + TPI * j + lrow) * D + 64 * h + lcol);
        } else {
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            const int tok = t0 + TPI * j + lrow;
            b.x[h][j] = tok < T ? *reinterpret_cast<const u32x4*>(X + tok * D + 64 * h + lcol)
                                : u32x4{0u, 0u, 0u, 0u};
          }
        }
      };
      auto load_u = [&](frag (&dst)[NF], int t0) {
        const int t = t0 + ln;
        if (FIX && t0 + 32 <= T) {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const int a = f / KS, ks = f - a * KS;
            const elem* up = Useg + (a * T + t) * r + g * half + ks * SLOT;
            if constexpr (SLOT == 8) dst[f] = *reinterpret_cast<const u32x4*>(up);
            else dst[f] = Tr::f(*up);
          }
          return;
        }
        const bool valid = t < T;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f < nfrag) {
            const int a = f / KS, ks = f - a * KS;
            const int k0 = g * half + ks * SLOT;
            const elem* up = Useg + (a * T + t) * r + k0;
            if constexpr (SLOT == 8) {
              u32x4 v = {0u, 0u, 0u, 0u};
              if (valid && k0 < r) {
                if (uvec) {
                  v = *reinterpret_cast<const u32x4*>(up);
                } else {
                  uint16_t tmp[8];
#pragma unroll
                  for (int jj = 0; jj < 8; ++jj) tmp[jj] = (k0 + jj < r) ? up[jj] : (uint16_t)0;
                  v = *reinterpret_cast<u32x4*>(tmp);
                }
              }
              dst[f] = v;
            } else {
              dst[f] = (valid && k0 < r) ? Tr::f(*up) : 0.f;
            }
          }
        }
      };

      // one tile: MFMAs on `cu`; the next tile's U goes to `nu` before the MFMAs start
      auto run_tile = [&](int it, frag (&cu)[NF], frag (&nu)[NF]) {
        const int t0 = first + it * kCorrRowsPerIter;
        const int tn = t0 + kCorrRowsPerIter;
        const bool more = it + 1 < n_my;
        if (more) load_u(nu, tn);
        const bool full = t0 + 32 <= T;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          // ---- two 32-channel MFMA blocks of this half into the staging tile
#pragma unroll 1
          for (int cbl = 0; cbl < 2; ++cbl) {
            const int cb = 2 * h + cbl;
            const elem* ap = wt + (cb * 32 + ln) * RS + g * half;
            floatx16 acc, tmp;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              if (FIX || f < nfrag) {
                const int a = f / KS, ks = f - a * KS;
                frag af;
                if constexpr (SLOT == 8) {
                  af = *reinterpret_cast<const u32x4*>(ap + a * D * RS + ks * SLOT);
                } else {
                  af = ap[a * D * RS + ks];
                }
                if (ks == 0) {
                  floatx16 z;
#pragma unroll
                  for (int i = 0; i < 16; ++i) z[i] = 0.f;
                  tmp = Tr::mma(af, cu[f], z);
                } else {
                  tmp = Tr::mma(af, cu[f], tmp);
                }
                if (ks == KS - 1) {
                  const float wa = wsh[a];
#pragma unroll
                  for (int i = 0; i < 16; ++i) acc[i] += wa * tmp[i];
                }
              }
            }
            float* sp = stage + ln * kStageRow + cbl * 32 + 16 * g;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<floatx4*>(sp + 4 * q) =
                  floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          // ---- add X, round once, coalesced store
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            const int row = TPI * j + lrow;
            const int tok = t0 + row;
            float dv[VEC], xv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
              *reinterpret_cast<floatx4*>(&dv[e]) =
                  *reinterpret_cast<const floatx4*>(stage + row * kStageRow + lcol + e);
            unpack_in<Tr>(b.x[h][j], xv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) dv[e] += xv[e];
            const u32x4 o = pack_out<Tr>(dv);
            if (full || tok < T) {
              *reinterpret_cast<u32x4*>(Y + tok * D + 64 * h + lcol) = o;
              if constexpr (POOL_OUT) {
                float fo[VEC];
                unpack_in<Tr>(o, fo);
#pragma unroll
                for (int e = 0; e < VEC; ++e) qs[h][e] += fo[e];
              }
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          if (more) load_x(h, tn);  // this half of X is consumed
        }
      };

      if (n_my > 0) {
#pragma unroll
        for (int h = 0; h < NH; ++h) load_x(h, first);
        load_u(b.u, first);
      }
      for (int it = 0; it < n_my; it += 2) {
        run_tile(it, b.u, u2);
        if (it + 1 < n_my) run_tile(it + 1, u2, b.u);
      }
    }

    if constexpr (POOL_OUT) {
      // token sums of the stored output: lanes sharing a channel -> waves in fixed order
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float v = qs[h][e];
#pragma unroll
          for (int off = LPT; off < kWave; off <<= 1) v += __shfl_xor(v, off, 64);
          if (lane < LPT) red[wave][64 * h + lcol + e] = v;
        }
      __syncthreads();
      if (tid < D) {
        const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        next_partials[(((size_t)x * S + s) * n_chunks + chunk) * D + tid] = v;
      }
    }
    __syncthreads();  // LDS (W^T, weights, staging, item id) is free for the next item
  }
}

static int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// ------------------------------------------------------------------------- launchers
template <class Tr, int D>
static hipError_t pool_partials_t(const void* K, const void* V, int S, int T, float* partials,
                                  int n_tiles, hipStream_t st) {
  dim3 grid(n_tiles, S, 2);
  hipLaunchKernelGGL((pool_partials_kernel<Tr, D>), grid, dim3(kBlock), 0, st,
                     (const typename Tr::elem*)K, (const typename Tr::elem*)V, T, partials,
                     n_tiles);
  return hipGetLastError();
}

hipError_t launch_pool_partials(const void* K, const void* V, int S, int T, int d, int dtype,
                                float* partials, int n_tiles, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (dtype == KVC_BF16)
    return d == 128 ? pool_partials_t<TrBF16, 128>(K, V, S, T, partials, n_tiles, st)
                    : pool_partials_t<TrBF16, 64>(K, V, S, T, partials, n_tiles, st);
  return d == 128 ? pool_partials_t<TrF32, 128>(K, V, S, T, partials, n_tiles, st)
                  : pool_partials_t<TrF32, 64>(K, V, S, T, partials, n_tiles, st);
}

hipError_t launch_reduce_pool(const float* partials, int n_tiles, int T, int S, int d,
                              float* q_out, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL((reduce_pool_kernel<128>), dim3(S), dim3(kWave), 0, st, partials,
                       n_tiles, T, q_out);
  else
    hipLaunchKernelGGL((reduce_pool_kernel<64>), dim3(S), dim3(kWave), 0, st, partials,
                       n_tiles, T, q_out);
  return hipGetLastError();
}

hipError_t launch_score(const float* partials, int n_tiles, int T, const float* q_in,
                        const float* desc, int S, int d, int A, float tau, float* q_ws,
                        float* w_ws, float* score_ws, uint8_t* mask_ws, float* q_out,
                        float* score_out, float* w_out, uint8_t* mask_out, int* ctr,
                        hipStream_t st) {
  (void)q_ws;
  if (S == 0) return hipSuccess;
  float* so = score_out ? score_out : score_ws;
  if (d == 128)
    hipLaunchKernelGGL((score_kernel<128>), dim3(S), dim3(kWave), 0, st, partials, n_tiles, T,
                       q_in, desc, A, tau, w_ws, mask_ws, q_out, so, w_out, mask_out, ctr);
  else
    hipLaunchKernelGGL((score_kernel<64>), dim3(S), dim3(kWave), 0, st, partials, n_tiles, T,
                       q_in, desc, A, tau, w_ws, mask_ws, q_out, so, w_out, mask_out, ctr);
  return hipGetLastError();
}

template <class Tr, int D, int NA, int KSC, int NFG>
static hipError_t correct_v(const void* K, const void* V, int S, int T, const void* U,
                            const void* W, int A, int r, int rp, const float* w,
                            const uint8_t* mask, const void* K_fb, const void* V_fb,
                            void* K_out, void* V_out, float* next_partials, int* ctr,
                            hipStream_t st) {
  using elem = typename Tr::elem;
  const int PADK = 16 / (int)sizeof(elem);
  const size_t lds = 4ull * 32 * kStageRow * sizeof(float) +
                     (size_t)A * D * (rp + PADK) * sizeof(elem);
  const int n_chunks = T > 0 ? ceil_div(T, kChunk) : 1;
  const int n_items = S * 2 * n_chunks;
  const int grid = n_items < 2 * device_cus() ? n_items : 2 * device_cus();
  auto k_pool = correct_kernel<Tr, D, NA, KSC, NFG, true>;
  auto k_plain = correct_kernel<Tr, D, NA, KSC, NFG, false>;
  if (lds > 48 * 1024) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_pool),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_plain),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  }
  hipLaunchKernelGGL(next_partials ? k_pool : k_plain, dim3(grid), dim3(kBlock), lds, st,
                     (const elem*)K, (const elem*)V, (const elem*)U, (const elem*)W, w, mask,
                     (const elem*)K_fb, (const elem*)V_fb, (elem*)K_out, (elem*)V_out,
                     next_partials, T, S, A, r, rp, n_chunks, n_items, ctr);
  return hipGetLastError();
}

// Compile-time variants for the common anchor shapes (bf16, r = 32 with A in {1, 2, 4, 6, 8},
// r = 16 or 64 with A = 4); every other shape takes the runtime-general kernel with the
// smallest register-resident fragment count that holds A * (rp / 2 / SLOT).
template <class Tr, int D>
static hipError_t correct_t(const void* K, const void* V, int S, int T, const void* U,
                            const void* W, int A, int r, const float* w, const uint8_t* mask,
                            const void* K_fb, const void* V_fb, void* K_out, void* V_out,
                            float* next_partials, int* ctr, hipStream_t st) {
  const int rp = (r + Tr::RPAD - 1) / Tr::RPAD * Tr::RPAD;
#define KVC_ARGS K, V, S, T, U, W, A, r, rp, w, mask, K_fb, V_fb, K_out, V_out, next_partials, ctr, st
  if constexpr (Tr::SLOT == 8 && D == 128) {
    if (r == 32) {
      switch (A) {
        case 1: return correct_v<Tr, D, 1, 2, 0>(KVC_ARGS);
        case 2: return correct_v<Tr, D, 2, 2, 0>(KVC_ARGS);
        case 4: return correct_v<Tr, D, 4, 2, 0>(KVC_ARGS);
        case 6: return correct_v<Tr, D, 6, 2, 0>(KVC_ARGS);
        case 8: return correct_v<Tr, D, 8, 2, 0>(KVC_ARGS);
        default: break;
      }
    }
    if (r == 16 && A == 4) return correct_v<Tr, D, 4, 1, 0>(KVC_ARGS);
    if (r == 64 && A == 4) return correct_v<Tr, D, 4, 4, 0>(KVC_ARGS);
  }
  const int nfrag = A * (rp / 2 / Tr::SLOT);
  constexpr int F0 = Tr::MAXF / 4, F1 = Tr::MAXF / 2, F2 = Tr::MAXF;
  if (nfrag <= F0) return correct_v<Tr, D, 0, 0, F0>(KVC_ARGS);
  if (nfrag <= F1) return correct_v<Tr, D, 0, 0, F1>(KVC_ARGS);
  return correct_v<Tr, D, 0, 0, F2>(KVC_ARGS);
#undef KVC_ARGS
}

hipError_t launch_correct(const void* K, const void* V, int S, int T, int d, int dtype,
                          const void* U, const void* W, int A, int r, const float* w,
                          const uint8_t* mask, const void* K_fb, const void* V_fb, void* K_out,
                          void* V_out, float* next_partials, int* ctr, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (dtype == KVC_BF16)
    return d == 128 ? correct_t<TrBF16, 128>(K, V, S, T, U, W, A, r, w, mask, K_fb, V_fb, K_out,
                                             V_out, next_partials, ctr, st)
                    : correct_t<TrBF16, 64>(K, V, S, T, U, W, A, r, w, mask, K_fb, V_fb, K_out,
                                            V_out, next_partials, ctr, st);
  return d == 128 ? correct_t<TrF32, 128>(K, V, S, T, U, W, A, r, w, mask, K_fb, V_fb, K_out,
                                          V_out, next_partials, ctr, st)
                  : correct_t<TrF32, 64>(K, V, S, T, U, W, A, r, w, mask, K_fb, V_fb, K_out,
                                         V_out, next_partials, ctr, st);
}

}  // namespace kvc
