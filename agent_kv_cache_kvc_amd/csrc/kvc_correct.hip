// Online correction of a reused shared-context KV cache on gfx950.
//
// KVCMAS, thelatestinai listing, Fig. 1: the reused cache of a shared segment is matched
// against the segment's online anchors (pooled descriptor vs. anchor descriptors, cosine),
// the anchors' low-rank corrections are combined with similarity weights (softmax) and
// added to K and V; a segment whose best match is below tau falls back to dense prefill.
//
// Kernels (all deterministic: fixed-order reductions, no floating-point atomics)
//   pool_partials_kernel  token sums of K and V per chunk                    (HBM stream)
//   reduce_pool_kernel    chunk sums -> q (the pooling entry point)
//   score_kernel          chunk sums or q -> cosines, softmax, score, mask  (one wave/segment)
//   correct_kernel        X' = X + sum_a w_a U_a W_a on MFMA, or copy-through (HBM stream);
//                         optionally the chunk sums of its output (the next pooled descriptor)
#include <hip/hip_runtime.h>

#include <type_traits>

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

// Tiles of 32 tokens per wave in one work item; the item's X stays in registers, 64 VGPRs
// per lane (bf16 d=128: 2 tiles, 256 tokens per item; f32 d=128: 1 tile, 128 tokens).
template <class Tr, int D>
constexpr int item_tiles() {
  return item_tiles_for(D * (int)sizeof(typename Tr::elem));
}

// Coalesced layout of a 32-token wave tile: access j of lane l covers token TPI j + l / LPT
// and channels 64 h + VEC (l % LPT) ... of half h (TPI = 64 / LPT tokens per access).
template <class Tr, int D>
struct Tile {
  static constexpr int NH = D / 64;        // 64-channel halves
  static constexpr int JN = Tr::LPT / 2;   // coalesced accesses per half per 32 tokens
  static constexpr int TPI = kWave / Tr::LPT;
  u32x4 v[NH][JN];
};

constexpr int kStageRow = 68;  // floats per staged token row (64 + 4: conflict-free rows)

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

// One wave's 32-token tile starting at token t0 of a [T, D] segment (zeros past T).  LAST: issued
// as non-temporal loads, so single-use lines leave L2 first (every read of K, V and the fallback
// caches in this file is a single use).
template <class Tr, int D, bool LAST = false>
__device__ __forceinline__ void load_tile(const typename Tr::elem* __restrict__ X, int t0, int T,
                                          int lrow, int lcol, Tile<Tr, D>& tile) {
  using TL = Tile<Tr, D>;
  auto ld = [](const typename Tr::elem* p) -> u32x4 {
    if constexpr (LAST) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
  };
  if (t0 + 32 <= T) {
#pragma unroll
    for (int h = 0; h < TL::NH; ++h)
#pragma unroll
      for (int j = 0; j < TL::JN; ++j)
        tile.v[h][j] = ld(X + (size_t)(t0 + TL::TPI * j + lrow) * D + 64 * h + lcol);
  } else {
#pragma unroll
    for (int h = 0; h < TL::NH; ++h)
#pragma unroll
      for (int j = 0; j < TL::JN; ++j) {
        const int tok = t0 + TL::TPI * j + lrow;
        tile.v[h][j] = tok < T ? ld(X + (size_t)tok * D + 64 * h + lcol) : u32x4{0u, 0u, 0u, 0u};
      }
  }
}

template <class Tr, int D>
__device__ __forceinline__ void add_tile(const Tile<Tr, D>& tile, float (&qs)[D / 64][Tr::VEC]) {
  using TL = Tile<Tr, D>;
#pragma unroll
  for (int h = 0; h < TL::NH; ++h)
#pragma unroll
    for (int j = 0; j < TL::JN; ++j) {
      float fv[Tr::VEC];
      unpack_in<Tr>(tile.v[h][j], fv);
#pragma unroll
      for (int e = 0; e < Tr::VEC; ++e) qs[h][e] += fv[e];
    }
}

// ------------------------------------------------------------------------- chunk sums
// A lane adds its tokens in (tile, access) order, then the lanes sharing a channel are added
// by a butterfly and the 4 waves in fixed order.  Every pooled sum in this file (inputs and
// outputs) takes this order over the same chunks, so the pooled descriptor of a cache does
// not depend on which pass computed it.
// The wave's sums of every channel into red[wave] (no barrier).
template <class Tr, int D>
__device__ __forceinline__ void wave_sums(float (&qs)[D / 64][Tr::VEC], float (*red)[D],
                                          int tid) {
  constexpr int NH = D / 64, VEC = Tr::VEC, LPT = Tr::LPT;
  const int lane = tid % kWave, wave = tid / kWave;
  const int lcol = VEC * (lane % LPT);
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float v = qs[h][e];
#pragma unroll
      for (int off = LPT; off < kWave; off <<= 1) v += __shfl_xor(v, off, 64);
      if (lane < LPT) red[wave][64 * h + lcol + e] = v;
    }
}

// The four waves' sums of channel tid (after a barrier that follows wave_sums).
template <int D>
__device__ __forceinline__ float join_sums(const float (*red)[D], int tid) {
  return ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

template <class Tr, int D>
__device__ __forceinline__ float finish_sums(float (&qs)[D / 64][Tr::VEC], float (*red)[D],
                                             int tid) {
  wave_sums<Tr, D>(qs, red, tid);
  __syncthreads();
  float out = 0.f;
  if (tid < D) out = join_sums<D>(red, tid);
  return out;  // valid for tid < D; the caller synchronises before `red` is written again
}

// grid (n_chunks, S, 2): chunk sums of K (z = 0) and V (z = 1).
template <class Tr, int D>
__global__ __launch_bounds__(kBlock) void pool_partials_kernel(
    const typename Tr::elem* __restrict__ K, const typename Tr::elem* __restrict__ V, int T,
    float* __restrict__ partials, int n_chunks) {
  constexpr int NT = item_tiles<Tr, D>();
  __shared__ float red[4][D];
  const int chunk = blockIdx.x, s = blockIdx.y, x = blockIdx.z, S = gridDim.y;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const typename Tr::elem* X = (x == 0 ? K : V) + (size_t)s * T * D;
  const int first = chunk * NT * kRowsPerPass + wave * 32;
  Tile<Tr, D> xr[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl)
    load_tile<Tr, D, true>(X, first + tl * kRowsPerPass, T, lane / Tr::LPT, Tr::VEC * (lane % Tr::LPT),
                     xr[tl]);
  float qs[D / 64][Tr::VEC];
#pragma unroll
  for (int h = 0; h < D / 64; ++h)
#pragma unroll
    for (int e = 0; e < Tr::VEC; ++e) qs[h][e] = 0.f;
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) add_tile<Tr, D>(xr[tl], qs);
  const float v = finish_sums<Tr, D>(qs, red, tid);
  if (tid < D) partials[(((size_t)x * S + s) * n_chunks + chunk) * D + tid] = v;
}

// ------------------------------------------------------------------------- matching
// Chunk sums -> pooled descriptor [mean K ; mean V]; one wave, lane holds channels
// lane + 64 i.  The sums are added in chunk order; loads go out 16 chunks at a time.
template <int D>
__device__ __forceinline__ void pooled_query(const float* __restrict__ partials, int n_chunks,
                                             int T, int s, int S, int lane,
                                             float (&q)[2 * D / kWave]) {
  constexpr int PER = 2 * D / kWave;
  constexpr int kJoin = 16;  // chunk sums loaded per round trip
  float sum[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sum[i] = 0.f;
  for (int c0 = 0; c0 < n_chunks; c0 += kJoin) {
    float v[kJoin][PER];
#pragma unroll
    for (int u = 0; u < kJoin; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = lane + kWave * i;
        const int x = c / D, ch = c % D;
        v[u][i] = (c0 + u < n_chunks)
                      ? partials[(((size_t)x * S + s) * n_chunks + c0 + u) * D + ch]
                      : 0.f;
      }
#pragma unroll
    for (int u = 0; u < kJoin; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (c0 + u < n_chunks) sum[i] += v[u][i];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) q[i] = T > 0 ? sum[i] / (float)T : 0.f;
}

// One wave: s_a = cos(q, desc_a) (0 when a norm is 0), w = softmax(s), score = max_a s_a
// (NaN if any s_a is NaN), fallback = !(score >= tau).  Lane a < A returns w_a.
template <int D>
__device__ __forceinline__ float segment_weights(const float (&q)[2 * D / kWave],
                                                 const float* __restrict__ desc, int s, int A,
                                                 float tau, int lane, float& score,
                                                 uint8_t& fall) {
  constexpr int PER = 2 * D / kWave;
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
  score = nan ? __uint_as_float(0x7fc00000u) : best;
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
  fall = !(score >= tau);
  float wv = 0.f;
#pragma unroll
  for (int a = 0; a < kMaxA; ++a)
    if (a == lane) wv = ex[a] / z;
  return wv;
}

template <int D>
__global__ __launch_bounds__(kWave) void reduce_pool_kernel(const float* __restrict__ partials,
                                                            int n_chunks, int T,
                                                            float* __restrict__ q_out) {
  constexpr int PER = 2 * D / kWave;
  const int s = blockIdx.x, S = gridDim.x, lane = threadIdx.x;
  float q[PER];
  pooled_query<D>(partials, n_chunks, T, s, S, lane, q);
#pragma unroll
  for (int i = 0; i < PER; ++i) q_out[(size_t)s * 2 * D + lane + kWave * i] = q[i];
}

// One wave per segment; also resets the work counter of the correction pass that follows.
template <int D>
__global__ __launch_bounds__(kWave) void score_kernel(
    const float* __restrict__ partials, int n_chunks, int T, const float* __restrict__ q_in,
    const float* __restrict__ desc, int A, float tau, float* __restrict__ w_ws,
    uint8_t* __restrict__ mask_ws, float* __restrict__ score_out, float* __restrict__ w_out,
    uint8_t* __restrict__ mask_out, int* __restrict__ ctr) {
  constexpr int PER = 2 * D / kWave;
  const int s = blockIdx.x, S = gridDim.x, lane = threadIdx.x;
  if (s == 0 && lane == 0) *ctr = 0;
  float q[PER];
  if (q_in != nullptr) {
#pragma unroll
    for (int i = 0; i < PER; ++i) q[i] = q_in[(size_t)s * 2 * D + lane + kWave * i];
  } else {
    pooled_query<D>(partials, n_chunks, T, s, S, lane, q);
  }
  float score;
  uint8_t fall;
  const float wv = segment_weights<D>(q, desc, s, A, tau, lane, score, fall);
  if (lane < A) {
    w_ws[(size_t)s * A + lane] = wv;
    if (w_out) w_out[(size_t)s * A + lane] = wv;
  }
  if (lane == 0) {
    mask_ws[s] = fall;
    mask_out[s] = fall;
    if (score_out) score_out[s] = score;
  }
}

// Online anchor pool: one workgroup (4 waves) per segment.  The pool's valid slots (the
// first count[s] of Vc) are scored like segment_weights, wave w taking slots w, w + 4, ... (the
// same per-wave arithmetic, so a score is bit-identical to kvc_correct's for the same
// descriptor); wave 0 then selects the A best (a NaN ranks last, ties go to the lower slot)
// and publishes their softmax weights (temperature 1) and slots; positions past the valid
// count repeat the best slot with weight 0.  score = best valid score (NaN if any valid score
// is NaN, -inf for an empty pool); fallback = !(score >= tau).  Resets *ctr.
template <int D>
__global__ __launch_bounds__(kBlock) void select_kernel(
    const float* __restrict__ partials, int n_chunks, int T, const float* __restrict__ q_in,
    const float* __restrict__ desc, const int* __restrict__ count, int Vc, int A, float tau,
    float* __restrict__ w_ws, int* __restrict__ slot_ws, uint8_t* __restrict__ mask_ws,
    float* __restrict__ score_out, float* __restrict__ w_out, int* __restrict__ slot_out,
    uint8_t* __restrict__ mask_out, int* __restrict__ ctr) {
  constexpr int PER = 2 * D / kWave;
  constexpr int NW = kBlock / kWave;
  __shared__ float sc_lds[kMaxPool];
  const int s = blockIdx.x, S = gridDim.x;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (s == 0 && threadIdx.x == 0) *ctr = 0;
  int n = count[s];
  n = n < 0 ? 0 : (n > Vc ? Vc : n);
  if (wave < n) {
    float q[PER];
    if (q_in != nullptr) {
#pragma unroll
      for (int i = 0; i < PER; ++i) q[i] = q_in[(size_t)s * 2 * D + lane + kWave * i];
    } else {
      pooled_query<D>(partials, n_chunks, T, s, S, lane, q);
    }
    float qq = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) qq += q[i] * q[i];
    const float nq = sqrtf(wave_sum(qq));
    for (int v = wave; v < n; v += NW) {
      const float* dv = desc + ((size_t)s * Vc + v) * 2 * D;
      float dd = 0.f, dq = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const float x = dv[lane + kWave * i];
        dd += x * x;
        dq += x * q[i];
      }
      dd = wave_sum(dd);
      dq = wave_sum(dq);
      const float den = nq * sqrtf(dd);
      if (lane == 0) sc_lds[v] = (den == 0.f) ? 0.f : dq / den;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float sc[kMaxPool];
  bool nan = false;
#pragma unroll
  for (int v = 0; v < kMaxPool; ++v) {
    sc[v] = v < n ? sc_lds[v] : 0.f;
    nan |= v < n && (sc[v] != sc[v]);
  }
  const int nsel = A < n ? A : n;
  uint32_t taken = 0u;
  int sel[kMaxPool];
  float ss[kMaxPool];
#pragma unroll
  for (int i = 0; i < kMaxPool; ++i) {
    sel[i] = 0;
    ss[i] = 0.f;
    if (i < nsel) {
      int best = -1;
      float bv = 0.f;
#pragma unroll
      for (int v = 0; v < kMaxPool; ++v) {
        if (v < n && !((taken >> v) & 1u)) {
          const float c = sc[v];
          if (best < 0 || (!(c != c) && ((bv != bv) || c > bv))) {
            best = v;
            bv = c;
          }
        }
      }
      sel[i] = best;
      ss[i] = bv;
      taken |= 1u << best;
    }
  }
  const float score = n == 0 ? -INFINITY : (nan ? __uint_as_float(0x7fc00000u) : ss[0]);
  float ex[kMaxPool];
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPool; ++i) {
    ex[i] = 0.f;
    if (i < nsel) {
      ex[i] = expf(ss[i] - ss[0]);
      z += ex[i];
    }
  }
  float wv = 0.f;
  int sv = 0;
#pragma unroll
  for (int i = 0; i < kMaxPool; ++i)
    if (i == lane) {
      wv = i < nsel ? ex[i] / z : 0.f;
      sv = i < nsel ? sel[i] : sel[0];
    }
  const uint8_t fall = !(score >= tau);
  if (lane < A) {
    w_ws[(size_t)s * A + lane] = wv;
    slot_ws[(size_t)s * A + lane] = sv;
    if (w_out) w_out[(size_t)s * A + lane] = wv;
    if (slot_out) slot_out[(size_t)s * A + lane] = sv;
  }
  if (lane == 0) {
    mask_ws[s] = fall;
    mask_out[s] = fall;
    if (score_out) score_out[s] = score;
  }
}

// ------------------------------------------------------------------------- correction
// Persistent workgroups (4 waves) take work items from a counter.  A work item is
// (segment, K|V, chunk of NT x 128 tokens); each wave owns NT tiles of 32 tokens, loads
// them into registers at the start of the item and keeps them there until X' is stored.
//
// MFMA: (delta X)^T = W^T U^T per 32-channel block; A operand = W_a^T staged in LDS (rows in
// operand order, see cinv32), B operand = U_a rows (8 consecutive k per lane, straight from
// HBM); result register i of lane l = (token l % 32, channel 16 (l / 32) + i).  Each anchor's
// product is finished in float32 and scaled by its weight, so w never passes through bf16.
// k layout: r is padded to rp (multiple of 2*SLOT); lane half g covers k in
// [g*rp/2, (g+1)*rp/2), MFMA step ks takes SLOT consecutive k from there.  The MFMA result
// goes through a per-wave LDS tile [32][64 + 4] floats to meet the coalesced layout of X;
// the next tile's U (double-buffered) is requested before the current tile's MFMAs.

struct CorrectArgs {
  const void* K;
  const void* V;
  const void* U;
  const void* W;
  const float* w_ws;       // [S][A] weights (from the matching kernel)
  const uint8_t* mask;     // [S] fallback flags (from the matching kernel)
  const void* K_fb;
  const void* V_fb;
  void* K_out;
  void* V_out;
  float* next_partials;    // chunk sums of the output, or null
  int* ctr;                // work counter (reset by the matching kernel)
  const int* slot_ws;      // SEL: [S][A] pool slot of each selected anchor
  int Vc;                  // SEL: pool slots per segment (U, W hold Vc anchors per segment)
  int n_t;                 // MT: targets corrected from one read of the source
  const void* tU[kMaxTargets];   // MT: per-target factors, outputs and fallback caches; the
  const void* tW[kMaxTargets];   //     weights and flags of target j are w_ws + j S A and
  void* tK[kMaxTargets];         //     mask + j S
  void* tV[kMaxTargets];
  const void* tKfb[kMaxTargets];
  const void* tVfb[kMaxTargets];
  int T, S, A, r, rp, n_chunks, n_items;
};

// NA > 0: compile-time anchor count NA and MFMA steps per anchor KSC (r = 2 KSC SLOT);
// NA == 0: runtime A and r with up to NFG register-resident fragments.
// SEL: anchor a of segment s is pool slot slot_ws[s][a] of Vc slots per segment
// (the online anchor pool); otherwise anchor a is slot a of A.
// MT: each item's tiles of the source are read once and corrected for n_t
// targets in turn (one source, several agents), each with its own factors, weights, flag,
// output and fallback cache.
template <class Tr, int D, int NA, int KSC, int NFG, bool POOL_OUT, bool SEL = false,
          bool MT = false>
__global__ __launch_bounds__(kBlock, 2) void correct_kernel(CorrectArgs args) {
  static_assert(!(MT && (SEL || POOL_OUT)), "several targets: plain correction only");
  using elem = typename Tr::elem;
  using frag = typename Tr::frag;
  using TL = Tile<Tr, D>;
  constexpr bool FIX = NA > 0;
  constexpr int NF = FIX ? NA * KSC : NFG;
  constexpr int NT = item_tiles<Tr, D>();
  constexpr int VEC = Tr::VEC;
  constexpr int SLOT = Tr::SLOT;
  constexpr int LPT = Tr::LPT;
  constexpr int TPI = TL::TPI;
  constexpr int NH = TL::NH, JN = TL::JN;
  constexpr int PADK = 16 / sizeof(elem);
  // CMP (compact LDS, bf16 anchor counts of 6 and more at r = 32): W^T rows are stored
  // unpadded with their 16-byte chunks XOR-swizzled by bits 2-3 of the row (the 16 rows that
  // one quarter-wave reads then fall into 16 distinct bank groups), and the MFMA results are
  // staged one 32-channel block at a time.  Two workgroups then fit in a CU's 160 KB of LDS at
  // A = 6 (about 70 KB each); at A = 8 one does (about 87 KB), and the launcher sizes the
  // persistent grid from the occupancy it gets.
  constexpr bool CMP = NA >= 6 && SLOT == 8 && KSC == 2;
  constexpr int SROW = CMP ? 36 : kStageRow;  // floats per staged token row

  const elem* __restrict__ K = static_cast<const elem*>(args.K);
  const elem* __restrict__ V = static_cast<const elem*>(args.V);
  const elem* __restrict__ U = static_cast<const elem*>(args.U);
  const elem* __restrict__ W = static_cast<const elem*>(args.W);
  const elem* K_fb = static_cast<const elem*>(args.K_fb);
  const elem* V_fb = static_cast<const elem*>(args.V_fb);
  elem* K_out = static_cast<elem*>(args.K_out);
  elem* V_out = static_cast<elem*>(args.V_out);
  const int T = args.T, S = args.S, n_chunks = args.n_chunks;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ float wsh[kMaxA];
  __shared__ int ssl[kMaxA];
  __shared__ float red[4][D];
  __shared__ int s_item;
  __shared__ int s_mask;

  elem* wt = reinterpret_cast<elem*>(smem_raw + 4 * 32 * SROW * sizeof(float));
  const int A = FIX ? NA : args.A;
  const int r = FIX ? 2 * KSC * SLOT : args.r;
  const int rp = FIX ? 2 * KSC * SLOT : args.rp;
  const int RS = rp + PADK;
  const int half = rp / 2;
  // LDS element of W^T row `row` (operand order), rank index k
  auto widx = [&](int row, int k) -> int {
    if constexpr (CMP) return row * rp + ((((k >> 3) ^ (row >> 2)) & 3) << 3) + (k & 7);
    else return row * RS + k;
  };
  const int KS = FIX ? KSC : half / SLOT;  // MFMA steps per anchor
  const int nfrag = A * KS;
  const bool uvec = FIX || (r % VEC) == 0;
  const int n_ci = 2 * n_chunks;             // items per segment
  const int nslot = SEL ? args.Vc : A;       // anchors stored per segment
  int* const ctr = args.ctr;
  const int n_items = args.n_items;
  if (threadIdx.x == 0) s_item = atomicAdd(ctr, 1);
  __syncthreads();
  int item = __builtin_amdgcn_readfirstlane(s_item);
  // POOL_OUT: an item leaves its waves' chunk sums in `red`; they are joined and stored after
  // the item's closing barrier, at the top of the loop (before the next item's first barrier,
  // after which `red` may be written again)
  [[maybe_unused]] long long pend = -1;  // (x S + s) n_chunks + chunk of the item whose sums wait
  for (;;) {
    // lane-derived values are recomputed per item (kept out of the loop-carried registers)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    if constexpr (POOL_OUT) {
      if (pend >= 0 && tid < D) args.next_partials[pend * D + tid] = join_sums<D>(red, tid);
    }
    if (item >= n_items) break;
    // the next item is requested now and read at the end of this one (the counter's round
    // trip overlaps the item)
    int nxt = 0;
    if (tid == 0) nxt = atomicAdd(ctr, 1);
    {
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane >> 5, ln = lane & 31;
    float* stage = reinterpret_cast<float*>(smem_raw) + wave * 32 * SROW;
    const int lrow = lane / LPT;               // token within a coalesced access
    const int lcol = VEC * (lane % LPT);       // channel offset within a half row

    // items run through the segments (and each segment's chunks) in the reverse of the
    // pooling kernel's order, so the first ones read what that kernel read last
    const int rs = item / n_ci;
    const int s = S - 1 - rs;
    const int ci = n_ci - 1 - (item - rs * n_ci);
    const int x = ci / n_chunks, chunk = ci - x * n_chunks;
    const size_t seg = (size_t)s * T * D;
    const elem* X = (x == 0 ? K : V) + seg;
    elem* Y = (x == 0 ? K_out : V_out) + seg;
    const elem* Xfb = (x == 0 ? K_fb : V_fb);
    const int first = chunk * NT * kRowsPerPass + wave * 32;
    const int n_my =
        first < T ? min(NT, (T - first + kRowsPerPass - 1) / kRowsPerPass) : 0;

    // ---- this wave's tiles of X, held in registers for the whole item (a segment already
    //      known to fall back to a fallback cache loads that cache instead)
    const bool fb_known = !MT && Xfb != nullptr && args.mask[s] != 0;
    const elem* Xsrc = fb_known ? Xfb + seg : X;
    TL xr[NT];
#pragma unroll
    for (int tl = 0; tl < NT; ++tl)
      load_tile<Tr, D, true>(Xsrc, first + tl * kRowsPerPass, T, lrow, lcol, xr[tl]);

    float qs[NH][VEC];
    if constexpr (POOL_OUT) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) qs[h][e] = 0.f;
    }

    // one target, or (MT) each target in turn on the same source tiles
    for (int tj = 0; tj < (MT ? args.n_t : 1); ++tj) {
    const elem* Ut = U;
    const elem* Wt = W;
    elem* Yt = Y;
    const elem* Xfbt = Xfb;
    const float* w_src = args.w_ws;
    const uint8_t* m_src = args.mask;
    if constexpr (MT) {
      Ut = static_cast<const elem*>(args.tU[tj]);
      Wt = static_cast<const elem*>(args.tW[tj]);
      Yt = static_cast<elem*>(x == 0 ? args.tK[tj] : args.tV[tj]) + seg;
      Xfbt = static_cast<const elem*>(x == 0 ? args.tKfb[tj] : args.tVfb[tj]);
      w_src += (size_t)tj * S * A;
      m_src += (size_t)tj * S;
    }

    if constexpr (SEL) {
      if (tid < A) ssl[tid] = args.slot_ws[(size_t)s * A + tid];
      __syncthreads();
    }

    // ---- stage W_a^T of this segment in LDS, rows in MFMA operand order (zero for k >= r); a
    //      falling-back segment stages nothing (its factors are not read)
    const bool pre_masked = m_src[s] != 0;  // same address in every lane
    if (FIX && SLOT == 8 && !pre_masked) {
      // bf16, r a multiple of 8: each step takes an 8 x 8 block (rank indices 8 kb .., channels
      // 8 cg ..; 16-byte coalesced loads along the channels), transposes it in registers and
      // writes 8 operand rows of 8 rank indices as 16-byte LDS stores
      const elem* Wseg = Wt + ((size_t)x * S + s) * nslot * r * D;
      constexpr int CGN = D / 8, KBN = FIX ? 2 * KSC * SLOT / 8 : 1;
      for (int q = tid; q < NA * KBN * CGN; q += kBlock) {
        const int cg = q % CGN, kb = (q / CGN) % KBN, a = q / (CGN * KBN);
        const elem* src = Wseg + ((size_t)(SEL ? ssl[a] : a) * r + 8 * kb) * D + 8 * cg;
        u32x4 in[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) in[i] = *reinterpret_cast<const u32x4*>(src + (size_t)i * D);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t lo = in[2 * k][j >> 1], hi = in[2 * k + 1][j >> 1];
            o[k] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          const int c = 8 * cg + j;
          *reinterpret_cast<u32x4*>(&wt[widx(a * D + (c & ~31) + cinv32(c & 31), 8 * kb)]) = o;
        }
      }
    } else if (!pre_masked) {
      const elem* Wseg = Wt + ((size_t)x * S + s) * nslot * r * D;
      const int n_w = A * r * (D / VEC);
      for (int q = tid; q < n_w; q += kBlock) {
        // k varies fastest across lanes, so the transposed LDS writes are contiguous
        const int k = q % r;
        const int rest = q / r;
        const int c0 = (rest % (D / VEC)) * VEC;
        const int a = rest / (D / VEC);
        elem v[VEC];
        *reinterpret_cast<u32x4*>(v) =
            *reinterpret_cast<const u32x4*>(Wseg + ((size_t)(SEL ? ssl[a] : a) * r + k) * D + c0);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int c = c0 + j;
          wt[widx(a * D + (c & ~31) + cinv32(c & 31), k)] = v[j];
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
    }

    {
      if (tid == 0) s_mask = m_src[s];
      if (tid < A) wsh[tid] = w_src[(size_t)s * A + tid];
    }
    __syncthreads();
    const bool masked = s_mask != 0;

    if (MT && masked) {
      // dense-prefill stand-in of this target: its fallback cache (copied tile by tile, the
      // source tiles stay in registers for the next target) or the source
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        const int t0 = first + tl * kRowsPerPass;
        if (tl < n_my) {
          TL fb;
          if (Xfbt != nullptr) load_tile<Tr, D, true>(Xfbt + seg, t0, T, lrow, lcol, fb);
          const TL& src = Xfbt != nullptr ? fb : xr[tl];
#pragma unroll
          for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int j = 0; j < JN; ++j) {
              const int tok = t0 + TPI * j + lrow;
              if (tok < T)
                __builtin_nontemporal_store(
                    src.v[h][j], reinterpret_cast<u32x4*>(Yt + (size_t)tok * D + 64 * h + lcol));
            }
        }
      }
    } else if (masked) {
      // dense-prefill stand-in: the fallback cache, or the source, bit for bit
      if (Xfb != nullptr && !fb_known) {
#pragma unroll
        for (int tl = 0; tl < NT; ++tl)
          load_tile<Tr, D, true>(Xfb + seg, first + tl * kRowsPerPass, T, lrow, lcol, xr[tl]);
      }
      const bool store = Xfb != nullptr || Y != X;  // in place with no fallback: unchanged
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        const int t0 = first + tl * kRowsPerPass;
        if (tl < n_my) {
#pragma unroll
          for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int j = 0; j < JN; ++j) {
              const int tok = t0 + TPI * j + lrow;
              if (tok < T) {
                if (store)  // non-temporal: the output is not read again by this kernel
                  __builtin_nontemporal_store(
                      xr[tl].v[h][j], reinterpret_cast<u32x4*>(Y + (size_t)tok * D + 64 * h + lcol));
                if constexpr (POOL_OUT) {
                  float fv[VEC];
                  unpack_in<Tr>(xr[tl].v[h][j], fv);
#pragma unroll
                  for (int e = 0; e < VEC; ++e) qs[h][e] += fv[e];
                }
              }
            }
        }
      }
    } else {
      const elem* Useg = Ut + ((size_t)x * S + s) * nslot * (size_t)T * r;
      auto load_u = [&](frag (&dst)[NF], int t0) {
        const int t = t0 + ln;
        if (FIX && t0 + 32 <= T) {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const int a = f / KS, ks = f - a * KS;
            const elem* up =
                Useg + ((size_t)(SEL ? ssl[a] : a) * T + t) * r + g * half + ks * SLOT;
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
            const elem* up = Useg + ((size_t)(SEL ? ssl[a] : a) * T + t) * r + k0;
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

      // one tile of this wave: MFMAs on `cu`; the next tile's U goes to `nu` first
      auto run_tile = [&](auto tl_c, frag (&cu)[NF], frag (&nu)[NF]) {
        constexpr int tl = decltype(tl_c)::value;
        const int t0 = first + tl * kRowsPerPass;
        if constexpr (CMP) {
          // one U buffer live at a time (registers): this tile's U is loaded here
          if (tl > 0) load_u(cu, t0);
        } else {
          if (tl + 1 < n_my) load_u(nu, t0 + kRowsPerPass);
        }
        const bool full = t0 + 32 <= T;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          // ---- two 32-channel MFMA blocks of this half into the staging tile
#pragma unroll 1
          for (int cbl = 0; cbl < 2; ++cbl) {
            const int cb = 2 * h + cbl;
            const elem* ap = wt + (cb * 32 + ln) * RS + g * half;  // padded layout only
            floatx16 acc, tmp;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              if (FIX || f < nfrag) {
                const int a = f / KS, ks = f - a * KS;
                frag af;
                if constexpr (CMP) {
                  af = *reinterpret_cast<const u32x4*>(
                      wt + widx(a * D + cb * 32 + ln, g * half + ks * SLOT));
                } else if constexpr (SLOT == 8) {
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
            float* sp = stage + ln * SROW + (CMP ? 0 : cbl * 32) + 16 * g;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<floatx4*>(sp + 4 * q) =
                  floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
            if constexpr (CMP) {
              // this block's 32 channels: the lanes that hold them add X, round and store
              __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
              for (int j = 0; j < JN; ++j) {
                const int row = TPI * j + lrow;
                const int tok = t0 + row;
                if ((lcol >> 5) == cbl) {
                  float dv[VEC], xv[VEC];
#pragma unroll
                  for (int e = 0; e < VEC; e += 4)
                    *reinterpret_cast<floatx4*>(&dv[e]) = *reinterpret_cast<const floatx4*>(
                        stage + row * SROW + (lcol & 31) + e);
                  unpack_in<Tr>(xr[tl].v[h][j], xv);
#pragma unroll
                  for (int e = 0; e < VEC; ++e) dv[e] += xv[e];
                  const u32x4 o = pack_out<Tr>(dv);
                  if (full || tok < T) {
                    // an ordinary store: the two 64-byte halves of each 128-byte line are
                    // written by the two blocks and meet in L2 (as non-temporal stores they
                    // went out as separate half-line writes, measured 5% slower)
                    *reinterpret_cast<u32x4*>(Yt + (size_t)tok * D + 64 * h + lcol) = o;
                    if constexpr (POOL_OUT) {
                      float fo[VEC];
                      unpack_in<Tr>(o, fo);
#pragma unroll
                      for (int e = 0; e < VEC; ++e) qs[h][e] += fo[e];
                    }
                  }
                }
              }
              __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            }
          }
          if constexpr (CMP) continue;
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
            unpack_in<Tr>(xr[tl].v[h][j], xv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) dv[e] += xv[e];
            const u32x4 o = pack_out<Tr>(dv);
            if (full || tok < T) {
              __builtin_nontemporal_store(  // the output is not read again here
                  o, reinterpret_cast<u32x4*>(Yt + (size_t)tok * D + 64 * h + lcol));
              if constexpr (POOL_OUT) {
                float fo[VEC];
                unpack_in<Tr>(o, fo);
#pragma unroll
                for (int e = 0; e < VEC; ++e) qs[h][e] += fo[e];
              }
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        }
      };

      frag ua[NF], ub[NF];
      if (n_my > 0) {
        load_u(ua, first);
        run_tile(std::integral_constant<int, 0>{}, ua, ub);
      }
      if constexpr (NT >= 2) {
        if (n_my > 1) run_tile(std::integral_constant<int, 1>{}, ub, ua);
      }
      if constexpr (NT >= 4) {
        if (n_my > 2) run_tile(std::integral_constant<int, 2>{}, ua, ub);
        if (n_my > 3) run_tile(std::integral_constant<int, 3>{}, ub, ua);
      }
    }

    if constexpr (MT) __syncthreads();  // LDS (W^T, weights) is free for the next target
    }

    if constexpr (POOL_OUT) {
      // token sums of the stored output, in the order of the input chunk sums
      wave_sums<Tr, D>(qs, red, tid);
      pend = ((long long)x * S + s) * n_chunks + chunk;
    }
    }
    if (tid == 0) s_item = nxt;
    __syncthreads();  // LDS (W^T, weights, staging, chunk sums, item id) is free for the next item
    item = __builtin_amdgcn_readfirstlane(s_item);
  }
}

static int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Workgroups of `k` (kBlock threads, `lds` bytes of dynamic LDS) resident per CU, from the
// runtime's occupancy calculator (at least 1; at most 2, the persistent grid's target).  Cached
// per kernel and LDS size.
static int resident_per_cu(const void* k, size_t lds) {
  struct Entry { const void* k; size_t lds; int dev; int n; };
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  (void)hipGetDevice(&dev);
  for (int i = 0; i < used; ++i)
    if (cache[i].k == k && cache[i].lds == lds && cache[i].dev == dev) return cache[i].n;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kBlock, lds) != hipSuccess || n < 1)
    n = 1;
  if (n > 2) n = 2;
  if (used < 64) cache[used++] = Entry{k, lds, dev, n};
  return n;
}

// ------------------------------------------------------------------------- launchers
template <class Tr, int D>
static hipError_t pool_partials_t(const void* K, const void* V, int S, int T, float* partials,
                                  int n_chunks, hipStream_t st) {
  dim3 grid(n_chunks, S, 2);
  hipLaunchKernelGGL((pool_partials_kernel<Tr, D>), grid, dim3(kBlock), 0, st,
                     (const typename Tr::elem*)K, (const typename Tr::elem*)V, T, partials,
                     n_chunks);
  return hipGetLastError();
}

hipError_t launch_pool_partials(const void* K, const void* V, int S, int T, int d, int dtype,
                                float* partials, int n_chunks, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (dtype == KVC_BF16)
    return d == 128 ? pool_partials_t<TrBF16, 128>(K, V, S, T, partials, n_chunks, st)
                    : pool_partials_t<TrBF16, 64>(K, V, S, T, partials, n_chunks, st);
  return d == 128 ? pool_partials_t<TrF32, 128>(K, V, S, T, partials, n_chunks, st)
                  : pool_partials_t<TrF32, 64>(K, V, S, T, partials, n_chunks, st);
}

hipError_t launch_reduce_pool(const float* partials, int n_chunks, int T, int S, int d,
                              float* q_out, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL((reduce_pool_kernel<128>), dim3(S), dim3(kWave), 0, st, partials,
                       n_chunks, T, q_out);
  else
    hipLaunchKernelGGL((reduce_pool_kernel<64>), dim3(S), dim3(kWave), 0, st, partials,
                       n_chunks, T, q_out);
  return hipGetLastError();
}

hipError_t launch_score(const float* partials, int n_chunks, int T, const float* q_in,
                        const float* desc, int S, int d, int A, float tau, float* w_ws,
                        uint8_t* mask_ws, float* score_out, float* w_out, uint8_t* mask_out,
                        int* ctr, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL((score_kernel<128>), dim3(S), dim3(kWave), 0, st, partials, n_chunks,
                       T, q_in, desc, A, tau, w_ws, mask_ws, score_out, w_out, mask_out, ctr);
  else
    hipLaunchKernelGGL((score_kernel<64>), dim3(S), dim3(kWave), 0, st, partials, n_chunks,
                       T, q_in, desc, A, tau, w_ws, mask_ws, score_out, w_out, mask_out, ctr);
  return hipGetLastError();
}

hipError_t launch_select(const float* partials, int n_chunks, int T, const float* q_in,
                         const float* desc, const int* count, int Vc, int S, int d, int A,
                         float tau, float* w_ws, int* slot_ws, uint8_t* mask_ws,
                         float* score_out, float* w_out, int* slot_out, uint8_t* mask_out,
                         int* ctr, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL((select_kernel<128>), dim3(S), dim3(kBlock), 0, st, partials, n_chunks, T,
                       q_in, desc, count, Vc, A, tau, w_ws, slot_ws, mask_ws, score_out, w_out,
                       slot_out, mask_out, ctr);
  else
    hipLaunchKernelGGL((select_kernel<64>), dim3(S), dim3(kBlock), 0, st, partials, n_chunks, T,
                       q_in, desc, count, Vc, A, tau, w_ws, slot_ws, mask_ws, score_out, w_out,
                       slot_out, mask_out, ctr);
  return hipGetLastError();
}

template <class Tr, int D, int NA, int KSC, int NFG, bool SEL = false, bool MT = false>
static hipError_t correct_v(const CorrectLaunch& L, hipStream_t st) {
  const int PADK = 16 / (int)sizeof(typename Tr::elem);
  constexpr bool CMP = NA >= 6 && Tr::SLOT == 8 && KSC == 2;  // as in correct_kernel
  const size_t lds = 4ull * 32 * (CMP ? 36 : kStageRow) * sizeof(float) +
                     (size_t)L.A * D * (L.rp + (CMP ? 0 : PADK)) * sizeof(typename Tr::elem);
  CorrectArgs a{};
  a.K = L.K;
  a.V = L.V;
  a.U = L.U;
  a.W = L.W;
  a.w_ws = L.w_ws;
  a.mask = L.mask_ws;
  a.K_fb = L.K_fb;
  a.V_fb = L.V_fb;
  a.K_out = L.K_out;
  a.V_out = L.V_out;
  a.next_partials = L.next_partials;
  a.ctr = L.ctr;
  a.slot_ws = L.slot_ws;
  a.Vc = L.Vc;
  a.n_t = L.n_t;
  for (int j = 0; j < kMaxTargets; ++j) {
    a.tU[j] = L.tU[j];
    a.tW[j] = L.tW[j];
    a.tK[j] = L.tK[j];
    a.tV[j] = L.tV[j];
    a.tKfb[j] = L.tKfb[j];
    a.tVfb[j] = L.tVfb[j];
  }
  a.T = L.T;
  a.S = L.S;
  a.A = L.A;
  a.r = L.r;
  a.rp = L.rp;
  a.n_chunks = chunks_of(L.T, L.d, L.dtype);
  a.n_items = L.S * 2 * a.n_chunks;
  const bool pool = L.next_partials != nullptr;
  void (*k)(CorrectArgs);
  if constexpr (SEL) {
    k = correct_kernel<Tr, D, NA, KSC, NFG, false, true>;
  } else if constexpr (MT) {
    k = correct_kernel<Tr, D, NA, KSC, NFG, false, false, true>;
  } else {
    k = pool ? correct_kernel<Tr, D, NA, KSC, NFG, true> : correct_kernel<Tr, D, NA, KSC, NFG, false>;
  }
  if (lds > 48 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int cap = resident_per_cu(reinterpret_cast<const void*>(k), lds) * device_cus();
  const int grid = a.n_items < cap ? a.n_items : cap;
  hipLaunchKernelGGL(k, dim3(grid), dim3(kBlock), lds, st, a);
  return hipGetLastError();
}

// Compile-time variants for the common anchor shapes (bf16, r = 32 with A in {1, 2, 4, 6, 8},
// r = 16 or 64 with A = 4); every other shape takes the runtime-general kernel with the
// smallest register-resident fragment count that holds A * (rp / 2 / SLOT).
template <class Tr, int D>
static hipError_t correct_t(CorrectLaunch L, hipStream_t st) {
  L.rp = (L.r + Tr::RPAD - 1) / Tr::RPAD * Tr::RPAD;
  if constexpr (Tr::SLOT == 8 && D == 128) {
    if (L.r == 32) {
      switch (L.A) {
        case 1: return correct_v<Tr, D, 1, 2, 0>(L, st);
        case 2: return correct_v<Tr, D, 2, 2, 0>(L, st);
        case 4: return correct_v<Tr, D, 4, 2, 0>(L, st);
        case 6: return correct_v<Tr, D, 6, 2, 0>(L, st);
        case 8: return correct_v<Tr, D, 8, 2, 0>(L, st);
        default: break;
      }
    }
    if (L.r == 16 && L.A == 4) return correct_v<Tr, D, 4, 1, 0>(L, st);
    if (L.r == 64 && L.A == 4) return correct_v<Tr, D, 4, 4, 0>(L, st);
  }
  const int nfrag = L.A * (L.rp / 2 / Tr::SLOT);
  constexpr int F0 = Tr::MAXF / 4, F1 = Tr::MAXF / 2, F2 = Tr::MAXF;
  if (nfrag <= F0) return correct_v<Tr, D, 0, 0, F0>(L, st);
  if (nfrag <= F1) return correct_v<Tr, D, 0, 0, F1>(L, st);
  return correct_v<Tr, D, 0, 0, F2>(L, st);
}

// The pooled correction (slot indirection): the 8B-shaped anchors (bf16, d = 128, A = 4,
// r = 32) take their compile-time variant, every other shape the runtime-general kernel.
template <class Tr, int D>
static hipError_t correct_sel_t(CorrectLaunch L, hipStream_t st) {
  L.rp = (L.r + Tr::RPAD - 1) / Tr::RPAD * Tr::RPAD;
  if constexpr (Tr::SLOT == 8 && D == 128) {
    if (L.r == 32 && L.A == 4) return correct_v<Tr, D, 4, 2, 0, true>(L, st);
  }
  const int nfrag = L.A * (L.rp / 2 / Tr::SLOT);
  constexpr int F0 = Tr::MAXF / 4, F1 = Tr::MAXF / 2, F2 = Tr::MAXF;
  if (nfrag <= F0) return correct_v<Tr, D, 0, 0, F0, true>(L, st);
  if (nfrag <= F1) return correct_v<Tr, D, 0, 0, F1, true>(L, st);
  return correct_v<Tr, D, 0, 0, F2, true>(L, st);
}

// The multi-target correction: the 8B-shaped anchors (bf16, d = 128, A = 4, r = 32) take
// their compile-time variant, every other shape the runtime-general kernel.
template <class Tr, int D>
static hipError_t correct_mt_t(CorrectLaunch L, hipStream_t st) {
  L.rp = (L.r + Tr::RPAD - 1) / Tr::RPAD * Tr::RPAD;
  if constexpr (Tr::SLOT == 8 && D == 128) {
    if (L.r == 32 && L.A == 4) return correct_v<Tr, D, 4, 2, 0, false, true>(L, st);
  }
  const int nfrag = L.A * (L.rp / 2 / Tr::SLOT);
  constexpr int F0 = Tr::MAXF / 4, F1 = Tr::MAXF / 2, F2 = Tr::MAXF;
  if (nfrag <= F0) return correct_v<Tr, D, 0, 0, F0, false, true>(L, st);
  if (nfrag <= F1) return correct_v<Tr, D, 0, 0, F1, false, true>(L, st);
  return correct_v<Tr, D, 0, 0, F2, false, true>(L, st);
}

hipError_t launch_correct(const CorrectLaunch& L, hipStream_t st) {
  if (L.S == 0) return hipSuccess;
  if (L.n_t > 0) {
    if (L.dtype == KVC_BF16)
      return L.d == 128 ? correct_mt_t<TrBF16, 128>(L, st) : correct_mt_t<TrBF16, 64>(L, st);
    return L.d == 128 ? correct_mt_t<TrF32, 128>(L, st) : correct_mt_t<TrF32, 64>(L, st);
  }
  if (L.slot_ws != nullptr) {
    if (L.dtype == KVC_BF16)
      return L.d == 128 ? correct_sel_t<TrBF16, 128>(L, st) : correct_sel_t<TrBF16, 64>(L, st);
    return L.d == 128 ? correct_sel_t<TrF32, 128>(L, st) : correct_sel_t<TrF32, 64>(L, st);
  }
  if (L.dtype == KVC_BF16)
    return L.d == 128 ? correct_t<TrBF16, 128>(L, st) : correct_t<TrBF16, 64>(L, st);
  return L.d == 128 ? correct_t<TrF32, 128>(L, st) : correct_t<TrF32, 64>(L, st);
}

}  // namespace kvc
