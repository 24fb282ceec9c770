// Correction for every anchor shape outside the specialised correction kernel's register and
// LDS budget (1 <= r <= d, A * r <= 256 in general; the specialised kernel takes A <= 16 and
// r <= 64 with A * ceil(r/16) * 16 <= 256 for bf16, A * ceil(r/8) * 8 <= 64 for fp32).
//
// KVCMAS, thelatestinai listing, Fig. 1(b): the segment's anchors are matched by cosine
// similarity, combined with softmax weights, and their low-rank corrections are added to K
// and V; Fig. 1(a): a segment whose best match is below tau falls back.  Fig. 13 varies the
// delta rank r_delta up to the full head dimension.
//
// Kernels
//   score_general_kernel    q -> cosines of any number of anchors, softmax, score, flag
//                           (one wave per segment, the scores held in LDS)
//   correct_general_kernel  X' = X + sum_a w_a U_a W_a as ONE contraction over the anchors'
//                           concatenated rank index k = a r + j (K = A r <= 256):
//                           (delta X)^T = Wt^T U^T with Wt[k, :] = w_a W_a[j, :] formed in
//                           float32 and staged in LDS 64 rows of k at a time (bf16: split as
//                           hi + lo bf16, two MFMAs per step, so the weighted factor is carried
//                           to about 2^-17), U read straight from memory (16-byte rows when r is
//                           a multiple of 8, element by element otherwise); a falling-back
//                           segment is copied from the fallback cache (or the source).
// One workgroup per (128-token tile, segment, K|V); each wave owns 32 tokens and all d
// channels; results are stored once, rounded to nearest even.
#include <hip/hip_runtime.h>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kGenKC = 64;  // rows of the concatenated rank index staged per step

// Inverse of cmap32 (channel within a 32-block -> MFMA operand row)
__device__ __forceinline__ int gen_cinv32(int c) {
  return 8 * ((c >> 2) & 3) + 4 * (c >> 4) + (c & 3);
}

// sum over the wave, fixed butterfly order (every lane gets the same bits)
__device__ __forceinline__ float gen_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace

// One wave per segment: s_a = cos(q, desc_a) (0 when a norm is 0), w = softmax(s), score =
// max_a s_a (NaN if any s_a is NaN), fallback = !(score >= tau).  q: [S][2D] float32.
template <int D>
__global__ __launch_bounds__(kWave) void score_general_kernel(
    const float* __restrict__ q_in, const float* __restrict__ desc, int A, float tau,
    float* __restrict__ w_ws, uint8_t* __restrict__ mask_ws, float* __restrict__ score_out,
    float* __restrict__ w_out, uint8_t* __restrict__ mask_out) {
  constexpr int PER = 2 * D / kWave;
  __shared__ float sc[kMaxAnchorsGeneral];
  const int s = blockIdx.x, lane = threadIdx.x;
  float q[PER];
  float qq = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    q[i] = q_in[(size_t)s * 2 * D + lane + kWave * i];
    qq += q[i] * q[i];
  }
  const float nq = sqrtf(gen_wave_sum(qq));
  float best = -INFINITY;
  bool nan = false;
  for (int a = 0; a < A; ++a) {
    const float* da = desc + ((size_t)s * A + a) * 2 * D;
    float dd = 0.f, dq = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const float v = da[lane + kWave * i];
      dd += v * v;
      dq += v * q[i];
    }
    dd = gen_wave_sum(dd);
    dq = gen_wave_sum(dq);
    const float den = nq * sqrtf(dd);
    const float c = (den == 0.f) ? 0.f : dq / den;
    if (lane == 0) sc[a] = c;
    nan |= (c != c);
    best = fmaxf(best, c);
  }
  __syncthreads();
  const float score = nan ? __uint_as_float(0x7fc00000u) : best;
  // softmax: each lane's anchors a = lane + 64 i, the lane sums joined in a fixed order
  float z = 0.f;
  for (int a = lane; a < A; a += kWave) z += expf(sc[a] - score);
  z = gen_wave_sum(z);
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

struct GenArgs {
  const void* K;
  const void* V;
  const void* U;         // [2][S][nslot][T][r]
  const void* W;         // [2][S][nslot][r][D]
  const float* w_ws;     // [S][A]
  const uint8_t* mask;   // [S]
  const int* slot_ws;    // [S][A] pool slots of the selected anchors, or null (slot a = a)
  int nslot;             // anchors stored per segment (A, or the pool capacity)
  const void* K_fb;
  const void* V_fb;
  void* K_out;
  void* V_out;
  int T, S, A, r;
};

template <typename E, int D>
__global__ __launch_bounds__(kBlock) void correct_general_kernel(GenArgs g) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int NB = D / 32;                 // 32-channel MFMA blocks
  constexpr int KP = kGenKC + (BF ? 8 : 4);  // LDS row stride of the staged factor (elements)
  constexpr int EV = 16 / sizeof(E);         // elements per 16-byte access
  __shared__ __align__(16) E whi[D * KP];
  __shared__ __align__(16) E wlo[BF ? D * KP : 1];
  __shared__ float wsh[kMaxAnchorsGeneral];
  __shared__ int ssl[kMaxAnchorsGeneral];

  const int tile = blockIdx.x, s = blockIdx.y, x = blockIdx.z;
  const int T = g.T, S = g.S, A = g.A, r = g.r;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int ln = lane & 31, hg = lane >> 5;
  const size_t seg = (size_t)s * T * D;
  const E* X = static_cast<const E*>(x == 0 ? g.K : g.V) + seg;
  E* Y = static_cast<E*>(x == 0 ? g.K_out : g.V_out) + seg;
  const E* Xfb = static_cast<const E*>(x == 0 ? g.K_fb : g.V_fb);
  const int t0 = tile * kRowsPerPass + wave * 32;

  if (g.mask[s] != 0) {  // same address in every lane: the whole workgroup copies
    const E* src = Xfb != nullptr ? Xfb + seg : X;
    if (src == Y) return;  // in place without a fallback cache: unchanged
    const int first = tile * kRowsPerPass * D;
    const int last = min(T, (tile + 1) * kRowsPerPass) * D;
    for (int e = first + tid * EV; e < last; e += kBlock * EV)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src + e),
                                  reinterpret_cast<u32x4*>(Y + e));
    return;
  }

  for (int a = tid; a < A; a += kBlock) {
    wsh[a] = g.w_ws[(size_t)s * A + a];
    ssl[a] = g.slot_ws != nullptr ? g.slot_ws[(size_t)s * A + a] : a;
  }
  const E* Ubase = static_cast<const E*>(g.U) + ((size_t)x * S + s) * g.nslot * (size_t)T * r;
  const E* Wbase = static_cast<const E*>(g.W) + ((size_t)x * S + s) * g.nslot * (size_t)r * D;
  const int Kt = A * r;
  const int t = t0 + ln;  // this lane's token in the B operand and the result

  floatx16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;

  for (int kc = 0; kc < Kt; kc += kGenKC) {
    __syncthreads();  // weights and slots visible; the previous step's factor is consumed
    // ---- stage Wt rows [kc, kc + 64): channel c of row k at LDS row gen_cinv32 order
    for (int e = tid; e < kGenKC * D; e += kBlock) {
      const int kk = e / D, c = e % D;
      const int kg = kc + kk;
      float v = 0.f;
      if (kg < Kt) {
        const int a = kg / r, j = kg - a * r;
        float wv;
        if constexpr (BF) wv = bf16_to_f32(Wbase[((size_t)ssl[a] * r + j) * D + c]);
        else wv = Wbase[((size_t)ssl[a] * r + j) * D + c];
        v = wsh[a] * wv;
      }
      const int row = (c & ~31) + gen_cinv32(c & 31);
      if constexpr (BF) {
        const uint16_t h = f32_to_bf16(v);
        whi[row * KP + kk] = h;
        wlo[row * KP + kk] = f32_to_bf16(v - bf16_to_f32(h));
      } else {
        whi[row * KP + kk] = v;
      }
    }
    __syncthreads();
    if constexpr (BF) {
#pragma unroll 1
      for (int ks = 0; ks < kGenKC / 16; ++ks) {
        const int k0 = kc + 16 * ks + 8 * hg;  // this lane's 8 consecutive k
        u32x4 uf = {0u, 0u, 0u, 0u};
        if (t < T && k0 < Kt) {
          const int a0 = k0 / r, j0 = k0 - a0 * r;
          if ((r & 7) == 0) {  // 8 consecutive k of one anchor: one 16-byte row piece
            uf = *reinterpret_cast<const u32x4*>(Ubase + ((size_t)ssl[a0] * T + t) * r + j0);
          } else {
            uint16_t tmp[8];
            int a = a0, j = j0;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              tmp[q] = (k0 + q < Kt) ? Ubase[((size_t)ssl[a] * T + t) * r + j] : (uint16_t)0;
              if (++j == r) { j = 0; ++a; }
            }
            uf = *reinterpret_cast<const u32x4*>(tmp);
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int row = b * 32 + ln;
          const u32x4 ah = *reinterpret_cast<const u32x4*>(&whi[row * KP + 16 * ks + 8 * hg]);
          const u32x4 al = *reinterpret_cast<const u32x4*>(&wlo[row * KP + 16 * ks + 8 * hg]);
          acc[b] = mfma_bf16(ah, uf, acc[b]);
          acc[b] = mfma_bf16(al, uf, acc[b]);
        }
      }
    } else {
#pragma unroll 2
      for (int ks = 0; ks < kGenKC / 2; ++ks) {
        const int k = kc + 2 * ks + hg;
        float uf = 0.f;
        if (t < T && k < Kt) {
          const int a = k / r, j = k - a * r;
          uf = Ubase[((size_t)ssl[a] * T + t) * r + j];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float af = whi[(b * 32 + ln) * KP + 2 * ks + hg];
          acc[b] = mfma_f32(af, uf, acc[b]);
        }
      }
    }
  }

  // ---- epilogue: lane (token t, half hg) holds channels 32 b + 16 hg + i of block b
  if (t < T) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c0 = 32 * b + 16 * hg;
      const E* xp = X + (size_t)t * D + c0;
      E* yp = Y + (size_t)t * D + c0;
      if constexpr (BF) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        typedef float f2_t __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(xp + 8 * h);
          u32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float lo = __uint_as_float(raw[j] << 16) + acc[b][8 * h + 2 * j];
            const float hi = __uint_as_float(raw[j] & 0xffff0000u) + acc[b][8 * h + 2 * j + 1];
            o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{lo, hi}, bf16x2_t));
          }
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(yp + 8 * h));
        }
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          floatx4 v = *reinterpret_cast<const floatx4*>(xp + 4 * h);
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] += acc[b][4 * h + j];
          __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(yp + 4 * h));
        }
      }
    }
  }
}

hipError_t launch_score_general(const float* q, const float* desc, int S, int d, int A,
                                float tau, float* w_ws, uint8_t* mask_ws, float* score_out,
                                float* w_out, uint8_t* mask_out, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL((score_general_kernel<128>), dim3(S), dim3(kWave), 0, st, q, desc, A, tau,
                       w_ws, mask_ws, score_out, w_out, mask_out);
  else
    hipLaunchKernelGGL((score_general_kernel<64>), dim3(S), dim3(kWave), 0, st, q, desc, A, tau,
                       w_ws, mask_ws, score_out, w_out, mask_out);
  return hipGetLastError();
}

hipError_t launch_correct_general(const CorrectLaunch& L, hipStream_t st) {
  if (L.S == 0 || L.T == 0) return hipSuccess;
  GenArgs g{};
  g.K = L.K;
  g.V = L.V;
  g.U = L.U;
  g.W = L.W;
  g.w_ws = L.w_ws;
  g.mask = L.mask_ws;
  g.slot_ws = L.slot_ws;
  g.nslot = L.slot_ws != nullptr ? L.Vc : L.A;
  g.K_fb = L.K_fb;
  g.V_fb = L.V_fb;
  g.K_out = L.K_out;
  g.V_out = L.V_out;
  g.T = L.T;
  g.S = L.S;
  g.A = L.A;
  g.r = L.r;
  const dim3 grid(ceil_div(L.T, kRowsPerPass), L.S, 2);
  if (L.dtype == KVC_BF16) {
    if (L.d == 128)
      hipLaunchKernelGGL((correct_general_kernel<uint16_t, 128>), grid, dim3(kBlock), 0, st, g);
    else
      hipLaunchKernelGGL((correct_general_kernel<uint16_t, 64>), grid, dim3(kBlock), 0, st, g);
  } else {
    if (L.d == 128)
      hipLaunchKernelGGL((correct_general_kernel<float, 128>), grid, dim3(kBlock), 0, st, g);
    else
      hipLaunchKernelGGL((correct_general_kernel<float, 64>), grid, dim3(kBlock), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace kvc
