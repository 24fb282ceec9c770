// Float64 wave helpers (DPP moves and sums, lane reads) and the float32 multisection on
// Sturm counts of a symmetric tridiagonal matrix, shared by the eigensolvers of the fit
// (kvc_fit.hip) and of the warm-started refit (kvc_warm.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace kvc {

// lanes whose DPP source lies outside the row read 0
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const int2 h = __builtin_bit_cast(int2, x);
  int2 o;
  o.x = __builtin_amdgcn_mov_dpp(h.x, CTRL, 0xf, 0xf, true);
  o.y = __builtin_amdgcn_mov_dpp(h.y, CTRL, 0xf, 0xf, true);
  return __builtin_bit_cast(double, o);
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}

// sum over aligned groups of N lanes (4, 8 or 16); every lane of the group gets it
template <int N>
__device__ __forceinline__ double group_sum_d(double v) {
  v += dpp_d<0xB1>(v);  // quad_perm [1, 0, 3, 2]
  v += dpp_d<0x4E>(v);  // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) v += dpp_d<0x141>(v);   // row_half_mirror
  if constexpr (N >= 16) v += dpp_d<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ double readlane_d(double v, int lane) {
  const int2 h = __builtin_bit_cast(int2, v);
  int2 o;
  o.x = __builtin_amdgcn_readlane(h.x, lane);
  o.y = __builtin_amdgcn_readlane(h.y, lane);
  return __builtin_bit_cast(double, o);
}

// a value that is the same on every lane, moved to scalar registers
__device__ __forceinline__ double uniform_d(double v) {
  const int2 h = __builtin_bit_cast(int2, v);
  int2 o;
  o.x = __builtin_amdgcn_readfirstlane(h.x);
  o.y = __builtin_amdgcn_readfirstlane(h.y);
  return __builtin_bit_cast(double, o);
}

// wavefront sum in a fixed order (rows of 16 lanes, then the four rows); uniform result
__device__ __forceinline__ double wave_sum_d(double v) {
  v = group_sum_d<16>(v);
  return ((readlane_d(v, 0) + readlane_d(v, 16)) + readlane_d(v, 32)) + readlane_d(v, 48);
}

template <int CTRL>
__device__ __forceinline__ float dpp_fl(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf,
                                                            0xf, true));
}

// The ev-th smallest eigenvalue of the symmetric tridiagonal matrix (diagonal df, squared
// off-diagonals shifted by one: e2s[j] = e_{j-1}^2 > 0, e2s[0] = 0) by P-point multisection on
// Sturm counts, P aligned lanes per eigenvalue (q = lane within the group).  Each step splits
// [lo, hi] into P + 1 parts; the new interval ends at the lowest point with more than ev
// eigenvalues below it and starts at the highest point under that one, so it always brackets
// the eigenvalue even where rounding makes the counts non-monotone.  4 points x 13 steps or
// 8 points x 10 steps shrink the start interval more than 2^30 times.  The Sturm chain reads
// the matrix 8 entries at a time (16-byte LDS reads), the next 8 loaded while the current 8
// are used, so LDS latency stays off the chain.
template <int P, int D, int NIT = (P == 4 ? 13 : 10)>
__device__ float multisect(int ev, float lo, float hi, const float* df, const float* e2s, int q) {
  static_assert(P == 4 || P == 8, "groups of 4 or 8 lanes");
  static_assert(D % 8 == 0, "chunks of 8");
  const float4* d4 = reinterpret_cast<const float4*>(df);
  const float4* e4 = reinterpret_cast<const float4*>(e2s);
  for (int it = 0; it < NIT; ++it) {
    const float mid = lo + (float)(q + 1) * ((hi - lo) * (1.f / (P + 1)));
    // Sturm count: the number of negative pivots of T - mid I (the first pivot is
    // df[0] - mid: its e2s term is 0 * rcp(1))
    float qv = 1.f;
    int cnt = 0;
    float4 da = d4[0], db = d4[1], ea = e4[0], eb = e4[1];
#pragma unroll 2
    for (int jb = 0; jb < D; jb += 8) {
      const int nx = jb + 8 < D ? jb / 4 + 2 : jb / 4;  // the last chunk reloads itself
      const float4 nda = d4[nx], ndb = d4[nx + 1], nea = e4[nx], neb = e4[nx + 1];
      const float dv[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
      const float ev2[8] = {ea.x, ea.y, ea.z, ea.w, eb.x, eb.y, eb.z, eb.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        qv = (dv[u] - mid) - ev2[u] * __builtin_amdgcn_rcpf(qv);
        cnt += qv < 0.f;
      }
      da = nda; db = ndb; ea = nea; eb = neb;
    }
    float h = cnt > ev ? mid : hi;
    h = fminf(h, dpp_fl<0xB1>(h));
    h = fminf(h, dpp_fl<0x4E>(h));
    if constexpr (P == 8) h = fminf(h, dpp_fl<0x141>(h));
    float l = mid < h ? mid : lo;
    l = fmaxf(l, dpp_fl<0xB1>(l));
    l = fmaxf(l, dpp_fl<0x4E>(l));
    if constexpr (P == 8) l = fmaxf(l, dpp_fl<0x141>(l));
    lo = l;
    hi = h;
  }
  return 0.5f * (lo + hi);
}

}  // namespace kvc
