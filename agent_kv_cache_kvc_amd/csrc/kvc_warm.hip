// Warm-started refit of the rank-r anchor from an updated Gram matrix, gfx950.
//
// KVCMAS keeps a delta's anchor as a compact low-rank state (metraipolis abstract) while the
// shared context keeps changing (same abstract; thelatestinai listing, Figs. 10-11: shared
// tokens accumulate over the workflow).  After rows are appended, G = delta^T delta moves
// little and its new top-r eigenvectors lie close to the previous W.  This kernel starts from
// that W instead of solving the d x d eigenproblem from scratch:
//
//   Q0   = [W_prev^T, E] on 32 columns: the previous rows plus, for r < 32, fixed +-1
//          directions made orthogonal to them;
//   loop (at most kWarmMaxIt times):
//     Z  = G Q (the first pass: G Q0; later passes: G times the previous pass's Ritz vectors
//          and the rest of its Q)
//     Q  = Z R^-1 with R^T R = Z^T Z (Cholesky QR after scaling the columns to unit norm,
//          a second pass when the first Cholesky factor is poorly conditioned)
//     H  = Q^T G Q, its r largest eigenpairs (Householder tridiagonalisation in float64,
//          float32 multisection on Sturm counts, float64 inverse iteration,
//          back-transformation)
//     X  = Q Y_r (Ritz vectors), G X = (G Q) Y_r
//     accept when every Ritz vector's residual |G x_i - rho_i x_i| is within 2^-28 of the
//     Gershgorin bound of G and X^T X = I to 1e-8 (W is stored in float32; the bounds below
//     carry the measured defect); otherwise iterate.  After the first pass the block grows
//     to 48 columns (16 more fixed directions orthogonal to it), which sets the convergence
//     of the r wanted vectors against the next ones.
//
// The effective rank is then decided from the Ritz vectors alone and must be certain
// (rho_i = x_i^T G x_i, C_k = sum of the k largest eigenvalues of G, need = energy trace G):
//   C_k >= sum of the k largest rho_i                        (Ky Fan: any k orthonormal
//                                                            vectors give a lower bound)
//   C_j <= max_i [sum of the j - i largest rho + i mu] + sqrt(j) (|G X - X diag(rho)|_F +
//          2 |F|_F)                                          with F the off-diagonal part of
//          X^T G X and mu >= the largest eigenvalue of G on the complement of X
//          (mu^2 <= |G|_F^2 - |X^T G X|_F^2, taken with (1e-13 + 4 r defect) |G|_F^2 added;
//          the residual term with 2 r defect times the Gershgorin bound added),
// each side widened by k (3 r defect(X) + 1e-12) times the Gershgorin bound for rounding and
// for X being orthonormal only to its measured defect (max |X^T X - I|).  k is kept when C_k >= need is proven
// and C_{k-1} < need is proven (k <= r); otherwise, or when the iteration does not converge,
// the matrix is marked (kWarmMiss) and the full eigensolver of the fit decides it.
//
// One workgroup of D / 16 waves per matrix (wave w owns rows 16 w .. 16 w + 15 of every
// n x 48 block); products on the float64 MFMA v_mfma_f64_16x16x4_f64, whose 16 x 16 result
// holds row g + 4 v, column i in register v of lane 16 g + i.
#include <hip/hip_runtime.h>

#include "kvc_device.h"
#include "kvc_eig_common.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kWarmM = 48;   // columns of the iterated block
constexpr int kWarmQS = 50;  // row stride (doubles) of the n x 48 block in LDS
constexpr int kWarmSS = 49;  // row stride of the 48 x 48 block
constexpr int kWarmMaxIt = 3;
constexpr int kWarmNW = 8;             // waves of the largest workgroup (d = 128)

typedef double double4v __attribute__((ext_vector_type(4)));

// LDS of the refit (one matrix per workgroup).  The phases below are separate functions
// (not inlined): each gets its own register allocation, and they hand their results to
// each other through these arrays.
extern __shared__ __align__(16) double w_lds[];  // QB [D][kWarmQS], then SM [48][kWarmSS]
__shared__ double w_red[2 * kWarmNW];
__shared__ double w_red3[kWarmNW][3];
__shared__ double w_stat[3];  // |G|_F^2, Gershgorin bound, trace
__shared__ double w_dvec[kWarmM], w_evec[kWarmM], w_tau[kWarmM], w_dsc[kWarmM], w_rdg[kWarmM];
__shared__ __align__(16) double w_vs[kWarmM], w_ws[kWarmM];
__shared__ __align__(16) float w_df[kWarmM], w_e2s[kWarmM];
__shared__ float w_lam[kEigMaxR];
__shared__ double w_col[kWarmNW][kEigMaxR];
__shared__ double w_res2[kEigMaxR], w_rho[kEigMaxR];
__shared__ double w_amax[kWarmNW][kEigMaxR];
__shared__ int w_aidx[kWarmNW][kEigMaxR];
__shared__ int w_flag[2];
__shared__ double w_resp;  // the previous pass's largest residual norm

__device__ __forceinline__ double4v mfma64(double a, double b, double4v c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// +-1 entry (i, j) of the extra start directions (a fixed integer hash)
__device__ __forceinline__ double warm_pattern(int i, int j) {
  uint32_t h = (uint32_t)i * 0x9E3779B1u + (uint32_t)j * 0x85EBCA77u + 0x27D4EB2Fu;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return (h & 1u) ? 1.0 : -1.0;
}

template <int NW>
__device__ __forceinline__ double wg_sum(double v) {
  v = wave_sum_d(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) w_red[threadIdx.x / kWave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += w_red[w];
  return s;
}

template <int NW>
__device__ __forceinline__ double wg_max(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if (threadIdx.x % kWave == 0) w_red[threadIdx.x / kWave] = v;
  __syncthreads();
  double s = w_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) s = fmax(s, w_red[w]);
  return s;
}

// one pass over the workgroup for three values: a sum, a maximum and a sum (waves in order)
template <int NW>
__device__ __forceinline__ void wg_sum_max_sum(double& a, double& b, double& c) {
  a = wave_sum_d(a);
  c = wave_sum_d(c);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) b = fmax(b, __shfl_xor(b, off, 64));
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    const int w = threadIdx.x / kWave;
    w_red3[w][0] = a;
    w_red3[w][1] = b;
    w_red3[w][2] = c;
  }
  __syncthreads();
  a = w_red3[0][0];
  b = w_red3[0][1];
  c = w_red3[0][2];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    a += w_red3[w][0];
    b = fmax(b, w_red3[w][1]);
    c += w_red3[w][2];
  }
}

// element e of the upper triangle (row-major, diagonal included) of an n x n matrix
__device__ __forceinline__ void tri_ij(int e, int n, int& i, int& j) {
  int a = 0;
  while (e >= n - a) { e -= n - a; ++a; }
  i = a;
  j = a + e;
}

// G fragment for the A operand: lane (g, i0) of wave w holds G[16 w + i0][4 kb + g]; the lower
// triangle of G defines the symmetric matrix
template <int D>
__device__ __forceinline__ double g_at(const double* Gm, int kb, int w, int g, int i0) {
  const int row = 16 * w + i0, col = 4 * kb + g;
  return Gm[row >= col ? row * D + col : col * D + row];
}

// acc[J] = G B for the first nt 16-column tiles of the block B in QB (B operand: row
// 4 kb + g).  G is read from global memory (L2) for every product, eight fragments at a time
// with the next eight in flight; the B operands are read two k-steps at a time (the memory
// clobber keeps the compiler from hoisting every LDS read of the loop ahead of the MFMAs).
template <int D, bool STATS = false>
__device__ __forceinline__ void product(const double* Gm, double4v* acc, int nt,
                                        double* ss = nullptr, double* ra = nullptr) {
  constexpr int KB = D / 4, NG = KB / 8, QS = kWarmQS;
  const int w = threadIdx.x / kWave, g = (threadIdx.x % kWave) / 16, i0 = threadIdx.x % 16;
  const double* QB = w_lds;
  double gA[2][8];
#pragma unroll
  for (int u = 0; u < 8; ++u) gA[0][u] = g_at<D>(Gm, u, w, g, i0);
#pragma unroll
  for (int J = 0; J < 3; ++J)
    if (J < nt) acc[J] = double4v{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if (gi + 1 < NG) {
#pragma unroll
      for (int u = 0; u < 8; ++u) gA[(gi + 1) & 1][u] = g_at<D>(Gm, 8 * (gi + 1) + u, w, g, i0);
    }
    if constexpr (STATS) {  // |G|_F^2 and this lane's share of its row's absolute sum
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        *ss = fma(gA[gi & 1][u], gA[gi & 1][u], *ss);
        *ra += fabs(gA[gi & 1][u]);
      }
    }
#pragma unroll
    for (int k2 = 0; k2 < 8; k2 += 2) {
      const int kb = 8 * gi + k2;
      double b[2][3];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int J = 0; J < 3; ++J)
          b[u][J] = J < nt ? QB[(4 * (kb + u) + g) * QS + 16 * J + i0] : 0.0;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int J = 0; J < 3; ++J)
          if (J < nt) acc[J] = mfma64(gA[gi & 1][k2 + u], b[u][J], acc[J]);
      asm volatile("" ::: "memory");
    }
  }
}

// upper tile t (row-major over I <= J) of an NT x NT grid of 16 x 16 tiles
template <int NT>
__device__ __forceinline__ void tile_ij(int t, int& I, int& J) {
  int a = 0;
  while (t >= NT - a) { t -= NT - a; ++a; }
  I = a;
  J = a + t;
}

// SM tiles (I, J), I <= J < NT, of P^T R summed over the waves in order: each wave's part is
// the product of its 16 rows of P and R (both in the result layout), three tiles at a time.
template <int D, int NT>
__device__ __forceinline__ void sym_tiles_to_sm(const double4v* P, const double4v* R) {
  constexpr int NW = D / 16, SS = kWarmSS, NTILE = NT * (NT + 1) / 2;
  const int w = threadIdx.x / kWave, g = (threadIdx.x % kWave) / 16, i0 = threadIdx.x % 16;
  double* SM = w_lds + D * kWarmQS;
#pragma unroll
  for (int t0 = 0; t0 < NTILE; t0 += 3) {
    double4v part[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      int I, J;
      tile_ij<NT>(t0 + q, I, J);
      part[q] = double4v{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int v = 0; v < 4; ++v) part[q] = mfma64(P[I][v], R[J][v], part[q]);
    }
    for (int ww = 0; ww < NW; ++ww) {
      if (w == ww) {
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          int I, J;
          tile_ij<NT>(t0 + q, I, J);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            double* p = SM + (16 * I + g + 4 * v) * SS + 16 * J + i0;
            *p = (ww == 0 ? 0.0 : *p) + part[q][v];
          }
        }
      }
      __syncthreads();
    }
  }
}

// extra start directions: QB columns [c0, c1) get the fixed +-1 pattern, made orthogonal to
// the columns [0, c0) (taken as orthonormal rows of a basis: E -= B (B^T E)); C = B^T E goes
// through SM
template <int D>
__device__ __attribute__((noinline)) void warm_extras(int c0, int c1) {
  constexpr int NW = D / 16, NTH = kWave * NW, QS = kWarmQS, SS = kWarmSS;
  const int tid = threadIdx.x, ne = c1 - c0;
  double* QB = w_lds;
  double* SM = w_lds + D * QS;
  for (int e = tid; e < ne * D; e += NTH) {
    const int j = c0 + e / D, i = e % D;
    QB[i * QS + j] = warm_pattern(i, j);
  }
  __syncthreads();
  for (int e = tid; e < c0 * ne; e += NTH) {  // C = B^T E  (c0 x ne)
    const int a = e / ne, b = e - a * ne;
    double c = 0.0;
#pragma unroll 4
    for (int i = 0; i < D; ++i) c = fma(QB[i * QS + a], QB[i * QS + c0 + b], c);
    SM[a * SS + b] = c;
  }
  __syncthreads();
  for (int e = tid; e < D * ne; e += NTH) {  // E -= B C
    const int i = e / ne, b = e - i * ne;
    double v = QB[i * QS + c0 + b];
    for (int a = 0; a < c0; ++a) v = fma(-QB[i * QS + a], SM[a * SS + b], v);
    QB[i * QS + c0 + b] = v;
  }
  __syncthreads();
}

// SM tiles (I, J), I <= J < NT, of B^T B for the block B in QB (MQ = 16 NT columns), each tile
// by one wave over all D rows (no cross-wave sum); both triangles of SM are written
template <int D, int NT>
__device__ __forceinline__ void gram_tiles_from_qb() {
  constexpr int NW = D / 16, QS = kWarmQS, SS = kWarmSS, NTILE = NT * (NT + 1) / 2;
  const int w = threadIdx.x / kWave, g = (threadIdx.x % kWave) / 16, i0 = threadIdx.x % 16;
  const double* QB = w_lds;
  double* SM = w_lds + D * QS;
  for (int t = w; t < NTILE; t += NW) {
    int I, J;
    tile_ij<NT>(t, I, J);
    double4v acc = double4v{0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int kb = 0; kb < D / 4; ++kb) {
      const double* row = QB + (4 * kb + g) * QS + i0;
      acc = mfma64(row[16 * I], row[16 * J], acc);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      SM[(16 * I + g + 4 * v) * SS + 16 * J + i0] = acc[v];
      SM[(16 * J + i0) * SS + 16 * I + g + 4 * v] = acc[v];
    }
  }
  __syncthreads();
}

// ---- phase 1: Z = G B with B the block in QB, then Cholesky QR of Z into QB (one pass, a
//      second when the first factor's smallest pivot is below 1e-4).  Returns 0 when Z is
//      numerically rank-deficient (uniform).
template <int D, int MQ, bool FIRST>
__device__ __attribute__((noinline)) int warm_zchol(const double* Gm) {
  constexpr int NW = D / 16, NTH = kWave * NW, NT = MQ / 16, QS = kWarmQS, SS = kWarmSS;
  constexpr int NTRI = MQ * (MQ + 1) / 2, OWN = (NTRI + NTH - 1) / NTH;
  const int tid = threadIdx.x, w = tid / kWave, g = (tid % kWave) / 16, i0 = tid % 16;
  double* QB = w_lds;
  double* SM = w_lds + D * QS;
  double4v acc[3];
  if constexpr (FIRST) {
    // the statistics of G ride on the first product: |G|_F^2, the Gershgorin bound (row sums
    // of |G|: a lane holds a quarter of its row), the trace; published in w_stat
    double ss = 0.0, ra = 0.0;
    double tr = tid < D ? Gm[tid * D + tid] : 0.0;  // issued before the product's loads
    product<D, true>(Gm, acc, NT, &ss, &ra);
    ra += __shfl_xor(ra, 16, 64);
    ra += __shfl_xor(ra, 32, 64);
    wg_sum_max_sum<NW>(ss, ra, tr);
    if (tid == 0) {
      w_stat[0] = ss;
      w_stat[1] = ra;
      w_stat[2] = tr;
    }
    // a zero, infinite or NaN G is left to the full eigensolver (uniform)
    if (!(tr > 0.0) || !(ss < 1e300) || !(ra < 1e300) || !(tr < 1e300)) return 0;
  } else {
    product<D>(Gm, acc, NT);
  }
  __syncthreads();  // every wave has read QB as a B operand
#pragma unroll
  for (int J = 0; J < NT; ++J)
#pragma unroll
    for (int v = 0; v < 4; ++v) QB[(16 * w + g + 4 * v) * QS + 16 * J + i0] = acc[J][v];
  int own_i[OWN], own_j[OWN];
#pragma unroll
  for (int u = 0; u < OWN; ++u) {
    const int e = tid + u * NTH;
    if (e < NTRI) tri_ij(e, MQ, own_i[u], own_j[u]);
    else { own_i[u] = -1; own_j[u] = -1; }
  }
  __syncthreads();  // Z complete in QB
  for (int pass = 0; pass < 2; ++pass) {
    // S = Z^T Z in SM
    gram_tiles_from_qb<D, NT>();
    // unit diagonal: S' = D S D with D = diag(S)^-1/2
    if (tid < MQ) {
      const double sd = SM[tid * SS + tid];
      w_dsc[tid] = sd > 0.0 && sd < 1e300 ? 1.0 / sqrt(sd) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < OWN; ++u)
      if (own_i[u] >= 0) SM[own_i[u] * SS + own_j[u]] *= w_dsc[own_i[u]] * w_dsc[own_j[u]];
    __syncthreads();
    // right-looking Cholesky on the upper triangle: row k stays U[k][j] = R[k][k] R[k][j]
#pragma unroll 1
    for (int k = 0; k < MQ; ++k) {
      const double inv = 1.0 / SM[k * SS + k];
#pragma unroll
      for (int u = 0; u < OWN; ++u) {
        const int i = own_i[u], j = own_j[u];
        if (i > k) SM[i * SS + j] -= SM[k * SS + i] * SM[k * SS + j] * inv;
      }
      __syncthreads();
    }
    // R = rows of U scaled by 1 / sqrt(U[k][k]); the smallest pivot decides the second pass
    double pmin = 1.0;
    if (tid < MQ) {
      const double pv = SM[tid * SS + tid];
      pmin = pv;
      w_rdg[tid] = pv > 0.0 && pv < 1e300 ? 1.0 / sqrt(pv) : 0.0;
    }
    pmin = -wg_max<NW>(-(pmin == pmin ? pmin : -1.0));  // NaN counts as a failure
#pragma unroll
    for (int u = 0; u < OWN; ++u)
      if (own_i[u] >= 0) SM[own_i[u] * SS + own_j[u]] *= w_rdg[own_i[u]];
    __syncthreads();
    if (!(pmin > 1e-18)) return 0;  // (uniform) numerically rank-deficient
    // q R = z D, row by row: four lanes per row of Z (wave w: its own 16 rows); lane p keeps
    // the solved q_k of its residue class k = p mod 4 in registers, so only R is read from
    // LDS (the same entries on every row: broadcast reads, independent of the solve)
    {
      const int row = tid / 4, p = tid % 4;
      double* qr = QB + row * QS;
      double z[MQ / 4], qk[MQ / 4];
#pragma unroll
      for (int u = 0; u < MQ / 4; ++u) z[u] = qr[4 * u + p];
#pragma unroll
      for (int j = 0; j < MQ; ++j) {
        double s = 0.0;
#pragma unroll
        for (int u = 0; u < MQ / 4; ++u)
          if (4 * u < j) s = 4 * u + p < j ? fma(qk[u], SM[(4 * u + p) * SS + j], s) : s;
        s += dpp_d<0xB1>(s);
        s += dpp_d<0x4E>(s);
        const double zj = __shfl(z[j / 4], (tid & ~3) + (j % 4), 64);  // z_j from its lane
        const double q = (zj * w_dsc[j] - s) * w_rdg[j];
        if (p == j % 4) qk[j / 4] = q;
      }
#pragma unroll
      for (int u = 0; u < MQ / 4; ++u) qr[4 * u + p] = qk[u];
    }
    if (pmin >= 1e-4) break;  // (uniform) orthonormal to about 1e-12 after one pass
#pragma unroll
    for (int J = 0; J < NT; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[J][v] = QB[(16 * w + g + 4 * v) * QS + 16 * J + i0];
    __syncthreads();  // SM is rewritten by the second pass
  }
  __syncthreads();  // Q complete in QB
  return 1;
}

// ---- phase 2: H = Q^T G Q into SM (both triangles)
template <int D, int MQ>
__device__ __attribute__((noinline)) void warm_rayleigh(const double* Gm) {
  constexpr int NW = D / 16, NTH = kWave * NW, NT = MQ / 16, QS = kWarmQS, SS = kWarmSS;
  const int tid = threadIdx.x, w = tid / kWave, g = (tid % kWave) / 16, i0 = tid % 16;
  const double* QB = w_lds;
  double* SM = w_lds + D * QS;
  double4v yacc[3], acc[3];
  product<D>(Gm, yacc, NT);
#pragma unroll
  for (int J = 0; J < NT; ++J)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[J][v] = QB[(16 * w + g + 4 * v) * QS + 16 * J + i0];
  sym_tiles_to_sm<D, NT>(acc, yacc);
  for (int e = tid; e < MQ * MQ; e += NTH) {
    const int i = e / MQ, j = e - i * MQ;
    if (i > j) SM[i * SS + j] = SM[j * SS + i];
  }
  __syncthreads();
}

// ---- phase 3: the r largest eigenpairs of H (SM): Householder tridiagonalisation (one wave,
//      lane i = row i; the reflector of step k stays in column k below the diagonal; a step
//      touches the trailing columns in batches of eight, the row entries and the broadcast
//      v, w of a batch read together; v and w vanish left of column k + 1 and p is cleared at
//      and above row k), 8-point multisection for the eigenvalues, inverse iteration and
//      back-transformation for the vectors; Y_r (48 x 16 NC, zero past r) into SM.
template <int D, int MQ>
__device__ __attribute__((noinline)) void warm_small_eig(int r) {
  constexpr int NW = D / 16, NTH = kWave * NW, SS = kWarmSS, RPL = MQ / 16;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  double* SM = w_lds + D * kWarmQS;
  const int NC = (r + 15) / 16;
  if (w == 0) {
    const int i = l;
    const bool row_ok = i < MQ;
    double* hrow = SM + (row_ok ? i : 0) * SS;
#pragma unroll 1
    for (int k = 0; k < MQ - 2; ++k) {
      // x = column k below the diagonal, broadcast; H x over the trailing columns, with
      // x.x and x.Hx in one reduction (H v = H x - alpha H e_{k+1}, so no second pass)
      const bool act = row_ok && i > k;
      const double x = act ? hrow[k] : 0.0;
      const double hk1 = act ? hrow[k + 1] : 0.0;  // H[i][k+1]
      if (row_ok) w_vs[i] = x;
      const int jb0 = (k + 1) & ~7;  // first batch holding a trailing column
      double pa = 0.0, pb = 0.0;
#pragma unroll 2
      for (int jb = jb0; jb < MQ; jb += 8) {
        double h[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) h[u] = hrow[jb + u];
        const double2 v01 = *reinterpret_cast<const double2*>(w_vs + jb);
        const double2 v23 = *reinterpret_cast<const double2*>(w_vs + jb + 2);
        const double2 v45 = *reinterpret_cast<const double2*>(w_vs + jb + 4);
        const double2 v67 = *reinterpret_cast<const double2*>(w_vs + jb + 6);
        pa = fma(h[0], v01.x, fma(h[2], v23.x, fma(h[4], v45.x, fma(h[6], v67.x, pa))));
        pb = fma(h[1], v01.y, fma(h[3], v23.y, fma(h[5], v45.y, fma(h[7], v67.y, pb))));
      }
      const double hx = act ? pa + pb : 0.0;
      double s1 = x * x, s2 = x * hx;  // both sums over the wave, rows of 16 first
      s1 = group_sum_d<16>(s1);
      s2 = group_sum_d<16>(s2);
      const double nx2 = ((readlane_d(s1, 0) + readlane_d(s1, 16)) + readlane_d(s1, 32)) +
                         readlane_d(s1, 48);
      const double xhx = ((readlane_d(s2, 0) + readlane_d(s2, 16)) + readlane_d(s2, 32)) +
                         readlane_d(s2, 48);
      const double x0 = readlane_d(x, k + 1), hx0 = readlane_d(hx, k + 1);
      const double b00 = readlane_d(hk1, k + 1);  // H[k+1][k+1]
      // |x| and t = 2 / v.v = 1 / (|x| (|x| + |x_0|)) from the hardware reciprocal square
      // root and reciprocal, two Newton steps each (x = 0: alpha = t = 0, no change)
      double y = __builtin_amdgcn_rsq(nx2);
      y = y * fma(-0.5 * nx2 * y, y, 1.5);
      y = y * fma(-0.5 * nx2 * y, y, 1.5);
      const double nx = nx2 * y;
      const double den = nx + fabs(x0);
      double rd = __builtin_amdgcn_rcp(den);
      rd = rd * fma(-den, rd, 2.0);
      rd = rd * fma(-den, rd, 2.0);
      const double alpha = nx2 > 0.0 ? (x0 >= 0.0 ? -nx : nx) : 0.0;
      const double t = nx2 > 0.0 ? y * rd : 0.0;
      const double v = i == k + 1 ? x0 - alpha : x;
      const double p = act ? t * (hx - alpha * hk1) : 0.0;
      const double K = 0.5 * t * t * (xhx - 2.0 * alpha * hx0 + alpha * alpha * b00);
      const double wv = p - K * v;
      if (row_ok) {
        w_vs[i] = v;
        w_ws[i] = wv;
      }
      if (act) {
#pragma unroll 2
        for (int jb = jb0; jb < MQ; jb += 8) {
          double h[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) h[u] = hrow[jb + u];
          double vv[8], ww[8];
#pragma unroll
          for (int u = 0; u < 8; u += 2) {
            const double2 a = *reinterpret_cast<const double2*>(w_vs + jb + u);
            const double2 b = *reinterpret_cast<const double2*>(w_ws + jb + u);
            vv[u] = a.x; vv[u + 1] = a.y; ww[u] = b.x; ww[u + 1] = b.y;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) hrow[jb + u] = h[u] - (v * ww[u] + wv * vv[u]);
        }
        hrow[k] = v;
      }
      if (i == 0) {
        w_dvec[k] = SM[k * SS + k];
        w_evec[k] = alpha;
        w_tau[k] = t;
      }
    }
    if (i == 0) {
      w_dvec[MQ - 2] = SM[(MQ - 2) * SS + MQ - 2];
      w_evec[MQ - 2] = SM[(MQ - 1) * SS + MQ - 2];
      w_dvec[MQ - 1] = SM[(MQ - 1) * SS + MQ - 1];
      w_evec[MQ - 1] = 0.0;
      w_tau[MQ - 2] = 0.0;
      w_tau[MQ - 1] = 0.0;
    }
  }
  __syncthreads();

  // the r largest eigenvalues of the tridiagonal matrix (8-point multisection)
  double glo = 0.0, ghi = 0.0;
  if (tid < MQ) {
    w_df[tid] = (float)w_dvec[tid];
    w_e2s[tid] = tid >= 1 ? fmaxf((float)(w_evec[tid - 1] * w_evec[tid - 1]), 1e-36f) : 0.f;
    const double rad = (tid > 0 ? fabs(w_evec[tid - 1]) : 0.0) + fabs(w_evec[tid]);
    glo = w_dvec[tid] - rad;
    ghi = w_dvec[tid] + rad;
  }
  const double hmax = wg_max<NW>(tid < MQ ? ghi : -1e300);
  const double hmin = -wg_max<NW>(tid < MQ ? -glo : -1e300);
  const double span = fmax(hmax - hmin, 1e-300);
  const float lo_s = (float)(hmin - 1e-6 * span), hi_s = (float)(hmax + 1e-6 * span);
  if (tid < 8 * r) {
    // 11 steps: 9^11 > 2^34 times below the Gershgorin width (the inverse iteration's
    // vectors for close eigenvalues stay orthogonal to about 1e-11)
    const float lam = multisect<8, MQ, 11>(MQ - 1 - tid / 8, lo_s, hi_s, w_df, w_e2s, tid % 8);
    if (tid % 8 == 0) w_lam[tid / 8] = lam;
  }
  __syncthreads();

    // ---- inverse iteration (16 lanes per vector, RPL rows per lane), back-transformation,
    //      Y_r into SM after every reflector has been read
    double z[RPL];
    const int L = tid % 16;
    constexpr int VPB = NTH / 16;  // vectors per batch
    double ybuf[(kEigMaxR + VPB - 1) / VPB][RPL];
#pragma unroll
    for (int bt = 0; bt < (kEigMaxR + VPB - 1) / VPB; ++bt) {
      const int vec = bt * VPB + tid / 16;
      if (bt * VPB >= r) break;  // uniform
      const double lam = vec < r ? (double)w_lam[vec] : 0.0;
      const double tiny = 1e-300 + 1e-16 * fmax(fabs((double)w_lam[0]), 1e-300);
      double Rrp[RPL], Rc1[RPL], Rml[RPL], Ry[RPL];
      unsigned sw = 0;
      auto rhs0 = [&](int j) { return 1.0 + 0.1 * (double)((j * (2 * vec + 3)) % 7); };
      {
        double cb = w_dvec[0] - lam, cc = w_evec[0], ry = rhs0(0);
#pragma unroll 1
        for (int b = 0; b < 16; ++b) {
          const bool own = L == b;
#pragma unroll
          for (int u = 0; u < RPL; ++u) {
            const int j = b * RPL + u;
            if (j < MQ - 1) {
              const double na = w_evec[j], nb = w_dvec[j + 1] - lam;
              const double nc = j + 1 < MQ - 1 ? w_evec[j + 1] : 0.0;
              const double ny = rhs0(j + 1);
              const bool swp = fabs(na) > fabs(cb);
              const double piv = swp ? na : cb, oth = swp ? cb : na;
              const double pg = fabs(piv) > tiny ? piv : (piv < 0.0 ? -tiny : tiny);
              double rp = __builtin_amdgcn_rcp(pg);  // 1 / pivot, two Newton steps
              rp = rp * fma(-pg, rp, 2.0);
              rp = rp * fma(-pg, rp, 2.0);
              const double mlt = oth * rp;
              const double c1 = swp ? nb : cc, yj = swp ? ny : ry;
              const double nry = swp ? ry - mlt * ny : ny - mlt * ry;
              const double ncb = swp ? cc - mlt * nb : nb - mlt * cc;
              const double ncc = swp ? -mlt * nc : nc;
              if (own) {
                Rrp[u] = rp; Rc1[u] = c1; Rml[u] = mlt; Ry[u] = yj;
                sw |= (unsigned)swp << u;
              }
              cb = ncb; cc = ncc; ry = nry;
            } else {
              const double pg = fabs(cb) > tiny ? cb : (cb < 0.0 ? -tiny : tiny);
              if (own) { Rrp[u] = 1.0 / pg; Rc1[u] = 0.0; Rml[u] = 0.0; Ry[u] = ry; }
            }
          }
        }
      }
      auto back_solve = [&]() {
        double x1 = 0.0, x2 = 0.0, sq = 0.0;
#pragma unroll 1
        for (int b = 15; b >= 0; --b) {
          const bool own = L == b;
#pragma unroll
          for (int u = RPL - 1; u >= 0; --u) {
            const int j = b * RPL + u;
            const double c2 = ((sw >> u) & 1u) && j + 1 < MQ - 1 ? w_evec[j + 1] : 0.0;
            const double xj = (Ry[u] - Rc1[u] * x1 - c2 * x2) * Rrp[u];
            if (own) { Ry[u] = xj; sq += xj * xj; }
            x2 = x1;
            x1 = xj;
          }
          x1 = dpp_d<0x101>(x1);  // row_shl:1
          x2 = dpp_d<0x101>(x2);
        }
        sq = group_sum_d<16>(sq);
        return sq > 0.0 ? 1.0 / sqrt(sq) : 0.0;
      };
      const double s1 = back_solve();
      {
        const double halo = dpp_d<0x101>(Ry[0]);
        double ry = s1 * Ry[0];
#pragma unroll 1
        for (int b = 0; b < 16; ++b) {
          const bool own = L == b;
#pragma unroll
          for (int u = 0; u < RPL; ++u) {
            const int j = b * RPL + u;
            if (j < MQ - 1) {
              const double ny = s1 * (u + 1 < RPL ? Ry[u + 1 < RPL ? u + 1 : 0] : halo);
              const bool swp = (sw >> u) & 1u;
              const double mlt = Rml[u];
              const double out = swp ? ny : ry;
              ry = swp ? ry - mlt * ny : ny - mlt * ry;
              if (own) Ry[u] = out;
            } else if (own) {
              Ry[u] = ry;
            }
          }
          ry = dpp_d<0x111>(ry);  // row_shr:1
        }
      }
      const double s2 = back_solve();
#pragma unroll
      for (int u = 0; u < RPL; ++u) z[u] = s2 * Ry[u];
      // y = H_0 H_1 ... H_{MQ-3} z
      #pragma unroll 1
      for (int k = MQ - 3; k >= 0; --k) {
        double vk[RPL], s = 0.0;
#pragma unroll
        for (int u = 0; u < RPL; ++u) {
          const int j = L * RPL + u;
          vk[u] = j > k ? SM[j * SS + k] : 0.0;
          s = fma(vk[u], z[u], s);
        }
        s = group_sum_d<16>(s) * w_tau[k];
#pragma unroll
        for (int u = 0; u < RPL; ++u) z[u] = fma(-s, vk[u], z[u]);
      }
#pragma unroll
      for (int u = 0; u < RPL; ++u) ybuf[bt][u] = z[u];
    }
    __syncthreads();  // every reflector has been read
#pragma unroll
    for (int bt = 0; bt < (kEigMaxR + VPB - 1) / VPB; ++bt) {
      const int vec = bt * VPB + tid / 16;
      if (bt * VPB >= 16 * NC) break;
      if (vec < 16 * NC) {
#pragma unroll
        for (int u = 0; u < RPL; ++u)
          SM[(L * RPL + u) * SS + vec] = vec < r ? ybuf[bt][u] : 0.0;
      }
    }
    __syncthreads();

}

// ---- phase 4: X = Q Y_r (written over the first r columns of Q in QB), G X, X^T G X and
//      X^T X, the residuals, the decision (convergence; the effective rank proven from the
//      Ritz values), and when accepted W.  Returns 0 (not converged: iterate), 1 (converged;
//      *k_out holds k or -1 when it is not proven) or 2 (not converged and not worth another
//      pass: the sum of the r Ritz values, a lower bound on that of the r largest eigenvalues,
//      stays 0.1% short of the energy threshold, so k_eff > r or the block is far off; or the
//      residual, shrinking at the rate of the last two passes, would not reach the tolerance
//      in the passes left).  Giving up only saves time: such a matrix takes the full solve,
//      as does one that runs out of passes.
template <int D, int MQ>
__device__ __attribute__((noinline)) int warm_check(const double* Gm, int r, double energy,
                                                    double gf2, double gersh, double trace,
                                                    float* W_m, int* k_out, int it) {
  constexpr int NW = D / 16, NTH = kWave * NW, QS = kWarmQS, SS = kWarmSS;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave, g = l / 16, i0 = l % 16;
  double* QB = w_lds;
  double* SM = w_lds + D * QS;
  const int NC = (r + 15) / 16;
  double4v xacc[2], gxacc[2];  // result layout; tile 1 only when r > 16
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    xacc[c] = double4v{0.0, 0.0, 0.0, 0.0};
    gxacc[c] = double4v{0.0, 0.0, 0.0, 0.0};
  }
  {
    const double* arow = QB + (16 * w + i0) * QS + g;
#pragma unroll
    for (int kb = 0; kb < MQ / 4; ++kb) {
      const double a = arow[4 * kb];
      const double* brow = SM + (4 * kb + g) * SS + i0;
      xacc[0] = mfma64(a, brow[0], xacc[0]);
      if (NC > 1) xacc[1] = mfma64(a, brow[16], xacc[1]);
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (c >= NC) continue;
      const int col = 16 * c + i0;
      if (col >= r) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) QB[(16 * w + g + 4 * v) * QS + col] = xacc[c][v];
    }
  }
  __syncthreads();  // X complete in QB; every wave has read Y_r from SM
  product<D>(Gm, gxacc, NC);
  // X^T X (SM[1024 ..], stride 32): tile (c1, c2), c1 <= c2, from X in QB over all rows, one
  // wave per tile
  {
    const int nt = NC * (NC + 1) / 2;
    if (w < nt) {
      const int c1 = w == 2 ? 1 : 0, c2 = w == 0 ? 0 : 1;
      double4v t = double4v{0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
      for (int kb = 0; kb < D / 4; ++kb) {
        const double* row = QB + (4 * kb + g) * QS + i0;
        t = mfma64(row[16 * c1], row[16 * c2], t);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        SM[1024 + (16 * c1 + g + 4 * v) * 32 + 16 * c2 + i0] = t[v];
        SM[1024 + (16 * c2 + i0) * 32 + 16 * c1 + g + 4 * v] = t[v];
      }
    }
  }
  // X^T G X (SM[0 ..], stride 32): each wave's rows, summed over the waves in order
  {
    double4v pp[2][2];
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        pp[c1][c2] = double4v{0.0, 0.0, 0.0, 0.0};
        if (c1 < NC && c2 < NC) {
#pragma unroll
          for (int v = 0; v < 4; ++v) pp[c1][c2] = mfma64(xacc[c1][v], gxacc[c2][v], pp[c1][c2]);
        }
      }
    for (int ww = 0; ww < NW; ++ww) {
      if (w == ww) {
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            if (c1 >= NC || c2 >= NC) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              double* pa = SM + (16 * c1 + g + 4 * v) * 32 + 16 * c2 + i0;
              *pa = (ww == 0 ? 0.0 : *pa) + pp[c1][c2][v];
            }
          }
      }
      __syncthreads();
    }
  }
  // residual of each Ritz vector: |G x_c - rho_c x_c|^2 over the rows, then the waves
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c >= NC) continue;
    const int col = 16 * c + i0;
    const double rc = col < r ? SM[col * 32 + col] : 0.0;
    double s = 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const double d = gxacc[c][v] - rc * xacc[c][v];
      s = fma(d, d, s);
    }
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    if (g == 0 && col < r) w_col[w][col] = s;
  }
  // |X^T G X|_F^2, the orthonormality defect of X, the off-diagonal part of X^T G X
  double af = 0.0, dx = 0.0, ff = 0.0;
  for (int e = tid; e < r * r; e += NTH) {
    const int a = e / r, b = e - a * r;
    const double xv = SM[1024 + a * 32 + b] - (a == b ? 1.0 : 0.0);
    const double av = SM[a * 32 + b];
    dx = fmax(dx, xv == xv ? fabs(xv) : 1e300);
    af = fma(av, av, af);
    if (a != b) ff = fma(av, av, ff);
  }
  wg_sum_max_sum<NW>(af, dx, ff);  // (its barriers also publish w_col)
  const double a_f2 = af, defect = dx, f_f2 = ff;
  if (tid < r) {
    double s = 0.0;
    for (int ww = 0; ww < NW; ++ww) s += w_col[ww][tid];
    w_res2[tid] = s;
    w_rho[tid] = SM[tid * 32 + tid];
  }
  __syncthreads();

    // ---- decision (wave 0, lane c for Ritz pair c, then shared): convergence, then the
    //      effective rank from the Ritz values (see the header)
    if (w == 0) {
      const int c = l;
      const bool on = c < r;
      const double r2 = on ? w_res2[c] : 0.0;
      const double rc = on ? w_rho[c] : 0.0;
      double rmx = on ? (r2 == r2 ? r2 : 1e300) : 0.0;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) rmx = fmax(rmx, __shfl_xor(rmx, off, 64));
      const double rsum = wave_sum_d(r2);
      const double tol = 0x1p-28 * gersh;
      const bool conv = defect <= 1e-8 && sqrt(rmx) <= tol;  // uniform
      int kk = -1;
      bool give_up = false;
      if (!conv) {
        const double rho_r = wave_sum_d(rc);  // the r Ritz values
        const double res = sqrt(rmx);
        give_up = rho_r < (1.0 - 1e-3) * energy * trace;
        if (it >= 1 && !give_up) {
          double pred = res;  // after the passes left, at the last pass's rate
          for (int q = it + 1; q < kWarmMaxIt; ++q) pred *= res / fmax(w_resp, 1e-300);
          give_up = pred > tol;
        }
        if (l == 0) w_resp = res;
      }
      if (conv) {
        double* rsd = w_col[0];  // the Ritz values, descending
        double* csum = w_col[1];  // their running sums
        int rank = 0;
        for (int c2 = 0; c2 < r; ++c2) {
          const double o = w_rho[c2];
          rank += (o > rc) || (o == rc && c2 < c);
        }
        if (on) rsd[rank] = rc;
        const double sv = on ? rsd[c] : 0.0;
        double cum = sv;  // C_{c+1}: the c + 1 largest
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const double o = __shfl_up(cum, off, 64);
          if (c >= off) cum += o;
        }
        if (on) csum[c] = cum;
        const double unit = (3.0 * r * defect + 1e-12) * gersh;
        const double need_hi = energy * trace * (1.0 + 1e-13);
        const double need_lo = energy * trace * (1.0 - 1e-13);
        const double mu = sqrt(fmax(gf2 - a_f2, 0.0) + (1e-13 + 4.0 * r * defect) * gf2);
        const double bres = sqrt(rsum) + 2.0 * sqrt(f_f2) + 2.0 * r * defect * gersh;
        const unsigned long long bal = __ballot(on && cum - (c + 1) * unit >= need_hi);
        if (bal) {
          const int k = __ffsll((long long)bal);  // the first lane that proves C_k >= need, + 1
          const int j = k - 1;
          double cand = -1e300;
          if (c <= j) cand = (j - c == 0 ? 0.0 : csum[j - c - 1]) + c * mu;
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) cand = fmax(cand, __shfl_xor(cand, off, 64));
          const double up = cand + sqrt((double)j) * bres + j * unit;
          kk = up < need_lo ? k : -1;
        }
      }
      if (l == 0) {
        w_flag[0] = conv ? 1 : (give_up ? 2 : 0);
        w_flag[1] = kk;
      }
    }
    __syncthreads();
    if (w_flag[0] != 1) return w_flag[0];  // (uniform) not converged: iterate or give up
    {
      const int k_cert = w_flag[1];
      *k_out = k_cert;
      if (k_cert >= 0) {
        // canonical sign: the largest |entry| of each row positive (the first one on ties)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (c >= NC) continue;
          const int col = 16 * c + i0;
          double best = -1.0, bval = 0.0;
          int bidx = D;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 16 * w + g + 4 * v;
            const double a = fabs(xacc[c][v]);
            if (a > best || (a == best && row < bidx)) { best = a; bidx = row; bval = xacc[c][v]; }
          }
#pragma unroll
          for (int off = 16; off <= 32; off *= 2) {
            const double ob = __shfl_xor(best, off, 64), ov = __shfl_xor(bval, off, 64);
            const int oi = __shfl_xor(bidx, off, 64);
            if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; bval = ov; }
          }
          if (g == 0 && col < r) {
            w_amax[w][col] = best;
            w_aidx[w][col] = bidx;
            w_col[w][col] = bval;
          }
        }
        __syncthreads();
        if (tid < r) {
          double best = -1.0, bval = 0.0;
          int bidx = D;
          for (int ww = 0; ww < NW; ++ww) {
            const double a = w_amax[ww][tid];
            const int ix = w_aidx[ww][tid];
            if (a > best || (a == best && ix < bidx)) { best = a; bidx = ix; bval = w_col[ww][tid]; }
          }
          w_rho[tid] = bval < 0.0 ? -1.0 : 1.0;  // rho is no longer needed: it holds the sign
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (c >= NC) continue;
          const int col = 16 * c + i0;
          if (col >= r) continue;
          const double sg = w_rho[col];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 16 * w + g + 4 * v;
            W_m[(size_t)col * D + row] = (float)(sg * xacc[c][v]);
          }
        }
      }
    }
  return 1;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(4 * D, D == 128 ? 4 : 2) void refit_warm_kernel(
    const double* __restrict__ G, const float* __restrict__ W_prev, int r, double energy,
    float* __restrict__ W_out, int32_t* __restrict__ k_eff_out, int32_t* __restrict__ warm_out) {
  constexpr int NTH = kWave * (D / 16), QS = kWarmQS;
  double* QB = w_lds;
  const int m = blockIdx.x, tid = threadIdx.x;
  const double* Gm = G + (size_t)m * D * D;

  int k_cert = -1;
  {
    // ---- Q0 = [W_prev^T, E] on 32 columns, E orthogonal to the rows of W_prev (r < 32)
    for (int e = tid; e < r * D; e += NTH) {
      const int j = e / D, i = e - j * D;
      QB[i * QS + j] = (double)W_prev[((size_t)m * r + j) * D + i];
    }
    __syncthreads();
    if (r < 32) warm_extras<D>(r, 32);
    // ---- passes: Z = G B, Cholesky QR, Rayleigh-Ritz, check; B for the next pass is the
    //      Ritz vectors of this one and the remaining columns of its Q (left in QB)
    // the first pass uses 32 columns (the previous rows and, for r < 32, extra directions);
    // later passes all 48
    float* W_m = W_out + (size_t)m * r * D;
#pragma unroll 1
    for (int it = 0; it < kWarmMaxIt; ++it) {
      int kc = -1, conv = 0;
      if (it == 0) {
        if (!warm_zchol<D, 32, true>(Gm)) break;
        warm_rayleigh<D, 32>(Gm);
        warm_small_eig<D, 32>(r);
        conv = warm_check<D, 32>(Gm, r, energy, w_stat[0], w_stat[1], w_stat[2], W_m, &kc, it);
      } else {
        if (it == 1) warm_extras<D>(32, kWarmM);  // the block grows to 48 columns
        if (!warm_zchol<D, kWarmM, false>(Gm)) break;
        warm_rayleigh<D, kWarmM>(Gm);
        warm_small_eig<D, kWarmM>(r);
        conv = warm_check<D, kWarmM>(Gm, r, energy, w_stat[0], w_stat[1], w_stat[2], W_m, &kc,
                                     it);
      }
      if (conv == 1) {
        k_cert = kc;
        break;
      }
      if (conv == 2) break;  // not worth another pass: the full solve takes it
    }
  }
  if (tid == 0) {
    k_eff_out[m] = k_cert >= 0 ? k_cert : kWarmMiss;
    if (warm_out) warm_out[m] = k_cert >= 0 ? 1 : 0;
  }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(ceil_div(n, kBlock)), dim3(kBlock), 0, st, p, n, v);
  return hipGetLastError();
}

// G [M][D][D] (float64, lower triangle read), W_prev [M][r][D] -> W_out (rows of matrices
// whose refit converged and whose k_eff is proven), k_eff_out (k, or kWarmMiss), warm_out
// (1 / 0, may be null).
hipError_t launch_refit_warm_kernel(const double* G, int M, int d, int r, double energy,
                                    const float* W_prev, float* W_out, int32_t* k_eff,
                                    int32_t* warm, hipStream_t st) {
  if (d == 128) {
    const size_t lds = (size_t)(128 * kWarmQS + kWarmM * kWarmSS) * sizeof(double);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(refit_warm_kernel<128>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(refit_warm_kernel<128>, dim3(M), dim3(4 * 128), lds, st, G, W_prev, r,
                       energy, W_out, k_eff, warm);
  } else {
    const size_t lds = (size_t)(64 * kWarmQS + kWarmM * kWarmSS) * sizeof(double);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(refit_warm_kernel<64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(refit_warm_kernel<64>, dim3(M), dim3(4 * 64), lds, st, G, W_prev, r,
                       energy, W_out, k_eff, warm);
  }
  return hipGetLastError();
}

}  // namespace kvc
