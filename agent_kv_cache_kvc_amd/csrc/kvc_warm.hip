// Warm-started refit of the rank-r anchor from an updated Gram matrix, gfx950.
//
// KVCMAS keeps a delta's anchor as a compact low-rank state (metraipolis abstract) while the
// shared context keeps changing (same abstract; thelatestinai listing, Figs. 10-11: shared
// tokens accumulate over the workflow).  After rows are appended, G = delta^T delta moves
// little and its new top-r eigenvectors lie close to the previous W.  This kernel starts from
// that W instead of solving the d x d eigenproblem from scratch:
//
//   Q0   = [W_prev^T, E]: the previous rows plus 48 - r fixed +-1 directions made orthogonal
//          to them (the 48-column block holds the convergence of the r wanted vectors
//          against the next ones);
//   loop (at most kWarmMaxIt times):
//     Z  = G Q (the first pass: G Q0; later passes: the previous G Q)
//     Q  = Z R^-1 with R^T R = Z^T Z (Cholesky QR after scaling the columns to unit norm,
//          a second pass when the first Cholesky factor is poorly conditioned)
//     H  = Q^T G Q (48 x 48), its r largest eigenpairs (Householder tridiagonalisation in
//          float64, float32 multisection on Sturm counts, float64 inverse iteration,
//          back-transformation)
//     X  = Q Y_r (Ritz vectors), G X = (G Q) Y_r
//     accept when every Ritz vector's residual |G x_i - rho_i x_i| is within 2^-28 of the
//     Gershgorin bound of G and X^T X = I to 1e-10; otherwise iterate from G Q.
//
// The effective rank is then decided from the Ritz vectors alone and must be certain
// (rho_i = x_i^T G x_i, C_k = sum of the k largest eigenvalues of G, need = energy trace G):
//   C_k >= sum of the k largest rho_i                        (Ky Fan: any k orthonormal
//                                                            vectors give a lower bound)
//   C_j <= max_i [sum of the j - i largest rho + i mu] + sqrt(j) (|G X - X diag(rho)|_F +
//          2 |F|_F)                                          with F the off-diagonal part of
//          X^T G X and mu >= the largest eigenvalue of G on the complement of X
//          (mu^2 <= |G|_F^2 - |X^T G X|_F^2),
// each side widened by k (3 r defect(X) + 1e-12) times the Gershgorin bound for rounding and
// for X being orthonormal only to its measured defect.  k is kept when C_k >= need is proven
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
constexpr int kWarmRpl = kWarmM / 16;  // rows per lane of a 48-long vector (16 lanes)

typedef double double4v __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ double wg_sum(double v, double* red) {
  v = wave_sum_d(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[w];
  return s;
}

template <int NW>
__device__ __forceinline__ double wg_max(double v, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) s = fmax(s, red[w]);
  return s;
}

// element e of the upper triangle (row-major, diagonal included) of an n x n matrix
__device__ __forceinline__ void tri_ij(int e, int n, int& i, int& j) {
  int a = 0;
  while (e >= n - a) { e -= n - a; ++a; }
  i = a;
  j = a + e;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(4 * D, D == 128 ? 4 : 2) void refit_warm_kernel(
    const double* __restrict__ G, const float* __restrict__ W_prev, int r, double energy,
    float* __restrict__ W_out, int32_t* __restrict__ k_eff_out, int32_t* __restrict__ warm_out) {
  constexpr int NW = D / 16, NTH = kWave * NW, KB = D / 4;
  constexpr int MQ = kWarmM, QS = kWarmQS, SS = kWarmSS, NTRI = MQ * (MQ + 1) / 2;
  constexpr int OWN = (NTRI + NTH - 1) / NTH;  // upper-triangle elements per thread
  constexpr int RPL = kWarmRpl;
  extern __shared__ __align__(16) double lds[];
  double* QB = lds;           // [D][QS]: Q0, Z, Q, then G Q
  double* SM = lds + D * QS;  // [MQ][SS]: Gram, Cholesky factor, H, reflectors, Y, X^T G X
  __shared__ double red[2 * NW];
  __shared__ double dvec[MQ], evec[MQ], tauv[MQ], vs[MQ], wsv[MQ], dsc[MQ], rdg[MQ];
  __shared__ __align__(16) float df[MQ], e2s[MQ];
  __shared__ float lamf[kEigMaxR];
  __shared__ double colred[NW][kEigMaxR];
  __shared__ double res2[kEigMaxR], rho[kEigMaxR];
  __shared__ int s_flag[2];
  __shared__ double s_amax[NW][kEigMaxR];
  __shared__ int s_aidx[NW][kEigMaxR];

  const int m = blockIdx.x, tid = threadIdx.x;
  const int w = tid / kWave, l = tid % kWave, g = l / 16, i0 = l % 16;
  const double* Gm = G + (size_t)m * D * D;
  const int NC = (r + 15) / 16;  // 16-column tiles of the Ritz block (1 or 2)

  // G fragments for the A operand: lane (g, i0) of wave w holds G[16 w + i0][4 kb + g]; the
  // lower triangle of G defines the symmetric matrix
  auto g_at = [&](int kb, int w, int g, int i0) {
    const int row = 16 * w + i0, col = 4 * kb + g;
    return Gm[row >= col ? row * D + col : col * D + row];
  };
  // acc[J] = G Q for the three 16-column tiles, Q from QB (B operand: row 4 kb + g).  G is
  // read again for every product (L2), so its 32 fragments live only here; the B operands
  // are read two k-steps at a time (the memory clobber keeps the compiler from hoisting
  // every LDS read of the loop ahead of the MFMAs)
  auto product = [&](double4v (&acc)[3], int w, int g, int i0) {
    double gA[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) gA[kb] = g_at(kb, w, g, i0);
#pragma unroll
    for (int J = 0; J < 3; ++J) acc[J] = double4v{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k2 = 0; k2 < KB; k2 += 2) {
      double b[2][3];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int J = 0; J < 3; ++J) b[u][J] = QB[(4 * (k2 + u) + g) * QS + 16 * J + i0];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int J = 0; J < 3; ++J) acc[J] = mfma64(gA[k2 + u], b[u][J], acc[J]);
      asm volatile("" ::: "memory");
    }
  };

  // SM tiles (I, J), I <= J, of P^T R summed over the waves in order: each wave's part is the
  // product of its 16 rows of P and R (both in the result layout), three tiles at a time
  auto sym_tiles_to_sm = [&](const double4v (&P)[3], const double4v (&R)[3], int w, int g,
                             int i0) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      double4v part[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const int t = 3 * half + q;  // tiles (0,0) (0,1) (0,2) | (1,1) (1,2) (2,2)
        const int I = t < 3 ? 0 : (t < 5 ? 1 : 2), J = t < 3 ? t : (t < 5 ? t - 2 : 2);
        part[q] = double4v{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int v = 0; v < 4; ++v) part[q] = mfma64(P[I][v], R[J][v], part[q]);
      }
      for (int ww = 0; ww < NW; ++ww) {
        if (w == ww) {
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            const int t = 3 * half + q;
            const int I = t < 3 ? 0 : (t < 5 ? 1 : 2), J = t < 3 ? t : (t < 5 ? t - 2 : 2);
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
  };

  // ---- statistics of G: |G|_F^2, trace, Gershgorin bound
  double ss = 0.0, ra = 0.0;
#pragma unroll 8
  for (int kb = 0; kb < KB; ++kb) {
    const double gv = g_at(kb, w, g, i0);
    ss = fma(gv, gv, ss);
    ra += fabs(gv);
  }
  ra += __shfl_xor(ra, 16, 64);  // the row's four column groups
  ra += __shfl_xor(ra, 32, 64);
  const double gf2 = wg_sum<NW>(ss, red);
  const double gersh = wg_max<NW>(ra, red);
  const double trace = wg_sum<NW>(tid < D ? Gm[tid * D + tid] : 0.0, red);
  bool miss = !(trace > 0.0) || !(gf2 < 1e300) || !(gersh < 1e300) || !(trace < 1e300);

  // ---- Q0 = [W_prev^T, E], E orthogonal to the rows of W_prev
  const int ne = MQ - r;
  if (!miss) {
    for (int e = tid; e < MQ * D; e += NTH) {
      const int j = e / D, i = e - j * D;
      QB[i * QS + j] = j < r ? (double)W_prev[((size_t)m * r + j) * D + i] : warm_pattern(i, j);
    }
    __syncthreads();
    for (int e = tid; e < r * ne; e += NTH) {  // C = W_prev E  (r x ne) -> SM
      const int a = e / ne, b = e - a * ne;
      double c = 0.0;
#pragma unroll 4
      for (int i = 0; i < D; ++i) c = fma(QB[i * QS + a], QB[i * QS + r + b], c);
      SM[a * SS + b] = c;
    }
    __syncthreads();
    for (int e = tid; e < D * ne; e += NTH) {  // E -= W_prev^T C
      const int i = e / ne, b = e - i * ne;
      double v = QB[i * QS + r + b];
      for (int a = 0; a < r; ++a) v = fma(-QB[i * QS + a], SM[a * SS + b], v);
      QB[i * QS + r + b] = v;
    }
    __syncthreads();
  }

  int own_i[OWN], own_j[OWN];
#pragma unroll
  for (int u = 0; u < OWN; ++u) {
    const int e = tid + u * NTH;
    if (e < NTRI) tri_ij(e, MQ, own_i[u], own_j[u]);
    else { own_i[u] = -1; own_j[u] = -1; }
  }

  double4v acc[3];   // the current block in the result layout (Z, then Q)
  double4v yacc[3];  // G Q
  if (!miss) {  // Z = G Q0
    int tq = threadIdx.x;
    asm volatile("" : "+v"(tq));
    product(acc, tq / kWave, (tq % kWave) / 16, tq % 16);
  }
  bool done = false;
  int k_cert = -1;
#pragma unroll 1
  for (int it = 0; it < kWarmMaxIt && !miss && !done; ++it) {
    // the lane coordinates again behind an opaque move: addresses derived from them are
    // formed inside each phase instead of being held in registers across the whole pass
    int tq = threadIdx.x;
    asm volatile("" : "+v"(tq));
    const int tid = tq, w = tq / kWave, l = tq % kWave, g = l / 16, i0 = l % 16;
    // ---- Cholesky QR of Z into QB (the first pass stores Z = G Q0; later passes find G Q
    //      there already, each wave in its own rows)
    __syncthreads();  // every wave has read QB as a B operand
#pragma unroll
    for (int J = 0; J < 3; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        double* p = QB + (16 * w + g + 4 * v) * QS + 16 * J + i0;
        if (it == 0) *p = acc[J][v];
        else acc[J][v] = *p;
      }
    for (int pass = 0; pass < 2; ++pass) {
      // S = Z^T Z: each wave's 16 rows, the upper 16 x 16 tiles (I <= J), summed over the
      // waves in order into SM (three tiles at a time)
      sym_tiles_to_sm(acc, acc, w, g, i0);
      // unit diagonal: S' = D S D with D = diag(S)^-1/2
      if (tid < MQ) {
        const double sd = SM[tid * SS + tid];
        dsc[tid] = sd > 0.0 && sd < 1e300 ? 1.0 / sqrt(sd) : 0.0;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < OWN; ++u)
        if (own_i[u] >= 0) SM[own_i[u] * SS + own_j[u]] *= dsc[own_i[u]] * dsc[own_j[u]];
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
        rdg[tid] = pv > 0.0 && pv < 1e300 ? 1.0 / sqrt(pv) : 0.0;
      }
      pmin = -wg_max<NW>(-(pmin == pmin ? pmin : -1.0), red);  // NaN counts as a failure
#pragma unroll
      for (int u = 0; u < OWN; ++u)
        if (own_i[u] >= 0) SM[own_i[u] * SS + own_j[u]] *= rdg[own_i[u]];
      __syncthreads();
      if (!(pmin > 1e-18)) { miss = true; break; }  // (uniform) numerically rank-deficient
      // q R = z D, row by row: four lanes per row of Z in place (wave w: its own 16 rows)
      {
        const int row = tid / 4, p = tid % 4;
        double* qr = QB + row * QS;
        #pragma unroll 1
        for (int j = 0; j < MQ; ++j) {
          double s = 0.0;
          for (int k = p; k < j; k += 4) s = fma(qr[k], SM[k * SS + j], s);
          s += dpp_d<0xB1>(s);
          s += dpp_d<0x4E>(s);
          const double q = (qr[j] * dsc[j] - s) * rdg[j];
          if (p == 0) qr[j] = q;
        }
      }
#pragma unroll
      for (int J = 0; J < 3; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[J][v] = QB[(16 * w + g + 4 * v) * QS + 16 * J + i0];
      if (pmin >= 1e-4) break;  // (uniform) orthonormal to about 1e-12 after one pass
      __syncthreads();          // SM is rewritten by the second pass
    }
    if (miss) break;
    __syncthreads();  // Q complete in QB

    // ---- G Q, and H = Q^T G Q (Q in the result layout again from QB)
    product(yacc, w, g, i0);
#pragma unroll
    for (int J = 0; J < 3; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[J][v] = QB[(16 * w + g + 4 * v) * QS + 16 * J + i0];
    {
      sym_tiles_to_sm(acc, yacc, w, g, i0);
      // the lower triangle from the upper one
      for (int e = tid; e < MQ * MQ; e += NTH) {
        const int i = e / MQ, j = e - i * MQ;
        if (i > j) SM[i * SS + j] = SM[j * SS + i];
      }
      __syncthreads();
    }

    // ---- Householder tridiagonalisation of H (one wave, lane i = row i); the reflector of
    //      step k stays in column k below the diagonal
    if (w == 0) {
      const int i = l;
      const bool row_ok = i < MQ;
      #pragma unroll 1
      for (int k = 0; k < MQ - 2; ++k) {
        const bool act = row_ok && i > k;
        const double x = act ? SM[i * SS + k] : 0.0;
        const double nx2 = wave_sum_d(x * x);
        const double x0 = readlane_d(x, k + 1);
        double alpha = 0.0, t = 0.0;
        if (nx2 > 0.0) {
          const double nx = sqrt(nx2);
          alpha = x0 >= 0.0 ? -nx : nx;
          t = 1.0 / (nx * (nx + fabs(x0)));  // 2 / v.v
        }
        const double v = i == k + 1 ? x0 - alpha : x;
        if (row_ok) vs[i] = v;
        double p = 0.0;
        if (act) {
          for (int j = k + 1; j < MQ; ++j) p = fma(SM[i * SS + j], vs[j], p);
          p *= t;
        }
        const double K = 0.5 * t * wave_sum_d(v * p);
        const double wv = p - K * v;
        if (row_ok) wsv[i] = wv;
        if (act) {
          for (int j = k + 1; j < MQ; ++j) SM[i * SS + j] -= v * wsv[j] + wv * vs[j];
          SM[i * SS + k] = v;
        }
        if (i == 0) {
          dvec[k] = SM[k * SS + k];
          evec[k] = alpha;
          tauv[k] = t;
        }
      }
      if (i == 0) {
        dvec[MQ - 2] = SM[(MQ - 2) * SS + MQ - 2];
        evec[MQ - 2] = SM[(MQ - 1) * SS + MQ - 2];
        dvec[MQ - 1] = SM[(MQ - 1) * SS + MQ - 1];
        evec[MQ - 1] = 0.0;
        tauv[MQ - 2] = 0.0;
        tauv[MQ - 1] = 0.0;
      }
    }
    __syncthreads();

    // ---- the r largest eigenvalues of the tridiagonal matrix (8-point multisection)
    double glo = 0.0, ghi = 0.0;
    if (tid < MQ) {
      df[tid] = (float)dvec[tid];
      e2s[tid] = tid >= 1 ? fmaxf((float)(evec[tid - 1] * evec[tid - 1]), 1e-36f) : 0.f;
      const double rad = (tid > 0 ? fabs(evec[tid - 1]) : 0.0) + fabs(evec[tid]);
      glo = dvec[tid] - rad;
      ghi = dvec[tid] + rad;
    }
    const double hmax = wg_max<NW>(tid < MQ ? ghi : -1e300, red);
    const double hmin = -wg_max<NW>(tid < MQ ? -glo : -1e300, red);
    const double span = fmax(hmax - hmin, 1e-300);
    const float lo_s = (float)(hmin - 1e-6 * span), hi_s = (float)(hmax + 1e-6 * span);
    if (tid < 8 * r) {
      const float lam = multisect<8, MQ>(MQ - 1 - tid / 8, lo_s, hi_s, df, e2s, tid % 8);
      if (tid % 8 == 0) lamf[tid / 8] = lam;
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
      const double lam = vec < r ? (double)lamf[vec] : 0.0;
      const double tiny = 1e-300 + 1e-16 * fmax(fabs((double)lamf[0]), 1e-300);
      double Rrp[RPL], Rc1[RPL], Rml[RPL], Ry[RPL];
      unsigned sw = 0;
      auto rhs0 = [&](int j) { return 1.0 + 0.1 * (double)((j * (2 * vec + 3)) % 7); };
      {
        double cb = dvec[0] - lam, cc = evec[0], ry = rhs0(0);
#pragma unroll 1
        for (int b = 0; b < 16; ++b) {
          const bool own = L == b;
#pragma unroll
          for (int u = 0; u < RPL; ++u) {
            const int j = b * RPL + u;
            if (j < MQ - 1) {
              const double na = evec[j], nb = dvec[j + 1] - lam;
              const double nc = j + 1 < MQ - 1 ? evec[j + 1] : 0.0;
              const double ny = rhs0(j + 1);
              const bool swp = fabs(na) > fabs(cb);
              const double piv = swp ? na : cb, oth = swp ? cb : na;
              const double pg = fabs(piv) > tiny ? piv : (piv < 0.0 ? -tiny : tiny);
              const double rp = 1.0 / pg;
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
            const double c2 = ((sw >> u) & 1u) && j + 1 < MQ - 1 ? evec[j + 1] : 0.0;
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
        s = group_sum_d<16>(s) * tauv[k];
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

    // ---- X = Q Y_r; then G Q over Q in QB (each wave its own rows) and G X = (G Q) Y_r
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
      for (int J = 0; J < 3; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) QB[(16 * w + g + 4 * v) * QS + 16 * J + i0] = yacc[J][v];
#pragma unroll
      for (int kb = 0; kb < MQ / 4; ++kb) {
        const double a = arow[4 * kb];
        const double* brow = SM + (4 * kb + g) * SS + i0;
        gxacc[0] = mfma64(a, brow[0], gxacc[0]);
        if (NC > 1) gxacc[1] = mfma64(a, brow[16], gxacc[1]);
        asm volatile("" ::: "memory");
      }
    }
    __syncthreads();  // every wave has read Y_r from SM
    // X^T G X (SM[0 ..]) and X^T X (SM[1024 ..]), NC x NC tiles of stride 32, each summed
    // over the waves in order
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      double4v pp[2][2];
#pragma unroll
      for (int c1 = 0; c1 < 2; ++c1)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          pp[c1][c2] = double4v{0.0, 0.0, 0.0, 0.0};
          if (c1 < NC && c2 < NC) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              pp[c1][c2] = mfma64(xacc[c1][v], which == 0 ? gxacc[c2][v] : xacc[c2][v],
                                  pp[c1][c2]);
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
                double* pa = SM + 1024 * which + (16 * c1 + g + 4 * v) * 32 + 16 * c2 + i0;
                *pa = (ww == 0 ? 0.0 : *pa) + pp[c1][c2][v];
              }
            }
        }
        __syncthreads();
      }
    }
    if (tid < r) rho[tid] = SM[tid * 32 + tid];
    __syncthreads();
    // residual of each Ritz vector: |G x_c - rho_c x_c|^2 over the rows, then the waves
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (c >= NC) continue;
      const int col = 16 * c + i0;
      const double rc = col < r ? rho[col] : 0.0;
      double s = 0.0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const double d = gxacc[c][v] - rc * xacc[c][v];
        s = fma(d, d, s);
      }
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (g == 0 && col < r) colred[w][col] = s;
    }
    __syncthreads();
    if (tid < r) {
      double s = 0.0;
      for (int ww = 0; ww < NW; ++ww) s += colred[ww][tid];
      res2[tid] = s;
    }
    // orthonormality defect of X, |X^T G X|_F^2 and its off-diagonal part
    double dx = 0.0, af = 0.0, ff = 0.0;
    for (int e = tid; e < r * r; e += NTH) {
      const int a = e / r, b = e - a * r;
      const double xv = SM[1024 + a * 32 + b] - (a == b ? 1.0 : 0.0);
      const double av = SM[a * 32 + b];
      dx = fmax(dx, xv == xv ? fabs(xv) : 1e300);
      af = fma(av, av, af);
      if (a != b) ff = fma(av, av, ff);
    }
    const double defect = wg_max<NW>(dx, red);
    const double a_f2 = wg_sum<NW>(af, red);
    const double f_f2 = wg_sum<NW>(ff, red);

    // ---- decision (thread 0, then shared)
    if (tid == 0) {
      int ok = 0, kk = -1;
      double rmax = 0.0, rsum = 0.0;
      for (int c = 0; c < r; ++c) {
        rmax = fmax(rmax, res2[c] == res2[c] ? res2[c] : 1e300);
        rsum += res2[c];
      }
      const bool conv = defect <= 1e-10 && sqrt(rmax) <= 0x1p-28 * gersh;
      if (conv) {
        ok = 1;
        // the effective rank from the Ritz vectors (see the header)
        double rs[kEigMaxR];
        for (int c = 0; c < r; ++c) {  // descending insertion sort
          double x = rho[c];
          int p = c;
          while (p > 0 && rs[p - 1] < x) { rs[p] = rs[p - 1]; --p; }
          rs[p] = x;
        }
        const double unit = (3.0 * r * defect + 1e-12) * gersh;
        const double need_hi = energy * trace * (1.0 + 1e-13);
        const double need_lo = energy * trace * (1.0 - 1e-13);
        const double mu = sqrt(fmax(gf2 - a_f2, 0.0) + (1e-13 + 4.0 * r * defect) * gf2);
        const double bres = sqrt(rsum) + 2.0 * sqrt(f_f2) + 2.0 * r * defect * gersh;
        double cum = 0.0;
        for (int k = 1; k <= r; ++k) {
          cum += rs[k - 1];
          if (cum - k * unit >= need_hi) { kk = k; break; }
        }
        if (kk > 0) {
          const int j = kk - 1;
          double best = -1e300;
          for (int i = 0; i <= j; ++i) {
            double c = 0.0;
            for (int q = 0; q < j - i; ++q) c += rs[q];
            best = fmax(best, c + i * mu);
          }
          const double up = best + sqrt((double)j) * bres + j * unit;
          if (!(up < need_lo)) kk = -1;
        }
      }
      s_flag[0] = ok;
      s_flag[1] = kk;
    }
    __syncthreads();
    if (s_flag[0]) {  // (uniform) converged: the Ritz vectors are the rows of W
      done = true;
      k_cert = s_flag[1];
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
            s_amax[w][col] = best;
            s_aidx[w][col] = bidx;
            colred[w][col] = bval;
          }
        }
        __syncthreads();
        if (tid < r) {
          double best = -1.0, bval = 0.0;
          int bidx = D;
          for (int ww = 0; ww < NW; ++ww) {
            const double a = s_amax[ww][tid];
            const int ix = s_aidx[ww][tid];
            if (a > best || (a == best && ix < bidx)) { best = a; bidx = ix; bval = colred[ww][tid]; }
          }
          rho[tid] = bval < 0.0 ? -1.0 : 1.0;  // rho is no longer needed: it holds the sign
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (c >= NC) continue;
          const int col = 16 * c + i0;
          if (col >= r) continue;
          const double sg = rho[col];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 16 * w + g + 4 * v;
            W_out[((size_t)m * r + col) * D + row] = (float)(sg * xacc[c][v]);
          }
        }
      }
    }
  }

  if (tid == 0) {
    const bool keep = done && k_cert >= 0;
    k_eff_out[m] = keep ? k_cert : kWarmMiss;
    if (warm_out) warm_out[m] = keep ? 1 : 0;
  }
}

// G [M][D][D] (float64, lower triangle read), W_prev [M][r][D] -> W_out (rows of matrices
// whose refit converged and whose k_eff is certain), k_eff_out (k, or kWarmMiss), warm_out
// (1 / 0, may be null).
__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(ceil_div(n, kBlock)), dim3(kBlock), 0, st, p, n, v);
  return hipGetLastError();
}

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
