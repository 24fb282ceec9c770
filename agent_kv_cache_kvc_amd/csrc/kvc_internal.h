// Internal definitions shared by the HIP translation units of libkvc (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

// ---------------------------------------------------------------- launch geometry
constexpr int kWave = 64;             // CDNA wavefront width
constexpr int kBlock = 256;           // 4 waves per workgroup everywhere
constexpr int kPoolRows = 256;        // tokens per pooling workgroup
constexpr int kCorrRowsPerIter = 128; // tokens per correction workgroup iteration (4 waves x 32)
constexpr int kCorrIters = 4;         // iterations per correction workgroup (512 tokens)
constexpr int kMaxA = 16;             // anchors per segment held in registers
constexpr int kMaxKSlots = 256;       // A * ceil16(r) bound of the LDS-staged factors
constexpr int kMaxR = 64;             // rank bound of the correction kernel
constexpr int kJacobiMaxSweeps = 40;  // hard cap: every workgroup leaves the sweep loop

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// ---------------------------------------------------------------- correction workspace
struct CorrectLayout {
  int S, T, d, A;
  int n_pool_tiles;   // pooling partials per segment and per K|V
  int n_corr_tiles;   // correction workgroups per segment and per K|V
  size_t off_pool;    // float [2][S][n_pool_tiles][d]
  size_t off_next;    // float [2][S][n_corr_tiles][d]   (pooled output partials)
  size_t off_q;       // float [S][2d]
  size_t off_w;       // float [S][A]
  size_t off_score;   // float [S]
  size_t off_mask;    // uint8 [S]
  size_t off_ctr;     // int [1]: work counter of the correction pass
  size_t bytes;
};

inline CorrectLayout correct_layout(int L, int H, int T, int d, int A) {
  CorrectLayout c{};
  c.S = L * H;
  c.T = T;
  c.d = d;
  c.A = A;
  c.n_pool_tiles = T > 0 ? ceil_div(T, kPoolRows) : 1;
  c.n_corr_tiles = T > 0 ? ceil_div(T, kCorrRowsPerIter * kCorrIters) : 1;
  size_t o = 0;
  c.off_pool = o;  o = align_up(o + sizeof(float) * 2ull * c.S * c.n_pool_tiles * d, 256);
  c.off_next = o;  o = align_up(o + sizeof(float) * 2ull * c.S * c.n_corr_tiles * d, 256);
  c.off_q = o;     o = align_up(o + sizeof(float) * (size_t)c.S * 2 * d, 256);
  c.off_w = o;     o = align_up(o + sizeof(float) * (size_t)c.S * A, 256);
  c.off_score = o; o = align_up(o + sizeof(float) * (size_t)c.S, 256);
  c.off_mask = o;  o = align_up(o + (size_t)c.S, 256);
  c.off_ctr = o;   o = align_up(o + sizeof(int), 256);
  c.bytes = o;
  return c;
}

// ---------------------------------------------------------------- fit workspace
struct FitLayout {
  int M, T, d, r;
  int rpad;         // r rounded up to 32 (rows of the bf16 hi/lo factor copies)
  int slab;         // rows staged per Gram iteration
  int nsplit;       // Gram partials per matrix
  int chunk;        // rows per Gram workgroup (multiple of slab)
  int nblk;         // upper-triangular 32x32 blocks of G
  size_t off_gram;  // float [M][nsplit][nblk][16][64]
  size_t off_whi;   // bf16 [M][rpad][d]
  size_t off_wlo;   // bf16 [M][rpad][d]
  size_t off_sweeps;// int [M]
  size_t bytes;
};

inline FitLayout fit_layout(int M, int T, int d, int r, int target_wgs = 2048) {
  FitLayout f{};
  f.M = M; f.T = T; f.d = d; f.r = r;
  f.rpad = (r + 31) / 32 * 32;
  f.slab = 16384 / d;  // 128 rows at d = 128, 256 at d = 64
  int nb = d / 32;
  f.nblk = nb * (nb + 1) / 2;
  int max_split = T > 0 ? ceil_div(T, f.slab) : 1;
  int want = M > 0 ? ceil_div(target_wgs, M) : 1;
  int ns = want < 1 ? 1 : (want > max_split ? max_split : want);
  int slabs_per = T > 0 ? ceil_div(ceil_div(T, f.slab), ns) : 1;
  f.chunk = slabs_per * f.slab;
  f.nsplit = T > 0 ? ceil_div(T, f.chunk) : 1;
  size_t o = 0;
  f.off_gram = o;   o = align_up(o + sizeof(float) * (size_t)M * f.nsplit * f.nblk * 1024, 256);
  f.off_whi = o;    o = align_up(o + 2ull * M * f.rpad * d, 256);
  f.off_wlo = o;    o = align_up(o + 2ull * M * f.rpad * d, 256);
  f.off_sweeps = o; o = align_up(o + sizeof(int) * (size_t)M, 256);
  f.bytes = o;
  return f;
}

// ---------------------------------------------------------------- launchers (.hip files)
hipError_t launch_pool_partials(const void* K, const void* V, int S, int T, int d, int dtype,
                                float* partials, int n_tiles, hipStream_t st);
hipError_t launch_score(const float* partials, int n_tiles, int T, const float* q_in,
                        const float* desc, int S, int d, int A, float tau, float* q_ws,
                        float* w_ws, float* score_ws, uint8_t* mask_ws, float* q_out,
                        float* score_out, float* w_out, uint8_t* mask_out, int* ctr,
                        hipStream_t st);
hipError_t launch_correct(const void* K, const void* V, int S, int T, int d, int dtype,
                          const void* U, const void* W, int A, int r, const float* w,
                          const uint8_t* mask, const void* K_fb, const void* V_fb, void* K_out,
                          void* V_out, float* next_partials, int* ctr, hipStream_t st);
hipError_t launch_reduce_pool(const float* partials, int n_tiles, int T, int S, int d,
                              float* q_out, hipStream_t st);
hipError_t launch_fit(const void* delta, const FitLayout& f, int dtype, double energy,
                      float* U_out, float* W_out, int32_t* k_eff, float* eig, char* ws,
                      hipStream_t st);

}  // namespace kvc
