// One 128 x 128 fp32 MFMA tile and its K loop, shared by the plain / step
// GEMM kernels (gemm.hip) and the fused projection + scan (fused.hip).
//
// Tiling: a workgroup computes a TBM x 128 tile of C (TBM = 128 with 4
// waves, or 256 with 8 waves); each wave owns 64 x 64 (2 x 2 MFMA tiles of
// 32 x 32, 64 accumulators per lane).  K advances 16 at a time through
// double-buffered LDS tiles; global loads for step k+1 are in flight while
// the matrix cores work on step k.
//
// Operand layout of v_mfma_f32_32x32x2_f32 (one 32x32x2 product per wave):
// lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator r of
// lane l is C[8*(r/4) + 4*(l/32) + r%4][l % 32].
//
// Paired columns (step mode and the fused projection + scan): the tile's 128
// B-columns are 64 channels d taken twice -- each wave's first 32 columns are
// k[:, d] and its next 32 are p[:, d] for the same d -- so accumulator set
// j = 0 of a lane holds k and set j = 1 holds p of the same (row, d).
#pragma once

#include "internal.hpp"

namespace sr {
namespace gt {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int PAD = 4;  // LDS row padding (floats) against bank conflicts

enum Mode { kPlain = 0, kStep = 1 };  // kStep: paired k / p columns

struct GemmParams {
  int64_t M, N, K;
  const float* A;
  int64_t lda;
  const float* Bm;
  int64_t ldb;
  float* C;
  int64_t ldc;
  // step mode
  int64_t D_h;
  const float* h_prev;
  float* h_next;
  // step mode with time decay of the carried state (rate null: none)
  const float* rate;     // [D_h]
  const float* gap;      // [M] gap preceding the token, per row
  int log1p_gap;
  uint32_t* saturated;   // or null: OR-ed with 1 when a rate * gap exceeds the clamp
  // split-K: blockIdx.z covers K rows [z*k_split, (z+1)*k_split); with
  // `partial` set, raw tile sums go to partial[z][M][Ncols] for a reduction.
  int64_t k_split;
  float* partial;
  int64_t ncols;
  int64_t tiles_n;  // tiles along N (blockIdx.x = m_tile * tiles_n + n_tile)
};

// Global column of B (and C) for block column c of the tile starting at n0.
template <int MODE>
__device__ __forceinline__ int64_t b_col(const GemmParams& P, int64_t n0, int c) {
  if (MODE == kPlain) return n0 + c;
  // step: n0 is the first channel of the tile (64 channels per tile).
  const int wn = c / 64, within = c % 64, half = within / 32, j = within % 32;
  return int64_t(half) * P.D_h + n0 + 32 * wn + j;
}

template <int MODE>
__device__ __forceinline__ bool b_col_ok(const GemmParams& P, int64_t n0, int c) {
  if (MODE == kPlain) return n0 + c < P.N;
  const int wn = c / 64, j = (c % 64) % 32;
  return n0 + 32 * wn + j < P.D_h;
}

// The K loop of one tile of TBM (128 or 256) rows x BN columns, run by
// 2 * TBM threads: TBM / 64 x 2 waves, each owning 64 x 64 (2 x 2 MFMA tiles
// of 32 x 32).  A rows row0 .. row0 + rows - 1 (the rest of the tile reads
// zeros), B columns from n0 (MODE decides how), K in [k_begin, k_end).
// Leaves the sums in acc and ends with a barrier, after which As / Bs are
// free.  FULL: the host has checked that every row, column and K step of
// the tile is in range and the operands allow 16-byte loads, so the loads
// need no tests and walk two pointers.
template <int MODE, int TBM, bool FULL = false>
__device__ __forceinline__ void tile_mainloop(const GemmParams& P, int64_t row0, int64_t rows,
                                              int64_t n0, int64_t k_begin, int64_t k_end,
                                              float (&As)[2][BK][TBM + PAD],
                                              float (&Bs)[2][BK][BN + PAD],
                                              floatx16 (&acc)[2][2]) {
  static_assert(TBM == 128 || TBM == 256, "tile rows");
  constexpr int NTH = 2 * TBM;
  constexpr int BPER = BK * BN / NTH;      // B floats per thread: 8 or 4
  constexpr int BTPR = BN / BPER;          // threads per B row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Global -> register staging: A tile TBM x 16 (8 floats per thread, one
  // row), B tile 16 x 128 (BPER floats per thread, one k row).
  const int a_row = tid >> 1, a_k = (tid & 1) * 8;
  const int b_k = tid / BTPR, b_c = (tid % BTPR) * BPER;
  const bool a_vec = (P.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(P.A) & 15) == 0);
  const bool b_vec = (P.ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(P.Bm) & 15) == 0) &&
                     (MODE == kPlain || P.D_h % 4 == 0);
  float ra[8], rb[BPER];
  const float* a_ptr = P.A + (row0 + a_row) * P.lda + k_begin + a_k;
  const float* b_ptr = P.Bm + (k_begin + b_k) * P.ldb + b_col<MODE>(P, n0, b_c);

  auto load_full = [&]() {
    const float4* sa = reinterpret_cast<const float4*>(a_ptr);
    const float4 u = sa[0], v = sa[1];
    ra[0] = u.x; ra[1] = u.y; ra[2] = u.z; ra[3] = u.w;
    ra[4] = v.x; ra[5] = v.y; ra[6] = v.z; ra[7] = v.w;
    const float4* sb = reinterpret_cast<const float4*>(b_ptr);
#pragma unroll
    for (int q = 0; q < BPER / 4; ++q) {
      const float4 w = sb[q];
      rb[4 * q + 0] = w.x; rb[4 * q + 1] = w.y; rb[4 * q + 2] = w.z; rb[4 * q + 3] = w.w;
    }
    a_ptr += BK;
    b_ptr += BK * P.ldb;
  };
  auto load_tiles = [&](int64_t k0) {
    const bool row_ok = a_row < rows;
    const int64_t gm = row0 + a_row;
    const int64_t gk = k0 + a_k;
    if (row_ok && a_vec && gk + 8 <= k_end) {
      const float4* src = reinterpret_cast<const float4*>(P.A + gm * P.lda + gk);
      const float4 u = src[0], v = src[1];
      ra[0] = u.x; ra[1] = u.y; ra[2] = u.z; ra[3] = u.w;
      ra[4] = v.x; ra[5] = v.y; ra[6] = v.z; ra[7] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        ra[j] = (row_ok && gk + j < k_end) ? P.A[gm * P.lda + gk + j] : 0.0f;
    }
    const int64_t bk = k0 + b_k;
    const int64_t gc = b_col<MODE>(P, n0, b_c);
    if (bk < k_end && b_vec && b_col_ok<MODE>(P, n0, b_c + BPER - 1)) {
      const float4* src = reinterpret_cast<const float4*>(P.Bm + bk * P.ldb + gc);
#pragma unroll
      for (int v = 0; v < BPER / 4; ++v) {
        const float4 u = src[v];
        rb[4 * v + 0] = u.x; rb[4 * v + 1] = u.y; rb[4 * v + 2] = u.z; rb[4 * v + 3] = u.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < BPER; ++j)
        rb[j] = (bk < k_end && b_col_ok<MODE>(P, n0, b_c + j))
                    ? P.Bm[bk * P.ldb + b_col<MODE>(P, n0, b_c + j)]
                    : 0.0f;
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) As[buf][a_k + j][a_row] = ra[j];
#pragma unroll
    for (int j = 0; j < BPER; ++j) Bs[buf][b_k][b_c + j] = rb[j];
  };

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int n_k = k_end > k_begin ? int((k_end - k_begin + BK - 1) / BK) : 0;
  if constexpr (FULL) load_full(); else load_tiles(k_begin);
  store_tiles(0);
  __syncthreads();
  const int kl = lane >> 5, ml = lane & 31;
  for (int kt = 0; kt < n_k; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_k) {
      if constexpr (FULL) load_full(); else load_tiles(k_begin + int64_t(kt + 1) * BK);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[buf][2 * kk + kl][wm * 64 + i * 32 + ml];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[buf][2 * kk + kl][wn * 64 + j * 32 + ml];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < n_k) store_tiles(buf ^ 1);
    __syncthreads();
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Renumbering so that each XCD gets a contiguous range of tile ids
// keeps tiles that share operands on one L2.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t bid, uint32_t n) {
  const uint32_t per = n / 8;
  return bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
}

}  // namespace gt
}  // namespace sr
