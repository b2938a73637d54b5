// fp32 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x2_f32), for the minGRU
// projections [k | p] = x W_in and y = h W_out, and the single-token step whose
// epilogue applies the recurrence.  The tile and its K loop are in
// gemm_tile.hpp.
//
// Step mode (the single-token step of the minGRU profile's sequential guide):
// with paired k / p columns one lane holds k and p of the same (row, d), and
// the epilogue computes
//     z = sigma(k), h_next = (1 - z) h_prev + z g(p) = h_prev + z (g(p) - h_prev)
// without writing [k | p] anywhere.

#include "gemm_tile.hpp"

namespace sr {
namespace {

using namespace gt;

// sigma(k) from e = e^{-|k|}: 1/(1+e) for k >= 0, e/(1+e) below.
__device__ __forceinline__ float sigmoid_f(float k) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(-fabsf(k) * kLog2e);
  const float big = __builtin_amdgcn_rcpf(1.0f + e);
  return k >= 0.0f ? big : e * big;
}

__device__ __forceinline__ float g_act(float p) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float ep = __builtin_amdgcn_exp2f(fminf(p, 0.0f) * kLog2e);
  return p >= 0.0f ? p + 0.5f : ep * __builtin_amdgcn_rcpf(1.0f + ep);
}

// The carried state entering the step for one (row, channel): h_prev (zero
// when absent), with time decay first scaled by exp(-min(rate_d * gap_row,
// 1e4)) (the token boundary comes before the token's write; exp(-1e4) is
// zero in float32, so the clamp changes no value and only marks saturation).
__device__ __forceinline__ float carried_state(const GemmParams& P, int64_t row, int64_t d) {
  float hp = P.h_prev ? P.h_prev[row * P.D_h + d] : 0.0f;
  if (P.rate != nullptr) {
    constexpr float kClamp = 1.0e4f, kLog2e = 1.4426950408889634f;
    const float gap = P.log1p_gap ? log1pf(P.gap[row]) : P.gap[row];
    const float e = P.rate[d] * gap;
    if (e > kClamp && P.saturated != nullptr)
      __hip_atomic_fetch_or(P.saturated, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    hp *= __builtin_amdgcn_exp2f(fminf(e, kClamp) * -kLog2e);
  }
  return hp;
}

// h_next = (1 - z) h + z g(p) with z = sigma(k), h the carried state,
// evaluated as the interpolation h + z (g(p) - h): the complement 1 - z is
// never rounded on its own, so a gate that keeps almost all of the state
// (z tiny) moves it by exactly z times the gap to the candidate, and h = g(p)
// is a fixed point.
__device__ __forceinline__ float step_value(float k, float p, float h) {
  return fmaf(sigmoid_f(k), g_act(p) - h, h);
}

__device__ __forceinline__ void step_update(const GemmParams& P, int64_t row, int64_t d, float k,
                                            float p) {
  P.h_next[row * P.D_h + d] = step_value(k, p, carried_state(P, row, d));
}

// One TBM x 128 tile per workgroup; blockIdx.x numbers the tiles (N tiles
// fastest, so consecutive tiles share their A rows; renumbered per XCD),
// blockIdx.z the K slice.
template <int MODE, int TBM, bool FULL>
__global__ __launch_bounds__(2 * TBM) void gemm_f32_kernel(const GemmParams P) {
  __shared__ float As[2][BK][TBM + PAD];
  __shared__ float Bs[2][BK][BN + PAD];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int kl = lane >> 5, ml = lane & 31;
  const uint32_t tile = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t m0 = int64_t(tile / uint32_t(P.tiles_n)) * TBM;
  const int64_t n0 = int64_t(tile % uint32_t(P.tiles_n)) * (MODE == kPlain ? BN : BN / 2);
  const int64_t k_begin = int64_t(blockIdx.z) * P.k_split;
  const int64_t k_end = (k_begin + P.k_split < P.K) ? k_begin + P.k_split : P.K;
  floatx16 acc[2][2];
  tile_mainloop<MODE, TBM, FULL>(P, m0, P.M - m0, n0, k_begin, k_end, As, Bs, acc);

  // Epilogue.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * 64 + i * 32 + (r / 4) * 8 + kl * 4 + (r % 4);
      if (row >= P.M) continue;
      if (P.partial != nullptr) {
        // Split-K: store this K slice's sums; the reduction applies the rest.
        float* part = P.partial + (int64_t(blockIdx.z) * P.M + row) * P.ncols;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (MODE == kPlain) {
            const int64_t col = n0 + wn * 64 + j * 32 + ml;
            if (col < P.N) part[col] = acc[i][j][r];
          } else {
            const int64_t d = n0 + 32 * wn + ml;
            if (d < P.D_h) part[j * P.D_h + d] = acc[i][j][r];
          }
        }
      } else if (MODE == kPlain) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = n0 + wn * 64 + j * 32 + ml;
          if (col < P.N) P.C[row * P.ldc + col] = acc[i][j][r];
        }
      } else {
        const int64_t d = n0 + 32 * wn + ml;
        if (d < P.D_h) step_update(P, row, d, acc[i][0][r], acc[i][1][r]);
      }
    }
  }
}

// Products with at most kSmallM rows (a step over a few streams): a
// 128-row MFMA tile would spend its whole K loop on them, so they run on
// fp32 FMAs instead.  A workgroup of 1024 threads owns CB columns (step
// mode: CB/2 channels, k then p) and all rows; thread (c, s) accumulates
// column c over the s-th of 1024/CB K slices, and the slices are summed in
// LDS in slice order (deterministic), then stored or used by the step
// update.  Narrower column blocks give more workgroups and shorter K loops
// (the loop is latency-bound: a few dozen loads per thread).
constexpr int kSmallM = 16;
constexpr int kSmallThreads = 1024;

template <int MODE, int MR, int CB>
__global__ __launch_bounds__(kSmallThreads) void small_m_kernel(const GemmParams P) {
  constexpr int SL = kSmallThreads / CB;  // K slices
  constexpr int HC = CB / 2;              // step mode: channels per block
  __shared__ float red[SL][MR][CB];
  const int c = threadIdx.x % CB, sl = threadIdx.x / CB;
  int64_t col;
  bool col_ok;
  if (MODE == kPlain) {
    col = int64_t(blockIdx.x) * CB + c;
    col_ok = col < P.N;
  } else {
    const int64_t ch = int64_t(blockIdx.x) * HC + (c % HC);
    col = (c < HC ? 0 : P.D_h) + ch;
    col_ok = ch < P.D_h;
  }
  const int64_t ks = (P.K + SL - 1) / SL;
  const int64_t k0 = sl * ks, k1 = (k0 + ks < P.K) ? k0 + ks : P.K;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  if (col_ok) {
    // Eight B loads in flight per round.
    const float* bp = P.Bm + k0 * P.ldb + col;
    int64_t k = k0;
    for (; k + 8 <= k1; k += 8, bp += 8 * P.ldb) {
      float b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) b[u] = bp[u * P.ldb];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int m = 0; m < MR; ++m)
          if (m < P.M) acc[m] = fmaf(P.A[m * P.lda + k + u], b[u], acc[m]);
    }
    for (; k < k1; ++k, bp += P.ldb) {
      const float b = *bp;
#pragma unroll
      for (int m = 0; m < MR; ++m)
        if (m < P.M) acc[m] = fmaf(P.A[m * P.lda + k], b, acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) red[sl][m][c] = acc[m];
  __syncthreads();
  // Thread (c, m): the slices of (row m, column c), in order.
  if (threadIdx.x < CB * MR) {
    const int rc = threadIdx.x % CB, m = threadIdx.x / CB;
    if (m < P.M) {
      float v = 0.0f;
#pragma unroll 8
      for (int q = 0; q < SL; ++q) v += red[q][m][rc];
      if (MODE == kPlain) {
        const int64_t oc = int64_t(blockIdx.x) * CB + rc;
        if (oc < P.N) P.C[m * P.ldc + oc] = v;
      } else if (rc < HC) {
        const int64_t ch = int64_t(blockIdx.x) * HC + rc;
        if (ch < P.D_h) {
          float vp = 0.0f;
#pragma unroll 8
          for (int q = 0; q < SL; ++q) vp += red[q][m][rc + HC];
          step_update(P, m, ch, v, vp);
        }
      }
    }
  }
}

// Products with a few hundred rows (the step over a batch of streams): the
// 128 x 128 tiles would be too few to fill the part, and splitting K across
// workgroups costs a round trip of the slices' sums through HBM.  Instead a
// workgroup owns a narrow tile of TM (64 or 32) rows x 64 columns (step
// mode: the k and p columns of 32 channels, so that a lane holds k and p of
// the same (row, d)) and splits K over its KG waves: wave g computes the
// whole tile (TM / 32 x 2 MFMA tiles of 32 x 32) over the g-th share of K,
// staged through its own LDS buffers.  The waves' sums meet in LDS and are
// added in wave order (deterministic), by all threads, which then store or
// apply the step update.
constexpr int kNarrowCols = 64;
constexpr int kNarrowMaxM = 512;
// Up to kNarrowWideMaxM rows the narrow tiles also replace a 128 x 128
// tiling that would leave CUs idle (fewer than 512 tiles; it would split K
// across workgroups and add a reduction launch) when K is at most
// kNarrowWideMaxK; with deeper K the split 128 x 128 tiles are faster.
// Measured (one process): layer forward B=2 T=1024 D=512 78 -> 54 us,
// B=2 T=2048 D=512 100 -> 94 us, step B=2048 D=512 67 -> 42 us, step B=1024
// D=1024 81 -> 68 us; with K = 2048 (B=2 T=1024 D=2048) 449 -> 456 us.
constexpr int kNarrowWideMaxM = 4096;
constexpr int kNarrowWideMaxK = 1024;
constexpr int kNarrowSK = 16; // K per pipeline stage

// Waves (K groups) per workgroup and stage buffers per wave, by tile height.
// A wave keeps kStages - 1 stages loading while it multiplies one: a stage
// holds only 32 (64-row tiles) or 16 (32-row tiles) MFMAs per wave, too
// short to cover a load's latency alone.  For 64-row tiles deeper prefetch
// beats more waves: four waves with three stages each (one wave per SIMD)
// against eight waves that fit only two (step B=256 D=2048, x_t W_in:
// 41.7 -> 36.9 us; a fourth stage, operands read into registers a half
// stage ahead, or the loads spread between the MFMAs gained nothing or
// lost).  The 32-row tiles keep eight waves (four are no faster).
constexpr int narrow_waves(int TM) { return TM == 64 ? 4 : 8; }
constexpr int narrow_stages(int, bool full) { return full ? 3 : 2; }

template <int TM, bool FULL>
struct Narrow {
  static constexpr int kKG = narrow_waves(TM);
  static constexpr int kRI = TM / 32;                       // row blocks per wave
  static constexpr int kThreads = 64 * kKG;
  static constexpr int kAPer = TM * kNarrowSK / 64;         // A floats per thread
  static constexpr int kBPer = kNarrowSK * kNarrowCols / 64;  // B floats per thread (16)
  // A is staged row-major, [row][k], B as [k][col].  Full tiles are loaded
  // straight from global memory into LDS (16 bytes per lane, the lanes of an
  // instruction filling 1 KiB in lane order), so their rows are unpadded and
  // the four 16-byte chunks of an A row are stored in the order chunk ^
  // ((row >> 1) & 3): the 16-byte reads of eight consecutive rows then hit
  // distinct banks.  The register-staged path pads rows instead (A rows of
  // 20 floats: 16-byte aligned, eight consecutive rows in distinct banks).
  static constexpr int kLdA = FULL ? kNarrowSK : kNarrowSK + 4;
  static constexpr int kLdB = FULL ? kNarrowCols : kNarrowCols + PAD;
  static constexpr int kLdR = kNarrowCols + PAD;
  static constexpr int kStageFloats = TM * kLdA + kNarrowSK * kLdB;
  static constexpr int kStages = narrow_stages(TM, FULL);
  static constexpr int kStageLoads = (TM * kNarrowSK + kNarrowSK * kNarrowCols) / 256;
  static constexpr int kStagingFloats = kKG * kStages * kStageFloats;
  static_assert(kStageLoads * 256 == TM * kNarrowSK + kNarrowSK * kNarrowCols, "whole loads");
  static constexpr int kRedFloats = kKG * TM * kLdR;  // the waves' sums, over the staging
  static constexpr int kSmemFloats = kStagingFloats > kRedFloats ? kStagingFloats : kRedFloats;
  static_assert(TM == 32 || TM == 64, "tile rows");
  static_assert(kAPer % 4 == 0 && kBPer % 4 == 0, "16-byte staging");
  static_assert(!FULL || (kLdA == 16 && kLdB == 64), "direct loads fill unpadded 1 KiB blocks");
  static_assert(FULL ? kStages == 3 : kStages == 2, "the K loops below");
  static_assert(kSmemFloats * 4 <= 160 * 1024, "LDS of one CU");
};

// Copies 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's bytes land at lds_block + 16 l, for the
// wave-uniform lds_block.  Completion is tracked by vmcnt.
__device__ __forceinline__ void load_lds16(const float* src, float* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_block, 16, 0, 0);
}

// Waits until this wave's direct loads have landed in LDS (vmcnt) and its
// LDS reads have returned (lgkmcnt), so that the next stage may read the one
// buffer and overwrite the other.
__device__ __forceinline__ void wait_stage() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }
// The same, leaving the last N direct loads (one later stage) in flight.
template <int N>
__device__ __forceinline__ void wait_stage_but() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void put4(float* r, int q, float4 v) {
  r[4 * q] = v.x; r[4 * q + 1] = v.y; r[4 * q + 2] = v.z; r[4 * q + 3] = v.w;
}
__device__ __forceinline__ float4 get4(const float* r, int q) {
  return make_float4(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]);
}

// Global column of B for tile column c (plain: n0 + c; step: k of channel
// n0 + c for c < 32, p of channel n0 + c - 32 after).
template <int MODE>
__device__ __forceinline__ int64_t narrow_col(const GemmParams& P, int64_t n0, int c) {
  if (MODE == kPlain) return n0 + c;
  return int64_t(c / 32) * P.D_h + n0 + (c % 32);
}
template <int MODE>
__device__ __forceinline__ bool narrow_col_ok(const GemmParams& P, int64_t n0, int c) {
  return MODE == kPlain ? n0 + c < P.N : n0 + (c % 32) < P.D_h;
}

template <int MODE, int TM, bool FULL>
__global__ __launch_bounds__(64 * narrow_waves(TM)) void narrow_kernel(const GemmParams P) {
  using G = Narrow<TM, FULL>;
  constexpr int SK = kNarrowSK, KG = G::kKG, RI = G::kRI;
  __shared__ __align__(16) float smem[G::kSmemFloats];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's K group
  const int kl = lane >> 5, ml = lane & 31;
  const int64_t cols = MODE == kPlain ? P.N : P.D_h;
  const int64_t tiles_m = (P.M + TM - 1) / TM;
  const uint32_t tile = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t m0 = int64_t(tile % uint32_t(tiles_m)) * TM;  // row tiles of a column tile adjacent
  const int64_t n0 = int64_t(tile / uint32_t(tiles_m)) * (MODE == kPlain ? kNarrowCols : kNarrowCols / 2);

  // This wave's K stages.
  const int64_t n_kt = (P.K + SK - 1) / SK;
  const int64_t per = (n_kt + KG - 1) / KG;
  const int64_t kt0 = g * per;
  const int64_t kt1 = kt0 + per < n_kt ? kt0 + per : n_kt;
  const int iters = int(per);  // the same for every wave

  // This wave's kStages stages, kStageFloats apart: A [TM][kLdA], then B [SK][kLdB].
  float* const stages = smem + g * G::kStages * G::kStageFloats;
  auto stage_at = [&](int buf) { return stages + buf * G::kStageFloats; };
  // Offset of A's 4-float chunk (row, k .. k + 3) in a stage (swizzled when full).
  auto a_off = [](int row, int k) {
    return row * G::kLdA + (FULL ? (((k >> 2) ^ ((row >> 1) & 3)) << 2) : k);
  };
  auto b_off = [](int k, int c) { return TM * G::kLdA + k * G::kLdB + c; };

  // Staging, in float4 chunks.  A chunk q of a lane: row q * 16 + lane / 4,
  // k (lane % 4) * 4, so one load instruction covers 16 whole row segments
  // (16 cache lines, not 64).  B chunk q: k row q * 4 + lane / 16, columns
  // (lane % 16) * 4: four whole 256-byte row segments per instruction.
  constexpr int kAQ = G::kAPer / 4, kBQ = G::kBPer / 4;
  static_assert(kAQ * 16 == TM && kBQ * 4 == SK && SK == 16, "staging chunks cover the stage");
  const int a_r = lane >> 2, a_k = (lane & 3) * 4;
  const int b_k = lane >> 4, b_c = (lane & 15) * 4;
  const bool a_vec = (P.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(P.A) & 15) == 0);
  const bool b_vec = (P.ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(P.Bm) & 15) == 0) &&
                     (MODE == kPlain || P.D_h % 4 == 0);
  const bool b_cols_ok = narrow_col_ok<MODE>(P, n0, b_c + 3);  // the chunk's last column
  const int64_t gc = narrow_col<MODE>(P, n0, b_c);
  float ra[4 * kAQ], rb[4 * kBQ];  // plain floats: kept in registers
  // Full tiles: the lane's A chunk goes to slot lane % 4 of its row, which
  // holds chunk (lane % 4) ^ ((row >> 1) & 3) (row = q * 16 + a_r, and
  // q * 16 does not change (row >> 1) & 3).
  const int a_kf = FULL ? (((lane & 3) ^ ((a_r >> 1) & 3)) << 2) : a_k;
  const float* a_ptr = P.A + (m0 + a_r) * P.lda + kt0 * SK + a_kf;
  const float* b_ptr = P.Bm + (kt0 * SK + b_k) * P.ldb + gc;

  // Full tiles, the next K stage into the stage at dst: instruction q of A
  // fills rows q*16 .. q*16+15 (1 KiB), instruction q of B k rows q*4 .. q*4+3.
  auto issue_direct = [&](float* dst) {
#pragma unroll
    for (int q = 0; q < kAQ; ++q) load_lds16(a_ptr + q * 16 * P.lda, dst + q * 256);
#pragma unroll
    for (int q = 0; q < kBQ; ++q) load_lds16(b_ptr + q * 4 * P.ldb, dst + b_off(0, 0) + q * 256);
    a_ptr += SK;
    b_ptr += SK * P.ldb;
  };

  // K stage kt of this wave (zeros past the wave's range, K, M or N).
  auto load_checked = [&](int64_t kt) {
    const bool in = kt < kt1;
    const int64_t k_lim = in ? (kt + 1) * SK < P.K ? (kt + 1) * SK : P.K : 0;
    const int64_t ka = kt * SK + a_k;
#pragma unroll
    for (int q = 0; q < kAQ; ++q) {
      const int64_t gm = m0 + q * 16 + a_r;
      const bool row_ok = gm < P.M;
      if (row_ok && a_vec && ka + 4 <= k_lim) {
        put4(ra, q, *reinterpret_cast<const float4*>(P.A + gm * P.lda + ka));
      } else {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (row_ok && ka + j < k_lim) ? P.A[gm * P.lda + ka + j] : 0.0f;
        put4(ra, q, make_float4(v[0], v[1], v[2], v[3]));
      }
    }
#pragma unroll
    for (int q = 0; q < kBQ; ++q) {
      const int64_t kb = kt * SK + q * 4 + b_k;
      const bool k_ok = kb < k_lim;
      if (k_ok && b_vec && b_cols_ok) {
        put4(rb, q, *reinterpret_cast<const float4*>(P.Bm + kb * P.ldb + gc));
      } else {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[j] = (k_ok && narrow_col_ok<MODE>(P, n0, b_c + j))
                     ? P.Bm[kb * P.ldb + narrow_col<MODE>(P, n0, b_c + j)]
                     : 0.0f;
        put4(rb, q, make_float4(v[0], v[1], v[2], v[3]));
      }
    }
  };
  auto store_stage = [&](float* dst) {
#pragma unroll
    for (int q = 0; q < kAQ; ++q) *reinterpret_cast<float4*>(dst + a_off(q * 16 + a_r, a_k)) = get4(ra, q);
#pragma unroll
    for (int q = 0; q < kBQ; ++q) *reinterpret_cast<float4*>(dst + b_off(q * 4 + b_k, b_c)) = get4(rb, q);
  };

  // Step mode: thread t finishes the (row, channel) pairs t, t + kThreads,
  // ... of the tile (channels fastest); their carried states are read now,
  // so that those loads are not waited for after the K loop.
  constexpr int kCh = kNarrowCols / 2;
  constexpr int kPairs = MODE == kStep ? TM * kCh / G::kThreads : 1;
  float carried[kPairs];
  if constexpr (MODE == kStep) {
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      const int e = tid + q * G::kThreads;
      const int64_t grow = m0 + e / kCh, d = n0 + e % kCh;
      carried[q] = (grow < P.M && d < cols) ? carried_state(P, grow, d) : 0.0f;
    }
  }

  floatx16 acc[RI][2];
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // The MFMAs of the stage at cur.  K order within a stage: MFMA s (s < SK /
  // 2) takes k = s from lanes 0..31 and k = SK / 2 + s from lanes 32..63 (the
  // same for A and B), so a lane reads its A values of all SK / 2 MFMAs with
  // 16-byte reads.
  auto mfma_stage = [&](const float* cur) {
    float a[RI][SK / 2];
#pragma unroll
    for (int i = 0; i < RI; ++i)
#pragma unroll
      for (int q = 0; q < SK / 8; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(cur + a_off(i * 32 + ml, kl * (SK / 2) + 4 * q));
        a[i][4 * q + 0] = v.x; a[i][4 * q + 1] = v.y; a[i][4 * q + 2] = v.z; a[i][4 * q + 3] = v.w;
      }
#pragma unroll
    for (int s = 0; s < SK / 2; ++s) {
      float b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = cur[b_off(kl * (SK / 2) + s, j * 32 + ml)];
#pragma unroll
      for (int i = 0; i < RI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j], acc[i][j], 0, 0, 0);
    }
  };
  // Each wave stages and reads only its own buffers, so the K loop needs no
  // workgroup barrier: a wave's LDS accesses take effect in its issue order,
  // and its direct loads are waited for (vmcnt) before it reads them.
  if constexpr (FULL) {
    // Three stages b0, b1, b2 in rotation; stage it is multiplied from
    // buffer it % 3 while stages it + 1 and it + 2 load.  One function with
    // three restrict pointers, so that the compiler sees that reading one
    // buffer does not wait for the loads into the other two.
    auto pipeline = [&](float* __restrict__ b0, float* __restrict__ b1, float* __restrict__ b2) {
      constexpr int L = G::kStageLoads;
      issue_direct(b0);
      if (iters > 1) {
        issue_direct(b1);
        wait_stage_but<L>();
      } else {
        wait_stage();
      }
      auto step = [&](const float* __restrict__ cur, float* __restrict__ nxt, int it) {
        const bool more = it + 2 < iters;
        if (more) issue_direct(nxt);
        mfma_stage(cur);
        if (more) wait_stage_but<L>(); else wait_stage();
      };
      for (int it = 0; it < iters; it += 3) {
        step(b0, b2, it);
        if (it + 1 < iters) step(b1, b0, it + 1);
        if (it + 2 < iters) step(b2, b1, it + 2);
      }
    };
    pipeline(stage_at(0), stage_at(1), stage_at(2));
  } else {
    load_checked(kt0);
    store_stage(stage_at(0));
    for (int it = 0; it < iters; ++it) {
      const int buf = it & 1;
      if (it + 1 < iters) load_checked(kt0 + it + 1);
      mfma_stage(stage_at(buf));
      if (it + 1 < iters) store_stage(stage_at(buf ^ 1));
    }
  }
  __syncthreads();  // every wave is done with the staging LDS

  // The waves' sums: red[g][row][c] over the staging LDS.
  float* red = smem;
  constexpr int kRedWave = TM * G::kLdR;
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + (r / 4) * 8 + kl * 4 + (r % 4);
        red[g * kRedWave + row * G::kLdR + j * 32 + ml] = acc[i][j][r];
      }
  __syncthreads();
  if (MODE == kPlain) {
    // Thread t: elements t, t + kThreads, ... of the TM x 64 tile (columns fastest).
#pragma unroll
    for (int q = 0; q < TM * kNarrowCols / G::kThreads; ++q) {
      const int e = tid + q * G::kThreads;
      const int row = e / kNarrowCols, c = e % kNarrowCols;
      float v = red[row * G::kLdR + c];
#pragma unroll
      for (int h = 1; h < KG; ++h) v += red[h * kRedWave + row * G::kLdR + c];
      const int64_t grow = m0 + row, gcol = n0 + c;
      if (grow < P.M && gcol < cols) P.C[grow * P.ldc + gcol] = v;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      const int e = tid + q * G::kThreads;
      const int row = e / kCh, c = e % kCh;
      float k = red[row * G::kLdR + c], p = red[row * G::kLdR + kCh + c];
#pragma unroll
      for (int h = 1; h < KG; ++h) {
        k += red[h * kRedWave + row * G::kLdR + c];
        p += red[h * kRedWave + row * G::kLdR + kCh + c];
      }
      const int64_t grow = m0 + row, d = n0 + c;
      if (grow < P.M && d < cols) P.h_next[grow * P.D_h + d] = step_value(k, p, carried[q]);
    }
  }
}

// Split-K reductions: the K slices' sums are added in slice order (so the
// result does not depend on scheduling), then stored or used by the step.
__global__ void reduce_plain_kernel(const float* part, int S, int64_t M, int64_t N, float* C,
                                    int64_t ldc) {
  const int64_t n = M * N, stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    float s = 0.0f;
    for (int z = 0; z < S; ++z) s += part[int64_t(z) * n + i];
    C[(i / N) * ldc + (i % N)] = s;
  }
}

__global__ void reduce_step_kernel(const GemmParams P, int S) {
  const int64_t n = P.M * P.D_h, stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t plane = P.M * P.ncols;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t row = i / P.D_h, d = i % P.D_h;
    float k = 0.0f, p = 0.0f;
    for (int z = 0; z < S; ++z) {
      k += P.partial[int64_t(z) * plane + row * P.ncols + d];
      p += P.partial[int64_t(z) * plane + row * P.ncols + P.D_h + d];
    }
    step_update(P, row, d, k, p);
  }
}

}  // namespace

namespace {

// Tiles of the 128 x 128 tiling (step mode: 64 channels per tile).
int64_t tiles_128(int64_t M, int64_t N, bool step) {
  return ((M + BM - 1) / BM) * (step ? (N / 2 + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN);
}

// K slices of the 128 x 128 tiling: enough workgroups for two per CU on a
// 256-CU part, each K slice at least 256 deep; small problems split K,
// large ones (whole-sequence projections) do not.
int splits_128(int64_t M, int64_t N, int64_t K, bool step) {
  if (K < 2 * 256) return 1;  // nothing worth splitting (and K = 0 has no slices)
  const int64_t tiles = tiles_128(M, N, step);
  if (tiles <= 0 || tiles >= 512) return 1;
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t by_k = K / 256;
  if (s > by_k) s = by_k;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  // Slices are whole multiples of the K step.
  const int64_t k_split = ((K + s - 1) / s + BK - 1) / BK * BK;
  return int((K + k_split - 1) / k_split);
}

// Products that run on the narrow tiles (at most kSmallM rows: the FMA path).
bool narrow_applies(int64_t M, int64_t N, int64_t K, bool step) {
  if (M <= kNarrowMaxM) return true;
  return M <= kNarrowWideMaxM && K <= kNarrowWideMaxK && tiles_128(M, N, step) < 512;
}

}  // namespace

int gemm_splits(int64_t M, int64_t N, int64_t K, bool step) {
  return narrow_applies(M, N, K, step) ? 1 : splits_128(M, N, K, step);
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool step) {
  const int s = gemm_splits(M, N, K, step);
  return s > 1 ? align_up(size_t(s) * size_t(M) * size_t(N) * 4, kAlign) : 0;
}

namespace {

template <int MODE, int CB>
void launch_small_m_cb(const GemmParams& P, int64_t n_cols, hipStream_t stream) {
  const int64_t blocks = (n_cols + (MODE == kPlain ? CB : CB / 2) - 1) / (MODE == kPlain ? CB : CB / 2);
  const dim3 grid{uint32_t(blocks)}, block{kSmallThreads};
  if (P.M <= 2)
    hipLaunchKernelGGL((small_m_kernel<MODE, 2, CB>), grid, block, 0, stream, P);
  else if (P.M <= 4)
    hipLaunchKernelGGL((small_m_kernel<MODE, 4, CB>), grid, block, 0, stream, P);
  else if (P.M <= 8)
    hipLaunchKernelGGL((small_m_kernel<MODE, 8, CB>), grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL((small_m_kernel<MODE, kSmallM, CB>), grid, block, 0, stream, P);
}

template <int MODE>
hipError_t launch_small_m(const GemmParams& P, hipStream_t stream) {
  // The widest column block that still gives 64 workgroups (16 at least).
  const int64_t n_cols = MODE == kPlain ? P.N : P.D_h;   // columns, or channels in step mode
  const int64_t per64 = MODE == kPlain ? 64 : 32, per32 = per64 / 2;
  if ((n_cols + per64 - 1) / per64 >= 64)
    launch_small_m_cb<MODE, 64>(P, n_cols, stream);
  else if ((n_cols + per32 - 1) / per32 >= 64)
    launch_small_m_cb<MODE, 32>(P, n_cols, stream);
  else
    launch_small_m_cb<MODE, 16>(P, n_cols, stream);
  return hipGetLastError();
}

template <int MODE, int TM>
void launch_narrow_tm(bool full, uint32_t tiles, const GemmParams& P, hipStream_t stream) {
  const dim3 grid{tiles}, block{uint32_t(Narrow<TM, true>::kThreads)};
  if (full)
    hipLaunchKernelGGL((narrow_kernel<MODE, TM, true>), grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL((narrow_kernel<MODE, TM, false>), grid, block, 0, stream, P);
}

// 64-row tiles when they alone give about a workgroup per CU, else 32-row
// tiles (twice as many).
template <int MODE>
sr_status launch_narrow(const GemmParams& P, hipStream_t stream, bool check_only) {
  const int64_t col_tiles = MODE == kPlain ? (P.N + kNarrowCols - 1) / kNarrowCols
                                           : (P.D_h + kNarrowCols / 2 - 1) / (kNarrowCols / 2);
  const int64_t tiles64 = ((P.M + 63) / 64) * col_tiles;
  const int tm = tiles64 >= 192 ? 64 : 32;
  const int64_t tiles = ((P.M + tm - 1) / tm) * col_tiles;
  if (tiles > int64_t(0x7FFFFFFF) / 512)
    return fail(SR_ERR_UNSUPPORTED, "GEMM of %lld narrow tiles too large", (long long)tiles);
  if (check_only) return SR_OK;
  const auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool full = P.K > 0 && P.M % tm == 0 &&
                    (MODE == kPlain ? P.N % kNarrowCols == 0 : P.D_h % (kNarrowCols / 2) == 0) &&
                    P.K % (int64_t(kNarrowSK) * narrow_waves(tm)) == 0 && P.lda % 4 == 0 &&
                    P.ldb % 4 == 0 && al16(P.A) && al16(P.Bm);
  if (tm == 64)
    launch_narrow_tm<MODE, 64>(full, uint32_t(tiles), P, stream);
  else
    launch_narrow_tm<MODE, 32>(full, uint32_t(tiles), P, stream);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SR_ERR_HIP, "narrow GEMM launch: %s", hipGetErrorString(err));
  return SR_OK;
}

template <int MODE, int TBM>
void launch_tiles(bool full, dim3 grid, const GemmParams& P, hipStream_t stream) {
  if (full)
    hipLaunchKernelGGL((gemm_f32_kernel<MODE, TBM, true>), grid, dim3(2 * TBM), 0, stream, P);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<MODE, TBM, false>), grid, dim3(2 * TBM), 0, stream, P);
}

sr_status launch_mode(int mode, GemmParams P, float* ws, hipStream_t stream, bool check_only) {
  if (P.M <= kSmallM) {
    if (P.M > 0 && (mode == kPlain ? P.N : P.D_h) > int64_t(0x7FFFFFFF) * 32)
      return fail(SR_ERR_UNSUPPORTED, "GEMM too wide");
    if (check_only) return SR_OK;
    const hipError_t e = mode == kPlain ? launch_small_m<kPlain>(P, stream)
                                        : launch_small_m<kStep>(P, stream);
    if (e != hipSuccess) return fail(SR_ERR_HIP, "small GEMM launch: %s", hipGetErrorString(e));
    return SR_OK;
  }
  if (narrow_applies(P.M, P.ncols, P.K, mode == kStep))
    return mode == kPlain ? launch_narrow<kPlain>(P, stream, check_only)
                          : launch_narrow<kStep>(P, stream, check_only);
  const int64_t cols_per_tile = mode == kPlain ? BN : BN / 2;
  const int64_t n_cols = mode == kPlain ? P.N : P.D_h;
  P.tiles_n = (n_cols + cols_per_tile - 1) / cols_per_tile;
  // Large plain products (enough 256-row tiles to fill the part twice over)
  // use 256-row tiles and no K split; the rest 128-row tiles, splitting K
  // when there are too few tiles.
  const int64_t tiles_256 = ((P.M + 255) / 256) * P.tiles_n;
  const bool big = mode == kPlain && tiles_256 >= 512;
  const int tbm = big ? 256 : BM;
  const int S = big ? 1 : gemm_splits(P.M, P.ncols, P.K, mode == kStep);
  P.k_split = S > 1 ? ((P.K + S - 1) / S + BK - 1) / BK * BK : (P.K > 0 ? P.K : 1);
  P.partial = S > 1 ? ws : nullptr;
  if (S > 1 && ws == nullptr) return fail(SR_ERR_INVALID_ARGUMENT, "GEMM split-K workspace missing");
  const int64_t tiles = ((P.M + tbm - 1) / tbm) * P.tiles_n;
  if (tiles > 0x7FFFFFFF / (2 * tbm))
    return fail(SR_ERR_UNSUPPORTED, "GEMM of %lld tiles too large", (long long)tiles);
  if (check_only) return SR_OK;
  const dim3 grid{uint32_t(tiles), 1, uint32_t(S)};
  // Every tile full (rows, columns, whole K steps in every slice) and
  // 16-byte operands: the loads need no range tests.
  const auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool full = P.K > 0 && P.M % tbm == 0 && n_cols % cols_per_tile == 0 && P.K % BK == 0 &&
                    P.k_split % BK == 0 && P.K % P.k_split == 0 && P.lda % 4 == 0 &&
                    P.ldb % 4 == 0 && al16(P.A) && al16(P.Bm) && (mode == kPlain || P.D_h % 4 == 0);
  if (mode == kPlain && big)
    launch_tiles<kPlain, 256>(full, grid, P, stream);
  else if (mode == kPlain)
    launch_tiles<kPlain, BM>(full, grid, P, stream);
  else
    launch_tiles<kStep, BM>(full, grid, P, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SR_ERR_HIP, "GEMM launch: %s", hipGetErrorString(err));
  if (S > 1) {
    const int64_t n = P.M * (mode == kPlain ? P.N : P.D_h);
    const int64_t blocks = (n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048;
    if (mode == kPlain)
      hipLaunchKernelGGL(reduce_plain_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream,
                         (const float*)ws, S, P.M, P.N, P.C, P.ldc);
    else
      hipLaunchKernelGGL(reduce_step_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream, P, S);
    err = hipGetLastError();
    if (err != hipSuccess) return fail(SR_ERR_HIP, "split-K reduction launch: %s", hipGetErrorString(err));
  }
  return SR_OK;
}

}  // namespace

sr_status launch_gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                          const float* Bm, int64_t ldb, float* C, int64_t ldc, float* ws,
                          hipStream_t stream, bool check_only) {
  if (M == 0 || N == 0) return SR_OK;
  GemmParams P{};
  P.M = M; P.N = N; P.K = K;
  P.A = A; P.lda = lda; P.Bm = Bm; P.ldb = ldb; P.C = C; P.ldc = ldc;
  P.ncols = N;
  return launch_mode(kPlain, P, ws, stream, check_only);
}

sr_status launch_step_in(int64_t Bsz, int64_t D_in, int64_t D_h, const float* x_t,
                         const float* W_in, const float* h_prev, float* h_next, float* ws,
                         hipStream_t stream, const StepDecay* decay, bool check_only) {
  if (Bsz == 0 || D_h == 0) return SR_OK;
  GemmParams P{};
  P.M = Bsz; P.N = 2 * D_h; P.K = D_in;
  P.A = x_t; P.lda = D_in; P.Bm = W_in; P.ldb = 2 * D_h; P.C = nullptr; P.ldc = 0;
  P.D_h = D_h; P.h_prev = h_prev; P.h_next = h_next;
  if (decay != nullptr) {
    P.rate = decay->rate;
    P.gap = decay->gap;
    P.log1p_gap = decay->log1p_gap;
    P.saturated = decay->saturated;
  }
  P.ncols = 2 * D_h;
  return launch_mode(kStep, P, ws, stream, check_only);
}

}  // namespace sr
