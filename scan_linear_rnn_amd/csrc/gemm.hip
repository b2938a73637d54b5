// fp32 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x2_f32), for the minGRU
// projections [k | p] = x W_in and y = h W_out, and the single-token step whose
// epilogue applies the recurrence.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of C; its four
// waves each own 64 x 64 (2 x 2 MFMA tiles of 32 x 32, 64 accumulators per
// lane).  K advances 16 at a time through double-buffered LDS tiles; global
// loads for step k+1 are in flight while the matrix cores work on step k.
//
// Operand layout of v_mfma_f32_32x32x2_f32 (one 32x32x2 product per wave):
// lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator r of
// lane l is C[8*(r/4) + 4*(l/32) + r%4][l % 32].
//
// Step mode (the single-token step of the minGRU profile's sequential guide):
// the workgroup's 128 B-columns are 64 channels d taken twice -- each wave's
// first 32 columns are k[:, d] and its next 32 are p[:, d] for the same d --
// so one lane holds k and p of the same (row, d) and the epilogue computes
//     z = sigma(k), a = 1 - z = sigma(-k), h_next = a h_prev + z g(p)
// without writing [k | p] anywhere.

#include "internal.hpp"

namespace sr {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int PAD = 4;  // LDS row padding (floats) against bank conflicts

enum Mode { kPlain = 0, kStep = 1 };

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

__device__ __forceinline__ float sigmoid_pos_neg(float k, float& one_minus) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(-fabsf(k) * kLog2e);
  const float big = __builtin_amdgcn_rcpf(1.0f + e);
  const float small = e * big;
  one_minus = k >= 0.0f ? small : big;
  return k >= 0.0f ? big : small;
}

__device__ __forceinline__ float g_act(float p) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float ep = __builtin_amdgcn_exp2f(fminf(p, 0.0f) * kLog2e);
  return p >= 0.0f ? p + 0.5f : ep * __builtin_amdgcn_rcpf(1.0f + ep);
}

// h_next = (1 - z) h_prev + z g(p) with z = sigma(k), for one (row, channel).
// With time decay the carried state is first scaled by
// exp(-min(rate_d * gap_row, 1e4)) (the token boundary comes before the
// token's write; exp(-1e4) is zero in float32, so the clamp changes no value
// and only marks saturation).
__device__ __forceinline__ void step_update(const GemmParams& P, int64_t row, int64_t d, float k,
                                            float p) {
  float a;
  const float z = sigmoid_pos_neg(k, a);
  float hp = P.h_prev ? P.h_prev[row * P.D_h + d] : 0.0f;
  if (P.rate != nullptr) {
    constexpr float kClamp = 1.0e4f, kLog2e = 1.4426950408889634f;
    const float gap = P.log1p_gap ? log1pf(P.gap[row]) : P.gap[row];
    const float e = P.rate[d] * gap;
    if (e > kClamp && P.saturated != nullptr)
      __hip_atomic_fetch_or(P.saturated, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    hp *= __builtin_amdgcn_exp2f(fminf(e, kClamp) * -kLog2e);
  }
  P.h_next[row * P.D_h + d] = fmaf(a, hp, z * g_act(p));
}

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmParams P) {
  __shared__ float As[2][BK][BM + PAD];
  __shared__ float Bs[2][BK][BN + PAD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = int64_t(blockIdx.x) * BM;
  const int64_t n0 = int64_t(blockIdx.y) * (MODE == kPlain ? BN : BN / 2);

  // Global -> register staging: A tile 128 x 16 (8 floats per thread, one row),
  // B tile 16 x 128 (8 floats per thread, one k row).
  const int a_row = tid >> 1, a_k = (tid & 1) * 8;
  const int b_k = tid >> 4, b_c = (tid & 15) * 8;
  const bool a_vec = (P.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(P.A) & 15) == 0);
  const bool b_vec = (P.ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(P.Bm) & 15) == 0) &&
                     (MODE == kPlain || P.D_h % 4 == 0);
  float ra[8], rb[8];
  const int64_t k_begin = int64_t(blockIdx.z) * P.k_split;
  const int64_t k_end = (k_begin + P.k_split < P.K) ? k_begin + P.k_split : P.K;

  auto load_tiles = [&](int64_t k0) {
    const int64_t gm = m0 + a_row;
    const int64_t gk = k0 + a_k;
    if (gm < P.M && a_vec && gk + 8 <= k_end) {
      const float4* src = reinterpret_cast<const float4*>(P.A + gm * P.lda + gk);
      const float4 u = src[0], v = src[1];
      ra[0] = u.x; ra[1] = u.y; ra[2] = u.z; ra[3] = u.w;
      ra[4] = v.x; ra[5] = v.y; ra[6] = v.z; ra[7] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        ra[j] = (gm < P.M && gk + j < k_end) ? P.A[gm * P.lda + gk + j] : 0.0f;
    }
    const int64_t bk = k0 + b_k;
    const int64_t gc = b_col<MODE>(P, n0, b_c);
    if (bk < k_end && b_vec && b_col_ok<MODE>(P, n0, b_c + 7)) {
      const float4* src = reinterpret_cast<const float4*>(P.Bm + bk * P.ldb + gc);
      const float4 u = src[0], v = src[1];
      rb[0] = u.x; rb[1] = u.y; rb[2] = u.z; rb[3] = u.w;
      rb[4] = v.x; rb[5] = v.y; rb[6] = v.z; rb[7] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        rb[j] = (bk < k_end && b_col_ok<MODE>(P, n0, b_c + j))
                    ? P.Bm[bk * P.ldb + b_col<MODE>(P, n0, b_c + j)]
                    : 0.0f;
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) As[buf][a_k + j][a_row] = ra[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) Bs[buf][b_k][b_c + j] = rb[j];
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t n_k = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;
  load_tiles(k_begin);
  store_tiles(0);
  __syncthreads();
  const int kl = lane >> 5, ml = lane & 31;
  for (int64_t kt = 0; kt < n_k; ++kt) {
    const int buf = int(kt & 1);
    if (kt + 1 < n_k) load_tiles(k_begin + (kt + 1) * BK);
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
    if (kt + 1 < n_k) {
      store_tiles(buf ^ 1);
    }
    __syncthreads();
  }

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

int gemm_splits(int64_t M, int64_t N, int64_t K, bool step) {
  // Enough workgroups for two per CU on a 256-CU part, each K slice at
  // least 256 deep; small problems (the single-token step) split K, large
  // ones (whole-sequence projections) do not.
  const int64_t tiles = ((M + BM - 1) / BM) * (step ? (N / 2 + BN / 2 - 1) / (BN / 2)
                                                    : (N + BN - 1) / BN);
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

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool step) {
  const int s = gemm_splits(M, N, K, step);
  return s > 1 ? align_up(size_t(s) * size_t(M) * size_t(N) * 4, kAlign) : 0;
}

namespace {

sr_status launch_mode(int mode, GemmParams P, int64_t tiles_m, int64_t tiles_n, float* ws,
                      hipStream_t stream) {
  const int S = gemm_splits(P.M, P.ncols, P.K, mode == kStep);
  P.k_split = S > 1 ? ((P.K + S - 1) / S + BK - 1) / BK * BK : (P.K > 0 ? P.K : 1);
  P.partial = S > 1 ? ws : nullptr;
  if (S > 1 && ws == nullptr) return fail(SR_ERR_INVALID_ARGUMENT, "GEMM split-K workspace missing");
  if (tiles_m > 0x7FFFFFFF || tiles_n > 65535)
    return fail(SR_ERR_UNSUPPORTED, "GEMM grid %lld x %lld too large", (long long)tiles_m,
                (long long)tiles_n);
  const dim3 grid{uint32_t(tiles_m), uint32_t(tiles_n), uint32_t(S)};
  if (mode == kPlain)
    hipLaunchKernelGGL(gemm_f32_kernel<kPlain>, grid, dim3(256), 0, stream, P);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<kStep>, grid, dim3(256), 0, stream, P);
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
                          hipStream_t stream) {
  if (M == 0 || N == 0) return SR_OK;
  GemmParams P{};
  P.M = M; P.N = N; P.K = K;
  P.A = A; P.lda = lda; P.Bm = Bm; P.ldb = ldb; P.C = C; P.ldc = ldc;
  P.ncols = N;
  return launch_mode(kPlain, P, (M + BM - 1) / BM, (N + BN - 1) / BN, ws, stream);
}

sr_status launch_step_in(int64_t Bsz, int64_t D_in, int64_t D_h, const float* x_t,
                         const float* W_in, const float* h_prev, float* h_next, float* ws,
                         hipStream_t stream, const StepDecay* decay) {
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
  return launch_mode(kStep, P, (Bsz + BM - 1) / BM, (D_h + BN / 2 - 1) / (BN / 2), ws, stream);
}

}  // namespace sr
