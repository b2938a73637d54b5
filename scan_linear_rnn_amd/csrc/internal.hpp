// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "scanrnn.h"

namespace sr {

// Records a printf-style message as the calling thread's last error and
// returns `code`.
sr_status fail(sr_status code, const char* fmt, ...);

// Empties the calling thread's last-error text (each entry point starts so).
void clear_last_error();

// Polls of an unwritten look-back word after which a scan gives up (marks
// the workspace, publishes NaN): process-wide, SCANRNN_LOOKBACK_SPIN_LIMIT
// unless scanrnn_set_lookback_spin_limit lowered it.
uint32_t lookback_spin_limit();

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr size_t kAlign = 256;

// ---------------------------------------------------------------- scan engine
//
// The workspace of one scan: a 256-byte header (ticket counter, status word)
// followed by one 64-bit state word per (chunk along T, batch row, channel).

struct ScanGeometry {
  int V;             // channels per lane
  int N;             // time steps per lane
  int W;             // waves per workgroup (stacked along T)
  int64_t Dc;        // channels per workgroup = 64 * V
  int64_t Tc;        // time steps per workgroup = W * N
  int64_t n_dtiles;  // ceil(D / Dc)
  int64_t n_tchunks; // ceil(T / Tc)
};

// Largest workspace any geometry needs for a [B,T,D] scan.
size_t scan_workspace_bytes(int64_t B, int64_t T, int64_t D);

enum class ScanOp { kMinGRU, kMinMax };

struct ScanRequest {
  ScanOp op;
  sr_dtype in_dtype;   // k,p (minGRU) or r,s (MinMax, fp32 only)
  int64_t B, T, D;
  const void* in0;     // k or r
  const void* in1;     // p or s
  int64_t ld_in;       // row stride of in0/in1, elements
  const float* init;   // h0 / x0 [B,D] or nullptr (zero state)
  float* out;          // [B,T,D] contiguous
  float* last;         // [B,D] or nullptr
  void* workspace;
  hipStream_t stream;
  // Time decay of the carried state (minGRU only; none when decay_rate is null).
  const float* decay_rate = nullptr;  // [D]
  const float* delta_t = nullptr;     // [B,T], contiguous
  int log1p_delta = 0;
  uint32_t* saturated = nullptr;      // device flag, OR-ed with 1 on saturation
  // Run every check the launch makes, then return without enqueuing
  // anything (so that a call of several launches can check them all first).
  bool check_only = false;
};

sr_status launch_scan(const ScanRequest& rq);

// Chooses the geometry a request will use (exposed for sizing and tests).
ScanGeometry choose_geometry(const ScanRequest& rq);

// Fused input projection + scan (fused.hip): h = scan(x W_in), the [k|p]
// tile never leaving the workgroup.  Used for large enough problems (see
// fused_forward_applies); its workspace is the look-back words of its own
// 256-step tiles.
struct FusedRequest {
  int64_t B, T, D_in, D_h;
  const float* x;      // [B,T,D_in]
  const float* W_in;   // [D_in, 2*D_h]
  const float* h0;     // [B,D_h] or nullptr
  float* h;            // [B,T,D_h]
  float* h_last;       // [B,D_h] or nullptr
  void* workspace;
  hipStream_t stream;
  const float* decay_rate = nullptr;  // time decay, as in ScanRequest
  const float* delta_t = nullptr;
  int log1p_delta = 0;
  uint32_t* saturated = nullptr;
  bool check_only = false;  // as in ScanRequest
};

bool fused_forward_applies(int64_t B, int64_t T, int64_t D_h);
size_t fused_workspace_bytes(int64_t B, int64_t T, int64_t D_h);
sr_status launch_fused_forward(const FusedRequest& rq);

// Backward pass of a scan (reverse time, same engine).
struct BackwardRequest {
  ScanOp op;
  sr_dtype in_dtype;    // k,p (minGRU); r,s are fp32
  int64_t B, T, D;
  const void* in0;      // k or r
  const void* in1;      // p or s
  int64_t ld_in;
  const float* fwd;     // forward outputs [B,T,D] (h_t or x_{t+1})
  const float* fwd0;    // forward initial state [B,D] (null = zero; required for MinMax)
  const float* grad;    // upstream gradient [B,T,D]
  const float* grad_last;  // gradient on the returned final state [B,D] or null
  float* d0;            // dk or dr [B,T,D]
  float* d1;            // dp or ds [B,T,D]
  float* dinit;         // dh0 or dx0 [B,D] or null
  // Time decay of the carried state (minGRU only; none when decay_rate is null).
  const float* decay_rate;  // [D]
  const float* delta_t;     // [B,T]
  int log1p_delta;
  void* workspace;
  hipStream_t stream;
};

sr_status launch_scan_backward(const BackwardRequest& rq);
size_t scan_backward_workspace_bytes(int64_t B, int64_t T, int64_t D);

// ---------------------------------------------------------------- GEMM
//
// C[M,N] = A[M,K] * B[K,N], fp32, row-major with leading dimensions.  Small
// problems split K across workgroups; `ws` must then hold
// gemm_workspace_bytes(M, N, K, false) bytes (it may be null when that is 0).
// With check_only, every check is made and nothing is enqueued.
sr_status launch_gemm_f32(int64_t M, int64_t N, int64_t K,
                          const float* A, int64_t lda,
                          const float* Bm, int64_t ldb,
                          float* C, int64_t ldc, float* ws, hipStream_t stream,
                          bool check_only = false);

// Time decay of the carried state in the step (see mingru_step_decayed).
struct StepDecay {
  const float* rate;     // [D_h]
  const float* gap;      // [Bsz]
  int log1p_gap;
  uint32_t* saturated;   // or null
};

// Step kernel: h_next = (1 - z) gamma h_prev + z g(p) with [k|p] = x_t W_in
// (gamma = 1 without decay), computed as one GEMM whose epilogue applies the
// update.  `ws`: as above with gemm_workspace_bytes(Bsz, 2*D_h, D_in, true).
sr_status launch_step_in(int64_t Bsz, int64_t D_in, int64_t D_h,
                         const float* x_t, const float* W_in,
                         const float* h_prev, float* h_next, float* ws, hipStream_t stream,
                         const StepDecay* decay = nullptr, bool check_only = false);

// Number of K slices a GEMM of this shape uses, and the workspace they need.
int gemm_splits(int64_t M, int64_t N, int64_t K, bool step);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool step);

// One MinMax step over n channels (x_next may alias x_prev).
sr_status launch_minmax_step(const float* r, const float* s, const float* x_prev, float* x_next,
                             int64_t n, hipStream_t stream);

// Copies n floats (src may be null: writes zeros).
sr_status launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream);

}  // namespace sr
