// C ABI entry points: argument validation, workspace carving, launches.
//
// Every check runs before anything is enqueued, so a non-OK status means
// nothing was launched and no output was touched.  No HIP call is made on a
// validation failure, which also lets the checks run on a machine without a
// GPU.

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.hpp"

namespace sr {

namespace {
thread_local char g_last_error[512] = "";
std::atomic<uint32_t> g_spin_limit{SCANRNN_LOOKBACK_SPIN_LIMIT};

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// n = a * b * c without overflow, all non-negative.
bool prod3(int64_t a, int64_t b, int64_t c, int64_t* n) {
  int64_t ab;
  return mul_ok(a, b, &ab) && mul_ok(ab, c, n);
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

struct FwdLayout {
  size_t scan_bytes, kp_off, kp_bytes, h_off, h_bytes, g_off, g_bytes, total;
};

// Workspace of a forward call: the scan's look-back words, the staged [k|p]
// (unless the projection is fused into the scan) and h when the projections
// run, and split-K partial sums of the GEMMs.
FwdLayout forward_layout(int64_t B, int64_t T, int64_t D_in, int64_t D_h, int64_t D_out,
                         bool w_in, bool w_out) {
  FwdLayout L{};
  const bool fused = w_in && fused_forward_applies(B, T, D_h);
  L.scan_bytes = align_up(fused ? fused_workspace_bytes(B, T, D_h) : scan_workspace_bytes(B, T, D_h),
                          kAlign);
  L.kp_off = L.scan_bytes;
  L.kp_bytes = w_in && !fused ? align_up(size_t(B) * size_t(T) * size_t(2 * D_h) * 4, kAlign) : 0;
  L.h_off = L.kp_off + L.kp_bytes;
  L.h_bytes = w_out ? align_up(size_t(B) * size_t(T) * size_t(D_h) * 4, kAlign) : 0;
  L.g_off = L.h_off + L.h_bytes;
  const size_t g_in = w_in && !fused ? gemm_workspace_bytes(B * T, 2 * D_h, D_in, false) : 0;
  const size_t g_out = w_out ? gemm_workspace_bytes(B * T, D_out, D_h, false) : 0;
  L.g_bytes = g_in > g_out ? g_in : g_out;
  L.total = L.g_off + L.g_bytes;
  return L;
}

size_t step_workspace(int64_t B, int64_t D_in, int64_t D_h, int64_t D_out) {
  const size_t a = gemm_workspace_bytes(B, 2 * D_h, D_in, true);
  const size_t b = gemm_workspace_bytes(B, D_out, D_h, false);
  return a > b ? a : b;
}

sr_status check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return SR_OK;
  if (ws == nullptr) return fail(SR_ERR_INVALID_ARGUMENT, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, kAlign)) return fail(SR_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (have < need)
    return fail(SR_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", have, need);
  return SR_OK;
}

#define SR_REQUIRE(cond, ...)                                   \
  do {                                                          \
    if (!(cond)) return fail(SR_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
  } while (0)

// Time decay of the carried state: the rate per channel, the gap per token.
struct Decay {
  const float* rate;
  const float* delta_t;
  int log1p_delta;
  uint32_t* saturated;
};

// n_rate channels need a rate and n_gap tokens a gap.
sr_status check_decay(const Decay& d, int64_t n_rate, int64_t n_gap) {
  SR_REQUIRE(n_rate == 0 || d.rate != nullptr, "decay_rate is NULL");
  SR_REQUIRE(n_gap == 0 || d.delta_t != nullptr, "delta_t is NULL");
  SR_REQUIRE(d.log1p_delta == 0 || d.log1p_delta == 1, "log1p_delta must be 0 or 1 (got %d)",
             d.log1p_delta);
  SR_REQUIRE(aligned(d.rate, 4) && aligned(d.delta_t, 4) && aligned(d.saturated, 4),
             "decay pointers must be 4-byte aligned");
  return SR_OK;
}

sr_status forward_impl(int64_t B, int64_t T, int64_t D_in, int64_t D_h, int64_t D_out,
                       const float* x, const float* W_in, const void* k, const void* p,
                       int64_t ld_kp, sr_dtype kp_dtype, const float* h0, const float* W_out,
                       float* y, float* h_last, void* workspace, size_t workspace_bytes,
                       void* stream, const Decay* dec) {
  SR_REQUIRE(B >= 0 && T >= 0 && D_in >= 0 && D_h >= 0 && D_out >= 0,
             "sizes must be non-negative (B=%lld T=%lld D_in=%lld D_h=%lld D_out=%lld)",
             (long long)B, (long long)T, (long long)D_in, (long long)D_h, (long long)D_out);
  int64_t n_kp, n_x, n_y, n_h;
  SR_REQUIRE(prod3(B, T, 2 * D_h, &n_kp) && prod3(B, T, D_in, &n_x) && prod3(B, T, D_out, &n_y) &&
                 prod3(B, T, D_h, &n_h),
             "tensor sizes overflow int64");
  const bool w_in = W_in != nullptr, w_out = W_out != nullptr;
  if (!w_out)
    SR_REQUIRE(D_out == D_h, "without W_out the output width D_out (%lld) must equal D_h (%lld)",
               (long long)D_out, (long long)D_h);
  SR_REQUIRE(n_y == 0 || y != nullptr, "y is NULL");
  SR_REQUIRE(aligned(y, 4) && aligned(h0, 4) && aligned(h_last, 4) && aligned(W_out, 4) &&
                 aligned(W_in, 4) && aligned(x, 4),
             "fp32 pointers must be 4-byte aligned");
  if (w_in) {
    SR_REQUIRE(k == nullptr && p == nullptr, "with W_in the projected k and p must be NULL");
    SR_REQUIRE(n_x == 0 || x != nullptr, "x is NULL while W_in is given");
  } else {
    SR_REQUIRE(x == nullptr, "x must be NULL when W_in is NULL (pass k and p instead)");
    SR_REQUIRE(kp_dtype == SR_F32 || kp_dtype == SR_BF16, "kp_dtype %d unsupported", int(kp_dtype));
    SR_REQUIRE(n_h == 0 || (k != nullptr && p != nullptr), "k or p is NULL");
    SR_REQUIRE(ld_kp >= D_h, "ld_kp (%lld) must be >= D_h (%lld)", (long long)ld_kp, (long long)D_h);
    const size_t esz = kp_dtype == SR_BF16 ? 2 : 4;
    SR_REQUIRE(aligned(k, esz) && aligned(p, esz), "k and p must be aligned to their element size");
    int64_t span;
    SR_REQUIRE(prod3(B, T, ld_kp, &span), "k/p extent overflows int64");
  }
  if (dec != nullptr) {
    sr_status st = check_decay(*dec, n_h > 0 ? D_h : 0, n_h > 0 ? B * T : 0);
    if (st != SR_OK) return st;
  }
  const FwdLayout L = forward_layout(B, T, D_in, D_h, D_out, w_in, w_out);
  sr_status st = check_workspace(workspace, workspace_bytes, L.total);
  if (st != SR_OK) return st;

  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  float* kp_buf = w_in ? reinterpret_cast<float*>(ws + L.kp_off) : nullptr;
  float* h_buf = w_out ? reinterpret_cast<float*>(ws + L.h_off) : y;
  float* g_buf = L.g_bytes ? reinterpret_cast<float*>(ws + L.g_off) : nullptr;

  if (B == 0 || D_h == 0) {
    // No channels: y has no elements unless D_out > 0 with W_out (then y = 0).
    if (w_out && n_y > 0) return launch_copy_or_zero(y, nullptr, n_y, s);
    return SR_OK;
  }
  // The launches of the call; run once with check_only (every launch's own
  // checks, nothing enqueued), then for real, so that a failing check never
  // leaves earlier launches behind.
  const bool fused = w_in && T > 0 && fused_forward_applies(B, T, D_h);
  auto run = [&](bool check_only) -> sr_status {
    sr_status st2;
    if (fused) {
      FusedRequest fr{};
      fr.B = B;
      fr.T = T;
      fr.D_in = D_in;
      fr.D_h = D_h;
      fr.x = x;
      fr.W_in = W_in;
      fr.h0 = h0;
      fr.h = h_buf;
      fr.h_last = h_last;
      fr.workspace = ws;
      fr.stream = s;
      if (dec != nullptr) {
        fr.decay_rate = dec->rate;
        fr.delta_t = dec->delta_t;
        fr.log1p_delta = dec->log1p_delta;
        fr.saturated = dec->saturated;
      }
      fr.check_only = check_only;
      st2 = launch_fused_forward(fr);
      if (st2 != SR_OK || !w_out) return st2;
      return launch_gemm_f32(B * T, D_out, D_h, h_buf, D_h, W_out, D_out, y, D_out, g_buf, s,
                             check_only);
    }
    if (w_in && T > 0) {
      st2 = launch_gemm_f32(B * T, 2 * D_h, D_in, x, D_in, W_in, 2 * D_h, kp_buf, 2 * D_h, g_buf, s,
                            check_only);
      if (st2 != SR_OK) return st2;
    }
    ScanRequest rq{};
    rq.op = ScanOp::kMinGRU;
    rq.in_dtype = w_in ? SR_F32 : kp_dtype;
    rq.B = B;
    rq.T = T;
    rq.D = D_h;
    rq.in0 = w_in ? static_cast<const void*>(kp_buf) : k;
    rq.in1 = w_in ? static_cast<const void*>(kp_buf + D_h) : p;
    rq.ld_in = w_in ? 2 * D_h : ld_kp;
    rq.init = h0;
    rq.out = h_buf;
    rq.last = h_last;
    rq.workspace = ws;
    rq.stream = s;
    if (dec != nullptr) {
      rq.decay_rate = dec->rate;
      rq.delta_t = dec->delta_t;
      rq.log1p_delta = dec->log1p_delta;
      rq.saturated = dec->saturated;
    }
    rq.check_only = check_only;
    st2 = launch_scan(rq);
    if (st2 != SR_OK) return st2;
    if (w_out && T > 0)
      st2 = launch_gemm_f32(B * T, D_out, D_h, h_buf, D_h, W_out, D_out, y, D_out, g_buf, s,
                            check_only);
    return st2;
  };
  st = run(true);
  return st != SR_OK ? st : run(false);
}

sr_status step_impl(int64_t B, int64_t D_in, int64_t D_h, int64_t D_out, const float* x_t,
                    const float* W_in, const float* W_out, const float* h_prev, float* h_next,
                    float* y_t, void* workspace, size_t workspace_bytes, void* stream,
                    const Decay* dec) {
  SR_REQUIRE(B >= 0 && D_in >= 0 && D_h >= 0 && D_out >= 0,
             "sizes must be non-negative (B=%lld D_in=%lld D_h=%lld D_out=%lld)", (long long)B,
             (long long)D_in, (long long)D_h, (long long)D_out);
  int64_t n_x, n_h, n_y, n_w;
  SR_REQUIRE(prod3(B, D_in, 1, &n_x) && prod3(B, D_h, 1, &n_h) && prod3(B, D_out, 1, &n_y) &&
                 prod3(D_in, 2 * D_h, 1, &n_w),
             "tensor sizes overflow int64");
  SR_REQUIRE(W_in != nullptr || n_w == 0, "W_in is NULL");
  SR_REQUIRE(x_t != nullptr || n_x == 0, "x_t is NULL");
  SR_REQUIRE(h_next != nullptr || n_h == 0, "h_next is NULL");
  if (W_out == nullptr)
    SR_REQUIRE(D_out == D_h, "without W_out the output width D_out (%lld) must equal D_h (%lld)",
               (long long)D_out, (long long)D_h);
  else
    SR_REQUIRE(y_t != nullptr || n_y == 0, "y_t is NULL while W_out is given");
  SR_REQUIRE(aligned(x_t, 4) && aligned(W_in, 4) && aligned(W_out, 4) && aligned(h_prev, 4) &&
                 aligned(h_next, 4) && aligned(y_t, 4),
             "fp32 pointers must be 4-byte aligned");
  if (dec != nullptr) {
    sr_status st = check_decay(*dec, n_h > 0 ? D_h : 0, n_h > 0 ? B : 0);
    if (st != SR_OK) return st;
  }
  sr_status st = check_workspace(workspace, workspace_bytes, step_workspace(B, D_in, D_h, D_out));
  if (st != SR_OK) return st;
  if (B == 0) return SR_OK;
  hipStream_t s = as_stream(stream);
  float* g_buf = static_cast<float*>(workspace);
  StepDecay sd{};
  if (dec != nullptr) sd = StepDecay{dec->rate, dec->delta_t, dec->log1p_delta, dec->saturated};
  // Checked first, then launched (as in forward_impl).
  auto run = [&](bool check_only) -> sr_status {
    sr_status st2 = launch_step_in(B, D_in, D_h, x_t, W_in, h_prev, h_next, g_buf, s,
                                   dec != nullptr ? &sd : nullptr, check_only);
    if (st2 != SR_OK) return st2;
    if (W_out != nullptr)
      return launch_gemm_f32(B, D_out, D_h, h_next, D_h, W_out, D_out, y_t, D_out, g_buf, s,
                             check_only);
    if (y_t != nullptr && y_t != h_next && !check_only) return launch_copy_or_zero(y_t, h_next, n_h, s);
    return SR_OK;
  };
  st = run(true);
  return st != SR_OK ? st : run(false);
}

}  // namespace

uint32_t lookback_spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

namespace {

sr_status mingru_backward_impl(int64_t B, int64_t T, int64_t D, const void* k, const void* p,
                               int64_t ld_kp, sr_dtype kp_dtype, const float* h0, const float* h,
                               const float* dh, const float* dh_last, float* dk, float* dp,
                               float* dh0, void* workspace, size_t workspace_bytes, void* stream,
                               const Decay* dec) {
  SR_REQUIRE(B >= 0 && T >= 0 && D >= 0, "sizes must be non-negative (B=%lld T=%lld D=%lld)",
             (long long)B, (long long)T, (long long)D);
  int64_t n, span;
  SR_REQUIRE(prod3(B, T, D, &n), "tensor sizes overflow int64");
  SR_REQUIRE(kp_dtype == SR_F32 || kp_dtype == SR_BF16, "kp_dtype %d unsupported", int(kp_dtype));
  SR_REQUIRE(ld_kp >= D, "ld_kp (%lld) must be >= D (%lld)", (long long)ld_kp, (long long)D);
  SR_REQUIRE(prod3(B, T, ld_kp, &span), "k/p extent overflows int64");
  SR_REQUIRE(n == 0 || (k && p && h && dh && dk && dp), "k, p, h, dh, dk and dp are required");
  const size_t esz = kp_dtype == SR_BF16 ? 2 : 4;
  SR_REQUIRE(aligned(k, esz) && aligned(p, esz), "k and p must be aligned to their element size");
  SR_REQUIRE(aligned(h0, 4) && aligned(h, 4) && aligned(dh, 4) && aligned(dh_last, 4) &&
                 aligned(dk, 4) && aligned(dp, 4) && aligned(dh0, 4),
             "fp32 pointers must be 4-byte aligned");
  if (dec != nullptr) {
    sr_status st = check_decay(*dec, n > 0 ? D : 0, n > 0 ? B * T : 0);
    if (st != SR_OK) return st;
  }
  sr_status st = check_workspace(workspace, workspace_bytes,
                                 mingru_scan_backward_workspace_size(B, T, D));
  if (st != SR_OK) return st;
  BackwardRequest rq{};
  rq.op = ScanOp::kMinGRU;
  rq.in_dtype = kp_dtype;
  rq.B = B; rq.T = T; rq.D = D;
  rq.in0 = k; rq.in1 = p; rq.ld_in = ld_kp;
  rq.fwd = h; rq.fwd0 = h0; rq.grad = dh; rq.grad_last = dh_last;
  rq.d0 = dk; rq.d1 = dp; rq.dinit = dh0;
  if (dec != nullptr && n > 0) {
    rq.decay_rate = dec->rate;
    rq.delta_t = dec->delta_t;
    rq.log1p_delta = dec->log1p_delta;
  }
  rq.workspace = workspace;
  rq.stream = as_stream(stream);
  return launch_scan_backward(rq);
}

}  // namespace

void clear_last_error() { g_last_error[0] = '\0'; }

sr_status fail(sr_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace sr

using namespace sr;

extern "C" {

const char* scanrnn_last_error(void) { return g_last_error; }

const char* scanrnn_version(void) { return "0.1.0"; }

size_t mingru_forward_workspace_size(int64_t B, int64_t T, int64_t D_in, int64_t D_h,
                                     int64_t D_out, int has_w_in, int has_w_out) {
  int64_t n;
  if (B < 0 || T < 0 || D_in < 0 || D_h < 0 || D_out < 0 || !prod3(B, T, 2 * D_h, &n)) return 0;
  return forward_layout(B, T, D_in, D_h, D_out, has_w_in != 0, has_w_out != 0).total;
}

sr_status mingru_forward(int64_t B, int64_t T, int64_t D_in, int64_t D_h, int64_t D_out,
                         const float* x, const float* W_in, const void* k, const void* p,
                         int64_t ld_kp, sr_dtype kp_dtype, const float* h0, const float* W_out,
                         float* y, float* h_last, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_last_error[0] = '\0';
  return forward_impl(B, T, D_in, D_h, D_out, x, W_in, k, p, ld_kp, kp_dtype, h0, W_out, y, h_last,
                      workspace, workspace_bytes, stream, nullptr);
}

sr_status mingru_forward_decayed(int64_t B, int64_t T, int64_t D_in, int64_t D_h, int64_t D_out,
                                 const float* x, const float* W_in, const void* k, const void* p,
                                 int64_t ld_kp, sr_dtype kp_dtype, const float* decay_rate,
                                 const float* delta_t, int log1p_delta, uint32_t* saturated,
                                 const float* h0, const float* W_out, float* y, float* h_last,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  const Decay dec{decay_rate, delta_t, log1p_delta, saturated};
  return forward_impl(B, T, D_in, D_h, D_out, x, W_in, k, p, ld_kp, kp_dtype, h0, W_out, y, h_last,
                      workspace, workspace_bytes, stream, &dec);
}

size_t mingru_step_workspace_size(int64_t B, int64_t D_in, int64_t D_h, int64_t D_out) {
  int64_t n;
  if (B < 0 || D_in < 0 || D_h < 0 || D_out < 0 || !prod3(B, 2 * D_h + D_out, D_in + D_h + 1, &n))
    return 0;
  return step_workspace(B, D_in, D_h, D_out);
}

sr_status mingru_step(int64_t B, int64_t D_in, int64_t D_h, int64_t D_out, const float* x_t,
                      const float* W_in, const float* W_out, const float* h_prev, float* h_next,
                      float* y_t, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  return step_impl(B, D_in, D_h, D_out, x_t, W_in, W_out, h_prev, h_next, y_t, workspace,
                   workspace_bytes, stream, nullptr);
}

sr_status mingru_step_decayed(int64_t B, int64_t D_in, int64_t D_h, int64_t D_out,
                              const float* x_t, const float* W_in, const float* W_out,
                              const float* decay_rate, const float* delta_t, int log1p_delta,
                              uint32_t* saturated, const float* h_prev, float* h_next, float* y_t,
                              void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  const Decay dec{decay_rate, delta_t, log1p_delta, saturated};
  return step_impl(B, D_in, D_h, D_out, x_t, W_in, W_out, h_prev, h_next, y_t, workspace,
                   workspace_bytes, stream, &dec);
}

size_t minmax_scan_workspace_size(int64_t B, int64_t T, int64_t D) {
  int64_t n;
  if (B < 0 || T < 0 || D < 0 || !prod3(B, T, D, &n)) return 0;
  return align_up(scan_workspace_bytes(B, T, D), kAlign);
}

sr_status minmax_scan(int64_t B, int64_t T, int64_t D, const float* r, const float* s,
                      const float* x0, float* x_out, float* x_last, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  SR_REQUIRE(B >= 0 && T >= 0 && D >= 0, "sizes must be non-negative (B=%lld T=%lld D=%lld)",
             (long long)B, (long long)T, (long long)D);
  int64_t n, nbd;
  SR_REQUIRE(prod3(B, T, D, &n) && prod3(B, D, 1, &nbd), "tensor sizes overflow int64");
  SR_REQUIRE(n == 0 || (r != nullptr && s != nullptr && x_out != nullptr), "r, s or x_out is NULL");
  SR_REQUIRE(nbd == 0 || x0 != nullptr, "x0 is required");
  SR_REQUIRE(aligned(r, 4) && aligned(s, 4) && aligned(x0, 4) && aligned(x_out, 4) &&
                 aligned(x_last, 4),
             "fp32 pointers must be 4-byte aligned");
  sr_status st = check_workspace(workspace, workspace_bytes, minmax_scan_workspace_size(B, T, D));
  if (st != SR_OK) return st;
  ScanRequest rq{};
  rq.op = ScanOp::kMinMax;
  rq.in_dtype = SR_F32;
  rq.B = B;
  rq.T = T;
  rq.D = D;
  rq.in0 = r;
  rq.in1 = s;
  rq.ld_in = D;
  rq.init = x0;
  rq.out = x_out;
  rq.last = x_last;
  rq.workspace = workspace;
  rq.stream = as_stream(stream);
  return launch_scan(rq);
}

sr_status minmax_step(int64_t B, int64_t D, const float* r_t, const float* s_t,
                      const float* x_prev, float* x_next, void* stream) {
  g_last_error[0] = '\0';
  SR_REQUIRE(B >= 0 && D >= 0, "sizes must be non-negative (B=%lld D=%lld)", (long long)B,
             (long long)D);
  int64_t n;
  SR_REQUIRE(prod3(B, D, 1, &n), "tensor sizes overflow int64");
  SR_REQUIRE(n == 0 || (r_t && s_t && x_prev && x_next), "r_t, s_t, x_prev and x_next are required");
  SR_REQUIRE(aligned(r_t, 4) && aligned(s_t, 4) && aligned(x_prev, 4) && aligned(x_next, 4),
             "fp32 pointers must be 4-byte aligned");
  return launch_minmax_step(r_t, s_t, x_prev, x_next, n, as_stream(stream));
}

size_t mingru_scan_backward_workspace_size(int64_t B, int64_t T, int64_t D) {
  int64_t n;
  if (B < 0 || T < 0 || D < 0 || !prod3(B, T, D, &n)) return 0;
  return align_up(scan_backward_workspace_bytes(B, T, D), kAlign);
}

size_t minmax_scan_backward_workspace_size(int64_t B, int64_t T, int64_t D) {
  return mingru_scan_backward_workspace_size(B, T, D);
}

sr_status mingru_scan_backward(int64_t B, int64_t T, int64_t D, const void* k, const void* p,
                               int64_t ld_kp, sr_dtype kp_dtype, const float* h0, const float* h,
                               const float* dh, const float* dh_last, float* dk, float* dp,
                               float* dh0, void* workspace, size_t workspace_bytes,
                               void* stream) {
  g_last_error[0] = '\0';
  return mingru_backward_impl(B, T, D, k, p, ld_kp, kp_dtype, h0, h, dh, dh_last, dk, dp, dh0,
                              workspace, workspace_bytes, stream, nullptr);
}

sr_status mingru_scan_backward_decayed(int64_t B, int64_t T, int64_t D, const void* k,
                                       const void* p, int64_t ld_kp, sr_dtype kp_dtype,
                                       const float* decay_rate, const float* delta_t,
                                       int log1p_delta, const float* h0, const float* h,
                                       const float* dh, const float* dh_last, float* dk, float* dp,
                                       float* dh0, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  g_last_error[0] = '\0';
  const Decay dec{decay_rate, delta_t, log1p_delta, nullptr};
  return mingru_backward_impl(B, T, D, k, p, ld_kp, kp_dtype, h0, h, dh, dh_last, dk, dp, dh0,
                              workspace, workspace_bytes, stream, &dec);
}

sr_status minmax_scan_backward(int64_t B, int64_t T, int64_t D, const float* r, const float* s,
                               const float* x0, const float* x_out, const float* dx,
                               const float* dx_last, float* dr, float* ds, float* dx0,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  SR_REQUIRE(B >= 0 && T >= 0 && D >= 0, "sizes must be non-negative (B=%lld T=%lld D=%lld)",
             (long long)B, (long long)T, (long long)D);
  int64_t n, nbd;
  SR_REQUIRE(prod3(B, T, D, &n) && prod3(B, D, 1, &nbd), "tensor sizes overflow int64");
  SR_REQUIRE(n == 0 || (r && s && x_out && dx && dr && ds), "r, s, x_out, dx, dr and ds are required");
  SR_REQUIRE(nbd == 0 || x0 != nullptr, "x0 is required");
  SR_REQUIRE(aligned(r, 4) && aligned(s, 4) && aligned(x0, 4) && aligned(x_out, 4) &&
                 aligned(dx, 4) && aligned(dx_last, 4) && aligned(dr, 4) && aligned(ds, 4) &&
                 aligned(dx0, 4),
             "fp32 pointers must be 4-byte aligned");
  sr_status st = check_workspace(workspace, workspace_bytes,
                                 minmax_scan_backward_workspace_size(B, T, D));
  if (st != SR_OK) return st;
  BackwardRequest rq{};
  rq.op = ScanOp::kMinMax;
  rq.in_dtype = SR_F32;
  rq.B = B; rq.T = T; rq.D = D;
  rq.in0 = r; rq.in1 = s; rq.ld_in = D;
  rq.fwd = x_out; rq.fwd0 = x0; rq.grad = dx; rq.grad_last = dx_last;
  rq.d0 = dr; rq.d1 = ds; rq.dinit = dx0;
  rq.workspace = workspace;
  rq.stream = as_stream(stream);
  return launch_scan_backward(rq);
}

sr_status scanrnn_set_lookback_spin_limit(uint32_t polls) {
  g_last_error[0] = '\0';
  SR_REQUIRE(polls <= SCANRNN_LOOKBACK_SPIN_LIMIT, "spin limit %u above the default %u", polls,
             (unsigned)SCANRNN_LOOKBACK_SPIN_LIMIT);
  g_spin_limit.store(polls, std::memory_order_relaxed);
  return SR_OK;
}

sr_status scanrnn_workspace_status(const void* workspace, void* stream) {
  g_last_error[0] = '\0';
  SR_REQUIRE(workspace != nullptr, "workspace is NULL");
  uint32_t flag = 0;
  hipStream_t s = as_stream(stream);
  hipError_t err = hipMemcpyAsync(&flag, static_cast<const char*>(workspace) + 4, 4,
                                  hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return fail(SR_ERR_HIP, "reading workspace status: %s", hipGetErrorString(err));
  if (flag & 1u) return fail(SR_ERR_LOOKBACK_TIMEOUT, "a scan gave up waiting for a predecessor tile");
  if (flag & 2u)
    return fail(SR_ERR_GATE_RANGE, "a gate logit beyond the fp32 range of sigma (|k| > ~87.3) was met");
  return SR_OK;
}

}  // extern "C"
