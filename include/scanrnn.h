/*
 * scanrnn.h -- C ABI of the MI355X (gfx950) minGRU / MinMax scan library.
 *
 * What the calls compute
 * ----------------------
 * minGRU layer (the log-space minGRU layer profiled on openvist.com as
 * "Mingru Pytorch"; intro and "Requirements & limits": a log-space numerically
 * stable layer with a parallel mode and a token-by-token mode that carries the
 * hidden state):
 *
 *     [k_t | p_t] = x_t W_in                 (k: first D_h columns, p: next D_h)
 *     z_t = sigma(k_t),   htilde_t = g(p_t),  g(v) = v + 1/2 (v >= 0), sigma(v) (v < 0)
 *     h_t = (1 - z_t) h_{t-1} + z_t htilde_t       t = 1..T, h_0 carried (absent = 0)
 *     y_t = h_t W_out                        (absent W_out: y_t = h_t)
 *
 * evaluated as an associative scan over t of the affine maps
 * h -> a_t h + b_t.  The log-space coefficients log a_t = log(1 - z_t) =
 * -softplus(k_t) and log b_t = log z_t + log g(p_t) are exponentiated in
 * closed form (a_t = sigma(-k_t), b_t = sigma(k_t) g(p_t), no cancelling
 * 1 - x), and composed maps carry their coefficient A together with its
 * complement 1 - A, so that a long memory (A near 1) keeps 1 - A to a few
 * ulps -- what the log-space form's -softplus(k) keeps -- while the state
 * itself stays linear (a signed h_0 needs no logarithm).  The single-token
 * step evaluates h_{t-1} + z_t (g(p_t) - h_{t-1}).
 *
 * Range.  For |k| above about 87.3 the smaller of sigma(k) and sigma(-k) is
 * below the smallest normal fp32 number and flushes to zero, and the term it
 * multiplies (the candidate's share for very negative k, the carried state
 * for very positive k) is dropped; every other term keeps full accuracy.
 * The scans report such gate logits through scanrnn_workspace_status
 * (SR_ERR_GATE_RANGE); the results are still written.
 *
 * MinMax neuron (minmaxrnc PyPI page, "The model" item 3):
 *
 *     x_{t+1} = max(min(r_t, x_t), s_t)   element-wise, by a prefix scan.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers; the caller owns every buffer,
 *   including the workspace.  The library keeps no pointer after a call
 *   returns and holds no global mutable state except a thread-local error
 *   string, the look-back poll bound (scanrnn_set_lookback_spin_limit) and
 *   the device array of mingru_scan_noalloc (with the caller-owned-buffer
 *   rule its one exception).
 * - Tensors are row-major, innermost (feature) dimension fastest; a [B,T,D]
 *   tensor is B*T rows of D elements.  Pointers must be aligned to their
 *   element size; wider alignment (8 or 16 bytes) lets the library use
 *   vector loads.
 * - Sizes are int64.  B*T*D may exceed 2^31; offsets are computed in 64 bits.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream).  Buffers must stay alive until the enqueued work completes.
 * - Arguments are validated before anything is enqueued: on any non-OK status
 *   nothing was launched and no output was written.  A failed HIP launch
 *   returns SR_ERR_HIP.  scanrnn_last_error() gives the text of the last
 *   non-OK status on the calling thread.  No C++ exception crosses the ABI.
 * - Calls are reentrant; concurrent calls must use distinct workspaces.
 * - Workspace: at least *_workspace_size(...) bytes, 256-byte aligned,
 *   contents need not be initialised (the call resets what it uses, on the
 *   stream, before the scan).
 * - Determinism: minmax_scan is bit-exact (min and max only select).  The
 *   minGRU calls agree with the sequential definition within rounding; the
 *   order in which partial results are combined does not depend on timing,
 *   so repeated calls give identical bits.
 */
#ifndef SCANRNN_H
#define SCANRNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SR_OK = 0,
  SR_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad stride     */
  SR_ERR_UNSUPPORTED = 2,        /* valid request the library does not handle   */
  SR_ERR_WORKSPACE_TOO_SMALL = 3,
  SR_ERR_HIP = 4,                /* a HIP runtime call failed                   */
  SR_ERR_LOOKBACK_TIMEOUT = 5,   /* reported by scanrnn_workspace_status only   */
  SR_ERR_GATE_RANGE = 6          /* reported by scanrnn_workspace_status only   */
} sr_status;

/* Element type of k and p: one of these values, passed as a 32-bit integer
 * so that whatever a caller sends is a valid value of the type; any other
 * value is rejected with SR_ERR_INVALID_ARGUMENT. */
enum { SR_F32 = 0, SR_BF16 = 1 };
typedef int32_t sr_dtype;

/* Bytes of workspace mingru_forward needs.  has_w_in / has_w_out say whether
 * the call will pass W_in / W_out.  W_out needs B*T*D_h floats to stage h.
 * With W_in, large problems (at least 512 tiles of 256 steps x 64 channels)
 * compute the projection inside the scan and need no more; smaller ones
 * stage [k|p] (B*T*2*D_h floats) and split-K partial sums. */
size_t mingru_forward_workspace_size(int64_t B, int64_t T, int64_t D_in, int64_t D_h,
                                     int64_t D_out, int has_w_in, int has_w_out);

/*
 * Parallel mode: the whole sequence at once (minGRU profile, guide "Install
 * and apply the minGRU layer": the output has the input's shape).
 *
 *   x      [B,T,D_in] fp32; read only when W_in != NULL.
 *   W_in   [D_in, 2*D_h] fp32, or NULL: then k and p are given directly
 *          (scan-only use) and x must be NULL.
 *   k, p   rows of the pre-projected gate logits / candidate pre-activations,
 *          element (b,t,d) at k[(b*T + t)*ld_kp + d]; dtype kp_dtype
 *          (SR_F32 or SR_BF16).  ld_kp >= D_h, so k and p may be the two
 *          halves of one [B,T,2*D_h] buffer.  Used only when W_in == NULL.
 *   h0     [B,D_h] fp32 carried state, or NULL (zero state).
 *   W_out  [D_h, D_out] fp32, or NULL (then D_out must equal D_h, y = h).
 *   y      [B,T,D_out] fp32 output.
 *   h_last [B,D_h] fp32, or NULL: receives h_T (h0, or zeros, when T == 0).
 */
sr_status mingru_forward(int64_t B, int64_t T, int64_t D_in, int64_t D_h, int64_t D_out,
                         const float* x, const float* W_in,
                         const void* k, const void* p, int64_t ld_kp, sr_dtype kp_dtype,
                         const float* h0, const float* W_out,
                         float* y, float* h_last,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mingru_step needs: none up to 512 streams, nor up to
 * 4096 streams while D_in and D_h are at most 1024 (the K range is then
 * split inside each workgroup); otherwise split-K partial sums. */
size_t mingru_step_workspace_size(int64_t B, int64_t D_in, int64_t D_h, int64_t D_out);

/*
 * Sequential mode, one token (minGRU profile, guide "Process a sequence
 * sequentially with carried hidden state"; the minGRU tutorial's Step 3: the
 * base step returns the new hidden state, which is also its output).
 *
 *   x_t    [B,D_in] fp32;  W_in [D_in,2*D_h] fp32 (required).
 *   W_out  [D_h,D_out] fp32 or NULL (then D_out must equal D_h).
 *   h_prev [B,D_h] fp32 or NULL (zero state).
 *   h_next [B,D_h] fp32; may be the same buffer as h_prev.
 *   y_t    [B,D_out] fp32, or NULL when W_out is NULL (the output is h_next;
 *          a non-NULL y_t then receives a copy).
 */
sr_status mingru_step(int64_t B, int64_t D_in, int64_t D_h, int64_t D_out,
                      const float* x_t, const float* W_in, const float* W_out,
                      const float* h_prev, float* h_next, float* y_t,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Time decay of the carried state (the decay contract of the minGRU tutorial
 * "Your first delta model", Step 5 "Adding time decay": each event comes with
 * the gap delta_t preceding it; the carried state is scaled by gamma once per
 * token, at the token boundary, before that token's own write; a zero gap is
 * gamma = exp(0) = 1; a rate * gap above about 1e4 saturates float32 and
 * wipes the memory, through a clamp, and is reported; log1p_delta compresses
 * the gaps).  On the minGRU's vector state:
 *
 *     gap_t  = log1p(delta_t) if log1p_delta else delta_t
 *     gamma  = exp(-min(decay_rate_d * gap_t, 1e4))
 *     h_t    = (1 - z_t) (gamma_t h_{t-1}) + z_t g(p_t)
 *
 *   decay_rate  [D_h] fp32 per-channel rate, >= 0 and finite.
 *   delta_t     [B,T] fp32 (sequence call) or [B] (step), contiguous, >= 0
 *               and finite.  Other values are outside the contract.
 *   log1p_delta 0 or 1.
 *   saturated   device uint32 or NULL: set to 1 (atomic OR, never cleared by
 *               the library) when some decay_rate_d * gap_t, rounded to fp32,
 *               exceeds 1e4.  exp(-1e4) is 0 in fp32, so the clamp changes no
 *               value; the flag says large gaps were not distinguished.
 *
 * Everything else is as in mingru_forward / mingru_step, with the same
 * workspace sizes (mingru_forward_workspace_size, mingru_step_workspace_size).
 */
sr_status mingru_forward_decayed(int64_t B, int64_t T, int64_t D_in, int64_t D_h, int64_t D_out,
                                 const float* x, const float* W_in,
                                 const void* k, const void* p, int64_t ld_kp, sr_dtype kp_dtype,
                                 const float* decay_rate, const float* delta_t, int log1p_delta,
                                 uint32_t* saturated,
                                 const float* h0, const float* W_out,
                                 float* y, float* h_last,
                                 void* workspace, size_t workspace_bytes, void* stream);

sr_status mingru_step_decayed(int64_t B, int64_t D_in, int64_t D_h, int64_t D_out,
                              const float* x_t, const float* W_in, const float* W_out,
                              const float* decay_rate, const float* delta_t, int log1p_delta,
                              uint32_t* saturated,
                              const float* h_prev, float* h_next, float* y_t,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace minmax_scan needs. */
size_t minmax_scan_workspace_size(int64_t B, int64_t T, int64_t D);

/*
 * MinMax neuron over a sequence (minmaxrnc PyPI page, "The model" item 3;
 * "Quick start" carries the state across calls).
 *
 *   r, s   [B,T,D] fp32 inputs of steps t = 0..T-1.
 *   x0     [B,D] fp32 initial state (required).
 *   x_out  [B,T,D] fp32: x_out[:,t,:] = x_{t+1}.
 *   x_last [B,D] fp32 or NULL: receives x_T (x0 when T == 0).
 * Results are bit-exact; NaN inputs are outside the contract.
 */
sr_status minmax_scan(int64_t B, int64_t T, int64_t D,
                      const float* r, const float* s, const float* x0,
                      float* x_out, float* x_last,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * One MinMax step for a single token, O(1) work and O(D) memory per token
 * (minmaxrnc page, "Key properties": efficient inference as a true RNN;
 * "Quick start": generation steps one token at a time carrying the state):
 *     x_next = max(min(r_t, x_prev), s_t)   element-wise over [B, D].
 * x_next may be the same buffer as x_prev.  No workspace.  Bit-exact.
 */
sr_status minmax_step(int64_t B, int64_t D, const float* r_t, const float* s_t,
                      const float* x_prev, float* x_next, void* stream);

/* Bytes of workspace the backward calls need. */
size_t mingru_scan_backward_workspace_size(int64_t B, int64_t T, int64_t D);
size_t minmax_scan_backward_workspace_size(int64_t B, int64_t T, int64_t D);

/*
 * Backward pass of the minGRU scan (the layers are trained: minGRU profile,
 * "Requirements & limits", training entry point).  For L with dL/dh_t = dh
 * on every output h_t (the scan-only mingru_forward's y) and dL/dh_T =
 * dh_last, returns
 *     dk_t = G_t z_t (1 - z_t) (g(p_t) - h_{t-1}),  dp_t = G_t z_t g'(p_t),
 *     dh0  = (1 - z_1) G_1,   with  G_t = dh_t + (1 - z_{t+1}) G_{t+1}.
 *
 *   k, p     the forward inputs (rows of ld_kp elements, kp_dtype).
 *   h0       [B,D] forward initial state or NULL (zero).
 *   h        [B,T,D] fp32 forward outputs h_1..h_T.
 *   dh       [B,T,D] fp32 upstream gradient;  dh_last [B,D] or NULL.
 *   dk, dp   [B,T,D] fp32 outputs (contiguous).  dh0 [B,D] or NULL.
 */
sr_status mingru_scan_backward(int64_t B, int64_t T, int64_t D,
                               const void* k, const void* p, int64_t ld_kp, sr_dtype kp_dtype,
                               const float* h0, const float* h, const float* dh,
                               const float* dh_last, float* dk, float* dp, float* dh0,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of the time-decayed minGRU scan (mingru_forward_decayed
 * without projections; decay contract of the delta tutorial, Step 5
 * "Adding time decay").  With gamma_t = exp(-min(decay_rate_d * gap_t, 1e4))
 * and c_t = (1 - z_t) gamma_t:
 *     dk_t = G_t z_t (1 - z_t) (g(p_t) - gamma_t h_{t-1}),  dp_t = G_t z_t g'(p_t),
 *     dh0  = c_1 G_1,   with  G_t = dh_t + c_{t+1} G_{t+1}.
 * decay_rate [D], delta_t [B,T] and log1p_delta as in mingru_forward_decayed
 * (the rates and gaps get no gradient); everything else and the workspace
 * size (mingru_scan_backward_workspace_size) as in mingru_scan_backward.
 */
sr_status mingru_scan_backward_decayed(int64_t B, int64_t T, int64_t D,
                                       const void* k, const void* p, int64_t ld_kp,
                                       sr_dtype kp_dtype,
                                       const float* decay_rate, const float* delta_t,
                                       int log1p_delta,
                                       const float* h0, const float* h, const float* dh,
                                       const float* dh_last, float* dk, float* dp, float* dh0,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of the MinMax scan (minmaxrnc page, "Key properties": the
 * gradient through the state path neither vanishes nor explodes -- it is
 * routed, unchanged, to the operand each step selects).  Gradients dx on
 * x_out and dx_last on x_T; r, s, x0 and x_out are the forward's.  Ties
 * (measure zero) route to the state: s only if strictly above min(r, x),
 * r only if strictly below x.  dr, ds [B,T,D], dx0 [B,D] or NULL.
 */
sr_status minmax_scan_backward(int64_t B, int64_t T, int64_t D,
                               const float* r, const float* s, const float* x0,
                               const float* x_out, const float* dx, const float* dx_last,
                               float* dr, float* ds, float* dx0,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The scan-only mingru_forward (W_in and W_out NULL, y = h) for callers that
 * cannot allocate -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc: no workspace argument and no allocation
 * of any kind.  Its look-back words live in a fixed device array of
 * mingru_scan_noalloc_max_workspace() bytes (32 MiB), one per GPU, held
 * until the process ends; requests needing more (scan workspace above that:
 * B * ceil(T/144) * D * 8 + 256 bytes) return SR_ERR_UNSUPPORTED before any
 * HIP call.  Every call on a GPU shares that GPU's array and resets it
 * first, on `stream`: calls in one stream are ordered and safe, calls that
 * overlap on one GPU (several streams, several host threads) race.  Results
 * are those of mingru_forward on the same inputs, bit for bit.  The first
 * call on a device looks up that device's copy of the array.
 *
 *   k, p, ld_kp, kp_dtype, h0   as in mingru_forward (scan-only use).
 *   h       [B,T,D] fp32 output;  h_last [B,D] fp32 or NULL.
 */
size_t mingru_scan_noalloc_max_workspace(void);
sr_status mingru_scan_noalloc(int64_t B, int64_t T, int64_t D,
                              const void* k, const void* p, int64_t ld_kp, sr_dtype kp_dtype,
                              const float* h0, float* h, float* h_last, void* stream);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* scanrnn_last_error(void);

/* Polls of a predecessor's unwritten look-back word after which a scan tile
 * gives up: it marks its workspace (see scanrnn_workspace_status) and
 * carries NaN for that channel instead of waiting longer (minGRU results are
 * NaN from there on; MinMax's min and max drop a NaN operand, so there only
 * the status shows it).  The default bound is never reached in normal
 * operation (predecessors are running, and publish within microseconds). */
#define SCANRNN_LOOKBACK_SPIN_LIMIT (1u << 20)

/* Lowers the bound above for scans launched afterwards by this process (all
 * threads; launches already enqueued keep theirs).  Meant for tests of the
 * timeout path: 0 gives up at the first unwritten word met.  polls above
 * SCANRNN_LOOKBACK_SPIN_LIMIT: SR_ERR_INVALID_ARGUMENT, nothing changed.
 * Pass SCANRNN_LOOKBACK_SPIN_LIMIT to restore the default. */
sr_status scanrnn_set_lookback_spin_limit(uint32_t polls);

/* Waits for `stream`, then reports what the scans that used `workspace` since
 * its last reset met: SR_ERR_LOOKBACK_TIMEOUT if one gave up waiting for a
 * predecessor chunk (a bounded wait that should never expire), else
 * SR_ERR_GATE_RANGE if a minGRU scan (forward, fused forward) met a gate
 * logit beyond the fp32 range of sigma (|k| above about 87.3; see the range
 * note at the top), else SR_OK. */
sr_status scanrnn_workspace_status(const void* workspace, void* stream);

/* Library version, "major.minor.patch". */
const char* scanrnn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SCANRNN_H */
