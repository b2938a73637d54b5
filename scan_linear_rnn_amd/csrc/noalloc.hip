// The scan-only minGRU forward without a caller workspace: its look-back
// words live in a fixed device array, so the call allocates nothing (for
// callers that cannot allocate: code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// `scratch` is one file-scope device array; every GPU that loads the library
// holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (in host code it only stands for the symbol): the
// first call on a device looks up that device's address of the array with
// hipGetSymbolAddress, with the device current, and keeps it; every later
// use goes through the kept address.  Calls on one GPU share the array and
// the call's launches reset what they use (the header and the look-back
// words) with a fill kernel first, so calls that overlap on one GPU (two
// streams at once) race; calls in one stream do not.

#include <mutex>

#include "internal.hpp"

namespace sr {
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB: look-back words of 3.9 M (tile, channel)s
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// This device's address of `scratch` (looked up once per device).
sr_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(SR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SR_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || ptr == nullptr)
      return fail(SR_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(err));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SR_OK;
}

}  // namespace
}  // namespace sr

using namespace sr;

extern "C" size_t mingru_scan_noalloc_max_workspace(void) { return kScratchBytes; }

extern "C" sr_status mingru_scan_noalloc(int64_t B, int64_t T, int64_t D, const void* k,
                                         const void* p, int64_t ld_kp, sr_dtype kp_dtype,
                                         const float* h0, float* h, float* h_last, void* stream) {
  clear_last_error();
  // Every check that needs no GPU comes first: a request beyond the scratch
  // array is refused before any HIP call.
  if (B < 0 || T < 0 || D < 0)
    return fail(SR_ERR_INVALID_ARGUMENT, "sizes must be non-negative (B=%lld T=%lld D=%lld)",
                (long long)B, (long long)T, (long long)D);
  int64_t n = 0;
  if (__builtin_mul_overflow(B, T, &n) || __builtin_mul_overflow(n, D, &n))
    return fail(SR_ERR_INVALID_ARGUMENT, "tensor sizes overflow int64");
  if (kp_dtype != SR_F32 && kp_dtype != SR_BF16)
    return fail(SR_ERR_INVALID_ARGUMENT, "kp_dtype %d unsupported", int(kp_dtype));
  if (ld_kp < D)
    return fail(SR_ERR_INVALID_ARGUMENT, "ld_kp (%lld) must be >= D (%lld)", (long long)ld_kp,
                (long long)D);
  int64_t span = 0;
  if (__builtin_mul_overflow(B, T, &span) || __builtin_mul_overflow(span, ld_kp, &span))
    return fail(SR_ERR_INVALID_ARGUMENT, "k/p extent overflows int64");
  if (n > 0 && (k == nullptr || p == nullptr || h == nullptr))
    return fail(SR_ERR_INVALID_ARGUMENT, "k, p and h are required");
  const size_t esz = kp_dtype == SR_BF16 ? 2 : 4;
  if (!aligned(k, esz) || !aligned(p, esz))
    return fail(SR_ERR_INVALID_ARGUMENT, "k and p must be aligned to their element size");
  if (!aligned(h0, 4) || !aligned(h, 4) || !aligned(h_last, 4))
    return fail(SR_ERR_INVALID_ARGUMENT, "fp32 pointers must be 4-byte aligned");
  const size_t need = scan_workspace_bytes(B, T, D);
  if (need > kScratchBytes)
    return fail(SR_ERR_UNSUPPORTED,
                "scan of B=%lld T=%lld D=%lld needs %zu bytes of look-back words, more than the "
                "%zu-byte no-alloc scratch (use mingru_forward with a workspace)",
                (long long)B, (long long)T, (long long)D, need, kScratchBytes);
  if (B == 0 || D == 0) return SR_OK;
  void* ws = nullptr;
  sr_status st = scratch_for_current_device(&ws);
  if (st != SR_OK) return st;
  ScanRequest rq{};
  rq.op = ScanOp::kMinGRU;
  rq.in_dtype = kp_dtype;
  rq.B = B;
  rq.T = T;
  rq.D = D;
  rq.in0 = k;
  rq.in1 = p;
  rq.ld_in = ld_kp;
  rq.init = h0;
  rq.out = h;
  rq.last = h_last;
  rq.workspace = ws;
  rq.stream = static_cast<hipStream_t>(stream);
  rq.check_only = true;
  st = launch_scan(rq);
  if (st != SR_OK) return st;
  rq.check_only = false;
  return launch_scan(rq);
}
