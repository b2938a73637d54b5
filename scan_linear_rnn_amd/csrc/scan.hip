// Single-pass chunked scan engine for gfx950, instantiated for the minGRU
// recurrence and the MinMax neuron.
//
// What is scanned.  Both recurrences are, per channel, a chain of maps
// h_t = f_t(h_{t-1}) drawn from a family closed under composition, so the
// whole sequence can be evaluated as a prefix scan over the maps (the minGRU
// profile's parallel mode; the minmaxrnc page, "Key properties": all states in
// O(log T) depth, and "The model" item 3: the neuron is computed by a prefix
// scan).
//
//   minGRU : f_t(h) = a_t h + b_t, with the log-space coefficients
//            log a_t = log(1 - z_t) = -softplus(k_t) and
//            log b_t = log z_t + log g(p_t), exponentiated in closed form
//            (a_t = sigma(-k_t), b_t = sigma(k_t) g(p_t)).  A composed map is
//            the pair (A, B): h -> A h + B.  0 < a <= 1 and b > 0 make every
//            composed pair a contraction with A in [0, 1] and B >= 0, so the
//            pair cannot overflow and an underflowing A is its exact limit.
//   MinMax : f_t(x) = max(min(r_t, x), s_t).  Applying (R1, S1) then (R2, S2)
//            is the clamp (min(R1, R2), max(min(R2, S1), S2)) -- exact, since
//            min and max only select.
//
// How (one launch, every input element read once, every output written once):
//   * A workgroup owns a tile of Dc = 64*V channels x Tc = W*N steps of one
//     batch row.  Lanes run along the channels, so every load and store is
//     coalesced along D; wave w of the workgroup owns steps [w*N, (w+1)*N).
//   * Phase 1 (all waves): each lane loads its N x V inputs, turns them into
//     maps (the fused activation -> coefficient transform), keeps the maps in
//     registers and composes them into one map per channel.
//   * Phase 2 (wave 0): the W per-wave maps meet in LDS; wave 0 forms each
//     wave's exclusive prefix and the tile's map, publishes the tile's map,
//     then looks back along T through the tiles before it (decoupled
//     look-back) until it finds one that published its end state, and
//     publishes this tile's end state in turn.
//   * Phase 3 (all waves): each lane starts from the state entering its run
//     and re-applies its register-resident maps, storing h (or x) per step.
//
// Look-back words.  Each (tile, batch row, channel) has one 64-bit word,
// written and read with relaxed device-scope atomics (a single dwordx2 access
// that bypasses the non-coherent per-XCD L2).  The high half says what the
// word holds: kTagEmpty (not written in this launch), kTagState (the low half
// is the state after the tile), anything else (the tile's map, high half =
// the map's first component).  A word is thus self-validating and needs no
// release/acquire fence.  Tiles take their position from a ticket counter
// in execution order, so a tile only ever waits on tiles that are already
// running.  The wait is bounded; if it ever expires the tile records a
// timeout in the workspace header and produces NaN rather than hanging.
//
// Determinism.  A tile that finds the end state of tile i and the maps of
// tiles i+1..j-1 applies those maps to the state one by one in order, which
// is exactly how tile i+1..j-1 compute their own end states; the state
// entering tile j is therefore the same bits however far the look-back went.

#include "internal.hpp"

#include <cstdarg>
#include <cstdio>

namespace sr {
namespace {

constexpr uint32_t kTagEmpty = 0xFFFFFFFFu;
constexpr uint32_t kTagState = 0xFFFFFFFEu;
constexpr uint32_t kCanonNaN = 0x7FC00000u;
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr size_t kHeaderBytes = 256;
constexpr int kWaves = 8;            // waves per workgroup
constexpr int kElemsPerLane = 32;    // N * V: maps each lane keeps in registers

struct Pair {
  float u, v;
};

struct MinGRUOp {
  static __device__ __forceinline__ Pair identity() { return {1.0f, 0.0f}; }
  // The map "apply f, then s".
  static __device__ __forceinline__ Pair compose(Pair f, Pair s) {
    return {f.u * s.u, fmaf(s.u, f.v, s.v)};
  }
  static __device__ __forceinline__ float apply(Pair m, float h) { return fmaf(m.u, h, m.v); }
  // (k, p) -> (a, b) = (e^{-softplus(k)}, e^{log sigma(k) + log g(p)}).
  // With e = e^{-|k|} in (0, 1]: sigma(|k|) = 1/(1+e), sigma(-|k|) = e/(1+e),
  // so neither a nor z = sigma(k) is formed by a cancelling 1 - x.
  static __device__ __forceinline__ Pair element(float k, float p) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float e = __builtin_amdgcn_exp2f(-fabsf(k) * kLog2e);
    const float big = __builtin_amdgcn_rcpf(1.0f + e);
    const float small = e * big;
    const bool kpos = k >= 0.0f;
    const float z = kpos ? big : small;
    const float a = kpos ? small : big;
    // g(p) = p + 1/2 (p >= 0), sigma(p) = e^p / (1 + e^p) (p < 0).
    const float ep = __builtin_amdgcn_exp2f(fminf(p, 0.0f) * kLog2e);
    const float g = p >= 0.0f ? p + 0.5f : ep * __builtin_amdgcn_rcpf(1.0f + ep);
    return {a, z * g};
  }
};

struct MinMaxOp {
  static __device__ __forceinline__ Pair identity() { return {INFINITY, -INFINITY}; }
  static __device__ __forceinline__ Pair compose(Pair f, Pair s) {
    return {fminf(f.u, s.u), fmaxf(fminf(s.u, f.v), s.v)};
  }
  static __device__ __forceinline__ float apply(Pair m, float x) {
    return fmaxf(fminf(m.u, x), m.v);
  }
  static __device__ __forceinline__ Pair element(float r, float s) { return {r, s}; }
};

// ------------------------------------------------------------------ loads

// Raw vector of V inputs as loaded from memory, and its conversion to float.
template <typename TIn, int V> struct Raw;

template <> struct Raw<uint16_t, 1> {  // bf16
  using type = uint16_t;
  static __device__ __forceinline__ void unpack(type r, float (&f)[1]) {
    f[0] = __uint_as_float(uint32_t(r) << 16);
  }
};
template <> struct Raw<uint16_t, 2> {
  using type = uint32_t;
  static __device__ __forceinline__ void unpack(type r, float (&f)[2]) {
    f[0] = __uint_as_float(r << 16);
    f[1] = __uint_as_float(r & 0xFFFF0000u);
  }
};
template <> struct Raw<uint16_t, 4> {
  using type = uint2;
  static __device__ __forceinline__ void unpack(type r, float (&f)[4]) {
    f[0] = __uint_as_float(r.x << 16);
    f[1] = __uint_as_float(r.x & 0xFFFF0000u);
    f[2] = __uint_as_float(r.y << 16);
    f[3] = __uint_as_float(r.y & 0xFFFF0000u);
  }
};
template <> struct Raw<float, 1> {
  using type = float;
  static __device__ __forceinline__ void unpack(type r, float (&f)[1]) { f[0] = r; }
};
template <> struct Raw<float, 2> {
  using type = float2;
  static __device__ __forceinline__ void unpack(type r, float (&f)[2]) {
    f[0] = r.x;
    f[1] = r.y;
  }
};
template <> struct Raw<float, 4> {
  using type = float4;
  static __device__ __forceinline__ void unpack(type r, float (&f)[4]) {
    f[0] = r.x;
    f[1] = r.y;
    f[2] = r.z;
    f[3] = r.w;
  }
};

template <int V> struct OutVec;
template <> struct OutVec<1> {
  static __device__ __forceinline__ void store(float* p, const float (&h)[1]) { *p = h[0]; }
};
template <> struct OutVec<2> {
  static __device__ __forceinline__ void store(float* p, const float (&h)[2]) {
    *reinterpret_cast<float2*>(p) = make_float2(h[0], h[1]);
  }
};
template <> struct OutVec<4> {
  static __device__ __forceinline__ void store(float* p, const float (&h)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(h[0], h[1], h[2], h[3]);
  }
};

// ------------------------------------------------------------ look-back words

__device__ __forceinline__ uint64_t load_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_word(uint64_t* p, uint64_t w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack_map(Pair m) {
  uint32_t hi = __float_as_uint(m.u);
  // Only NaN inputs can produce these bit patterns; keep them off the tags.
  if (hi == kTagEmpty || hi == kTagState) hi = kCanonNaN;
  return (uint64_t(hi) << 32) | __float_as_uint(m.v);
}
__device__ __forceinline__ uint64_t pack_state(float h) {
  return (uint64_t(kTagState) << 32) | __float_as_uint(h);
}
__device__ __forceinline__ Pair unpack_map(uint64_t w) {
  return {__uint_as_float(uint32_t(w >> 32)), __uint_as_float(uint32_t(w))};
}

struct ScanParams {
  const void* in0;
  const void* in1;
  int64_t ld_in;
  float* out;
  const float* init;
  float* last;
  int64_t B, T, D;
  int64_t n_dtiles, n_tchunks, n_chains;
  uint32_t* counter;  // header word 0: ticket counter
  uint32_t* status;   // header word 1: timeout flag
  uint64_t* state;    // [n_tchunks][B][D] look-back words
};

// Wave 0's look-back for its V channels: returns the state entering tile
// `tchunk` of batch row b.
template <class Op, int V>
__device__ __forceinline__ void lookback(const ScanParams& P, int64_t tchunk, int64_t b,
                                         int64_t d, float (&hin)[V]) {
  const size_t stride = size_t(P.B) * size_t(P.D);
  const uint64_t* col = P.state + size_t(b) * size_t(P.D) + size_t(d);
  int64_t i[V];
  bool done[V];
#pragma unroll
  for (int c = 0; c < V; ++c) {
    i[c] = tchunk - 1;
    done[c] = false;
    hin[c] = (P.init != nullptr) ? P.init[size_t(b) * P.D + d + c] : 0.0f;
  }
  // Backward: find the nearest earlier tile whose end state is published.
  uint32_t spins = 0;
  bool timed_out = false;
  while (true) {
    bool all_done = true;
    uint64_t w[V];
#pragma unroll
    for (int c = 0; c < V; ++c)
      if (!done[c]) w[c] = load_word(col + size_t(i[c]) * stride + c);
    bool waiting = false;
#pragma unroll
    for (int c = 0; c < V; ++c) {
      if (done[c]) continue;
      const uint32_t hi = uint32_t(w[c] >> 32);
      if (hi == kTagState) {
        hin[c] = __uint_as_float(uint32_t(w[c]));
        done[c] = true;
      } else if (hi != kTagEmpty) {
        // A published map: step further back (tile 0 publishes only its
        // state, so i never passes below 0; the guard keeps it that way).
        if (--i[c] < 0) done[c] = true;  // hin keeps the initial state
      } else {
        waiting = true;
      }
      all_done = all_done && done[c];
    }
    if (all_done) break;
    if (waiting) {
      if (++spins > kSpinLimit) {
        timed_out = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  if (timed_out) {
    __hip_atomic_store(P.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int c = 0; c < V; ++c) hin[c] = __uint_as_float(kCanonNaN);
    return;
  }
  // Forward: apply the maps of tiles i+1 .. tchunk-1 in order.
#pragma unroll
  for (int c = 0; c < V; ++c) {
    float h = hin[c];
    for (int64_t m = (i[c] < 0 ? 0 : i[c] + 1); m < tchunk; ++m) {
      const uint64_t wm = load_word(col + size_t(m) * stride + c);
      if (uint32_t(wm >> 32) == kTagState)
        h = __uint_as_float(uint32_t(wm));  // tile m finished meanwhile: same value
      else
        h = Op::apply(unpack_map(wm), h);
    }
    hin[c] = h;
  }
}

template <class Op, typename TIn, int V>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(4)))
void chunk_scan_kernel(const ScanParams P) {
  constexpr int N = kElemsPerLane / V;
  constexpr int W = kWaves;
  using R = Raw<TIn, V>;
  __shared__ uint32_t s_ticket;
  __shared__ Pair s_pre[W][64 * V];
  __shared__ float s_hin[64 * V];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_ticket = atomicAdd(P.counter, 1u);
  __syncthreads();
  // Tickets, chains and tiles all fit in 32 bits (checked on the host).
  const uint32_t ticket = s_ticket;
  const uint32_t n_chains = uint32_t(P.n_chains), n_dtiles = uint32_t(P.n_dtiles);
  const uint32_t chain = ticket % n_chains;
  const int64_t tchunk = ticket / n_chains;
  const int64_t b = chain / n_dtiles;
  const int64_t d = int64_t(chain % n_dtiles) * (64 * V) + lane * V;
  const bool lane_on = d < P.D;
  const int64_t tw = tchunk * (W * N) + wave * N;  // first step of this wave's run

  // Phase 1: load, transform, compose.  Loads outside the tensor are
  // redirected to a valid element and their maps replaced by the identity,
  // so the loads need no branches.
  const TIn* in0 = static_cast<const TIn*>(P.in0);
  const TIn* in1 = static_cast<const TIn*>(P.in1);
  const int64_t dl = lane_on ? d : 0;
  typename R::type raw0[N], raw1[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int64_t t = (tw + n < P.T) ? tw + n : P.T - 1;
    const size_t off = size_t(b * P.T + t) * size_t(P.ld_in) + size_t(dl);
    raw0[n] = *reinterpret_cast<const typename R::type*>(in0 + off);
    raw1[n] = *reinterpret_cast<const typename R::type*>(in1 + off);
  }
  Pair e[N][V];
  Pair agg[V];
#pragma unroll
  for (int c = 0; c < V; ++c) agg[c] = Op::identity();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float x0[V], x1[V];
    R::unpack(raw0[n], x0);
    R::unpack(raw1[n], x1);
    const bool ok = lane_on && (tw + n < P.T);
#pragma unroll
    for (int c = 0; c < V; ++c) {
      const Pair el = Op::element(x0[c], x1[c]);
      e[n][c] = ok ? el : Op::identity();
      agg[c] = Op::compose(agg[c], e[n][c]);
    }
  }
#pragma unroll
  for (int c = 0; c < V; ++c) s_pre[wave][lane * V + c] = agg[c];
  __syncthreads();

  // Phase 2: wave 0 combines the waves and looks back along T.
  if (wave == 0) {
    Pair run[V];
#pragma unroll
    for (int c = 0; c < V; ++c) run[c] = Op::identity();
#pragma unroll
    for (int w = 0; w < W; ++w) {
#pragma unroll
      for (int c = 0; c < V; ++c) {
        const Pair a = s_pre[w][lane * V + c];
        s_pre[w][lane * V + c] = run[c];  // exclusive prefix of wave w
        run[c] = Op::compose(run[c], a);
      }
    }
    float hin[V];
    uint64_t* slot = P.state + (size_t(tchunk) * size_t(P.B) + size_t(b)) * size_t(P.D) + size_t(d);
    if (lane_on) {
      if (tchunk == 0) {
#pragma unroll
        for (int c = 0; c < V; ++c)
          hin[c] = (P.init != nullptr) ? P.init[size_t(b) * P.D + d + c] : 0.0f;
      } else {
#pragma unroll
        for (int c = 0; c < V; ++c) store_word(slot + c, pack_map(run[c]));
        lookback<Op, V>(P, tchunk, b, d, hin);
      }
      if (tchunk + 1 < P.n_tchunks) {
#pragma unroll
        for (int c = 0; c < V; ++c) store_word(slot + c, pack_state(Op::apply(run[c], hin[c])));
      }
    } else {
#pragma unroll
      for (int c = 0; c < V; ++c) hin[c] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < V; ++c) s_hin[lane * V + c] = hin[c];
  }
  __syncthreads();

  // Phase 3: replay the maps from the state entering this wave's run.
  float h[V];
#pragma unroll
  for (int c = 0; c < V; ++c) h[c] = Op::apply(s_pre[wave][lane * V + c], s_hin[lane * V + c]);
  float* out = P.out + size_t(b * P.T) * size_t(P.D) + size_t(d);
#pragma unroll
  for (int n = 0; n < N; ++n) {
#pragma unroll
    for (int c = 0; c < V; ++c) h[c] = Op::apply(e[n][c], h[c]);
    const int64_t t = tw + n;
    if (lane_on && t < P.T) {
      OutVec<V>::store(out + size_t(t) * size_t(P.D), h);
      if (P.last != nullptr && t == P.T - 1) {
#pragma unroll
        for (int c = 0; c < V; ++c) P.last[size_t(b) * P.D + d + c] = h[c];
      }
    }
  }
}

// Resets a scan workspace: header words to zero, look-back words to
// kTagEmpty (all bits set).
__global__ void reset_workspace_kernel(uint4* ws, size_t n_header16, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    ws[i] = (i < n_header16) ? make_uint4(0, 0, 0, 0)
                             : make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
}

__global__ void copy_or_zero_kernel(float* dst, const float* src, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : 0.0f;
}

template <class Op, typename TIn, int V>
hipError_t launch_v(const ScanParams& P, hipStream_t stream) {
  const int64_t n_blocks = P.n_chains * P.n_tchunks;
  hipLaunchKernelGGL((chunk_scan_kernel<Op, TIn, V>), dim3(uint32_t(n_blocks)),
                     dim3(64 * kWaves), 0, stream, P);
  return hipGetLastError();
}

template <class Op, typename TIn>
hipError_t launch_op(int V, const ScanParams& P, hipStream_t stream) {
  switch (V) {
    case 4: return launch_v<Op, TIn, 4>(P, stream);
    case 2: return launch_v<Op, TIn, 2>(P, stream);
    default: return launch_v<Op, TIn, 1>(P, stream);
  }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

ScanGeometry choose_geometry(const ScanRequest& rq) {
  const size_t esz = rq.in_dtype == SR_BF16 ? 2 : 4;
  int V = 1;
  for (int cand : {4, 2}) {
    const bool fits = rq.D % cand == 0 && rq.ld_in % cand == 0 &&
                      aligned(rq.in0, esz * cand) && aligned(rq.in1, esz * cand) &&
                      aligned(rq.out, 4 * cand);
    if (!fits) continue;
    // Prefer the widest vector that leaves no more idle lanes than V = 1 does.
    const int64_t tiles_c = (rq.D + 64 * cand - 1) / (64 * cand);
    const int64_t tiles_1 = (rq.D + 63) / 64;
    if (tiles_c * 64 * cand <= tiles_1 * 64) {
      V = cand;
      break;
    }
  }
  ScanGeometry g;
  g.V = V;
  g.N = kElemsPerLane / V;
  g.W = kWaves;
  g.Dc = 64 * V;
  g.Tc = int64_t(g.W) * g.N;
  g.n_dtiles = (rq.D + g.Dc - 1) / g.Dc;
  g.n_tchunks = (rq.T + g.Tc - 1) / g.Tc;
  return g;
}

size_t scan_workspace_bytes(int64_t B, int64_t T, int64_t D) {
  // The shortest tile along T (V = 4) needs the most look-back words.
  const int64_t min_tc = int64_t(kWaves) * (kElemsPerLane / 4);
  const int64_t n_tchunks = (T + min_tc - 1) / min_tc;
  return kHeaderBytes + align_up(size_t(n_tchunks) * size_t(B) * size_t(D) * 8, kAlign);
}

sr_status launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream) {
  if (n <= 0) return SR_OK;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream, dst, src, n);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SR_ERR_HIP, "copy kernel launch: %s", hipGetErrorString(err));
  return SR_OK;
}

sr_status launch_scan(const ScanRequest& rq) {
  if (rq.B == 0 || rq.D == 0) return SR_OK;
  if (rq.T == 0) {
    if (rq.last != nullptr) return launch_copy_or_zero(rq.last, rq.init, rq.B * rq.D, rq.stream);
    return SR_OK;
  }
  const ScanGeometry g = choose_geometry(rq);
  ScanParams P;
  P.in0 = rq.in0;
  P.in1 = rq.in1;
  P.ld_in = rq.ld_in;
  P.out = rq.out;
  P.init = rq.init;
  P.last = rq.last;
  P.B = rq.B;
  P.T = rq.T;
  P.D = rq.D;
  P.n_dtiles = g.n_dtiles;
  P.n_tchunks = g.n_tchunks;
  P.n_chains = rq.B * g.n_dtiles;
  // HIP caps a 1-D grid at 2^32 work-items.
  if (P.n_chains * P.n_tchunks * (64 * kWaves) > int64_t(0xFFFFFFFFu))
    return fail(SR_ERR_UNSUPPORTED, "scan of %lld tiles exceeds one launch's grid",
                (long long)(P.n_chains * P.n_tchunks));
  char* ws = static_cast<char*>(rq.workspace);
  P.counter = reinterpret_cast<uint32_t*>(ws);
  P.status = reinterpret_cast<uint32_t*>(ws) + 1;
  P.state = reinterpret_cast<uint64_t*>(ws + kHeaderBytes);

  const size_t used = kHeaderBytes + size_t(g.n_tchunks) * size_t(rq.B) * size_t(rq.D) * 8;
  const size_t n16 = (used + 15) / 16;
  const size_t blocks = (n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096;
  hipLaunchKernelGGL(reset_workspace_kernel, dim3(uint32_t(blocks)), dim3(256), 0, rq.stream,
                     reinterpret_cast<uint4*>(ws), kHeaderBytes / 16, n16);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SR_ERR_HIP, "workspace reset launch: %s", hipGetErrorString(err));

  if (rq.op == ScanOp::kMinMax)
    err = launch_op<MinMaxOp, float>(g.V, P, rq.stream);
  else if (rq.in_dtype == SR_BF16)
    err = launch_op<MinGRUOp, uint16_t>(g.V, P, rq.stream);
  else
    err = launch_op<MinGRUOp, float>(g.V, P, rq.stream);
  if (err != hipSuccess) return fail(SR_ERR_HIP, "scan launch: %s", hipGetErrorString(err));
  return SR_OK;
}

}  // namespace sr
