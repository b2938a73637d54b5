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
//   * Phase 2 (one thread per channel): the W per-wave maps meet in LDS and
//     give each wave's exclusive prefix and the tile's map, which is
//     published.  Then all threads fetch, in one round trip, the look-back
//     words of the preceding tiles of the same channels into LDS (decoupled
//     look-back with a window); the nearest published end state, followed by
//     the maps of the tiles after it, gives the state entering the tile.
//     Only if the window holds no usable end state does the thread walk back
//     one tile at a time.  The tile's end state is then published.
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
constexpr int kWaves = 12;           // waves per workgroup
constexpr int kElemsPerLane = 24;    // N * V: maps each lane keeps in registers
constexpr int kWavesPerSimd = 6;     // register budget: waves resident per SIMD
constexpr int kWindowTiles = 4;      // preceding tiles whose look-back words one round trip fetches

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

// Buffer resources: a 128-bit descriptor (base, byte extent) lets a wave
// address its rows with one per-lane byte offset plus a per-row scalar
// offset, instead of a 64-bit address per load; reads past the extent return
// zero instead of faulting.  Word 3 is the gfx9-family raw-buffer format.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the streaming accesses: non-temporal (each input element is
// read once and each output written once, so they should not displace
// anything in L2 / the MALL).
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes <= 0 ? 0 : (bytes > int64_t(0xFFFFFFFF) ? int64_t(0xFFFFFFFF) : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(uint32_t(n)), kRsrcWord3);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// V inputs of type TIn as loaded (raw bits), and their conversion to float.
template <typename TIn, int V> struct Raw;

template <> struct Raw<uint16_t, 1> {  // bf16
  using type = uint32_t;
  static __device__ __forceinline__ type load(rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStreamPolicy);
  }
  static __device__ __forceinline__ void unpack(type x, float (&f)[1]) {
    f[0] = __uint_as_float(x << 16);
  }
};
template <> struct Raw<uint16_t, 2> {
  using type = uint32_t;
  static __device__ __forceinline__ type load(rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStreamPolicy);
  }
  static __device__ __forceinline__ void unpack(type x, float (&f)[2]) {
    f[0] = __uint_as_float(x << 16);
    f[1] = __uint_as_float(x & 0xFFFF0000u);
  }
};
template <> struct Raw<float, 1> {
  using type = uint32_t;
  static __device__ __forceinline__ type load(rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStreamPolicy);
  }
  static __device__ __forceinline__ void unpack(type x, float (&f)[1]) { f[0] = __uint_as_float(x); }
};
template <> struct Raw<float, 2> {
  using type = u32x2;
  static __device__ __forceinline__ type load(rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamPolicy);
  }
  static __device__ __forceinline__ void unpack(type x, float (&f)[2]) {
    f[0] = __uint_as_float(x.x);
    f[1] = __uint_as_float(x.y);
  }
};

template <int V> struct OutVec;
template <> struct OutVec<1> {
  static __device__ __forceinline__ void store(rsrc_t r, int voff, int soff, const float (&h)[1]) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(h[0]), r, voff, soff, kStreamPolicy);
  }
};
template <> struct OutVec<2> {
  static __device__ __forceinline__ void store(rsrc_t r, int voff, int soff, const float (&h)[2]) {
    u32x2 v;
    v.x = __float_as_uint(h[0]);
    v.y = __float_as_uint(h[1]);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, kStreamPolicy);
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

// Look-back along T for one channel, one tile at a time: used when the
// window fetched in one round trip holds no usable end state.  Returns the
// state entering tile `tchunk` of batch row b, channel d.
template <class Op>
__device__ float lookback_serial(const ScanParams& P, int64_t tchunk, int64_t b, int64_t d) {
  const size_t plane = size_t(P.B) * size_t(P.D);
  const uint64_t* col = P.state + size_t(b) * size_t(P.D) + size_t(d);
  float h = (P.init != nullptr) ? P.init[size_t(b) * P.D + d] : 0.0f;
  // Backward: find the nearest earlier tile whose end state is published.
  int64_t i = tchunk - 1;
  uint32_t spins = 0;
  while (i >= 0) {
    const uint64_t w = load_word(col + size_t(i) * plane);
    const uint32_t hi = uint32_t(w >> 32);
    if (hi == kTagState) {
      h = __uint_as_float(uint32_t(w));
      break;
    }
    if (hi != kTagEmpty) {
      --i;  // a published map: keep walking (tile 0 publishes only its state)
      continue;
    }
    if (++spins > kSpinLimit) {
      __hip_atomic_store(P.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return __uint_as_float(kCanonNaN);
    }
    __builtin_amdgcn_s_sleep(8);  // ~512 cycles between polls of an unwritten word
  }
  // Forward: apply the maps of tiles i+1 .. tchunk-1 in order.
  for (int64_t m = i + 1; m < tchunk; ++m) {
    const uint64_t wm = load_word(col + size_t(m) * plane);
    if (uint32_t(wm >> 32) == kTagState)
      h = __uint_as_float(uint32_t(wm));  // tile m finished meanwhile: same value
    else
      h = Op::apply(unpack_map(wm), h);
  }
  return h;
}

template <class Op, typename TIn, int V>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd)))
void chunk_scan_kernel(const ScanParams P) {
  constexpr int N = kElemsPerLane / V;
  constexpr int W = kWaves;
  using R = Raw<TIn, V>;
  __shared__ uint32_t s_ticket;
  __shared__ Pair s_pre[W][64 * V];
  __shared__ uint64_t s_win[kWindowTiles][64 * V];
  __shared__ float s_hin[64 * V];

  const int lane = threadIdx.x & 63;
  // The wave index and the ticket are the same in every lane of a wave;
  // saying so keeps the buffer descriptors built from them in scalar
  // registers (otherwise each buffer access becomes a uniformity loop).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x == 0) s_ticket = atomicAdd(P.counter, 1u);
  __syncthreads();
  // Tickets, chains and tiles all fit in 32 bits (checked on the host).
  const uint32_t ticket = __builtin_amdgcn_readfirstlane(s_ticket);
  const uint32_t n_chains = uint32_t(P.n_chains), n_dtiles = uint32_t(P.n_dtiles);
  const uint32_t chain = ticket % n_chains;
  const int64_t tchunk = ticket / n_chains;
  const int64_t b = chain / n_dtiles;
  const int64_t d = int64_t(chain % n_dtiles) * (64 * V) + lane * V;
  const bool lane_on = d < P.D;
  const int64_t tw = tchunk * (W * N) + wave * N;  // first step of this wave's run

  // Phase 1: load, transform, compose.  Loads need no branches: past the
  // end of the tensor they return zero, and every map outside [0,T) x [0,D)
  // is replaced by the identity.
  // The wave's rows start at (b, tw); row n of the run is n*ld elements on.
  const int64_t esz = sizeof(TIn);
  const int64_t row0 = b * P.T + tw;
  const int64_t dtile_first = int64_t(chain % n_dtiles) * (64 * V);
  const int64_t base_el = row0 * P.ld_in + dtile_first;
  const int64_t end_el = (P.B * P.T - 1) * P.ld_in + P.D;  // one past the last element
  const rsrc_t r0 = make_rsrc(static_cast<const TIn*>(P.in0) + base_el, (end_el - base_el) * esz);
  const rsrc_t r1 = make_rsrc(static_cast<const TIn*>(P.in1) + base_el, (end_el - base_el) * esz);
  const int voff_in = int(lane * V * esz);
  const int row_bytes = int(P.ld_in * esz);
  typename R::type raw0[N], raw1[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    raw0[n] = R::load(r0, voff_in, n * row_bytes);
    raw1[n] = R::load(r1, voff_in, n * row_bytes);
  }
  Pair e[N][V];
  Pair agg[V];
#pragma unroll
  for (int c = 0; c < V; ++c) agg[c] = Op::identity();
  // Steps [0, nvalid) of the run lie inside the sequence (a wave-uniform
  // bound, so the test is a scalar branch); lanes past D are reset below.
  // Out-of-range maps are still replayed in phase 3 but never stored.
  const int64_t rem = P.T - tw;
  const int nvalid = rem <= 0 ? 0 : (rem >= N ? N : int(rem));
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float x0[V], x1[V];
    R::unpack(raw0[n], x0);
    R::unpack(raw1[n], x1);
#pragma unroll
    for (int c = 0; c < V; ++c) e[n][c] = Op::element(x0[c], x1[c]);
    if (n < nvalid) {
#pragma unroll
      for (int c = 0; c < V; ++c) agg[c] = Op::compose(agg[c], e[n][c]);
    }
    // Keep the scheduler from interleaving many steps' temporaries while
    // all of the run's loads are still holding their registers.
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!lane_on) {
#pragma unroll
    for (int c = 0; c < V; ++c) agg[c] = Op::identity();
  }
#pragma unroll
  for (int c = 0; c < V; ++c) s_pre[wave][lane * V + c] = agg[c];
  __syncthreads();

  // Phase 2: one thread per channel combines the waves' maps and resolves
  // the state entering the tile.
  constexpr int Dc = 64 * V;
  constexpr int kWin = kWindowTiles;
  const int tid = threadIdx.x;
  const int64_t dtile0 = int64_t(chain % n_dtiles) * Dc;
  const bool chan_thread = tid < Dc;
  const int64_t dc = dtile0 + tid;
  const bool chan_on = chan_thread && dc < P.D;
  const size_t plane = size_t(P.B) * size_t(P.D);  // words per tile index
  Pair run = Op::identity();
  if (chan_thread) {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const Pair a = s_pre[w][tid];
      s_pre[w][tid] = run;  // exclusive prefix of wave w
      run = Op::compose(run, a);
    }
  }
  float hin = 0.0f;
  if (tchunk == 0) {
    if (chan_on && P.init != nullptr) hin = P.init[size_t(b) * P.D + dc];
  } else {
    if (chan_on) store_word(P.state + size_t(tchunk) * plane + size_t(b) * P.D + dc, pack_map(run));
    // All threads fetch the words of the kWin preceding tiles into LDS in
    // one round trip; position -1 stands for the initial state.
    const int c = tid % Dc;
    const int64_t dd = dtile0 + c;
    for (int q = tid / Dc; q < kWin; q += (64 * W) / Dc) {
      const int64_t m = tchunk - 1 - q;
      uint64_t w = pack_state(__uint_as_float(kCanonNaN));
      if (dd < P.D) {
        if (m >= 0)
          w = load_word(P.state + size_t(m) * plane + size_t(b) * P.D + dd);
        else if (m == -1)
          w = pack_state(P.init != nullptr ? P.init[size_t(b) * P.D + dd] : 0.0f);
      }
      s_win[q][c] = w;
    }
  }
  __syncthreads();
  if (tchunk > 0 && chan_on) {
    // Nearest published end state in the window, provided no tile between
    // it and this one is still unwritten.
    int found = -1;
    for (int q = 0; q < kWin; ++q) {
      const uint32_t hi = uint32_t(s_win[q][tid] >> 32);
      if (hi == kTagState) {
        found = q;
        break;
      }
      if (hi == kTagEmpty) break;
    }
    if (found >= 0) {
      float h = __uint_as_float(uint32_t(s_win[found][tid]));
      for (int q = found - 1; q >= 0; --q) h = Op::apply(unpack_map(s_win[q][tid]), h);
      hin = h;
    } else {
      hin = lookback_serial<Op>(P, tchunk, b, dc);
    }
  }
  if (chan_on) {
    s_hin[tid] = hin;
    if (tchunk + 1 < P.n_tchunks)
      store_word(P.state + size_t(tchunk) * plane + size_t(b) * P.D + dc,
                 pack_state(Op::apply(run, hin)));
  }
  __syncthreads();

  // Phase 3: replay the maps from the state entering this wave's run.
  float h[V];
#pragma unroll
  for (int c = 0; c < V; ++c) h[c] = Op::apply(s_pre[wave][lane * V + c], s_hin[lane * V + c]);
  const int64_t out_base = row0 * P.D + dtile_first;
  const rsrc_t ro = make_rsrc(P.out + out_base, (P.B * P.T * P.D - out_base) * 4);
  const int voff_out = lane * V * 4;
  const int out_row_bytes = int(P.D * 4);
#pragma unroll
  for (int n = 0; n < N; ++n) {
#pragma unroll
    for (int c = 0; c < V; ++c) h[c] = Op::apply(e[n][c], h[c]);
    const int64_t t = tw + n;
    if (lane_on && t < P.T) {
      OutVec<V>::store(ro, voff_out, n * out_row_bytes, h);
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
  return V == 2 ? launch_v<Op, TIn, 2>(P, stream) : launch_v<Op, TIn, 1>(P, stream);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

ScanGeometry choose_geometry(const ScanRequest& rq) {
  // Two channels per lane when the data allows it: 128-channel tiles keep
  // many independent chains along T (so few tiles of a chain are in flight
  // at once and the look-back window reaches a finished tile), with 4-byte
  // bf16 / 8-byte fp32 accesses that still cover whole cache lines per wave.
  const size_t esz = rq.in_dtype == SR_BF16 ? 2 : 4;
  int V = 1;
  const bool v2 = rq.D % 2 == 0 && rq.ld_in % 2 == 0 && aligned(rq.in0, esz * 2) &&
                  aligned(rq.in1, esz * 2) && aligned(rq.out, 8);
  const int64_t tiles_2 = (rq.D + 127) / 128, tiles_1 = (rq.D + 63) / 64;
  if (v2 && tiles_2 * 128 <= tiles_1 * 64) V = 2;
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
  // The shortest tile along T (V = 2) needs the most look-back words.
  const int64_t min_tc = int64_t(kWaves) * (kElemsPerLane / 2);
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
