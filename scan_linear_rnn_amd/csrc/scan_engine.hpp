// Device-side building blocks shared by the scans (forward and backward):
// the two associative operators, buffer-descriptor access, the look-back
// words and the windowed decoupled look-back that resolves the state entering
// a tile.  Included by scan.hip and scan_bwd.hip.
#pragma once

#include "internal.hpp"
#include "scan_addr.hpp"

namespace sr {
namespace eng {


constexpr uint32_t kTagEmpty = 0xFFFFFFFFu;
constexpr uint32_t kTagState = 0xFFFFFFFEu;
constexpr uint32_t kCanonNaN = 0x7FC00000u;
constexpr size_t kHeaderBytes = 256;
// Bit pattern of the smallest normal fp32 number: a non-negative gate factor
// whose bits are below it has flushed.
constexpr uint32_t kMinNormalBits = 0x00800000u;
// Bits of the workspace status word (header word 1).
constexpr uint32_t kStatusTimeout = 1u;    // a look-back wait gave up
constexpr uint32_t kStatusGateRange = 2u;  // a gate logit beyond the fp32 range of sigma
constexpr int kWaves = addr::kFwdWaves;               // waves per workgroup
constexpr int kElemsPerLane = addr::kFwdElemsPerLane; // N * V: maps each lane keeps in registers
constexpr int kWavesPerSimd = 6;     // register budget: waves resident per SIMD
constexpr int kWindowTiles = 4;      // most preceding tiles whose look-back words one round trip fetches

struct Pair {
  float u, v;
};

// An affine map h -> a h + b carried with its complement c = 1 - a.  Both a
// and c are kept because each is the accurate one in its own range: a long
// run of steps that each keep most of the state (a near 1) has 1 - a far
// below an ulp of 1, so a product of rounded a's loses it, while the sum of
// the steps' complements keeps it to a few ulps; a run that forgets (c near
// 1) has a tiny a that the product keeps and 1 - c does not.  This is the
// log-space form's point (log(1 - z) = -softplus(k) carries the retained
// fraction without the cancelling 1 - z) kept in linear arithmetic: the
// composed state never needs a logarithm.
struct Affine {
  float a, c, b;
};

struct MinGRUOp {
  using Step = Affine;  // one step's map, as the transform produces it
  using Agg = Affine;   // a composed map
  static __device__ __forceinline__ Agg identity() { return {1.0f, 0.0f, 0.0f}; }
  // The coefficient of a composed map: 1 - C while C < 1/2 (A within half an
  // ulp of 1's spacing, and C accurate to a few ulps), else the product A.
  static __device__ __forceinline__ float coef(Agg f) { return f.c < 0.5f ? 1.0f - f.c : f.a; }
  // Folds one step into a run (sequentially, in registers): "f, then s".
  // C = C_f + A_f c_s adds non-negative terms, so it never cancels.
  static __device__ __forceinline__ Agg push(Agg f, Step s) {
    return {f.a * s.a, fmaf(f.a, s.c, f.c), fmaf(s.a, f.b, s.b)};
  }
  // Composes two runs, "f, then s", each side's coefficient the accurate one.
  static __device__ __forceinline__ Agg compose(Agg f, Agg s) {
    const float fa = coef(f), sa = coef(s);
    return {fa * sa, fmaf(fa, s.c, f.c), fmaf(sa, f.b, s.b)};
  }
  // The map a composed run applies (what phase 3 and the look-back words use).
  static __device__ __forceinline__ Pair map(Agg f) { return {coef(f), f.b}; }
  static __device__ __forceinline__ Pair step_map(Step s) { return {s.a, s.b}; }
  static __device__ __forceinline__ float apply(Pair m, float h) { return fmaf(m.u, h, m.v); }
  // (k, p) -> a = e^{-softplus(k)} = sigma(-k), its complement c = z =
  // sigma(k), and b = e^{log z + log g(p)} = z g(p), without a cancelling
  // 1 - x anywhere.  With e = e^{-|k|} and ep = e^{-|p|} in (0, 1]:
  // sigma(|k|) = 1/(1+e), sigma(-|k|) = e/(1+e), and for p < 0,
  // g(p) = sigma(p) = ep/(1+ep).  (1/(1+e) is exactly 1 when e is below half
  // an ulp of 1, so a gate at rest keeps the state exactly.)  Every value is
  // formed for both signs and selected, so the transform has no branch.
  static __device__ __forceinline__ Step element(float k, float p) {
    constexpr float kNegLog2e = -1.4426950408889634f;
    const float e = __builtin_amdgcn_exp2f(fabsf(k) * kNegLog2e);
    const float ep = __builtin_amdgcn_exp2f(fabsf(p) * kNegLog2e);
    const float big = __builtin_amdgcn_rcpf(1.0f + e);  // 1 / (1 + e)
    const float small = e * big;                        // e / (1 + e)
    const float sig_p = ep * __builtin_amdgcn_rcpf(1.0f + ep);
    const bool kpos = k >= 0.0f;
    const float z = kpos ? big : small;
    const float a = kpos ? small : big;
    const float g = p >= 0.0f ? p + 0.5f : sig_p;
    return {a, z, z * g};
  }
  // The smaller of sigma(k) and sigma(-k) of a step: below the smallest
  // normal fp32 number (|k| beyond ~87.3) it has flushed, and the term it
  // multiplies is dropped.  Kernels keep the minimum of this over their steps
  // and report out-of-range gates in the workspace status.  Both factors are
  // non-negative, so their bit patterns order like their values (one integer
  // min3 per step, and no NaN canonicalisation).
  static __device__ __forceinline__ uint32_t gate_floor(Step s, uint32_t lo) {
    const uint32_t x = __float_as_uint(s.a), y = __float_as_uint(s.c);
    const uint32_t m = x < y ? x : y;
    return lo < m ? lo : m;
  }
  static constexpr bool kHasGateRange = true;
  // Time decay of the carried state: the step's coefficient a becomes a gamma
  // with gamma = e^{-x}, and its complement 1 - a gamma = c + a (1 - gamma),
  // where om = 1 - gamma must itself be accurate for small x (see decay_factors).
  static __device__ __forceinline__ Step decayed(Step s, float gamma, float om) {
    return {s.a * gamma, fmaf(s.a, om, s.c), s.b};
  }
};

// gamma = e^{-x} = 2^y and om = 1 - gamma for x = rate * gap >= 0 (y = nx2 =
// -x log2(e) <= 0), both accurate.  For x < 1/8 the complement is y Q(y), Q a
// cubic fitted to (1 - 2^y) / y on [-log2(e)/8, 0] (decay_poly.py: relative
// error of y Q(y) below 1.4e-7 in fp32), with no cancelling subtraction;
// above it 1 - gamma loses at most a factor 8.5 to cancellation (gamma <=
// 0.883).  Evaluated in y directly (no conversion to x), the cubic costs
// three fused multiply-adds and a multiply per element.
__device__ __forceinline__ void decay_factors(float nx2, float& gamma, float& om) {
  constexpr float kYSmall = -0.18033688011112042f;  // -log2(e) / 8
  gamma = __builtin_amdgcn_exp2f(nx2);
  const float q = fmaf(fmaf(fmaf(-0.00914925244f, nx2, -0.0554514937f), nx2, -0.2402246f), nx2,
                       -0.693147182f);
  om = nx2 > kYSmall ? q * nx2 : 1.0f - gamma;
}

// The scan over time-decayed steps (the decayed forward scan).  A step's
// coefficient is a gamma, gamma = 2^y with y = -x log2(e) <= 0 its decay; as
// decay factors multiply, a composed run keeps its gates' part and its decay
// part apart: (a, c = 1 - a) of the gates exactly as MinGRUOp composes them,
// and y, the sum of its steps' y (non-positive terms: no cancellation).  Its
// coefficient is a 2^y and its complement c + a (1 - 2^y), a sum of
// non-negative terms, both accurate and formed once per composed run
// (decay_factors on the run's y) instead of once per step.  With every y
// zero the results are those of MinGRUOp, bit for bit.
struct AffineDecay {
  float a, c, y, b;
};
struct DecayedStep {
  float a, c, y, full, b;  // full = a 2^y, the step's whole coefficient
};

struct MinGRUDecayOp {
  using Step = DecayedStep;
  using Agg = AffineDecay;
  static __device__ __forceinline__ Agg identity() { return {1.0f, 0.0f, 0.0f, 0.0f}; }
  // The gates' coefficient alone, the accurate one of a and 1 - c.
  static __device__ __forceinline__ float gate_coef(Agg f) { return f.c < 0.5f ? 1.0f - f.c : f.a; }
  // The whole coefficient: 1 - C while C < 1/2, else a 2^y.
  static __device__ __forceinline__ float coef(Agg f) {
    float gamma, om;
    decay_factors(f.y, gamma, om);
    const float fa = gate_coef(f);
    const float C = fmaf(fa, om, f.c);
    return C < 0.5f ? 1.0f - C : fa * gamma;
  }
  static __device__ __forceinline__ Agg push(Agg f, Step s) {
    return {f.a * s.a, fmaf(f.a, s.c, f.c), f.y + s.y, fmaf(s.full, f.b, s.b)};
  }
  static __device__ __forceinline__ Agg compose(Agg f, Agg s) {
    const float fa = gate_coef(f), sa = gate_coef(s);
    return {fa * sa, fmaf(fa, s.c, f.c), f.y + s.y, fmaf(coef(s), f.b, s.b)};
  }
  static __device__ __forceinline__ Pair map(Agg f) { return {coef(f), f.b}; }
  static __device__ __forceinline__ Pair step_map(Step s) { return {s.full, s.b}; }
  static __device__ __forceinline__ float apply(Pair m, float h) { return fmaf(m.u, h, m.v); }
  static __device__ __forceinline__ Step element(float k, float p) {
    const Affine e = MinGRUOp::element(k, p);
    return {e.a, e.c, 0.0f, e.a, e.b};
  }
  // The step with its decay y = -x log2(e) applied to the carried state.
  static __device__ __forceinline__ Step decay(Step s, float y) {
    return {s.a, s.c, y, s.a * __builtin_amdgcn_exp2f(y), s.b};
  }
  static __device__ __forceinline__ uint32_t gate_floor(Step s, uint32_t lo) {
    return MinGRUOp::gate_floor(Affine{s.a, s.c, s.b}, lo);
  }
  static constexpr bool kHasGateRange = true;
};

struct MinMaxOp {
  using Step = Pair;
  using Agg = Pair;
  static __device__ __forceinline__ Agg identity() { return {INFINITY, -INFINITY}; }
  // "f, then s": the clamp (min(R_f, R_s), max(min(R_s, S_f), S_s)).
  static __device__ __forceinline__ Agg compose(Agg f, Agg s) {
    return {fminf(f.u, s.u), fmaxf(fminf(s.u, f.v), s.v)};
  }
  static __device__ __forceinline__ Agg push(Agg f, Step s) { return compose(f, s); }
  static __device__ __forceinline__ Pair map(Agg f) { return f; }
  static __device__ __forceinline__ Pair step_map(Step s) { return s; }
  static __device__ __forceinline__ float apply(Pair m, float x) {
    return fmaxf(fminf(m.u, x), m.v);
  }
  static __device__ __forceinline__ Step element(float r, float s) { return {r, s}; }
  static __device__ __forceinline__ uint32_t gate_floor(Step, uint32_t lo) { return lo; }
  static constexpr bool kHasGateRange = false;
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
  int window;         // look-back words fetched per tile in the first round trip, 1..kWindowTiles
  uint32_t spin_limit;  // polls of an unwritten look-back word before giving up
  // Time decay of the carried state (minGRU only; unused when rate is null).
  const float* rate;     // [D] per-channel decay rate
  const float* gap;      // [B,T] gap preceding each token
  int log1p_gap;         // gaps are compressed with log1p first
  uint32_t* saturated;   // or null: OR-ed with 1 when a rate * gap exceeds the clamp
};

// Time decay (the decay contract of the minGRU tutorials' "Adding time decay"
// step): the carried state is scaled by exp(-min(rate * gap, kDecayClamp))
// at the token boundary, before the token's own write.  exp(-x) is already
// zero in float32 for x above ~104, so the clamp changes no value and is not
// applied; it marks where large gaps stop being distinguishable, which is
// reported as saturation.  For rate >= 0, rounding is monotone in the gap, so
// some rate * gap_n exceeds the clamp exactly when rate * max_n gap_n does.
constexpr float kDecayClamp = 1.0e4f;
constexpr float kNegLog2e = -1.4426950408889634f;

// Look-back along T for one channel, used when the window fetched in one
// round trip holds no usable end state.  Returns the state entering tile
// `tchunk` of batch row b, channel d.  Walks back kB words per
// round trip to the nearest published end state (position -1 stands for the
// initial state; an unwritten word is polled, bounded), then applies the maps
// of the tiles after it one by one in order, again kB loads per
// round trip.  One apply per tile, in order, from an end state: the same fma
// sequence as the tiles' own end states, whatever the depth reached.
constexpr int kSerialBatch = 4;  // default words per round trip (register cost: 2 VGPRs each)

template <class Op, int kB>
__device__ float lookback_serial(const ScanParams& P, int64_t tchunk, int64_t b, int64_t d) {
  const size_t plane = size_t(P.B) * size_t(P.D);
  const uint64_t* col = P.state + size_t(b) * size_t(P.D) + size_t(d);
  const float h_init = (P.init != nullptr) ? P.init[size_t(b) * P.D + d] : 0.0f;
  float h = h_init;
  // Backward.  tchunk >= 1, and the batch that reaches position -1 holds the
  // initial state there, so the loop ends with an end state found.
  int64_t top = tchunk - 1;
  int64_t found = -1;
  uint32_t spins = 0;
  for (;;) {
    uint64_t w[kB];
#pragma unroll
    for (int q = 0; q < kB; ++q)
      w[q] = top - q >= 0 ? load_word(col + size_t(top - q) * plane) : pack_state(h_init);
    // First position (nearest tile) that is not a published map.
    int stop = kB;
#pragma unroll
    for (int q = kB - 1; q >= 0; --q) {
      const uint32_t hi = uint32_t(w[q] >> 32);
      if (hi == kTagState || hi == kTagEmpty) stop = q;
    }
    if (stop == kB) {  // kB maps: the next batch
      top -= kB;
      continue;
    }
    uint64_t ws = 0;
#pragma unroll
    for (int q = 0; q < kB; ++q)
      if (q == stop) ws = w[q];
    if (uint32_t(ws >> 32) == kTagState) {
      h = __uint_as_float(uint32_t(ws));
      found = top - stop;
      break;
    }
    // Tile top - stop has not published yet: poll its word.
    if (++spins > P.spin_limit) {
      __hip_atomic_fetch_or(P.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return __uint_as_float(kCanonNaN);
    }
    __builtin_amdgcn_s_sleep(8);  // ~512 cycles between polls of an unwritten word
    top -= stop;
  }
  // Forward: the maps of tiles found+1 .. tchunk-1, in order.  Every one was
  // seen published above; one that has meanwhile become an end state holds
  // the same value the apply would give.
  for (int64_t m0 = found + 1; m0 < tchunk; m0 += kB) {
    uint64_t w[kB];
#pragma unroll
    for (int q = 0; q < kB; ++q) w[q] = m0 + q < tchunk ? load_word(col + size_t(m0 + q) * plane) : 0;
#pragma unroll
    for (int q = 0; q < kB; ++q) {
      if (m0 + q < tchunk) {
        if (uint32_t(w[q] >> 32) == kTagState)
          h = __uint_as_float(uint32_t(w[q]));
        else
          h = Op::apply(unpack_map(w[q]), h);
      }
    }
  }
  return h;
}


// Where a ticket's tile lies: its position along the scan, batch row and
// first channel (tickets, chains and tiles fit in 32 bits: checked on the
// host).
struct Tile {
  int64_t tchunk, b, d0;
};

__device__ __forceinline__ Tile decode_ticket(const ScanParams& P, uint32_t ticket, int64_t Dc) {
  const uint32_t n_chains = uint32_t(P.n_chains), n_dtiles = uint32_t(P.n_dtiles);
  const uint32_t chain = ticket % n_chains;
  Tile t;
  t.tchunk = ticket / n_chains;
  t.b = chain / n_dtiles;
  t.d0 = int64_t(chain % n_dtiles) * Dc;
  return t;
}

// Phase 2 of every scan, run by the whole workgroup after the barrier that
// follows phase 1 (which left each wave's map of each channel in s_pre).
// One thread per channel turns s_pre[w] into wave w's exclusive prefix and
// forms the tile's map, which is published; all threads then fetch the
// look-back words of the P.window preceding tiles in one round trip.
// The nearest published end state, followed by the maps of the tiles after
// it applied one by one in order, gives the state entering the tile, written
// to s_hin; only if the window holds no usable end state does a thread walk
// back further (lookback_serial, SB words per round trip).  The tile's end
// state is published last.  Ends with a
// barrier, after which s_pre and s_hin are ready for phase 3.  W is the
// number of segments along T (waves of the scan kernel), NT the number of
// threads in the workgroup (a multiple of Dc, at least Dc).
template <class Op, int W, int Dc, int NT = 64 * W, int SB = kSerialBatch>
__device__ __forceinline__ void resolve_tile(const ScanParams& P, const Tile& tl,
                                             typename Op::Agg (&s_pre)[W][Dc],
                                             uint64_t (&s_win)[kWindowTiles][Dc],
                                             float (&s_hin)[Dc]) {
  const int kWin = P.window;  // in [1, kWindowTiles], uniform over the launch
  const int tid = threadIdx.x;
  const bool chan_thread = tid < Dc;
  const int64_t dc = tl.d0 + tid;
  const bool chan_on = chan_thread && dc < P.D;
  const size_t plane = size_t(P.B) * size_t(P.D);  // words per tile index
  typename Op::Agg run = Op::identity();
  if (chan_thread) {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const typename Op::Agg a = s_pre[w][tid];
      s_pre[w][tid] = run;  // exclusive prefix of wave w
      run = Op::compose(run, a);
    }
  }
  float hin = 0.0f;
  if (tl.tchunk == 0) {
    if (chan_on && P.init != nullptr) hin = P.init[size_t(tl.b) * P.D + dc];
  } else {
    if (chan_on)
      store_word(P.state + size_t(tl.tchunk) * plane + size_t(tl.b) * P.D + dc, pack_map(Op::map(run)));
    // All threads fetch the words of the kWin preceding tiles into LDS in
    // one round trip; position -1 stands for the initial state.
    const int c = tid % Dc;
    const int64_t dd = tl.d0 + c;
    static_assert(NT % Dc == 0 && NT >= Dc, "one or more full sets of channel threads");
    for (int q = tid / Dc; q < kWin; q += NT / Dc) {
      const int64_t m = tl.tchunk - 1 - q;
      uint64_t w = pack_state(__uint_as_float(kCanonNaN));
      if (dd < P.D) {
        if (m >= 0)
          w = load_word(P.state + size_t(m) * plane + size_t(tl.b) * P.D + dd);
        else if (m == -1)
          w = pack_state(P.init != nullptr ? P.init[size_t(tl.b) * P.D + dd] : 0.0f);
      }
      s_win[q][c] = w;
    }
  }
  __syncthreads();
  if (tl.tchunk > 0 && chan_on) {
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
      hin = lookback_serial<Op, SB>(P, tl.tchunk, tl.b, dc);
    }
  }
  if (chan_on) {
    s_hin[tid] = hin;
    if (tl.tchunk + 1 < P.n_tchunks)
      store_word(P.state + size_t(tl.tchunk) * plane + size_t(tl.b) * P.D + dc,
                 pack_state(Op::apply(Op::map(run), hin)));
  }
  __syncthreads();
}

// Takes a ticket (one thread, broadcast through LDS) and decodes the tile.
__device__ __forceinline__ uint32_t take_ticket(const ScanParams& P, uint32_t* s_ticket) {
  if (threadIdx.x == 0) *s_ticket = atomicAdd(P.counter, 1u);
  __syncthreads();
  // Every lane of every wave holds the same ticket; saying so keeps the
  // buffer descriptors built from it in scalar registers.
  return __builtin_amdgcn_readfirstlane(*s_ticket);
}

// Resets a scan workspace: header words to zero, look-back words to
// kTagEmpty (all bits set).  Defined in scan.hip.
sr_status reset_workspace(void* ws, size_t used_bytes, hipStream_t stream);

}  // namespace eng
}  // namespace sr
