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
//     further, a few words per round trip.  The tile's end state is then
//     published.
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

#include <type_traits>

#include "scan_engine.hpp"

namespace sr {
namespace eng {

// Resets a scan workspace: header words to zero, look-back words to
// kTagEmpty (all bits set).
__global__ void reset_workspace_kernel(uint4* ws, size_t n_header16, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    ws[i] = (i < n_header16) ? make_uint4(0, 0, 0, 0)
                             : make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
}

sr_status reset_workspace(void* ws, size_t used, hipStream_t stream) {
  const size_t n16 = (used + 15) / 16;
  const size_t blocks = (n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096;
  hipLaunchKernelGGL(reset_workspace_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(ws), kHeaderBytes / 16, n16);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SR_ERR_HIP, "workspace reset launch: %s", hipGetErrorString(err));
  return SR_OK;
}

}  // namespace eng

namespace {
using namespace eng;

// E: maps each lane keeps (N * V); kElemsPerLane except for the MinMax
// scan's shorter tiles (choose_geometry).
template <class Op, typename TIn, int V, bool kDecay, int E = kElemsPerLane>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd)))
void chunk_scan_kernel(const ScanParams P) {
  static_assert(E % V == 0 && E <= kElemsPerLane, "whole runs within the register budget");
  constexpr int N = E / V;
  constexpr int W = kWaves;
  using R = Raw<TIn, V>;
  using Agg = typename Op::Agg;
  __shared__ uint32_t s_ticket;
  __shared__ Agg s_pre[W][64 * V];
  __shared__ uint64_t s_win[kWindowTiles][64 * V];
  __shared__ float s_hin[64 * V];

  const int lane = threadIdx.x & 63;
  // The wave index is the same in every lane of a wave; saying so keeps the
  // buffer descriptors built from it in scalar registers (otherwise each
  // buffer access becomes a uniformity loop).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ticket = take_ticket(P, &s_ticket);
  const uint32_t n_chains = uint32_t(P.n_chains), n_dtiles = uint32_t(P.n_dtiles);
  const uint32_t chain = ticket % n_chains;
  const int64_t tchunk = ticket / n_chains;
  const int64_t b = chain / n_dtiles;
  const int64_t dtile_first = int64_t(chain % n_dtiles) * (64 * V);
  const int64_t d = dtile_first + lane * V;
  const bool lane_on = d < P.D;
  const int64_t tw = tchunk * (W * N) + wave * N;  // first step of this wave's run
  // The run's rows and the lane's channel, clamped so that every load stays
  // inside the tensor (scan_addr.hpp); steps [0, nvalid) of the run lie
  // inside the sequence (wave-uniform).
  addr::FwdRun run = addr::fwd_run(P.T, P.D, V, N, tw, dtile_first, lane);
  // The row clamps depend on the wave only: said so, they stay in scalar
  // registers (a per-lane row offset would need a loop per buffer load).
  run.nvalid = __builtin_amdgcn_readfirstlane(run.nvalid);
  run.n_last = __builtin_amdgcn_readfirstlane(run.n_last);
  const int nvalid = run.nvalid;
  const int64_t t_base = run.t_base;

  // Phase 1: load, transform, compose.
  const int64_t esz = sizeof(TIn);
  const int64_t base_el = (b * P.T + t_base) * P.ld_in + dtile_first;
  const int64_t end_el = (P.B * P.T - 1) * P.ld_in + P.D;  // one past the last element
  const rsrc_t r0 = make_rsrc(static_cast<const TIn*>(P.in0) + base_el, (end_el - base_el) * esz);
  const rsrc_t r1 = make_rsrc(static_cast<const TIn*>(P.in1) + base_el, (end_el - base_el) * esz);
  const int voff_in = int(run.lane_ch * esz);
  const int row_bytes = int(P.ld_in * esz);  // N * row_bytes < 2^31: checked on the host
  // Time decay: -rate * log2(e) for each of the lane's channels, and the gap
  // of step n of the run held by lane n (one load per wave; the step's gap
  // is then read from that lane, so it is uniform across the wave).  Rates
  // past D and gaps past T are zero: no decay, no saturation.  Issued before
  // the input loads so that the first step does not wait for all of them.
  float nrate[V];
  float gap_l = 0.0f, gap_max = 0.0f;
  typename Raw<float, V>::type rate_raw{};
  if constexpr (kDecay) {
    // Buffer loads throughout: channels past D, lanes >= N and steps past T
    // fall outside the descriptors' extents (per-lane offsets, soffset 0)
    // and read zero, with no branch (a branch around a load would make the
    // wave wait for it right there).
    const int64_t n_gaps = nvalid;
    const rsrc_t rg = make_rsrc(P.gap + (tw < P.T ? b * P.T + tw : 0), n_gaps * 4);
    gap_l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, lane * 4, 0, 0));
    const rsrc_t rr = make_rsrc(P.rate + dtile_first, (P.D - dtile_first) * 4);
    rate_raw = Raw<float, V>::load(rr, lane * V * 4, 0);
  }
  typename R::type raw0[N], raw1[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int soff = addr::fwd_row(run, n) * row_bytes;  // scalar
    raw0[n] = R::load(r0, voff_in, soff);
    raw1[n] = R::load(r1, voff_in, soff);
  }
  if constexpr (kDecay) {
    if (P.log1p_gap) gap_l = log1pf(gap_l);  // after the input loads are issued
    Raw<float, V>::unpack(rate_raw, nrate);
#pragma unroll
    for (int c = 0; c < V; ++c) nrate[c] *= kNegLog2e;
  }
  Pair e[N][V];
  Agg agg[V];
#pragma unroll
  for (int c = 0; c < V; ++c) agg[c] = Op::identity();
  uint32_t gate_lo = 0x3F800000u;  // bits of 1.0f
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float x0[V], x1[V];
    R::unpack(raw0[n], x0);
    R::unpack(raw1[n], x1);
    typename Op::Step st[V], raw_st[V];
#pragma unroll
    for (int c = 0; c < V; ++c) st[c] = raw_st[c] = Op::element(x0[c], x1[c]);
    if constexpr (kDecay) {
      const float gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gap_l), n));
      gap_max = fmaxf(gap_max, gn);
#pragma unroll
      for (int c = 0; c < V; ++c) st[c] = Op::decay(st[c], nrate[c] * gn);
    }
#pragma unroll
    for (int c = 0; c < V; ++c) e[n][c] = Op::step_map(st[c]);
    // Steps inside the sequence join the run's map and the gate check (one
    // wave-uniform test per step).
    if (n < nvalid) {
#pragma unroll
      for (int c = 0; c < V; ++c) {
        agg[c] = Op::push(agg[c], st[c]);
        gate_lo = Op::gate_floor(raw_st[c], gate_lo);
      }
    }
    // Keep the scheduler from interleaving many steps' temporaries while
    // all of the run's loads are still holding their registers.
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!lane_on) {
#pragma unroll
    for (int c = 0; c < V; ++c) agg[c] = Op::identity();
  }
  // Flags: a gate logit beyond the fp32 range of sigma (valid steps and
  // channels only), and time-decay saturation.
  if constexpr (Op::kHasGateRange) {
    if (__builtin_amdgcn_ballot_w64(gate_lo < kMinNormalBits && lane_on) != 0 && lane == 0)
      __hip_atomic_fetch_or(P.status, kStatusGateRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if constexpr (kDecay) {
    if (P.saturated != nullptr) {
      bool sat = false;
#pragma unroll
      for (int c = 0; c < V; ++c) sat = sat || (d + c < P.D && P.rate[d + c] * gap_max > kDecayClamp);
      if (__builtin_amdgcn_ballot_w64(sat) != 0 && lane == 0)
        __hip_atomic_fetch_or(P.saturated, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
#pragma unroll
  for (int c = 0; c < V; ++c) s_pre[wave][lane * V + c] = agg[c];
  __syncthreads();

  // Phase 2: the state entering the tile (decoupled look-back).
  resolve_tile<Op, W, 64 * V>(P, Tile{tchunk, b, dtile_first}, s_pre, s_win, s_hin);

  // Phase 3: replay the maps from the state entering this wave's run and
  // store the valid steps (a scalar bound; lanes past D store nothing).
  if (lane_on) {
    float h[V];
#pragma unroll
    for (int c = 0; c < V; ++c)
      h[c] = Op::apply(Op::map(s_pre[wave][lane * V + c]), s_hin[lane * V + c]);
    const int64_t out_base = (b * P.T + t_base) * P.D + dtile_first;
    const rsrc_t ro = make_rsrc(P.out + out_base, (P.B * P.T * P.D - out_base) * 4);
    const int voff_out = lane * V * 4;
    const int out_row_bytes = int(P.D * 4);  // N * out_row_bytes < 2^31: checked on the host
    const int64_t n_final = P.T - 1 - tw;   // the step holding h_T, if in this run
#pragma unroll
    for (int n = 0; n < N; ++n) {
#pragma unroll
      for (int c = 0; c < V; ++c) h[c] = Op::apply(e[n][c], h[c]);
      if (n < nvalid) {
        OutVec<V>::store(ro, voff_out, n * out_row_bytes, h);
        if (P.last != nullptr && n == n_final) {
#pragma unroll
          for (int c = 0; c < V; ++c) P.last[size_t(b) * P.D + d + c] = h[c];
        }
      }
    }
  }
}

// One MinMax step for every channel: x_next = max(min(r, x_prev), s).
__global__ void minmax_step_kernel(const float* r, const float* s, const float* x_prev,
                                   float* x_next, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    x_next[i] = MinMaxOp::apply(Pair{r[i], s[i]}, x_prev[i]);
}

__global__ void copy_or_zero_kernel(float* dst, const float* src, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : 0.0f;
}

template <class Op, typename TIn, int V, bool kDecay, int E = kElemsPerLane>
hipError_t launch_v(const ScanParams& P, hipStream_t stream) {
  const int64_t n_blocks = P.n_chains * P.n_tchunks;
  hipLaunchKernelGGL((chunk_scan_kernel<Op, TIn, V, kDecay, E>), dim3(uint32_t(n_blocks)),
                     dim3(64 * kWaves), 0, stream, P);
  return hipGetLastError();
}

template <class Op, typename TIn, bool kDecay = false>
hipError_t launch_op(const ScanGeometry& g, const ScanParams& P, hipStream_t stream) {
  if constexpr (std::is_same_v<Op, MinMaxOp>) {
    if (g.V == 1 && g.N == addr::kFwdElemsPerLaneShort)
      return launch_v<Op, TIn, 1, kDecay, addr::kFwdElemsPerLaneShort>(P, stream);
  }
  return g.V == 2 ? launch_v<Op, TIn, 2, kDecay>(P, stream) : launch_v<Op, TIn, 1, kDecay>(P, stream);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

ScanGeometry choose_geometry(const ScanRequest& rq) {
  // Two channels per lane when the data allows it, the 128-channel tiles pad
  // no more than 64-channel ones, and they still leave at least 32 chains
  // (batch rows x channel tiles): 4-byte bf16 / 8-byte fp32 accesses cover
  // whole cache lines per wave.  With fewer chains, about 512 resident tiles
  // put dozens of tiles of each chain in flight at once, and nearly every
  // tile waits on predecessors that are still loading (serial look-back,
  // ~11 tiles deep at 8 chains); one channel per lane doubles the chains and
  // halves that depth, which outweighs its 128-byte row segments.  Measured
  // (bf16, one launch): 1 x 65536 x 1024 128.3 -> 120.9 us, 8 x 65536 x 256
  // 213.7 -> 204.4 us; equal at 32 chains (4 x 65536 x 1024), and 48 chains
  // are better with two channels per lane.
  const size_t esz = rq.in_dtype == SR_BF16 ? 2 : 4;
  int V = 1;
  const bool v2 = rq.D % 2 == 0 && rq.ld_in % 2 == 0 && aligned(rq.in0, esz * 2) &&
                  aligned(rq.in1, esz * 2) && aligned(rq.out, 8);
  const int64_t tiles_2 = (rq.D + 127) / 128, tiles_1 = (rq.D + 63) / 64;
  constexpr int64_t kMinChains = 32;
  if (v2 && tiles_2 * 128 <= tiles_1 * 64 && rq.B * tiles_2 >= kMinChains) V = 2;
  ScanGeometry g;
  g.V = V;
  g.N = kElemsPerLane / V;
  // The MinMax scan with one channel per lane and at least 16 chains takes
  // 240-step tiles (20 steps per lane) instead of 288: its maps are two
  // selections, so a tile's work is almost all loads and stores, and the
  // shorter tiles even out the last of the launch.  Measured (fp32, median
  // of 50 launches after 100, one process): 8 x 32768 x 192 (24 chains)
  // 120.7 -> 116.9 us, 32 x 32768 x 192 436.1 -> 427.6 us, 8 x 131072 x 192
  // 418.8 -> 415.0 us; with 3 chains (1 x 262144 x 192) 153.5 -> 171.4 us
  // and with two channels per lane (8 x 65536 x 1024) 1106 -> 1113 us, so
  // those keep 288.
  constexpr int64_t kShortMinChains = 16;
  if (rq.op == ScanOp::kMinMax && V == 1 && rq.B * tiles_1 >= kShortMinChains)
    g.N = addr::kFwdElemsPerLaneShort;
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

sr_status launch_minmax_step(const float* r, const float* s, const float* x_prev, float* x_next,
                             int64_t n, hipStream_t stream) {
  if (n <= 0) return SR_OK;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(minmax_step_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream, r, s, x_prev,
                     x_next, n);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SR_ERR_HIP, "MinMax step launch: %s", hipGetErrorString(err));
  return SR_OK;
}

// First look-back window.  About 512 tiles are resident at once (two
// workgroups per CU on 256 CUs); spread over n_chains chains, a tile's
// nearest finished predecessor is about 512 / n_chains tiles back, so that
// many words are fetched first: 1 when predecessors have usually finished
// (fewer window reads), up to kWindowTiles.  Measured: 64 x 8192 x 1024
// bf16 720 -> 705 us with 1 word instead of 4; 8 x 65536 x 1024 best at 4.
static int lookback_window(int64_t n_chains) {
  constexpr int64_t kResidentTiles = 512;
  const int64_t per_chain = (kResidentTiles + n_chains - 1) / n_chains;
  return int(per_chain < 1 ? 1 : (per_chain > kWindowTiles ? kWindowTiles : per_chain));
}

sr_status launch_scan(const ScanRequest& rq) {
  if (rq.B == 0 || rq.D == 0) return SR_OK;
  if (rq.T == 0) {
    if (rq.last != nullptr && !rq.check_only)
      return launch_copy_or_zero(rq.last, rq.init, rq.B * rq.D, rq.stream);
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
  // A wave addresses its rows with 32-bit scalar offsets of up to N rows.
  const int64_t esz = rq.in_dtype == SR_BF16 ? 2 : 4;
  const int64_t max_row_bytes = rq.ld_in * esz > rq.D * 4 ? rq.ld_in * esz : rq.D * 4;
  if (max_row_bytes * g.N > int64_t(0x7FFFFFFF))
    return fail(SR_ERR_UNSUPPORTED, "scan rows of %lld bytes are too long",
                (long long)max_row_bytes);
  if (rq.check_only) return SR_OK;
  char* ws = static_cast<char*>(rq.workspace);
  P.counter = reinterpret_cast<uint32_t*>(ws);
  P.status = reinterpret_cast<uint32_t*>(ws) + 1;
  P.state = reinterpret_cast<uint64_t*>(ws + kHeaderBytes);
  P.window = lookback_window(P.n_chains);
  P.spin_limit = lookback_spin_limit();
  P.rate = rq.decay_rate;
  P.gap = rq.delta_t;
  P.log1p_gap = rq.log1p_delta;
  P.saturated = rq.saturated;

  const size_t used = kHeaderBytes + size_t(g.n_tchunks) * size_t(rq.B) * size_t(rq.D) * 8;
  sr_status st = reset_workspace(ws, used, rq.stream);
  if (st != SR_OK) return st;
  hipError_t err;
  const bool decay = rq.decay_rate != nullptr;
  if (rq.op == ScanOp::kMinMax)
    err = launch_op<MinMaxOp, float>(g, P, rq.stream);
  else if (decay && rq.in_dtype == SR_BF16)
    err = launch_op<MinGRUDecayOp, uint16_t, true>(g, P, rq.stream);
  else if (decay)
    err = launch_op<MinGRUDecayOp, float, true>(g, P, rq.stream);
  else if (rq.in_dtype == SR_BF16)
    err = launch_op<MinGRUOp, uint16_t>(g, P, rq.stream);
  else
    err = launch_op<MinGRUOp, float>(g, P, rq.stream);
  if (err != hipSuccess) return fail(SR_ERR_HIP, "scan launch: %s", hipGetErrorString(err));
  return SR_OK;
}

}  // namespace sr
