// Backward pass of the two scans on the same engine, run in reverse time.
//
// The gradient of a linear recurrence is again a linear recurrence, backward
// in time (the chain rule; the MinMax page's "Key properties" note that
// gradients through the MinMax state path neither vanish nor explode, and the
// minGRU profile's "Requirements & limits" name a training entry point).  With
// dL/dh_t = dh_t given for every output:
//
//   minGRU : G_t = a_{t+1} G_{t+1} + dh_t      (a = 1 - z = sigma(-k))
//            dk_t = G_t z_t a_t (g(p_t) - h_{t-1}),  dp_t = G_t z_t g'(p_t),
//            dh_0 = a_1 G_1
//            With time decay (the delta tutorial's "Adding time decay": the
//            carried state is scaled by gamma_t = exp(-lambda_d gap_t) before
//            token t's write) a_t becomes a_t gamma_t in G and dh_0, and
//            h_{t-1} becomes gamma_t h_{t-1} in dk_t; rates and gaps get no
//            gradient.
//   MinMax : Gamma_{t+1} = c_{t+1} Gamma_{t+2} + dx_{t+1}, c in {0, 1} the
//            "state passes through" indicator of the step; dr_t / ds_t get
//            Gamma_{t+1} where r_t / s_t was selected, dx_0 = c_0 Gamma_1.
//
// Both are scans of affine maps G -> c G + x, so the forward engine's affine
// operator, look-back and determinism carry over unchanged.  Scan position u
// is time t = T-1-u; the step's map is (coefficient of the next step, the
// step's upstream gradient), with the coefficient of the last time step set
// to 1 so that the gradient on the returned final state enters as the
// initial state.  Phase 3 turns each G_t into the step's input gradients from
// the step's inputs and the forward state before it.
//
// Reading for MinMax ties (measure zero for continuous inputs): s is selected
// only if strictly greater than min(r, x), r only if strictly smaller than x;
// otherwise the state passes.

#include <type_traits>

#include "scan_engine.hpp"

namespace sr {
namespace {
using namespace eng;

constexpr int kBwdWaves = addr::kBwdWaves;
constexpr int kBwdElemsPerLane = addr::kBwdElemsPerLane;  // N * V steps kept per lane
constexpr int kBwdWavesPerSimd = 4;

struct BwdParams {
  ScanParams core;      // look-back context; core.init = gradient on the final state
  const void* in0;      // k (minGRU) or r (MinMax)
  const void* in1;      // p or s
  int64_t ld_in;
  const float* fwd;     // forward outputs [B,T,D]: h_t (minGRU), x_{t+1} (MinMax)
  const float* fwd0;    // forward initial state [B,D] (may be null for minGRU)
  const float* grad;    // upstream gradient on every output [B,T,D]
  float* d0;            // dk / dr  [B,T,D]
  float* d1;            // dp / ds  [B,T,D]
  float* dinit;         // dh0 / dx0 [B,D] or null
  const float* rate;    // time decay (minGRU): [D] per-channel rate
  const float* gap;     // [B,T] gap preceding each token
  int log1p_gap;        // gaps compressed with log1p first
};

__device__ __forceinline__ void sig_pair(float k, float& z, float& a) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(-fabsf(k) * kLog2e);
  const float big = __builtin_amdgcn_rcpf(1.0f + e);
  const float small = e * big;
  z = k >= 0.0f ? big : small;  // sigma(k)
  a = k >= 0.0f ? small : big;  // 1 - sigma(k)
}

// g(p) and g'(p).
__device__ __forceinline__ void g_and_slope(float p, float& g, float& gs) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float ep = __builtin_amdgcn_exp2f(fminf(p, 0.0f) * kLog2e);
  const float sp = ep * __builtin_amdgcn_rcpf(1.0f + ep);  // sigma(p) for p < 0
  g = p >= 0.0f ? p + 0.5f : sp;
  gs = p >= 0.0f ? 1.0f : sp * (1.0f - sp);
}

// MinMax selection at one step: 0 the state passes, 1 r selected, 2 s selected.
__device__ __forceinline__ int selection(float r, float s, float x) {
  return s > fminf(r, x) ? 2 : (r < x ? 1 : 0);
}

enum Kind { kMinGRU = 0, kMinMax = 1 };

// V channels per lane, N steps per lane, W waves.  The wave's rows, at scan
// step n, are t_n = t_hi - n; loads are clamped into [0, T) and addressed
// from the lowest row any of them touches, so every buffer offset is
// non-negative and small.
template <int KIND, typename TIn, int V, int N, int W, bool kDecay, int SB>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(kBwdWavesPerSimd)))
void scan_backward_kernel(const BwdParams Q) {
  using R = Raw<TIn, V>;
  using RF = Raw<float, V>;
  // The reverse maps G -> coef G + grad compose as the forward's do; with
  // time decay their runs keep the gates' part and the summed log2 decay
  // apart (MinGRUDecayOp), so each step's decay needs no complement.
  using Op = std::conditional_t<KIND == kMinGRU && kDecay, MinGRUDecayOp, MinGRUOp>;
  constexpr int Dc = 64 * V;
  const ScanParams& P = Q.core;
  __shared__ uint32_t s_ticket;
  __shared__ typename Op::Agg s_pre[W][Dc];
  __shared__ uint64_t s_win[kWindowTiles][Dc];
  __shared__ float s_hin[Dc];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ticket = take_ticket(P, &s_ticket);
  const Tile tl = decode_ticket(P, ticket, Dc);
  const int64_t d = tl.d0 + lane * V;
  const bool lane_on = d < P.D;
  const int64_t T = P.T;
  // The run's rows (clamped into [0, T), addressed from the lowest one) and
  // the lane's channel, so that every access stays inside its tensor
  // (scan_addr.hpp).
  addr::BwdRun run = addr::bwd_run(T, P.D, V, N, tl.tchunk, wave, W, tl.d0, lane);
  // The row offsets depend on the wave only: said so, they stay in scalar
  // registers (a per-lane row offset would need a loop per buffer access).
  run.nvalid = __builtin_amdgcn_readfirstlane(run.nvalid);
  run.rbase = (int64_t(__builtin_amdgcn_readfirstlane(int(run.rbase >> 32))) << 32) |
              uint32_t(__builtin_amdgcn_readfirstlane(int(run.rbase)));
  run.t_hi = (int64_t(__builtin_amdgcn_readfirstlane(int(run.t_hi >> 32))) << 32) |
             uint32_t(__builtin_amdgcn_readfirstlane(int(run.t_hi)));
  const int64_t t_hi = run.t_hi;
  const int nvalid = run.nvalid;
  auto soff = [&](int64_t row, int64_t row_bytes) -> int {
    return int(addr::bwd_row(run, T, row) * row_bytes);
  };
  const int64_t row0 = tl.b * T + run.rbase;

  // Descriptors over the inputs, the forward states and the gradients.
  const int64_t esz = sizeof(TIn);
  const int64_t in_base = row0 * Q.ld_in + tl.d0;
  const int64_t in_end = (P.B * T - 1) * Q.ld_in + P.D;
  const rsrc_t r0 = make_rsrc(static_cast<const TIn*>(Q.in0) + in_base, (in_end - in_base) * esz);
  const rsrc_t r1 = make_rsrc(static_cast<const TIn*>(Q.in1) + in_base, (in_end - in_base) * esz);
  const int64_t f_base = row0 * P.D + tl.d0;
  const int64_t f_end = P.B * T * P.D;
  const rsrc_t rf = make_rsrc(Q.fwd + f_base, (f_end - f_base) * 4);
  const rsrc_t rg = make_rsrc(Q.grad + f_base, (f_end - f_base) * 4);
  const int vin = int(run.lane_ch * esz), vf = int(run.lane_ch * 4);
  const int64_t in_row = Q.ld_in * esz, f_row = P.D * 4;

  // Time decay: -rate * log2(e) for the lane's channels, and lane i holding
  // the gap of time t_hi + 1 - i (i = 0 .. N; rows clamped into [0, T), and
  // only the in-range ones are used), so that step n reads the gaps of its
  // following step (lane n) and of itself (lane n + 1) with readlane.  Both
  // are loaded before the step inputs, so that the first step does not wait
  // for all of those.
  float nrate[V];
  float gap_l = 0.0f;
  typename RF::type rate_raw{};
  if constexpr (kDecay) {
    const rsrc_t rr = make_rsrc(Q.rate + tl.d0, (P.D - tl.d0) * 4);
    rate_raw = RF::load(rr, lane * V * 4, 0);
    const int64_t gt = t_hi + 1 - lane;
    const int64_t grow = gt < 0 ? 0 : (gt > T - 1 ? T - 1 : gt);
    const rsrc_t rgap = make_rsrc(Q.gap + tl.b * T, T * 4);
    gap_l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rgap, int(grow * 4), 0, 0));
  }

  // Step inputs.  minGRU: in0 rows t_n+1 .. t_n (k), in1 rows t_n (p),
  // fwd rows t_n - 1 (h_{t-1}).  MinMax: in0/in1 rows t_n+1 .. t_n (r, s),
  // fwd rows t_n .. t_n - 1 (x_{t+1} .. x_t).
  typename R::type i0[N + 1], i1[N + 1];
  typename RF::type fw[N + 1], gr[N];
#pragma unroll
  for (int i = 0; i <= N; ++i) {
    i0[i] = R::load(r0, vin, soff(t_hi + 1 - i, in_row));
    if (KIND == kMinMax || i < N) i1[i] = R::load(r1, vin, soff(KIND == kMinMax ? t_hi + 1 - i : t_hi - i, in_row));
    if (KIND == kMinMax || i < N) fw[i] = RF::load(rf, vf, soff(KIND == kMinMax ? t_hi - i : t_hi - 1 - i, f_row));
    if (i < N) gr[i] = RF::load(rg, vf, soff(t_hi - i, f_row));
  }
  if constexpr (kDecay) {
    float rv[V];
    RF::unpack(rate_raw, rv);
#pragma unroll
    for (int c = 0; c < V; ++c) nrate[c] = rv[c] * kNegLog2e;
    if (Q.log1p_gap) gap_l = log1pf(gap_l);  // after the input loads are issued
  }
  // The log2 decay y and the factor gamma = 2^y of time t_hi + 1 - i (i = 0
  // .. N) for each of the lane's channels, formed once here: phase 1 and
  // phase 3 both use them.
  constexpr int ND = kDecay ? N + 1 : 1;
  float ylog[ND][V], gamma_at[ND][V];
  if constexpr (kDecay) {
#pragma unroll
    for (int i = 0; i <= N; ++i) {
      const float gp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gap_l), i));
#pragma unroll
      for (int c = 0; c < V; ++c) {
        ylog[i][c] = nrate[c] * gp;
        gamma_at[i][c] = __builtin_amdgcn_exp2f(ylog[i][c]);
      }
    }
  }
  // The decay factor and log2 decay of step (t_hi + 1 - i) for each of the
  // lane's channels (the plain scan: 1 and 0).
  auto decay_at = [&](int i, float (&gam)[V], float (&y)[V]) {
#pragma unroll
    for (int c = 0; c < V; ++c) {
      gam[c] = 1.0f;
      y[c] = 0.0f;
    }
    if constexpr (kDecay) {
#pragma unroll
      for (int c = 0; c < V; ++c) {
        gam[c] = gamma_at[i][c];
        y[c] = ylog[i][c];
      }
    }
  };

  // The forward state before step 0 (for t = 0).
  float init_state[V];
#pragma unroll
  for (int c = 0; c < V; ++c)
    init_state[c] = (lane_on && Q.fwd0 != nullptr) ? Q.fwd0[size_t(tl.b) * P.D + d + c] : 0.0f;

  // The coefficient of the map of step n of the run (time t = t_hi - n):
  // that of the following step, a_{t+1} gamma_{t+1} (minGRU) or whether the
  // state passes step t+1 (MinMax), with its complement; 1 (complement 0)
  // for t = T - 1, where the gradient on the returned final state enters.
  auto step_coef = [&](int n, float (&coef)[V], float (&comp)[V]) {
    if (KIND == kMinGRU) {
      float kn[V], gam[V], yv[V];
      R::unpack(i0[n], kn);  // k_{t+1}
      decay_at(n, gam, yv);  // gamma_{t+1}
#pragma unroll
      for (int c = 0; c < V; ++c) {
        float z, a, om = 0.0f;
        sig_pair(kn[c], z, a);
        if constexpr (kDecay) {
          float unused;
          decay_factors(yv[c], unused, om);
        }
        coef[c] = a * gam[c];
        comp[c] = fmaf(a, om, z);  // 1 - a gamma = z + a (1 - gamma)
      }
    } else {
      float rn[V], sn[V], xn[V];
      R::unpack(i0[n], rn);   // r_{t+1}
      R::unpack(i1[n], sn);   // s_{t+1}
      RF::unpack(fw[n], xn);  // x_{t+1}
#pragma unroll
      for (int c = 0; c < V; ++c) {
        coef[c] = selection(rn[c], sn[c], xn[c]) == 0 ? 1.0f : 0.0f;
        comp[c] = 1.0f - coef[c];
      }
    }
    if (t_hi - n == T - 1) {
#pragma unroll
      for (int c = 0; c < V; ++c) {
        coef[c] = 1.0f;
        comp[c] = 0.0f;
      }
    }
  };

  // Phase 1: the maps G -> coef G + grad of the run's steps, composed with
  // their complements 1 - coef (see Affine).  The maps are not kept: phase 3
  // gets each step's coefficient as the one it forms for the step before
  // (bit for bit the same arithmetic), and the gradient is still loaded.
  typename Op::Agg agg[V];
#pragma unroll
  for (int c = 0; c < V; ++c) agg[c] = Op::identity();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float gv[V];
    RF::unpack(gr[n], gv);
    if constexpr (KIND == kMinGRU && kDecay) {
      // Step n's map: the gates' part of the following step (a, z), its
      // log2 decay y, and its whole coefficient a 2^y, formed as step_coef
      // forms it (phase 3 replays with that one); identity gates and no
      // decay at t = T - 1.
      float kn[V];
      R::unpack(i0[n], kn);  // k_{t+1}
      const bool last = t_hi - n == T - 1;
      if (n < nvalid) {
#pragma unroll
        for (int c = 0; c < V; ++c) {
          float z, a;
          sig_pair(kn[c], z, a);
          const DecayedStep st =
              last ? DecayedStep{1.0f, 0.0f, 0.0f, 1.0f, gv[c]}
                   : DecayedStep{a, z, ylog[n][c], a * gamma_at[n][c], gv[c]};
          agg[c] = Op::push(agg[c], st);
        }
      }
    } else {
      float coef[V], comp[V];
      step_coef(n, coef, comp);
      if (n < nvalid) {
#pragma unroll
        for (int c = 0; c < V; ++c) agg[c] = Op::push(agg[c], Affine{coef[c], comp[c], gv[c]});
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!lane_on) {
#pragma unroll
    for (int c = 0; c < V; ++c) agg[c] = Op::identity();
  }
#pragma unroll
  for (int c = 0; c < V; ++c) s_pre[wave][lane * V + c] = agg[c];
  __syncthreads();

  // Phase 2: the gradient entering the tile (decoupled look-back), its
  // fallback walking SB words per round trip (chosen per launch).
  resolve_tile<Op, W, Dc, 64 * W, SB>(P, tl, s_pre, s_win, s_hin);

  // Phase 3: replay to get G at every step and form the input gradients.
  // coef_next: the coefficient of the next step's map (the first from the
  // step after the run, then each step's own pass_or_a).
  float G[V], coef_next[V];
#pragma unroll
  for (int c = 0; c < V; ++c)
    G[c] = Op::apply(Op::map(s_pre[wave][lane * V + c]), s_hin[lane * V + c]);
  {
    float comp0[V];
    step_coef(0, coef_next, comp0);
  }
  const rsrc_t o0 = make_rsrc(Q.d0 + f_base, (f_end - f_base) * 4);
  const rsrc_t o1 = make_rsrc(Q.d1 + f_base, (f_end - f_base) * 4);
  uint32_t gate_lo = 0x3F800000u;  // smallest sigma(+-k_t) of the valid steps (bits)
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int64_t t = t_hi - n;
    {
      float gv[V];
      RF::unpack(gr[n], gv);
#pragma unroll
      for (int c = 0; c < V; ++c) G[c] = MinGRUOp::apply(Pair{coef_next[c], gv[c]}, G[c]);
    }
    float o0v[V], o1v[V], pass_or_a[V];
    if (KIND == kMinGRU) {
      float kt[V], pt[V], hp[V], gam[V], yv[V];
      R::unpack(i0[n + 1], kt);
      R::unpack(i1[n], pt);
      RF::unpack(fw[n], hp);
      decay_at(n + 1, gam, yv);  // gamma_t
#pragma unroll
      for (int c = 0; c < V; ++c) {
        const float h_prev = (t == 0 ? init_state[c] : hp[c]) * gam[c];
        float z, a, g, gs;
        sig_pair(kt[c], z, a);
        g_and_slope(pt[c], g, gs);
        if (n < nvalid) gate_lo = MinGRUOp::gate_floor(Affine{a, z, 0.0f}, gate_lo);
        // z a first, then the difference, then G: z a can sit at the bottom
        // of the normal range (|k| near 87), and G z a would go subnormal.
        o0v[c] = ((z * a) * (g - h_prev)) * G[c];
        o1v[c] = G[c] * z * gs;
        pass_or_a[c] = a * gam[c];
      }
    } else {
      float rt[V], st[V], xt[V];
      R::unpack(i0[n + 1], rt);
      R::unpack(i1[n + 1], st);
      RF::unpack(fw[n + 1], xt);
#pragma unroll
      for (int c = 0; c < V; ++c) {
        const float x_prev = t == 0 ? init_state[c] : xt[c];
        const int sel = selection(rt[c], st[c], x_prev);
        o0v[c] = sel == 1 ? G[c] : 0.0f;
        o1v[c] = sel == 2 ? G[c] : 0.0f;
        pass_or_a[c] = sel == 0 ? 1.0f : 0.0f;
      }
    }
#pragma unroll
    for (int c = 0; c < V; ++c) coef_next[c] = pass_or_a[c];
    if (lane_on && n < nvalid) {
      OutVec<V>::store(o0, vf, soff(t, f_row), o0v);
      OutVec<V>::store(o1, vf, soff(t, f_row), o1v);
      if (t == 0 && Q.dinit != nullptr) {
#pragma unroll
        for (int c = 0; c < V; ++c) Q.dinit[size_t(tl.b) * P.D + d + c] = pass_or_a[c] * G[c];
      }
    }
  }
  if (KIND == kMinGRU) {
    if (__builtin_amdgcn_ballot_w64(gate_lo < kMinNormalBits && lane_on) != 0 && lane == 0)
      __hip_atomic_fetch_or(P.status, kStatusGateRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Look-back fallback: with many chains a tile's walk is short and one word
// per round trip costs this register-bound kernel least; with few chains
// dozens of tiles of a chain are in flight together and walks are long, and
// four words per round trip pay off.  Measured (bf16, one process): B=8
// T=65536 D=1024 (64 chains) 1818 / 1826 / 1863 us with 1 / 2 / 4 words;
// 1 x 65536 x 1024 (8 chains) 314 / 297 / 285 us; 1 x 262144 x 256 (2
// chains) 644 / 618 / 520 us; at 16 chains all within 1.6%.
constexpr int64_t kFewChains = 16;

template <int KIND, typename TIn, int V, bool kDecay = false>
hipError_t launch_bwd_v(const BwdParams& Q, hipStream_t stream) {
  constexpr int N = kBwdElemsPerLane / V;
  static_assert(N + 1 <= 64, "one lane per gap of the run");
  const int64_t n_blocks = Q.core.n_chains * Q.core.n_tchunks;
  if (Q.core.n_chains < kFewChains)
    hipLaunchKernelGGL((scan_backward_kernel<KIND, TIn, V, N, kBwdWaves, kDecay, 4>),
                       dim3(uint32_t(n_blocks)), dim3(64 * kBwdWaves), 0, stream, Q);
  else
    hipLaunchKernelGGL((scan_backward_kernel<KIND, TIn, V, N, kBwdWaves, kDecay, 1>),
                       dim3(uint32_t(n_blocks)), dim3(64 * kBwdWaves), 0, stream, Q);
  return hipGetLastError();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

size_t scan_backward_workspace_bytes(int64_t B, int64_t T, int64_t D) {
  const int64_t min_tc = int64_t(kBwdWaves) * (kBwdElemsPerLane / 2);
  const int64_t n_tchunks = (T + min_tc - 1) / min_tc;
  return kHeaderBytes + align_up(size_t(n_tchunks) * size_t(B) * size_t(D) * 8, kAlign);
}

sr_status launch_scan_backward(const BackwardRequest& rq) {
  if (rq.B == 0 || rq.D == 0) return SR_OK;
  if (rq.T == 0) {
    // Nothing to scan: the gradient on the initial state is the one on the
    // returned final state (which then is the initial state itself).
    if (rq.dinit != nullptr) return launch_copy_or_zero(rq.dinit, rq.grad_last, rq.B * rq.D, rq.stream);
    return SR_OK;
  }
  const size_t esz = rq.in_dtype == SR_BF16 ? 2 : 4;
  const bool v2 = rq.D % 2 == 0 && rq.ld_in % 2 == 0 && aligned(rq.in0, 2 * esz) &&
                  aligned(rq.in1, 2 * esz) && aligned(rq.fwd, 8) && aligned(rq.grad, 8) &&
                  aligned(rq.d0, 8) && aligned(rq.d1, 8) &&
                  (rq.D + 127) / 128 * 128 <= (rq.D + 63) / 64 * 64;
  const int V = v2 ? 2 : 1;
  const int64_t Dc = 64 * V, Tc = int64_t(kBwdWaves) * (kBwdElemsPerLane / V);
  BwdParams Q{};
  ScanParams& P = Q.core;
  P.init = rq.grad_last;
  P.B = rq.B;
  P.T = rq.T;
  P.D = rq.D;
  P.n_dtiles = (rq.D + Dc - 1) / Dc;
  P.n_tchunks = (rq.T + Tc - 1) / Tc;
  P.n_chains = rq.B * P.n_dtiles;
  if (P.n_chains * P.n_tchunks * (64 * kBwdWaves) > int64_t(0xFFFFFFFFu))
    return fail(SR_ERR_UNSUPPORTED, "backward scan of %lld tiles exceeds one launch's grid",
                (long long)(P.n_chains * P.n_tchunks));
  char* ws = static_cast<char*>(rq.workspace);
  P.counter = reinterpret_cast<uint32_t*>(ws);
  P.status = reinterpret_cast<uint32_t*>(ws) + 1;
  P.state = reinterpret_cast<uint64_t*>(ws + kHeaderBytes);
  P.window = kWindowTiles;
  P.spin_limit = lookback_spin_limit();
  Q.in0 = rq.in0;
  Q.in1 = rq.in1;
  Q.ld_in = rq.ld_in;
  Q.fwd = rq.fwd;
  Q.fwd0 = rq.fwd0;
  Q.grad = rq.grad;
  Q.d0 = rq.d0;
  Q.d1 = rq.d1;
  Q.dinit = rq.dinit;
  Q.rate = rq.decay_rate;
  Q.gap = rq.delta_t;
  Q.log1p_gap = rq.log1p_delta;
  const bool decay = rq.decay_rate != nullptr;
  if (decay && rq.op != ScanOp::kMinGRU)
    return fail(SR_ERR_UNSUPPORTED, "time decay applies to the minGRU scan only");
  sr_status st = reset_workspace(ws, kHeaderBytes + size_t(P.n_tchunks) * size_t(P.B) * size_t(P.D) * 8,
                                 rq.stream);
  if (st != SR_OK) return st;
  hipError_t err;
  if (rq.op == ScanOp::kMinMax)
    err = V == 2 ? launch_bwd_v<kMinMax, float, 2>(Q, rq.stream) : launch_bwd_v<kMinMax, float, 1>(Q, rq.stream);
  else if (decay && rq.in_dtype == SR_BF16)
    err = V == 2 ? launch_bwd_v<kMinGRU, uint16_t, 2, true>(Q, rq.stream)
                 : launch_bwd_v<kMinGRU, uint16_t, 1, true>(Q, rq.stream);
  else if (decay)
    err = V == 2 ? launch_bwd_v<kMinGRU, float, 2, true>(Q, rq.stream)
                 : launch_bwd_v<kMinGRU, float, 1, true>(Q, rq.stream);
  else if (rq.in_dtype == SR_BF16)
    err = V == 2 ? launch_bwd_v<kMinGRU, uint16_t, 2>(Q, rq.stream)
                 : launch_bwd_v<kMinGRU, uint16_t, 1>(Q, rq.stream);
  else
    err = V == 2 ? launch_bwd_v<kMinGRU, float, 2>(Q, rq.stream) : launch_bwd_v<kMinGRU, float, 1>(Q, rq.stream);
  if (err != hipSuccess) return fail(SR_ERR_HIP, "backward scan launch: %s", hipGetErrorString(err));
  return SR_OK;
}

}  // namespace sr
