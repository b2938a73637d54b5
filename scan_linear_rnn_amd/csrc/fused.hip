// Fused input projection and minGRU scan for gfx950: [k | p] = x W_in is
// computed a tile at a time on the matrix cores and scanned in the same
// workgroup, so k and p never travel to HBM and back (16 bytes per element
// in fp32).  The minGRU profile's parallel mode, with the layer's projection
// feeding the scan directly.
//
// A workgroup owns 256 consecutive steps of one batch row and 64 channels:
// the 256 x 128 MFMA tile of gemm_tile.hpp (8 waves) with paired columns, so
// lane (kl, ml) of wave (wm, wn) holds k and p of channel 32*wn + ml for the
// 32 rows wm*64 + 32*i + 8*q + 4*kl + j (i, j, q in 0..1, 0..3, 0..3).  The scan
// of the tile runs on that layout:
//   1. each lane turns its 32 (k, p) into maps, in the accumulator
//      registers, and composes each run of 4 consecutive rows (8 runs);
//   2. along T the runs of a wave alternate between lane ml and lane ml + 32
//      (run 2n + kl of the wave's 64 rows is run n of lane kl), so the two
//      lanes swap their runs and both walk the 16 runs in order, each keeping
//      the prefix that enters its own runs;
//   3. the four wave rows along T (wm = 0..3) meet in LDS and the tile is
//      linked to its predecessors along T by the engine's windowed look-back
//      (scan_engine.hpp), exactly as in the stand-alone scan;
//   4. each lane replays its maps from the state entering its runs and stores
//      h.
// Tiles take tickets in execution order, so a tile only waits on tiles that
// are already running (see scan.hip).  Time decay (the minGRU tutorials'
// "Adding time decay" step) scales each map's coefficient by
// exp(-rate_d * gap_t) as in the stand-alone scan.

#include "gemm_tile.hpp"
#include "scan_engine.hpp"

namespace sr {
namespace {

using namespace gt;
using namespace eng;

constexpr int kTileT = 256;    // steps per tile (the 256-row GEMM tile)
constexpr int kTileD = BN / 2; // channels per tile (paired k / p columns)

struct FusedParams {
  GemmParams g;  // A = x [B*T, D_in], Bm = W_in [D_in, 2*D_h], K = D_in
  ScanParams s;  // look-back context; out = h [B,T,D_h], D = D_h
};

// Register budget: 4 waves per SIMD (two workgroups per CU), as the plain
// 256-row GEMM runs; measured 17.3 ms against 19.1 ms at the compiler's own
// choice (2 waves per SIMD) on a 131072 x 4096 x 2048 projection (B=256,
// T=512, D=2048).  Within it the epilogue keeps the per-row maps in the
// accumulators, the runs' entry prefixes in the K loop's staging LDS and
// its row tests relative to the lane's first row: 121 VGPRs without decay,
// no spills (the decayed variant spills 25 dwords once per tile).  Before,
// 65 dwords (prefixes and 64-bit row indices) spilled and were reloaded per
// tile, at no measurable cost (16.66 vs 16.69 ms on that projection).
template <bool kDecay, bool kFull>
__global__ __launch_bounds__(2 * kTileT) __attribute__((amdgpu_waves_per_eu(4)))
void fused_proj_scan_kernel(const FusedParams F) {
  __shared__ float As[2][BK][kTileT + PAD];
  __shared__ float Bs[2][BK][BN + PAD];
  __shared__ uint32_t s_ticket;
  __shared__ Affine s_pre[kTileT / 64][kTileD];
  __shared__ uint64_t s_win[kWindowTiles][kTileD];
  __shared__ float s_hin[kTileD];
  __shared__ float s_gap[kTileT];

  const ScanParams& P = F.s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int kl = lane >> 5, ml = lane & 31;
  const uint32_t ticket = take_ticket(P, &s_ticket);
  const Tile tl = decode_ticket(P, ticket, kTileD);
  const int64_t t0 = tl.tchunk * kTileT;
  const int64_t rows = P.T - t0 < kTileT ? P.T - t0 : kTileT;
  // Row tests in the epilogue compare the row's offset within the lane's
  // runs (a constant there) with these per-lane bounds, so that no per-row
  // index is kept across the look-back.
  const int row_base = wm * 64 + (lane >> 5) * 4;  // the lane's first row in the tile
  const int rows_rel = int(rows) - row_base;      // rows [0, rows) are inside the sequence
  const int c = wn * 32 + ml;  // channel within the tile
  const int64_t d = tl.d0 + c;
  const bool chan_ok = d < P.D;

  float rate = 0.0f, nrate = 0.0f;
  if constexpr (kDecay) {
    if (tid < kTileT) {
      float gp = tid < rows ? P.gap[tl.b * P.T + t0 + tid] : 0.0f;
      if (P.log1p_gap) gp = log1pf(gp);
      s_gap[tid] = gp;  // published by the K loop's barriers
    }
    rate = chan_ok ? P.rate[d] : 0.0f;
    nrate = rate * kNegLog2e;
  }

  floatx16 acc[2][2];
  tile_mainloop<kStep, kTileT, kFull>(F.g, tl.b * P.T + t0, rows, tl.d0, 0, F.g.K, As, Bs, acc);

  // 1. Maps in place of the sums (set 0 <- coefficient, set 1 <- offset);
  // rows past T become the identity.  Each run of 4 rows (run n = (i, q),
  // n = 4*i + q) is composed as its maps are formed, with the complements
  // (see Affine), which are not kept per row.
  bool sat = false;
  uint32_t gate_lo = 0x3F800000u;  // bits of 1.0f
  Affine mine[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int i = n / 4, q = n % 4;
    Affine run_n = MinGRUOp::identity();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * q + j;
      const int lr = wm * 64 + i * 32 + q * 8 + kl * 4 + j;
      const bool in_seq = i * 32 + q * 8 + j < rows_rel;  // lr < rows
      Affine m = MinGRUOp::element(acc[i][0][r], acc[i][1][r]);
      if (in_seq) gate_lo = MinGRUOp::gate_floor(m, gate_lo);
      if constexpr (kDecay) {
        const float gp = s_gap[lr];
        float gamma, om;
        decay_factors(nrate * gp, gamma, om);
        m = MinGRUOp::decayed(m, gamma, om);
        sat = sat || (rate * gp > kDecayClamp);
      }
      if (!in_seq) m = MinGRUOp::identity();
      acc[i][0][r] = m.a;
      acc[i][1][r] = m.b;
      run_n = MinGRUOp::push(run_n, m);
    }
    mine[n] = run_n;
  }
  if constexpr (kDecay) {
    if (P.saturated != nullptr && __builtin_amdgcn_ballot_w64(sat) != 0 && lane == 0)
      __hip_atomic_fetch_or(P.saturated, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (__builtin_amdgcn_ballot_w64(gate_lo < kMinNormalBits && chan_ok) != 0 && lane == 0)
    __hip_atomic_fetch_or(P.status, kStatusGateRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // 2. The partner lane's runs (lane ^ 32), then the prefix over the wave's
  // 16 runs in T order: run 2n is lane kl = 0's run n, run 2n + 1 lane 1's.
  // The prefixes entering the lane's runs wait for step 4 in the staging LDS
  // of the K loop, which is free now (in registers they would spill).
  float* const pre = &As[0][0][0];  // [8][2][512]: run n's (u, v) of thread tid
  static_assert(8 * 2 * 2 * kTileT <= 2 * BK * (kTileT + PAD), "prefixes fit the staging LDS");
  auto put_pre = [&](int n, Pair m) {
    pre[(2 * n) * (2 * kTileT) + tid] = m.u;
    pre[(2 * n + 1) * (2 * kTileT) + tid] = m.v;
  };
  Affine run = MinGRUOp::identity();
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const Affine other = {__shfl_xor(mine[n].a, 32), __shfl_xor(mine[n].c, 32),
                          __shfl_xor(mine[n].b, 32)};
    const Affine even = kl == 0 ? mine[n] : other;
    const Affine odd = kl == 0 ? other : mine[n];
    if (kl == 0) put_pre(n, MinGRUOp::map(run));
    run = MinGRUOp::compose(run, even);
    if (kl == 1) put_pre(n, MinGRUOp::map(run));
    run = MinGRUOp::compose(run, odd);
  }
  // 3. Wave rows along T, then the look-back across tiles.
  if (kl == 0) s_pre[wm][c] = run;
  __syncthreads();
  resolve_tile<MinGRUOp, kTileT / 64, kTileD, 2 * kTileT, 2>(P, tl, s_pre, s_win, s_hin);

  // 4. Replay and store.  One buffer descriptor over the tile's rows of h:
  // the lane's row and channel in the vector offset, the step's row within
  // the lane's runs in the (wave-uniform) scalar offset, so that no 64-bit
  // address per row is formed and kept across the look-back (the compiler
  // had spilled 32 of them).  Rows past T are skipped explicitly: the range
  // check does not cover the scalar offset.
  const float h_wave = MinGRUOp::apply(MinGRUOp::map(s_pre[wm][c]), s_hin[c]);
  const int64_t row_bytes = P.D * 4;
  const rsrc_t ro = make_rsrc(P.out + (tl.b * P.T + t0) * P.D, rows * row_bytes);
  const int vo = int((wm * 64 + kl * 4) * row_bytes + d * 4);
  // The row that is step T - 1 (its state is h_T), relative to row_base, or
  // -1 (no row of the lane's runs).
  const int last_rel =
      (P.last != nullptr && P.T - 1 - t0 < kTileT) ? int(P.T - 1 - t0) - row_base : -1;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int i = n / 4, q = n % 4;
    const Pair pn = {pre[(2 * n) * (2 * kTileT) + tid], pre[(2 * n + 1) * (2 * kTileT) + tid]};
    float h = MinGRUOp::apply(pn, h_wave);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rel = i * 32 + q * 8 + j;  // the row is row_base + rel
      h = MinGRUOp::apply(Pair{acc[i][0][4 * q + j], acc[i][1][4 * q + j]}, h);
      if (chan_ok && rel < rows_rel) {
        // Default cache policy (not streaming): the output projection that
        // usually follows reads h, and mid-sized h stays in the Infinity Cache.
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(h), ro, vo, int(rel * row_bytes), 0);
        if (rel == last_rel) P.last[tl.b * P.D + d] = h;
      }
    }
  }
}

}  // namespace

bool fused_forward_applies(int64_t B, int64_t T, int64_t D_h) {
  // Worth it when the tiles alone fill the part several times over; smaller
  // problems keep the split-K projection, which spreads its K loop over more
  // workgroups.
  if (B <= 0 || T <= 0 || D_h <= 0) return false;
  // A tile's rows of h are addressed with 32-bit byte offsets.
  if (int64_t(kTileT) * D_h * 4 > int64_t(0x7FFFFFFF)) return false;
  const int64_t tiles = B * ((D_h + kTileD - 1) / kTileD) * ((T + kTileT - 1) / kTileT);
  return tiles >= 512 && tiles * 2 * kTileT <= int64_t(0xFFFFFFFFu);
}

size_t fused_workspace_bytes(int64_t B, int64_t T, int64_t D_h) {
  const int64_t n_tchunks = (T + kTileT - 1) / kTileT;
  return eng::kHeaderBytes + align_up(size_t(n_tchunks) * size_t(B) * size_t(D_h) * 8, kAlign);
}

sr_status launch_fused_forward(const FusedRequest& rq) {
  // fused_forward_applies has checked the grid; nothing else can fail before
  // the launch.
  if (rq.check_only) return SR_OK;
  FusedParams F{};
  GemmParams& g = F.g;
  g.M = rq.B * rq.T;
  g.N = 2 * rq.D_h;
  g.K = rq.D_in;
  g.A = rq.x;
  g.lda = rq.D_in;
  g.Bm = rq.W_in;
  g.ldb = 2 * rq.D_h;
  g.D_h = rq.D_h;
  ScanParams& P = F.s;
  P.out = rq.h;
  P.init = rq.h0;
  P.last = rq.h_last;
  P.B = rq.B;
  P.T = rq.T;
  P.D = rq.D_h;
  P.n_dtiles = (rq.D_h + kTileD - 1) / kTileD;
  P.n_tchunks = (rq.T + kTileT - 1) / kTileT;
  P.n_chains = rq.B * P.n_dtiles;
  char* ws = static_cast<char*>(rq.workspace);
  P.counter = reinterpret_cast<uint32_t*>(ws);
  P.status = reinterpret_cast<uint32_t*>(ws) + 1;
  P.state = reinterpret_cast<uint64_t*>(ws + eng::kHeaderBytes);
  P.window = eng::kWindowTiles;
  P.spin_limit = lookback_spin_limit();
  P.rate = rq.decay_rate;
  P.gap = rq.delta_t;
  P.log1p_gap = rq.log1p_delta;
  P.saturated = rq.saturated;
  const int64_t tiles = P.n_chains * P.n_tchunks;
  const size_t used = eng::kHeaderBytes + size_t(P.n_tchunks) * size_t(rq.B) * size_t(rq.D_h) * 8;
  sr_status st = eng::reset_workspace(ws, used, rq.stream);
  if (st != SR_OK) return st;
  // Every tile full (whole 256-step tiles, whole channel tiles, K a
  // positive multiple of 16) with 16-byte operands: the K loop needs no range
  // tests.  (It loads its first K step unconditionally, so K = 0, where x may
  // be NULL, takes the checked loop.)
  const auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool full = rq.D_in > 0 && rq.T % kTileT == 0 && rq.D_h % kTileD == 0 && rq.D_in % BK == 0 &&
                    rq.D_in % 4 == 0 && al16(rq.x) && al16(rq.W_in);
  const dim3 grid{uint32_t(tiles)}, block{2 * kTileT};
  if (rq.decay_rate != nullptr && full)
    hipLaunchKernelGGL((fused_proj_scan_kernel<true, true>), grid, block, 0, rq.stream, F);
  else if (rq.decay_rate != nullptr)
    hipLaunchKernelGGL((fused_proj_scan_kernel<true, false>), grid, block, 0, rq.stream, F);
  else if (full)
    hipLaunchKernelGGL((fused_proj_scan_kernel<false, true>), grid, block, 0, rq.stream, F);
  else
    hipLaunchKernelGGL((fused_proj_scan_kernel<false, false>), grid, block, 0, rq.stream, F);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SR_ERR_HIP, "fused projection + scan launch: %s", hipGetErrorString(err));
  return SR_OK;
}

}  // namespace sr
