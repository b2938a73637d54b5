// Where one wave of a scan kernel reads and writes: the row (time step) and
// channel clamps that keep every buffer access inside its tensor.
//
// A wave addresses its rows through a buffer descriptor with a per-lane byte
// offset (the channel) and a per-row scalar offset.  The descriptor's range
// check covers the per-lane offset only, so these clamps -- not the range
// check -- keep the accesses in bounds: rows past the run's last valid step
// re-read that step, a run wholly outside the sequence reads a row that
// exists, and lanes past D re-read channel D - V.  Maps built from re-read
// values are replaced by the identity or never stored.
//
// Host and device: the kernels call these, and a host program checks every
// access they imply against the tensors' extents over many shapes.
#pragma once

#include <cstdint>

namespace sr {
namespace addr {

// Tile geometry of the two scan kernels: waves per workgroup (stacked along
// T) and maps each lane keeps in registers (steps x channels per lane).
constexpr int kFwdWaves = 12;
constexpr int kFwdElemsPerLane = 24;
// The MinMax scan's shorter tiles (one channel per lane, 20 steps per lane)
// for launches with enough chains.
constexpr int kFwdElemsPerLaneShort = 20;
constexpr int kBwdWaves = 8;
constexpr int kBwdElemsPerLane = 16;

// The forward scan: wave w of tile tchunk reads steps tw .. tw + N - 1,
// tw = tchunk * (W * N) + w * N, of batch row b, channels d0 + lane*V ..
struct FwdRun {
  int64_t t_base;  // step of the descriptor's first row: tw, or T - 1 past the end
  int nvalid;      // steps of the run inside the sequence
  int n_last;      // highest row (relative to t_base) any step reads
  int64_t lane_ch; // the lane's first channel, relative to d0
};

__host__ __device__ inline FwdRun fwd_run(int64_t T, int64_t D, int V, int N, int64_t tw,
                                          int64_t d0, int lane) {
  FwdRun r;
  const int64_t rem = T - tw;
  r.nvalid = rem <= 0 ? 0 : (rem >= N ? N : int(rem));
  r.t_base = tw < T ? tw : T - 1;
  r.n_last = r.nvalid > 0 ? r.nvalid - 1 : 0;
  const int64_t d = d0 + int64_t(lane) * V;
  r.lane_ch = (d < D - V ? d : D - V) - d0;
  return r;
}

// Row read by step n of the run, relative to t_base.
__host__ __device__ inline int fwd_row(const FwdRun& r, int n) { return n < r.n_last ? n : r.n_last; }

// The backward scan runs in reverse time: wave w of tile tchunk handles steps
// t_hi, t_hi - 1, .. t_hi - N + 1, t_hi = T - 1 - (tchunk * (W * N) + w * N),
// and reads rows t_hi + 1 .. t_hi - N (the neighbours of its steps), each
// clamped into [0, T) and addressed from rbase, the lowest row read.
struct BwdRun {
  int64_t t_hi;
  int nvalid;
  int64_t rbase;
  int64_t lane_ch;
};

__host__ __device__ inline BwdRun bwd_run(int64_t T, int64_t D, int V, int N, int64_t tchunk,
                                          int w, int W, int64_t d0, int lane) {
  BwdRun r;
  r.t_hi = T - 1 - (tchunk * (int64_t(W) * N) + int64_t(w) * N);
  r.nvalid = r.t_hi < 0 ? 0 : (r.t_hi + 1 >= N ? N : int(r.t_hi + 1));
  r.rbase = r.t_hi - N > 0 ? r.t_hi - N : 0;
  const int64_t d = d0 + int64_t(lane) * V;
  r.lane_ch = (d < D - V ? d : D - V) - d0;
  return r;
}

// Row offset (relative to rbase) at which time step `row` is read.
__host__ __device__ inline int64_t bwd_row(const BwdRun& r, int64_t T, int64_t row) {
  const int64_t c = row < 0 ? 0 : (row > T - 1 ? T - 1 : row);
  return c - r.rbase;
}

}  // namespace addr
}  // namespace sr
