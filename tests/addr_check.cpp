// Host check of the scan kernels' buffer addressing (scan_addr.hpp): for
// every tile, wave, lane and step of a sweep of shapes, the element each load
// and store touches lies inside its tensor, and the valid ones are exactly the
// intended (batch row, step, channel).  Compiled as HIP (the helpers are
// host + device functions) and run on the host only; prints the number of
// accesses checked and "ok", or the first violation and exit status 1.
// Built with -DPLANT_UNCLAMPED_ROWS it checks an unclamped forward row offset
// instead (a planted mistake the check must report).
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "scan_addr.hpp"

using namespace sr::addr;

static long long g_checks = 0;

static void fail(const char* what, long long B, long long T, long long D, long long ld, int V,
                 long long tile, int w, int lane, int n, long long got, long long lo, long long hi) {
  std::printf("VIOLATION %s: B=%lld T=%lld D=%lld ld=%lld V=%d tile=%lld wave=%d lane=%d n=%d "
              "element=%lld allowed [%lld, %lld]\n",
              what, B, T, D, ld, V, tile, w, lane, n, got, lo, hi);
  std::exit(1);
}

// The forward scan kernel: W waves of N = E / V steps per lane.
static void check_forward(int64_t B, int64_t T, int64_t D, int64_t ld, int V, int W, int E) {
  const int N = E / V;
  const int64_t Dc = 64 * V, Tc = int64_t(W) * N;
  const int64_t n_dtiles = (D + Dc - 1) / Dc, n_tchunks = (T + Tc - 1) / Tc;
  const int64_t in_last = (B * T - 1) * ld + D - 1;  // last element of k / p
  for (int64_t b = 0; b < B; ++b)
    for (int64_t dt = 0; dt < n_dtiles; ++dt)
      for (int64_t tc = 0; tc < n_tchunks; ++tc)
        for (int w = 0; w < W; ++w) {
          const int64_t d0 = dt * Dc, tw = tc * Tc + int64_t(w) * N;
          for (int lane = 0; lane < 64; ++lane) {
            const FwdRun r = fwd_run(T, D, V, N, tw, d0, lane);
            const int64_t d = d0 + int64_t(lane) * V;
            const int64_t base = (b * T + r.t_base) * ld + d0;  // descriptor base
            if (r.lane_ch < 0) fail("negative lane offset", B, T, D, ld, V, tc, w, lane, -1, r.lane_ch, 0, 0);
            for (int n = 0; n < N; ++n) {
#ifdef PLANT_UNCLAMPED_ROWS
              // The planted mistake: step n read at row n with no clamp.
              const int row = n;
#else
              const int row = fwd_row(r, n);
#endif
              if (row < 0) fail("negative row offset", B, T, D, ld, V, tc, w, lane, n, row, 0, 0);
              for (int c = 0; c < V; ++c) {
                const int64_t e = base + int64_t(row) * ld + r.lane_ch + c;
                ++g_checks;
                if (e < 0 || e > in_last) fail("forward load", B, T, D, ld, V, tc, w, lane, n, e, 0, in_last);
                if (n < r.nvalid && d < D && e != (b * T + tw + n) * ld + d + c)
                  fail("forward load (wrong element)", B, T, D, ld, V, tc, w, lane, n, e,
                       (b * T + tw + n) * ld + d + c, (b * T + tw + n) * ld + d + c);
              }
              // Stores: valid steps, lanes inside D, rows of D elements.
              if (n < r.nvalid && d < D) {
                for (int c = 0; c < V; ++c) {
                  const int64_t e = (b * T + r.t_base + n) * D + d0 + int64_t(lane) * V + c;
                  ++g_checks;
                  if (e < 0 || e > B * T * D - 1 || e != (b * T + tw + n) * D + d + c)
                    fail("forward store", B, T, D, ld, V, tc, w, lane, n, e, 0, B * T * D - 1);
                }
              }
            }
          }
        }
}

// The backward scan kernel: W waves of N = E / V steps per lane, reverse time.
static void check_backward(int64_t B, int64_t T, int64_t D, int64_t ld, int V, int W, int E) {
  const int N = E / V;
  const int64_t Dc = 64 * V, Tc = int64_t(W) * N;
  const int64_t n_dtiles = (D + Dc - 1) / Dc, n_tchunks = (T + Tc - 1) / Tc;
  const int64_t in_last = (B * T - 1) * ld + D - 1;  // k / p (or r / s)
  const int64_t f_last = B * T * D - 1;              // h, dh, dk, dp
  for (int64_t b = 0; b < B; ++b)
    for (int64_t dt = 0; dt < n_dtiles; ++dt)
      for (int64_t tc = 0; tc < n_tchunks; ++tc)
        for (int w = 0; w < W; ++w) {
          const int64_t d0 = dt * Dc;
          for (int lane = 0; lane < 64; ++lane) {
            const BwdRun r = bwd_run(T, D, V, N, tc, w, W, d0, lane);
            const int64_t d = d0 + int64_t(lane) * V;
            const int64_t in_base = (b * T + r.rbase) * ld + d0;
            const int64_t f_base = (b * T + r.rbase) * D + d0;
            if (r.rbase < 0 || r.rbase > T - 1)
              fail("descriptor base row", B, T, D, ld, V, tc, w, lane, -1, r.rbase, 0, T - 1);
            // Rows the kernel reads: t_hi + 1 - i (i = 0..N) and t_hi - 1 - i,
            // t_hi - i (i = 0..N-1): all of t_hi - N .. t_hi + 1.
            for (int64_t row = r.t_hi - N; row <= r.t_hi + 1; ++row) {
              const int64_t ro = bwd_row(r, T, row);
              if (ro < 0) fail("negative row offset", B, T, D, ld, V, tc, w, lane, int(row), ro, 0, 0);
              for (int c = 0; c < V; ++c) {
                const int64_t ei = in_base + ro * ld + r.lane_ch + c;
                const int64_t ef = f_base + ro * D + r.lane_ch + c;
                g_checks += 2;
                if (ei < 0 || ei > in_last) fail("backward input load", B, T, D, ld, V, tc, w, lane, int(row), ei, 0, in_last);
                if (ef < 0 || ef > f_last) fail("backward state load", B, T, D, ld, V, tc, w, lane, int(row), ef, 0, f_last);
                if (row >= 0 && row < T && d < D) {
                  if (ei != (b * T + row) * ld + d + c)
                    fail("backward input load (wrong element)", B, T, D, ld, V, tc, w, lane, int(row), ei, 0, 0);
                  if (ef != (b * T + row) * D + d + c)
                    fail("backward state load (wrong element)", B, T, D, ld, V, tc, w, lane, int(row), ef, 0, 0);
                }
              }
            }
            // Stores: steps t_hi - n for n < nvalid, lanes inside D.
            for (int n = 0; n < r.nvalid && d < D; ++n) {
              const int64_t t = r.t_hi - n;
              for (int c = 0; c < V; ++c) {
                const int64_t e = f_base + bwd_row(r, T, t) * D + r.lane_ch + c;
                ++g_checks;
                if (e != (b * T + t) * D + d + c || e < 0 || e > f_last)
                  fail("backward store", B, T, D, ld, V, tc, w, lane, n, e, 0, f_last);
              }
            }
          }
        }
}

int main() {
  // The kernels' own geometry (scan_addr.hpp).
  const int64_t Ts[] = {1, 2, 5, 19, 20, 21, 23, 24, 25, 143, 144, 145, 239, 240, 241, 287, 288, 289, 300, 1000};
  const int64_t Ds[] = {1, 2, 3, 16, 63, 64, 65, 127, 128, 130, 192, 200, 257};
  const int64_t Bs[] = {1, 2, 3};
  for (int64_t B : Bs)
    for (int64_t T : Ts)
      for (int64_t D : Ds)
        for (int64_t extra : {int64_t(0), int64_t(1), int64_t(64)})
          for (int V : {1, 2}) {
            const int64_t ld = D + extra;
            if (V == 2 && (D % 2 || ld % 2)) continue;
            check_forward(B, T, D, ld, V, kFwdWaves, kFwdElemsPerLane);
            if (V == 1) check_forward(B, T, D, ld, V, kFwdWaves, kFwdElemsPerLaneShort);
            check_backward(B, T, D, ld, V, kBwdWaves, kBwdElemsPerLane);
          }
  std::printf("forward and backward addressing: %lld accesses checked, all inside their tensors\n",
              g_checks);
  std::printf("ok\n");
  return 0;
}
