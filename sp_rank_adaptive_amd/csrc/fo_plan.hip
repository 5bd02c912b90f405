// Schedule model for the chunked AG-GEMM (host only).
//
// FlashOverlap's scheduler predicts when each piece lands and how long its
// sub-task runs, and orders the work so that no compute waits on the tail
// (euno.news "Methodology" step 3: an analytical model of the dependency
// graph; gist.science technical summary §2: work on incoming data first, the
// slice already present last).  This model covers the two decisions the
// persistent AG kernel leaves to its caller:
//  - order: peers by expected landing time, the local chunk last;
//  - split: how many ways the chunk that lands last is split along k.
// Splitting that chunk lets every idle workgroup share its tiles, which pays
// when the GPU is idle at the last landing (slow links); when every workgroup
// is still busy with earlier chunks (fast links), the split units queue behind
// them and the extra partial traffic only adds time.
//
// The model simulates the kernel's ready-first claims.  One simulated
// workgroup per launch workgroup takes, whenever it is free, the first unit
// in priority order whose chunk has landed; the units of a split chunk are
// followed by its reduce units.  A running unit's rate falls linearly from
// what one workgroup reaches alone to an equal share of the whole GPU's rate
// as more workgroups run (rates are recomputed at every event).  The
// constants are calibrated on MI355X measurements of the TP=8 MLP
// up-projection share (4096 x 1792 x 4096 in 8 chunks): about 900 TFLOP/s
// with every workgroup busy, one chunk alone about 1.8 times faster per
// workgroup, and about 5 us from a flag store to the first claim of that
// chunk.  Over ring arrivals at 50, 153, 400 and 1000 GB/s per link (peers
// starting with the consumer kernel) its completions came within 3% of the
// measured ones, and its split was the best measured one or within 2% of it;
// on the long-sequence QKV share (16384 x 1280 x 8192 in 16 chunks, 50 GB/s)
// it also picks the best measured split.
#include "fo_internal.hpp"

#include <algorithm>
#include <vector>

namespace fo {
namespace {

constexpr int kPlanMaxSplit = 8;
constexpr double kFlagLatencyNs = 5000.0;       // flag store -> first claim
constexpr double kDefaultTflops = 900.0;        // every workgroup busy
constexpr double kAloneSpeedup = 1.8;           // one workgroup alone vs shared
constexpr double kHbmBytesPerNs = 5000.0;       // 5 TB/s, shared
constexpr double kWgBytesPerNsMax = 60.0;       // one workgroup alone
constexpr double kUnitFixedNs = 1500.0;         // claim and bookkeeping per unit
constexpr double kClaimQueueNs = 10.0;          // per workgroup claiming at the same instant
constexpr double kSplitMarginNs = 500.0;        // a larger split must win by more

struct Sim {
  int grid = 0, tiles = 0, kt_total = 0;
  int64_t bm = 0, bn = 0, k = 0;
  double rate_all = 0;   // FLOP per ns with every workgroup busy
  double rate_one = 0;   // FLOP per ns of one workgroup alone
};

// Split factor the launch actually uses for a requested one (every split must
// own at least one 64-wide k stage).
int effective_split(int sk, int kt_total) {
  if (sk > kt_total) sk = kt_total;
  int kt_per = (kt_total + sk - 1) / sk;
  while (sk > 1 && (int64_t)(sk - 1) * kt_per >= kt_total) {
    --sk;
    kt_per = (kt_total + sk - 1) / sk;
  }
  return sk < 1 ? 1 : sk;
}

// Predicted completion (ns after t0) of one AG launch: an event-driven
// simulation with processor sharing.  A running unit holds an amount of work
// measured in nanoseconds of a workgroup running alone; while `active` units
// run, each advances at speed min(1, share / alone) where share is the
// whole-GPU rate divided among them.  Claims are made by idle workgroups at
// each event in priority order; a claim costs a fixed time plus a term that
// grows with the number of workgroups claiming at that instant (they queue on
// the same claim counters).  A reduce unit waits, holding its workgroup, until
// every split of its tile has finished.
double simulate(const Sim &s, int R, const int *order, const double *avail, const int *split) {
  struct Chunk {
    int units = 0, next = 0, red_units = 0, red_next = 0, S = 1;
    std::vector<int> tile_left;          // splits of the tile still running
    std::vector<double> tile_done;       // when the last split finished (-1: not yet)
    std::vector<int> ready_tiles;        // tiles in the order their splits finished
  };
  enum { IDLE, RUN, WAIT_TILE, GONE };
  struct Wg {
    int state = IDLE;
    double work = 0;                     // ns at the alone rate
    int chunk = -1, tile = -1, red = 0;
  };
  std::vector<Chunk> ch(R);
  for (int c = 0; c < R; ++c) {
    Chunk &q = ch[c];
    q.S = split[c];
    q.units = s.tiles * q.S;
    if (q.S > 1) {
      q.red_units = s.tiles * RED_SLICES;
      q.tile_left.assign(s.tiles, q.S);
      q.tile_done.assign(s.tiles, -1.0);
    }
  }
  const double alone_flop = s.rate_one;                  // FLOP per ns
  const double alone_bytes = kWgBytesPerNsMax;           // bytes per ns
  const double tile_out = (double)s.bm * (double)s.bn * 4.0;
  std::vector<Wg> wg(s.grid);
  double t = 0, done = 0;
  int left_total = 0;
  for (int c = 0; c < R; ++c) left_total += ch[c].units + ch[c].red_units;
  while (left_total > 0) {
    // claims by idle workgroups: those that find work queue on the counters
    int idle = 0, claimable = 0;
    for (const Wg &g : wg) idle += g.state == IDLE;
    for (int c = 0; c < R; ++c)
      if (avail[c] <= t) claimable += (ch[c].units - ch[c].next) + (ch[c].red_units - ch[c].red_next);
    const double claim_ns = kUnitFixedNs + kClaimQueueNs * std::min(idle, claimable);
    double next_avail = -1;
    bool any_unclaimed = false;
    for (Wg &g : wg) {
      if (g.state != IDLE) continue;
      bool took = false;
      for (int pi = 0; pi < R && !took; ++pi) {
        const int c = order[pi];
        Chunk &q = ch[c];
        const bool gemm_left = q.next < q.units;
        const bool red_left = !gemm_left && q.red_next < q.red_units;
        if (!gemm_left && !red_left) continue;
        any_unclaimed = true;
        if (avail[c] > t) {
          if (next_avail < 0 || avail[c] < next_avail) next_avail = avail[c];
          continue;
        }
        g.chunk = c;
        if (gemm_left) {
          const int u = q.next++;
          g.tile = u / q.S;
          g.red = 0;
          g.work = claim_ns + 2.0 * (double)s.bm * (double)s.bn * (double)s.k / q.S / alone_flop +
                   tile_out / alone_bytes;
          g.state = RUN;
        } else {
          const int v = q.red_next++;
          g.tile = v / RED_SLICES;   // index into the ready list
          g.red = 1;
          g.work = claim_ns + tile_out / RED_SLICES * (q.S + 1) / alone_bytes;
          g.state = WAIT_TILE;
        }
        took = true;
      }
    }
    // reduce units whose tile has finished start running
    for (Wg &g : wg)
      if (g.state == WAIT_TILE && g.tile < (int)ch[g.chunk].ready_tiles.size()) g.state = RUN;
    int active = 0;
    for (const Wg &g : wg) active += g.state == RUN;
    if (!any_unclaimed)
      for (Wg &g : wg)
        if (g.state == IDLE) g.state = GONE;
    if (active == 0) {
      if (next_avail < 0) break;   // nothing can progress (cannot happen with valid input)
      t = next_avail;
      continue;
    }
    // a workgroup's rate falls linearly from the alone rate (one running)
    // to an equal share of the whole GPU's (all running)
    const double busy_frac = (double)active / s.grid;
    const double speed = (1.0 + (kAloneSpeedup - 1.0) * (1.0 - busy_frac)) / kAloneSpeedup;
    double dt = -1;
    for (const Wg &g : wg)
      if (g.state == RUN && (dt < 0 || g.work / speed < dt)) dt = g.work / speed;
    if (next_avail > t && next_avail - t < dt) dt = next_avail - t;
    t += dt;
    for (Wg &g : wg) {
      if (g.state != RUN) continue;
      g.work -= dt * speed;
      if (g.work > 1e-6) continue;
      Chunk &q = ch[g.chunk];
      if (!g.red && q.S > 1 && --q.tile_left[g.tile] == 0) {
        q.tile_done[g.tile] = t;
        q.ready_tiles.push_back(g.tile);
      }
      g.state = IDLE;
      --left_total;
      done = std::max(done, t);
    }
  }
  return done;
}

}  // namespace
}  // namespace fo

using namespace fo;

extern "C" fo_status fo_plan_ag_schedule(int64_t m, int64_t n, int64_t k, int32_t nchunks, int32_t local,
                                         const int64_t *arrival_ns, double gemm_tflops,
                                         int32_t num_workgroups, int32_t *order_out, int32_t *split_out,
                                         int64_t *predicted_ns) {
  const int R = nchunks;
  if (!arrival_ns || !order_out || !split_out) return FO_ERR_NULL;
  if (R < 1 || R > FO_MAX_CHUNKS || m <= 0 || n <= 0 || k <= 0 || m % R != 0) return FO_ERR_SHAPE;
  if (local < 0 || local >= R) return FO_ERR_SCHEDULE;
  for (int c = 0; c < R; ++c)
    if (c != local && arrival_ns[c] < 0) return FO_ERR_SCHEDULE;
  int grid = num_workgroups;
  if (grid <= 0) grid = device_num_cus();
  if (grid <= 0) return FO_ERR_HIP;

  // order: peers by landing time (ties by ring distance), local last
  std::vector<int> peers;
  for (int s = 1; s < R; ++s) peers.push_back(((local - s) % R + R) % R);
  std::stable_sort(peers.begin(), peers.end(),
                   [&](int a, int b) { return arrival_ns[a] < arrival_ns[b]; });
  for (int i = 0; i < R - 1; ++i) order_out[i] = peers[i];
  order_out[R - 1] = local;

  Sim s;
  s.grid = grid;
  const int64_t mc = m / R;
  const TileCfg t = choose_tile(mc, n, k, R, grid, /*leave_room=*/true);
  s.bm = t.bm;
  s.bn = t.bn;
  s.k = k;
  s.tiles = (int)(((mc + t.bm - 1) / t.bm) * ((n + t.bn - 1) / t.bn));
  s.kt_total = (int)((k + 63) / 64);
  const double tflops = gemm_tflops > 0 ? gemm_tflops : kDefaultTflops;
  s.rate_all = tflops * 1e3;                       // FLOP per ns, whole GPU
  s.rate_one = s.rate_all / grid * kAloneSpeedup;  // one workgroup alone

  std::vector<double> avail(R);
  for (int c = 0; c < R; ++c) avail[c] = c == local ? 0.0 : (double)arrival_ns[c] + kFlagLatencyNs;
  const int tail = R > 1 ? order_out[R - 2] : -1;   // the peer that lands last

  // Predicted completion for every split of the last-landing chunk.
  std::vector<int> split(R, 1);
  const int cands[4] = {1, 2, 4, 8};
  double pred_by[4] = {-1, -1, -1, -1};
  for (int i = 0; i < 4; ++i) {
    const int want = cands[i];
    const int sk = effective_split(std::min(want, kPlanMaxSplit), s.kt_total);
    double pred = -1;
    if ((tail >= 0 && sk == want) || (tail < 0 && want == 1)) {
      if (tail >= 0) split[tail] = sk;
      pred = simulate(s, R, order_out, avail.data(), split.data());
      if (tail >= 0) split[tail] = 1;
    }
    pred_by[i] = pred;
    if (predicted_ns) predicted_ns[i] = pred < 0 ? -1 : (int64_t)pred;
  }
  // Split decision: the earliest predicted completion; a larger split must
  // win by more than kSplitMarginNs.
  for (int c = 0; c < R; ++c) split_out[c] = 1;
  if (tail >= 0) {
    double best = pred_by[0];
    int best_s = 1;
    for (int i = 1; i < 4; ++i)
      if (pred_by[i] >= 0 && pred_by[i] < best - kSplitMarginNs) { best = pred_by[i]; best_s = cands[i]; }
    split_out[tail] = best_s;
  }
  return FO_OK;
}
