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
//
// Beyond the order and split of one launch, the model also covers:
//  - the links: when each message lands on a ring (one incoming link, the
//    peers' chunks one after another) or a full mesh (a link per peer, all
//    at once), with each chunk optionally streamed as several messages;
//  - the number of messages each peer chunk is streamed in: only the last
//    message's share of the work is left after the last landing, while
//    small pieces cost more per unit (fo_plan_ag_stream);
//  - calibration: the rates, the alone speed-up and the latencies are taken
//    from measured launches of the shape (fo_plan_calibrate) instead of the
//    defaults below;
//  - the reduce-scatter side: when the shard is complete for the unfused,
//    fused and ring forms of GEMM-RS, given when the incoming partials land
//    (fo_plan_rs_form).
// The kernel's claim-ahead is modelled too: a workgroup with nothing landed
// to do holds a unit of the next chunk in priority order and starts it as
// soon as that chunk lands, without a claim.
#include "fo_internal.hpp"

#include <algorithm>
#include <math.h>
#include <vector>

namespace fo {
namespace {

constexpr int kPlanMaxSplit = 8;
// Defaults of the calibration (fo_plan_calib), measured on MI355X on the
// TP=8 MLP up-projection share.
constexpr double kFlagLatencyNs = 5000.0;       // flag store -> first claim by a claim walk
constexpr double kReserveLatencyNs = 2000.0;    // flag store -> a held unit's first loads
constexpr double kDefaultTflops = 900.0;        // every workgroup busy
constexpr double kAloneSpeedup = 1.8;           // one workgroup alone vs shared
constexpr double kHbmBytesPerNs = 5000.0;       // 5 TB/s, shared
constexpr double kWgBytesPerNsMax = 60.0;       // one workgroup alone
constexpr double kUnitFixedNs = 1500.0;         // claim and bookkeeping per unit
constexpr double kClaimQueueNs = 10.0;          // per workgroup claiming at the same instant
constexpr double kSplitMarginNs = 500.0;        // a larger split must win by more
constexpr double kLaunchNs = 4000.0;            // a launch's start and end, dispatch included

struct Sim {
  int grid = 0, tiles = 0, kt_total = 0;
  int64_t bm = 0, bn = 0, k = 0;
  double rate_all = 0;   // FLOP per ns with every workgroup busy
  double rate_one = 0;   // FLOP per ns of one workgroup alone
  double alone_speedup = kAloneSpeedup;
  double unit_fixed_ns = kUnitFixedNs;
  double reserve_ns = kReserveLatencyNs;
};

// Calibration with defaults for the fields left <= 0.
fo_plan_calib calib_or_default(const fo_plan_calib *c) {
  fo_plan_calib o{};
  o.gemm_tflops = (c && c->gemm_tflops > 0) ? c->gemm_tflops : kDefaultTflops;
  o.alone_speedup = (c && c->alone_speedup > 0) ? c->alone_speedup : kAloneSpeedup;
  o.flag_latency_ns = (c && c->flag_latency_ns > 0) ? c->flag_latency_ns : kFlagLatencyNs;
  o.reserve_latency_ns = (c && c->reserve_latency_ns > 0) ? c->reserve_latency_ns : kReserveLatencyNs;
  o.unit_fixed_ns = (c && c->unit_fixed_ns > 0) ? c->unit_fixed_ns : kUnitFixedNs;
  o.hbm_gbps = (c && c->hbm_gbps > 0) ? c->hbm_gbps : kHbmBytesPerNs;
  return o;
}

// The simulation's view of one launch shape (tile, rates) under a calibration.
Sim make_sim(int64_t mc, int64_t n, int64_t k, int R, int grid, const fo_plan_calib &cal) {
  Sim s;
  s.grid = grid;
  const TileCfg t = choose_tile(mc, n, k, R, grid, /*leave_room=*/true);
  s.bm = t.bm;
  s.bn = t.bn;
  s.k = k;
  s.tiles = (int)(((mc + t.bm - 1) / t.bm) * ((n + t.bn - 1) / t.bn));
  s.kt_total = (int)((k + 63) / 64);
  s.rate_all = cal.gemm_tflops * 1e3;                          // FLOP per ns, whole GPU
  s.rate_one = s.rate_all / grid * cal.alone_speedup;          // one workgroup alone
  s.alone_speedup = cal.alone_speedup;
  s.unit_fixed_ns = cal.unit_fixed_ns;
  s.reserve_ns = cal.reserve_latency_ns;
  return s;
}

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
// whole-GPU rate divided among them.  Idle workgroups claim at each event in
// priority order: a landed chunk's unit after its flag latency, at a fixed
// cost plus a term that grows with the number of workgroups claiming at that
// instant (they queue on the same claim counters); with nothing landed to
// do, a workgroup holds a unit of the first chunk in priority order that has
// units left (claim-ahead) and starts it reserve_ns after that chunk lands,
// without a claim.  A reduce unit waits, holding its workgroup, until every
// split of its tile has finished.
double simulate(const Sim &s, int R, const int *order, const double *land, double flag_latency_ns,
                const int *split) {
  struct Chunk {
    int units = 0, next = 0, red_units = 0, red_next = 0, S = 1;
    std::vector<int> tile_left;          // splits of the tile still running
    std::vector<int> ready_tiles;        // tiles in the order their splits finished
  };
  enum { IDLE, RUN, WAIT_TILE, HELD, GONE };
  struct Wg {
    int state = IDLE;
    double work = 0;                     // ns at the alone rate
    double start = 0;                    // HELD: when the unit starts
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
    }
  }
  std::vector<double> avail(R);
  for (int c = 0; c < R; ++c) avail[c] = land[c] < 0 ? 0.0 : land[c] + flag_latency_ns;   // < 0: present
  const double alone_flop = s.rate_one;                  // FLOP per ns
  const double alone_bytes = kWgBytesPerNsMax;           // bytes per ns
  const double tile_out = (double)s.bm * (double)s.bn * 4.0;
  auto gemm_work = [&](const Chunk &q) {
    return 2.0 * (double)s.bm * (double)s.bn * (double)s.k / q.S / alone_flop + tile_out / alone_bytes;
  };
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
    const double claim_ns = s.unit_fixed_ns + kClaimQueueNs * std::min(idle, claimable);
    double next_event = -1;
    bool any_unclaimed = false;
    auto note = [&](double te) { if (te > t && (next_event < 0 || te < next_event)) next_event = te; };
    for (Wg &g : wg) {
      if (g.state != IDLE) continue;
      bool took = false;
      int ahead = -1;                    // first chunk with GEMM units left that has not landed
      for (int pi = 0; pi < R && !took; ++pi) {
        const int c = order[pi];
        Chunk &q = ch[c];
        const bool gemm_left = q.next < q.units;
        const bool red_left = !gemm_left && q.red_next < q.red_units;
        if (!gemm_left && !red_left) continue;
        any_unclaimed = true;
        if (avail[c] > t) {
          note(avail[c]);
          if (gemm_left && ahead < 0) ahead = c;
          continue;
        }
        g.chunk = c;
        if (gemm_left) {
          const int u = q.next++;
          g.tile = u / q.S;
          g.red = 0;
          g.work = claim_ns + gemm_work(q);
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
      if (!took && ahead >= 0) {         // claim ahead
        Chunk &q = ch[ahead];
        const int u = q.next++;
        g.chunk = ahead;
        g.tile = u / q.S;
        g.red = 0;
        g.work = gemm_work(q);
        g.start = land[ahead] + s.reserve_ns;
        g.state = HELD;
        note(g.start);
      }
    }
    // held units whose chunk has landed, and reduce units whose tile has
    // finished, start running
    for (Wg &g : wg) {
      if (g.state == HELD && g.start <= t) g.state = RUN;
      if (g.state == WAIT_TILE && g.tile < (int)ch[g.chunk].ready_tiles.size()) g.state = RUN;
      if (g.state == HELD) note(g.start);
    }
    int active = 0;
    for (const Wg &g : wg) active += g.state == RUN;
    if (!any_unclaimed)
      for (Wg &g : wg)
        if (g.state == IDLE) g.state = GONE;
    if (active == 0) {
      if (next_event < 0) break;   // nothing can progress (cannot happen with valid input)
      t = next_event;
      continue;
    }
    // a workgroup's rate falls linearly from the alone rate (one running)
    // to an equal share of the whole GPU's (all running)
    const double busy_frac = (double)active / s.grid;
    const double speed = (1.0 + (s.alone_speedup - 1.0) * (1.0 - busy_frac)) / s.alone_speedup;
    double dt = -1;
    for (const Wg &g : wg)
      if (g.state == RUN && (dt < 0 || g.work / speed < dt)) dt = g.work / speed;
    if (next_event > t && next_event - t < dt) dt = next_event - t;
    t += dt;
    for (Wg &g : wg) {
      if (g.state != RUN) continue;
      g.work -= dt * speed;
      if (g.work > 1e-6) continue;
      Chunk &q = ch[g.chunk];
      if (!g.red && q.S > 1 && --q.tile_left[g.tile] == 0) q.ready_tiles.push_back(g.tile);
      g.state = IDLE;
      --left_total;
      done = std::max(done, t);
    }
  }
  return done;
}

// Order (peers by landing time, ties in ring order from local, local last)
// and the predicted completion for each split {1, 2, 4, 8} of the peer that
// lands last (-1 where that split is not possible); returns the chosen split
// (the earliest, a larger one only if it wins by more than kSplitMarginNs).
int plan_launch(const Sim &s, int R, int local, const double *land, double flag_latency_ns, int32_t *order,
                double pred[4], int sub = 1) {
  // pieces that land (land >= 0) by landing time, ties by their chunk's ring
  // distance from local and then by piece; then the pieces already present
  std::vector<int> peers, present;
  const int Rc = R / sub;
  for (int d = 0; d < Rc; ++d) {
    const int c = ((local / sub - d) % Rc + Rc) % Rc;
    for (int j = 0; j < sub; ++j) (land[c * sub + j] < 0 ? present : peers).push_back(c * sub + j);
  }
  std::stable_sort(peers.begin(), peers.end(), [&](int a, int b) { return land[a] < land[b]; });
  std::sort(present.begin(), present.end());
  int n = 0;
  for (int c : peers) order[n++] = c;
  for (int c : present) order[n++] = c;
  const int tail = peers.empty() ? -1 : peers.back();
  std::vector<int> split(R, 1);
  const int cands[4] = {1, 2, 4, 8};
  for (int i = 0; i < 4; ++i) {
    const int want = cands[i];
    const int sk = effective_split(std::min(want, kPlanMaxSplit), s.kt_total);
    pred[i] = -1;
    if ((tail >= 0 && sk == want) || (tail < 0 && want == 1)) {
      if (tail >= 0) split[tail] = sk;
      pred[i] = simulate(s, R, order, land, flag_latency_ns, split.data());
      if (tail >= 0) split[tail] = 1;
    }
  }
  int best_s = 1;
  double best = pred[0];
  for (int i = 1; i < 4; ++i)
    if (pred[i] >= 0 && pred[i] < best - kSplitMarginNs) { best = pred[i]; best_s = cands[i]; }
  return best_s;
}

// Landing time of each of a chunk's `sub` messages: chunk c of the ring lands
// its last byte at its ring step times the chunk's link time; on a mesh every
// peer sends at once on its own link.
void link_arrivals(int R, int local, double chunk_ns, int topology, int sub, std::vector<double> &land) {
  land.assign((size_t)R * sub, 0.0);
  for (int d = 1; d < R; ++d) {
    const int c = ((local - d) % R + R) % R;
    const double t_begin = topology == FO_LINK_MESH ? 0.0 : (d - 1) * chunk_ns;
    for (int j = 0; j < sub; ++j) land[(size_t)c * sub + j] = t_begin + (j + 1) * chunk_ns / sub;
  }
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
  fo_plan_calib in{};
  in.gemm_tflops = gemm_tflops;
  const fo_plan_calib cal = calib_or_default(&in);
  const Sim sim = make_sim(m / R, n, k, R, grid, cal);
  std::vector<double> land(R);
  for (int c = 0; c < R; ++c) land[c] = c == local ? -1.0 : (double)arrival_ns[c];
  double pred[4];
  const int best = plan_launch(sim, R, local, land.data(), cal.flag_latency_ns, order_out, pred);
  for (int c = 0; c < R; ++c) split_out[c] = 1;
  if (R > 1) split_out[order_out[R - 2]] = best;
  if (predicted_ns)
    for (int i = 0; i < 4; ++i) predicted_ns[i] = pred[i] < 0 ? -1 : (int64_t)pred[i];
  return FO_OK;
}

extern "C" fo_status fo_plan_link_arrivals(int32_t nchunks, int32_t local, int64_t chunk_bytes, double link_gbps,
                                           int32_t topology, int32_t sub, int64_t *arrival_ns) {
  const int R = nchunks;
  if (!arrival_ns) return FO_ERR_NULL;
  if (R < 1 || sub < 1 || (int64_t)R * sub > FO_MAX_CHUNKS || chunk_bytes <= 0) return FO_ERR_SHAPE;
  if (local < 0 || local >= R || link_gbps <= 0 || (topology != FO_LINK_RING && topology != FO_LINK_MESH))
    return FO_ERR_SCHEDULE;
  std::vector<double> land;
  link_arrivals(R, local, (double)chunk_bytes / link_gbps, topology, sub, land);
  for (int i = 0; i < R * sub; ++i) arrival_ns[i] = (i / sub == local) ? 0 : (int64_t)llround(land[i]);
  return FO_OK;
}

extern "C" fo_status fo_plan_calibrate(int64_t m, int64_t n, int64_t k, int32_t nchunks, double all_present_ns,
                                       double chunk_alone_ns, double tail_unsplit_ns, int32_t num_workgroups,
                                       fo_plan_calib *out) {
  const int R = nchunks;
  if (!out) return FO_ERR_NULL;
  if (R < 1 || R > FO_MAX_CHUNKS || m <= 0 || n <= 0 || k <= 0 || m % R != 0) return FO_ERR_SHAPE;
  if (all_present_ns <= kLaunchNs) return FO_ERR_SCHEDULE;
  int grid = num_workgroups;
  if (grid <= 0) grid = device_num_cus();
  if (grid <= 0) return FO_ERR_HIP;
  fo_plan_calib cal = calib_or_default(nullptr);
  // the whole-GPU rate: the launch's flops over its time less start and end
  cal.gemm_tflops = 2.0 * (double)m * (double)n * (double)k / (all_present_ns - kLaunchNs) / 1e3;
  // the alone speed-up A from one chunk's unsplit launch, whose `tiles` units
  // run alone: D = (F/r + E A) / (1 + (A - 1) f), with F a tile's flops, r
  // the per-workgroup share of the whole-GPU rate, E its output time alone
  // and f the idle fraction of the grid
  if (chunk_alone_ns > kLaunchNs) {
    const Sim s0 = make_sim(m / R, n, k, R, grid, cal);
    const double F = 2.0 * (double)s0.bm * (double)s0.bn * (double)k;
    const double r = s0.rate_all / grid;
    const double E = (double)s0.bm * (double)s0.bn * 4.0 / kWgBytesPerNsMax;
    const double f = 1.0 - std::min(1.0, (double)s0.tiles / grid);
    const double D = chunk_alone_ns - kLaunchNs - cal.unit_fixed_ns;
    const double den = D * f - E;
    if (D > 0 && den > 0) cal.alone_speedup = std::min(4.0, std::max(1.0, (F / r - D * (1.0 - f)) / den));
    // the latency from a landing to a held unit's first loads: an unsplit
    // last chunk landing on an idle GPU ends one unit after its landing
    if (tail_unsplit_ns > 0) {
      const Sim s1 = make_sim(m / R, n, k, R, grid, cal);
      const double speed = (1.0 + (s1.alone_speedup - 1.0) * f) / s1.alone_speedup;
      const double unit = (F / s1.rate_one + E) / speed;
      cal.reserve_latency_ns = std::max(200.0, tail_unsplit_ns - unit);
    }
  }
  *out = cal;
  return FO_OK;
}

extern "C" fo_status fo_plan_ag_stream(int64_t m, int64_t n, int64_t k, int32_t nchunks, int32_t local,
                                       double link_gbps, int32_t topology, const fo_plan_calib *calib,
                                       int32_t num_workgroups, int32_t *sub_out, int32_t *order_out,
                                       int32_t *split_out, int64_t *predicted_ns) {
  const int R = nchunks;
  if (!sub_out || !order_out || !split_out) return FO_ERR_NULL;
  if (R < 1 || R > FO_MAX_CHUNKS || m <= 0 || n <= 0 || k <= 0 || m % R != 0) return FO_ERR_SHAPE;
  if (local < 0 || local >= R || link_gbps <= 0 || (topology != FO_LINK_RING && topology != FO_LINK_MESH))
    return FO_ERR_SCHEDULE;
  int grid = num_workgroups;
  if (grid <= 0) grid = device_num_cus();
  if (grid <= 0) return FO_ERR_HIP;
  const fo_plan_calib cal = calib_or_default(calib);
  const int64_t mc = m / R;
  const double chunk_ns = (double)(mc * k * 2) / link_gbps;
  const int subs[4] = {1, 2, 4, 8};
  double best = -1;
  int best_sub = 1, best_split = 1;
  std::vector<int32_t> order(FO_MAX_CHUNKS), best_order(FO_MAX_CHUNKS);
  for (int si = 0; si < 4; ++si) {
    const int sub = subs[si];
    double pred[4] = {-1, -1, -1, -1};
    if ((int64_t)R * sub <= FO_MAX_CHUNKS && mc % sub == 0 && (sub == 1 || R > 1)) {
      const int R2 = R * sub;
      const Sim sim = make_sim(mc / sub, n, k, R2, grid, cal);
      std::vector<double> land;
      link_arrivals(R, local, chunk_ns, topology, sub, land);
      for (int j = 0; j < sub; ++j) land[(size_t)local * sub + j] = -1.0;
      const int sk = plan_launch(sim, R2, local * sub, land.data(), cal.flag_latency_ns, order.data(), pred, sub);
      const double p = pred[sk == 1 ? 0 : sk == 2 ? 1 : sk == 4 ? 2 : 3];
      // more messages must win by more than the margin
      if (p >= 0 && (best < 0 || p < best - kSplitMarginNs)) {
        best = p;
        best_sub = sub;
        best_split = sk;
        best_order = order;
      }
    }
    if (predicted_ns)
      for (int i = 0; i < 4; ++i) predicted_ns[si * 4 + i] = pred[i] < 0 ? -1 : (int64_t)pred[i];
  }
  const int R2 = R * best_sub;
  *sub_out = best_sub;
  for (int i = 0; i < R2; ++i) {
    order_out[i] = best_order[i];
    split_out[i] = 1;
  }
  // the piece that lands last is the last of the landing pieces in the order
  if (R > 1) split_out[best_order[R2 - best_sub - 1]] = best_split;
  return FO_OK;
}

extern "C" fo_status fo_plan_rs_form(int64_t m, int64_t n, int64_t k, int32_t nchunks, int32_t local,
                                     const int64_t *arrival_ns, const fo_plan_calib *calib, int32_t num_workgroups,
                                     int32_t *form_out, int64_t *predicted_ns) {
  const int R = nchunks;
  if (!arrival_ns || !form_out) return FO_ERR_NULL;
  if (R < 1 || R > FO_MAX_CHUNKS || m <= 0 || n <= 0 || k <= 0 || m % R != 0) return FO_ERR_SHAPE;
  if (local < 0 || local >= R) return FO_ERR_SCHEDULE;
  for (int c = 0; c < R; ++c)
    if (c != local && arrival_ns[c] < 0) return FO_ERR_SCHEDULE;
  int grid = num_workgroups;
  if (grid <= 0) grid = device_num_cus();
  if (grid <= 0) return FO_ERR_HIP;
  const fo_plan_calib cal = calib_or_default(calib);
  // the GEMM-RS launch; every chunk's partial is ready at its end (one round)
  const double t_gemm = kLaunchNs + 2.0 * (double)m * (double)n * (double)k / (cal.gemm_tflops * 1e3);
  const double part = (double)(m / R) * (double)n * 4.0;         // one fp32 partial
  const double shard = (double)(m / R) * (double)n * 2.0;        // the bf16 shard
  const double hbm = cal.hbm_gbps;                               // bytes per ns
  // incoming partials in landing order (the reduce's summation order)
  std::vector<double> land;
  for (int d = 1; d < R; ++d) land.push_back((double)arrival_ns[((local - d) % R + R) % R]);
  std::sort(land.begin(), land.end());
  // progressive reduce from `start`: each pass adds the run of partials
  // landed by then (read the running sum and the run, write the sum; the
  // last pass writes the shard)
  auto progressive = [&](double start) {
    double t = start;
    size_t added = 0;
    const double poll = cal.reserve_latency_ns;
    while (added < land.size()) {
      size_t run = 0;
      while (added + run < land.size() && land[added + run] + poll <= t) ++run;
      if (run == 0) { t = land[added] + poll; continue; }
      const bool last = added + run == land.size();
      t += ((double)(run + 1) * part + (last ? shard : part)) / hbm;
      added += run;
    }
    if (land.empty()) t += (part + shard) / hbm;
    return t;
  };
  const double unfused = progressive(t_gemm + kLaunchNs);        // a second launch behind the GEMM
  const double fused = progressive(t_gemm);                      // shard units after the GEMM units
  // ring: the local chunk's accumulated partial is the last message; its sum
  // with the local partial is the shard
  const double last = land.empty() ? 0.0 : land.back();
  const double ring = std::max(t_gemm, last + cal.reserve_latency_ns) + (2.0 * part + shard) / hbm;
  const double pred[3] = {unfused, fused, ring};
  int best = 0;
  for (int i = 1; i < 3; ++i)
    if (pred[i] < pred[best] - kSplitMarginNs) best = i;
  *form_out = best;
  if (predicted_ns)
    for (int i = 0; i < 3; ++i) predicted_ns[i] = (int64_t)pred[i];
  return FO_OK;
}
