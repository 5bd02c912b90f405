// C ABI of the one-GPU FlashOverlap hot path: argument validation, schedule
// expansion (default rank-adaptive order, split policy), launch sizing.
// Declarations, argument meaning and error behaviour: include/flashoverlap.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fo_internal.hpp"

namespace fo {

namespace {

constexpr int kMaxDevices = 64;
constexpr uint64_t kDefaultTimeoutNs = 10ull * 1000 * 1000 * 1000;
constexpr int kMaxSplit = 8;
constexpr int kMinSplitStages = 16;   // automatic split: k stages per split, at least
constexpr int kMinSelfSplit = 4;     // split units sum their own slices only from this split up
// Largest k: a tile's operand rows (at most 256 of them) are addressed with
// 32-bit byte offsets, and an offset of 2^30 past a row block must lie beyond
// it (it stands for "k past the end", which reads as zero).
constexpr int64_t kMaxK = (int64_t)1 << 21;

struct DevInfo {
  int cus = 0;
  int lds = 0;
  uint64_t wall_hz = 0;
  hipError_t err = hipSuccess;
};

DevInfo g_dev[kMaxDevices];
std::once_flag g_once[kMaxDevices];
thread_local char g_hip_err[256] = "";

void record(hipError_t e) {
  const char *s = hipGetErrorString(e);
  strncpy(g_hip_err, s ? s : "unknown HIP error", sizeof(g_hip_err) - 1);
  g_hip_err[sizeof(g_hip_err) - 1] = 0;
}

const DevInfo *dev_info() {
  int d = 0;
  hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) { record(e); return nullptr; }
  if (d < 0 || d >= kMaxDevices) return nullptr;
  std::call_once(g_once[d], [d]() {
    DevInfo &I = g_dev[d];
    int khz = 0;
    I.err = hipDeviceGetAttribute(&I.cus, hipDeviceAttributeMultiprocessorCount, d);
    if (I.err == hipSuccess)
      I.err = hipDeviceGetAttribute(&I.lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, d);
    if (I.err == hipSuccess) I.err = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, d);
    I.wall_hz = (uint64_t)khz * 1000ull;
  });
  if (g_dev[d].err != hipSuccess) { record(g_dev[d].err); return nullptr; }
  return &g_dev[d];
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

fo_status check_schedule(const fo_schedule *s) {
  if (!s) return FO_ERR_NULL;
  if (s->nchunks < 1 || s->nchunks > FO_MAX_CHUNKS) return FO_ERR_SHAPE;
  if (s->local < 0 || s->local >= s->nchunks) return FO_ERR_SCHEDULE;
  if (s->epoch == 0) return FO_ERR_SCHEDULE;
  if (s->mode != FO_SCHED_READY_FIRST && s->mode != FO_SCHED_STRICT) return FO_ERR_SCHEDULE;
  if (s->max_workgroups < 0) return FO_ERR_SCHEDULE;
  if (s->order) {
    uint64_t seen = 0;
    for (int i = 0; i < s->nchunks; ++i) {
      const int c = s->order[i];
      if (c < 0 || c >= s->nchunks || (seen >> c) & 1ull) return FO_ERR_ORDER;
      seen |= 1ull << c;
    }
  }
  if (s->split)
    for (int i = 0; i < s->nchunks; ++i)
      if (s->split[i] < 1 || s->split[i] > kMaxSplit) return FO_ERR_SCHEDULE;
  return FO_OK;
}

// Default priority: peers in ring arrival order local-1, local-2, ..., then local.
void expand_order(const fo_schedule *s, int32_t *order) {
  const int R = s->nchunks;
  if (s->order) {
    for (int i = 0; i < R; ++i) order[i] = s->order[i];
    return;
  }
  for (int i = 1; i < R; ++i) order[i - 1] = ((s->local - i) % R + R) % R;
  order[R - 1] = s->local;
}

uint64_t ns_to_ticks(uint64_t ns, uint64_t hz) {
  const long double t = (long double)ns * (long double)hz / 1e9L;
  return t > 1.8e19L ? ~0ull : (uint64_t)t;
}

struct GemmPlan {
  TileCfg tile;
  int64_t mc;
  int tiles_m, tiles_n, tiles;
  int kt_total;
  size_t counter_bytes, partial_offset, total_bytes;
  int ready_off;
};

// Workspace bound over every tile configuration the library may pick.
GemmPlan plan_workspace(int64_t m, int64_t n, int64_t k, int R) {
  GemmPlan p{};
  p.mc = m / R;
  // every tile shape the launch may pick: the most tiles per chunk (counters
  // and ready lists) and the largest padded chunk area (split partials)
  const int64_t most_tiles = max_tiles_per_chunk(p.mc, n);
  const int64_t padded = max_padded_tile_area(p.mc, n);
  (void)k;
  p.ready_off = (int)(WS_TILE_CTR + R * most_tiles);
  p.counter_bytes = WS_HEADER_BYTES + 2 * (size_t)R * most_tiles * sizeof(uint32_t);
  p.partial_offset = (p.counter_bytes + 255) & ~(size_t)255;
  p.total_bytes = p.partial_offset + (size_t)kMaxSplit * padded * sizeof(float);
  return p;
}

GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k, int R, int grid, bool leave_room) {
  GemmPlan p = plan_workspace(m, n, k, R);
  p.tile = choose_tile(p.mc, n, k, R, grid, leave_room);
  p.tiles_m = (int)((p.mc + p.tile.bm - 1) / p.tile.bm);
  p.tiles_n = (int)((n + p.tile.bn - 1) / p.tile.bn);
  p.tiles = p.tiles_m * p.tiles_n;
  p.kt_total = (int)((k + 63) / 64);
  return p;
}

// The fused reduce of fo_gemm_rs_reduce.
struct FusedRs {
  void *shard;
  bool shard_bf16;
  const float *const *incoming;   // host [R] of device pointers
  bool ring;                      // ring form: incoming[c] is chunk c's accumulated partial (may be null)
};

// Zeroes n 32-bit words with vector stores (a kernel rather than a memset, so
// the clearing can sit inside a captured stream).
__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

fo_status run_gemm(const void *x, const void *w, void *y, bool y_bf16, uint32_t *done,
                   bool rs_mode, int64_t m, int64_t n, int64_t k, const fo_schedule *s,
                   void *ws, size_t ws_bytes, void *stream, const FusedRs *fz = nullptr,
                   bool clear_counters = false) {
  if (!x || !w || !y || !s) return FO_ERR_NULL;
  fo_status st = check_schedule(s);
  if (st != FO_OK) return st;
  const int R = s->nchunks;
  if (m <= 0 || n <= 0 || k <= 0 || m % R != 0) return FO_ERR_SHAPE;
  if (m / R > (int64_t)1 << 30 || n > (int64_t)1 << 30 || k > kMaxK) return FO_ERR_SHAPE;
  if (k % 8 != 0 || !aligned16(x) || !aligned16(w)) return FO_ERR_ALIGN;
  if (!aligned16(y) && !y_bf16) return FO_ERR_ALIGN;
  if (rs_mode && s->arrived && !fz) return FO_ERR_SCHEDULE;
  if (fz) {
    if (!fz->shard || !fz->incoming) return FO_ERR_NULL;
    // direct form: every peer's partial is required (incoming[local] is
    // ignored); ring form: any entry may be null (no incoming partial)
    auto used = [&](int c) { return fz->ring ? fz->incoming[c] != nullptr : c != s->local; };
    for (int c = 0; c < R; ++c)
      if (!fz->ring && c != s->local && !fz->incoming[c]) return FO_ERR_NULL;
    if (n % 4 != 0 || !aligned16(fz->shard)) return FO_ERR_ALIGN;
    for (int c = 0; c < R; ++c)
      if (used(c) && !aligned16(fz->incoming[c])) return FO_ERR_ALIGN;
    if ((m / R) * n * 4 >= ((int64_t)1 << 31)) return FO_ERR_SHAPE;
    if (s->split)
      for (int c = 0; c < R; ++c)
        if (s->split[c] != 1) return FO_ERR_SCHEDULE;
    const size_t shard_bytes = (size_t)(m / R) * n * (fz->shard_bf16 ? 2 : 4);
    if (overlaps(fz->shard, shard_bytes, y, (size_t)m * n * 4) ||
        overlaps(fz->shard, shard_bytes, x, (size_t)m * k * 2) ||
        overlaps(fz->shard, shard_bytes, w, (size_t)n * k * 2))
      return FO_ERR_ALIAS;
    // incoming partials are read while the launch writes the partials and
    // the shard
    const size_t inc_bytes = (size_t)(m / R) * n * 4;
    for (int c = 0; c < R; ++c)
      if (used(c) && (overlaps(fz->incoming[c], inc_bytes, fz->shard, shard_bytes) ||
                      overlaps(fz->incoming[c], inc_bytes, y, (size_t)m * n * 4)))
        return FO_ERR_ALIAS;
  }
  const size_t ybytes = (size_t)m * n * (y_bf16 ? 2 : 4);
  if (overlaps(y, ybytes, x, (size_t)m * k * 2) || overlaps(y, ybytes, w, (size_t)n * k * 2))
    return FO_ERR_ALIAS;
  if (!ws) return FO_ERR_WORKSPACE;
  if (ws_bytes < plan_workspace(m, n, k, R).total_bytes || !aligned16(ws)) return FO_ERR_WORKSPACE;

  const DevInfo *I = dev_info();
  if (!I) return FO_ERR_HIP;

  // Workgroups: one per CU.  With arrival flags the tile configuration must
  // leave registers free on every SIMD, so the one-wave timer and flag
  // kernels of a copy engine emulator can run beside the persistent grid.
  // Every workgroup of the persistent grid must be resident at once (a
  // workgroup may wait for units that others hold, and the first units are
  // assigned by workgroup index), and each takes one CU's LDS: the grid is
  // capped at one workgroup per CU.
  const int full = I->cus;
  const int grid_cap = (s->max_workgroups > 0 && s->max_workgroups < full) ? s->max_workgroups : full;
  const GemmPlan p = plan_gemm(m, n, k, R, grid_cap, s->arrived != nullptr);

  GemmArgs a{};
  a.x = static_cast<const uint16_t *>(x);
  a.w = static_cast<const uint16_t *>(w);
  a.y = y;
  a.y_bf16 = y_bf16 ? 1 : 0;
  a.rs_mode = rs_mode ? 1 : 0;
  a.m = m; a.n = n; a.k = k;
  a.R = R;
  a.mc = (int32_t)p.mc;
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  // Rectangles of each chunk's tile grid, one per XCD: among the shapes
  // whose largest rectangle holds the fewest tiles (an XCD with more tiles
  // than the others makes its neighbours' workgroups steal one contended
  // claim at a time), the one that minimises the operand rows one XCD
  // streams over all R chunks (X rows of its row band in every chunk plus W
  // rows of its column band).
  {
    const int shapes[4][2] = {{1, 8}, {2, 4}, {4, 2}, {8, 1}};
    int64_t best[3] = {-1, -1, -1};   // empty rectangles, largest rectangle, cost
    for (const auto &sh : shapes) {
      const int gm = sh[0], gn = sh[1];
      const int64_t key[3] = {(gm > p.tiles_m || gn > p.tiles_n) ? 1 : 0,
                              (int64_t)((p.tiles_m + gm - 1) / gm) * ((p.tiles_n + gn - 1) / gn),
                              (int64_t)R * ((p.tiles_m + gm - 1) / gm) * p.tile.bm +
                                  (int64_t)((p.tiles_n + gn - 1) / gn) * p.tile.bn};
      bool better = best[0] < 0;
      for (int q = 0; q < 3 && !better; ++q) {
        if (key[q] != best[q]) { better = key[q] < best[q]; break; }
      }
      if (better) {
        for (int q = 0; q < 3; ++q) best[q] = key[q];
        a.gm = gm; a.gn = gn;
      }
    }
    for (int g = 0; g < XCDS; ++g) {
      const int i = g / a.gn, j = g % a.gn;
      const int rows = (i + 1) * p.tiles_m / a.gm - i * p.tiles_m / a.gm;
      const int cols = (j + 1) * p.tiles_n / a.gn - j * p.tiles_n / a.gn;
      a.gtiles[g] = rows * cols;
    }
  }
  a.local = s->local;
  a.strict = s->mode == FO_SCHED_STRICT ? 1 : 0;
  a.arrived = fz ? nullptr : s->arrived;   // fused: the flags gate the incoming partials only
  a.done_flags = done;
  a.epoch = s->epoch;
  a.timeout_ticks = ns_to_ticks(s->timeout_ns ? s->timeout_ns : kDefaultTimeoutNs, I->wall_hz);
  a.status = s->status;
  a.stamps = s->stamps;
  a.ws32 = static_cast<uint32_t *>(ws);
  a.partials = reinterpret_cast<float *>(static_cast<char *>(ws) + p.partial_offset);
  expand_order(s, a.order);

  // Split policy.
  int split[FO_MAX_CHUNKS];
  for (int c = 0; c < R; ++c) split[c] = 1;
  if (s->split) {
    for (int c = 0; c < R; ++c) split[c] = s->split[c];
  } else if (s->arrived && R > 1 && !rs_mode) {
    // the last peer in priority order is the chunk expected to land last
    int tail = -1;
    for (int i = R - 1; i >= 0; --i)
      if (a.order[i] != s->local) { tail = a.order[i]; break; }
    // Split so its tiles fill the GPU, but keep at least kMinSplitStages
    // 64-wide k stages per split: a shorter split spends as much on writing
    // and reducing its partial tile as on its k-loop.  (On the TP=8 MLP share,
    // k = 4096, split 4 was the best measured at every link bandwidth from 50
    // to 400 GB/s and split 8 up to 9% slower; on the QKV share, k = 8192,
    // split 8 was the best at 50 GB/s.)
    int sk = (grid_cap + p.tiles - 1) / p.tiles;
    if (sk > kMaxSplit) sk = kMaxSplit;
    if (sk > p.kt_total / kMinSplitStages) sk = p.kt_total / kMinSplitStages;
    if (sk < 1) sk = 1;
    if (tail >= 0) split[tail] = sk;
  }
  int64_t total_units = 0;
  size_t ctr_used = 0, part_used = 0;
  for (int c = 0; c < R; ++c) {
    int sk = split[c];
    if (sk > p.kt_total) sk = p.kt_total;
    int kt_per = (p.kt_total + sk - 1) / sk;
    // every split must own at least one k stage
    while (sk > 1 && (int64_t)(sk - 1) * kt_per >= p.kt_total) {
      --sk;
      kt_per = (p.kt_total + sk - 1) / sk;
    }
    a.split[c] = sk;
    a.kslice[c] = kt_per * 64;
    a.units[c] = p.tiles * sk;
    a.red_units[c] = sk > 1 ? p.tiles * RED_SLICES : 0;
    if (sk > 1) {
      a.ctr_base[c] = (int32_t)ctr_used;
      a.part_base[c] = (int32_t)part_used;
      ctr_used += (size_t)p.tiles;
      part_used += (size_t)p.tiles * sk;
    } else {
      a.ctr_base[c] = -1;
      a.part_base[c] = -1;
    }
    total_units += a.units[c] + a.red_units[c];
  }
  // Split chunks without reduce units: each split unit sums its own row
  // slices of its tile once the tile's splits are all written, so no
  // workgroup claims a reduce unit on one shared counter after the GEMM
  // units.  A unit then waits for the other splits of its tile.  The claimed
  // units of each XCD group form a prefix of the group's split-fastest
  // numbering, so at most S - 1 units per group and split chunk wait at a
  // time; with at least XCDS x (sum of the splits) workgroups some workgroup
  // is always free to claim the rest (and under round-robin assignment each
  // XCD has at least S workgroups, so a tile spans at most two rounds).
  // A split of 2 or 3 leaves each unit a third or more of its tile to sum,
  // one round trip per few rows: there reduce units on the idle workgroups
  // were faster (measured on the TP=8 MLP chunk alone), so every split
  // chunk must be split at least kMinSelfSplit ways.
  a.self_reduce = 0;
  if (!fz) {
    int64_t units = 0, split_sum = 0;
    bool deep = true;
    for (int c = 0; c < R; ++c) {
      units += a.units[c];
      if (a.split[c] > 1) {
        split_sum += a.split[c];
        deep = deep && a.split[c] >= kMinSelfSplit;
      }
    }
    const int64_t g = units < grid_cap ? units : grid_cap;
    if (split_sum > 0 && deep && g >= (int64_t)XCDS * split_sum && tile_self_reduce(p.tile)) {
      a.self_reduce = 1;
      total_units = units;
      for (int c = 0; c < R; ++c) a.red_units[c] = 0;
    }
  }
  if (fz) {
    // Direct form: the local chunk's tiles get shard units (RED_SLICES row
    // slices each) and a ready list; the incoming partials are summed in
    // priority order.  Ring form: so do the tiles of every chunk with an
    // incoming partial (inc[] indexed by chunk), and of the local chunk.
    a.fused = 1;
    a.ring = fz->ring ? 1 : 0;
    a.shard = fz->shard;
    a.shard_bf16 = fz->shard_bf16 ? 1 : 0;
    a.inc_arrived = s->arrived;
    a.ninc = 0;
    for (int c = 0; c < R; ++c) {
      const bool units = fz->ring ? (fz->incoming[c] != nullptr || c == s->local) : c == s->local;
      if (!units) continue;
      a.red_units[c] = p.tiles * RED_SLICES;
      a.ctr_base[c] = (int32_t)ctr_used;
      ctr_used += (size_t)p.tiles;
      total_units += a.red_units[c];
    }
    a.nshard = 0;
    for (int i = 0; i < R; ++i)
      if (a.red_units[a.order[i]] > 0) a.shard_seq[a.nshard++] = a.order[i];
    if (fz->ring) {
      for (int c = 0; c < R; ++c) a.inc[c] = fz->incoming[c];
    } else {
      for (int i = 0; i < R; ++i) {
        const int q = a.order[i];
        if (q == s->local) continue;
        a.inc[a.ninc] = fz->incoming[q];
        a.inc_chunk[a.ninc] = q;
        ++a.ninc;
      }
    }
  }
  a.ready_off = p.ready_off;
  if (part_used > 0 && ws_bytes < p.partial_offset + part_used * partial_slot_bytes(p.tile))
    return FO_ERR_WORKSPACE;
  if (total_units > (int64_t)1 << 30) return FO_ERR_SHAPE;
  a.total_units = (int32_t)total_units;
  a.grid = (int32_t)(total_units < grid_cap ? total_units : grid_cap);
  if (a.grid < 1) a.grid = 1;
  // Without arrival flags and reduce units, every unit is assigned
  // statically when that is balanced: no workgroup gets a second unit (2), or
  // every XCD group holds the same number of units and every XCD the same
  // number of workgroups (1: round-robin over the XCD's workgroups).
  a.static_rr = 0;
  a.all_unsplit = 1;
  for (int c = 0; c < R; ++c) a.all_unsplit = a.all_unsplit && a.split[c] == 1;
  for (int g = 0; g < XCDS; ++g) {
    int64_t units_g = 0;
    for (int c = 0; c < R; ++c) units_g += (int64_t)a.gtiles[g] * a.split[c];
    a.gunits[g] = (int32_t)units_g;
  }
  {
    bool ok = true;
    for (int c = 0; c < R && ok; ++c) ok = a.red_units[c] == 0;
    bool equal = (a.grid % XCDS) == 0, single = true;
    int64_t units0 = -1;
    for (int g = 0; g < XCDS && ok; ++g) {
      int64_t units_g = 0;
      for (int c = 0; c < R; ++c) units_g += (int64_t)a.gtiles[g] * a.split[c];
      const int64_t wgs_g = (a.grid - g + XCDS - 1) / XCDS;
      if (units0 < 0) units0 = units_g;
      equal = equal && units_g == units0;
      single = single && units_g <= wgs_g;
    }
    if (a.arrived == nullptr) a.static_rr = !ok ? 0 : single ? 2 : equal ? 1 : 0;
    // With flags and no group holding more units than its XCD has
    // workgroups, a workgroup whose first claim got a unit leaves after it:
    // the units number at most the workgroups, so every unit not taken by a
    // first claim leaves a workgroup whose first claim failed, and those keep
    // claiming until no work is left.
    a.one_unit = (a.arrived != nullptr && ok && single) ? 1 : 0;
  }
  // A launch whose claims are all static, with no split chunks, reduce
  // units, flags or stamps, touches no counter: its workgroups skip the exit
  // count too.
  a.no_counters = (a.static_rr != 0 && a.all_unsplit && !fz && !done && !s->stamps) ? 1 : 0;
  if (fz) {
    // shard units are assigned statically (workgroup b takes b, b + grid,
    // ... of each chunk with shard units, in priority order) only when every
    // workgroup's static first claim is a GEMM unit, so no dynamic claim of a
    // shard unit can happen.  Dynamic claims of a ring chunk's units wait for
    // its landing; hundreds of workgroups claiming at each landing would queue
    // on the counters.
    bool exact = true;
    for (int g = 0; g < XCDS; ++g) {
      const int64_t wgs_g = (a.grid - g + XCDS - 1) / XCDS;
      exact = exact && (int64_t)a.gunits[g] == wgs_g;
    }
    a.fused_static = exact ? 1 : 0;
  }

  if (clear_counters) {
    // the counters (claims, completions, split tiles, ready lists) start at zero
    const int64_t words = (int64_t)(p.counter_bytes / sizeof(uint32_t));
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t *>(ws), words);
    const hipError_t ez = hipGetLastError();
    if (ez != hipSuccess) { record(ez); return FO_ERR_HIP; }
  }
  hipError_t e = launch_gemm(a, p.tile, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) { record(e); return FO_ERR_HIP; }
  return FO_OK;
}

// Workspace of fo_ag_gemm_noalloc: one array per GPU, held from the library's
// load until the process ends, shared by every such call on that GPU.  Host
// code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, once per device (scratch_address).
constexpr size_t kNoAllocBytes = FO_NOALLOC_SCRATCH_BYTES;

}  // namespace
}  // namespace fo

static __device__ __align__(256) unsigned char scratch[fo::kNoAllocBytes];

namespace fo {
namespace {

void *g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of this GPU's scratch array (the current device), looked up
// on the first call on that device with the device current.
void *scratch_address() {
  int d = 0;
  const hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) { record(e); return nullptr; }
  if (d < 0 || d >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[d], [d]() {
    void *ptr = nullptr;
    g_scratch_err[d] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[d] = g_scratch_err[d] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[d] != hipSuccess) { record(g_scratch_err[d]); return nullptr; }
  return g_scratch[d];
}

}  // namespace

int device_num_cus() {
  const DevInfo *I = dev_info();
  return I ? I->cus : 0;
}

uint64_t device_wall_hz() {
  const DevInfo *I = dev_info();
  return I ? I->wall_hz : 0;
}

}  // namespace fo

using namespace fo;

extern "C" {

size_t fo_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t nchunks) {
  if (m <= 0 || n <= 0 || k <= 0 || nchunks < 1 || nchunks > FO_MAX_CHUNKS || m % nchunks) return 0;
  if (m / nchunks > (int64_t)1 << 30 || n > (int64_t)1 << 30 || k > kMaxK) return 0;
  return plan_workspace(m, n, k, nchunks).total_bytes;
}

fo_status fo_ag_gemm(const void *x, const void *w, void *y, fo_dtype y_dtype, int64_t m, int64_t n,
                     int64_t k, const fo_schedule *s, void *ws, size_t ws_bytes, void *stream) {
  if (y_dtype != FO_F32 && y_dtype != FO_BF16) return FO_ERR_DTYPE;
  return run_gemm(x, w, y, y_dtype == FO_BF16, nullptr, false, m, n, k, s, ws, ws_bytes, stream);
}

fo_status fo_ag_gemm_noalloc(const void *x, const void *w, void *y, fo_dtype y_dtype, int64_t m, int64_t n,
                             int64_t k, const fo_schedule *s, void *stream) {
  if (y_dtype != FO_F32 && y_dtype != FO_BF16) return FO_ERR_DTYPE;
  if (!x || !w || !y || !s) return FO_ERR_NULL;
  // the problem's workspace bound must fit the scratch array
  const size_t need = fo_workspace_bytes(m, n, k, s->nchunks);
  if (need > kNoAllocBytes) return FO_ERR_WORKSPACE;
  // need == 0 means an invalid shape, which the validation in run_gemm
  // reports before it looks at the workspace
  void *ws = need ? scratch_address() : nullptr;
  if (need && !ws) return FO_ERR_HIP;
  return run_gemm(x, w, y, y_dtype == FO_BF16, nullptr, false, m, n, k, s, ws, kNoAllocBytes, stream,
                  nullptr, true);
}

fo_status fo_a2a_gemm(const void *const *pieces, const void *w, void *y, fo_dtype y_dtype, int64_t m,
                      int64_t n, int64_t k, const fo_schedule *s, void *ws, size_t ws_bytes, void *stream) {
  if (y_dtype != FO_F32 && y_dtype != FO_BF16) return FO_ERR_DTYPE;
  if (!pieces || !w || !y || !s) return FO_ERR_NULL;
  fo_status st = check_schedule(s);
  if (st != FO_OK) return st;
  const int P = s->nchunks;
  for (int q = 0; q < P; ++q)
    if (!pieces[q]) return FO_ERR_NULL;
  if (m <= 0 || n <= 0 || k <= 0 || k % P != 0) return FO_ERR_SHAPE;
  if (m > (int64_t)1 << 30 || n > (int64_t)1 << 30 || k > kMaxK) return FO_ERR_SHAPE;
  const int64_t kp = k / P;
  if (kp % 8 != 0 || !aligned16(w)) return FO_ERR_ALIGN;
  for (int q = 0; q < P; ++q)
    if (!aligned16(pieces[q])) return FO_ERR_ALIGN;
  const bool bf = y_dtype == FO_BF16;
  if (!aligned16(y) && !bf) return FO_ERR_ALIGN;
  if (s->split)
    for (int q = 0; q < P; ++q)
      if (s->split[q] != 1) return FO_ERR_SCHEDULE;
  const size_t ybytes = (size_t)m * n * (bf ? 2 : 4);
  if (overlaps(y, ybytes, w, (size_t)n * k * 2)) return FO_ERR_ALIAS;
  for (int q = 0; q < P; ++q)
    if (overlaps(y, ybytes, pieces[q], (size_t)m * kp * 2)) return FO_ERR_ALIAS;
  if (!ws || ws_bytes < WS_HEADER_BYTES || !aligned16(ws)) return FO_ERR_WORKSPACE;

  const DevInfo *I = dev_info();
  if (!I) return FO_ERR_HIP;
  A2aArgs a{};
  for (int q = 0; q < P; ++q) a.piece[q] = static_cast<const uint16_t *>(pieces[q]);
  a.w = static_cast<const uint16_t *>(w);
  a.y = y;
  a.y_bf16 = bf ? 1 : 0;
  a.m = m; a.n = n; a.k = k;
  a.kp = (int32_t)kp;
  a.P = P;
  a.local = s->local;
  // default order: the piece already present, then the peers' pieces in the
  // order pairwise exchange delivers them (local-1, local-2, ...)
  if (s->order) {
    for (int i = 0; i < P; ++i) a.order[i] = s->order[i];
  } else {
    for (int i = 0; i < P; ++i) a.order[i] = ((s->local - i) % P + P) % P;
  }
  a.tiles_m = (int32_t)((m + A2A_BM - 1) / A2A_BM);
  a.tiles_n = (int32_t)((n + A2A_BN - 1) / A2A_BN);
  {
    // the rectangle shape whose operand rows per XCD are fewest
    const int shapes[4][2] = {{1, 8}, {2, 4}, {4, 2}, {8, 1}};
    int64_t best = -1;
    for (const auto &sh : shapes) {
      const int gm = sh[0], gn = sh[1];
      int64_t cost = (int64_t)((a.tiles_m + gm - 1) / gm) * A2A_BM + (int64_t)((a.tiles_n + gn - 1) / gn) * A2A_BN;
      if (gm > a.tiles_m || gn > a.tiles_n) cost += (int64_t)1 << 40;   // empty rectangles
      if (best < 0 || cost < best) { best = cost; a.gm = gm; a.gn = gn; }
    }
    for (int g = 0; g < XCDS; ++g) {
      const int i = g / a.gn, j = g % a.gn;
      const int rows = (i + 1) * a.tiles_m / a.gm - i * a.tiles_m / a.gm;
      const int cols = (j + 1) * a.tiles_n / a.gn - j * a.tiles_n / a.gn;
      a.gtiles[g] = rows * cols;
    }
  }
  // one workgroup per CU at most (the whole grid resident), none without a
  // tile: each XCD's workgroups share its rectangle's tiles
  const int full = I->cus;
  const int cap = (s->max_workgroups > 0 && s->max_workgroups < full) ? s->max_workgroups : full;
  int grid = 0;
  for (int g = 0; g < XCDS; ++g) {
    const int wgs_g = (cap - g + XCDS - 1) / XCDS;
    const int use = a.gtiles[g] < wgs_g ? a.gtiles[g] : wgs_g;
    // workgroup b sits on XCD b % 8: the grid must reach rank use - 1 on XCD g
    if (use > 0 && (use - 1) * XCDS + g + 1 > grid) grid = (use - 1) * XCDS + g + 1;
    // a workgroup computes only its own XCD's rectangle: every rectangle
    // with tiles needs a workgroup, whatever the cap
    if (a.gtiles[g] > 0 && grid < g + 1) grid = g + 1;
  }
  a.grid = grid < 1 ? 1 : grid;
  a.arrived = s->arrived;
  a.epoch = s->epoch;
  a.timeout_ticks = ns_to_ticks(s->timeout_ns ? s->timeout_ns : kDefaultTimeoutNs, I->wall_hz);
  a.status = s->status;
  a.stamps = s->stamps;
  a.ws32 = static_cast<uint32_t *>(ws);
  const hipError_t e = launch_a2a(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) { record(e); return FO_ERR_HIP; }
  return FO_OK;
}

namespace {

// Query-split attention workspace: counters, then one partial slot per
// (head, query tile, key chunk).
struct QsaPlan {
  int64_t conv_off;
  size_t part_offset, vt_offset, total;
};

// Workspace: counters (stage claims and the rest of the header, one per
// query tile, one per (chunk, head) conversion), the partial slots, then the
// fp16 value images.
QsaPlan qsa_plan(int64_t seq, int64_t heads, int32_t R) {
  const int64_t tiles = seq / QSA_BQ;
  QsaPlan p{};
  p.conv_off = QSA_DONE + heads * tiles;
  p.part_offset = ((size_t)(p.conv_off + (int64_t)R * heads) * sizeof(uint32_t) + 255) & ~(size_t)255;
  p.vt_offset = p.part_offset + (size_t)heads * tiles * R * (QSA_BQ * QSA_D + 2 * QSA_BQ) * sizeof(float);
  p.total = p.vt_offset + (size_t)heads * seq * QSA_D * sizeof(uint16_t);
  return p;
}

fo_status qsa_shape(int64_t seq, int32_t heads, int32_t head_dim, int32_t R) {
  if (R < 1 || R > QSA_MAX_CHUNKS) return FO_ERR_SHAPE;
  if (seq <= 0 || heads <= 0 || head_dim != QSA_D || seq % R != 0) return FO_ERR_SHAPE;
  const int64_t chunk = seq / R;
  if (chunk % QSA_BQ != 0) return FO_ERR_SHAPE;
  // a chunk of qkv rows is addressed with 32-bit byte offsets
  if (chunk * 3 * (int64_t)heads * QSA_D * 2 >= ((int64_t)1 << 31) || seq > ((int64_t)1 << 30)) return FO_ERR_SHAPE;
  return FO_OK;
}

}  // namespace

size_t fo_qsa_workspace_bytes(int64_t seq, int32_t heads, int32_t head_dim, int32_t nchunks) {
  if (qsa_shape(seq, heads, head_dim, nchunks) != FO_OK) return 0;
  return qsa_plan(seq, heads, nchunks).total;
}

fo_status fo_qsa_attention(const void *qkv, void *o, fo_dtype o_dtype, int64_t seq, int32_t heads,
                           int32_t head_dim, int32_t causal, const fo_schedule *s, void *ws, size_t ws_bytes,
                           void *stream) {
  if (o_dtype != FO_F32 && o_dtype != FO_BF16) return FO_ERR_DTYPE;
  if (!qkv || !o || !s) return FO_ERR_NULL;
  fo_status st = check_schedule(s);
  if (st != FO_OK) return st;
  const int R = s->nchunks;
  st = qsa_shape(seq, heads, head_dim, R);
  if (st != FO_OK) return st;
  if (causal != 0 && causal != 1) return FO_ERR_SCHEDULE;
  if (s->split)
    for (int c = 0; c < R; ++c)
      if (s->split[c] != 1) return FO_ERR_SCHEDULE;
  const bool bf = o_dtype == FO_BF16;
  if (!aligned16(qkv) || !aligned16(o)) return FO_ERR_ALIGN;
  const size_t obytes = (size_t)seq * heads * QSA_D * (bf ? 2 : 4);
  if (overlaps(o, obytes, qkv, (size_t)seq * 3 * heads * QSA_D * 2)) return FO_ERR_ALIAS;
  const QsaPlan plan = qsa_plan(seq, heads, R);
  if (!ws || ws_bytes < plan.total || !aligned16(ws)) return FO_ERR_WORKSPACE;
  if (overlaps(ws, plan.total, o, obytes) || overlaps(ws, plan.total, qkv, (size_t)seq * 3 * heads * QSA_D * 2))
    return FO_ERR_ALIAS;

  const DevInfo *I = dev_info();
  if (!I) return FO_ERR_HIP;
  QsaArgs a{};
  a.qkv = static_cast<const uint16_t *>(qkv);
  a.o = o;
  a.o_bf16 = bf ? 1 : 0;
  a.S = (int32_t)seq;
  a.H = heads;
  a.R = R;
  a.causal = causal;
  a.chunk = (int32_t)(seq / R);
  a.tiles = a.chunk / QSA_BQ;
  a.local = s->local;
  // default order: the local chunk, then the others in ring landing order
  if (s->order) {
    for (int i = 0; i < R; ++i) a.order[i] = s->order[i];
  } else {
    for (int i = 0; i < R; ++i) a.order[i] = ((s->local - i) % R + R) % R;
  }
  // Stage s: the (query chunk, key chunk) pairs whose later chunk in `order`
  // is order[s]: the new chunk's queries against the earlier chunks' keys
  // and the earlier queries against its keys, then the new chunk with
  // itself.  With the causal mask, pairs whose keys all follow the queries
  // are empty and left out.
  int np = 0;
  const int per_pair = heads * a.tiles;
  // With arrival flags, two groups of 4 waves share each block (one
  // workgroup per CU): the blocks of the chunk that lands last then use every
  // CU.  With every chunk present, one group per workgroup and two workgroups
  // per CU.
  a.groups = s->arrived != nullptr ? 2 : 1;
  a.conv_units = heads * (a.chunk / (a.groups * QSA_BKV));   // (head, key tiles of one unit) of the chunk
  for (int sg = 0; sg < R; ++sg) {
    a.stage_pair0[sg] = np;
    const int cs = a.order[sg];
    auto add = [&](int qc, int kc) {
      if (causal && kc > qc) return;
      a.pair_q[np] = (int8_t)qc;
      a.pair_k[np] = (int8_t)kc;
      ++np;
    };
    for (int p = 0; p < sg; ++p) {
      add(cs, a.order[p]);
      add(a.order[p], cs);
    }
    add(cs, cs);
    a.stage_units[sg] = (np - a.stage_pair0[sg]) * per_pair;
    // each stage opens with the conversion units of its new chunk; with the
    // causal mask the stage's last pair is its diagonal one
    a.stage_units[sg] += a.conv_units;
    a.stage_big[sg] = causal ? a.stage_units[sg] - per_pair : a.stage_units[sg];
  }
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)QSA_D));
  const int64_t blocks = (int64_t)np * per_pair;
  const int full = a.groups == 2 ? I->cus : 2 * I->cus;   // 8 waves per CU either way
  const int cap = (s->max_workgroups > 0 && s->max_workgroups < full) ? s->max_workgroups : full;
  a.grid = (int32_t)(blocks < cap ? blocks : cap);
  if (a.grid < 1) a.grid = 1;
  // With arrival flags every claim group needs a workgroup of its own: a
  // group's workgroups claim its conversion units before any block, and a
  // block may wait for the conversions dealt to any group.  (Workgroups
  // with nothing left to claim leave at once.)
  if (s->arrived != nullptr && a.grid < XCDS) a.grid = XCDS < full ? XCDS : full;
  a.arrived = s->arrived;
  a.epoch = s->epoch;
  a.timeout_ticks = ns_to_ticks(s->timeout_ns ? s->timeout_ns : kDefaultTimeoutNs, I->wall_hz);
  a.status = s->status;
  a.stamps = s->stamps;
  a.ws32 = static_cast<uint32_t *>(ws);
  a.part = reinterpret_cast<float *>(static_cast<char *>(ws) + plan.part_offset);
  a.vt = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + plan.vt_offset);
  a.conv_off = (int32_t)plan.conv_off;
  const hipError_t e = launch_qsa(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) { record(e); return FO_ERR_HIP; }
  return FO_OK;
}

fo_status fo_gemm_rs(const void *x, const void *w, float *partial, uint32_t *done, int64_t m,
                     int64_t n, int64_t k, const fo_schedule *s, void *ws, size_t ws_bytes,
                     void *stream) {
  return run_gemm(x, w, partial, false, done, true, m, n, k, s, ws, ws_bytes, stream);
}

fo_status fo_gemm_rs_reduce(const void *x, const void *w, float *partial, uint32_t *done,
                            void *shard, fo_dtype shard_dtype, const float *const *incoming,
                            int64_t m, int64_t n, int64_t k, const fo_schedule *s, void *ws,
                            size_t ws_bytes, void *stream) {
  if (shard_dtype != FO_F32 && shard_dtype != FO_BF16) return FO_ERR_DTYPE;
  const FusedRs fz{shard, shard_dtype == FO_BF16, incoming, false};
  return run_gemm(x, w, partial, false, done, true, m, n, k, s, ws, ws_bytes, stream, &fz);
}

fo_status fo_gemm_rs_ring(const void *x, const void *w, float *partial, uint32_t *done, void *shard,
                          fo_dtype shard_dtype, const float *const *incoming, int64_t m, int64_t n,
                          int64_t k, const fo_schedule *s, void *ws, size_t ws_bytes, void *stream) {
  if (shard_dtype != FO_F32 && shard_dtype != FO_BF16) return FO_ERR_DTYPE;
  const FusedRs fz{shard, shard_dtype == FO_BF16, incoming, true};
  return run_gemm(x, w, partial, false, done, true, m, n, k, s, ws, ws_bytes, stream, &fz);
}

fo_status fo_chunk_reduce(void *dst, fo_dtype dst_dtype, const float *const *srcs, int64_t n,
                          const fo_schedule *s, void *stream) {
  if (!dst || !srcs || !s) return FO_ERR_NULL;
  fo_status st = check_schedule(s);
  if (st != FO_OK) return st;
  if (dst_dtype != FO_F32 && dst_dtype != FO_BF16) return FO_ERR_DTYPE;
  const int R = s->nchunks;
  if (n <= 0) return FO_ERR_SHAPE;
  if (n % 4 != 0) return FO_ERR_ALIGN;
  for (int i = 0; i < R; ++i) {
    if (!srcs[i]) return FO_ERR_NULL;
    if (!aligned16(srcs[i])) return FO_ERR_ALIGN;
  }
  if (!aligned16(dst)) return FO_ERR_ALIGN;
  const size_t nb = (size_t)n * 4, db = (size_t)n * (dst_dtype == FO_BF16 ? 2 : 4);
  // dst may equal srcs[local] exactly (fp32, in place); any other overlap is refused
  for (int i = 0; i < R; ++i) {
    if (dst_dtype == FO_F32 && i == s->local && dst == (const void *)srcs[i]) continue;
    if (overlaps(dst, db, srcs[i], nb)) return FO_ERR_ALIAS;
  }
  for (int i = 0; i < R; ++i)
    for (int j = i + 1; j < R; ++j)
      if (overlaps(srcs[i], nb, srcs[j], nb)) return FO_ERR_ALIAS;

  const DevInfo *I = dev_info();
  if (!I) return FO_ERR_HIP;

  int32_t order[FO_MAX_CHUNKS];
  expand_order(s, order);
  ReduceArgs a{};
  int q = 0;
  a.src[q] = srcs[s->local];
  a.chunk_of[q++] = s->local;
  for (int i = 0; i < R; ++i) {
    if (order[i] == s->local) continue;
    a.src[q] = srcs[order[i]];
    a.chunk_of[q++] = order[i];
  }
  a.dst = dst;
  a.dst_bf16 = dst_dtype == FO_BF16 ? 1 : 0;
  a.acc = dst_dtype == FO_F32 ? static_cast<float *>(dst) : const_cast<float *>(srcs[s->local]);
  a.R = R;
  a.n4 = n / 4;
  a.arrived = s->arrived;
  a.epoch = s->epoch;
  a.timeout_ticks = ns_to_ticks(s->timeout_ns ? s->timeout_ns : kDefaultTimeoutNs, I->wall_hz);
  a.status = s->status;
  a.stamps = s->stamps;

  // 8 vectors of every source per lane per step: the most bytes in flight
  // measured best (8 x 2^27 sources: 5.7 TB/s, against 5.1 with 2 vectors).
  // Those registers leave room for one workgroup per CU (and for the
  // emulator's one-wave kernels beside it).  Without flags the grid is 8
  // workgroups per CU, run one after another on each CU; with flags every
  // workgroup must be resident (each waits for its sources in passes), so
  // the grid is one per CU.
  int grid = s->max_workgroups > 0 ? s->max_workgroups : (a.arrived ? I->cus : I->cus * 8);
  const int64_t min_per = 256 * 8;   // one full step of the workgroup
  // a workgroup's range is addressed with 32-bit byte offsets (at most 1 GiB
  // per workgroup; the grid grows past max_workgroups if it must)
  const int64_t max_per = ((int64_t)1 << 30) / 16;
  int64_t per = (a.n4 + grid - 1) / grid;
  if (per < min_per) per = min_per;
  per = (per + 255) / 256 * 256;
  if (per > max_per) per = max_per;
  a.per_wg4 = per;
  grid = (int)((a.n4 + per - 1) / per);
  hipError_t e = launch_reduce(a, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) { record(e); return FO_ERR_HIP; }
  return FO_OK;
}

fo_status fo_emulate_arrivals(void *const *dst, const void *const *src, const size_t *bytes,
                              const int64_t *issue_ns, const int64_t *release_ns,
                              const int32_t *chunk_id, int32_t count, uint32_t *arrived,
                              uint32_t epoch, uint64_t *stamps, void *stream) {
  return fo_emulate_arrivals_gated(nullptr, 0, dst, src, bytes, issue_ns, release_ns, chunk_id, count,
                                   arrived, epoch, stamps, stream);
}

fo_status fo_emulate_arrivals_gated(const uint64_t *gate, uint64_t gate_timeout_ns, void *const *dst,
                                    const void *const *src, const size_t *bytes,
                                    const int64_t *issue_ns, const int64_t *release_ns,
                                    const int32_t *chunk_id, int32_t count, uint32_t *arrived,
                                    uint32_t epoch, uint64_t *stamps, void *stream) {
  if (count < 0) return FO_ERR_SHAPE;
  if (count == 0) return FO_OK;
  if (!dst || !src || !bytes || !release_ns || !chunk_id || !arrived || !stamps) return FO_ERR_NULL;
  if (epoch == 0) return FO_ERR_SCHEDULE;
  for (int i = 0; i < count; ++i) {
    if (chunk_id[i] < 0 || chunk_id[i] >= FO_MAX_CHUNKS) return FO_ERR_SCHEDULE;
    if (release_ns[i] < 0 || (issue_ns && (issue_ns[i] < 0 || issue_ns[i] > release_ns[i])))
      return FO_ERR_SCHEDULE;
    if (bytes[i] && (!dst[i] || !src[i])) return FO_ERR_NULL;
  }
  const DevInfo *I = dev_info();
  if (!I) return FO_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto issue_at = [&](int i) -> uint64_t { return (uint64_t)(issue_ns ? issue_ns[i] : release_ns[i]); };
  const uint64_t gate_ns = gate_timeout_ns ? gate_timeout_ns : kDefaultTimeoutNs;
  hipError_t e = launch_emu_start(stamps, ns_to_ticks(issue_at(0), I->wall_hz), gate,
                                  ns_to_ticks(gate_ns, I->wall_hz), st);
  for (int i = 0; i < count && e == hipSuccess; ++i) {
    if (bytes[i]) e = hipMemcpyAsync(dst[i], src[i], bytes[i], hipMemcpyDeviceToDeviceNoCU, st);
    if (e != hipSuccess) break;
    const uint64_t next = (i + 1 < count) ? ns_to_ticks(issue_at(i + 1), I->wall_hz) : 0;
    e = launch_emu_flag(stamps, ns_to_ticks((uint64_t)release_ns[i], I->wall_hz), next,
                        arrived + chunk_id[i], epoch, stamps + 1 + chunk_id[i], st);
  }
  if (e != hipSuccess) { record(e); return FO_ERR_HIP; }
  return FO_OK;
}

fo_status fo_emulate_sends(const uint32_t *done, uint32_t epoch, void *const *dst, const void *const *src,
                           const size_t *bytes, const int32_t *chunk_id, const int64_t *link_ns, int32_t count,
                           uint64_t timeout_ns, int32_t *status, uint64_t *stamps, void *stream) {
  if (count < 0) return FO_ERR_SHAPE;
  if (count == 0) return FO_OK;
  if (!done || !dst || !src || !bytes || !chunk_id || !link_ns || !stamps) return FO_ERR_NULL;
  if (epoch == 0) return FO_ERR_SCHEDULE;
  for (int i = 0; i < count; ++i) {
    if (chunk_id[i] < 0 || chunk_id[i] >= FO_MAX_CHUNKS || link_ns[i] < 0) return FO_ERR_SCHEDULE;
    if (bytes[i] && (!dst[i] || !src[i])) return FO_ERR_NULL;
  }
  const DevInfo *I = dev_info();
  if (!I) return FO_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint64_t tmo = ns_to_ticks(timeout_ns ? timeout_ns : kDefaultTimeoutNs, I->wall_hz);
  hipError_t e = hipSuccess;
  for (int i = 0; i < count && e == hipSuccess; ++i) {
    e = launch_emu_wait_flag(done + chunk_id[i], epoch, tmo, status, stamps + 2 * i, st);
    if (e == hipSuccess && bytes[i]) e = hipMemcpyAsync(dst[i], src[i], bytes[i], hipMemcpyDeviceToDeviceNoCU, st);
    if (e == hipSuccess) e = launch_emu_hold(stamps + 2 * i, ns_to_ticks((uint64_t)link_ns[i], I->wall_hz),
                                             stamps + 2 * i + 1, st);
  }
  if (e != hipSuccess) { record(e); return FO_ERR_HIP; }
  return FO_OK;
}

fo_status fo_device_info(int32_t *num_cus, int32_t *lds_bytes_per_cu, uint64_t *wall_clock_hz) {
  const DevInfo *I = dev_info();
  if (!I) return FO_ERR_HIP;
  if (num_cus) *num_cus = I->cus;
  if (lds_bytes_per_cu) *lds_bytes_per_cu = I->lds;
  if (wall_clock_hz) *wall_clock_hz = I->wall_hz;
  return FO_OK;
}

const char *fo_status_string(fo_status st) {
  switch (st) {
    case FO_OK: return "ok";
    case FO_ERR_NULL: return "a required pointer is NULL";
    case FO_ERR_SHAPE: return "invalid shape (non-positive size, m % R != 0 or R out of range)";
    case FO_ERR_ALIGN: return "pointer not 16-byte aligned or k/n not a multiple of the vector width";
    case FO_ERR_DTYPE: return "unsupported dtype";
    case FO_ERR_ORDER: return "order is not a permutation of 0..R-1";
    case FO_ERR_SCHEDULE: return "invalid schedule (local, epoch, mode, split or arrival times)";
    case FO_ERR_WORKSPACE: return "workspace missing or too small";
    case FO_ERR_HIP: return "HIP runtime error";
    case FO_ERR_TIMEOUT: return "a flag wait exceeded the timeout";
    case FO_ERR_ALIAS: return "buffers overlap";
    default: return "unknown status";
  }
}

const char *fo_last_hip_error(void) { return g_hip_err; }

}  // extern "C"
