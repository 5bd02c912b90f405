// Persistent chunked GEMM for gfx950: bf16 MFMA (16x16x32), fp32 accumulate,
// operand tiles copied straight into an LDS ring by the buffer-load DMA path,
// work claimed chunk by chunk as the chunks' epoch flags show them landed.
//
// This is the partitioned computation of FlashOverlap (euno.news
// "Methodology" step 2: the GEMM is split into sub-tasks on the same row
// slices that are communicated) with the rank-adaptive order of the
// gist.science technical summary §2: work whose input depends on incoming
// chunks is claimed in `order` as soon as it lands; the chunk already present
// (local) is taken whenever nothing else is ready, so after the last landing
// only that chunk's work remains (Flash-AG), and in GEMM-RS mode the chunk that
// stays local is produced last (Flash-RS).
//
// Layout and schedule
//  - One persistent workgroup per CU computes BM x BN output tiles.  Its
//    compute waves form a WGM x WGN grid, each wave owning a block of 16x16
//    MFMA tiles: 4 waves (one per SIMD) or 8 (two per SIMD, under a register
//    cap that leaves room for a one-wave kernel beside the grid).  In the
//    producer/consumer layout 4 of the 8 waves only issue and wait for the
//    copies while the other 4 only read fragments and multiply.
//  - Operand tiles of BM x BK (X rows) and BN x BK (W rows = output columns)
//    sit in an LDS ring of STAGES buffers with a 16-byte XOR swizzle, so the
//    fragment reads of 8 consecutive rows hit distinct bank groups.
//  - The copy engine behind the buffer loads writes each stage straight into
//    LDS (no register staging, no LDS store instructions); STAGES-1 stages are
//    in flight while one is multiplied, one barrier per stage.
//  - Each chunk's tile grid is cut into 8 rectangles, one per XCD (workgroup
//    b runs on XCD b % 8); a workgroup claims from its own XCD's rectangle
//    first, so each XCD's L2 serves a few X row blocks and W column blocks to
//    its 32 CUs, and steals from the chunk's other rectangles when its own is
//    empty.  The host picks the rectangle shape that minimises the operand
//    rows one XCD streams over all chunks.
#include "fo_device.hpp"
#include "fo_internal.hpp"
#include "fo_tile.hpp"

#include <stdio.h>
#include <stdlib.h>
#include <type_traits>
#include <utility>

namespace fo {

struct ClaimState {
  uint64_t acquired;   // bit c: this workgroup has done the acquire for chunk c
  int taken;           // units taken so far (static round-robin)
};

struct Unit {
  int c;      // chunk, -1 finished, -2 abort
  int tm, tn; // tile row / column inside the chunk
  int sp;     // split index, or the row slice of a reduce unit
  int first;  // 1 for the first unit of group 0 (chunk start stamp)
  int red;    // 1: reduce unit (sum a split tile's partials over one row slice)
};

__device__ __forceinline__ uint32_t group_units(const GemmArgs &a, int c, int g) {
  return (uint32_t)(a.gtiles[g] * a.split[c]);
}

// Without arrival flags every chunk is present from the start, so each
// workgroup's first unit is assigned statically: the q-th workgroup of XCD g
// takes the q-th unit of group g in priority order, with no atomic.  The
// claim counter of (c, g) then counts the units after these: this returns
// how many units of (c, g) the static assignment covers.
__device__ __forceinline__ uint32_t static_units(const GemmArgs &a, int c, int g) {
  if (a.arrived != nullptr) return 0;
  const int wgs = (a.grid - g + XCDS - 1) / XCDS;   // workgroups on XCD g
  int off = 0;
  for (int sidx = 0; sidx < a.R; ++sidx) {
    const int cc = a.order[sidx];
    const int nu = (int)group_units(a, cc, g);
    if (cc == c) {
      const int left = wgs - off;
      return left <= 0 ? 0u : (uint32_t)(left < nu ? left : nu);
    }
    off += nu;
  }
  return 0u;
}

// Group g of a chunk is rectangle (g / gn, g % gn) of the chunk's tile grid,
// cut into gm row bands and gn column bands; its tiles are numbered row by
// row.  Rectangle g is the XCD g queue, so an XCD streams a few X row blocks
// and a few W column blocks instead of every row block of the chunk.
__device__ __forceinline__ void group_tile(const GemmArgs &a, int g, int tl, int &tm, int &tn) {
  const int i = g / a.gn, j = g - (g / a.gn) * a.gn;
  const int rlo = i * a.tiles_m / a.gm;
  const int clo = j * a.tiles_n / a.gn, chi = (j + 1) * a.tiles_n / a.gn;
  const int ncols = chi - clo;
  tm = rlo + tl / ncols;
  tn = clo + tl - (tl / ncols) * ncols;
}

// Reduce unit v of chunk c: wait (wave 0, all lanes) until the v / RED_SLICES-th
// tile of the chunk is published on its ready list, then fill r.  A split
// tile is published once all its splits are written: every split unit waits
// for its written-through stores before it counts itself, and the tile
// counter reads S only after all S splits counted themselves.  The reduce
// unit then reads the partials with system-coherent loads, which do not hit
// a stale line in any cache, so it needs no fence (an acquire fence would
// invalidate the XCD's whole L2 once per reduce unit).  An unsplit tile (the
// fused shard units) is published by its only unit after its written-through
// stores and read the same way.  On abort or timeout r.c = -2.
__device__ __forceinline__ void take_reduce_unit(const GemmArgs &a, int c, uint32_t v, Unit &r) {
  const int lane = threadIdx.x & 63;
  uint32_t e = 0;
  if (lane == 0) {
    const uint32_t *slot = a.ws32 + a.ready_off + a.ctr_base[c] + v / RED_SLICES;
    const uint64_t t0 = now_ticks();
    while ((e = load_relaxed(slot)) == 0u) {
      if (load_relaxed(a.ws32 + WS_ABORT) || now_ticks() - t0 > a.timeout_ticks) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  e = __builtin_amdgcn_readfirstlane(e);
  if (e == 0u) {   // abort or timeout while waiting
    if (lane == 0) {
      if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(a.ws32 + WS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    r.c = -2;
    return;
  }
  const int tile = (int)e - 1;
  if (a.split[c] > 1) {
    if (lane == 0) {
      const uint32_t *ctr = a.ws32 + WS_TILE_CTR + a.ctr_base[c] + tile;
      const uint64_t t0 = now_ticks();   // bounded like every other wait
      while (load_relaxed_agent(ctr) < (uint32_t)a.split[c] && now_ticks() - t0 <= a.timeout_ticks)
        __builtin_amdgcn_s_sleep(1);
    }
  }
  r.c = c;
  r.tm = tile / a.tiles_n;
  r.tn = tile - r.tm * a.tiles_n;
  r.sp = (int)(v % RED_SLICES);
  r.first = 0;
  r.red = 1;
}

// Wave 0 of a workgroup picks the next unit (all 64 lanes call this).
// One round trip reads every arrival flag and every claim counter in
// parallel across the lanes; then a scan in priority order takes the first
// chunk that has landed and has work: a GEMM unit (its own XCD's group if
// that has work, else the group with the most left) with one fetch-add, or,
// once every GEMM unit of a split chunk is claimed, one of its reduce units.
// A reduce unit may be claimed before its tile is published; it then waits
// for a split that is already running, never for unclaimed work.
// STRICT mode only looks at the first chunk in order that still has work.
__device__ Unit claim_unit(const GemmArgs &a, ClaimState &st, int xg, int &rank_hint) {
  const int lane = threadIdx.x & 63;
  const int R = a.R;
  uint64_t wait_from = 0;
  Unit r{-1, 0, 0, 0, 0, 0};
  // First claim of a workgroup: the q-th unit of its own XCD's group in
  // priority order (q = its rank on the XCD).  Without flags it is taken
  // statically (see static_units).  With flags it is the q-th unit over the
  // landed chunks, taken as if no unit were claimed yet (true at the start
  // of a call), so only the flags are read before the fetch-add; if that
  // shows the group exhausted, the general claim below takes over.
  // Static round-robin (no arrival flags, no reduce units, XCD groups of
  // equal size): the q-th workgroup of XCD g takes units q, q + W, q + 2W, ...
  // of group g in priority order (W = workgroups on the XCD), with no atomic.
  // Claims by hundreds of workgroups at once would otherwise queue on the
  // counters' cache lines.  When no workgroup gets a second unit
  // (static_rr == 2) the first unit comes from the static first claim below
  // and the next claim ends the workgroup.
  // Fused shard units with one GEMM unit per workgroup: after its static
  // first unit, workgroup b takes shard units b, b + grid, ... of each chunk
  // that has them, in priority order (no claim counter; a unit waits for its
  // chunk's incoming partials itself).
  if (a.fused_static && rank_hint < 0) {
    // the t-th shard unit of this workgroup: units b, b + grid, ... of each
    // chunk with shard units (every such chunk has the same number), chunks
    // in priority order (the landing order)
    const int t = st.taken++;
    const int b = (int)blockIdx.x;
    const int U = a.red_units[a.shard_seq[0]];
    const int nu = U > b ? (U - b + a.grid - 1) / a.grid : 0;
    if (nu == 0 || t >= nu * a.nshard) return r;
    const int i = t / nu;
    take_reduce_unit(a, a.shard_seq[i], (uint32_t)(b + (t - i * nu) * a.grid), r);
    return r;
  }
  if (a.static_rr == 2 && rank_hint < 0) return r;   // one unit per workgroup: done
  if (a.one_unit && st.taken == 1) return r;          // first claim got a unit: done
  if (a.static_rr == 1) {
    const int wgs = (a.grid - xg + XCDS - 1) / XCDS;
    uint32_t q = (uint32_t)((int)(blockIdx.x / XCDS) + st.taken * wgs);
    ++st.taken;
    rank_hint = -1;
    if (q >= (uint32_t)a.gunits[xg]) return r;   // this workgroup's share is done
    if (a.all_unsplit) {
      // every chunk holds gtiles[g] units in group g: no walk over the order
      const int gt = a.gtiles[xg];
      const int sidx = (int)q / gt, tl = (int)q - sidx * gt;
      r.c = a.order[sidx];
      r.sp = 0;
      group_tile(a, xg, tl, r.tm, r.tn);
      r.first = (xg == 0 && tl == 0);
      r.red = 0;
      return r;
    }
    for (int sidx = 0; sidx < R; ++sidx) {
      const int c = a.order[sidx];
      const uint32_t nu = group_units(a, c, xg);
      if (q < nu) {
        const int S = a.split[c];
        const int tl = (int)q / S;
        r.c = c;
        r.sp = (int)q - tl * S;
        group_tile(a, xg, tl, r.tm, r.tn);
        r.first = (xg == 0 && q == 0);
        r.red = 0;
        return r;
      }
      q -= nu;
    }
    return r;
  }
  if (rank_hint >= 0 && a.arrived == nullptr) {
    uint32_t q = (uint32_t)rank_hint;
    rank_hint = -1;
    for (int sidx = 0; sidx < R; ++sidx) {
      const int c = a.order[sidx];
      const uint32_t nu = group_units(a, c, xg);
      if (q < nu) {
        const int S = a.split[c];
        const int tl = (int)q / S;
        r.c = c;
        r.sp = (int)q - tl * S;
        group_tile(a, xg, tl, r.tm, r.tn);
        r.first = (xg == 0 && q == 0);
        r.red = 0;
        return r;
      }
      q -= nu;
    }
  }
  if (rank_hint >= 0 && !a.strict) {
    bool ok = false;
    if (lane < R) {
      const int c = a.order[lane];
      ok = a.arrived == nullptr || c == a.local || epoch_reached(load_relaxed(a.arrived + c), a.epoch);
    }
    const uint64_t landed = __ballot(ok);
    uint32_t q = (uint32_t)rank_hint;
    int pick = -1;
    for (int sidx = 0; sidx < R; ++sidx) {
      if (!((landed >> sidx) & 1)) continue;
      const uint32_t nu = group_units(a, a.order[sidx], xg);
      if (q < nu) { pick = a.order[sidx]; break; }
      q -= nu;
    }
    if (pick >= 0) {
      rank_hint = -1;
      if (a.arrived != nullptr && pick != a.local) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
      st.acquired |= 1ull << pick;
      uint32_t u = 0;
      if (lane == 0) u = fetch_add_relaxed(a.ws32 + WS_CLAIM + pick * XCDS + xg, 1u);
      u = __builtin_amdgcn_readfirstlane(u);
      if (u < group_units(a, pick, xg)) {
        const int S = a.split[pick];
        const int tl = (int)u / S;
        st.taken = 1;
        r.c = pick;
        r.sp = (int)u - tl * S;
        group_tile(a, xg, tl, r.tm, r.tn);
        r.first = (xg == 0 && u == 0);
        r.red = 0;
        return r;
      }
    }
  }
  for (;;) {
    // landed[s]: chunk order[s] usable; red[s]: split chunk with reduce units left
    // ring form: a chunk's shard units wait for its incoming partial, so they
    // are claimable only once it has landed (blocked: units left, not landed)
    bool ok = false, redp = false, blk = false;
    if (lane < R) {
      const int c = a.order[lane];
      ok = a.arrived == nullptr || c == a.local ||
           epoch_reached(load_relaxed(a.arrived + c), a.epoch);
      if (a.red_units[c] > 0) redp = load_relaxed(a.ws32 + WS_RED_CLAIM + c) < (uint32_t)a.red_units[c];
      if (redp && a.ring && a.inc_arrived != nullptr && a.inc[c] != nullptr &&
          !epoch_reached(load_relaxed(a.inc_arrived + c), a.epoch)) {
        redp = false;
        blk = true;
      }
    }
    const uint64_t landed = __ballot(ok);
    const uint64_t red_left = __ballot(redp);
    const uint64_t red_blocked = __ballot(blk);
    // GEMM units left per (order position, group), 8 positions per batch of
    // 64 lanes; each batch is looked at as it is read (no arrays indexed at
    // run time: the compiler would keep them in registers across the whole
    // persistent loop).  has_work covers every batch read so far; the walk
    // stops early only at a pick or at a chunk with work left, so has_work is
    // nonzero whenever the walk did not reach the end.
    const int nb = (R + 7) / 8;
    uint64_t has_work = 0;
    int pick_s = -1, pick_g = -1, pick_red = 0;
    bool stop = false;
#pragma nounroll
    for (int b = 0; b < nb && !stop; ++b) {
      const int pidx = b * 64 + lane;
      uint32_t lv = 0;
      if (pidx < R * XCDS) {
        const int sidx = pidx / XCDS, g = pidx % XCDS;
        const int c = a.order[sidx];
        const uint32_t cnt = load_relaxed(a.ws32 + WS_CLAIM + c * XCDS + g) + static_units(a, c, g);
        const uint32_t tot = group_units(a, c, g);
        lv = cnt < tot ? tot - cnt : 0;
      }
      const uint64_t gmb = __ballot(lv > 0);
      for (uint64_t mm = gmb; mm; mm &= mm - 1) has_work |= 1ull << (b * 8 + __builtin_ctzll(mm) / XCDS);
      const int s_end = R < b * 8 + 8 ? R : b * 8 + 8;
      for (int sidx = b * 8; sidx < s_end; ++sidx) {
        const uint64_t gm = (gmb >> ((sidx % 8) * XCDS)) & 0xFFull;
        const bool redw = ((red_left >> sidx) & 1) && gm == 0;
        if (!gm && !redw) continue;
        const bool is_landed = (landed >> sidx) & 1;
        if (!is_landed) {
          if (a.strict) { stop = true; break; }   // strict: the first chunk with work decides
          continue;
        }
        if (gm) {
          // first claim of a workgroup: the q-th workgroup of an XCD skips the
          // first q units its XCD's group has left (in priority order over
          // landed chunks), so the XCD's workgroups start on distinct units
          if (rank_hint >= 0 && !a.strict && ((gm >> xg) & 1)) {
            const uint32_t own = __shfl(lv, (sidx % 8) * XCDS + xg);
            if ((uint32_t)rank_hint >= own) { rank_hint -= (int)own; continue; }
          }
          pick_s = sidx;
          if ((gm >> xg) & 1) {
            pick_g = xg;
          } else {
            uint32_t best = 0;
            for (uint64_t g2 = gm; g2; g2 &= g2 - 1) {
              const int g = __builtin_ctzll(g2);
              const uint32_t lg = __shfl(lv, (sidx % 8) * XCDS + g);
              if (lg > best) { best = lg; pick_g = g; }
            }
          }
        } else {
          pick_s = sidx;
          pick_red = 1;
        }
        stop = true;
        break;
      }
    }
    if (pick_s < 0 && rank_hint >= 0) {   // fewer units than workgroups: normal claim
      rank_hint = -1;
      continue;
    }
    rank_hint = -1;
    if (pick_s >= 0) {
      const int c = a.order[pick_s];
      if (!((st.acquired >> c) & 1ull)) {
        // first use of a landed peer chunk: make the copy's data visible
        if (a.arrived != nullptr && c != a.local) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
        st.acquired |= 1ull << c;
      }
      if (pick_red) {
        uint32_t v = 0;
        if (lane == 0) v = fetch_add_relaxed(a.ws32 + WS_RED_CLAIM + c, 1u);
        v = __builtin_amdgcn_readfirstlane(v);
        if (v >= (uint32_t)a.red_units[c]) continue;   // all taken: look again
        take_reduce_unit(a, c, v, r);
        return r;
      }
      uint32_t u = 0;
      if (lane == 0) u = fetch_add_relaxed(a.ws32 + WS_CLAIM + c * XCDS + pick_g, 1u);
      u = __builtin_amdgcn_readfirstlane(u) + static_units(a, c, pick_g);
      if (u < group_units(a, c, pick_g)) {
        const int S = a.split[c];
        const int tl = (int)u / S;
        r.c = c;
        r.sp = (int)u - tl * S;
        group_tile(a, pick_g, tl, r.tm, r.tn);
        r.first = (pick_g == 0 && u == 0);
        r.red = 0;
        return r;
      }
      continue;   // lost the race for the last unit: look again
    }
    if (has_work == 0 && red_left == 0 && red_blocked == 0) { r.c = -1; return r; }   // every unit claimed
    // Claim ahead: GEMM work is left only in chunks that have not landed.
    // Take a unit of the first such chunk in priority order now (own XCD's
    // group first) and wait for that chunk's flag alone, so the unit starts
    // as soon as the chunk lands, without a walk over every counter after
    // the landing.  The wait depends on the flag only (set from outside the
    // launch), never on another workgroup.
    if (has_work != 0 && a.arrived != nullptr) {
      const int sidx = __builtin_ctzll(has_work);   // first position with GEMM work (not landed)
      const int c = a.order[sidx];
      if (!((landed >> sidx) & 1ull)) {
        uint32_t u = 0;
        int g_got = -1;
        for (int t = 0; t < XCDS && g_got < 0; ++t) {
          const int g = (xg + t) % XCDS;
          if (group_units(a, c, g) == 0u) continue;
          if (lane == 0) u = fetch_add_relaxed(a.ws32 + WS_CLAIM + c * XCDS + g, 1u);
          u = __builtin_amdgcn_readfirstlane(u);
          if (u < group_units(a, c, g)) g_got = g;
        }
        if (g_got >= 0) {
          bool ok = true;
          if (lane == 0) {
            const uint64_t t0 = now_ticks();
            while (!epoch_reached(load_relaxed(a.arrived + c), a.epoch)) {
              if (load_relaxed(a.ws32 + WS_ABORT) || now_ticks() - t0 > a.timeout_ticks) { ok = false; break; }
              __builtin_amdgcn_s_sleep(1);
            }
          }
          if (!__builtin_amdgcn_readfirstlane((int)ok)) {
            if (lane == 0) {
              if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(a.ws32 + WS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            r.c = -2;
            return r;
          }
          if (!((st.acquired >> c) & 1ull)) {   // first use of the landed chunk
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
            st.acquired |= 1ull << c;
          }
          const int S = a.split[c];
          const int tl = (int)u / S;
          r.c = c;
          r.sp = (int)u - tl * S;
          group_tile(a, g_got, tl, r.tm, r.tn);
          r.first = (g_got == 0 && u == 0);
          r.red = 0;
          return r;
        }
        continue;   // that chunk's units are all taken: look again
      }
    }
    // Work is left only in chunks that have not landed (or, in STRICT mode,
    // behind one), and only a landing can change that: other workgroups'
    // claims only remove work.  So until the landed set changes, only the
    // flags and the abort word are read, one line each, rather than every
    // claim counter: hundreds of waiting workgroups would otherwise queue on
    // the counters' memory channel and delay the claims after a landing.
    if (wait_from == 0) wait_from = now_ticks();
    for (;;) {
      if (load_relaxed(a.ws32 + WS_ABORT)) { r.c = -2; return r; }
      if (now_ticks() - wait_from > a.timeout_ticks) {
        if (lane == 0) {
          if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
          __hip_atomic_store(a.ws32 + WS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        r.c = -2;
        return r;
      }
      __builtin_amdgcn_s_sleep(4);
      bool now_ok = false, now_blk = false;
      if (lane < R) {
        const int c = a.order[lane];
        now_ok = a.arrived == nullptr || c == a.local || epoch_reached(load_relaxed(a.arrived + c), a.epoch);
        if (((red_blocked >> lane) & 1) && a.inc_arrived != nullptr)
          now_blk = !epoch_reached(load_relaxed(a.inc_arrived + c), a.epoch);
      }
      if (__ballot(now_ok) != landed || __ballot(now_blk) != red_blocked) break;
    }
  }
}

// Output piece writer: 4 consecutive fp32 values at (row, col) of a row-major
// destination with leading dimension ld, stored as fp32 or bf16 (round to
// nearest even), masked to ncols columns.  With wt (fp32 only) the store is
// written through to memory.
__device__ __forceinline__ void put4(char *base, int64_t ld, int64_t row, int64_t col, int64_t ncols,
                                     bool bf16, bool vec_ok, bool wt, const f32x4 &val) {
  if (wt) {
    float *q = reinterpret_cast<float *>(base) + row * ld + col;
    if (vec_ok && col + 4 <= ncols) {
      store_wt16(q, val);
    } else {
      for (int e = 0; e < 4 && col + e < ncols; ++e)
        __hip_atomic_store(q + e, val[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    return;
  }
  if (vec_ok && col + 4 <= ncols) {
    if (bf16) {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(val[0]) | ((uint32_t)f32_to_bf16_rne(val[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(val[2]) | ((uint32_t)f32_to_bf16_rne(val[3]) << 16);
      *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(base) + row * ld + col) = u32x2{lo, hi};
    } else {
      *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(base) + row * ld + col) = val;
    }
  } else {
    for (int e = 0; e < 4 && col + e < ncols; ++e) {
      if (bf16)
        reinterpret_cast<uint16_t *>(base)[row * ld + col + e] = f32_to_bf16_rne(val[e]);
      else
        reinterpret_cast<float *>(base)[row * ld + col + e] = val[e];
    }
  }
}

// Reduce unit: row slice `slice` of split tile `tile` of chunk c, whose S
// partials are all written (through to memory); reads them with
// system-coherent loads, sums them in split order 0..S-1 and stores the
// output rows.
template <int BM, int BN, int NTT>
__device__ __forceinline__ void reduce_unit(const GemmArgs &a, int c, int tile, int slice, int64_t row0,
                                         int64_t rowlim, int64_t col0) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // computed per unit, not kept live across the loop
  const int64_t N = a.n;
  const int S = a.split[c];
  const size_t pbase = (size_t)a.part_base[c] + (size_t)tile * S;
  const float *P = a.partials + pbase * (size_t)(BM * BN);
  constexpr int ROWS = BM / RED_SLICES;
  constexpr int PPR = BN / 4;                       // pieces per row
  static_assert(BM % RED_SLICES == 0, "slices");
  const int r0 = slice * ROWS;
  const bool vec_ok = (N & 3) == 0;
  // one resource over the tile's S partials (at most 8 x 256 x 256 fp32)
  const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(P, S * BM * BN * 4);
  for (int pc = tid; pc < ROWS * PPR; pc += NTT) {
    const int rr = r0 + pc / PPR, cc = pc - (pc / PPR) * PPR;
    const int off = (rr * BN + cc * 4) * 4;
    f32x4 t[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < S)
        t[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, off + q * (BM * BN * 4), 0, 1 | 2));
    f32x4 sum = t[0];
#pragma unroll
    for (int q = 1; q < 8; ++q)
      if (q < S) sum = sum + t[q];
    const int64_t row = row0 + rr;
    if (row < rowlim && col0 + cc * 4 < N)
      put4(reinterpret_cast<char *>(a.y), N, row, col0 + cc * 4, N, a.y_bf16 != 0, vec_ok,
           a.done_flags != nullptr, sum);
  }
}

// Split unit sp of a split tile when split units reduce their own slices:
// sums row slices sp, sp + S, ... (of RED_SLICES) over the tile's S partials
// in split order 0..S-1, as reduce units would, and stores the output rows.
// With own_lds the unit's own partial rows come from its LDS staging (row
// stride SROW floats; the unit did not write them out), the other splits'
// rows from memory with system-coherent loads.  Each thread issues the loads
// of U pieces for every partial before it adds, so the slices cost a round
// trip per U pieces rather than one per slice.  One instance for every S (a
// switch over S instances displaced the k-loop's registers).
template <int BM, int BN, int NTT, int SROW>
__device__ __forceinline__ void reduce_own_slices(const GemmArgs &a, int c, int tile, int sp, int64_t row0,
                                                  int64_t rowlim, int64_t col0, const float *stg, bool own_lds) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // computed per unit, not kept live across the loop
  const int64_t N = a.n;
  const int S = a.split[c];
  const float *P = a.partials + ((size_t)a.part_base[c] + (size_t)tile * S) * (size_t)(BM * BN);
  constexpr int ROWS = BM / RED_SLICES;
  constexpr int PPR = BN / 4;                       // 16-byte pieces per row
  constexpr int PPS = ROWS * PPR;                   // pieces per slice
  constexpr int SMAX = 8;                           // largest split
  constexpr int U = 2;                              // pieces per thread per batch (3 or more put
                                                    // scratch traffic into the 128x224 k-loop)
  const int npc = ((RED_SLICES - sp + S - 1) / S) * PPS;
  const bool vec_ok = (N & 3) == 0;
  const bool wt = a.done_flags != nullptr;
  const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(P, S * BM * BN * 4);
  for (int base = tid; base < npc; base += U * NTT) {
    f32x4 t[U][SMAX];
    int rr[U], cc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pc = base + u * NTT;
      const int j = pc / PPS, w = pc - (pc / PPS) * PPS;
      rr[u] = (sp + j * S) * ROWS + w / PPR;
      cc[u] = w - (w / PPR) * PPR;
      const int off = (rr[u] * BN + cc[u] * 4) * 4;
#pragma unroll
      for (int q = 0; q < SMAX; ++q) {
        t[u][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (q < S && pc < npc && !(own_lds && q == sp))
          t[u][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, off + q * (BM * BN * 4), 0, 1 | 2));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pc = base + u * NTT;
      if (pc >= npc) continue;
      const f32x4 own = own_lds ? *reinterpret_cast<const f32x4 *>(stg + rr[u] * SROW + cc[u] * 4)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 sum = (own_lds && sp == 0) ? own : t[u][0];
#pragma unroll
      for (int q = 1; q < SMAX; ++q)
        if (q < S) sum = sum + ((own_lds && q == sp) ? own : t[u][q]);
      const int64_t row = row0 + rr[u];
      if (row < rowlim && col0 + cc[u] * 4 < N)
        put4(reinterpret_cast<char *>(a.y), N, row, col0 + cc[u] * 4, N, a.y_bf16 != 0, vec_ok, wt, sum);
    }
  }
}

// Shard unit (fo_gemm_rs_reduce, fo_gemm_rs_ring): row slice `slice` of a
// tile of chunk c, whose partial is in memory (written through by its unit).
// Sums the partial and the incoming partials in summation order (fp32, left
// to right) and stores the result:
//  - direct form (c = local): the incoming partials are inc[0 .. ninc-1]
//    (priority order without local: the order fo_chunk_reduce uses, so the
//    bits match the unfused pair); the sum goes to the shard (fp32, or bf16
//    rounded to nearest even);
//  - ring form: the one incoming partial is inc[c] (none if null), the
//    accumulated partial from the predecessor; the sum goes to the shard for
//    the local chunk and back over the partial rows (written through, to be
//    forwarded) for the others.
// Each wave keeps its running sums in registers and adds, whenever it finds
// some, the longest run of pending sources whose flags show the epoch: only
// the sources that land last are left to read after the last landing, and
// all of them are read together when they are already there.  The partial and
// the incoming partials are read with system-coherent loads: a copy engine or
// another XCD wrote them during the launch.  Returns false after a timeout
// (status set, the launch aborted).  No barrier: the waves of the workgroup
// run through it independently.
template <int BM, int BN, int NTT>
__device__ __forceinline__ bool shard_unit(const GemmArgs &a, int c, int slice, int64_t row0, int64_t rowlim,
                                           int64_t col0) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // computed per unit, not kept live across the loop
  const int lane = tid & 63;
  const int64_t N = a.n;
  const int bytes = (int)((int64_t)a.mc * N * 4);              // one chunk of fp32 rows (< 2 GiB)
  const int64_t lrow0 = row0 - (int64_t)c * a.mc;              // first row inside the chunk
  float *const prow = reinterpret_cast<float *>(a.y) + (int64_t)c * a.mc * N;
  const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(prow, bytes);
  const bool ring = a.ring != 0;
  const int ninc = ring ? (a.inc[c] != nullptr ? 1 : 0) : a.ninc;
  constexpr int ROWS = BM / RED_SLICES;
  constexpr int PPR = BN / 4;                       // 16-byte pieces per row
  constexpr int PER = (ROWS * PPR + NTT - 1) / NTT; // pieces per thread
  constexpr int KB = 8;                             // sources whose loads are issued together
  const int r0 = slice * ROWS;
  int off[PER];
  bool ok[PER];
  f32x4 v[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int pc = tid + q * NTT;
    const int rr = r0 + pc / PPR, cc = pc - (pc / PPR) * PPR;
    const int64_t col = col0 + cc * 4;
    ok[q] = pc < ROWS * PPR && row0 + rr < rowlim && col < N;
    off[q] = ok[q] ? (int)(((lrow0 + rr) * N + col) * 4) : 0;
    v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ok[q]) v[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, off[q], 0, 1 | 2 | 16));
  }
  const uint64_t t0 = now_ticks();
  int s = 0;
  while (s < ninc) {
    // sources s .. e-1 have landed (lane i looks at source i's flag)
    int e = ninc;
    if (a.inc_arrived) {
      bool landed = true;
      if (lane < ninc)
        landed = epoch_reached(load_relaxed(a.inc_arrived + (ring ? c : a.inc_chunk[lane])), a.epoch);
      const uint64_t pending = ~__ballot(landed) >> s;
      if (pending) e = s + __builtin_ctzll(pending);
      if (e == s) {
        bool out = false;
        if (lane == 0) out = (now_ticks() - t0 > a.timeout_ticks) || load_relaxed(a.ws32 + WS_ABORT) != 0u;
        if (__ballot(out)) {
          if (lane == 0) {
            if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(a.ws32 + WS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          return false;
        }
        __builtin_amdgcn_s_sleep(4);
        continue;
      }
    }
    // the loads of up to KB sources are issued together, then added in
    // summation order
    for (; s < e; s += KB) {
      f32x4 t[KB][PER];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
#pragma unroll
        for (int q = 0; q < PER; ++q) t[k][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s + k < e) {
          const __amdgpu_buffer_rsrc_t ri = uniform_rsrc(ring ? a.inc[c] : a.inc[s + k], bytes);
#pragma unroll
          for (int q = 0; q < PER; ++q)
            if (ok[q]) t[k][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, off[q], 0, 1 | 2 | 16));
        }
      }
#pragma unroll
      for (int k = 0; k < KB; ++k)
        if (s + k < e) {
#pragma unroll
          for (int q = 0; q < PER; ++q)
            if (ok[q]) v[q] += t[k][q];
        }
    }
    s = e;
  }
  // Every store is written through to memory: the unit is counted towards
  // done[c] once its stores are acknowledged, and a consumer of done[c] (a
  // copy engine, another stream) reads the rows without any cache
  // maintenance by this launch.
  const bool to_shard = !ring || c == a.local;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (!ok[q]) continue;
    const int64_t idx = off[q] / 4;
    if (!to_shard) {
      store_wt16(prow + idx, v[q]);
    } else if (a.shard_bf16) {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[q][0]) | ((uint32_t)f32_to_bf16_rne(v[q][1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[q][2]) | ((uint32_t)f32_to_bf16_rne(v[q][3]) << 16);
      store_wt8(reinterpret_cast<uint16_t *>(a.shard) + idx, u32x2{lo, hi});
    } else {
      store_wt16(reinterpret_cast<float *>(a.shard) + idx, v[q]);
    }
  }
  return true;
}

// The kernel's argument block behind a pointer the compiler cannot see
// through, taken once per unit: without it the compiler hoists every argument
// field the unit loop may read into registers for the whole kernel (and spills
// them), where the tiles need those registers for accumulators and fragments.
// The fields are reloaded with scalar loads from the argument segment.
__device__ __forceinline__ const GemmArgs &unit_args() {
  auto p = (const __attribute__((address_space(4))) GemmArgs *)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const GemmArgs *)p;
}

// Compute waves: a WGM x WGN grid of waves over the tile.  Copies:
//  - default: every 4 waves form a copy group that also issues the stage
//    copies (round v goes to copy group v % NCG);
//  - PC: four extra producer waves issue every copy and wait for it, so a
//    compute wave never stalls behind a full load queue; the two kinds of
//    wave share each SIMD;
//  - HP (8 compute waves): waves 0-3 issue every copy and also multiply,
//    waves 4-7 only multiply.  A wave that issues a burst of copies stalls
//    until the load queue takes them; the other wave on its SIMD then keeps
//    the matrix core busy, where in the default layout both would stall.
template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, bool PC, bool HP = false, bool RV = false>
__device__ __forceinline__ void gemm_body(const GemmArgs &a) {
  using C = Cfg<BM, BN, BK, STAGES, WGM, WGN>;
  constexpr int NCW = WGM * WGN;               // compute waves
  constexpr int NTT = 64 * NCW + (PC ? NT : 0);
  constexpr int NCG = (PC || HP) ? 1 : NTT / NT;   // copy groups of 4 waves
  static_assert(NTT % NT == 0, "whole copy groups");
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  __shared__ Unit s_unit;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool prod = !(PC || HP) || wave < 4;                             // issues stage copies
  const bool cons = !PC || wave >= 4;                                    // multiplies
  const int cwave = PC ? (wave >= 4 ? wave - 4 : 0) : wave;              // index among compute waves
  const int wm = cwave / WGN, wn = cwave % WGN;
  const int cg = __builtin_amdgcn_readfirstlane(wave >> 2);             // copy group
  const int cw = wave & 3;                                               // wave in its copy group
  const int64_t K = a.k, N = a.n;
  const int xg = (int)(blockIdx.x % XCDS);

  ClaimState st{0ull, 0};
  int rank_hint = (int)(blockIdx.x / XCDS);   // this workgroup's rank inside its XCD
  // The stage buffers are written only by the copy engine (asm below): hand
  // the buffer to an opaque asm so the compiler cannot assume it is never
  // written and fold the fragment reads away.
  asm volatile("" :: "v"(lds) : "memory");
  if (blockIdx.x == 0 && tid == 0 && a.stamps) store_u64_relaxed(a.stamps + 2 * a.R, now_ticks());

  for (;;) {
    const GemmArgs &a = unit_args();
    if (wave == 0) {
      const Unit u = claim_unit(a, st, xg, rank_hint);
      if (lane == 0) s_unit = u;
    }
    __syncthreads();
    Unit un = s_unit;
    un.c = __builtin_amdgcn_readfirstlane(un.c);
    un.tm = __builtin_amdgcn_readfirstlane(un.tm);
    un.tn = __builtin_amdgcn_readfirstlane(un.tn);
    un.sp = __builtin_amdgcn_readfirstlane(un.sp);
    un.red = __builtin_amdgcn_readfirstlane(un.red);
    const int c = un.c;
    if (c < 0) break;
    if (un.first && tid == 0 && a.stamps) store_u64_relaxed(a.stamps + c, now_ticks());

    const int S = a.split[c];
    const int sp = un.sp;
    const int tile = un.tm * a.tiles_n + un.tn;
    const int64_t row0 = (int64_t)c * a.mc + (int64_t)un.tm * BM;
    const int64_t rowlim = (int64_t)(c + 1) * a.mc;
    const int64_t col0 = (int64_t)un.tn * BN;
    const int64_t k0 = (int64_t)sp * a.kslice[c];
    const int64_t k1 = (k0 + a.kslice[c] < K) ? k0 + a.kslice[c] : K;
    const int KT = (int)((k1 - k0 + BK - 1) / BK);

    if (un.red) {
      if (a.fused)   // no split chunks: every reduce unit is a shard unit
        shard_unit<BM, BN, NTT>(a, c, un.sp, row0, rowlim, col0);
      else
        reduce_unit<BM, BN, NTT>(a, c, tile, un.sp, row0, rowlim, col0);
    } else {

    // Stage layout in LDS: BM rows of X then BN rows of W, ROWB bytes each,
    // 16-byte pieces XOR-swizzled.  Load round v of a stage fills LDS slots
    // [256 v, 256 v + 256) (wave w of copy group v % NCG, which issues round
    // v: 64 slots at m0 = base + 4096 v + 1024 w);
    // slot s holds row s / CH, piece s % CH, i.e. logical piece
    // (s % CH) ^ swz(row) of that row.  Thread t always fills slot t of a
    // round, so its row inside a round, its piece and hence its byte offset
    // in the operand are fixed; the round and the k position go into the
    // uniform offset.  Rows past the chunk end or past n read as zero (buffer
    // size), and so does k past the split's end (per-thread offset moved past
    // the buffer).
    const int nra = (int)((rowlim - row0 < BM) ? rowlim - row0 : BM);
    const int nrb = (int)((N - col0 < BN) ? N - col0 : BN);
    const __amdgpu_buffer_rsrc_t rsa = uniform_rsrc(a.x + row0 * K, (int)(nra * K * 2));
    const __amdgpu_buffer_rsrc_t rsb = uniform_rsrc(a.w + col0 * K, (int)(nrb * K * 2));
    const uint32_t lds0 = lds_addr(lds) + (uint32_t)(__builtin_amdgcn_readfirstlane(cw) * 1024);

    auto issue = [&](int stage) {
      const int kk = (int)(k0 + (int64_t)stage * BK);          // uniform
      // RV: the per-lane offset is recomputed from the thread index at each
      // issue.  In a layout whose k-loop needs nearly every register, the
      // offset kept live across the loop gets spilled, and its reload waits
      // for every copy in flight before the next stage's copies go out.
      int t = threadIdx.x;
      if constexpr (RV) asm volatile("" : "+v"(t));
      const int rtr = (t & (NT - 1)) / C::CH;
      const int rtch = ((t & (NT - 1)) % C::CH) ^ C::swz(rtr);
      const int vo = (kk + rtch * 8 < k1) ? (int)((rtr * K + rtch * 8) * 2) : 0x40000000;   // k past the end reads zero
      const uint32_t base = lds0 + (uint32_t)((stage % STAGES) * C::STAGE);
#pragma unroll
      for (int v = 0; v < C::V; ++v) {
        if (NCG > 1 && v % NCG != cg) continue;
        const bool isA = v < C::AV;
        const int rs = C::RSTEP * (isA ? v : v - C::AV);
        dma16(base + (uint32_t)(v * 4096), vo, isA ? rsa : rsb, (int)((rs * K + kk) * 2));
      }
    };

    // The first k-step starts the accumulators from an inline zero operand
    // instead of zero-filled registers: with zero-filled registers the
    // register allocator shares one zero and cannot keep each MFMA's result in
    // its accumulator registers, and copies accumulators every k-step.
    f32x4 acc[C::FM][C::FN];
    // One stage: read every fragment of k-step 0, then issue k-step 0's MFMAs
    // interleaved with the fragment reads of k-step 1, then k-step 1's MFMAs.
    // The schedule is pinned: left alone, the scheduler reuses one register
    // quad for all X fragments and waits for each read before its MFMAs.
    auto compute = [&](auto firstc, auto bufc) {
      constexpr bool first = decltype(firstc)::value;
      constexpr int buf = decltype(bufc)::value;
      const char *A = lds + buf * C::STAGE;
      const char *B = A + C::A_BYTES;
      if constexpr (PC && C::KS == 2) {
        // Both k-steps with few live fragments: k-step 0's MFMAs go column by
        // column; after column j its W fragment is dead and k-step 1's W
        // fragment j is read in its place, and k-step 1's X fragments are read
        // during the last column.  Peak: 2 FM + FN fragments.
        const int sw0 = (((lane >> 4) ^ C::swz(lane & 15)) << 4);
        const int sw1 = (((4 + (lane >> 4)) ^ C::swz(lane & 15)) << 4);
        auto rda = [&](int i, int swz) {
          return *reinterpret_cast<const bf16x8 *>(A + (wm * C::WTM + i * 16 + (lane & 15)) * C::ROWB + swz);
        };
        auto rdb = [&](int j, int swz) {
          return *reinterpret_cast<const bf16x8 *>(B + (wn * C::WTN + j * 16 + (lane & 15)) * C::ROWB + swz);
        };
        bf16x8 a0[C::FM], a1[C::FM], b0[C::FN], b1[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) a0[i] = rda(i, sw0);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) b0[j] = rdb(j, sw0);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
#pragma unroll
          for (int i = 0; i < C::FM; ++i) {
            if (first)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], b0[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
          }
          b1[j] = rdb(j, sw1);
          if (j == C::FN - 1) {
#pragma unroll
            for (int i = 0; i < C::FM; ++i) a1[i] = rda(i, sw1);
          }
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
        // pinned order (mask 0x100: LDS reads, 0x008: MFMA)
        __builtin_amdgcn_sched_group_barrier(0x100, C::FM + C::FN, 0);
        static_for<C::FN - 1>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, C::FM, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
        __builtin_amdgcn_sched_group_barrier(0x008, C::FM, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1 + C::FM, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, C::FM * C::FN, 0);
        return;
      } else {
      bf16x8 af[C::KS][C::FM], bfr[C::KS][C::FN];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int ch = ks * 4 + (lane >> 4);
        const int swz = ((ch ^ C::swz(lane & 15)) << 4);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
          af[ks][i] = *reinterpret_cast<const bf16x8 *>(A + (wm * C::WTM + i * 16 + (lane & 15)) * C::ROWB + swz);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          bfr[ks][j] = *reinterpret_cast<const bf16x8 *>(B + (wn * C::WTN + j * 16 + (lane & 15)) * C::ROWB + swz);
      }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            if (first && ks == 0)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][i], bfr[ks][j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
          }
      // pinned order (mask 0x100: LDS reads, 0x008: MFMA)
      constexpr int NF = C::FM + C::FN, NM = C::FM * C::FN;
      __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);
      if constexpr (C::KS == 2) {
        static_for<NF>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NM - NF, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      }
      }
    };

    // Wait until stage j has landed: the stages issued after it may stay in
    // flight (each stage is V copies per wave).
    auto wait_stage = [&](int j) {
      const int later = ((j + STAGES - 1 < KT) ? j + STAGES - 1 : KT) - (j + 1);
      if constexpr (NCG == 1) {
        wait_later<C::V, STAGES>(later);
      } else {
        static_assert(NCG == 2, "copy groups");
        if (cg == 0) wait_later<(C::V + 1) / 2, STAGES>(later);
        else wait_later<C::V / 2, STAGES>(later);
      }
    };

    // prologue: stages 0 .. STAGES-2 in flight.  The LDS buffers about to be
    // filled may still be read by the previous unit's last k-steps.
    __syncthreads();
    if (prod) {
#pragma unroll
      for (int p = 0; p < STAGES - 1; ++p)
        if (p < KT) issue(p);
    }

    // iteration j: wait for stage j; barrier (stage j visible to every wave,
    // and every wave is done with stage j-1, whose buffer is refilled next);
    // issue stage j+STAGES-1; multiply stage j (LDS buffer j % STAGES).
    // Iteration 0 is peeled; the rest are unrolled STAGES at a time so each
    // buffer offset is a constant.
    if (prod) wait_stage(0);
    __syncthreads();
    if (prod && STAGES - 1 < KT) issue(STAGES - 1);
    if (cons) compute(std::true_type{}, std::integral_constant<int, 0>{});
    for (int j0 = 1; j0 < KT; j0 += STAGES) {
      static_for<STAGES>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        const int j = j0 + p;
        if (j < KT) {
          if (prod) wait_stage(j);
          __syncthreads();
          if (prod && j + STAGES - 1 < KT) issue(j + STAGES - 1);
          if (cons) compute(std::false_type{}, std::integral_constant<int, (1 + p) % STAGES>{});
        }
      });
    }

    // Epilogue: stage the tile in LDS (the stage ring is idle now) so every
    // lane writes 16-byte row pieces; a tile too large for LDS goes in two
    // row halves (the waves of one half write their quadrants each pass).
    // Unsplit: the tile goes to the output.  Split: the fp32 partial goes to
    // its workspace slot (row-major BM x BN); the split that completes the
    // tile publishes it for the reduce units.
    {
      // Lane indices of the epilogue come from an opaque copy of the thread
      // index, so they are computed here, per unit, rather than hoisted to
      // the kernel's start and kept live (spilled) across the k-loop.
      int etid = threadIdx.x;
      asm volatile("" : "+v"(etid));
      const int elane = etid & 63, ewave = etid >> 6;
      const int ecw = PC ? (ewave >= 4 ? ewave - 4 : 0) : ewave;
      const bool econs = !PC || ewave >= 4;
      const int ewm = ecw / WGN, ewn = ecw % WGN;
      // padded fp32 row (spreads the staging writes over banks) when it fits
      constexpr int SROW = (BM / 2 * (BN + 4) * 4 <= C::LDS) ? BN + 4 : BN;
      constexpr int HALVES = (BM * SROW * 4 <= C::LDS) ? 1 : 2;
      static_assert(BM / HALVES * SROW * 4 <= C::LDS, "epilogue staging");
      static_assert(WGM % HALVES == 0, "a staging pass holds whole wave rows");
      constexpr int WPP = WGM / HALVES;                             // wave rows per pass
      constexpr int HROWS = BM / HALVES;
      constexpr int CPR = BN / 4;                                   // 16-byte pieces per row
      float *stg = reinterpret_cast<float *>(lds);
      const bool to_out = (S == 1);
      char *dbase = to_out ? reinterpret_cast<char *>(a.y)
                           : reinterpret_cast<char *>(a.partials + ((size_t)a.part_base[c] + (size_t)tile * S + sp) * (size_t)(BM * BN));
      const int64_t ld = to_out ? N : BN;
      const int64_t rbase = to_out ? row0 : 0, cbase = to_out ? col0 : 0;
      const int64_t rlim = to_out ? rowlim : BM, clim = to_out ? N : BN;
      const bool vec_ok = to_out ? (N & 3) == 0 : true;
      const bool bf = to_out && a.y_bf16;
      // split partials (read by reduce units on any XCD) and GEMM-RS output
      // (read by the consumer of the done flags) are written through
      const bool wt = !to_out || a.done_flags != nullptr || a.fused;
      // a split unit that sums its own slices keeps them in the LDS staging
      // (the whole tile is staged in one pass) instead of writing them out
      const bool own_lds = HALVES == 1 && !to_out && a.self_reduce;
#pragma unroll
      for (int h = 0; h < HALVES; ++h) {
        __syncthreads();
        if (econs && ewm / WPP == h) {
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int r = (ewm % WPP) * C::WTM + i * 16 + (elane >> 4) * 4 + v;
                stg[r * SROW + ewn * C::WTN + j * 16 + (elane & 15)] = acc[i][j][v];
              }
        }
        __syncthreads();
        for (int cidx = etid; cidx < HROWS * CPR; cidx += NTT) {
          const int r = cidx / CPR, cc = cidx - (cidx / CPR) * CPR;
          if constexpr (HALVES == 1)
            if (own_lds && ((r / (BM / RED_SLICES)) % S) == sp) continue;   // kept in LDS for this unit's sum
          const int64_t row = rbase + h * HROWS + r;
          const int64_t col = cbase + cc * 4;
          if (row >= rlim || col >= clim) continue;
          const f32x4 val = *reinterpret_cast<const f32x4 *>(stg + r * SROW + cc * 4);
          put4(dbase, ld, row, col, clim, bf, vec_ok, wt, val);
        }
      }
      if (a.fused && to_out && a.red_units[c] > 0) {
        // fused: publish the tile for its shard units once its
        // written-through stores are acknowledged
        wait_stores();
        __syncthreads();
        if (etid == 0) {
          const uint32_t idx = fetch_add_relaxed(a.ws32 + WS_RED_READY + c, 1u);
          store_relaxed_agent(a.ws32 + a.ready_off + a.ctr_base[c] + idx, (uint32_t)(tile + 1));
        }
      }
      if (!to_out) {
        // Publish the partial: once its write-through stores are acknowledged,
        // count the split.  The split that completes the tile lists it for
        // the reduce units, which read the tile counter before their reads
        // of the partials (see the reduce unit).
        wait_stores();
        __syncthreads();
        // Split units sum their own slices in every layout but the one that
        // needs every register in its k-loop (RV; the host enables it only
        // where tile_self_reduce says so): there the wait and the sums
        // displace the loop's registers.
        constexpr bool SR = !RV;
        bool ok = true;
        if (etid == 0) {
          uint32_t *ctr = a.ws32 + WS_TILE_CTR + a.ctr_base[c] + tile;
          const uint32_t old = fetch_add_relaxed(ctr, 1u);
          if (SR && a.self_reduce) {
            // wait for the tile's other splits (running or about to be
            // claimed by a free workgroup: the claimed units of a group form
            // a prefix of its split-fastest numbering, so at most S - 1
            // units per group and split chunk can wait here, and the host
            // enables this only with more workgroups than that)
            if (old != (uint32_t)(S - 1)) {
              const uint64_t t0 = now_ticks();
              while (load_relaxed_agent(ctr) < (uint32_t)S) {
                if (load_relaxed(a.ws32 + WS_ABORT) || now_ticks() - t0 > a.timeout_ticks) { ok = false; break; }
                __builtin_amdgcn_s_sleep(1);
              }
              if (!ok) {
                if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_SYSTEM);
                __hip_atomic_store(a.ws32 + WS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
            }
          } else if (old == (uint32_t)(S - 1)) {
            const uint32_t idx = fetch_add_relaxed(a.ws32 + WS_RED_READY + c, 1u);
            store_relaxed_agent(a.ws32 + a.ready_off + a.ctr_base[c] + idx, (uint32_t)(tile + 1));
          }
        }
        if constexpr (SR) {
          if (a.self_reduce) {
            // The other splits' partials are in memory (thread 0 read the
            // counter at S before the barrier; they are read with
            // system-coherent loads): sum this split's row slices in split
            // order 0..S-1, as a reduce unit would.
            if (__syncthreads_or(!ok)) break;
            reduce_own_slices<BM, BN, NTT, SROW>(a, c, tile, sp, row0, rowlim, col0, stg, own_lds);
          }
        }
      }
    }
    }   // GEMM unit

    // Completion accounting.  In GEMM-RS mode the chunk's done flag is
    // released after every output element of the chunk is in memory: each
    // unit waits for its write-through stores before it counts itself, and
    // the unit that completes the chunk acquires before releasing the flag.
    // Without done flags the counters only feed the stamps.
    if (a.done_flags) wait_stores();
    __syncthreads();
    if (tid == 0 && (a.done_flags || a.stamps)) {
      const uint32_t d = fetch_add_relaxed(a.ws32 + WS_CHUNK_DONE + c, 1u);
      if (d == (uint32_t)(a.units[c] + a.red_units[c] - 1)) {
        if (a.stamps) store_u64_relaxed(a.stamps + a.R + c, now_ticks());
        if (a.done_flags) {
          fence_acquire_agent();
          store_release(a.done_flags + c, a.epoch);
        }
      }
      if (a.stamps) {
        const uint32_t t = fetch_add_relaxed(a.ws32 + WS_TOTAL_DONE, 1u);
        if (t == (uint32_t)(a.total_units - 1)) store_u64_relaxed(a.stamps + 2 * a.R + 1, now_ticks());
      }
    }
  }

  // The last workgroup to leave returns every counter to zero for the next
  // call.  Every counter access is a device-scope atomic performed at the
  // device's coherence point, and each of a workgroup's counter atomics has
  // returned (its result steers the workgroup) before the workgroup counts
  // its exit; the last workgroup issues the resets after its own count has
  // returned.  No cache maintenance is needed, and none is paid: a release
  // fence here would write back the XCD's L2 once per workgroup.
  // The count goes in two levels (the workgroups of each XCD, then the XCDs)
  // so the exits do not queue on one counter; a launch that touched no
  // counter (static claims only, no flags, stamps or reduce units) skips it.
  if (tid == 0 && !a.no_counters) {
    const int xcd = (int)(blockIdx.x % XCDS);
    const int on_xcd = (a.grid - xcd + XCDS - 1) / XCDS;
    const int xcds = a.grid < XCDS ? a.grid : XCDS;
    bool last = fetch_add_relaxed(a.ws32 + WS_EXITED_X + xcd, 1u) == (uint32_t)(on_xcd - 1);
    if (last) last = fetch_add_relaxed(a.ws32 + WS_EXITED, 1u) == (uint32_t)(xcds - 1);
    if (last) {
      uint32_t *W = a.ws32;
      for (int g = 0; g < XCDS; ++g) store_relaxed_agent(W + WS_EXITED_X + g, 0u);
      for (int c = 0; c < a.R; ++c) {
        for (int g = 0; g < XCDS; ++g) store_relaxed_agent(W + WS_CLAIM + c * XCDS + g, 0u);
        store_relaxed_agent(W + WS_CHUNK_DONE + c, 0u);
        store_relaxed_agent(W + WS_RED_CLAIM + c, 0u);
        store_relaxed_agent(W + WS_RED_READY + c, 0u);
        if (a.ctr_base[c] >= 0) {
          const int ntiles = a.units[c] / a.split[c];
          for (int t = 0; t < ntiles; ++t) {
            store_relaxed_agent(W + WS_TILE_CTR + a.ctr_base[c] + t, 0u);
            store_relaxed_agent(W + a.ready_off + a.ctr_base[c] + t, 0u);
          }
        }
      }
      store_relaxed_agent(W + WS_TOTAL_DONE, 0u);
      store_relaxed_agent(W + WS_ABORT, 0u);
      store_relaxed_agent(W + WS_EXITED, 0u);
    }
  }
}

template <int BM, int BN, int BK, int STAGES>
__global__ void __launch_bounds__(NT, 1) gemm_kernel(GemmArgs a) {
  gemm_body<BM, BN, BK, STAGES, 2, 2, false>(a);
}

// Eight waves: two per SIMD.  The register cap leaves VGPRs free on every
// SIMD, so a one-wave kernel of a copy-engine emulator still fits beside the
// persistent grid.  On gfx950 the compiler counts this attribute in pairs of
// the unified VGPR/AGPR file: 120 caps each wave at 240, so two waves leave
// 32 of each lane's 512 registers free.
template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, bool PC, bool HP = false, bool RV = false>
__global__ void __launch_bounds__(2 * NT, 1) __attribute__((amdgpu_num_vgpr(120)))
gemm_kernel_w8(GemmArgs a) {
  gemm_body<BM, BN, BK, STAGES, WGM, WGN, PC, HP, RV>(a);
}

namespace {

struct Cand {
  int bm, bn, bk, stages;
  bool room;   // leaves registers free on every SIMD for a one-wave kernel
};

// Tile configurations compiled into the library (the launcher below maps
// each to its wave layout): 256 x 256 (k staged 64 at a time in two 64 KiB
// buffers, so every operand row piece is a whole 128-byte line) and 256 x 160,
// both as 8 waves in a 4 x 2 grid, half of them also issuing the copies (HP);
// 128 x 224 as 4 producer waves + 2 x 2 compute waves; 128 x 128 as 2 x 2
// waves.
constexpr Cand kCands[] = {{256, 256, 64, 2, true}, {256, 160, 64, 3, true},
                           {128, 224, 64, 3, true}, {128, 128, 64, 4, true}};

// Relative cost of a tile shape per output element: operand bytes staged per
// flop fall as 1/BM + 1/BN, so larger tiles run closer to the MFMA rate.
double tile_eff(int bm, int bn) { return 1.0 / (1.0 + 48.0 / bm + 48.0 / bn); }

bool parse_env_tile(Cand *out) {
  const char *e = getenv("FO_TILE");
  if (!e) return false;
  int bm = 0, bn = 0;
  if (sscanf(e, "%dx%d", &bm, &bn) != 2) return false;
  for (const Cand &c : kCands)
    if (c.bm == bm && c.bn == bn) { *out = c; return true; }
  return false;
}

}  // namespace

TileCfg choose_tile(int64_t mc, int64_t n, int64_t k, int R, int grid, bool leave_room) {
  (void)k;
  Cand pick{};
  if (parse_env_tile(&pick) && !(leave_room && !pick.room))
    return TileCfg{pick.bm, pick.bn, pick.stages};
  if (grid < 1) grid = 1;
  double best = 0;
  bool have = false;
  for (const Cand &c : kCands) {
    // with arrival flags a one-wave emulator kernel must still fit beside
    // the persistent grid
    if (leave_room && !c.room) continue;
    const int64_t tiles = ((mc + c.bm - 1) / c.bm) * ((n + c.bn - 1) / c.bn) * R;
    const int64_t waves = (tiles + grid - 1) / grid;
    const double cost = (double)waves * c.bm * c.bn / tile_eff(c.bm, c.bn);
    if (!have || cost < best) { best = cost; pick = c; have = true; }
  }
  return TileCfg{pick.bm, pick.bn, pick.stages};
}

int64_t max_padded_tile_area(int64_t mc, int64_t n) {
  int64_t best = 0;
  for (const Cand &c : kCands) {
    const int64_t a = (mc + c.bm - 1) / c.bm * c.bm * ((n + c.bn - 1) / c.bn * c.bn);
    if (a > best) best = a;
  }
  return best;
}

int64_t max_tiles_per_chunk(int64_t mc, int64_t n) {
  int64_t best = 0;
  for (const Cand &c : kCands) {
    const int64_t t = ((mc + c.bm - 1) / c.bm) * ((n + c.bn - 1) / c.bn);
    if (t > best) best = t;
  }
  return best;
}

size_t partial_slot_bytes(const TileCfg &t) { return (size_t)t.bm * t.bn * sizeof(float); }

// Split units may sum their own slices (GemmArgs::self_reduce) in every
// compiled layout but 256x256 (RV).
bool tile_self_reduce(const TileCfg &t) { return !(t.bm == 256 && t.bn == 256); }

hipError_t launch_gemm(const GemmArgs &a, const TileCfg &t, hipStream_t stream) {
  if (t.bm == 256 && t.bn == 256)
    hipLaunchKernelGGL((gemm_kernel_w8<256, 256, 64, 2, 4, 2, false, true, true>), dim3(a.grid), dim3(2 * NT), 0, stream, a);
  else if (t.bm == 256 && t.bn == 160)
    hipLaunchKernelGGL((gemm_kernel_w8<256, 160, 64, 3, 4, 2, false, true>), dim3(a.grid), dim3(2 * NT), 0, stream, a);
  else if (t.bm == 128 && t.bn == 224)
    hipLaunchKernelGGL((gemm_kernel_w8<128, 224, 64, 3, 2, 2, true>), dim3(a.grid), dim3(2 * NT), 0, stream, a);
  else if (t.bm == 128 && t.bn == 128)
    hipLaunchKernelGGL((gemm_kernel<128, 128, 64, 4>), dim3(a.grid), dim3(NT), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fo
