// Query-split attention for gfx950: O = softmax(scale * Q K^T [+ causal
// mask]) V per head, computed in blocks released as the sequence chunks land.
//
// Query-Split Attention (gist.science technical summary §2: attention
// decomposed into scores, softmax and weighted sum, so that more of it
// overlaps the communication).  Under sequence-parallel all-gather the rows
// of Q, K and V (the QKV projection's output for each token) arrive chunk by
// chunk.  The work is cut into blocks (head, 128-query tile, key chunk):
// every block needs its query chunk and its key chunk only, so blocks on
// chunks that have landed run while the rest is in flight, and the queries of
// the chunk that lands last are spread over all their key chunks instead of
// one long unit.  Each block leaves its row maxima, sums of exponentials and
// unnormalised weighted sums; the block that completes a query tile merges
// its tile's blocks in key-chunk order (so the bits never depend on landing
// times) and writes the output rows.
//
// Layout and schedule
//  - 8 waves per CU in either of two forms.  With every chunk present: two
//    workgroups of 4 waves per CU, each on its own block.  Under arrivals:
//    one workgroup of two groups of 4 waves per CU, sharing each block, group
//    g taking key tiles g, g + 2, ... with its own double-buffered LDS tiles,
//    maxima, sums and weighted sums; at the block's end group 1 hands its
//    state to group 0 through LDS, which merges the two.  The blocks of the
//    chunk that lands last then occupy every CU, each in about two thirds of
//    the time.  (Two independent workgroups overlap one's softmax with the
//    other's MFMAs; the two groups, in step at every barrier, do not, so the
//    all-present launch keeps the first form.)  Each wave owns 32 queries.  A key tile of 64 rows is copied into LDS by
//    the buffer-load DMA path (16-byte pieces XOR-swizzled by row); the
//    values of a key chunk are converted once to fp16 images, transposed, that
//    a block copies to LDS as they lie, so each lane reads its value fragments
//    as 16-byte pieces.
//  - Scores are computed transposed, S^T = K Q^T (bf16 MFMA, fp32
//    accumulate), so each lane holds one query's scores for 4 keys of every
//    16-key block: the softmax needs one cross-lane step per tile, and the
//    probabilities are already laid out as the second operand of
//    O^T = V^T P^T (fp16 MFMA, fp32 accumulate), whose rows for a query sit in
//    that query's lane.  Both operands of O^T take the keys of a 32-key
//    k-step in the same permuted order (4 from each of two 16-key blocks).
//  - Blocks are released in stages: stage s holds the blocks whose later
//    chunk is order[s], and opens once the chunks order[0..s] have landed.
//    Wave 0 claims the next block of the lowest open stage with one
//    fetch-add; a workgroup acquires (system scope) the first time it uses a
//    peer's chunk.
#include "fo_device.hpp"
#include "fo_internal.hpp"
#include "fo_tile.hpp"

namespace fo {

namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int QS_GT = 256;                      // threads of one group of 4 waves
constexpr int K_ROWB = QSA_D * 2;                  // 256 bytes per key row
constexpr int K_TILE = QSA_BKV * K_ROWB;           // 16 KiB
constexpr int VT_ROWB = QSA_BKV * 2;               // 64 fp16 keys per value row
constexpr int VT_TILE = QSA_D * VT_ROWB;           // 16 KiB
constexpr int QS_GLDS = 2 * K_TILE + 2 * VT_TILE;  // one group's tiles, both double-buffered
constexpr int SLOT_FLOATS = QSA_BQ * QSA_D + 2 * QSA_BQ;   // O [BQ][d], m [BQ], l [BQ]
constexpr int QS_EXITED = 576, QS_COMBINED = 577, QS_ABORT = 578, QS_EXITED_X = 584;
constexpr int QS_GROUPS = 8;   // claim groups per stage (one per XCD)
constexpr int QS_LINE = 32;    // words between the groups' counter lines: counter (g, s) at word 32 g + s
constexpr int QS_NEXT = 579;   // every chunk present: next unit past the workgroups' first ones
constexpr int QS_STATIC = 2;   // every chunk present: units each workgroup takes without a counter
constexpr float NEG_BIG = -1.0e30f;
constexpr float RESCALE_LOG2 = 8.0f;   // lazy rescale threshold (log2 units)

struct Blk {
  int h, qt, qc, kc;   // head, query tile over the whole sequence, query chunk, key chunk; qt < 0: stop
  int conv;            // 1: conversion unit (chunk qc, head h, key tiles G kc .. G kc + G - 1, one per group)
};

__device__ __forceinline__ void store_wt4(float *p, float v) {
  asm volatile("global_store_dword %0, %1, off sc0 sc1\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}

// Loads of data another workgroup wrote through during this launch, at
// system-coherent cache policy (sc0 sc1), without a fence.  The resource is
// the slot's (wave-uniform); the offset is per lane.
__device__ __forceinline__ f32x4 load_coherent16(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 1 | 2));
}

__device__ __forceinline__ float load_coherent4(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 1 | 2));
}

// Wave 0 (all lanes) claims the next unit.  Stage s is open once
// order[0..s] have all landed.  A stage's units are dealt to 8 groups
// (unit u to group u % 8), one claim counter each; the counters of a group
// share one 128-byte line (word 32 g + s), and the workgroups of the 8 XCDs
// (group = workgroup % 8) claim in their own group, so a claim reads and
// updates one line that an eighth of the workgroups use.  Among its group's
// open stages with units left the claim takes the largest next unit (a stage
// hands out its conversion units first, then its full pairs, then its
// diagonal blocks from the one with the most key tiles), the lowest stage on
// ties: with several stages open the long blocks start first and the short
// ones fill in at the end.  With its group exhausted it takes from the other
// groups the same way.  Waits (bounded) while units are left only in stages
// that are not open.
__device__ __forceinline__ int unit_key(const QsaArgs &a, int s, int u) {
  const int big = a.stage_big[s];
  const int key = u < a.conv_units ? 2 * a.tiles + 2 : u < big ? 2 * a.tiles + 1 : 2 * (a.tiles - (u - big) / a.H);
  return min(key, (1 << 22) - 1);   // ranks only; keeps the packed rank below 2^31
}

// Unit u of stage s as a block (or a conversion unit); the first use of a
// peer's chunk by this workgroup acquires (a copy engine wrote its rows
// during the launch).
__device__ __forceinline__ Blk decode_unit(const QsaArgs &a, int s, uint32_t u, uint32_t &acquired) {
  const int per_pair = a.H * a.tiles;
  const int big = a.stage_big[s];
  int pi, j;
  Blk b;
  b.conv = 0;
  if ((int)u < a.conv_units) {
    // convert the new chunk's value rows (head u / units per head, key
    // tiles G (u % units per head) .. + G - 1, one per group)
    const int nkt = a.chunk / (a.groups * QSA_BKV);
    b.conv = 1;
    b.qc = a.order[s];
    b.h = (int)u / nkt;
    b.kc = (int)u - b.h * nkt;
    b.qt = 0;
    if (a.arrived != nullptr && !((acquired >> b.qc) & 1u)) {
      if (b.qc != a.local) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
      acquired |= 1u << b.qc;
    }
    return b;
  }
  if ((int)u < big) {
    const int ub = (int)u - a.conv_units;
    pi = a.stage_pair0[s] + ub / per_pair;
    const int rem = ub - (ub / per_pair) * per_pair;
    b.h = rem / a.tiles;
    j = rem - b.h * a.tiles;
  } else {
    const int v = (int)u - big;
    pi = a.stage_pair0[s] + (big - a.conv_units) / per_pair;
    const int jj = v / a.H;
    b.h = v - jj * a.H;
    j = a.tiles - 1 - jj;
  }
  b.qc = a.pair_q[pi];
  b.kc = a.pair_k[pi];
  b.qt = b.qc * a.tiles + j;
  // first use of a peer's chunk by this workgroup: its rows were written
  // by a copy engine during the launch
  const uint32_t need = (1u << b.qc) | (1u << b.kc);
  if (a.arrived != nullptr && (need & ~acquired)) {
    uint32_t peers = need & ~acquired & ~(1u << a.local);
    if (peers) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
    acquired |= need;
  }
  return b;
}

__device__ Blk qsa_claim(const QsaArgs &a, uint32_t &acquired, uint64_t &wait_from, int &taken) {
  const int lane = threadIdx.x & 63;
  const int R = a.R;
  if (a.arrived == nullptr) {
    // Every chunk present: one sequence over all stages, largest first (the
    // conversion units, the full pairs, then the diagonal blocks from the
    // most key tiles down).  A workgroup's first two units are its index in
    // it and that plus the grid (no counter: the workgroups take them
    // together at the start and after the conversions); the later ones,
    // which finish at scattered times, come from one counter.
    uint32_t G;
    if (taken < QS_STATIC) {
      G = blockIdx.x + (uint32_t)(taken * a.grid);
    } else {
      uint32_t k = 0;
      if (lane == 0) k = fetch_add_relaxed(a.ws32 + QS_NEXT, 1u);
      G = (uint32_t)(QS_STATIC * a.grid) + __builtin_amdgcn_readfirstlane(k);
    }
    ++taken;
    const uint32_t nconv = (uint32_t)(R * a.conv_units);
    if (G < nconv) return decode_unit(a, (int)(G / a.conv_units), G % a.conv_units, acquired);
    G -= nconv;
    for (int s = 0; s < R; ++s) {
      const uint32_t nb = (uint32_t)(a.stage_big[s] - a.conv_units);
      if (G < nb) return decode_unit(a, s, (uint32_t)a.conv_units + G, acquired);
      G -= nb;
    }
    const uint32_t per_class = (uint32_t)(R * a.H);               // diagonal blocks of one size
    if (a.causal && G < per_class * (uint32_t)a.tiles) {
      const uint32_t jj = G / per_class, rem = G - jj * per_class;
      const int s = (int)(rem / a.H), h = (int)(rem - (rem / a.H) * a.H);
      return decode_unit(a, s, (uint32_t)a.stage_big[s] + jj * a.H + h, acquired);
    }
    return Blk{0, -1, 0, 0, 0};                                      // every unit taken
  }
  const int xg = (int)(blockIdx.x % QS_GROUPS);
  for (;;) {
    bool ok = false;
    if (lane < R) {
      const int c = a.order[lane];
      ok = a.arrived == nullptr || c == a.local || epoch_reached(load_relaxed(a.arrived + c), a.epoch);
    }
    const uint64_t landed = __ballot(ok);
    const int open = (~landed == 0ull) ? 64 : __builtin_ctzll(~landed);
    // rank of a candidate (stage st, group g, next unit u): key, then lower
    // stage, then lower group
    auto rank = [&](int st, int g, int u) { return (unit_key(a, st, u) << 8) | (127 - (st * QS_GROUPS + g)); };
    int best = -1;
    bool own_left = false;
    if (lane < R) {
      const uint32_t k = load_relaxed(a.ws32 + QS_LINE * xg + lane);
      const int u = (int)k * QS_GROUPS + xg;
      if (u < a.stage_units[lane]) {
        own_left = true;
        if (lane < open) best = rank(lane, xg, u);
      }
    }
    bool any_left = __ballot(own_left) != 0ull;
    if (__ballot(best >= 0) == 0ull) {
      // the own group has no open unit: look at every group
#pragma unroll
      for (int bt = 0; bt < (QSA_MAX_CHUNKS * QS_GROUPS + 63) / 64; ++bt) {
        const int idx = bt * 64 + lane;
        const int g = idx / QSA_MAX_CHUNKS, st = idx % QSA_MAX_CHUNKS;
        bool left = false;
        if (st < R && g < QS_GROUPS) {
          const uint32_t k = load_relaxed(a.ws32 + QS_LINE * g + st);
          const int u = (int)k * QS_GROUPS + g;
          if (u < a.stage_units[st]) {
            left = true;
            if (st < open) best = max(best, rank(st, g, u));
          }
        }
        any_left = any_left || __ballot(left) != 0ull;
      }
    }
    if (!any_left) return Blk{0, -1, 0, 0, 0};                     // every unit claimed
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off));
    best = __builtin_amdgcn_readfirstlane(best);
    if (best >= 0) {
      const int cand = 127 - (best & 127);
      const int s = cand / QS_GROUPS, g = cand % QS_GROUPS;
      uint32_t k = 0;
      if (lane == 0) k = fetch_add_relaxed(a.ws32 + QS_LINE * g + s, 1u);
      k = __builtin_amdgcn_readfirstlane(k);
      const uint32_t u = k * QS_GROUPS + (uint32_t)g;
      if (u >= (uint32_t)a.stage_units[s]) continue;                 // lost the race: look again
      return decode_unit(a, s, u, acquired);
    }
    if (wait_from == 0) wait_from = now_ticks();
    bool out = false;
    if (lane == 0) out = load_relaxed(a.ws32 + QS_ABORT) != 0u || now_ticks() - wait_from > a.timeout_ticks;
    if (__ballot(out)) {
      if (lane == 0) {
        if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(a.ws32 + QS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return Blk{0, -2, 0, 0, 0};
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Conversion unit (c, h, t): the value rows of key tile t of chunk c, head
// h, converted to fp16 and transposed into the image a block copies to LDS.
// The image of a key tile is [d][64 keys]; 16-byte piece P of row d holds
// the keys of k-group P = 4 k2 + g, in the order the score fragments hold
// them (32 k2 + 4 g + 0..3, then 32 k2 + 16 + 4 g + 0..3), and sits at
// piece P ^ (d % 8), so the fragment reads of 8 rows fall on 8 distinct bank
// groups.  Thread i of the group: k-group i % 8, head dims 4 (i / 8) .. + 4.
// Stores are written through.
__device__ __forceinline__ void qsa_convert(const QsaArgs &a, int c, int h, int t) {
  int tid = threadIdx.x & (QS_GT - 1);
  asm volatile("" : "+v"(tid));
  const int kg = tid & 7, dg = tid >> 3;
  const int k2 = kg >> 2, g = kg & 3;
  const int HD = a.H * QSA_D;
  const int64_t RS = 3 * (int64_t)HD;
  const int64_t row0 = (int64_t)c * a.chunk + (int64_t)t * QSA_BKV;
  const uint16_t *src = a.qkv + row0 * RS + 2 * HD + h * QSA_D + dg * 4;
  bf16x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = 32 * k2 + 4 * g + (i < 4 ? i : 12 + i);
    v[i] = *reinterpret_cast<const bf16x4 *>(src + (int64_t)key * RS);
  }
  uint16_t *dst = a.vt + ((int64_t)h * (a.S / QSA_BKV) + (int64_t)c * (a.chunk / QSA_BKV) + t) * (QSA_D * QSA_BKV);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f16x8 piece;
#pragma unroll
    for (int i = 0; i < 8; ++i) piece[i] = (_Float16)(float)v[i][e];
    const int row = dg * 4 + e;
    store_wt16(dst + row * QSA_BKV + ((kg ^ (row & 7)) << 3), __builtin_bit_cast(f32x4, piece));
  }
}

// One block: the 128 queries of tile b.qt against the keys of chunk b.kc, for
// head b.h; leaves the tile's row maxima m, sums l and unnormalised weighted
// sums O (fp32, written through) in the block's slot.  With G groups of 4
// waves, group grp (waves 4 grp .. 4 grp + 3) takes key tiles grp, grp + G,
// ...; wave w of every group owns queries 32 w .. 32 w + 31 of the tile.
template <int G>
__device__ __forceinline__ void qsa_block(const QsaArgs &a, char *lds_all, const Blk &b) {
  int tid_all = threadIdx.x;
  asm volatile("" : "+v"(tid_all));
  const int grp = G == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid_all >> 8);
  const int tid = tid_all & (QS_GT - 1);
  char *const lds = lds_all + grp * QS_GLDS;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // the same, in a scalar register
  const int g = lane >> 4, li = lane & 15;
  const int HD = a.H * QSA_D;
  const int64_t RS = 3 * (int64_t)HD;                     // qkv row stride (elements)
  const int q0 = b.qt * QSA_BQ;
  const int kbase = b.kc * a.chunk;
  const bool diag = a.causal && b.kc == b.qc;
  const int nkt_all = a.chunk / QSA_BKV;
  // with the causal mask, key tiles past the tile's last query are empty
  const int nkt = diag ? (q0 + QSA_BQ - 1 - kbase) / QSA_BKV + 1 : nkt_all;

  // Query fragments (second operand of S^T = K Q^T): lane (g, li) holds
  // query row q0 + 32 wave + 16 qb + li, head dims 32 ks + 8 g .. + 8.
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint16_t *qrow = a.qkv + (int64_t)(q0 + wave * 32 + qb * 16 + li) * RS + b.h * QSA_D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[qb][ks] = *reinterpret_cast<const bf16x8 *>(qrow + ks * 32);
  }
  // Opaque to the compiler once loaded: left alone it reloads them from
  // memory in every tile to free registers, and the waits for those reloads,
  // counted in order with the next tile's copies issued just before, made
  // every tile wait for its successor's copies before its first MFMA.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(qf[qb][ks]));

  // Copies into LDS by the buffer-load DMA path, both tiles double-buffered
  // (tile kt in buffer kt % 2).  Key tile: thread t fills 16-byte slot t of
  // each of 4 rounds (16 key rows per round); slot t holds row t / 16 of the
  // round, physical piece t % 16, i.e. logical piece (t % 16) ^ (row % 16).
  // Value tile: the converted image, 16 KiB copied as it lies, at
  // system-coherent cache policy (other workgroups wrote it in this launch).
  const __amdgpu_buffer_rsrc_t rsk =
      uniform_rsrc(a.qkv + (int64_t)kbase * RS + HD + b.h * QSA_D, (int)((int64_t)a.chunk * RS * 2));
  const __amdgpu_buffer_rsrc_t rsv =
      uniform_rsrc(a.vt + ((int64_t)b.h * (a.S / QSA_BKV) + (int64_t)b.kc * nkt_all) * (QSA_D * QSA_BKV),
                   nkt_all * VT_TILE);
  const uint32_t lds_w = lds_addr(lds) + (uint32_t)(wave_s * 1024);
  auto issue = [&](int kt) {   // the group's tile kt (its iteration kt / G) into buffer (kt / G) % 2
    const uint32_t kb = lds_w + (uint32_t)(((kt / G) & 1) * K_TILE);
    const uint32_t vb = lds_w + (uint32_t)(2 * K_TILE + ((kt / G) & 1) * VT_TILE);
    // the per-lane offsets are rebuilt at each issue from the lane id
    // (mbcnt, no memory) and the wave index (a scalar): kept live across the
    // tile loop they were spilled, and the reload's wait, counted in order
    // with the copies in flight, held back the issue
    int t = (wave_s << 6) | (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(t));
    const int k_voff = (int)(((t >> 4) * RS + (((t & 15) ^ (t >> 4)) * 8)) * 2);
#pragma unroll
    for (int rd = 0; rd < 4; ++rd)
      dma16(kb + (uint32_t)(rd * 4096), k_voff, rsk, (int)((int64_t)(kt * QSA_BKV + rd * 16) * RS * 2));
#pragma unroll
    for (int rd = 0; rd < 4; ++rd)
      dma16_coherent(vb + (uint32_t)(rd * 4096), t * 16, rsv, kt * VT_TILE + rd * 4096);
  };

  f32x4 o[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {NEG_BIG, NEG_BIG}, l[2] = {0.f, 0.f};

  // Pipeline: tile kt + 1's copies go out at the start of tile kt, into the
  // buffers tile kt - 1 used; one barrier per tile (tile kt + 1 landed, and
  // every wave is done with tile kt's buffers).
  __syncthreads();                 // the previous block's last tile is done with the buffers
  if (grp < nkt) issue(grp);
  wait_vm<0>();
  __syncthreads();
  // The probabilities of the group's current tile (fp16, laid out as the
  // second operand of O^T = V^T P^T), from score() to pv().
  f16x8 pf[2][2];
  // Scores of tile kt, S^T = K Q^T, and its online softmax; MASK: the tile
  // crosses the diagonal (uniform).
  auto score = [&](int kt, auto maskc) {
    const bool MASK = static_cast<bool>(maskc);
    const char *K = lds + ((kt / G) & 1) * K_TILE;
    // S^T = K Q^T: st[kb][qb], keys 16 kb + 4 g + v, query 16 qb + li
    // (the four key fragments of a group of 16 keys are read together, then
    // its eight MFMAs issued)
    f32x4 st[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8 *>(K + (kb * 16 + li) * K_ROWB + (((ks * 4 + g) ^ li) << 4));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          st[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[qb][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : st[kb][qb], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    // Online softmax per query, in log2 units.  The maximum is taken over
    // the raw scores (the scale is positive); the reference m a row's
    // probabilities are taken against moves up only when the tile's maximum
    // exceeds it by more than 2^8, so the weighted sums are rescaled only
    // then (any reference gives the same softmax; probabilities stay below
    // 2^8, well inside fp16).  The first tile always sets it.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = NEG_BIG;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float sv = st[kb][qb][v];
          if (MASK) {
            const int qrow = q0 + wave * 32 + qb * 16 + li;
            if (kbase + kt * QSA_BKV + kb * 16 + 4 * g + v > qrow) sv = -__builtin_inff();
            st[kb][qb][v] = sv;
          }
          mx = fmaxf(mx, sv);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxs = mx * a.scale_log2;
      const bool grow = mxs > m[qb] + RESCALE_LOG2;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mnew = grow ? mxs : m[qb];
        const float f = __builtin_amdgcn_exp2f(m[qb] - mnew);
        m[qb] = mnew;
        l[qb] *= f;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][qb] *= f;
      }
      const float nm = -m[qb];
      float sum = 0.f;
      _Float16 p16[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][qb][v], a.scale_log2, nm));
          sum += p;
          p16[kb][v] = (_Float16)p;
        }
      l[qb] += sum;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        pf[qb][k2] = f16x8{p16[2 * k2][0], p16[2 * k2][1], p16[2 * k2][2], p16[2 * k2][3],
                           p16[2 * k2 + 1][0], p16[2 * k2 + 1][1], p16[2 * k2 + 1][2], p16[2 * k2 + 1][3]};
    }
  };
  // O^T += V^T P^T for tile kt: value rows 16 db + li, the keys of k-group
  // 4 k2 + g
    // (the same key order as pf)
  auto pv = [&](int kt) {
    const char *VT = lds + 2 * K_TILE + ((kt / G) & 1) * VT_TILE;

    {
      // two groups of 16 value dims at a time: the next group's four
      // fragment reads are in flight while this group's eight MFMAs run
      // (read one at a time, each read's latency stood in front of two MFMAs)
      auto rdv = [&](int db, int k2) {
        return *reinterpret_cast<const f16x8 *>(VT + (db * 16 + li) * VT_ROWB + (((k2 * 4 + g) ^ (li & 7)) << 4));
      };
      f16x8 vf[2][2][2];
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) vf[0][dd][k2] = rdv(dd, k2);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      static_for<4>([&](auto gc) {
        constexpr int gi = decltype(gc)::value;
        constexpr int cur = gi & 1;
        if constexpr (gi + 1 < 4) {
#pragma unroll
          for (int dd = 0; dd < 2; ++dd)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) vf[cur ^ 1][dd][k2] = rdv(2 * (gi + 1) + dd, k2);
        }
#pragma unroll
        for (int dd = 0; dd < 2; ++dd)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              o[2 * gi + dd][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[cur][dd][k2], pf[qb][k2], o[2 * gi + dd][qb], 0, 0, 0);
        if constexpr (gi + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      });
    }
  };
  // Key tiles that end before the block's first query need no mask; on the
  // diagonal the last two tiles cross it.  Every tile ends in one barrier of
  // the whole workgroup (the group's next tile landed, every wave done with
  // the tile whose buffer is refilled next).
  const int nfree = diag ? (q0 - kbase) / QSA_BKV : nkt;
  if constexpr (G == 1) {
    // the mask known at compile time: unmasked tiles carry none of it
    auto step = [&](int kt, auto maskc) {
      if (kt + 1 < nkt) issue(kt + 1);
      score(kt, maskc);
      pv(kt);
      if (kt + 1 < nkt) {
        wait_vm<0>();
        __syncthreads();
      }
    };
    for (int kt = 0; kt < nfree; ++kt) step(kt, std::false_type{});
    if (diag) {
      step(nfree, std::true_type{});
      step(nfree + 1, std::true_type{});
    }
  } else {
    // the groups take the block's tiles in turn, one tile each per
    // iteration; a group with no tile left sits the last one out.  One tile
    // body with the mask as a run-time flag: two bodies made the compiler
    // move the accumulators between register sets at every tile.
    const int iters = (nkt + G - 1) / G;
    for (int it = 0; it < iters; ++it) {
      const int kt = G * it + grp;
      if (kt < nkt) {
        if (kt + G < nkt) issue(kt + G);
        score(kt, kt >= nfree);
        pv(kt);
      }
      if (it + 1 < iters) {
        wait_vm<0>();
        __syncthreads();
      }
    }
  }

  // Group 1 hands its maxima, partial sums and weighted sums to group 0,
  // lane by lane, through LDS (the tile buffers are free after the barrier);
  // group 0 merges them: M = max, each side scaled by 2^(its m - M).  Group
  // 0's first tile holds keys at or before every query of the tile, so its
  // maxima are finite.
  if constexpr (G == 2) {
  __syncthreads();
  float *xo = reinterpret_cast<float *>(lds_all + QS_GLDS) + (wave * 64 + lane) * 64;   // 64 floats per lane
  float *xm = reinterpret_cast<float *>(lds_all) + (wave * 64 + lane) * 4;              // m[2], l[2] per lane
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) *reinterpret_cast<f32x4 *>(xo + (db * 2 + qb) * 4) = o[db][qb];
    *reinterpret_cast<f32x4 *>(xm) = f32x4{m[0], m[1], l[0], l[1]};
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const f32x4 ml = *reinterpret_cast<const f32x4 *>(xm);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m1 = ml[qb], l1 = ml[2 + qb];
      const float mm = fmaxf(m[qb], m1);
      const float a0 = __builtin_amdgcn_exp2f(m[qb] - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
      l[qb] = l[qb] * a0 + l1 * a1;
      m[qb] = mm;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        o[db][qb] = o[db][qb] * a0 + *reinterpret_cast<const f32x4 *>(xo + (db * 2 + qb) * 4) * a1;
    }
  }
  }

  // the block's slot: O rows by query (value dims 16 db + 4 g + v in lane
  // (g, li) of query 16 qb + li), then m and l per query
  const int QT = a.S / QSA_BQ;
  float *slot = a.part + ((int64_t)(b.h * QT + b.qt) * a.R + b.kc) * SLOT_FLOATS;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = wave * 32 + qb * 16 + li;
#pragma unroll
    for (int db = 0; db < 8; ++db) store_wt16(slot + r * QSA_D + db * 16 + 4 * g, o[db][qb]);
    float lt = l[qb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (g == 0) {
      store_wt4(slot + QSA_BQ * QSA_D + r, m[qb]);
      store_wt4(slot + QSA_BQ * QSA_D + QSA_BQ + r, lt);
    }
  }
}

// Merge of a query tile's blocks (key chunks 0 .. nb-1, in that order): per
// query, M = max m, L = sum 2^(m - M) l, O = sum (2^(m - M) / L) O.  The
// maxima and sums go through LDS (the block's buffers are idle here), then
// each thread merges 16-byte pieces of output rows, the loads of two slots in
// flight together.
template <int NTH>
__device__ __forceinline__ void qsa_combine(const QsaArgs &a, char *lds, int h, int qt, int nb) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int QT = a.S / QSA_BQ;
  const float *slot0 = a.part + (int64_t)(h * QT + qt) * a.R * SLOT_FLOATS;
  float *s_m = reinterpret_cast<float *>(lds);                     // [nb][BQ]
  float *s_l = s_m + QSA_MAX_CHUNKS * QSA_BQ;                      // [nb][BQ]
  constexpr int PIECES = QSA_BQ * (QSA_D / 4);                     // 16-byte output pieces
  constexpr int PER = PIECES / NTH;
  constexpr int SB = NTH >= 512 ? 2 : 1;                           // slots whose loads are in flight together
                                                                   // (as many as the registers allow)
  auto slot_rs = [&](int j) { return uniform_rsrc(slot0 + (int64_t)j * SLOT_FLOATS, SLOT_FLOATS * 4); };
  // the first slots' rows go out before the maxima and sums (they do not
  // depend on the weights), so those round trips overlap
  f32x4 t[SB][PER];
#pragma unroll
  for (int jj = 0; jj < SB; ++jj)
    if (jj < nb) {
      const __amdgpu_buffer_rsrc_t rs = slot_rs(jj);
#pragma unroll
      for (int k = 0; k < PER; ++k) t[jj][k] = load_coherent16(rs, (tid + k * NTH) * 16);
    }
  __syncthreads();   // the block's last tile is done with LDS
  for (int idx = tid; idx < nb * QSA_BQ; idx += NTH) {
    const int j = idx / QSA_BQ, r = idx - (idx / QSA_BQ) * QSA_BQ;
    const __amdgpu_buffer_rsrc_t rs = slot_rs(j);
    s_m[idx] = load_coherent4(rs, (QSA_BQ * QSA_D + r) * 4);
    s_l[idx] = load_coherent4(rs, (QSA_BQ * QSA_D + QSA_BQ + r) * 4);
  }
  __syncthreads();
  if (tid < QSA_BQ) {
    float M = NEG_BIG;
    for (int j = 0; j < nb; ++j) M = fmaxf(M, s_m[j * QSA_BQ + tid]);
    float L = 0.f;
    for (int j = 0; j < nb; ++j) {
      const float w = __builtin_amdgcn_exp2f(s_m[j * QSA_BQ + tid] - M);
      s_m[j * QSA_BQ + tid] = w;
      L += w * s_l[j * QSA_BQ + tid];
    }
    for (int j = 0; j < nb; ++j) s_m[j * QSA_BQ + tid] /= L;     // the weights
  }
  __syncthreads();
  const int HD = a.H * QSA_D;
  f32x4 acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  // slots in order 0 .. nb-1 (fp32 adds in that order), SB loaded together
  for (int j0 = 0; j0 < nb; j0 += SB) {
    if (j0 > 0) {
#pragma unroll
      for (int jj = 0; jj < SB; ++jj)
        if (j0 + jj < nb) {
          const __amdgpu_buffer_rsrc_t rs = slot_rs(j0 + jj);
#pragma unroll
          for (int k = 0; k < PER; ++k) t[jj][k] = load_coherent16(rs, (tid + k * NTH) * 16);
        }
    }
#pragma unroll
    for (int jj = 0; jj < SB; ++jj)
      if (j0 + jj < nb) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const int r = (tid + k * NTH) / (QSA_D / 4);
          acc[k] += s_m[(j0 + jj) * QSA_BQ + r] * t[jj][k];
        }
      }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = tid + k * NTH;
    const int r = idx / (QSA_D / 4), c4 = idx - r * (QSA_D / 4);
    const int64_t off = (int64_t)(qt * QSA_BQ + r) * HD + h * QSA_D + 4 * c4;
    if (a.o_bf16) {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[k][0]) | ((uint32_t)f32_to_bf16_rne(acc[k][1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[k][2]) | ((uint32_t)f32_to_bf16_rne(acc[k][3]) << 16);
      *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.o) + off) = u32x2{lo, hi};
    } else {
      *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.o) + off) = acc[k];
    }
  }
}

// Two workgroups per CU under a register cap: on gfx950 the attribute counts
// pairs of the unified register file, so 120 caps each wave at 240 and the
// two waves of a SIMD leave 32 of each lane's 512 registers free, where the
// one-wave kernels of a copy-engine emulator still fit beside the grid.
// G groups of 4 waves per workgroup: G = 2, one workgroup per CU, when the
// chunks arrive during the launch (the last chunk's blocks then use every
// CU, each in half the time); G = 1, two workgroups per CU, when every chunk
// is present (independent workgroups overlap one's softmax with the other's
// MFMAs, where two groups of one workgroup, in step at each barrier, do not).
template <int G>
__global__ void __launch_bounds__(G * QS_GT, 2 / G) __attribute__((amdgpu_num_vgpr(120))) qsa_kernel(QsaArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[G * QS_GLDS];
  __shared__ Blk s_blk;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  asm volatile("" :: "v"(lds) : "memory");
  if (blockIdx.x == 0 && tid == 0 && a.stamps) store_u64_relaxed(a.stamps + 2 * a.R, now_ticks());
  uint32_t acquired = 0;
  int taken = 0;
  uint64_t wait_from = 0;
  for (;;) {
    if (wave == 0) {
      const Blk b = qsa_claim(a, acquired, wait_from, taken);
      if (lane == 0) s_blk = b;
    }
    __syncthreads();
    Blk b = s_blk;
    b.h = __builtin_amdgcn_readfirstlane(b.h);
    b.qt = __builtin_amdgcn_readfirstlane(b.qt);
    b.qc = __builtin_amdgcn_readfirstlane(b.qc);
    b.kc = __builtin_amdgcn_readfirstlane(b.kc);
    b.conv = __builtin_amdgcn_readfirstlane(b.conv);
    if (b.qt < 0) break;
    if (b.conv) {
      // group g converts key tile G kc + g; the unit counts once every
      // group's stores are acknowledged
      qsa_convert(a, b.qc, b.h, G * b.kc + (G == 1 ? 0 : (tid >> 8)));
      wait_stores();
      __syncthreads();
      if (tid == 0) fetch_add_relaxed(a.ws32 + a.conv_off + b.qc * a.H + b.h, 1u);
      continue;
    }
    // the key chunk's values for this head must all be converted (bounded wait)
    if (tid == 0) {
      const uint32_t *cc = a.ws32 + a.conv_off + b.kc * a.H + b.h;
      const uint64_t t0 = now_ticks();
      while (load_relaxed(cc) < (uint32_t)(a.chunk / (G * QSA_BKV))) {
        if (load_relaxed(a.ws32 + QS_ABORT) != 0u) break;
        if (now_ticks() - t0 > a.timeout_ticks) {
          if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          __hip_atomic_store(a.ws32 + QS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    qsa_block<G>(a, lds, b);
    // count the block once its stores are acknowledged; the block that
    // completes the tile merges it
    wait_stores();
    __syncthreads();
    const int nb = a.causal ? b.qc + 1 : a.R;
    if (tid == 0) {
      uint32_t *ctr = a.ws32 + QSA_DONE + b.h * (a.S / QSA_BQ) + b.qt;
      const uint32_t old = fetch_add_relaxed(ctr, 1u);
      s_last = old == (uint32_t)(nb - 1);
      if (s_last) store_relaxed_agent(ctr, 0u);   // the tile's last user: back to zero
    }
    __syncthreads();
    if (s_last) {
      qsa_combine<G * QS_GT>(a, lds, b.h, b.qt, nb);
      if (a.stamps) {
        __syncthreads();
        if (tid == 0) {
          const uint32_t t = fetch_add_relaxed(a.ws32 + QS_COMBINED, 1u);
          if (t == (uint32_t)(a.H * (a.S / QSA_BQ) - 1)) store_u64_relaxed(a.stamps + 2 * a.R + 1, now_ticks());
        }
      }
    }
  }
  // the last workgroup to leave returns the counters to zero (after an abort
  // the tiles' block counters too: their tiles were left unfinished)
  // (counted per XCD, then per XCD group, so the exits do not queue on one
  // counter)
  if (tid == 0) {
    const int xcd = (int)(blockIdx.x % XCDS);
    const int on_xcd = (a.grid - xcd + XCDS - 1) / XCDS;
    const int xcds = a.grid < XCDS ? a.grid : XCDS;
    bool last = fetch_add_relaxed(a.ws32 + QS_EXITED_X + xcd, 1u) == (uint32_t)(on_xcd - 1);
    if (last) last = fetch_add_relaxed(a.ws32 + QS_EXITED, 1u) == (uint32_t)(xcds - 1);
    if (last) {
      for (int g = 0; g < XCDS; ++g) store_relaxed_agent(a.ws32 + QS_EXITED_X + g, 0u);
      if (load_relaxed_agent(a.ws32 + QS_ABORT) != 0u)
        for (int t = 0; t < a.H * (a.S / QSA_BQ); ++t) store_relaxed_agent(a.ws32 + QSA_DONE + t, 0u);
      for (int g = 0; g < QS_GROUPS; ++g)
        for (int t = 0; t < a.R; ++t) store_relaxed_agent(a.ws32 + QS_LINE * g + t, 0u);
      for (int t = 0; t < a.R * a.H; ++t) store_relaxed_agent(a.ws32 + a.conv_off + t, 0u);
      store_relaxed_agent(a.ws32 + QS_COMBINED, 0u);
      store_relaxed_agent(a.ws32 + QS_NEXT, 0u);
      store_relaxed_agent(a.ws32 + QS_ABORT, 0u);
      store_relaxed_agent(a.ws32 + QS_EXITED, 0u);
    }
  }
}

}  // namespace

hipError_t launch_qsa(const QsaArgs &a, hipStream_t stream) {
  if (a.groups == 2)
    hipLaunchKernelGGL(qsa_kernel<2>, dim3(a.grid), dim3(2 * QS_GT), 0, stream, a);
  else
    hipLaunchKernelGGL(qsa_kernel<1>, dim3(a.grid), dim3(QS_GT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fo
