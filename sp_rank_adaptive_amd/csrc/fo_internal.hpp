// Internal launch interface between the C ABI (fo_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "flashoverlap.h"

namespace fo {

// Workspace layout (32-bit words from the start of the workspace).  Every
// counter is returned to zero by the last workgroup to leave the kernel, so
// the counters are zero again after each completed call.
constexpr int XCDS = 8;                      // work-queue groups (one per XCD)
constexpr int WS_CLAIM = 0;                  // [FO_MAX_CHUNKS][XCDS] unit claim counters
constexpr int WS_CHUNK_DONE = 512;           // [FO_MAX_CHUNKS] finished units per chunk
constexpr int WS_TOTAL_DONE = 576;           // finished units, all chunks
constexpr int WS_EXITED = 577;               // workgroups that have left the loop
constexpr int WS_ABORT = 578;                // set when a wait timed out
constexpr int WS_EXITED_X = 584;             // [XCDS] workgroups of each XCD that have left the loop
constexpr int WS_RED_CLAIM = 640;            // [FO_MAX_CHUNKS] reduce units claimed
constexpr int WS_RED_READY = 704;            // [FO_MAX_CHUNKS] split tiles published
constexpr int WS_TILE_CTR = 1024;            // split-K arrival counters, one per tile,
                                             // then the ready lists (same size)
constexpr size_t WS_HEADER_BYTES = 4096;     // bytes before the tile counters
constexpr int RED_SLICES = 8;                // reduce units (row slices) per split tile

// Output tile of one workgroup and the depth of its LDS stage ring.
struct TileCfg {
  int bm, bn, stages;
};

// Arrays the first claim and the unit set-up read start on their own
// 64-byte lines, so the first entries of each come in with one line.
struct GemmArgs {
  const uint16_t *x;          // bf16 [m][k]
  const uint16_t *w;          // bf16 [n][k]
  void *y;                    // [m][n] fp32 or bf16
  int32_t y_bf16;
  int32_t rs_mode;            // 1: GEMM-RS (done flags), 0: AG-GEMM
  int64_t m, n, k;
  int32_t R, mc;              // chunks, rows per chunk
  int32_t tiles_m, tiles_n;   // tiles per chunk
  int32_t gm, gn;             // each chunk's tile grid is cut into gm x gn rectangles
  int32_t gtiles[XCDS];       // tiles per rectangle (work-queue group)
  int32_t local;
  int32_t strict;
  int32_t total_units;
  int32_t grid;
  int32_t static_rr;          // every unit assigned statically: 1 round-robin per XCD, 2 one per workgroup
  int32_t no_counters;        // static claims, no reduce units, no flags or stamps: no counter is touched
  int32_t all_unsplit;        // 1: no chunk is split
  int32_t one_unit;           // flags: a workgroup whose first claim succeeds leaves after it
  int32_t self_reduce;        // split chunks have no reduce units: each split unit, once its tile's
                              // splits are all written, sums row slices sp, sp + S, ... of the tile
  // Fused reduce of the local chunk (fo_gemm_rs_reduce): the local chunk's
  // reduce units sum its partial and the incoming partials into the shard.
  int32_t fused;                      // 1: red_units[c] > 0 are shard units
  int32_t ring;                       // 1: ring form: chunk c's shard units add inc[c] (indexed by
                                      //    chunk, flag inc_arrived[c]) and write in place, the local
                                      //    chunk's to the shard; claimed only once inc[c] landed
  int32_t fused_static;               // 1: shard units assigned statically (b, b + grid, ...)
  int32_t nshard;                     // chunks with shard units
  int32_t shard_seq[FO_MAX_CHUNKS];   // those chunks in priority order
  int32_t shard_bf16;
  int32_t ninc;                       // incoming partials, in summation order
  void *shard;                        // [mc][n]
  const uint32_t *inc_arrived;        // device [R] flags of the incoming partials, or null
  const float *inc[FO_MAX_CHUNKS];    // incoming partials [mc][n] fp32
  int32_t inc_chunk[FO_MAX_CHUNKS];   // chunk id of inc[i] (its flag)
  alignas(64) int32_t gunits[XCDS];       // units per work-queue group over all chunks
  const uint32_t *arrived;    // device [R] or null
  uint32_t *done_flags;       // device [R] or null
  uint32_t epoch;
  uint64_t timeout_ticks;
  int32_t *status;
  uint64_t *stamps;
  uint32_t *ws32;             // counters
  float *partials;            // split-K partial tiles
  alignas(64) int32_t order[FO_MAX_CHUNKS];
  alignas(64) int32_t split[FO_MAX_CHUNKS];
  alignas(64) int32_t units[FO_MAX_CHUNKS];     // tiles * split
  int32_t ctr_base[FO_MAX_CHUNKS];  // split chunk: first tile counter / ready slot; -1 if unsplit
  int32_t part_base[FO_MAX_CHUNKS]; // split chunk: first partial tile (tile*S + split)
  alignas(64) int32_t kslice[FO_MAX_CHUNKS];    // k extent of one split (multiple of 64)
  int32_t red_units[FO_MAX_CHUNKS]; // split chunk: tiles * RED_SLICES reduce units, else 0
  int32_t ready_off;                // word offset of the ready lists (after the tile counters)
};

struct ReduceArgs {
  const float *src[FO_MAX_CHUNKS];  // in summation sequence: seq[0] = local
  int32_t chunk_of[FO_MAX_CHUNKS];  // chunk id of seq[i] (for the flags)
  void *dst;
  float *acc;                       // fp32 running sum between passes
  int32_t dst_bf16;
  int32_t R;
  int64_t n4;                       // number of float4 vectors
  int64_t per_wg4;                  // float4 vectors owned by one workgroup
  const uint32_t *arrived;
  uint32_t epoch;
  uint64_t timeout_ticks;
  int32_t *status;
  uint64_t *stamps;
};

// All-to-all GEMM (fo_a2a_gemm): y = sum over pieces of piece[q] times the
// column block q of W, each piece's k-range taken in `order` once it landed.
struct A2aArgs {
  const uint16_t *piece[FO_MAX_CHUNKS];   // bf16 [m][kp] each, indexed by piece id
  const uint16_t *w;                      // bf16 [n][k], k = P * kp
  void *y;                                // [m][n] fp32 or bf16
  int32_t y_bf16;
  int64_t m, n, k;
  int32_t kp;                             // k extent of one piece
  int32_t P, local;
  int32_t order[FO_MAX_CHUNKS];           // accumulation order of the pieces
  int32_t tiles_m, tiles_n, gm, gn;       // tile grid, cut into gm x gn rectangles
  int32_t gtiles[XCDS];                   // tiles per rectangle (one per XCD)
  int32_t grid;
  const uint32_t *arrived;                // device [P] or null
  uint32_t epoch;
  uint64_t timeout_ticks;
  int32_t *status;
  uint64_t *stamps;                       // [2P+2]: [2P] start, [2P+1] last tile written
  uint32_t *ws32;                         // counters (the workspace header)
};

constexpr int A2A_BM = 128, A2A_BN = 256;   // output tile of the all-to-all GEMM
hipError_t launch_a2a(const A2aArgs &a, hipStream_t stream);

// Query-split attention (fo_qsa_attention).  A block is (head, 128-query
// tile, key chunk); blocks are released in stages (stage s opens once the
// chunks order[0..s] have landed).
constexpr int QSA_MAX_CHUNKS = 16;
constexpr int QSA_BQ = 128, QSA_BKV = 64, QSA_D = 128;
constexpr int QSA_DONE = 1024;                  // word offset of the per-(head, tile) block counters
struct QsaArgs {
  const uint16_t *qkv;                          // bf16 [S][3*H*d]
  void *o;                                      // [S][H*d] fp32 or bf16
  int32_t o_bf16;
  int32_t S, H, R, causal;
  int32_t chunk;                                // rows per chunk
  int32_t tiles;                                // query tiles per chunk
  int32_t local;
  int32_t order[QSA_MAX_CHUNKS];
  int32_t stage_units[QSA_MAX_CHUNKS];          // blocks released by stage s
  int32_t stage_pair0[QSA_MAX_CHUNKS];          // first pair of stage s in pair_q / pair_k
  int32_t groups;                               // groups of 4 waves per workgroup (1 or 2)
  int32_t conv_units;                           // conversion units opening each stage (H * key tiles / groups)
  int32_t stage_big[QSA_MAX_CHUNKS];            // conversion units plus the blocks of stage s that hold
                                                // every key tile of their pair; the rest, with the
                                                // causal mask, are the stage's diagonal pair, by
                                                // query tile from the last
  int32_t conv_off;                             // word offset of the [R][H] conversion counters
  uint16_t *vt;                                 // fp16 value images [H][S / 64][d][64]
  int8_t pair_q[QSA_MAX_CHUNKS * QSA_MAX_CHUNKS];  // (query chunk, key chunk) pairs by stage
  int8_t pair_k[QSA_MAX_CHUNKS * QSA_MAX_CHUNKS];
  float scale_log2;                             // log2(e) / sqrt(d)
  int32_t grid;
  const uint32_t *arrived;
  uint32_t epoch;
  uint64_t timeout_ticks;
  int32_t *status;
  uint64_t *stamps;                             // [2R+2]: [2R] start, [2R+1] last output written
  uint32_t *ws32;                               // counters, then the partial slots
  float *part;                                  // per (head, query tile, key chunk): O [BQ][d], m [BQ], l [BQ]
};
hipError_t launch_qsa(const QsaArgs &a, hipStream_t stream);

// Tile configuration chosen for a problem (host).
TileCfg choose_tile(int64_t mc, int64_t n, int64_t k, int R, int grid, bool leave_room);
size_t partial_slot_bytes(const TileCfg &t);
// Bounds over every compiled tile configuration, for workspace sizing: the
// largest padded chunk area (rows and columns rounded up to whole tiles) and
// the most tiles per chunk.
int64_t max_padded_tile_area(int64_t mc, int64_t n);
int64_t max_tiles_per_chunk(int64_t mc, int64_t n);

hipError_t launch_gemm(const GemmArgs &a, const TileCfg &t, hipStream_t stream);
// Whether the layout of t lets split units sum their own slices (self_reduce).
bool tile_self_reduce(const TileCfg &t);
hipError_t launch_reduce(const ReduceArgs &a, int grid, hipStream_t stream);

// Emulator kernels.
hipError_t launch_emu_start(uint64_t *t0_slot, uint64_t wait_ticks, const uint64_t *gate,
                            uint64_t gate_ticks, hipStream_t s);
hipError_t launch_emu_flag(const uint64_t *t0_slot, uint64_t release_ticks,
                           uint64_t next_issue_ticks, uint32_t *flag, uint32_t epoch,
                           uint64_t *stamp_slot, hipStream_t s);

hipError_t launch_emu_wait_flag(const uint32_t *flag, uint32_t epoch, uint64_t timeout_ticks, int32_t *status,
                                uint64_t *start_slot, hipStream_t s);
hipError_t launch_emu_hold(const uint64_t *start_slot, uint64_t link_ticks, uint64_t *done_slot, hipStream_t s);

int device_num_cus();
uint64_t device_wall_hz();

}  // namespace fo
