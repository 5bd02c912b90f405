/*
 * flashoverlap.h - C ABI of the one-GPU FlashOverlap hot path for gfx950.
 *
 * FlashOverlap (arXiv 2604.24013) replaces the all-gather and reduce-scatter
 * collectives of tensor/data parallel training with decomposed peer-to-peer
 * pieces and schedules partitioned computation on those pieces so that no
 * compute waits for the last piece (abstract; gist.science technical summary
 * §2 "Methodology", Flash-AG and Flash-RS; euno.news "Methodology" steps 1-3).
 * This library is one rank's share of that work on one MI355X:
 *
 *   fo_ag_gemm       Y = AllGather(X) * W, computed chunk by chunk as peer
 *                    row-chunks of X land (Flash-AG).
 *   fo_gemm_rs       the partial outputs P_c = X[rows of c] * W for every
 *                    chunk c, peer-destined chunks first and the chunk that
 *                    stays local last (Flash-RS, rank-adaptive partial output
 *                    scheduling).
 *   fo_chunk_reduce  dst = sum of R partial chunks, each peer chunk added once
 *                    it has landed (the reduction inside reduce-scatter; DP
 *                    needs reduce-scatter, technical summary §1).
 *   fo_emulate_arrivals  enqueues the arrivals of emulated peers: SDMA copies
 *                    from a staging region of the same HBM, each released at
 *                    a programmable time and then flagged (the receive side of
 *                    the decomposed collective).
 *
 * Conventions shared by every call
 *  - Pointers named "device" are HIP device pointers on the current device;
 *    "host" pointers are read during the call only.  The caller owns every
 *    buffer, flag array, workspace and stream; the library keeps no pointer
 *    after the enqueued work completes and allocates no device memory.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream);
 *    calls return without synchronising.  Buffers must stay alive until the
 *    stream work completes.
 *  - Argument errors are reported synchronously and enqueue nothing.  Errors
 *    found on the device (a flag wait that exceeds its bound) are written to
 *    the optional device status word and the kernel exits cleanly.
 *  - Matrices are row-major.  bf16 operands are IEEE binary32's upper halves.
 *    W is the K x N weight stored as [n][k] (K contiguous, nn.Linear layout).
 *  - Chunk c of an m-row operand is rows [c*m/R, (c+1)*m/R); m % R == 0.
 *  - Epoch flags: chunk c counts as landed once (int32)(flag[c] - epoch) >= 0.
 *    The caller passes a new, larger epoch on every call and never resets
 *    flags.  Calls that share a workspace or flag array must not overlap.
 */
#ifndef FLASHOVERLAP_H
#define FLASHOVERLAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fo_status;
enum {
  FO_OK = 0,
  FO_ERR_NULL = 1,       /* a required pointer is NULL                        */
  FO_ERR_SHAPE = 2,      /* non-positive size, m % R != 0, R out of range,
                            k > 2^21 (GEMM calls)                             */
  FO_ERR_ALIGN = 3,      /* pointer not 16-byte aligned, k % 8 != 0, or n % 4
                            != 0 where fp32 rows are moved as 16-byte pieces */
  FO_ERR_DTYPE = 4,      /* unknown dtype, or a dtype the call cannot store   */
  FO_ERR_ORDER = 5,      /* order is not a permutation of 0..R-1              */
  FO_ERR_SCHEDULE = 6,   /* local out of range, epoch == 0, bad mode/split    */
  FO_ERR_WORKSPACE = 7,  /* workspace NULL or smaller than fo_workspace_bytes */
  FO_ERR_HIP = 8,        /* a HIP runtime call failed (see fo_last_hip_error) */
  FO_ERR_TIMEOUT = 9,    /* device-side: a flag wait exceeded timeout_ns      */
  FO_ERR_ALIAS = 10      /* buffers overlap in a way the call does not allow  */
};

typedef int32_t fo_dtype;
enum { FO_F32 = 0, FO_BF16 = 1 };

/* Chunk claim policy (euno.news "Methodology" step 3: no sub-task waits for
 * the last piece; technical summary §2: chunks that depend on incoming data
 * first, the slice that stays local last). */
enum {
  FO_SCHED_READY_FIRST = 0, /* claim work from the first chunk in `order` that
                               has landed and has work left                    */
  FO_SCHED_STRICT = 1       /* take chunks exactly in `order`, waiting for each */
};

/* Largest supported number of chunks (emulated ranks). */
#define FO_MAX_CHUNKS 64

/* The chunk-order / arrival-schedule argument taken by every call. */
typedef struct fo_schedule {
  int32_t         nchunks;     /* R, 1 <= R <= FO_MAX_CHUNKS                    */
  int32_t         local;       /* this rank's chunk, 0 <= local < R             */
  const int32_t  *order;       /* host [R]: permutation of 0..R-1, the compute
                                  priority.  NULL = default: peers in ring
                                  arrival order local-1, local-2, ..., local+1,
                                  then local last                               */
  const uint32_t *arrived;     /* device [R] epoch flags; NULL = every chunk is
                                  present.  arrived[local] is never read.  Used
                                  by fo_ag_gemm and fo_chunk_reduce only.       */
  uint32_t        epoch;       /* > 0; new and larger on every call             */
  uint32_t        mode;        /* FO_SCHED_READY_FIRST or FO_SCHED_STRICT       */
  uint64_t        timeout_ns;  /* bound on one flag wait; 0 = 10 s              */
  int32_t        *status;      /* device [1], optional: receives FO_ERR_TIMEOUT */
  uint64_t       *stamps;      /* device, optional wall-clock timeline (ticks of
                                  the device wall clock, rate from fo_device_info):
                                  GEMM calls: [2R+2] = per-chunk first claim,
                                  per-chunk completion, kernel start, last
                                  output written.  fo_chunk_reduce: [2] = first
                                  workgroup start, completion (the caller zeroes
                                  [1] before the call; it receives a maximum).  */
  const int32_t  *split;       /* host [R], optional split-K factor per chunk
                                  (1..8).  NULL = auto: 1 everywhere when
                                  arrived == NULL, otherwise the last peer in
                                  `order` (the chunk expected to land last) is
                                  split so its tiles fill the GPU, keeping at
                                  least 1024 of k per split.                   */
  int32_t         max_workgroups; /* 0 = auto.  GEMM calls cap it at one
                                     workgroup per CU (the persistent grid
                                     must be resident at once; larger values
                                     act as the cap).  fo_chunk_reduce: auto
                                     is one workgroup per CU with `arrived`
                                     (all resident while they wait) and 8
                                     per CU without; it may exceed the value
                                     so no workgroup owns more than 1 GiB.
                                     fo_qsa_attention: auto is 8 waves per
                                     CU; with `arrived` it runs at least 8
                                     workgroups (one per claim group).
                                     fo_a2a_gemm runs at least one workgroup
                                     on every XCD whose tile rectangle is not
                                     empty (up to 8).                          */
  int32_t         reserved;
} fo_schedule;

/* Workspace bytes that fo_ag_gemm / fo_gemm_rs need for an m x n x k problem
 * in R chunks with the automatic split policy (or any split vector whose split
 * chunks fit; the call checks).  The workspace starts with work counters and
 * ends with split-K partial tiles.  It must be zero-filled once before its
 * first use; every call leaves the counters zero again when it completes
 * (also after FO_ERR_TIMEOUT); the partial tiles need no initialisation. */
size_t fo_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t nchunks);

/* Chunked AG-GEMM (technical summary §2, Flash-AG; row/column-parallel
 * projections for MLP and QKV).
 *   x  device bf16 [m][k]: all R row-chunks.  Peer chunks are written by
 *      the caller (or fo_emulate_arrivals) and flagged in s->arrived.
 *   w  device bf16 [n][k] (the K x N weight, K contiguous).
 *   y  device [m][n], y_dtype FO_F32 or FO_BF16 (round to nearest even);
 *      y = x * W for every row, whatever the order or arrival times.
 *   ws device workspace of ws_bytes >= fo_workspace_bytes(m, n, k, R).
 * Each output tile is computed from bf16 MFMA products with fp32 accumulation
 * in a fixed k order, so a given shape, split vector and input give the same
 * bits on every run.  Sizes: 1 <= k <= 2^21 with k % 8 == 0; m/R and n at
 * most 2^30.  Errors: NULL, SHAPE, ALIGN, DTYPE, ORDER, SCHEDULE, WORKSPACE,
 * ALIAS (y overlapping x or w), HIP. */
fo_status fo_ag_gemm(const void *x, const void *w, void *y, fo_dtype y_dtype,
                     int64_t m, int64_t n, int64_t k,
                     const fo_schedule *s, void *ws, size_t ws_bytes,
                     void *stream);

/* fo_ag_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation, kernels and bits as fo_ag_gemm with its workspace taken
 * from a library-held device array instead of a caller buffer:
 *   - the array is FO_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the
 *     library's load until the process ends; a problem whose
 *     fo_workspace_bytes exceeds it is refused with FO_ERR_WORKSPACE;
 *   - every call on a GPU shares that GPU's array: its counters are cleared
 *     by a kernel at the start of each call (on `stream`), so calls that
 *     overlap on one GPU race and must be ordered by the caller;
 *   - nothing is allocated or freed, by this call or anything it calls.
 * Arguments, errors and results as fo_ag_gemm (without ws, ws_bytes). */
#define FO_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fo_status fo_ag_gemm_noalloc(const void *x, const void *w, void *y, fo_dtype y_dtype,
                             int64_t m, int64_t n, int64_t k,
                             const fo_schedule *s, void *stream);

/* Chunked GEMM-RS (technical summary §2, Flash-RS).
 *   x        device bf16 [m][k]; w device bf16 [n][k].
 *   partial  device fp32 [m][n]: partial[rows of c] = x[rows of c] * W.
 *   done     device [R] epoch flags, optional: done[c] = epoch is stored with
 *            release semantics once chunk c is complete, so a copy engine or
 *            a peer may send it on.  Every row of chunk c (and, in the fused
 *            calls below, of the shard) is written through to memory before
 *            its flag, so a consumer polling done[c] on another stream or
 *            engine reads final data.
 * Default order: peers in send order local-1, ..., local+1, then the local
 * chunk last.  s->arrived must be NULL (the input rows are local).
 * Errors as fo_ag_gemm. */
fo_status fo_gemm_rs(const void *x, const void *w, float *partial, uint32_t *done,
                     int64_t m, int64_t n, int64_t k,
                     const fo_schedule *s, void *ws, size_t ws_bytes,
                     void *stream);

/* Chunked GEMM-RS with the reduce of the local chunk fused in (technical
 * summary §2, Flash-RS: the partial that stays local is produced last, and
 * the final receive is absorbed by that last step).  Computes exactly what
 * fo_gemm_rs computes (partial and done flags, same bits) and, in the same
 * launch,
 *   shard = partial[rows of local] + incoming[order'[0]] + incoming[order'[1]]
 *           + ...
 * in fp32 left to right, where order' is the priority order without local:
 * the order and bits of fo_chunk_reduce(shard, srcs with srcs[local] =
 * partial rows of local, srcs[q] = incoming[q]).  Each tile of the local
 * chunk is split into row slices that any workgroup sums once the tile is
 * written and every incoming partial has landed.
 *   shard     device [m/R][n], shard_dtype FO_F32 or FO_BF16 (nearest even).
 *   incoming  host [R] array of device fp32 [m/R][n] pointers; incoming[local]
 *             is ignored.  With s->arrived, incoming[q] is read only after
 *             arrived[q] shows the epoch (system-coherent loads: a copy
 *             engine may write it during the call); the GEMM itself is not
 *             gated.  Shard units are taken after every GEMM unit; a
 *             workgroup holding one adds each run of landed partials as it
 *             lands, so only the partials that land last are read after the
 *             last landing.
 * n % 4 == 0 and (m/R) * n * 4 < 2^31 are required; split factors other
 * than 1 are rejected.  Errors as fo_gemm_rs, plus DTYPE, ALIAS (shard
 * overlapping partial, x or w; an incoming partial overlapping the shard or
 * partial). */
fo_status fo_gemm_rs_reduce(const void *x, const void *w, float *partial, uint32_t *done,
                            void *shard, fo_dtype shard_dtype, const float *const *incoming,
                            int64_t m, int64_t n, int64_t k, const fo_schedule *s,
                            void *ws, size_t ws_bytes, void *stream);

/* Ring form of the fused GEMM-RS (technical summary §2, Flash-RS: at each
 * step a rank adds its partial of the chunk passing through it to the
 * accumulated partial received from its predecessor and forwards the sum; the
 * chunk that stays local is the last step).  Computes fo_gemm_rs's partials
 * and, in the same launch, for every chunk c with incoming[c] != NULL:
 *   c != local: partial[rows of c] = partial[rows of c] + incoming[c]
 *               (fp32, in place, written through: the message to forward);
 *   c == local: shard = partial[rows of local] + incoming[local]
 *               (incoming[local] NULL: shard = partial rows of local).
 * done[c] = epoch is released once chunk c's rows (or the shard) are final.
 * With s->arrived, chunk c's sum starts only after arrived[c] shows the epoch
 * (system-coherent loads of incoming[c]); no workgroup waits on a landing
 * while GEMM work is left.  In a ring of R ranks the predecessor's message for chunk c
 * holds the partials of ranks c+1 .. local-1; the chunk with no incoming
 * partial (local-1, whose accumulation this rank starts) is sent as computed.
 *   shard, shard_dtype: as fo_gemm_rs_reduce.
 *   incoming  host [R] array of device fp32 [m/R][n] pointers, any NULL.
 * Requirements and errors as fo_gemm_rs_reduce. */
fo_status fo_gemm_rs_ring(const void *x, const void *w, float *partial, uint32_t *done,
                          void *shard, fo_dtype shard_dtype, const float *const *incoming,
                          int64_t m, int64_t n, int64_t k, const fo_schedule *s,
                          void *ws, size_t ws_bytes, void *stream);

/* Flash All-to-All GEMM (technical summary §2: Flash All-to-All, the
 * extension of the decomposed primitives to Ulysses parallelism; §1: Ulysses
 * parallelism needs all-to-all).  The all-to-all after head-parallel
 * attention hands this rank, from every rank q, its sequence rows of q's
 * heads: piece q, a column block of the output projection's input.  Computes
 *   y = [piece 0 | piece 1 | ... | piece P-1] * W
 *     = sum over q of piece[q] * (columns [q*k/P, (q+1)*k/P) of W)
 * with each piece's share multiplied once its flag shows it landed.
 *   pieces  host [P] array of device bf16 [m][k/P] pointers (each piece
 *           contiguous, as its message lands); P = s->nchunks.
 *   w       device bf16 [n][k] (the K x N weight, K contiguous).
 *   y       device [m][n], y_dtype FO_F32 or FO_BF16 (nearest even).
 *   s       order: the order in which every output tile adds the pieces
 *           (it fixes the bits); NULL = the local piece, then local-1,
 *           local-2, ... (the order a pairwise-exchange all-to-all delivers
 *           them).  arrived[q] gates piece q (never read for local; NULL =
 *           every piece present); a piece is read only after its flag shows
 *           the epoch, with one system-scope acquire per workgroup.  mode is
 *           not used; split must be NULL or all 1.  stamps, optional, [2P+2]:
 *           [2P] kernel start, [2P+1] last output tile written.
 *   ws      device workspace of at least 4096 bytes, zero-filled once (a
 *           fo_ag_gemm workspace serves; calls sharing it must not overlap).
 * Each output element is summed in fp32 from bf16 MFMA products, piece by
 * piece in `order` and k ascending inside a piece: a given order gives the
 * same bits whatever the landing times.  Sizes: k % P == 0, (k/P) % 8 == 0,
 * k <= 2^21, m and n at most 2^30.  Errors: NULL, SHAPE, ALIGN, DTYPE, ORDER,
 * SCHEDULE, WORKSPACE, ALIAS (y overlapping w or a piece), HIP;
 * FO_ERR_TIMEOUT in *status when a flag wait exceeds its bound. */
fo_status fo_a2a_gemm(const void *const *pieces, const void *w, void *y, fo_dtype y_dtype,
                      int64_t m, int64_t n, int64_t k, const fo_schedule *s,
                      void *ws, size_t ws_bytes, void *stream);

/* Query-Split Attention (technical summary §2: attention decomposed into
 * scores, softmax and weighted sum so that more computation overlaps the
 * communication).  For every head h:
 *   O_h = softmax(Q_h K_h^T / sqrt(d) [+ causal mask]) V_h
 * where the rows of Q, K and V (the QKV projection's output, one row per
 * token) arrive in R sequence chunks (chunk c = rows [c*S/R, (c+1)*S/R)).
 * The work is cut into blocks (head, 128 queries, key chunk), each released
 * once the chunks order[0..s] it needs have landed (s = the later of its two
 * chunks' positions in `order`), so blocks on landed chunks run while the
 * rest is in flight; each query tile's blocks are merged in key-chunk order.
 * Each stage first converts its new chunk's values to fp16 once (into the
 * workspace, transposed), which the stage's blocks then copy as they lie.
 *   qkv     device bf16 [S][3*H*d]: per row the queries of heads 0..H-1 (d
 *           each), then their keys, then their values.
 *   o       device [S][H*d], o_dtype FO_F32 or FO_BF16 (nearest even).
 *   head_dim must be 128; (S/R) % 128 == 0; 1 <= R <= 16.
 *   causal  1: token i attends to tokens 0..i; 0: to every token.
 *   s       order: stage order of the chunks (NULL = local, local-1,
 *           local-2, ...: the order a ring delivers them); arrived[c] gates
 *           chunk c (NULL = all present); split NULL or all 1; mode unused.
 *           stamps, optional, [2R+2]: [2R] start, [2R+1] last output row
 *           written.
 *   ws      device workspace of fo_qsa_workspace_bytes(S, H, d, R) bytes
 *           (counters, per-block partial results, and the fp16 values:
 *           H*S*d*2 bytes), zero-filled once (every call leaves its counters
 *           zero).
 * Scores are bf16 MFMA products accumulated in fp32; the softmax runs in
 * fp32 (base-2 exponentials); the weighted sum multiplies fp16
 * probabilities by the values converted to fp16 (values must lie within
 * fp16's range) with fp32 accumulation.  The bits depend on the inputs and R
 * only, never on the order or the landing times.  Errors: NULL, SHAPE,
 * ALIGN, DTYPE, ORDER, SCHEDULE, WORKSPACE, ALIAS (o or ws overlapping qkv,
 * ws overlapping o), HIP; FO_ERR_TIMEOUT in *status when a flag wait
 * exceeds its bound. */
size_t fo_qsa_workspace_bytes(int64_t seq, int32_t heads, int32_t head_dim, int32_t nchunks);
fo_status fo_qsa_attention(const void *qkv, void *o, fo_dtype o_dtype, int64_t seq, int32_t heads,
                           int32_t head_dim, int32_t causal, const fo_schedule *s,
                           void *ws, size_t ws_bytes, void *stream);

/* Chunk reduce-add (technical summary §1 DP reduce-scatter, §2 Flash-RS).
 *   srcs  host [R] array of device fp32 pointers, n elements each.
 *   dst   device, n elements of dst_dtype (FO_F32 or FO_BF16).
 * dst = srcs[local] + srcs[order'[0]] + srcs[order'[1]] + ... in fp32, added
 * left to right, where order' is `order` without `local`.  With s->arrived,
 * a source is read only after its flag shows the epoch (with system-scope
 * coherent loads, so a copy engine may have written it during the call); each
 * pass adds the longest run of pending sources (in that order) that have all
 * landed, so the bits never depend on arrival timing.
 * Intermediate fp32 sums of a multi-pass reduce are kept in dst when dst is
 * fp32 (dst may equal srcs[local]: in place) and in srcs[local] when dst is
 * bf16 (srcs[local] is then overwritten).  n % 4 == 0 and 16-byte aligned
 * pointers are required.  Errors: NULL, SHAPE, ALIGN, DTYPE, ORDER, SCHEDULE,
 * ALIAS, HIP. */
fo_status fo_chunk_reduce(void *dst, fo_dtype dst_dtype, const float *const *srcs,
                          int64_t n, const fo_schedule *s, void *stream);

/* Emulated peer arrivals on `stream` (a side stream, normally).  For each i in
 * 0..count-1 in array order: wait until issue_ns[i] after the call's start
 * t0, copy bytes[i] from src[i] to dst[i] on a DMA (SDMA) engine, wait until
 * release_ns[i] after t0 and after the copy, then record the device wall clock
 * in stamps[1 + chunk_id[i]] and store arrived[chunk_id[i]] = epoch, written
 * through to memory (the copy has completed before the store, in stream
 * order; a consumer acquires before reading the chunk).  stamps[0] receives
 * t0.
 *   dst, src, bytes, issue_ns, release_ns, chunk_id: host arrays [count];
 *   issue_ns may be NULL (each copy is issued at its release time); a zero
 *   bytes[i] releases only the flag (the data are already in place).
 *   arrived: device [R].
 *   stamps: device [2 + max chunk id], required: stamps[0] is the timeline's
 *   start, which every flag kernel of the call reads (NULL: FO_ERR_NULL).
 * Errors: NULL, SHAPE (count < 0), SCHEDULE (epoch 0, chunk id out of range,
 * negative or inverted times), HIP. */
fo_status fo_emulate_arrivals(void *const *dst, const void *const *src,
                              const size_t *bytes, const int64_t *issue_ns,
                              const int64_t *release_ns, const int32_t *chunk_id,
                              int32_t count, uint32_t *arrived, uint32_t epoch,
                              uint64_t *stamps, void *stream);

/* fo_emulate_arrivals whose timeline starts when a device word becomes
 * nonzero: the timer kernel first waits (at most gate_timeout_ns, 0 = 10 s)
 * until *gate != 0, then records t0; issue and release times count from
 * there.  With gate = the consumer kernel's start stamp (stamps[2R] of a
 * GEMM call, zeroed before the call) the emulated peers start sending when
 * the consumer starts, however long the host takes to enqueue the arrivals.
 * Each message is three operations on `stream`; with many messages the
 * runtime's queue fills and this call blocks the host until operations
 * retire, which the timer's gate holds back: enqueue the consumer before
 * the arrivals (or the host waits out the gate's timeout).
 * gate NULL behaves as fo_emulate_arrivals.  Errors as fo_emulate_arrivals. */
fo_status fo_emulate_arrivals_gated(const uint64_t *gate, uint64_t gate_timeout_ns,
                                    void *const *dst, const void *const *src,
                                    const size_t *bytes, const int64_t *issue_ns,
                                    const int64_t *release_ns, const int32_t *chunk_id,
                                    int32_t count, uint32_t *arrived, uint32_t epoch,
                                    uint64_t *stamps, void *stream);

/* Emulated peer sends of the reduce-scatter (technical summary §2, Flash-RS:
 * the partial outputs destined for peers are computed first so that their
 * sends start while the rest is computed).  On `stream` (a side stream,
 * normally), for each i in 0..count-1 in array order, one send after another
 * (one link):
 *   wait until done[chunk_id[i]] shows the epoch (the GEMM-RS launch released
 *   that chunk's rows; bounded by timeout_ns, 0 = 10 s; a timeout writes
 *   FO_ERR_TIMEOUT to *status if given and the send goes ahead), record
 *   stamps[2i] = start; copy bytes[i] from src[i] to dst[i] on a DMA (SDMA)
 *   engine; hold until link_ns[i] after the start (the modelled time on the
 *   link) and after the copy; record stamps[2i+1] = completion.
 *   done: device [R] flags written by fo_gemm_rs / fo_gemm_rs_reduce /
 *   fo_gemm_rs_ring; dst, src, bytes, chunk_id, link_ns: host [count];
 *   stamps: device [2*count] (device wall-clock ticks), required.
 * Errors: NULL, SHAPE (count < 0), SCHEDULE (epoch 0, chunk id out of range,
 * negative link time), HIP. */
fo_status fo_emulate_sends(const uint32_t *done, uint32_t epoch, void *const *dst,
                           const void *const *src, const size_t *bytes, const int32_t *chunk_id,
                           const int64_t *link_ns, int32_t count, uint64_t timeout_ns,
                           int32_t *status, uint64_t *stamps, void *stream);

/* Schedule model for fo_ag_gemm (host only; euno.news "Methodology" step 3:
 * the scheduler models the dependency graph of pieces and sub-tasks;
 * technical summary §2: work on incoming data first, the local slice last).
 * Given when each peer chunk is expected to land, returns the priority order
 * (peers by landing time, ties in ring order local-1, local-2, ...; the
 * local chunk last) and the split vector (1 everywhere except the chunk that
 * lands last, split 1, 2, 4 or 8 ways along k).  A simulation of the
 * kernel's ready-first claims over `num_workgroups` workgroups (processor
 * sharing of the GPU's rate among running units) predicts the completion for
 * each split; the earliest wins, a larger split by more than 0.5 us.  A chunk
 * landing on an idle GPU is split so every workgroup shares its tiles; one
 * landing while the workgroups are busy is not, since its split units would
 * queue behind them.  The result is meant for fo_schedule.order and .split.
 *   arrival_ns      host [R]: expected landing time of chunk c after t0
 *                   (the local chunk's entry is ignored).
 *   gemm_tflops     sustained rate of one launch with every workgroup busy;
 *                   <= 0 selects 900.
 *   num_workgroups  workgroups of the launch; <= 0 = one per CU of the
 *                   current device (needs a device).
 *   order_out, split_out  host [R].
 *   predicted_ns    host [4], optional: the predicted completion (ns after
 *                   t0) with the last chunk split 1, 2, 4, 8 ways; -1 where
 *                   that split is not possible (k too short, or R == 1).
 * Errors: NULL, SHAPE, SCHEDULE (local out of range, negative arrival), HIP
 * (no device when num_workgroups <= 0). */
fo_status fo_plan_ag_schedule(int64_t m, int64_t n, int64_t k, int32_t nchunks, int32_t local,
                              const int64_t *arrival_ns, double gemm_tflops,
                              int32_t num_workgroups, int32_t *order_out, int32_t *split_out,
                              int64_t *predicted_ns);

/* Calibration of the schedule model: measured facts of a launch shape on the
 * device.  Fields <= 0 take the defaults (measured on MI355X on the TP=8 MLP
 * up-projection share): 900 TFLOP/s, alone speed-up 1.8, 5 us from a flag
 * store to a claim walk's first unit, 2 us to a held unit's first loads,
 * 1.5 us of claim and bookkeeping per unit, 5 TB/s of HBM for the reduce. */
typedef struct fo_plan_calib {
  double gemm_tflops;         /* launch rate with every workgroup busy          */
  double alone_speedup;       /* a workgroup alone vs its share of a busy GPU   */
  double flag_latency_ns;     /* flag store -> first unit by a claim walk       */
  double reserve_latency_ns;  /* flag store -> first loads of a held unit       */
  double unit_fixed_ns;       /* claim and bookkeeping per unit                 */
  double hbm_gbps;            /* HBM rate of the reduce passes (bytes per ns)   */
} fo_plan_calib;

/* Calibrates the schedule model for an m x n x k AG-GEMM in R chunks from
 * measured launches (euno.news "Methodology" step 3; "Limitations": the
 * model assumes uniform links, so it is fitted per shape and device):
 *   all_present_ns   one launch with every chunk landed (required, > 4 us);
 *   chunk_alone_ns   one chunk's rows alone, unsplit (<= 0: keep default
 *                    alone speed-up);
 *   tail_unsplit_ns  measured exposed tail with the last chunk unsplit and
 *                    the GPU idle when it lands (<= 0: keep default latency).
 * Host only; num_workgroups <= 0 asks the current device for its CUs.
 * Errors: NULL, SHAPE, SCHEDULE, HIP. */
fo_status fo_plan_calibrate(int64_t m, int64_t n, int64_t k, int32_t nchunks, double all_present_ns,
                            double chunk_alone_ns, double tail_unsplit_ns, int32_t num_workgroups,
                            fo_plan_calib *out);

/* Link model (host only): when each message of the decomposed all-gather
 * lands, for chunks of chunk_bytes over links of link_gbps (bytes per ns),
 * each peer chunk streamed as `sub` messages.
 *   FO_LINK_RING  one incoming link: the chunk of ring distance d is sent in
 *                 [(d-1) T, d T] with T = chunk_bytes / link_gbps;
 *   FO_LINK_MESH  one link per peer: every peer sends in [0, T].
 * Message j of chunk c lands at the start of its chunk's window plus
 * (j + 1) T / sub.  arrival_ns: host [R * sub], message c * sub + j; the
 * local chunk's entries are 0.  Errors: NULL, SHAPE (R * sub > 64),
 * SCHEDULE. */
enum { FO_LINK_RING = 0, FO_LINK_MESH = 1 };
fo_status fo_plan_link_arrivals(int32_t nchunks, int32_t local, int64_t chunk_bytes, double link_gbps,
                                int32_t topology, int32_t sub, int64_t *arrival_ns);

/* Streamed schedule for fo_ag_gemm (host only): chooses how many messages
 * (1, 2, 4 or 8) each peer chunk of the AG-GEMM is streamed in, and the
 * split of the piece that lands last, by the earliest predicted completion
 * under the link model (more messages only when they win by more than
 * 0.5 us: small pieces cost more per unit).  With sub messages the launch
 * takes R * sub chunks of m / (R * sub) rows (piece c * sub + j = rows of
 * message j of chunk c); the local chunk's pieces are present (flag them,
 * and pass any one of them as local).
 *   calib           NULL or a calibration (fo_plan_calibrate).
 *   sub_out         the chosen number of messages per chunk.
 *   order_out, split_out  host [64]: the first R * sub entries are the
 *                   priority order and split vector for fo_schedule.
 *   predicted_ns    host [16], optional: completion predicted for messages
 *                   {1, 2, 4, 8} x split {1, 2, 4, 8} (row-major; -1 where
 *                   not possible).
 * Errors: NULL, SHAPE, SCHEDULE, HIP (no device when num_workgroups <= 0). */
fo_status fo_plan_ag_stream(int64_t m, int64_t n, int64_t k, int32_t nchunks, int32_t local,
                            double link_gbps, int32_t topology, const fo_plan_calib *calib,
                            int32_t num_workgroups, int32_t *sub_out, int32_t *order_out,
                            int32_t *split_out, int64_t *predicted_ns);

/* Reduce-scatter form (host only; technical summary §2, Flash-RS): given
 * when each peer's fp32 partial for the local chunk lands (arrival_ns host
 * [R], the local entry ignored), predicts when the bf16 shard is complete
 * for GEMM-RS then fo_chunk_reduce (0), fo_gemm_rs_reduce (1) and
 * fo_gemm_rs_ring with the accumulated partial landing last (2), and picks
 * the earliest (a later form only if it wins by more than 0.5 us).
 * predicted_ns host [3], optional.  Errors: NULL, SHAPE, SCHEDULE, HIP. */
fo_status fo_plan_rs_form(int64_t m, int64_t n, int64_t k, int32_t nchunks, int32_t local,
                          const int64_t *arrival_ns, const fo_plan_calib *calib, int32_t num_workgroups,
                          int32_t *form_out, int64_t *predicted_ns);

/* Device facts used to interpret stamps and size launches. */
fo_status fo_device_info(int32_t *num_cus, int32_t *lds_bytes_per_cu,
                         uint64_t *wall_clock_hz);

const char *fo_status_string(fo_status st);

/* Text of the last HIP error seen by the calling thread ("" if none). */
const char *fo_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FLASHOVERLAP_H */
