// All-to-all GEMM for gfx950: Y = sum over pieces q of A_q * W[:, block q],
// bf16 MFMA with fp32 accumulation, each piece's k-range multiplied as soon as
// its epoch flag shows it landed.
//
// Flash All-to-All (gist.science technical summary §2: the decomposed
// primitives extended to Ulysses parallelism; §1: Ulysses parallelism needs
// all-to-all).  After attention runs head-parallel, the all-to-all hands each
// rank, from every rank q, the rows of its sequence slice for q's heads: a
// column block A_q of the attention output, the contraction dimension of the
// output projection that follows.  Decomposed into peer-to-peer pieces, the
// projection proceeds piece by piece: the block already present first, then
// each peer's block as it lands, so after the last landing only that piece's
// share of the contraction is left in every tile.
//
// Layout and schedule
//  - One workgroup per CU computes 128 x 256 output tiles: 8 waves (two per
//    SIMD) in a 2 x 4 grid of 64 x 64 wave tiles; waves 0-3 also issue the
//    stage copies (the other wave on each SIMD keeps the matrix core busy
//    while one waits on a burst of copies).
//  - k is staged 64 at a time through a ring of 3 LDS buffers filled by the
//    buffer-load DMA path; a stage never straddles two pieces (a piece whose
//    extent is not a multiple of 64 ends in a stage whose missing columns
//    read as zero).
//  - Every tile adds the pieces in `order`, so the bits depend on the order
//    alone, never on landing times.  Wave 0 reads a piece's flag when the
//    copy of its first stage is due, and once a piece has landed performs one
//    system-scope acquire (the copy engine wrote the piece during the launch)
//    before any wave of the workgroup loads from it.
//  - Tiles are cut into 8 rectangles, one per XCD (workgroup b runs on XCD
//    b % 8), and each XCD's workgroups take its rectangle's tiles in turn.
#include "fo_device.hpp"
#include "fo_internal.hpp"
#include "fo_tile.hpp"

namespace fo {

namespace {

constexpr int A2A_BK = 64, A2A_STAGES = 3, A2A_WGM = 2, A2A_WGN = 4;

// Tile (tm, tn) of the tl-th tile of rectangle g, rectangles numbered row by
// row over a gm x gn cut of the tile grid (tiles inside a rectangle also row
// by row).
__device__ __forceinline__ void a2a_tile(const A2aArgs &a, int g, int tl, int &tm, int &tn) {
  const int i = g / a.gn, j = g - (g / a.gn) * a.gn;
  const int rlo = i * a.tiles_m / a.gm;
  const int clo = j * a.tiles_n / a.gn, chi = (j + 1) * a.tiles_n / a.gn;
  const int ncols = chi - clo;
  tm = rlo + tl / ncols;
  tn = clo + tl - (tl / ncols) * ncols;
}

// One stage of MFMAs (two 32-deep k-steps) from LDS buffer BUF: every X and W
// fragment of both k-steps is read, then the MFMAs follow in a pinned order.
template <typename C, bool FIRST, int BUF>
__device__ __forceinline__ void a2a_stage(f32x4 (&acc)[C::FM][C::FN], const char *lds, int wm, int wn, int lane) {
  const char *A = lds + BUF * C::STAGE;
  const char *B = A + C::A_BYTES;
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
        if (FIRST && ks == 0)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][i], bfr[ks][j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
      }
  // pinned order (mask 0x100: LDS reads, 0x008: MFMA): all reads of k-step 0,
  // then its MFMAs interleaved with the reads of k-step 1, then the rest
  constexpr int NF = C::FM + C::FN, NM = C::FM * C::FN;
  __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);
  static_for<NF>([&](auto) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  });
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * NM - NF, 0);
}

// Wave 0 (all lanes): extends `ready` (leading order positions known landed)
// past position pi, waiting for the flags (bounded), and takes every later
// position that has already landed.  Lane i reads position i's flag, so one
// round trip covers every piece.  Returns the new count (wave-uniform), or -1
// after a timeout or another workgroup's abort.  *peer: a peer's piece was
// taken (the caller acquires).
__device__ int a2a_poll(const A2aArgs &a, int ready, int pi, bool *peer) {
  const int lane = threadIdx.x & 63;
  const uint64_t t0 = now_ticks();
  for (;;) {
    bool landed = true, is_peer = false;
    if (lane < a.P) {
      const int q = a.order[lane];
      is_peer = a.arrived != nullptr && q != a.local;
      landed = !is_peer || epoch_reached(load_relaxed(a.arrived + q), a.epoch);
    }
    const uint64_t ok = __ballot(landed);
    const int r = (~ok == 0ull) ? 64 : __builtin_ctzll(~ok);   // leading landed positions
    const int rr = r < a.P ? r : a.P;
    if (rr > pi) {
      const uint64_t newly = __ballot(is_peer && lane >= ready && lane < rr);
      *peer = newly != 0ull;
      return rr;
    }
    bool out = false;
    if (lane == 0) out = load_relaxed(a.ws32 + WS_ABORT) != 0u || now_ticks() - t0 > a.timeout_ticks;
    if (__ballot(out)) {
      if (lane == 0) {
        if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(a.ws32 + WS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return -1;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN>
__global__ void __launch_bounds__(2 * NT, 1) __attribute__((amdgpu_num_vgpr(120)))
a2a_kernel(A2aArgs a) {
  using C = Cfg<BM, BN, BK, STAGES, WGM, WGN>;
  constexpr int NTT = 2 * NT;
  static_assert(WGM * WGN == 8, "eight compute waves");
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  // positions known landed, double-buffered by poll parity: a wave that reads
  // one slot late after a barrier still finds the value written before it
  __shared__ int s_ready[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool prod = wave < 4;                     // issues the stage copies
  const int wm = wave / WGN, wn = wave % WGN;
  const int cw = wave & 3;
  const int xg = (int)(blockIdx.x % XCDS);
  const int wgs = (a.grid - xg + XCDS - 1) / XCDS;  // workgroups on this XCD
  const int64_t K = a.k, N = a.n;
  const int kp = a.kp;
  const int KTP = (kp + BK - 1) / BK;             // stages per piece
  const int KT = a.P * KTP;
  asm volatile("" :: "v"(lds) : "memory");
  if (blockIdx.x == 0 && tid == 0 && a.stamps) store_u64_relaxed(a.stamps + 2 * a.P, now_ticks());

  int ready = 0;     // leading order positions whose pieces are known landed
  int slot = 0;
  bool aborted = false;
  int done_tiles = 0;

  for (int tl = (int)(blockIdx.x / XCDS); tl < a.gtiles[xg] && !aborted; tl += wgs) {
    int tm, tn;
    a2a_tile(a, xg, tl, tm, tn);
    const int64_t row0 = (int64_t)tm * BM, col0 = (int64_t)tn * BN;
    const int nra = (int)((a.m - row0 < BM) ? a.m - row0 : BM);
    const int nrb = (int)((N - col0 < BN) ? N - col0 : BN);
    const __amdgpu_buffer_rsrc_t rsb = uniform_rsrc(a.w + col0 * K, (int)(nrb * K * 2));
    const uint32_t lds0 = lds_addr(lds) + (uint32_t)(__builtin_amdgcn_readfirstlane(cw) * 1024);

    // Stage j: order position pi = j / KTP, piece q = order[pi], columns
    // [kin, kin + BK) of the piece.  X rows come from the piece (row stride
    // kp), W rows from the piece's column block of W (row stride k).  Thread
    // t fills slot t of each load round (see the chunked GEMM); columns past
    // the piece's end read as zero from both operands.
    auto issue = [&](int j) {
      const int pi = j / KTP;
      const int q = a.order[pi];
      const int kin = (j - pi * KTP) * BK;
      const __amdgpu_buffer_rsrc_t rsa = uniform_rsrc(a.piece[q] + row0 * kp, nra * kp * 2);
      int t = threadIdx.x;
      asm volatile("" : "+v"(t));
      const int rtr = (t & (NT - 1)) / C::CH;
      const int rtch = ((t & (NT - 1)) % C::CH) ^ C::swz(rtr);
      const bool in = kin + rtch * 8 < kp;
      const int voa = in ? (rtr * kp + rtch * 8) * 2 : 0x40000000;
      const int vob = in ? (int)((rtr * K + rtch * 8) * 2) : 0x40000000;
      const uint32_t base = lds0 + (uint32_t)((j % STAGES) * C::STAGE);
#pragma unroll
      for (int v = 0; v < C::V; ++v) {
        if (v < C::AV)
          dma16(base + (uint32_t)(v * 4096), voa, rsa, (C::RSTEP * v * kp + kin) * 2);
        else
          dma16(base + (uint32_t)(v * 4096), vob, rsb,
                (int)((C::RSTEP * (v - C::AV) * K + (int64_t)q * kp + kin) * 2));
      }
    };

    // Wave 0 makes sure the piece of stage j has landed before its copy is
    // issued; the barrier that follows publishes the count to every wave.
    // Returns false (every wave alike) after a timeout.
    auto need = [&](int j) { return j < KT && j / KTP >= ready; };
    auto poll = [&](int j) {
      if (wave == 0) {
        bool peer = false;
        const int r = __builtin_amdgcn_readfirstlane(a2a_poll(a, ready, j / KTP, &peer));
        if (peer) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");   // the landed pieces' bytes
        if (lane == 0) s_ready[slot] = r;
      }
    };
    auto take = [&]() {
      ready = __builtin_amdgcn_readfirstlane(s_ready[slot]);
      slot ^= 1;
      return ready >= 0;
    };

    f32x4 acc[C::FM][C::FN];
    auto wait_stage = [&](int j) {
      const int later = ((j + STAGES - 1 < KT) ? j + STAGES - 1 : KT) - (j + 1);
      wait_later<C::V, STAGES>(later);
    };

    // prologue: stages 0 .. STAGES-2 in flight (the buffers may still be read
    // by the previous tile's last stages: barrier first)
    __syncthreads();
    for (int p = 0; p < STAGES - 1 && p < KT && !aborted; ++p) {
      if (need(p)) {
        poll(p);
        __syncthreads();
        if (!take()) { aborted = true; break; }
      }
      if (prod) issue(p);
    }
    // iteration j: (poll for stage j+STAGES-1's piece); wait for stage j;
    // barrier; issue stage j+STAGES-1; multiply stage j
    auto iter = [&](int j, auto firstc, auto bufc) {
      const int jn = j + STAGES - 1;
      const bool nd = need(jn);
      if (nd) poll(jn);
      if (prod) wait_stage(j);
      __syncthreads();
      if (nd && !take()) return false;
      if (prod && jn < KT) issue(jn);
      a2a_stage<C, decltype(firstc)::value, decltype(bufc)::value>(acc, lds, wm, wn, lane);
      return true;
    };
    if (!aborted && !iter(0, std::true_type{}, std::integral_constant<int, 0>{})) aborted = true;
    for (int j0 = 1; j0 < KT && !aborted; j0 += STAGES) {
      static_for<STAGES>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        const int j = j0 + p;
        if (j < KT && !aborted && !iter(j, std::false_type{}, std::integral_constant<int, (1 + p) % STAGES>{}))
          aborted = true;
      });
    }
    if (aborted) {
      wait_vm<0>();      // no copy into LDS may still be in flight at exit
      break;
    }

    // Epilogue: the tile staged through LDS in padded fp32 rows, then stored
    // as 16-byte row pieces (fp32, or bf16 rounded to nearest even).
    {
      int etid = threadIdx.x;
      asm volatile("" : "+v"(etid));
      const int elane = etid & 63, ewave = etid >> 6;
      const int ewm = ewave / WGN, ewn = ewave % WGN;
      constexpr int SROW = BN + 4;
      static_assert(BM * SROW * 4 <= C::LDS, "epilogue staging");
      constexpr int CPR = BN / 4;
      float *stg = reinterpret_cast<float *>(lds);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = ewm * C::WTM + i * 16 + (elane >> 4) * 4 + v;
            stg[r * SROW + ewn * C::WTN + j * 16 + (elane & 15)] = acc[i][j][v];
          }
      __syncthreads();
      const bool vec_ok = (N & 3) == 0;
      for (int cidx = etid; cidx < BM * CPR; cidx += NTT) {
        const int r = cidx / CPR, cc = cidx - (cidx / CPR) * CPR;
        const int64_t row = row0 + r, col = col0 + cc * 4;
        if (row >= a.m || col >= N) continue;
        const f32x4 val = *reinterpret_cast<const f32x4 *>(stg + r * SROW + cc * 4);
        if (a.y_bf16) {
          uint16_t *q = reinterpret_cast<uint16_t *>(a.y) + row * N + col;
          if (vec_ok && col + 4 <= N) {
            const uint32_t lo = (uint32_t)f32_to_bf16_rne(val[0]) | ((uint32_t)f32_to_bf16_rne(val[1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_rne(val[2]) | ((uint32_t)f32_to_bf16_rne(val[3]) << 16);
            *reinterpret_cast<u32x2 *>(q) = u32x2{lo, hi};
          } else {
            for (int e = 0; e < 4 && col + e < N; ++e) q[e] = f32_to_bf16_rne(val[e]);
          }
        } else {
          float *q = reinterpret_cast<float *>(a.y) + row * N + col;
          if (vec_ok && col + 4 <= N) {
            *reinterpret_cast<f32x4 *>(q) = val;
          } else {
            for (int e = 0; e < 4 && col + e < N; ++e) q[e] = val[e];
          }
        }
      }
    }
    ++done_tiles;
  }

  // Completion stamp: the workgroup that finishes the last tile records it.
  // The last workgroup to leave returns the counters to zero; the exits are
  // counted per XCD, then per XCD group, so they do not queue on one
  // counter.  Without flags and stamps no counter is touched and nothing is
  // counted.
  __syncthreads();
  if (tid == 0 && (a.stamps || a.arrived)) {
    if (a.stamps && done_tiles > 0) {
      const int total = a.tiles_m * a.tiles_n;
      const uint32_t t = fetch_add_relaxed(a.ws32 + WS_TOTAL_DONE, (uint32_t)done_tiles);
      if ((int)(t + done_tiles) == total) store_u64_relaxed(a.stamps + 2 * a.P + 1, now_ticks());
    }
    const int xcd = (int)(blockIdx.x % XCDS);
    const int on_xcd = (a.grid - xcd + XCDS - 1) / XCDS;
    const int xcds = a.grid < XCDS ? a.grid : XCDS;
    bool last = fetch_add_relaxed(a.ws32 + WS_EXITED_X + xcd, 1u) == (uint32_t)(on_xcd - 1);
    if (last) last = fetch_add_relaxed(a.ws32 + WS_EXITED, 1u) == (uint32_t)(xcds - 1);
    if (last) {
      for (int g = 0; g < XCDS; ++g) store_relaxed_agent(a.ws32 + WS_EXITED_X + g, 0u);
      store_relaxed_agent(a.ws32 + WS_TOTAL_DONE, 0u);
      store_relaxed_agent(a.ws32 + WS_ABORT, 0u);
      store_relaxed_agent(a.ws32 + WS_EXITED, 0u);
    }
  }
}

}  // namespace

hipError_t launch_a2a(const A2aArgs &a, hipStream_t stream) {
  static_assert(A2A_BM == 128 && A2A_BN == 256, "tile");
  hipLaunchKernelGGL((a2a_kernel<A2A_BM, A2A_BN, A2A_BK, A2A_STAGES, A2A_WGM, A2A_WGN>), dim3(a.grid), dim3(2 * NT),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace fo
