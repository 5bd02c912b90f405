// Persistent chunked GEMM for gfx950: bf16 MFMA (16x16x32), fp32 accumulate,
// LDS-staged double-buffered tiles, work claimed chunk by chunk as the chunks'
// epoch flags show them landed.
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
// One workgroup = 4 waves (one per SIMD) computing a BM x BN output tile; each
// wave owns a (BM/2) x (BN/2) quadrant made of 16x16 MFMA blocks.  Operand
// tiles of BM x 64 (X rows) and BN x 64 (W rows, i.e. output columns) sit in
// LDS with a 16-byte XOR swizzle so the MFMA fragment reads of 8 consecutive
// rows hit distinct bank groups.
#include "fo_device.hpp"
#include "fo_internal.hpp"

namespace fo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;    // k depth of one LDS stage (two MFMA k-steps of 32)
constexpr int NT = 256;   // threads per workgroup

template <int BM, int BN>
struct Cfg {
  static constexpr int WTM = BM / 2, WTN = BN / 2;   // wave tile
  static constexpr int FM = WTM / 16, FN = WTN / 16; // MFMA blocks per wave
  static constexpr int AV = BM * 8 / NT;             // 16-byte loads per thread (X)
  static constexpr int BV = BN * 8 / NT;             // 16-byte loads per thread (W)
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile loads");
};

struct ClaimState {
  uint64_t landed;     // bit c: chunk c seen landed (acquire done)
  uint64_t exhausted;  // bit c: chunk c has no unit left
};

// Thread 0 of a workgroup: pick the next unit.  Returns the chunk (>= 0) and
// sets `unit`; -1 when every chunk is exhausted; -2 on abort or timeout.
__device__ int claim_unit(const GemmArgs &a, ClaimState &st, int &unit, uint64_t t_begin) {
  uint64_t wait_from = 0;
  for (;;) {
    bool waiting = false;
    for (int s = 0; s < a.R; ++s) {
      const int c = a.order[s];
      const uint64_t bit = 1ull << c;
      if (st.exhausted & bit) continue;
      if (!(st.landed & bit)) {
        if (a.arrived == nullptr || c == a.local) {
          st.landed |= bit;
        } else if (epoch_reached(load_relaxed(a.arrived + c), a.epoch)) {
          // flag seen: make the copy's data visible before any read of it
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
          st.landed |= bit;
        } else {
          waiting = true;
          if (a.strict) break;
          continue;
        }
      }
      const uint32_t u = fetch_add_relaxed(a.ws32 + WS_CLAIM + c, 1u);
      if ((int)u < a.units[c]) {
        unit = (int)u;
        return c;
      }
      st.exhausted |= bit;
    }
    if (!waiting) return -1;
    if (load_relaxed(a.ws32 + WS_ABORT)) return -2;
    const uint64_t t = now_ticks();
    if (wait_from == 0) wait_from = t;
    if (t - wait_from > a.timeout_ticks) {
      if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(a.ws32 + WS_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return -2;
    }
    (void)t_begin;
    __builtin_amdgcn_s_sleep(4);
  }
}

template <int BM, int BN>
__global__ void __launch_bounds__(NT, 1) gemm_kernel(GemmArgs a) {
  using C = Cfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  __shared__ int s_chunk, s_unit, s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t K = a.k, N = a.n;

  ClaimState st{0ull, 0ull};
  const uint64_t t_begin = now_ticks();
  if (blockIdx.x == 0 && tid == 0 && a.stamps) store_u64_relaxed(a.stamps + 2 * a.R, t_begin);

  for (;;) {
    if (tid == 0) {
      int u = 0;
      const int c = claim_unit(a, st, u, t_begin);
      s_chunk = c;
      s_unit = u;
    }
    __syncthreads();
    const int c = s_chunk;
    const int u = s_unit;
    if (c < 0) break;
    if (u == 0 && tid == 0 && a.stamps) store_u64_relaxed(a.stamps + c, now_ticks());

    const int S = a.split[c];
    const int tile = u / S;
    const int sp = u - tile * S;
    const int tm = tile / a.tiles_n;
    const int tn = tile - tm * a.tiles_n;
    const int64_t row0 = (int64_t)c * a.mc + (int64_t)tm * BM;
    const int64_t rowlim = (int64_t)(c + 1) * a.mc;
    const int64_t col0 = (int64_t)tn * BN;
    const int64_t k0 = (int64_t)sp * a.kslice[c];
    const int64_t k1 = (k0 + a.kslice[c] < K) ? k0 + a.kslice[c] : K;
    const int KT = (int)((k1 - k0 + BK - 1) / BK);

    u32x4 ra[C::AV], rb[C::BV];
    auto gload = [&](int64_t kk) {
#pragma unroll
      for (int v = 0; v < C::AV; ++v) {
        const int idx = tid + v * NT;
        const int r = idx >> 3, ch = idx & 7;
        const int64_t row = row0 + r, kc = kk + ch * 8;
        if (row < rowlim && kc < k1)
          ra[v] = *reinterpret_cast<const u32x4 *>(a.x + row * K + kc);
        else
          ra[v] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int v = 0; v < C::BV; ++v) {
        const int idx = tid + v * NT;
        const int r = idx >> 3, ch = idx & 7;
        const int64_t col = col0 + r, kc = kk + ch * 8;
        if (col < N && kc < k1)
          rb[v] = *reinterpret_cast<const u32x4 *>(a.w + col * K + kc);
        else
          rb[v] = u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto sstore = [&](int stage) {
      char *A = lds + stage * C::STAGE;
      char *B = A + C::A_BYTES;
#pragma unroll
      for (int v = 0; v < C::AV; ++v) {
        const int idx = tid + v * NT;
        const int r = idx >> 3, ch = idx & 7;
        *reinterpret_cast<u32x4 *>(A + r * 128 + ((ch ^ (r & 7)) << 4)) = ra[v];
      }
#pragma unroll
      for (int v = 0; v < C::BV; ++v) {
        const int idx = tid + v * NT;
        const int r = idx >> 3, ch = idx & 7;
        *reinterpret_cast<u32x4 *>(B + r * 128 + ((ch ^ (r & 7)) << 4)) = rb[v];
      }
    };

    f32x4 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gload(k0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) gload(k0 + (int64_t)(kt + 1) * BK);
      const char *A = lds + cur * C::STAGE;
      const char *B = A + C::A_BYTES;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ch = ks * 4 + (lane >> 4);
        const int swz = ((ch ^ (lane & 7)) << 4);
        bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const int r = wm * C::WTM + i * 16 + (lane & 15);
          af[i] = *reinterpret_cast<const bf16x8 *>(A + r * 128 + swz);
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int r = wn * C::WTN + j * 16 + (lane & 15);
          bfr[j] = *reinterpret_cast<const bf16x8 *>(B + r * 128 + swz);
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) sstore(cur ^ 1);
      __syncthreads();
    }

    bool write_out = true;
    if (S > 1) {
      // Deterministic split-K: every split stores its fp32 partial tile; the
      // split that arrives last sums the S partials in split order 0..S-1.
      const int ctr = a.ctr_base[c] + tile;
      const size_t pbase = (size_t)a.part_base[c] + (size_t)tile * S;
      f32x4 *mine = reinterpret_cast<f32x4 *>(a.partials + (pbase + sp) * (BM * BN));
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mine[((wave * C::FM + i) * C::FN + j) * 64 + lane] = acc[i][j];
      fence_release_agent();
      __syncthreads();
      if (tid == 0) {
        const uint32_t old = fetch_add_acq_rel(a.ws32 + WS_TILE_CTR + ctr, 1u);
        s_last = (old == (uint32_t)(S - 1));
      }
      __syncthreads();
      write_out = s_last != 0;
      if (write_out) {
        fence_acquire_agent();
        f32x4 sum[C::FM][C::FN];
        for (int q = 0; q < S; ++q) {
          const f32x4 *p = reinterpret_cast<const f32x4 *>(a.partials + (pbase + q) * (BM * BN));
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
              const f32x4 v = (q == sp) ? acc[i][j] : p[((wave * C::FM + i) * C::FN + j) * 64 + lane];
              sum[i][j] = (q == 0) ? v : sum[i][j] + v;
            }
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) acc[i][j] = sum[i][j];
      }
    }

    if (write_out) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int64_t col = col0 + wn * C::WTN + j * 16 + (lane & 15);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int64_t row = row0 + wm * C::WTM + i * 16 + (lane >> 4) * 4 + v;
            if (row < rowlim && col < N) {
              if (a.y_bf16)
                reinterpret_cast<uint16_t *>(a.y)[row * N + col] = f32_to_bf16_rne(acc[i][j][v]);
              else
                reinterpret_cast<float *>(a.y)[row * N + col] = acc[i][j][v];
            }
          }
        }
    }

    // Completion accounting; in GEMM-RS mode the chunk's done flag is released
    // after every output element of the chunk is stored.
    if (a.done_flags) fence_release_agent();
    __syncthreads();
    if (tid == 0) {
      const uint32_t d = fetch_add_acq_rel(a.ws32 + WS_CHUNK_DONE + c, 1u);
      if (d == (uint32_t)(a.units[c] - 1)) {
        if (a.stamps) store_u64_relaxed(a.stamps + a.R + c, now_ticks());
        if (a.done_flags) store_release(a.done_flags + c, a.epoch);
      }
      const uint32_t t = fetch_add_acq_rel(a.ws32 + WS_TOTAL_DONE, 1u);
      if (t == (uint32_t)(a.total_units - 1) && a.stamps)
        store_u64_relaxed(a.stamps + 2 * a.R + 1, now_ticks());
    }
  }

  // The last workgroup to leave returns every counter to zero for the next call.
  if (tid == 0) {
    const uint32_t e = fetch_add_acq_rel(a.ws32 + WS_EXITED, 1u);
    if (e == (uint32_t)(a.grid - 1)) {
      for (int c = 0; c < a.R; ++c) {
        a.ws32[WS_CLAIM + c] = 0u;
        a.ws32[WS_CHUNK_DONE + c] = 0u;
        if (a.ctr_base[c] >= 0) {
          const int ntiles = a.units[c] / a.split[c];
          for (int t = 0; t < ntiles; ++t) a.ws32[WS_TILE_CTR + a.ctr_base[c] + t] = 0u;
        }
      }
      a.ws32[WS_TOTAL_DONE] = 0u;
      a.ws32[WS_ABORT] = 0u;
      a.ws32[WS_EXITED] = 0u;
    }
  }
}

TileCfg choose_tile(int64_t mc, int64_t n, int64_t k) {
  (void)mc; (void)n; (void)k;
  return TileCfg{128, 128};
}

size_t partial_slot_bytes(const TileCfg &t) { return (size_t)t.bm * t.bn * sizeof(float); }

hipError_t launch_gemm(const GemmArgs &a, const TileCfg &t, hipStream_t stream) {
  if (t.bm == 128 && t.bn == 128) {
    hipLaunchKernelGGL((gemm_kernel<128, 128>), dim3(a.grid), dim3(NT), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fo
