// Chunk reduce-add for gfx950: dst = src[seq 0] + src[seq 1] + ... (fp32),
// each peer source read only after its epoch flag shows it landed.
//
// The reduction inside the decomposed reduce-scatter (gist.science technical
// summary §1: data parallelism needs reduce-scatter; §2: Flash-RS sums the
// partial outputs into the slice that stays local).  HBM-bound: each workgroup
// owns a contiguous range of 16-byte vectors and streams it with coalesced
// 16-byte loads per lane; no workgroup waits for another, so there is no grid
// barrier.  A pass adds the longest run of pending sources (in summation
// order) that have all landed; the per-element addition order is therefore
// fixed by the order argument alone, never by arrival timing.
#include "fo_device.hpp"
#include "fo_internal.hpp"

namespace fo {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int RT = 256;  // threads per workgroup
constexpr int RU = 8;    // vectors per thread per step (128 bytes of each source in flight per lane)
constexpr int KB = 8;    // sources whose loads are issued together

// 16 bytes of a source that a copy engine wrote after this grid started, read
// coherently at system scope (cache policy sc0 sc1, plus the streaming hint):
// a line of it that an XCD's L2 still holds from before the copy is not
// returned.  Every byte of a source is read once, so nothing is lost by not
// caching it, and no workgroup needs an acquire fence, which would invalidate
// its XCD's whole L2 (once per workgroup, several microseconds in total).
__device__ __forceinline__ f32x4 load_landed(__amdgpu_buffer_rsrc_t rs, int64_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)byte_off, 0, 1 | 2 | 16));
}

// PEER: sources are gated by arrival flags (read with load_landed);
// otherwise every source was written before the launch.
template <bool OUT_BF16, bool PEER>
__global__ void __launch_bounds__(RT) reduce_kernel(ReduceArgs a) {
  __shared__ int s_avail;
  const int tid = threadIdx.x;
  const int64_t beg = (int64_t)blockIdx.x * a.per_wg4;
  const int64_t end = (beg + a.per_wg4 < a.n4) ? beg + a.per_wg4 : a.n4;
  if (blockIdx.x == 0 && tid == 0 && a.stamps) store_u64_relaxed(a.stamps, now_ticks());
  if (beg >= end) return;

  int added = 0;
  while (added < a.R) {
    if (tid == 0) {
      int av = added;
      uint64_t wait_from = 0;
      for (;;) {
        av = added;
        while (av < a.R && (av == 0 || a.arrived == nullptr ||
                            epoch_reached(load_relaxed(a.arrived + a.chunk_of[av]), a.epoch)))
          ++av;
        if (av > added) break;
        const uint64_t t = now_ticks();
        if (wait_from == 0) wait_from = t;
        if (t - wait_from > a.timeout_ticks) {
          if (a.status) __hip_atomic_store(a.status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
          av = -1;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      s_avail = av;
    }
    __syncthreads();
    const int av = s_avail;
    __syncthreads();
    if (av < 0) return;
    const bool last = (av == a.R);
    const int first_src = (added == 0) ? 1 : added;
    const f32x4 *init = (added == 0) ? reinterpret_cast<const f32x4 *>(a.src[0])
                                     : reinterpret_cast<const f32x4 *>(a.acc);

    // One step: RU vectors per thread.  Loads of up to KB sources are issued
    // together (bytes in flight hide HBM latency), then added in summation
    // order.  `full`: every vector of the step is inside the range.  Every
    // byte is touched once, so loads and stores carry the streaming
    // (nontemporal) hint.
    auto step = [&](int64_t base, bool full) {
      f32x4 v[RU];
#pragma unroll
      for (int q = 0; q < RU; ++q) {
        const int64_t i = base + (int64_t)q * RT;
        if (full || i < end) v[q] = __builtin_nontemporal_load(init + i);
      }
      for (int s0 = first_src; s0 < av; s0 += KB) {
        f32x4 t[KB][RU];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          if (s0 + k < av) {
            const f32x4 *p = reinterpret_cast<const f32x4 *>(a.src[s0 + k]);
            if constexpr (PEER) {
              // this workgroup's range of the source; offsets past it read zero
              const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                  (void *)(p + beg), (short)0, (int)((end - beg) * 16), 0x00020000);
#pragma unroll
              for (int q = 0; q < RU; ++q) {
                const int64_t i = base + (int64_t)q * RT;
                if (full || i < end) t[k][q] = load_landed(rs, (i - beg) * 16);
              }
            } else {
#pragma unroll
              for (int q = 0; q < RU; ++q) {
                const int64_t i = base + (int64_t)q * RT;
                if (full || i < end) t[k][q] = __builtin_nontemporal_load(p + i);
              }
            }
          }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k)
          if (s0 + k < av) {
#pragma unroll
            for (int q = 0; q < RU; ++q) v[q] += t[k][q];
          }
      }
#pragma unroll
      for (int q = 0; q < RU; ++q) {
        const int64_t i = base + (int64_t)q * RT;
        if (!full && i >= end) continue;
        if (last && OUT_BF16) {
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[q][0]) | ((uint32_t)f32_to_bf16_rne(v[q][1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[q][2]) | ((uint32_t)f32_to_bf16_rne(v[q][3]) << 16);
          reinterpret_cast<u32x2 *>(a.dst)[i] = u32x2{lo, hi};
        } else if (last) {
          __builtin_nontemporal_store(v[q], reinterpret_cast<f32x4 *>(a.dst) + i);
        } else {
          __builtin_nontemporal_store(v[q], reinterpret_cast<f32x4 *>(a.acc) + i);
        }
      }
    };
    int64_t w = beg;
    for (; w + (int64_t)RT * RU <= end; w += (int64_t)RT * RU) step(w + tid, true);
    if (w < end) step(w + tid, false);
    added = av;
  }

  if (a.stamps) {
    __syncthreads();
    if (tid == 0)
      __hip_atomic_fetch_max(a.stamps + 1, now_ticks(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_reduce(const ReduceArgs &a, int grid, hipStream_t stream) {
  const bool peer = a.arrived != nullptr;
  if (a.dst_bf16 && peer)
    hipLaunchKernelGGL((reduce_kernel<true, true>), dim3(grid), dim3(RT), 0, stream, a);
  else if (a.dst_bf16)
    hipLaunchKernelGGL((reduce_kernel<true, false>), dim3(grid), dim3(RT), 0, stream, a);
  else if (peer)
    hipLaunchKernelGGL((reduce_kernel<false, true>), dim3(grid), dim3(RT), 0, stream, a);
  else
    hipLaunchKernelGGL((reduce_kernel<false, false>), dim3(grid), dim3(RT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fo
