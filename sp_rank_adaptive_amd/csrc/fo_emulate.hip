// Peer emulator kernels: one-wave timers that release emulated peer chunks.
//
// The decomposed collective's receive side (FlashOverlap abstract and
// euno.news "Methodology" step 1: the collective becomes directed
// peer-to-peer messages) is emulated on one GPU: each peer chunk is a copy
// from a staging region of the same HBM on a DMA engine, enqueued between these
// kernels on a side stream.  A timer kernel holds the stream until the copy's
// issue time; a flag kernel waits for the chunk's release time, records the
// device wall clock and stores the chunk's epoch flag, written through to
// memory.
// Each kernel is a single wave that sleeps between clock reads.
#include "fo_device.hpp"
#include "fo_internal.hpp"

namespace fo {

__device__ __forceinline__ void sleep_until(uint64_t t0, uint64_t offset) {
  while (now_ticks() - t0 < offset) __builtin_amdgcn_s_sleep(16);
}

// With a gate, the timeline starts once *gate is nonzero (the consumer
// kernel's start stamp, say), waiting at most gate_ticks.
__global__ void __launch_bounds__(64) emu_start_kernel(uint64_t *t0_slot, uint64_t wait_ticks,
                                                       const uint64_t *gate, uint64_t gate_ticks) {
  if (threadIdx.x != 0) return;
  if (gate) {
    const uint64_t g0 = now_ticks();
    while (__hip_atomic_load(gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == 0 &&
           now_ticks() - g0 < gate_ticks)
      __builtin_amdgcn_s_sleep(2);
  }
  const uint64_t t0 = now_ticks();
  store_u64_relaxed(t0_slot, t0);
  sleep_until(t0, wait_ticks);
}

__global__ void __launch_bounds__(64) emu_flag_kernel(const uint64_t *t0_slot, uint64_t release_ticks,
                                                      uint64_t next_issue_ticks, uint32_t *flag,
                                                      uint32_t epoch, uint64_t *stamp_slot) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = __hip_atomic_load(t0_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  sleep_until(t0, release_ticks);
  if (stamp_slot) store_u64_relaxed(stamp_slot, now_ticks());
  // The chunk's bytes were written by the copy engine, which finished before
  // this kernel started: there is nothing of this kernel's own to release.  A
  // release store would write back this XCD's whole L2 (dirty lines of the
  // concurrent GEMM included) before the flag becomes visible, delaying it by
  // microseconds; the flag store itself is written through to memory.
  __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  sleep_until(t0, next_issue_ticks);
}

// Send side: waits (bounded) until *flag shows the epoch (a chunk the
// producer has finished), then records the start of the send in
// *start_slot; a timeout writes FO_ERR_TIMEOUT to *status (if given) and
// still records the stamp, so the stream moves on.
__global__ void __launch_bounds__(64) emu_wait_flag_kernel(const uint32_t *flag, uint32_t epoch, uint64_t timeout_ticks,
                                                           int32_t *status, uint64_t *start_slot) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = now_ticks();
  while (!epoch_reached(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM), epoch)) {
    if (now_ticks() - t0 > timeout_ticks) {
      if (status) __hip_atomic_store(status, (int32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  // the flag's release ordered the producer's written-through rows before
  // it; the copy engine reads them after this kernel ends (stream order)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  store_u64_relaxed(start_slot, now_ticks());
}

// Send side: holds the stream until `link_ticks` after *start_slot (the
// modelled time the message occupies the link), then records the send's
// completion in *done_slot.
__global__ void __launch_bounds__(64) emu_hold_kernel(const uint64_t *start_slot, uint64_t link_ticks, uint64_t *done_slot) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = __hip_atomic_load(start_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  sleep_until(t0, link_ticks);
  store_u64_relaxed(done_slot, now_ticks());
}

hipError_t launch_emu_wait_flag(const uint32_t *flag, uint32_t epoch, uint64_t timeout_ticks, int32_t *status,
                                uint64_t *start_slot, hipStream_t s) {
  hipLaunchKernelGGL(emu_wait_flag_kernel, dim3(1), dim3(64), 0, s, flag, epoch, timeout_ticks, status, start_slot);
  return hipGetLastError();
}

hipError_t launch_emu_hold(const uint64_t *start_slot, uint64_t link_ticks, uint64_t *done_slot, hipStream_t s) {
  hipLaunchKernelGGL(emu_hold_kernel, dim3(1), dim3(64), 0, s, start_slot, link_ticks, done_slot);
  return hipGetLastError();
}

hipError_t launch_emu_start(uint64_t *t0_slot, uint64_t wait_ticks, const uint64_t *gate,
                            uint64_t gate_ticks, hipStream_t s) {
  hipLaunchKernelGGL(emu_start_kernel, dim3(1), dim3(64), 0, s, t0_slot, wait_ticks, gate, gate_ticks);
  return hipGetLastError();
}

hipError_t launch_emu_flag(const uint64_t *t0_slot, uint64_t release_ticks, uint64_t next_issue_ticks,
                           uint32_t *flag, uint32_t epoch, uint64_t *stamp_slot, hipStream_t s) {
  hipLaunchKernelGGL(emu_flag_kernel, dim3(1), dim3(64), 0, s, t0_slot, release_ticks, next_issue_ticks,
                     flag, epoch, stamp_slot);
  return hipGetLastError();
}

}  // namespace fo
