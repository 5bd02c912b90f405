// Device-side helpers shared by the gfx950 kernels: epoch flags with
// acquire/release ordering, the constant-rate wall clock, bounded waits.
//
// Synchronisation between the peer emulator (copy engine + flag store) and the
// consuming kernels is the "communication and computation synchronization that
// keeps data consistent and free of races" of the FlashOverlap key designs
// (shd-paper.top digest, key designs item 3).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fo {

// Device wall clock (constant rate, see hipDeviceAttributeWallClockRate).
__device__ __forceinline__ uint64_t now_ticks() {
  return (uint64_t)wall_clock64();
}

// True once an epoch flag has reached `epoch` (wrap-safe comparison).
__device__ __forceinline__ bool epoch_reached(uint32_t flag, uint32_t epoch) {
  return (int32_t)(flag - epoch) >= 0;
}

__device__ __forceinline__ uint32_t load_relaxed(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void store_release(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void store_u64_relaxed(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Device-wide counters (workspace): relaxed atomics, performed at the
// coherence point, so every XCD sees one count.
__device__ __forceinline__ uint32_t fetch_add_relaxed(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_relaxed_agent(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_relaxed_agent(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// On gfx950 an agent-scope release fence writes the XCD's L2 back to memory
// and an acquire fence invalidates it: both are paid by every workgroup on
// the XCD, so the kernels fence only where data actually changes hands.
__device__ __forceinline__ void fence_acquire_agent() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace fo
