// Building blocks of the gfx950 MFMA tile kernels (the chunked GEMM and the
// all-to-all GEMM): the LDS stage ring of a BM x BN tile, copies straight from
// global memory into LDS by the buffer-load DMA path, write-through stores and
// the waits between them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;   // threads of 4 waves (one copy group)
constexpr uint32_t kBufDword3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9)

// Tile of BM x BN outputs; k staged through an LDS ring of STAGES buffers,
// BK at a time (BK = 32 or 64: one or two MFMA k-steps per stage).  The
// compute waves form a WGM x WGN grid over the tile.
template <int BM, int BN, int BK, int STAGES, int WGM = 2, int WGN = 2>
struct Cfg {
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile
  static constexpr int FM = WTM / 16, FN = WTN / 16; // MFMA blocks per wave
  static constexpr int ROWB = BK * 2;                // LDS bytes per operand row
  static constexpr int CH = BK / 8;                  // 16-byte pieces per row
  static constexpr int RSTEP = NT / CH;              // rows covered by one load round
  static constexpr int AV = BM / RSTEP;              // load rounds per stage (X)
  static constexpr int BV = BN / RSTEP;              // load rounds per stage (W)
  static constexpr int V = AV + BV;
  static constexpr int KS = BK / 32;                 // MFMA k-steps per stage
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int B_BYTES = BN * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_RING = STAGES * STAGE;
  // The epilogue stages fp32 output rows padded by 4 floats (16 bytes), half
  // a tile at a time when the whole tile does not fit; the LDS block is the
  // larger of the ring and that staging area.
  static constexpr int EPI_HALF = BM / 2 * (BN + 4) * 4;
  static constexpr int LDS = LDS_RING > EPI_HALF ? LDS_RING : EPI_HALF;
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(STAGES >= 2 && STAGES <= 4, "STAGES");
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert(BM % RSTEP == 0 && BN % RSTEP == 0, "tile loads");
  static_assert(LDS + 64 <= 160 * 1024, "LDS");
  // 16-byte piece `ch` of row `r` lives at piece ch ^ swz(r): the fragment
  // reads of 8 consecutive rows then cover 8 distinct 16-byte bank groups.
  __device__ static constexpr int swz(int r) { return BK == 64 ? (r & 7) : ((r >> 1) & 3); }
};

// LDS byte address of a shared-memory pointer (the DMA destination base).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16-byte store written through every cache level to memory (system-scope
// cache policy).  Output that another agent or XCD consumes is stored this
// way, so a unit only has to wait for its own stores to be acknowledged
// (wait_stores) before it counts itself, instead of a release fence that
// writes back the whole L2 of its XCD.  The compiler does not track these
// stores: every path that issues them ends in wait_stores.
// The store reads its data registers after it issues, and the compiler,
// which sees only an asm statement, may write those registers with the very
// next instruction; the wait states after the store (the hardware's rule for
// stores of more than 8 bytes asks for one) cover that window.
__device__ __forceinline__ void store_wt16(void *p, const f32x4 &v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ void store_wt8(void *p, const u32x2 &v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc0 sc1\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ void wait_stores() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// 16 bytes per lane from a buffer resource straight into LDS: lane L's bytes
// land at m0 + 16 L.  Issued from asm so the compiler does not wait for
// every outstanding copy before each LDS read; waits are explicit
// (wait_vm) and a workgroup barrier follows them before any read.
__device__ __forceinline__ void dma16(uint32_t m0, int voff, __amdgpu_buffer_rsrc_t rs, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(rs),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
}

// dma16 at system-coherent cache policy (sc0 sc1): data other workgroups
// wrote through during this launch is read from the coherence point, never
// from a stale line of this XCD's L2.
__device__ __forceinline__ void dma16_coherent(uint32_t m0, int voff, __amdgpu_buffer_rsrc_t rs, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen sc0 sc1 lds"
               :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(rs),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
}

// Raw buffer resource over `bytes` bytes at p, built from wave-uniform
// (scalar) values so it can feed the scalar operand of a buffer load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *p, int bytes) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0,
                                          __builtin_amdgcn_readfirstlane(bytes), (int)kBufDword3);
}


// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

// Wait for this wave's copies of stage j when `later` stages issued after it
// may stay in flight (VR copies per stage and wave).
template <int VR, int STAGES>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (STAGES >= 4) { if (later >= 2) { wait_vm<2 * VR>(); return; } }
  if constexpr (STAGES >= 3) { if (later >= 1) { wait_vm<VR>(); return; } }
  wait_vm<0>();
}

}  // namespace fo
