// Device-side building blocks shared by the attention kernels for gfx950:
// fragment types, the LDS row layout of bf16 tiles (XOR-swizzled 16-byte
// chunks), global -> LDS copies, wave-level reductions and the bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bss {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kMaskFull = 0, kMaskChunk = 1, kMaskWindow = 2, kMaskBlock = 3;

template <bool B>
struct Bool {
  static constexpr bool value = B;
};

template <int D>
struct Shape {
  static constexpr int CPR = D / 8;                          // 16-byte chunks per token row in memory
  static constexpr int RB = D * 2;                           // bytes per token row in memory
  // 16-byte chunks per row in LDS: d = 80 rows get two extra chunks whose V
  // slots hold the constant pad of the last O^T tile (element 80 = 1, so that
  // O^T row 80 is the row sum of P); the DMA never writes them.
  static constexpr int LCPR = (D == 80) ? 12 : CPR;
  static constexpr int LRB = LCPR * 16;                      // bytes per row in LDS
  static constexpr int KS = D / 16;                          // k-steps of the Q.K product
  static constexpr int DT = (D + 31) / 32;                   // 32-row tiles of O^T
  static constexpr int TILE = kBN * LRB;                     // bytes of one K (or V) tile in LDS
  static constexpr int LOADS = 2 * kBN * LCPR / 64 / kWaves; // LDS-DMA wave-instructions per wave per tile
  // waves 0-1 fill the K tile, waves 2-3 the V tile, LOADS wave-instructions each
  static_assert(2 * LOADS == LCPR, "each wave must cover half of one tensor's tile");
  // the XOR swizzle repeats every 16 rows; that many rows span DMA_PERIOD loads
  static constexpr int DMA_PERIOD = 16 * LCPR / 64;
  static_assert(LOADS % DMA_PERIOD == 0, "loads per wave must be whole swizzle periods");
  static constexpr bool PAD_ROWSUM = (D % 32) != 0;
  // S^T tiles start from minus the reference (the C operand of the first
  // k-step), so the scores come out of the MFMA already shifted.
  static constexpr bool SEEDED = true;
  // d = 64 and 80 software-pipeline the tiles (the VALU work of one tile
  // runs beside the MFMAs of the next); at d >= 128 the second score block
  // that needs does not fit the registers, and other kernels take over.
  static constexpr bool PIPELINED = D < 128;
};

// Physical 16-byte chunk of logical chunk c in LDS row `row` (an XOR, so its
// own inverse).  Chosen so that the 16 rows read by one K-fragment load, and
// the 4 rows x 64 bytes read by 32 lanes of one transposed V load, fall in
// distinct banks of a 64-bank LDS:
//   d = 128 (16 chunks):  c ^ {row bits 0-1 -> bits 2-3, row bits 2-3 -> bits 0-1}
//   d = 64  (8 chunks):   c ^ {row bit 1 -> bit 2, row bits 2-3 -> bits 0-1}
//   d = 80  (12 chunks):  c ^ row bits 2-3  (stays inside each aligned group of 4)
template <int D>
__device__ __forceinline__ int phys_chunk(int row, int c) {
  if constexpr (D == 128) return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  else if constexpr (D == 64) return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  else return c ^ ((row >> 2) & 3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// A wave-uniform 64-bit value moved to scalar registers (readfirstlane yields
// int: widen through uint32_t so the low half is not sign-extended).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t a) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32)));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One 16-byte global -> LDS copy per lane: lane l writes LDS bytes
// [lds_base + 16 l, lds_base + 16 l + 16) from base + voffset.  base and
// lds_base must be wave-uniform.  Issued as inline assembly so the compiler
// does not treat every later LDS read as aliasing it (it would then wait for
// the whole prefetch before any LDS read); completion is tracked by the
// explicit vmcnt waits in the main loop.
__device__ __forceinline__ void dma16(uint64_t base, uint32_t voffset, uint32_t lds_base) {
  __asm__ volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voffset), "s"(base), "s"(lds_base)
      : "memory", "m0");
}
// Same, with the lanes set in `skip` left out (exec is narrowed and restored
// inside the statement, so no branch is needed).
__device__ __forceinline__ void dma16_skip(uint64_t base, uint32_t voffset, uint32_t lds_base,
                                           uint64_t skip) {
  uint64_t saved;
  __asm__ volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_andn2_b64 exec, exec, %4\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voffset), "s"(base), "s"(lds_base), "s"(skip)
      : "memory", "m0", "scc");  // s_andn2_b64 writes SCC
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)(p)));
}

__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Max (or sum) of x over lanes l and l^32.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Value of x held by lane (l mod 32), delivered to lanes l and l^32.
__device__ __forceinline__ float low_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]);
}

// An empty asm that claims to modify x: values derived from x inside a loop
// can then not be hoisted out of it (used to recompute cheap addresses
// instead of keeping a register for each).
template <typename T>
__device__ __forceinline__ void opaque(T& x) {
  __asm__ volatile("" : "+v"(x));
}

// max(a, b, c) in one instruction.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace dev
}  // namespace bss
