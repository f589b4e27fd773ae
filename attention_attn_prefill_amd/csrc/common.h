// Device-side helpers shared by the attention kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for -inf as a running maximum: exp2(x - kNegBig) never sees (-inf) - (-inf).
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) void lds_void;

// One global_load_lds_dwordx4: each lane copies 16 bytes from `g` to LDS byte address
// lds_off + 16 * lane. Written as asm so the compiler does not treat every later LDS read as
// a possible alias of the in-flight copy (it would wait for the copy before unrelated LDS
// reads); the caller awaits completion explicitly (vmcnt) before reading the data. The
// instruction writes no registers. An LDS DMA that follows a scalar write of M0 needs one
// wait state on this chip family (the compiler puts an s_nop there in its own code, but it
// does not look inside asm): without it the copy can take the previous M0 and land at
// another LDS address.
__device__ __forceinline__ void lds_dma_16(const void* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_off), "v"(g)
               : "memory", "m0");
}

// As lds_dma_16 with the address split into a wave-uniform 64-bit base (SGPRs) and a 32-bit
// per-lane byte offset: a tile loop then advances the base with scalar arithmetic and keeps
// the offsets fixed, instead of recomputing 64-bit lane addresses with vector instructions.
__device__ __forceinline__ void lds_dma_16s(const void* sbase, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}

// As lds_dma_16 with one dword per lane: LDS byte address lds_off + 4 * lane.
__device__ __forceinline__ void lds_dma_4(const void* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_off), "v"(g)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// 64-bit element offset of (block, head, slot, 0) in a [num_blocks][Hkv][bs][D] pool.
__device__ __forceinline__ int64_t pool_offset(int pb, int Hkv, int g, int bs, int slot, int D) {
  return (((int64_t)pb * Hkv + g) * bs + slot) * (int64_t)D;
}

}  // namespace attn
