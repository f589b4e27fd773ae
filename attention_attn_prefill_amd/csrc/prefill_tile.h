// Tile geometry and small helpers shared by the bf16 prefill kernels (gfx950, wave64).
#pragma once
#include "common.h"

namespace attn {

constexpr int kPrefillThreads = 256;
// keys per tile: 64 at D=64; 32 at D=128, which halves the LDS and score registers per
// workgroup so that three waves fit on a SIMD
template <int D>
constexpr int kTileKeys = D == 128 ? 32 : 64;
// The running max lags the true max by at most this much (log2 units), so probabilities stay
// below 2^kRescaleSlack; O and l share the same reference, so o = O / l is unchanged.
constexpr float kRescaleSlack = 8.0f;

__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// max / sum over lanes l and l ^ 32 (the two halves of a 32x32 accumulator column). The max is
// one v_max_f32 written out: fmaxf would first quiet both inputs (the exchanged value is not
// known to be canonical), two more instructions; scores are never NaN.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short i16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct PTile {
  static constexpr int ROWB = D * 2;                 // bytes of one K or V row
  static constexpr int CHUNKS = ROWB / 16;           // 16-byte chunks per row
  static constexpr int BN = kTileKeys<D>;            // keys per tile
  static constexpr int TILE = BN * ROWB;             // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * TILE;             // K tile then V tile
  static constexpr int INSTR = TILE / 1024;          // wave load instructions per tile
  static constexpr int PER_WAVE = INSTR / 4;         // ... per wave
  static constexpr int ROWS_PER_INSTR = 1024 / ROWB;
};

// Chunk swizzles (c = 16-byte chunk index inside a row). K: the 16 lanes of a ds_read_b128 pass
// read one chunk of 16 consecutive keys; V: a ds_read_b64_tr_b16 pass reads 64 bytes of 4
// consecutive keys. Both land on distinct 4-bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Query heads per workgroup (the waves of one workgroup share a KV head) and query-row chunks
// per head, for G = Hq / Hkv query heads per KV head.
inline void prefill_split(int Hq, int Hkv, int& HW, int& QW) {
  const int G = Hq / Hkv;
  HW = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  QW = 4 / HW;
}

}  // namespace attn
