// kv_cache_append: write new K/V rows into a paged cache, copying bf16 bits or quantizing to
// INT8 or FP8 E4M3 with a per-(token, KV head) fp16 scale.
//
// Paged placement follows "分页KV缓存：借鉴操作系统的内存管理" on the Tiny-Infer page
// ("从零构建CUDA推理引擎：Tiny-Infer项目的技术深度解析"): logical position -> (physical block
// from the table, slot inside the block). INT8 storage follows "推测性解码与INT8量化" there;
// FP8 E4M3 with a dynamic per-token scale follows "3.3 FP8量化支持" on the triton-fused-ops
// page. The scale rule (absmax / 127 or / 448, fp16, symmetric, ties-to-even) is this
// library's reading.
//
// With RoPE (kv_cache_append_rope, attn_rope_inplace) the K rows are rotated first: rotary
// position embedding applied where the rows already cross HBM, in the spirit of
// "3.1 RMSNorm + RoPE 融合" on the triton-fused-ops page ("Triton融合算子优化：LLM推理性能提升3倍
// 的工程实践"). The pages give no formula; this library takes the Llama convention: dimension
// i < D/2 pairs with i + D/2 and the pair turns by pos * base^(-2i/D). The frequencies come
// from an fp64 table built once per call on the host; the angle and its reduction modulo 2*pi are
// fp64 (positions reach tens of thousands of radians); sin, cos and the rotation are fp32,
// rounded to bf16 (RNE) when stored as bf16. Each (token, pair) angle is evaluated once per
// workgroup and shared by the token's heads through LDS.
//
// HBM-bound elementwise work: one thread moves 8 elements (16 B of bf16 input); the D / 8
// threads of one (token, head) row sit in adjacent lanes and reduce the row's absmax (and
// exchange RoPE partners) with cross-lane shuffles. Division is IEEE (correctly rounded) so
// codes match a CPU reference bit for bit.
#include "common.h"
#include "launch.h"
#include <hip/hip_fp16.h>
#include <cmath>

namespace attn {

// inv_freq[i] = base^(-2i/D), i < D/2: computed once on the host (fp64 pow) and passed by
// value, so no workgroup evaluates pow or waits for a table of its own.
struct RopeFreq {
  double f[64];
};

// The angle of a pair depends only on (position, pair index), so a workgroup computes each
// (token, pair) of its rows once: the (cos, sin) table of the tokens its rows cover,
// tokens t_a .. t_a + ntok - 1, one entry per thread (all threads take part), in LDS behind one
// barrier; every row of a token reads the token's table. Same arithmetic for every element as
// computing it in place.
template <int D>
__device__ __forceinline__ float2 rope_entry(int pos, int i, const RopeFreq& rf) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double ang = (double)pos * rf.f[i];
  const float r = (float)(ang - kTwoPi * rint(ang * (1.0 / kTwoPi)));  // in [-pi, pi]
  float sn, cs;
  sincosf(r, &sn, &cs);
  return make_float2(cs, sn);
}

template <int D, int ROWS>
__device__ __forceinline__ void rope_fill_all(float2 (*s_cs)[D / 2], int64_t t_a, int ntok,
                                              const int32_t* __restrict__ pos,
                                              const RopeFreq& rf) {
  for (int j = threadIdx.x; j < ntok * (D / 2); j += blockDim.x) {
    const int k = j / (D / 2), i = j % (D / 2);
    s_cs[k][i] = rope_entry<D>(pos[t_a + k], i, rf);
  }
  __syncthreads();
}

// Rotate the 8 values x (elements 8c .. 8c+7 of a D-wide row, c = lane's chunk) with the
// token's (cos, sin) table. The partner half of the row sits TPR/2 lanes away; every lane of
// the row must call.
template <int D>
__device__ __forceinline__ void rope8(float (&x)[8], int c, const float2* __restrict__ row_cs) {
  constexpr int TPR = D / 8;
  const bool lo_half = c < TPR / 2;
  const int i0 = (8 * c) % (D / 2);  // pairs i0 .. i0+7 (element d and d +- D/2 share one)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = __shfl_xor(x[e], TPR / 2, TPR);  // element d +- D/2
    const float2 t = row_cs[i0 + e];
    x[e] = lo_half ? fmaf(x[e], t.x, -y * t.y) : fmaf(y, t.y, x[e] * t.x);
  }
}

template <int D, int KV, bool ROPE>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ table, void* __restrict__ k_cache, void* __restrict__ v_cache,
    __half* __restrict__ k_scale, __half* __restrict__ v_scale, int64_t rows, int Hkv, int bs,
    int num_seqs, int max_blocks, int num_blocks, RopeFreq rf) {
  constexpr int TPR = D / 8;        // threads per (token, head) row
  constexpr int ROWS = 256 / TPR;   // rows per workgroup
  __shared__ float2 s_cs[ROPE ? ROWS : 1][ROPE ? D / 2 : 1];
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / TPR;
  const int c = (int)(gid % TPR);
  const bool in_range = row < rows;
  const int64_t r = in_range ? row : 0;
  const int64_t t = r / Hkv;
  const int g = (int)(r % Hkv);

  bool valid = in_range;
  int pb = 0, slot = 0;
  if (valid) {
    const int b = seq_idx[t], p = pos[t];
    valid = b >= 0 && b < num_seqs && p >= 0 && p < max_blocks * bs;
    if (valid) {
      pb = table[(int64_t)b * max_blocks + p / bs];
      slot = p % bs;
      valid = pb >= 0 && pb < num_blocks;
    }
  }
  const int64_t src = r * D + c * 8;
  const int64_t dst = pool_offset(pb, Hkv, g, bs, slot, D) + c * 8;
  u32x4 win[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  if (in_range) {
    win[0] = *reinterpret_cast<const u32x4*>(k_new + src);
    win[1] = *reinterpret_cast<const u32x4*>(v_new + src);
  }
  int cs_row = 0;  // this row's token's table
  if constexpr (ROPE) {
    const int64_t r0 = (int64_t)blockIdx.x * ROWS;
    const int64_t t_a = r0 / Hkv, t_b = (min(r0 + ROWS, rows) - 1) / Hkv;
    cs_row = in_range ? (int)(t - t_a) : 0;  // rows past the end read entry 0, store nothing
    rope_fill_all<D, ROWS>(s_cs, t_a, (int)(t_b - t_a + 1), pos, rf);
  }

#pragma unroll
  for (int which = 0; which < 2; ++which) {
    u32x4 w = win[which];
    const bool rot = ROPE && which == 0;  // RoPE turns K only
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
    if (rot) rope8<D>(x, c, s_cs[cs_row]);
    if constexpr (KV == kKvBf16) {
      uint16_t* out = reinterpret_cast<uint16_t*>(which == 0 ? k_cache : v_cache);
      if (rot) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
      }
      if (valid) *reinterpret_cast<u32x4*>(out + dst) = w;
    } else {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
      for (int m = 1; m < TPR; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, TPR));
      constexpr float kMaxCode = KV == kKvI8 ? 127.0f : 448.0f;  // INT8 / FP8 E4M3 largest
      const float s32 = __fdiv_rn(a, kMaxCode);
      const __half s16 = __float2half_rn(s32);
      const float sf = __half2float(s16);
      uint32_t packed[2] = {0u, 0u};
      if constexpr (KV == kKvI8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int code = 0;
          if (sf != 0.0f) {
            float qv = rintf(__fdiv_rn(x[i], sf));
            qv = fminf(fmaxf(qv, -127.0f), 127.0f);
            code = (int)qv;
          }
          packed[i / 4] |= ((uint32_t)code & 0xffu) << (8 * (i % 4));
        }
      } else if (sf != 0.0f) {
        // E4M3 of the clamped quotient, round to nearest even, by the hardware conversion
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float y0 = fminf(fmaxf(__fdiv_rn(x[i], sf), -448.0f), 448.0f);
          const float y1 = fminf(fmaxf(__fdiv_rn(x[i + 1], sf), -448.0f), 448.0f);
          const uint32_t two = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false) & 0xffffu;
          packed[i / 4] |= two << (8 * (i % 4));
        }
      }
      uint8_t* out = reinterpret_cast<uint8_t*>(which == 0 ? k_cache : v_cache);
      __half* sc = which == 0 ? k_scale : v_scale;
      if (valid) {
        u32x2 pk = {packed[0], packed[1]};
        *reinterpret_cast<u32x2*>(out + dst) = pk;
        if (c == 0) sc[((int64_t)pb * Hkv + g) * bs + slot] = s16;
      }
    }
  }
}

// In-place RoPE of bf16 rows x [T][H][D] at positions pos[T] (the query side of the fused
// append: Q is turned by the same rule before attention).
template <int D>
__global__ __launch_bounds__(256) void rope_rows_kernel(uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ pos,
                                                        int64_t rows, int H, RopeFreq rf) {
  constexpr int TPR = D / 8;
  constexpr int ROWS = 256 / TPR;
  __shared__ float2 s_cs[ROWS][D / 2];
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / TPR;
  const int c = (int)(gid % TPR);
  const bool in_range = row < rows;
  const int64_t r = in_range ? row : 0;
  u32x4 w = {0u, 0u, 0u, 0u};
  uint16_t* p = x + r * D + 8 * c;
  if (in_range) w = *reinterpret_cast<const u32x4*>(p);
  const int64_t t = r / H, r0 = (int64_t)blockIdx.x * ROWS;
  const int64_t t_a = r0 / H, t_b = (min(r0 + ROWS, rows) - 1) / H;
  const int cs_row = in_range ? (int)(t - t_a) : 0;  // rows past the end store nothing
  rope_fill_all<D, ROWS>(s_cs, t_a, (int)(t_b - t_a + 1), pos, rf);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
  rope8<D>(v, c, s_cs[cs_row]);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  if (in_range) *reinterpret_cast<u32x4*>(p) = w;
}

static RopeFreq rope_freq(int D, double base) {
  RopeFreq rf{};
  for (int i = 0; i < D / 2 && i < 64; ++i) rf.f[i] = std::pow(base, -2.0 * i / D);
  return rf;
}

template <bool ROPE>
static int launch_append(const AppendArgs& a, double rope_base, hipStream_t stream) {
  const RopeFreq rf = ROPE ? rope_freq(a.D, rope_base) : RopeFreq{};
  const int64_t rows = (int64_t)a.T * a.Hkv;
  const int tpr = a.D / 8;
  const int64_t threads = rows * tpr;
  const int block = 256;
  const int64_t grid = (threads + block - 1) / block;
  if (grid == 0) return 0;
#define ATTN_APPEND(DD, KV)                                                                    \
  hipLaunchKernelGGL((kv_append_kernel<DD, KV, ROPE>), dim3((unsigned)grid), dim3(block),       \
                     0, stream, (const uint16_t*)a.k_new, (const uint16_t*)a.v_new, a.seq_idx,  \
                     a.pos, a.block_table, a.k_cache, a.v_cache, (__half*)a.k_scale,            \
                     (__half*)a.v_scale, rows, a.Hkv, a.block_size, a.num_seqs,                 \
                     a.max_blocks_per_seq, a.num_blocks, rf)
  if (a.D == 64) {
    if (a.kv == kKvI8) ATTN_APPEND(64, kKvI8); else if (a.kv == kKvFp8) ATTN_APPEND(64, kKvFp8); else ATTN_APPEND(64, kKvBf16);
  } else {
    if (a.kv == kKvI8) ATTN_APPEND(128, kKvI8); else if (a.kv == kKvFp8) ATTN_APPEND(128, kKvFp8); else ATTN_APPEND(128, kKvBf16);
  }
#undef ATTN_APPEND
  return 0;
}

int launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  return launch_append<false>(a, 0.0, stream);
}

int launch_kv_append_rope(const AppendArgs& a, double rope_base, hipStream_t stream) {
  return launch_append<true>(a, rope_base, stream);
}

int launch_rope_rows(void* x, const int32_t* pos, int T, int H, int D, double rope_base,
                     hipStream_t stream) {
  const int64_t rows = (int64_t)T * H;
  const int64_t grid = (rows * (D / 8) + 255) / 256;
  if (grid == 0) return 0;
  const RopeFreq rf = rope_freq(D, rope_base);
  if (D == 64)
    hipLaunchKernelGGL(rope_rows_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (uint16_t*)x, pos, rows, H, rf);
  else
    hipLaunchKernelGGL(rope_rows_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (uint16_t*)x, pos, rows, H, rf);
  return 0;
}

}  // namespace attn
