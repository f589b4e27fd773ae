// Paged-KV single-token decode attention with the KV axis split across workgroups and a
// log-sum-exp merge of the partial results.
//
// Pages (title, section): the Tiny-Infer page ("从零构建CUDA推理引擎：Tiny-Infer项目的技术深度解析")
// -- "分页KV缓存：借鉴操作系统的内存管理" (fixed-size blocks, table from logical position to
// physical block), "技术架构与模块设计" (incremental decode against the cache), "推测性解码与INT8量化"
// (INT8 cache); the inference-lab page ("从零开始的LLM推理优化实验室：从PyTorch基线到Triton内核的完整实践")
// -- "KV缓存实验与长上下文优化" (sliding window); the triton-fused-ops page
// ("Triton融合算子优化：LLM推理性能提升3倍的工程实践") -- "一、LLM推理的算子瓶颈" (decode is bound by
// reading the KV cache from memory).
//
// Design (gfx950): one workgroup of 4 waves per (split, KV head g, sequence b). A split is a
// run of `C` consecutive logical tokens, block aligned. All G = Hq/Hkv query heads of g are
// served by the same workgroup, so every K/V byte is read from HBM once.
//   pass 1  QK^T on MFMA 16x16x32: A = 16 tokens of a K block (natural [token][d] rows),
//           B = Q^T of the G heads (padded to 16 columns). Scores (log2 units) go to LDS.
//   pass 2  per-head max and exp2 over the split's scores in LDS; row sums.
//   pass 3  PV on the VALU: each lane owns 8 consecutive d of one token, multiplies by the G
//           probabilities and accumulates; lanes are then reduced.
//   final   o = acc / l  (single split: bf16 output directly)  or a partial (o, lse) in fp32
//           workspace, merged by decode_merge_kernel.
#include "common.h"
#include "launch.h"
#include <hip/hip_fp16.h>
#include <algorithm>
#include <type_traits>

namespace attn {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = 4;
constexpr int kScoreFloats = 4096;  // LDS score buffer: G * split_tokens <= 4096

__device__ __forceinline__ int decode_ctx(const int32_t* ctx_lens, int b, int max_ctx,
                                          int max_blocks, int bs) {
  int c = ctx_lens[b];
  int cap = min(max_ctx, max_blocks * bs);
  return c < 0 ? 0 : (c > cap ? cap : c);
}

template <int D, int GP, bool I8>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const __half* __restrict__ k_scale,
    const __half* __restrict__ v_scale, const int32_t* __restrict__ table,
    const int32_t* __restrict__ ctx_lens, uint16_t* __restrict__ out,
    float* __restrict__ part_o, float* __restrict__ part_lse, int Hq, int Hkv, int G,
    int max_blocks, int num_blocks, int max_ctx, float scale_log2, int window, int C,
    int n_split) {
  constexpr int BS = 16;
  __shared__ float s_scores[kScoreFloats];
  __shared__ float s_red[kDecodeWaves][GP][D];
  __shared__ float s_m[GP], s_l[GP];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  const int ctx = decode_ctx(ctx_lens, b, max_ctx, max_blocks, BS);
  const int lo = window > 0 ? max(0, ctx - window) : 0;
  const int base = lo & ~(BS - 1);
  const int t_begin = base + split * C;
  if (ctx <= 0) {
    // Empty context: the output is defined as zero. Split 0 writes it (merge sees n_valid=0).
    if (split == 0 && n_split == 1) {
      for (int i = threadIdx.x; i < G * D; i += kDecodeThreads)
        out[((int64_t)b * Hq + g * G) * D + i] = 0;
    }
    return;
  }
  if (t_begin >= ctx) return;
  const int t_end = min(t_begin + C, ctx);
  const int nblk = (t_end - t_begin + BS - 1) / BS;
  const int lb0 = t_begin / BS;
  const int32_t* trow = table + (int64_t)b * max_blocks;

  // ---- pass 1: scores on MFMA -------------------------------------------------------------
  const int hq = lane & 15;    // MFMA column = query head within the group
  const int grp = lane >> 4;   // 0..3
  {
    constexpr int KSTEPS = D / 32;
    typedef typename std::conditional<I8, f16x8, bf16x8>::type frag_t;
    frag_t qf[KSTEPS];
    const uint16_t* qrow = q + ((int64_t)b * Hq + g * G + hq) * D;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      // k-step j covers d = 32j + 8*grp + e for bf16; for int8, the d set of step j is
      // 64*(j/2) + 16*grp + 8*(j%2) + e (one 16-byte load feeds two steps).
      const int d0 = I8 ? (64 * (j / 2) + 16 * grp + 8 * (j % 2)) : (32 * j + 8 * grp);
      u32x4 w = {0u, 0u, 0u, 0u};
      if (hq < G) w = *reinterpret_cast<const u32x4*>(qrow + d0);
      if constexpr (I8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[j][2 * e] = (_Float16)bf16_lo(w[e]);
          qf[j][2 * e + 1] = (_Float16)bf16_hi(w[e]);
        }
      } else {
        qf[j] = __builtin_bit_cast(bf16x8, w);
      }
    }

    for (int blk = wave; blk < nblk; blk += kDecodeWaves) {
      const int pb = trow[lb0 + blk];
      const bool ok = pb >= 0 && pb < num_blocks;
      const int tok = 4 * grp;  // first of this lane's 4 accumulator rows
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      float ksc[4] = {1.f, 1.f, 1.f, 1.f};
      if (ok) {
        const int64_t row = pool_offset(pb, Hkv, g, BS, lane & 15, D);
        if constexpr (I8) {
          const int8_t* kc = reinterpret_cast<const int8_t*>(k_cache) + row;
#pragma unroll
          for (int jj = 0; jj < D / 64; ++jj) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(kc + 64 * jj + 16 * grp);
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
              f16x8 a;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t word = w[2 * sub + e / 4];
                a[e] = (_Float16)(int)(int8_t)(word >> (8 * (e % 4)));
              }
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[2 * jj + sub], acc, 0, 0, 0);
            }
          }
          const __half* ks = k_scale + ((int64_t)pb * Hkv + g) * BS + tok;
#pragma unroll
          for (int i = 0; i < 4; ++i) ksc[i] = __half2float(ks[i]);
        } else {
          const uint16_t* kc = reinterpret_cast<const uint16_t*>(k_cache) + row;
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(kc + 32 * j + 8 * grp);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), qf[j],
                                                          acc, 0, 0, 0);
          }
        }
      }
      if (hq < G) {
        f32x4 s;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t_begin + blk * BS + tok + i;
          const bool vis = ok && t >= lo && t < t_end;
          s[i] = vis ? acc[i] * ksc[i] * scale_log2 : -INFINITY;
        }
        *reinterpret_cast<f32x4*>(&s_scores[hq * C + blk * BS + tok]) = s;
      }
    }
  }
  __syncthreads();

  // ---- pass 2: per-head max, probabilities, sums -----------------------------------------
  const int ntok = nblk * BS;
  for (int h = wave; h < G; h += kDecodeWaves) {
    float m = kNegBig;
    for (int i = lane; i < ntok; i += 64) m = fmaxf(m, s_scores[h * C + i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float l = 0.f;
    for (int i = lane; i < ntok; i += 64) {
      const float p = fast_exp2(s_scores[h * C + i] - m);
      s_scores[h * C + i] = p;
      l += p;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) {
      s_m[h] = m;
      s_l[h] = l;
    }
  }
  __syncthreads();

  // ---- pass 3: PV on the VALU ------------------------------------------------------------
  constexpr int CPR = D / 8;      // lanes per token row (8 elements each)
  constexpr int TPW = 64 / CPR;   // tokens per wave step
  const int c = lane % CPR, ts = lane / CPR;
  float acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  for (int blk = wave; blk < nblk; blk += kDecodeWaves) {
    const int pb = trow[lb0 + blk];
    if (!(pb >= 0 && pb < num_blocks)) continue;
#pragma unroll
    for (int tt = 0; tt < BS; tt += TPW) {
      const int slot = tt + ts;
      const int tpos = t_begin + blk * BS + slot;
      if (tpos < lo || tpos >= t_end) continue;  // masked slot: may hold anything (even NaN)
      const int64_t off = pool_offset(pb, Hkv, g, BS, slot, D) + 8 * c;
      float x[8];
      float vsc = 1.f;
      if constexpr (I8) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(
            reinterpret_cast<const int8_t*>(v_cache) + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)(int8_t)(w[e / 4] >> (8 * (e % 4)));
        vsc = __half2float(v_scale[((int64_t)pb * Hkv + g) * BS + slot]);
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const uint16_t*>(v_cache) + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_lo(w[e]);
          x[2 * e + 1] = bf16_hi(w[e]);
        }
      }
      const int li = blk * BS + slot;
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (h < G) {
          const float p = s_scores[h * C + li] * vsc;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, x[e], acc[h][e]);
        }
      }
    }
  }
  // reduce over the token slots of the wave (lanes with equal c)
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o);
  if (ts == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_red[wave][h][8 * c + e] = acc[h][e];
  }
  __syncthreads();

  for (int i = threadIdx.x; i < G * D; i += kDecodeThreads) {
    const int h = i / D, d = i % D;
    const float sum = s_red[0][h][d] + s_red[1][h][d] + s_red[2][h][d] + s_red[3][h][d];
    const float inv = 1.0f / s_l[h];
    const int head = g * G + h;
    if (n_split == 1) {
      out[((int64_t)b * Hq + head) * D + d] = (uint16_t)f32_to_bf16_bits(sum * inv);
    } else {
      const int64_t pi = ((int64_t)b * Hq + head) * n_split + split;
      part_o[pi * D + d] = sum * inv;
      if (d == 0) part_lse[pi] = s_m[h] + __log2f(s_l[h]);
    }
  }
}

// Merge the partials of one (sequence, query head): weights exp2(lse_s - max lse).
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ ctx_lens, uint16_t* __restrict__ out, int Hq, int max_blocks,
    int max_ctx, int window, int C, int n_split) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int ctx = decode_ctx(ctx_lens, b, max_ctx, max_blocks, 16);
  const int lo = window > 0 ? max(0, ctx - window) : 0;
  const int base = lo & ~15;
  const int n_valid = ctx > 0 ? min(n_split, (ctx - base + C - 1) / C) : 0;
  const int64_t pi = ((int64_t)b * Hq + h) * n_split;
  float M = -INFINITY;
  for (int s = 0; s < n_valid; ++s) M = fmaxf(M, part_lse[pi + s]);
  constexpr int EPT = D / 64;
  float acc[EPT] = {};
  float L = 0.f;
  for (int s = 0; s < n_valid; ++s) {
    const float w = fast_exp2(part_lse[pi + s] - M);
    L += w;
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = fmaf(w, part_o[(pi + s) * D + threadIdx.x + 64 * e], acc[e]);
  }
  const float inv = n_valid > 0 ? 1.0f / L : 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    out[((int64_t)b * Hq + h) * D + threadIdx.x + 64 * e] = (uint16_t)f32_to_bf16_bits(acc[e] * inv);
}

static int pow2_at_least(int g) {
  int p = 1;
  while (p < g) p <<= 1;
  return p;
}

DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int max_context_len, int window,
                       int split_tokens) {
  (void)D;
  DecodePlan p{};
  const int G = Hq / Hkv;
  const int GP = pow2_at_least(G);
  const int cap = (kScoreFloats / GP) & ~15;
  const int span = window > 0 ? std::min(max_context_len, window + 15) : max_context_len;
  int C = split_tokens;
  if (C == 0) {
    // Aim for about 8 workgroups per CU over the whole grid, splits of 128..cap tokens.
    const long long target = 2048;
    long long want = ((long long)B * Hkv * span + target - 1) / target;
    want = (want + 15) & ~15LL;
    C = (int)std::max<long long>(128, std::min<long long>(want, cap));
  }
  p.split_tokens = C;
  p.n_split = (span + C - 1) / C;
  if (p.n_split < 1) p.n_split = 1;
  if (p.n_split == 1) {
    p.workspace_bytes = 0;
  } else {
    const size_t parts = (size_t)B * Hq * p.n_split;
    const size_t o_bytes = parts * D * sizeof(float);
    const size_t lse_off = (o_bytes + 255) & ~(size_t)255;
    p.workspace_bytes = lse_off + parts * sizeof(float);
  }
  return p;
}

int launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int GP = pow2_at_least(G);
  const int C = a.plan.split_tokens, ns = a.plan.n_split;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (ns > 1) {
    const size_t parts = (size_t)a.B * a.Hq * ns;
    const size_t lse_off = (parts * a.D * sizeof(float) + 255) & ~(size_t)255;
    part_o = reinterpret_cast<float*>(a.workspace);
    part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + lse_off);
  }
  const float scale_log2 = a.scale * kLog2e;
  dim3 grid(ns, a.Hkv, a.B);
#define ATTN_DSPLIT(DD, GG, I8)                                                                 \
  hipLaunchKernelGGL((decode_split_kernel<DD, GG, I8>), grid, dim3(kDecodeThreads), 0, stream, \
                     (const uint16_t*)a.q, a.k_cache, a.v_cache, (const __half*)a.k_scale,      \
                     (const __half*)a.v_scale, a.block_table, a.context_lens, (uint16_t*)a.o,   \
                     part_o, part_lse, a.Hq, a.Hkv, G, a.max_blocks_per_seq, a.num_blocks,      \
                     a.max_context_len, scale_log2, a.window, C, ns)
#define ATTN_DSPLIT_G(DD, I8)                 \
  switch (GP) {                               \
    case 1: ATTN_DSPLIT(DD, 1, I8); break;    \
    case 2: ATTN_DSPLIT(DD, 2, I8); break;    \
    case 4: ATTN_DSPLIT(DD, 4, I8); break;    \
    case 8: ATTN_DSPLIT(DD, 8, I8); break;    \
    default: ATTN_DSPLIT(DD, 16, I8); break;  \
  }
  if (a.D == 64) {
    if (a.int8) { ATTN_DSPLIT_G(64, true) } else { ATTN_DSPLIT_G(64, false) }
  } else {
    if (a.int8) { ATTN_DSPLIT_G(128, true) } else { ATTN_DSPLIT_G(128, false) }
  }
#undef ATTN_DSPLIT_G
#undef ATTN_DSPLIT
  if (ns > 1) {
    dim3 mgrid(a.Hq, a.B);
    if (a.D == 64)
      hipLaunchKernelGGL(decode_merge_kernel<64>, mgrid, dim3(64), 0, stream, part_o, part_lse,
                         a.context_lens, (uint16_t*)a.o, a.Hq, a.max_blocks_per_seq,
                         a.max_context_len, a.window, C, ns);
    else
      hipLaunchKernelGGL(decode_merge_kernel<128>, mgrid, dim3(64), 0, stream, part_o, part_lse,
                         a.context_lens, (uint16_t*)a.o, a.Hq, a.max_blocks_per_seq,
                         a.max_context_len, a.window, C, ns);
  }
  return 0;
}

}  // namespace attn
