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
// Each wave walks the split in chunks of U blocks; for a chunk it
//   * issues the table lookups and every K and V load of the chunk at once (deep memory-level
//     parallelism: 16-32 KB in flight per wave),
//   * computes QK^T on MFMA 16x16x32: A = 16 tokens of a K block in their natural [token][d]
//     rows, B = Q^T of the G heads (padded to 16 columns); for INT8 the codes are widened to
//     fp16 (exact) and the per-token scale is applied to the fp32 score,
//   * runs the online softmax per head in the log2 domain, moving the running max (and
//     rescaling the accumulators) only when it grows by more than 8,
//   * hands the probabilities to the PV lanes through a small per-wave LDS slice and does PV on
//     the VALU, each lane owning 8 consecutive d of one token (coalesced V rows); the INT8 V
//     scale is folded into the probability.
// The 4 waves' (m, l, acc) are merged by log-sum-exp in LDS; the workgroup then writes the
// bf16 output (single split) or an fp32 partial (o, lse) merged by decode_merge_kernel.
#include "common.h"
#include "launch.h"
#include <hip/hip_fp16.h>
#include <algorithm>
#include <type_traits>

namespace attn {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = 4;
constexpr int kMaxSplitBlocks = kMaxSplitTokens / 16;  // the table slice is kept in LDS

__device__ __forceinline__ int decode_ctx(const int32_t* ctx_lens, int b, int max_ctx,
                                          int max_blocks, int bs) {
  int c = ctx_lens[b];
  int cap = min(max_ctx, max_blocks * bs);
  return c < 0 ? 0 : (c > cap ? cap : c);
}

// K/V cache reads are streamed once per call: non-temporal loads keep them from displacing
// reusable lines (the table slice, Q) and measured faster on MI355X for pure streaming.
template <typename V>
__device__ __forceinline__ V ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
}

// INT8 -> fp16 widening without conversions: with u = x ^ 0x80 (= x + 128 as a byte), the
// fp16 bit pattern 0x64uu is exactly 1024 + u = 1152 + x. One v_perm builds two such halves
// from a dword of codes (the 0x64 bytes come from the constant operand).
__device__ __forceinline__ uint32_t widen_lo(uint32_t u) { return __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u); }
__device__ __forceinline__ uint32_t widen_hi(uint32_t u) { return __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u); }
constexpr float kI8Bias = 1152.0f;

// xor-16 / xor-32 lane partners within a wave
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Chunks of U blocks (U*16 tokens, 8 KB of K+V for the bf16 D=128 and INT8 caches, 8 KB for
// bf16 D=64) are the unit of work of one wave: their K and V loads are all issued before any of
// them is consumed. Small chunks keep register use low, so more waves stay resident and more
// bytes are in flight per CU (measured better than larger per-wave batches).
template <int D, bool I8>
struct DecodeShape {
  static constexpr int BS = 16;
  static constexpr int U = (D == 64 || I8) ? 2 : 1;       // blocks per chunk
  static constexpr int KSTEPS = D / 32;                    // MFMA k-steps per block
  static constexpr int KLOADS = I8 ? D / 64 : D / 32;      // 16-byte K loads per lane per block
  static constexpr int VBYTES = I8 ? 8 : 16;               // bytes per lane per V load (8 elements)
  static constexpr int CPR = D / 8;                        // lanes per V row
  static constexpr int TPW = 64 / CPR;                     // tokens per V load instruction
  static constexpr int VLOADS = BS / TPW;                  // V loads per lane per block
};

template <int D, int GP, bool I8>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const __half* __restrict__ k_scale,
    const __half* __restrict__ v_scale, const int32_t* __restrict__ table,
    const int32_t* __restrict__ ctx_lens, uint16_t* __restrict__ out,
    float* __restrict__ part_o, float* __restrict__ part_lse, int Hq, int Hkv, int G,
    int max_blocks, int num_blocks, int max_ctx, float scale_log2, int window, int C,
    int n_split) {
  using SH = DecodeShape<D, I8>;
  constexpr int BS = SH::BS, U = SH::U, CT = U * BS;  // CT tokens per chunk
  // probabilities handed from the MFMA lanes to the PV lanes: fp32 [token][head] for bf16;
  // for INT8, fp16 pairs (token t, token t + 8) of p' = p * v_scale, [block][pair][head]
  __shared__ float s_p[kDecodeWaves][I8 ? 1 : CT][GP];
  __shared__ uint32_t s_pp[kDecodeWaves][I8 ? U : 1][8][GP];
  __shared__ float s_alpha[kDecodeWaves][GP];
  __shared__ float s_red[kDecodeWaves][GP][D];
  __shared__ float s_ml[kDecodeWaves][3][GP];
  __shared__ int s_pb[kMaxSplitBlocks];  // the split's slice of the block table

  // Grid (Hkv, B, n_split) with the split index slowest and reversed: consecutive workgroups
  // (dispatched round-robin over the XCDs) then belong to different sequences, so the XCDs
  // share ragged work evenly; splits that exist only for long contexts go first.
  const int split = n_split - 1 - blockIdx.z, g = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int ctx = decode_ctx(ctx_lens, b, max_ctx, max_blocks, BS);
  const int lo = window > 0 ? max(0, ctx - window) : 0;
  const int base = lo & ~(BS - 1);
  const int t_begin = base + split * C;
  if (ctx <= 0) {
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
  {
    const int32_t* trow = table + (int64_t)b * max_blocks + lb0;
    for (int i = threadIdx.x; i < nblk; i += kDecodeThreads) {
      const int e = trow[i];
      s_pb[i] = (e >= 0 && e < num_blocks) ? e : -1;  // -1: entry unusable, tokens skipped
    }
  }
  __syncthreads();

  // MFMA (QK^T) lane roles: column = query head, rows = 4 tokens of the block
  const int hq = lane & 15, grp = lane >> 4;
  // PV lane roles: 8 consecutive d of one token (bf16) or of a token pair (INT8)
  const int c8 = lane % SH::CPR, ts = lane / SH::CPR;

  typedef typename std::conditional<I8, f16x8, bf16x8>::type frag_t;
  frag_t qf[SH::KSTEPS];
  float qsum = 0.f;  // INT8: sum of this head's fp16 q values (the widened codes carry +1152)
  {
    const uint16_t* qrow = q + ((int64_t)b * Hq + g * G + hq) * D;
#pragma unroll
    for (int j = 0; j < SH::KSTEPS; ++j) {
      // bf16: step j covers d = 32j + 8*grp + e; INT8: one 16-byte load feeds steps 2jj,
      // 2jj+1 covering d = 64*jj + 16*grp + 8*sub + e.
      const int d0 = I8 ? (64 * (j / 2) + 16 * grp + 8 * (j % 2)) : (32 * j + 8 * grp);
      u32x4 w = {0u, 0u, 0u, 0u};
      if (hq < G) w = *reinterpret_cast<const u32x4*>(qrow + d0);
      if constexpr (I8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[j][2 * e] = (_Float16)bf16_lo(w[e]);
          qf[j][2 * e + 1] = (_Float16)bf16_hi(w[e]);
          qsum += (float)qf[j][2 * e] + (float)qf[j][2 * e + 1];
        }
      } else {
        qf[j] = __builtin_bit_cast(bf16x8, w);
      }
    }
    if constexpr (I8) {
      qsum += __shfl_xor(qsum, 16);
      qsum = sum_x32(qsum);
    }
  }
  const float bias = kI8Bias * qsum;

  float m_run = kNegBig;  // per head (lanes hq), log2 units
  float l_part = 0.f;     // this lane's share of the row sum
  float ps_part = 0.f;    // INT8: this lane's share of sum(p'), in the fp16 values used
  float acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  const int nchunk = (nblk + U - 1) / U;
  for (int ch = wave; ch < nchunk; ch += kDecodeWaves) {
    const int blk0 = ch * U;
    int pb[U];
    bool okb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = blk0 + u;
      pb[u] = __builtin_amdgcn_readfirstlane(blk < nblk ? s_pb[blk] : -1);
      okb[u] = pb[u] >= 0;
      if (!okb[u]) pb[u] = 0;
    }
    // ---- issue every load of the chunk -------------------------------------------------
    u32x4 kw[U][SH::KLOADS];
    typedef typename std::conditional<I8, u32x2, u32x4>::type vword_t;
    vword_t vw[U][SH::VLOADS];
    float ksc[U][4], vsc[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t brow = pool_offset(pb[u], Hkv, g, BS, 0, D);
      if constexpr (I8) {
        const int8_t* kc = reinterpret_cast<const int8_t*>(k_cache) + brow + (int64_t)hq * D;
#pragma unroll
        for (int jj = 0; jj < SH::KLOADS; ++jj)
          kw[u][jj] = ld_stream<u32x4>(kc + 64 * jj + 16 * grp);
        const int8_t* vc = reinterpret_cast<const int8_t*>(v_cache) + brow;
#pragma unroll
        for (int i = 0; i < SH::VLOADS; ++i)
          vw[u][i] = ld_stream<u32x2>(vc + (int64_t)(i * SH::TPW + ts) * D + 8 * c8);
        const int64_t srow = ((int64_t)pb[u] * Hkv + g) * BS + 4 * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ksc[u][i] = __half2float(k_scale[srow + i]);
          vsc[u][i] = __half2float(v_scale[srow + i]);
        }
      } else {
        const uint16_t* kc = reinterpret_cast<const uint16_t*>(k_cache) + brow + (int64_t)hq * D;
#pragma unroll
        for (int j = 0; j < SH::KLOADS; ++j)
          kw[u][j] = ld_stream<u32x4>(kc + 32 * j + 8 * grp);
        const uint16_t* vc = reinterpret_cast<const uint16_t*>(v_cache) + brow;
#pragma unroll
        for (int i = 0; i < SH::VLOADS; ++i)
          vw[u][i] = ld_stream<u32x4>(vc + (int64_t)(i * SH::TPW + ts) * D + 8 * c8);
      }
    }
    // ---- scores on MFMA ---------------------------------------------------------------
    float sc[U][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (I8) {
#pragma unroll
        for (int jj = 0; jj < SH::KLOADS; ++jj)
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const uint32_t w0 = kw[u][jj][2 * sub] ^ 0x80808080u;
            const uint32_t w1 = kw[u][jj][2 * sub + 1] ^ 0x80808080u;
            const u32x4 hv = {widen_lo(w0), widen_hi(w0), widen_lo(w1), widen_hi(w1)};
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, hv),
                                                        qf[2 * jj + sub], a4, 0, 0, 0);
          }
      } else {
#pragma unroll
        for (int j = 0; j < SH::KSTEPS; ++j)
          a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw[u][j]), qf[j], a4, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t_begin + (blk0 + u) * BS + 4 * grp + i;
        const bool vis = okb[u] && t >= lo && t < t_end;
        float s;
        if constexpr (I8)
          s = (a4[i] - bias) * ksc[u][i] * scale_log2;
        else
          s = a4[i] * scale_log2;
        sc[u][i] = vis ? s : -INFINITY;
        cmax = fmaxf(cmax, sc[u][i]);
      }
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = max_x32(cmax);
    // lazy rescale: move the running max only when it grows by more than 8 (log2 units)
    if (__builtin_amdgcn_ballot_w64(cmax > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
      ps_part *= alpha;
      if (grp == 0 && hq < GP) s_alpha[wave][hq] = alpha;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float al = s_alpha[wave][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al;
      }
    }
    // probabilities -> LDS
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(sc[u][i] - m_run);
        l_part += p;
        if constexpr (I8) {
          // masked tokens: p = 0 exactly, and their (possibly NaN) scale is not used
          const _Float16 pv16 = (_Float16)(sc[u][i] == -INFINITY ? 0.f : p * vsc[u][i]);
          ps_part += (float)pv16;
          const int t = 4 * grp + i;  // token inside block u: pair t & 7, element t >> 3
          if (hq < GP)
            reinterpret_cast<_Float16*>(&s_pp[wave][u][t & 7][hq])[t >> 3] = pv16;
        } else {
          if (hq < GP) s_p[wave][u * BS + 4 * grp + i][hq] = p;
        }
      }
    __builtin_amdgcn_wave_barrier();
    // ---- PV on the VALU -----------------------------------------------------------------
    if constexpr (I8) {
      // lane (ts, c8) owns tokens ts + TPW*i of each block; it pairs t = ts + TPW*pr with t + 8
      // and accumulates p'_t (1152 + x_t[d]) with v_dot2_f32_f16 (codes are finite, masked
      // tokens have p' = 0)
      constexpr int NPAIR = SH::VLOADS / 2;
      static_assert(SH::TPW * NPAIR == 8, "token pairs are (t, t + 8)");
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int pr = 0; pr < NPAIR; ++pr) {
          const int pair = ts + SH::TPW * pr;
          const u32x2 bw = vw[u][pr], cw = vw[u][pr + NPAIR];
          uint32_t xp[8];  // fp16 pairs (1152 + x_t, 1152 + x_{t+8}) for the lane's 8 d
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t bx = bw[k] ^ 0x80808080u, cx = cw[k] ^ 0x80808080u;
            const uint32_t i0 = __builtin_amdgcn_perm(cx, bx, 0x05010400u);  // b0 c0 b1 c1
            const uint32_t i1 = __builtin_amdgcn_perm(cx, bx, 0x07030602u);  // b2 c2 b3 c3
            xp[4 * k + 0] = widen_lo(i0);
            xp[4 * k + 1] = widen_hi(i0);
            xp[4 * k + 2] = widen_lo(i1);
            xp[4 * k + 3] = widen_hi(i1);
          }
          uint32_t pp[GP];
#pragma unroll
          for (int h4 = 0; h4 < GP; h4 += 4) {
            if constexpr (GP >= 4) {
              const u32x4 p4 = *reinterpret_cast<const u32x4*>(&s_pp[wave][u][pair][h4]);
              pp[h4] = p4[0]; pp[h4 + 1] = p4[1]; pp[h4 + 2] = p4[2]; pp[h4 + 3] = p4[3];
            } else {
#pragma unroll
              for (int h = 0; h < GP; ++h) pp[h] = s_pp[wave][u][pair][h];
            }
          }
#pragma unroll
          for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              acc[h][e] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pp[h]),
                                                 __builtin_bit_cast(f16x2, xp[e]), acc[h][e], false);
        }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < SH::VLOADS; ++i) {
          const int slot = i * SH::TPW + ts;
          const int tpos = t_begin + (blk0 + u) * BS + slot;
          if (!(okb[u] && tpos >= lo && tpos < t_end)) continue;  // masked slot may hold NaN
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(vw[u][i][e]);
            x[2 * e + 1] = bf16_hi(vw[u][i][e]);
          }
          float pv[GP];
#pragma unroll
          for (int h4 = 0; h4 < GP; h4 += 4) {
            if constexpr (GP >= 4) {
              const f32x4 p4 = *reinterpret_cast<const f32x4*>(&s_p[wave][u * BS + slot][h4]);
              pv[h4] = p4[0]; pv[h4 + 1] = p4[1]; pv[h4 + 2] = p4[2]; pv[h4 + 3] = p4[3];
            } else {
#pragma unroll
              for (int h = 0; h < GP; ++h) pv[h] = s_p[wave][u * BS + slot][h];
            }
          }
#pragma unroll
          for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv[h], x[e], acc[h][e]);
        }
    }
    __builtin_amdgcn_wave_barrier();  // the staging slices are rewritten by the next chunk
  }

  // ---- reduce inside the wave ------------------------------------------------------------
  // row sums: lanes hq, hq+16, hq+32, hq+48
  float l_w = l_part + __shfl_xor(l_part, 16);
  l_w = sum_x32(l_w);
  float ps_w = 0.f;
  if constexpr (I8) {
    ps_w = ps_part + __shfl_xor(ps_part, 16);
    ps_w = sum_x32(ps_w);
  }
  // PV accumulators: lanes with equal c8
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = SH::CPR; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o);
  if (grp == 0 && hq < GP) {
    s_ml[wave][0][hq] = m_run;
    s_ml[wave][1][hq] = l_w;
    s_ml[wave][2][hq] = ps_w;
  }
  __builtin_amdgcn_wave_barrier();
  if (ts == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float corr = I8 ? kI8Bias * s_ml[wave][2][h] : 0.f;  // remove the +1152 of the codes
#pragma unroll
      for (int e = 0; e < 8; ++e) s_red[wave][h][8 * c8 + e] = acc[h][e] - corr;
    }
  }
  __syncthreads();

  // ---- merge the 4 waves and write ---------------------------------------------------------
  for (int i = threadIdx.x; i < G * D; i += kDecodeThreads) {
    const int h = i / D, d = i % D;
    float M = s_ml[0][0][h];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_ml[w][0][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float wt = fast_exp2(s_ml[w][0][h] - M);  // waves that saw no token: l = 0, acc = 0
      num = fmaf(wt, s_red[w][h][d], num);
      den = fmaf(wt, s_ml[w][1][h], den);
    }
    const float inv = 1.0f / den;
    const int head = g * G + h;
    if (n_split == 1) {
      out[((int64_t)b * Hq + head) * D + d] = (uint16_t)f32_to_bf16_bits(num * inv);
    } else {
      const int64_t pi = ((int64_t)b * Hq + head) * n_split + split;
      part_o[pi * D + d] = num * inv;
      if (d == 0) part_lse[pi] = M + __log2f(den);
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
  (void)Hq;
  DecodePlan p{};
  const int span = window > 0 ? std::min(max_context_len, window + 15) : max_context_len;
  int C = split_tokens;
  if (C == 0) {
    // 2048-token splits for long spans, 1024 otherwise (a quarter of the span, at least 256,
    // for short contexts): enough workgroups to balance ragged contexts over the CUs, few
    // enough that the per-split prologue and the merge stay small (measured on MI355X).
    if (span >= 8192)
      C = 2048;
    else
      C = std::min(1024, std::max(256, ((span / 4) + 255) & ~255));
  }
  p.split_tokens = C;
  p.n_split = std::max(1, (span + C - 1) / C);
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
  dim3 grid(a.Hkv, a.B, ns);
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
