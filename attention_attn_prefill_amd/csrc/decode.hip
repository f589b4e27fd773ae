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
// Design (gfx950). All G = Hq/Hkv query heads of a KV head g are served by the same wave, so
// every K/V byte is read from HBM once. The work is the list of (sequence b, KV head g,
// 16-token block) triples that hold visible tokens; two launch shapes split it:
//  * balanced (the default): a persistent grid whose waves each take an equal contiguous range
//    of that list, so ragged context lengths cost no imbalance; a wave writes one partial per
//    (b, g) segment its range touches, or the final output when it holds a whole segment;
//  * fixed split (split_tokens > 0): one workgroup of 4 waves per (split of C tokens, g, b),
//    the waves merged in LDS.
// A wave walks its blocks in chunks of U blocks; for a chunk it
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
// Partials (o, lse) are merged by log-sum-exp in a second small kernel.
#include "common.h"
#include "launch.h"
#include <hip/hip_fp16.h>
#include <algorithm>
#include <climits>
#include <type_traits>

namespace attn {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = 4;
constexpr int kMaxSplitBlocks = kMaxSplitTokens / 16;  // the table slice is kept in LDS

// First key any of the QL query rows (positions ctx - QL .. ctx - 1) attends to.
__device__ __forceinline__ int first_key(int ctx, int QL, int window) {
  return window > 0 ? max(0, ctx - QL + 1 - window) : 0;
}

__device__ __forceinline__ int decode_ctx(const int32_t* ctx_lens, int b, int max_ctx,
                                          int max_blocks, int bs) {
  int c = ctx_lens[b];
  int cap = min(max_ctx, max_blocks * bs);
  return c < 0 ? 0 : (c > cap ? cap : c);
}

typedef short i16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_v2i32;

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

// FP8 E4M3 -> fp16 pair with gfx950's packed conversion (scale 1): every E4M3 value,
// subnormals included, is exact in fp16. fp8x2_lo / fp8x2_hi convert bytes 0, 1 / 2, 3 of u.
__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t u) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t u) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 1.0f, true));
}

// Byte caches run QK^T on fp16 MFMA, so each bf16 query column is brought into fp16 range
// first: multiplied by 2^k, k chosen from the column's largest magnitude so that it lands in
// [2^8, 2^9) (k clamped to [-126, 126]). The product is exact, every element within 2^-22 of
// the column maximum stays an fp16 normal (exact), and 2^-k is folded into the score scale.
// Without it a bf16 query element of magnitude >= 65520 would become inf, and elements below
// 2^-24 would flush to zero.
__device__ __forceinline__ int q_range_shift(float amax) {
  if (!(amax > 0.f)) return 0;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xff) - 127;  // floor(log2) for normals
  return min(126, max(-126, 8 - e));
}
__device__ __forceinline__ float pow2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

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
template <int D, int KV>
struct DecodeShape {
  static constexpr bool BYTE = KV != kKvBf16;              // one byte per cached element
  static constexpr int BS = 16;
  static constexpr int U = (D == 64 || BYTE) ? 2 : 1;     // blocks per chunk
  static constexpr int KSTEPS = D / 32;                    // MFMA k-steps per block
  static constexpr int KLOADS = BYTE ? D / 64 : D / 32;    // 16-byte K loads per lane per block
  static constexpr int VBYTES = BYTE ? 8 : 16;             // bytes per lane per V load (8 elements)
  static constexpr int CPR = D / 8;                        // lanes per V row
  static constexpr int TPW = 64 / CPR;                     // tokens per V load instruction
  static constexpr int VLOADS = BS / TPW;                  // V loads per lane per block
};

// Per-wave decode state: Q fragments, running max, row-sum shares and PV accumulators of the
// G heads of one (sequence, KV head). The LDS staging slices belong to the wave.
template <int D, int GP, int KV>
struct DecodeWave {
  static constexpr bool kMfmaPv = false;
  using SH = DecodeShape<D, KV>;
  static constexpr bool BYTE = SH::BYTE, I8 = KV == kKvI8, F8 = KV == kKvFp8;
  static constexpr int BS = SH::BS, U = SH::U, CT = U * BS;  // CT tokens per chunk
  typedef typename std::conditional<BYTE, f16x8, bf16x8>::type frag_t;
  typedef typename std::conditional<BYTE, u32x2, u32x4>::type vword_t;
  // probabilities handed from the MFMA lanes to the PV lanes: fp32 [token][head] for bf16;
  // for byte caches, fp16 pairs (token t, token t + 8) of p' = p * v_scale, [block][pair][head]
  struct Lds {
    float p[BYTE ? 1 : CT][GP];
    uint32_t pp[BYTE ? U : 1][8][GP];
    float alpha[GP];
  };

  int lane, hq, grp, c8, ts;
  frag_t qf[SH::KSTEPS];
  float bias;     // INT8: 1152 * sum of this head's fp16 q values (the widened codes carry +1152)
  float qscale;   // byte caches: 2^-k of this lane's column (its query was scaled by 2^k)
  float m_run;    // per head (lanes hq), log2 units
  float l_part;   // this lane's share of the row sum
  float ps_part;  // INT8: this lane's share of sum(p'), in the fp16 values used
  float acc[GP][8];
  int qpos, wlo;  // this lane's column: its query position and first key its window admits

  __device__ __forceinline__ void init(int lane_) {
    lane = lane_;
    hq = lane & 15;  // MFMA (QK^T) lane roles: column = query head, rows = 4 tokens of a block
    grp = lane >> 4;
    c8 = lane % SH::CPR;  // PV lane roles: 8 consecutive d of one token (bf16) or a token pair (INT8)
    ts = lane / SH::CPR;
  }

  // Q^T of the wave's columns, padded to 16: column c < G*QL is query row r = c / G (position
  // ctx - QL + r) of head g*G + c % G of sequence b; q is [B][QL][Hq][D].
  __device__ __forceinline__ void load_q(const uint16_t* __restrict__ q, int b, int g, int G,
                                         int QL, int Hq, int ctx, int window) {
    float qsum = 0.f;
    const int ncol = G * QL;
    const int r = hq / G, h = hq % G;
    const uint16_t* qrow = q + (((int64_t)b * QL + r) * Hq + g * G + h) * D;
    qpos = ctx - QL + r;
    wlo = window > 0 ? qpos - window + 1 : INT_MIN;
    u32x4 w[SH::KSTEPS];
#pragma unroll
    for (int j = 0; j < SH::KSTEPS; ++j) {
      // bf16: step j covers d = 32j + 8*grp + e; INT8: one 16-byte load feeds steps 2jj,
      // 2jj+1 covering d = 64*jj + 16*grp + 8*sub + e.
      const int d0 = BYTE ? (64 * (j / 2) + 16 * grp + 8 * (j % 2)) : (32 * j + 8 * grp);
      w[j] = (u32x4){0u, 0u, 0u, 0u};
      if (hq < ncol) w[j] = *reinterpret_cast<const u32x4*>(qrow + d0);
      if constexpr (!BYTE) qf[j] = __builtin_bit_cast(bf16x8, w[j]);
    }
    qscale = 1.f;
    if constexpr (BYTE) {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < SH::KSTEPS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[j][e])), fabsf(bf16_hi(w[j][e]))));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = max_x32(amax);
      const int k = q_range_shift(amax);
      const float up = pow2i(k);
      qscale = pow2i(-k);
#pragma unroll
      for (int j = 0; j < SH::KSTEPS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[j][2 * e] = (_Float16)(bf16_lo(w[j][e]) * up);
          qf[j][2 * e + 1] = (_Float16)(bf16_hi(w[j][e]) * up);
          qsum += (float)qf[j][2 * e] + (float)qf[j][2 * e + 1];
        }
    }
    if constexpr (I8) {
      qsum += __shfl_xor(qsum, 16);
      qsum = sum_x32(qsum);
    }
    bias = I8 ? kI8Bias * qsum : 0.f;
  }

  __device__ __forceinline__ void reset() {
    m_run = kNegBig;
    l_part = 0.f;
    ps_part = 0.f;
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  // The registers of one chunk in flight: blocks pb[u] (physical; okb[u] false = skip)
  // holding logical tokens t0 + 16u .. t0 + 16u + 15.
  struct Chunk {
    u32x4 kw[U][SH::KLOADS];
    vword_t vw[U][SH::VLOADS];
    float ksc[U][4], vsc[U][4];
    int pb[U];
    bool okb[U];
    int t0;
  };

  // Issue every load of a chunk (pb, okb and t0 already set).
  __device__ __forceinline__ void load(Chunk& c, const void* __restrict__ k_cache,
                                       const void* __restrict__ v_cache,
                                       const __half* __restrict__ k_scale,
                                       const __half* __restrict__ v_scale, int Hkv, int g,
                                       Lds&) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t brow = pool_offset(c.pb[u], Hkv, g, BS, 0, D);
      if constexpr (BYTE) {
        const int8_t* kc = reinterpret_cast<const int8_t*>(k_cache) + brow + (int64_t)hq * D;
#pragma unroll
        for (int jj = 0; jj < SH::KLOADS; ++jj)
          c.kw[u][jj] = ld_stream<u32x4>(kc + 64 * jj + 16 * grp);
        const int8_t* vc = reinterpret_cast<const int8_t*>(v_cache) + brow;
#pragma unroll
        for (int i = 0; i < SH::VLOADS; ++i)
          c.vw[u][i] = ld_stream<u32x2>(vc + (int64_t)(i * SH::TPW + ts) * D + 8 * c8);
        const int64_t srow = ((int64_t)c.pb[u] * Hkv + g) * BS + 4 * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c.ksc[u][i] = __half2float(k_scale[srow + i]);
          c.vsc[u][i] = __half2float(v_scale[srow + i]);
        }
      } else {
        const uint16_t* kc = reinterpret_cast<const uint16_t*>(k_cache) + brow + (int64_t)hq * D;
#pragma unroll
        for (int j = 0; j < SH::KLOADS; ++j)
          c.kw[u][j] = ld_stream<u32x4>(kc + 32 * j + 8 * grp);
        const uint16_t* vc = reinterpret_cast<const uint16_t*>(v_cache) + brow;
#pragma unroll
        for (int i = 0; i < SH::VLOADS; ++i)
          c.vw[u][i] = ld_stream<u32x4>(vc + (int64_t)(i * SH::TPW + ts) * D + 8 * c8);
      }
    }
  }

  // Online softmax + PV of a loaded chunk; tokens outside [lo, hi) are masked, and for each
  // column the tokens after its query position or left of its window.
  __device__ __forceinline__ void compute(const Chunk& c, int lo, int hi, float scale_log2,
                                          Lds& L, bool = false) {
    // ---- scores on MFMA -----------------------------------------------------------------
    float sc[U][4];
    float cmax = -INFINITY;
    const float sl = BYTE ? scale_log2 * qscale : scale_log2;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BYTE) {
#pragma unroll
        for (int jj = 0; jj < SH::KLOADS; ++jj)
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            u32x4 hv;
            if constexpr (I8) {
              const uint32_t w0 = c.kw[u][jj][2 * sub] ^ 0x80808080u;
              const uint32_t w1 = c.kw[u][jj][2 * sub + 1] ^ 0x80808080u;
              hv = (u32x4){widen_lo(w0), widen_hi(w0), widen_lo(w1), widen_hi(w1)};
            } else {
              const uint32_t w0 = c.kw[u][jj][2 * sub], w1 = c.kw[u][jj][2 * sub + 1];
              hv = (u32x4){fp8x2_lo(w0), fp8x2_hi(w0), fp8x2_lo(w1), fp8x2_hi(w1)};
            }
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, hv),
                                                        qf[2 * jj + sub], a4, 0, 0, 0);
          }
      } else {
#pragma unroll
        for (int j = 0; j < SH::KSTEPS; ++j)
          a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, c.kw[u][j]), qf[j], a4, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = c.t0 + u * BS + 4 * grp + i;
        const bool vis = c.okb[u] && t >= lo && t < hi && t <= qpos && t >= wlo;
        float s;
        if constexpr (I8)
          s = (a4[i] - bias) * c.ksc[u][i] * sl;
        else if constexpr (F8)
          s = a4[i] * c.ksc[u][i] * sl;
        else
          s = a4[i] * sl;
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
      if (grp == 0 && hq < GP) L.alpha[hq] = alpha;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float al = L.alpha[h];
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
        if constexpr (BYTE) {
          // masked tokens: p = 0 exactly, and their (possibly NaN) scale is not used
          const _Float16 pv16 = (_Float16)(sc[u][i] == -INFINITY ? 0.f : p * c.vsc[u][i]);
          ps_part += (float)pv16;
          const int t = 4 * grp + i;  // token inside block u: pair t & 7, element t >> 3
          if (hq < GP) reinterpret_cast<_Float16*>(&L.pp[u][t & 7][hq])[t >> 3] = pv16;
        } else {
          if (hq < GP) L.p[u * BS + 4 * grp + i][hq] = p;
        }
      }
    __builtin_amdgcn_wave_barrier();
    // ---- PV on the VALU -------------------------------------------------------------------
    if constexpr (BYTE) {
      // lane (ts, c8) owns tokens ts + TPW*i of each block; it pairs t = ts + TPW*pr with t + 8
      // and accumulates p'_t * widened(x_t[d]) with v_dot2_f32_f16 -- INT8: 1152 + x, FP8:
      // the E4M3 value (codes are finite, masked tokens have p' = 0)
      constexpr int NPAIR = SH::VLOADS / 2;
      static_assert(SH::TPW * NPAIR == 8, "token pairs are (t, t + 8)");
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int pr = 0; pr < NPAIR; ++pr) {
          const int pair = ts + SH::TPW * pr;
          const u32x2 bw = c.vw[u][pr], cw = c.vw[u][pr + NPAIR];
          uint32_t xp[8];  // fp16 pairs (token t, token t + 8) for the lane's 8 d
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t bx = I8 ? bw[k] ^ 0x80808080u : bw[k];
            const uint32_t cx = I8 ? cw[k] ^ 0x80808080u : cw[k];
            const uint32_t i0 = __builtin_amdgcn_perm(cx, bx, 0x05010400u);  // b0 c0 b1 c1
            const uint32_t i1 = __builtin_amdgcn_perm(cx, bx, 0x07030602u);  // b2 c2 b3 c3
            if constexpr (I8) {
              xp[4 * k + 0] = widen_lo(i0);
              xp[4 * k + 1] = widen_hi(i0);
              xp[4 * k + 2] = widen_lo(i1);
              xp[4 * k + 3] = widen_hi(i1);
            } else {
              xp[4 * k + 0] = fp8x2_lo(i0);
              xp[4 * k + 1] = fp8x2_hi(i0);
              xp[4 * k + 2] = fp8x2_lo(i1);
              xp[4 * k + 3] = fp8x2_hi(i1);
            }
          }
          uint32_t pp[GP];
#pragma unroll
          for (int h4 = 0; h4 < GP; h4 += 4) {
            if constexpr (GP >= 4) {
              const u32x4 p4 = *reinterpret_cast<const u32x4*>(&L.pp[u][pair][h4]);
              pp[h4] = p4[0]; pp[h4 + 1] = p4[1]; pp[h4 + 2] = p4[2]; pp[h4 + 3] = p4[3];
            } else {
#pragma unroll
              for (int h = 0; h < GP; ++h) pp[h] = L.pp[u][pair][h];
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
          const int tpos = c.t0 + u * BS + slot;
          if (!(c.okb[u] && tpos >= lo && tpos < hi)) continue;  // masked slot may hold NaN
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(c.vw[u][i][e]);
            x[2 * e + 1] = bf16_hi(c.vw[u][i][e]);
          }
          float pv[GP];
#pragma unroll
          for (int h4 = 0; h4 < GP; h4 += 4) {
            if constexpr (GP >= 4) {
              const f32x4 p4 = *reinterpret_cast<const f32x4*>(&L.p[u * BS + slot][h4]);
              pv[h4] = p4[0]; pv[h4 + 1] = p4[1]; pv[h4 + 2] = p4[2]; pv[h4 + 3] = p4[3];
            } else {
#pragma unroll
              for (int h = 0; h < GP; ++h) pv[h] = L.p[u * BS + slot][h];
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

  // Reduce inside the wave: returns this head's row sum l and sum(p') (lanes hq); afterwards
  // the lanes with ts == 0 hold the complete accumulators of d = 8*c8 .. 8*c8+7, with the
  // INT8 bias already removed.
  __device__ __forceinline__ void reduce(float& l_w, float& ps_w) {
    l_w = l_part + __shfl_xor(l_part, 16);  // lanes hq, hq+16, hq+32, hq+48
    l_w = sum_x32(l_w);
    ps_w = 0.f;
    if constexpr (I8) {
      ps_w = ps_part + __shfl_xor(ps_part, 16);
      ps_w = sum_x32(ps_w);
    }
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int o = SH::CPR; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o);
    if constexpr (I8) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float corr = kI8Bias * __shfl(ps_w, h);  // remove the +1152 of the codes
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] -= corr;
      }
    }
  }

  // f(column, d0, values) for each run of 8 consecutive d this lane holds (after reduce)
  template <typename F>
  __device__ __forceinline__ void emit(F&& f) const {
    if (ts == 0) {
#pragma unroll
      for (int h = 0; h < GP; ++h) f(h, 8 * c8, acc[h]);
    }
  }
};

// PV on MFMA (byte caches, and bf16 caches with 8 or more query columns): the same per-wave
// state as DecodeWave. A chunk is 32 tokens (two 16-token blocks). Row m of block MFMA u
// (u = 0, 1) is chunk token 8*(m/4) + 4u + m%4, so the score accumulator of lane (column c,
// group g) holds chunk tokens 8g .. 8g+7 -- the B operand of a 16x16x32 MFMA with the 32
// tokens as K. V goes global -> LDS (the wave's own slice, 16-byte chunks XOR-swizzled by row)
// and returns transposed: for byte caches ds_read_b64_tr_b8 gives lane (d, g) of slice s tokens
// 8g .. 8g+7 of d = 16s + lane % 16 (widened to fp16 exactly as K is); for bf16 two
// ds_read_b64_tr_b16 give 4 tokens each. Oᵀ accumulates in 16x16 tiles: lane (c, g) holds
// d = 16s + 4g .. 4g+3 of column c.
template <int D, int GP, int KV>
struct DecodeWaveM {
  static constexpr bool kMfmaPv = true;
  static constexpr bool I8 = KV == kKvI8, F8 = KV == kKvFp8, BF = KV == kKvBf16;
  static constexpr int ES = BF ? 2 : 1;           // bytes per cached element
  static constexpr int BS = 16, U = 2, CT = 32;  // CT tokens per chunk
  static constexpr int KLOADS = BF ? D / 32 : D / 64;  // 16-byte K loads per lane per block MFMA
  static constexpr int KSTEPS = D / 32;           // QK MFMA k-steps
  static constexpr int NS = D / 16;               // 16-d output slices
  static constexpr int ROWB = D * ES;             // bytes per V row
  static constexpr int VINSTR = CT * ROWB / 1024;  // 1 KB DMA instructions per chunk
  static constexpr int kLoads = U * KLOADS + (BF ? 0 : 2) + VINSTR;  // vector memory ops of load()
  static_assert(kLoads < 64, "vmcnt field");
  typedef typename std::conditional<BF, bf16x8, f16x8>::type frag_t;
  struct Lds {
    __attribute__((aligned(16))) uint8_t v[CT * ROWB];  // V, [token][16-byte chunk ^ swz]
  };
  // chunk swizzle of V row r: the rows one transposing read touches land on distinct banks
  // (bf16: an even XOR keeps the two chunks of a 32-byte read segment together)
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (BF) return D == 128 ? 2 * (r & 3) : 2 * ((r >> 1) & 1);
    return D == 128 ? (r & 7) : ((r >> 2) & 3);
  }

  int lane, hq, grp;
  frag_t qf[KSTEPS];
  float bias;     // INT8: 1152 * sum of this column's fp16 q values
  float qscale;   // byte caches: 2^-k of this lane's column (its query was scaled by 2^k)
  float m_run;    // this lane's column, log2 units
  float l_part;   // this lane's share of the column's row sum
  float ps_part;  // INT8: this lane's share of sum(p'), in the fp16 values used
  f32x4 o[NS];    // Oᵀ tiles
  int qpos, wlo;

  __device__ __forceinline__ void init(int lane_) {
    lane = lane_;
    hq = lane & 15;  // column (QK output, P operand, O tiles)
    grp = lane >> 4;
  }

  // Q^T of the wave's columns, padded to 16 (same rule as DecodeWave): bf16 step j covers
  // d = 32j + 8*grp + e; byte caches d = 64*(j/2) + 16*grp + 8*(j%2) + e.
  __device__ __forceinline__ void load_q(const uint16_t* __restrict__ q, int b, int g, int G,
                                         int QL, int Hq, int ctx, int window) {
    float qsum = 0.f;
    const int ncol = G * QL;
    const int r = hq / G, h = hq % G;
    const uint16_t* qrow = q + (((int64_t)b * QL + r) * Hq + g * G + h) * D;
    qpos = ctx - QL + r;
    wlo = window > 0 ? qpos - window + 1 : INT_MIN;
    u32x4 w[KSTEPS];
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      const int d0 = BF ? 32 * j + 8 * grp : 64 * (j / 2) + 16 * grp + 8 * (j % 2);
      w[j] = (u32x4){0u, 0u, 0u, 0u};
      if (hq < ncol) w[j] = *reinterpret_cast<const u32x4*>(qrow + d0);
      if constexpr (BF) qf[j] = __builtin_bit_cast(bf16x8, w[j]);
    }
    qscale = 1.f;
    if constexpr (!BF) {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[j][e])), fabsf(bf16_hi(w[j][e]))));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = max_x32(amax);
      const int k = q_range_shift(amax);
      const float up = pow2i(k);
      qscale = pow2i(-k);
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[j][2 * e] = (_Float16)(bf16_lo(w[j][e]) * up);
          qf[j][2 * e + 1] = (_Float16)(bf16_hi(w[j][e]) * up);
          qsum += (float)qf[j][2 * e] + (float)qf[j][2 * e + 1];
        }
    }
    if constexpr (I8) {
      qsum += __shfl_xor(qsum, 16);
      qsum = sum_x32(qsum);
    }
    bias = I8 ? kI8Bias * qsum : 0.f;
  }

  __device__ __forceinline__ void reset() {
    m_run = kNegBig;
    l_part = 0.f;
    ps_part = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) o[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  struct Chunk {
    u32x4 kw[U][KLOADS];  // K of this lane's row of block MFMA u
    u32x4 ksc8, vsc8;     // byte caches: fp16 scales of chunk tokens 8*grp .. 8*grp+7
    int pb[U];
    bool okb[U];
    int t0;
  };
  // physical block of chunk block i (0 or 1); a select, not an indexed access (a lane-varying
  // index would put the array in scratch memory)
  static __device__ __forceinline__ int blk_of(const Chunk& c, int i) { return i ? c.pb[1] : c.pb[0]; }

  // Issue every load of a chunk (pb, okb and t0 already set): K (and scales) to registers,
  // V to the wave's LDS slice (awaited in compute).
  __device__ __forceinline__ void load(Chunk& c, const void* __restrict__ k_cache,
                                       const void* __restrict__ v_cache,
                                       const __half* __restrict__ k_scale,
                                       const __half* __restrict__ v_scale, int Hkv, int g,
                                       Lds& L) {
    const char* kb = reinterpret_cast<const char*>(k_cache);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tok = 8 * (hq >> 2) + 4 * u + (hq & 3);  // this lane's row of block MFMA u
      const char* kc = kb + pool_offset(blk_of(c, tok >> 4), Hkv, g, BS, tok & 15, D) * ES;
#pragma unroll
      for (int j = 0; j < KLOADS; ++j)
        c.kw[u][j] = ld_stream<u32x4>(kc + (BF ? 2 * (32 * j + 8 * grp) : 64 * j + 16 * grp));
    }
    if constexpr (!BF) {
      const int64_t srow = ((int64_t)blk_of(c, grp >> 1) * Hkv + g) * BS + ((8 * grp) & 15);
      c.ksc8 = *reinterpret_cast<const u32x4*>(k_scale + srow);
      c.vsc8 = *reinterpret_cast<const u32x4*>(v_scale + srow);
    }
    const char* vb = reinterpret_cast<const char*>(v_cache);
#pragma unroll
    for (int n = 0; n < VINSTR; ++n) {
      const int off = n * 1024 + 16 * lane;  // LDS byte of this lane's 16 bytes
      const int r = off / ROWB, ch = (off % ROWB) / 16;
      const char* src = vb + pool_offset(blk_of(c, r >> 4), Hkv, g, BS, r & 15, D) * ES + 16 * (ch ^ swz(r));
      lds_dma_16(src, lds_addr(L.v + n * 1024));
    }
  }

  __device__ __forceinline__ float scale_of(u32x4 s8, int e) const {
    return __half2float(__builtin_bit_cast(__half, (uint16_t)(s8[e >> 1] >> (16 * (e & 1)))));
  }

  // Online softmax + PV of a loaded chunk (tokens outside [lo, hi) masked, and for each column
  // the tokens after its query position or left of its window). next_in_flight: the next
  // chunk's loads (kLoads of them) were issued after this chunk's.
  __device__ __forceinline__ void compute(const Chunk& c, int lo, int hi, float scale_log2,
                                          Lds& L, bool next_in_flight = false) {
    // ---- scores on MFMA (rows permuted: lane (column, grp) gets tokens 8grp + 4u + i) ------
    float sc[U][4];
    float cmax = -INFINITY;
    const bool okb = (grp >> 1) ? c.okb[1] : c.okb[0];  // the block of tokens 8grp .. 8grp+7
    const float sl = BF ? scale_log2 : scale_log2 * qscale;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j)
          a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, c.kw[u][j]), qf[j], a4, 0, 0, 0);
      } else {
#pragma unroll
        for (int jj = 0; jj < KLOADS; ++jj)
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            u32x4 hv;
            if constexpr (I8) {
              const uint32_t w0 = c.kw[u][jj][2 * sub] ^ 0x80808080u;
              const uint32_t w1 = c.kw[u][jj][2 * sub + 1] ^ 0x80808080u;
              hv = (u32x4){widen_lo(w0), widen_hi(w0), widen_lo(w1), widen_hi(w1)};
            } else {
              const uint32_t w0 = c.kw[u][jj][2 * sub], w1 = c.kw[u][jj][2 * sub + 1];
              hv = (u32x4){fp8x2_lo(w0), fp8x2_hi(w0), fp8x2_lo(w1), fp8x2_hi(w1)};
            }
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, hv),
                                                        qf[2 * jj + sub], a4, 0, 0, 0);
          }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * u + i;  // token 8grp + e of the chunk
        const int t = c.t0 + 8 * grp + e;
        const bool vis = okb && t >= lo && t < hi && t <= qpos && t >= wlo;
        float s;
        if constexpr (I8)
          s = (a4[i] - bias) * scale_of(c.ksc8, e) * sl;
        else if constexpr (F8)
          s = a4[i] * scale_of(c.ksc8, e) * sl;
        else
          s = a4[i] * sl;
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
#pragma unroll
      for (int s = 0; s < NS; ++s) o[s] *= alpha;  // this lane's column
    }
    // ---- probabilities: the B operand, tokens 8grp .. 8grp+7 -------------------------------
    // bf16: p rounded to bf16, and the row sum adds the rounded values (those PV uses);
    // byte caches: p' = p * v_scale in fp16
    frag_t pf;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * u + i;
        const float p = fast_exp2(sc[u][i] - m_run);
        if constexpr (BF) {
          const __bf16 pb16 = (__bf16)p;
          l_part += (float)pb16;
          pf[e] = pb16;
        } else {
          l_part += p;
          // masked tokens: p' = 0 exactly, and their (possibly NaN) scale is not used
          const _Float16 pv16 = (_Float16)(sc[u][i] == -INFINITY ? 0.f : p * scale_of(c.vsc8, e));
          ps_part += (float)pv16;
          pf[e] = pv16;
        }
      }
    // ---- PV on MFMA ------------------------------------------------------------------------
    // V of chunk tokens outside [lo, hi) or in an unusable block is zeroed: their p is 0, but
    // unwritten slots may hold NaN (0 * NaN = NaN). Lane bits: token 8grp + e is byte e (byte
    // caches) or half e of the two-read bf16 operand.
    u32x4 vmask = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    const bool ragged = !(c.okb[0] && c.okb[1] && c.t0 >= lo && c.t0 + CT <= hi);
    if (ragged) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = c.t0 + 8 * grp + e;
        if (!(okb && t >= lo && t < hi)) {
          if constexpr (BF)
            vmask[e >> 1] &= ~(0xffffu << (16 * (e & 1)));
          else
            vmask[e >> 2] &= ~(0xffu << (8 * (e & 3)));
        }
      }
    }
    if (next_in_flight)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (kLoads & 0xF) | ((kLoads >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // this chunk's V copy has landed in LDS
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      frag_t va;
      if constexpr (BF) {
        // rows 8grp + 4h + (lane%16)/4, elements 16s + 4(lane%4) .. +3: lane gets 4 tokens of d
        u32x4 w;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = 8 * grp + 4 * h + ((lane & 15) >> 2);
          const int chk = (2 * s + ((lane & 3) >> 1)) ^ swz(rr);
          const i16x4 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(L.v + rr * ROWB + 16 * chk + 8 * (lane & 1)));
          const u32x2 t2 = __builtin_bit_cast(u32x2, t4);
          w[2 * h] = t2[0] & vmask[2 * h];
          w[2 * h + 1] = t2[1] & vmask[2 * h + 1];
        }
        va = __builtin_bit_cast(bf16x8, w);
      } else {
        const int rr = 8 * grp + ((lane & 15) >> 1);  // the row this lane addresses
        const u32x2 raw = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                       (lds_v2i32*)(L.v + rr * ROWB + 16 * (s ^ swz(rr)) + 8 * (lane & 1))));
        const uint32_t w0 = raw[0] & vmask[0], w1 = raw[1] & vmask[1];
        u32x4 hv;
        if constexpr (I8) {
          const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
          hv = (u32x4){widen_lo(x0), widen_hi(x0), widen_lo(x1), widen_hi(x1)};
        } else {
          hv = (u32x4){fp8x2_lo(w0), fp8x2_hi(w0), fp8x2_lo(w1), fp8x2_hi(w1)};
        }
        va = __builtin_bit_cast(f16x8, hv);
      }
      if constexpr (BF)
        o[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[s], 0, 0, 0);
      else
        o[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pf, o[s], 0, 0, 0);
    }
  }

  // Row sum l and sum(p') of this lane's column (complete on every lane of the column); the
  // Oᵀ tiles are already complete, the INT8 bias is removed here.
  __device__ __forceinline__ void reduce(float& l_w, float& ps_w) {
    l_w = l_part + __shfl_xor(l_part, 16);
    l_w = sum_x32(l_w);
    ps_w = 0.f;
    if constexpr (I8) {
      ps_w = ps_part + __shfl_xor(ps_part, 16);
      ps_w = sum_x32(ps_w);
      const float corr = kI8Bias * ps_w;  // remove the +1152 of the codes
#pragma unroll
      for (int s = 0; s < NS; ++s) o[s] -= corr;
    }
  }

  // f(column, d0, values) for each run of 4 consecutive d this lane holds (columns < GP)
  template <typename F>
  __device__ __forceinline__ void emit(F&& f) const {
    if (hq < GP) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float v4[4] = {o[s][0], o[s][1], o[s][2], o[s][3]};
        f(hq, 16 * s + 4 * grp, v4);
      }
    }
  }
};

// bf16 caches with few columns stream best with PV on the VALU (measured); byte caches and
// 8 or more columns use the MFMA form
template <int D, int GP, int KV>
using DecodeWaveT = typename std::conditional<KV == kKvBf16 && GP < 8, DecodeWave<D, GP, KV>,
                                              DecodeWaveM<D, GP, KV>>::type;

// ---- fixed split: one workgroup of 4 waves per (split, g, b) --------------------------------
// VIRT: g counts virtual KV heads, R of them per cache head (more query columns per cache head
// than one MFMA tile holds); without it R is 1 and not read.
template <int D, int GP, int KV, bool VIRT>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const __half* __restrict__ k_scale,
    const __half* __restrict__ v_scale, const int32_t* __restrict__ table,
    const int32_t* __restrict__ ctx_lens, uint16_t* __restrict__ out,
    float* __restrict__ part_o, float* __restrict__ part_lse, int Hq, int Hkv, int G, int QL,
    int max_blocks, int num_blocks, int max_ctx, float scale_log2, int window, int C,
    int n_split, int R) {
  using W = DecodeWaveT<D, GP, KV>;
  constexpr int BS = W::BS, U = W::U;
  // the V staging slices are dead once every wave has left its loop, and the per-wave O
  // partials reuse their space (a barrier separates the two)
  __shared__ union {
    typename W::Lds lds[kDecodeWaves];
    float red[kDecodeWaves][GP][D];
  } s_u;
  __shared__ float s_ml[kDecodeWaves][2][GP];
  __shared__ int s_pb[kMaxSplitBlocks];  // the split's slice of the block table

  // Grid (Hkv, B, n_split) with the split index slowest and reversed: consecutive workgroups
  // (dispatched round-robin over the XCDs) then belong to different sequences, so the XCDs
  // share ragged work evenly; splits that exist only for long contexts go first.
  const int split = n_split - 1 - blockIdx.z, g = blockIdx.x, b = blockIdx.y;
  const int Hk = VIRT ? Hkv / R : Hkv, gk = VIRT ? g / R : g;  // the cache's heads, g's head
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int ncol = G * QL;
  const int ctx = decode_ctx(ctx_lens, b, max_ctx, max_blocks, BS);
  const int lo = first_key(ctx, QL, window);
  const int base = lo & ~(BS - 1);
  const int t_begin = base + split * C;
  if (ctx <= 0) {
    if (split == 0 && n_split == 1) {
      for (int i = threadIdx.x; i < ncol * D; i += kDecodeThreads) {
        const int c = i / D;
        out[(((int64_t)b * QL + c / G) * Hq + g * G + c % G) * D + i % D] = 0;
      }
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

  W w;
  w.init(lane);
  w.load_q(q, b, g, G, QL, Hq, ctx, window);
  w.reset();
  // this wave's chunks are ch = wave, wave + 4, ...
  const int nchunk = (nblk + U - 1) / U;
  typename W::Chunk cA;
  auto prep = [&](typename W::Chunk& c, int ch) {
    const int blk0 = ch * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = blk0 + u;
      const int e = __builtin_amdgcn_readfirstlane(blk < nblk ? s_pb[blk] : -1);
      c.okb[u] = e >= 0;
      c.pb[u] = c.okb[u] ? e : 0;
    }
    c.t0 = t_begin + blk0 * BS;
    w.load(c, k_cache, v_cache, k_scale, v_scale, Hk, gk, s_u.lds[wave]);
  };
  for (int ch = wave; ch < nchunk; ch += kDecodeWaves) {
    prep(cA, ch);
    w.compute(cA, lo, t_end, scale_log2, s_u.lds[wave]);
  }

  float l_w, ps_w;
  w.reduce(l_w, ps_w);
  if (w.grp == 0 && w.hq < GP) {
    s_ml[wave][0][w.hq] = w.m_run;
    s_ml[wave][1][w.hq] = l_w;
  }
  __syncthreads();  // every wave is done with the staging slices
  w.emit([&](int h, int d0, const auto& v) {
    constexpr int N = sizeof(v) / sizeof(v[0]);
#pragma unroll
    for (int e = 0; e < N; ++e) s_u.red[wave][h][d0 + e] = v[e];
  });
  __syncthreads();

  // ---- merge the 4 waves and write ---------------------------------------------------------
  for (int i = threadIdx.x; i < ncol * D; i += kDecodeThreads) {
    const int h = i / D, d = i % D;  // column h: query row h / G, head g*G + h % G
    float M = s_ml[0][0][h];
#pragma unroll
    for (int wv = 1; wv < kDecodeWaves; ++wv) M = fmaxf(M, s_ml[wv][0][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int wv = 0; wv < kDecodeWaves; ++wv) {
      const float wt = fast_exp2(s_ml[wv][0][h] - M);  // waves that saw no token: l = 0, acc = 0
      num = fmaf(wt, s_u.red[wv][h][d], num);
      den = fmaf(wt, s_ml[wv][1][h], den);
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    const int64_t orow = ((int64_t)b * QL + h / G) * Hq + g * G + h % G;  // query row, head
    if (n_split == 1) {
      out[orow * D + d] = (uint16_t)f32_to_bf16_bits(num * inv);
    } else {
      const int64_t pi = orow * n_split + split;
      part_o[pi * D + d] = num * inv;
      if (d == 0) part_lse[pi] = M + __log2f(den);
    }
  }
}

// Log-sum-exp merge of n partials (o_i, lse_i in log2 units) of one (sequence, query head),
// partial i at index first + i * stride, in one pass: the running max moves as partials
// arrive, and the loads of four partials are in flight together. One wave; lane l owns
// d = l + 64e. A partial whose piece saw no usable token has lse = -inf and weight 0.
template <int D>
__device__ __forceinline__ void merge_partials(const float* __restrict__ part_o,
                                               const float* __restrict__ part_lse,
                                               int64_t first, int64_t stride, int n,
                                               uint16_t* __restrict__ orow) {
  constexpr int EPT = D / 64, BATCH = 4;
  const int lane = threadIdx.x & 63;
  float M = -INFINITY, L = 0.f, acc[EPT] = {};
  for (int i = 0; i < n; i += BATCH) {
    float ls[BATCH], ov[BATCH][EPT];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int64_t idx = first + (int64_t)(i + k) * stride;
      ls[k] = i + k < n ? part_lse[idx] : -INFINITY;
#pragma unroll
      for (int e = 0; e < EPT; ++e) ov[k][e] = i + k < n ? part_o[idx * D + lane + 64 * e] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      if (ls[k] == -INFINITY) continue;
      if (ls[k] > M) {
        const float r = fast_exp2(M - ls[k]);  // M = -inf at first: r = 0
        L *= r;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] *= r;
        M = ls[k];
      }
      const float w = fast_exp2(ls[k] - M);
      L += w;
#pragma unroll
      for (int e = 0; e < EPT; ++e) acc[e] = fmaf(w, ov[k][e], acc[e]);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) orow[lane + 64 * e] = (uint16_t)f32_to_bf16_bits(acc[e] * inv);
}

// Fixed split: partials of (query row, head) are the n_valid splits that hold tokens.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ ctx_lens, uint16_t* __restrict__ out, int Hq, int QL,
    int max_blocks, int max_ctx, int window, int C, int n_split) {
  const int h = blockIdx.x, row = blockIdx.y, b = row / QL;  // row: query row b*QL + r
  const int ctx = decode_ctx(ctx_lens, b, max_ctx, max_blocks, 16);
  const int base = first_key(ctx, QL, window) & ~15;
  const int n_valid = ctx > 0 ? min(n_split, (ctx - base + C - 1) / C) : 0;
  merge_partials<D>(part_o, part_lse, ((int64_t)row * Hq + h) * n_split, 1, n_valid,
                    out + ((int64_t)row * Hq + h) * D);
}

// ---- balanced: persistent waves over equal ranges of the (b, g, block) list -----------------
// Sequence b contributes nvis(b) blocks per KV head (the blocks holding positions
// [lo_b, ctx_b)); the list orders blocks by (b, g, block). With T = Hkv * sum nvis and P waves,
// wave p owns list entries [p*q, min((p+1)*q, T)), q = ceil(T / P). The piece of segment
// s = b*Hkv + g that wave p holds goes to partial slot s + p: pieces of one segment sit in
// consecutive waves and segments follow in wave order, so the slots are distinct and there
// are at most B*Hkv + P of them.
__device__ __forceinline__ int visible_blocks(const int32_t* __restrict__ ctx_lens, int b,
                                              int max_ctx, int max_blocks, int window, int QL) {
  const int ctx = decode_ctx(ctx_lens, b, max_ctx, max_blocks, 16);
  if (ctx <= 0) return 0;
  return (ctx + 15) / 16 - first_key(ctx, QL, window) / 16;
}

template <int D, int GP, int KV, bool VIRT>
__global__ __launch_bounds__(kDecodeThreads) void decode_stream_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const __half* __restrict__ k_scale,
    const __half* __restrict__ v_scale, const int32_t* __restrict__ table,
    const int32_t* __restrict__ ctx_lens, uint16_t* __restrict__ out,
    int32_t* __restrict__ prefix_out, float* __restrict__ part_o, float* __restrict__ part_lse,
    int B, int Hq, int Hkv, int G, int QL, int max_blocks, int num_blocks, int max_ctx,
    float scale_log2, int R) {
  using W = DecodeWaveT<D, GP, KV>;
  constexpr int BS = W::BS, U = W::U;
  constexpr int NSLOT = W::kMfmaPv ? 2 : 1;  // MFMA form: the next chunk's V lands in slot 1
  __shared__ typename W::Lds s_lds[kDecodeWaves][NSLOT];
  __shared__ int s_pre[kStreamMaxB + 1];
  __shared__ int s_wsum[kDecodeWaves];
  __shared__ int s_tab[kDecodeWaves][2][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- prefix of visible blocks over the sequences (every workgroup; workgroup 0 also
  // stores it for the merge): per-thread runs, a scan inside each wave, then the wave totals
  {
    const int per = (B + kDecodeThreads - 1) / kDecodeThreads;
    const int b0 = tid * per;
    int run = 0;
    for (int i = 0; i < per && b0 + i < B; ++i)
      run += visible_blocks(ctx_lens, b0 + i, max_ctx, max_blocks, 0, QL);
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wave; ++w2) base += s_wsum[w2];
    run = base + incl - run;  // exclusive prefix of this thread's first sequence
    for (int i = 0; i < per && b0 + i < B; ++i) {
      s_pre[b0 + i] = run;
      run += visible_blocks(ctx_lens, b0 + i, max_ctx, max_blocks, 0, QL);
    }
    if (tid == kDecodeThreads - 1) s_pre[B] = base + incl;
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = tid; i <= B; i += kDecodeThreads) prefix_out[i] = s_pre[i];
  }

  const int64_t T = (int64_t)Hkv * s_pre[B];
  const int P = gridDim.x * kDecodeWaves;
  const int64_t qn = (T + P - 1) / P;
  const int p = blockIdx.x * kDecodeWaves + wave;
  const int64_t pos0 = p * qn;
  const int64_t end = min(pos0 + qn, T);
  if (pos0 >= end) return;  // no barrier follows

  // the segment holding entry pos0: the last b with Hkv * pre[b] <= pos0 (it has nvis(b) > 0)
  int b = 0;
  {
    int lo_b = 0, hi_b = B - 1;
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if ((int64_t)Hkv * s_pre[mid] <= pos0) lo_b = mid; else hi_b = mid - 1;
    }
    b = lo_b;
  }
  int nv = s_pre[b + 1] - s_pre[b];
  int g = (int)((pos0 - (int64_t)Hkv * s_pre[b]) / nv);
  const int Hk = VIRT ? Hkv / R : Hkv;  // the cache's KV heads; virtual head g reads g / R
  int gk = VIRT ? g / R : g;

  // Table entries of the wave's list range, 64 at a time: lane i of window k holds the entry
  // of list position pos0 + 64k + i. Windows are copied global -> LDS (two per wave) and the
  // next one is in flight while the current one is used, so neither a 64-entry boundary nor a
  // segment boundary waits on a table load; the copy is awaited only when a window begins
  // (a register copy of an in-flight load would make every later use wait for all loads).
  // The segment of each lane's position is found in the prefix (at or after sequence b_hint).
  auto fetch_window = [&](int64_t w0, int b_hint, int buf) {
    const int64_t e = w0 + lane;
    const int32_t* src = table;  // lanes past the range copy any valid entry, never used
    if (e < end) {
      int lo_b = b_hint, hi_b = B - 1;
      while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if ((int64_t)Hkv * s_pre[mid] <= e) lo_b = mid; else hi_b = mid - 1;
      }
      const int nvb = s_pre[lo_b + 1] - s_pre[lo_b];
      const int r = (int)(e - (int64_t)Hkv * s_pre[lo_b]);  // g * nvb + block
      src = table + (int64_t)lo_b * max_blocks + r % nvb;   // no window: block 0 is visible
    }
    lds_dma_4(src, lds_addr(&s_tab[wave][buf][0]));
  };
  int64_t wbase = pos0;
  int wk = 0;
  fetch_window(pos0, b, 0);
  if (pos0 + 64 < end) fetch_window(pos0 + 64, b, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int tab = s_tab[wave][0][lane];
  auto entry = [&](int64_t e) -> int {  // e: list position, visited in increasing order
    if (e - wbase >= 64) {
      wbase += 64;
      ++wk;
      // Window wk's copy was issued 64 list positions (at least 32 chunks) ago, and every
      // chunk since was computed after waiting for all loads older than the newest chunk's,
      // so it has landed: no wait here (a vmcnt(0) would also drain the MFMA form's other
      // chunk); the empty asm only keeps the compiler from reading the slice earlier.
      asm volatile("" ::: "memory");
      tab = s_tab[wave][wk & 1][lane];
      if (wbase + 64 < end) fetch_window(wbase + 64, b, (wk + 1) & 1);
    }
    return __builtin_amdgcn_readlane(tab, (int)(e - wbase));
  };

  // current piece: list positions [pos, pend) of segment (b, g), blocks j0 .. j1-1
  int64_t seg0 = (int64_t)Hkv * s_pre[b] + (int64_t)g * nv;
  int64_t pend = min(end, seg0 + nv);
  int j0 = (int)(pos0 - seg0), j1 = (int)(pend - seg0);
  int ctx = decode_ctx(ctx_lens, b, max_ctx, max_blocks, BS);
  int hi = min(j1 * BS, ctx);

  W w;
  w.init(lane);
  // MFMA form: the SIMD's issue arbiter favours older waves, so the workgroup dispatched first
  // on a CU streams faster than the second one (INT8 70B-shaped decode: ~161 against ~180 us to
  // finish the same work). The second half of the grid (the later workgroups) holds priority 1
  // for 3 of every 4 chunks, the first half for the remaining one: with equal shares (a flip
  // every 4 chunks) the earlier workgroups still end ~7 us first; 3 of 4 (or 5 of 8) evens them
  // out best (7 of 8 and always-high overshoot).
  const bool late = blockIdx.x >= gridDim.x / 2;
  int prio = W::kMfmaPv && late ? 1 : 0, nchunk = 0;
  if (prio) __builtin_amdgcn_s_setprio(1);
  typename W::Chunk cA;
  auto prep = [&](typename W::Chunk& c, int j, int slot) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = j + u < j1 ? entry(seg0 + j + u) : -1;
      c.okb[u] = e >= 0 && e < num_blocks;  // unusable entry: its tokens are skipped
      c.pb[u] = c.okb[u] ? e : 0;
    }
    c.t0 = j * BS;
    w.load(c, k_cache, v_cache, k_scale, v_scale, Hk, gk, s_lds[wave][slot]);
    if (W::kMfmaPv) {  // the later workgroups high for 3 chunks of 4, the earlier for 1 of 4
      const int want = (((++nchunk) & 3) != 0) == late ? 1 : 0;
      if (want != prio) {
        prio = want;
        if (prio) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
      }
    }
  };

  w.load_q(q, b, g, G, QL, Hq, ctx, 0);
  w.reset();
  prep(cA, j0, 0);
  const int ncol = G * QL;
  while (true) {
    // ---- the chunks of the piece; cA holds the first one's loads --------------------------
    if constexpr (W::kMfmaPv) {
      // two chunks in flight: the next chunk's loads are issued before this one is computed
      typename W::Chunk cB;
      for (int j = j0;; j += 2 * U) {
        const bool nb = j + U < j1;
        if (nb) prep(cB, j + U, 1);
        w.compute(cA, 0, hi, scale_log2, s_lds[wave][0], nb);
        if (!nb) break;
        const bool na = j + 2 * U < j1;
        if (na) prep(cA, j + 2 * U, 0);
        w.compute(cB, 0, hi, scale_log2, s_lds[wave][1], na);
        if (!na) break;
      }
    } else {
      for (int j = j0;; j += U) {
        if (j > j0) prep(cA, j, 0);
        w.compute(cA, 0, hi, scale_log2, s_lds[wave][0]);
        if (j + U >= j1) break;
      }
    }

    // ---- the next piece's Q and first chunk are issued before this one is written out -----
    const int ob = b, og = g;
    const bool whole = j0 == 0 && j1 == nv;
    const bool more = pend < end;
    if (more) {
      if (++g == Hkv) {  // next sequence with visible blocks (one exists: pend < T)
        g = 0;
        do ++b; while (b < B - 1 && s_pre[b + 1] == s_pre[b]);
        nv = s_pre[b + 1] - s_pre[b];
        ctx = decode_ctx(ctx_lens, b, max_ctx, max_blocks, BS);
      }
      gk = VIRT ? g / R : g;
      seg0 = pend;
      pend = min(end, seg0 + nv);
      j0 = 0;
      j1 = (int)(pend - seg0);
      hi = min(j1 * BS, ctx);
      w.load_q(q, b, g, G, QL, Hq, ctx, 0);
      prep(cA, 0, 0);
    }

    float l_w, ps_w;
    w.reduce(l_w, ps_w);
    const int64_t slot = (int64_t)ob * Hkv + og + p;
    // column h's row sum and max: lane h holds them (both lane layouts)
    float lcol[GP], mcol[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      lcol[h] = __shfl(l_w, h);
      mcol[h] = __shfl(w.m_run, h);
    }
    // column h: query row h / G, head g*G + h % G; v holds d0 .. d0 + N - 1
    w.emit([&](int h, int d0, const auto& v) {
      constexpr int N = sizeof(v) / sizeof(v[0]);
      if (h >= ncol) return;
      float lh, mh;
      if constexpr (W::kMfmaPv) {  // h is this lane's own column
        lh = l_w;
        mh = w.m_run;
      } else {
        lh = lcol[h];
        mh = mcol[h];
      }
      const float inv = lh > 0.f ? 1.0f / lh : 0.f;
      if (whole) {
        uint32_t o2[N / 2];
#pragma unroll
        for (int e = 0; e < N / 2; ++e) o2[e] = pack_bf16x2(v[2 * e] * inv, v[2 * e + 1] * inv);
        const int64_t orow = ((int64_t)ob * QL + h / G) * Hq + og * G + h % G;
        uint16_t* dst = out + orow * D + d0;
        if constexpr (N == 8)
          *reinterpret_cast<u32x4*>(dst) = (u32x4){o2[0], o2[1], o2[2], o2[3]};
        else
          *reinterpret_cast<u32x2*>(dst) = (u32x2){o2[0], o2[1]};
      } else {
        float* po = part_o + ((slot * ncol + h) * D + d0);
#pragma unroll
        for (int e = 0; e < N; e += 4)
          *reinterpret_cast<f32x4*>(po + e) = (f32x4){v[e] * inv, v[e + 1] * inv, v[e + 2] * inv, v[e + 3] * inv};
        if (d0 == 0) part_lse[slot * ncol + h] = lh > 0.f ? mh + __log2f(lh) : -INFINITY;
      }
    });
    if (!more) break;
    w.reset();
  }
}

// Merge for the balanced shape: column hl of KV head g of sequence b gathers the pieces of
// segment s = (b, g) from slots s + p0 .. s + p1; a segment held by one wave was written
// directly. One wave per column and kMergeCols columns per workgroup: an eighth of the
// workgroups that one column each would need (C3 -0.6 us, measured).
constexpr int kMergeCols = 8;
template <int D>
__global__ __launch_bounds__(64 * kMergeCols) void decode_stream_merge_kernel(
    const int32_t* __restrict__ prefix, const float* __restrict__ part_o,
    const float* __restrict__ part_lse, uint16_t* __restrict__ out, int B, int Hq, int Hkv,
    int G, int QL, int P) {
  const int ncol = G * QL;
  const int c = blockIdx.x * kMergeCols + (threadIdx.x >> 6);  // one column per wave
  if (c >= Hkv * ncol) return;
  const int g = c / ncol, hl = c % ncol, b = blockIdx.y;  // column hl of g
  const int nv = prefix[b + 1] - prefix[b];
  uint16_t* orow = out + (((int64_t)b * QL + hl / G) * Hq + g * G + hl % G) * D;
  if (nv == 0) {  // empty context: zeros
#pragma unroll
    for (int e = 0; e < D / 64; ++e) orow[(threadIdx.x & 63) + 64 * e] = 0;
    return;
  }
  const int64_t T = (int64_t)Hkv * prefix[B];
  const int64_t qn = (T + P - 1) / P;
  const int64_t seg0 = (int64_t)Hkv * prefix[b] + (int64_t)g * nv;
  const int64_t p0 = seg0 / qn, p1 = (seg0 + nv - 1) / qn;
  if (p0 == p1) return;
  const int64_t s = (int64_t)b * Hkv + g;
  merge_partials<D>(part_o, part_lse, (s + p0) * ncol + hl, ncol, (int)(p1 - p0 + 1), orow);
}

static int pow2_at_least(int g) {
  int p = 1;
  while (p < g) p <<= 1;
  return p;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return 256;  // MI355X
  }
  return cus;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodePlan plan_decode(int B, int QL, int Hq, int Hkv, int D, int max_context_len, int window,
                       int split_tokens) {
  DecodePlan p{};
  // keys the QL query rows of one sequence can attend to (block-rounded)
  const int span = window > 0 ? std::min(max_context_len, window + QL - 1 + 15) : max_context_len;
  const int ncol = (Hq / Hkv) * QL;  // query columns per (sequence, KV head)
  if (split_tokens == 0 && window == 0 && B <= kStreamMaxB) {
    // balanced shape (no window: context lengths, and so the work per sequence, can be
    // arbitrarily ragged): at most one wave per list entry and two 4-wave workgroups per CU.
    // Every wave gets the same amount of work, so the workgroup count must be a whole multiple
    // of the CU count; of 1, 2, 3, 4 and 8 workgroups per CU, 2 streams fastest (longer
    // ranges per wave mean fewer partials to write and merge, and the 8 waves still keep
    // enough loads in flight)
    const int64_t max_entries = (int64_t)B * Hkv * ((span + 15) / 16 + 1);
    const int64_t waves = std::min<int64_t>((int64_t)device_cus() * 8, max_entries);
    p.stream = true;
    p.stream_waves_max = (int)std::max<int64_t>(kDecodeWaves, waves);
    const size_t slots = (size_t)B * Hkv + p.stream_waves_max;
    p.prefix_off = 0;
    p.part_o_off = align256((size_t)(B + 1) * sizeof(int32_t));
    p.part_lse_off = p.part_o_off + align256(slots * ncol * D * sizeof(float));
    p.workspace_bytes = p.part_lse_off + slots * ncol * sizeof(float);
    return p;
  }
  int C = split_tokens;
  if (C == 0) {
    // fixed splits chosen by the library (a window bounds every sequence's span, or the batch
    // is too large for the balanced shape): 2048-token splits for long spans, else a quarter of
    // the span rounded to 256 within [256, 1024] (measured on MI355X)
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
    const size_t parts = (size_t)B * Hkv * ncol * p.n_split;
    p.part_o_off = 0;
    p.part_lse_off = align256(parts * D * sizeof(float));
    p.workspace_bytes = p.part_lse_off + parts * sizeof(float);
  }
  return p;
}

template <int D, int GP, int KV, bool VIRT>
static void launch_stream(const DecodeArgs& a, hipStream_t stream) {
  const auto kern = decode_stream_kernel<D, GP, KV, VIRT>;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kDecodeThreads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int wgs = std::max(1, std::min(device_cus() * per_cu, a.plan.stream_waves_max / kDecodeWaves));
  char* ws = reinterpret_cast<char*>(a.workspace);
  int32_t* prefix = reinterpret_cast<int32_t*>(ws + a.plan.prefix_off);
  float* part_o = reinterpret_cast<float*>(ws + a.plan.part_o_off);
  float* part_lse = reinterpret_cast<float*>(ws + a.plan.part_lse_off);
  const int G = a.Hq / a.Hkv;
  hipLaunchKernelGGL(kern, dim3(wgs), dim3(kDecodeThreads), 0, stream, (const uint16_t*)a.q,
                     a.k_cache, a.v_cache, (const __half*)a.k_scale, (const __half*)a.v_scale,
                     a.block_table, a.context_lens, (uint16_t*)a.o, prefix, part_o, part_lse, a.B,
                     a.Hq, a.Hkv, G, a.q_len, a.max_blocks_per_seq, a.num_blocks,
                     a.max_context_len, a.scale * kLog2e, a.kv_rep);
  const int merge_wgs = (a.Hkv * G * a.q_len + kMergeCols - 1) / kMergeCols;
  hipLaunchKernelGGL(decode_stream_merge_kernel<D>, dim3(merge_wgs, a.B), dim3(64 * kMergeCols), 0,
                     stream, prefix, part_o, part_lse, (uint16_t*)a.o, a.B, a.Hq, a.Hkv, G,
                     a.q_len, wgs * kDecodeWaves);
}

template <int D, int GP, int KV, bool VIRT>
static void launch_split(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int C = a.plan.split_tokens, ns = a.plan.n_split;
  char* ws = reinterpret_cast<char*>(a.workspace);
  float* part_o = ns > 1 ? reinterpret_cast<float*>(ws + a.plan.part_o_off) : nullptr;
  float* part_lse = ns > 1 ? reinterpret_cast<float*>(ws + a.plan.part_lse_off) : nullptr;
  hipLaunchKernelGGL((decode_split_kernel<D, GP, KV, VIRT>), dim3(a.Hkv, a.B, ns), dim3(kDecodeThreads),
                     0, stream, (const uint16_t*)a.q, a.k_cache, a.v_cache,
                     (const __half*)a.k_scale, (const __half*)a.v_scale, a.block_table,
                     a.context_lens, (uint16_t*)a.o, part_o, part_lse, a.Hq, a.Hkv, G, a.q_len,
                     a.max_blocks_per_seq, a.num_blocks, a.max_context_len, a.scale * kLog2e,
                     a.window, C, ns, a.kv_rep);
  if (ns > 1)
    hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(a.Hq, a.B * a.q_len), dim3(64), 0, stream,
                       part_o, part_lse, a.context_lens, (uint16_t*)a.o, a.Hq, a.q_len,
                       a.max_blocks_per_seq, a.max_context_len, a.window, C, ns);
}

template <int D, int GP, int KV>
static void launch_shape(const DecodeArgs& a, hipStream_t stream) {
  if (a.kv_rep > 1) {  // virtual KV heads
    if (a.plan.stream)
      launch_stream<D, GP, KV, true>(a, stream);
    else
      launch_split<D, GP, KV, true>(a, stream);
    return;
  }
  if (a.plan.stream)
    launch_stream<D, GP, KV, false>(a, stream);
  else
    launch_split<D, GP, KV, false>(a, stream);
}

template <int D, int KV>
static void launch_g(const DecodeArgs& a, hipStream_t stream) {
  switch (pow2_at_least(a.Hq / a.Hkv * a.q_len)) {  // MFMA columns: (query row, head) pairs
    case 1: launch_shape<D, 1, KV>(a, stream); break;
    case 2: launch_shape<D, 2, KV>(a, stream); break;
    case 4: launch_shape<D, 4, KV>(a, stream); break;
    case 8: launch_shape<D, 8, KV>(a, stream); break;
    default: launch_shape<D, 16, KV>(a, stream); break;
  }
}

template <int D>
static void launch_kv(const DecodeArgs& a, hipStream_t stream) {
  switch (a.kv) {
    case kKvI8: launch_g<D, kKvI8>(a, stream); break;
    case kKvFp8: launch_g<D, kKvFp8>(a, stream); break;
    default: launch_g<D, kKvBf16>(a, stream); break;
  }
}

int launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.D == 64)
    launch_kv<64>(a, stream);
  else
    launch_kv<128>(a, stream);
  return 0;
}

}  // namespace attn
