// fp32 tiled prefill attention with an online softmax (VALU path).
//
// Same method as the bf16 kernel (the Tiny-Infer page, "从零构建CUDA推理引擎：Tiny-Infer项目的技术深度解析",
// section "Flash Attention：内存与计算的重平衡": blocks of keys staged on chip, online softmax,
// the score matrix never stored) for fp32 tensors, where gfx950 has no bf16-rate matrix
// instruction that keeps full fp32 accuracy. It serves small fp32 problems, which are launch-
// latency bound; each thread owns D/64 x 64 elements of one query row, the K/V tile sits in
// LDS and is read by broadcast.
#include "common.h"
#include "launch.h"

namespace attn {

constexpr int kF32Threads = 64;
constexpr int kF32BN = 32;

template <int D>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int S, int Hq, int Hkv, int G, int n_qblk,
    float scale_log2, int causal, int window) {
  constexpr int TPR = D / 64;             // threads per query row
  constexpr int ROWS = kF32Threads / TPR;  // query rows per workgroup
  __shared__ float ks[kF32BN][D];
  __shared__ float vs[kF32BN][D];

  const int tid = threadIdx.x;
  const int part = tid % TPR;  // which 64-wide slice of d this thread owns
  const int rloc = tid / TPR;
  int id = blockIdx.x;
  const int qblk_rank = id % n_qblk;
  id /= n_qblk;
  const int h = id % Hq;
  const int b = id / Hq;
  const int g = h / G;
  const int qblk = causal ? (n_qblk - 1 - qblk_rank) : qblk_rank;
  const int q0 = qblk * ROWS;
  const int qp = q0 + rloc;
  const bool live = qp < S;

  float qv[64], acc[64];
  const float* qrow = q + (((int64_t)b * S + (live ? qp : 0)) * Hq + h) * D + 64 * part;
#pragma unroll
  for (int d = 0; d < 64; ++d) {
    qv[d] = live ? qrow[d] : 0.f;
    acc[d] = 0.f;
  }
  float m_run = kNegBig, l_run = 0.f;

  const int q_last = min(S - 1, q0 + ROWS - 1);
  const int kmin = window > 0 ? max(0, q0 - window + 1) : 0;
  const int kmax = causal ? q_last : S - 1;
  const int64_t kstride = (int64_t)Hkv * D;
  const float* kb = k + ((int64_t)b * S * Hkv + g) * D;
  const float* vb = v + ((int64_t)b * S * Hkv + g) * D;

  for (int k0 = (kmin / kF32BN) * kF32BN; k0 <= kmax; k0 += kF32BN) {
    __syncthreads();
    for (int i = tid; i < kF32BN * D; i += kF32Threads) {
      const int key = i / D, d = i % D;
      const bool in = k0 + key < S;
      ks[key][d] = in ? kb[(k0 + key) * kstride + d] : 0.f;
      vs[key][d] = in ? vb[(k0 + key) * kstride + d] : 0.f;
    }
    __syncthreads();
    float s[kF32BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < 64; ++d) dot = fmaf(qv[d], ks[j][64 * part + d], dot);
      if (TPR == 2) dot += __shfl_xor(dot, 1);
      const int key = k0 + j;
      bool vis = key < S;
      if (causal) vis = vis && key <= qp;
      if (window > 0) vis = vis && qp - key < window;
      s[j] = vis ? dot * scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      s[j] = fast_exp2(s[j] - m_new);
      rs += s[j];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 64; ++d) {
      float a = acc[d] * alpha;
#pragma unroll
      for (int j = 0; j < kF32BN; ++j) a = fmaf(s[j], vs[j][64 * part + d], a);
      acc[d] = a;
    }
  }
  if (live) {
    const float inv = 1.0f / l_run;
    float* orow = o + (((int64_t)b * S + qp) * Hq + h) * D + 64 * part;
#pragma unroll
    for (int d = 0; d < 64; ++d) orow[d] = acc[d] * inv;
    if (lse != nullptr && part == 0) lse[((int64_t)b * Hq + h) * S + qp] = (m_run + __log2f(l_run)) * kLn2;
  }
}

int launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int rows = kF32Threads / (a.D / 64);
  const int n_qblk = (a.S + rows - 1) / rows;
  const long long nwg = (long long)a.B * a.Hq * n_qblk;
  const float scale_log2 = a.scale * kLog2e;
  if (a.D == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)nwg), dim3(kF32Threads), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                       a.S, a.Hq, a.Hkv, G, n_qblk, scale_log2, a.causal, a.window);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)nwg), dim3(kF32Threads), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                       a.S, a.Hq, a.Hkv, G, n_qblk, scale_log2, a.causal, a.window);
  return 0;
}

}  // namespace attn
