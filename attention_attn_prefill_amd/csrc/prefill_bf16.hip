// Tiled causal / sliding-window prefill attention, bf16 in, fp32 accumulate, on gfx950 MFMA.
//
// Pages (title, section): the Tiny-Infer page ("从零构建CUDA推理引擎：Tiny-Infer项目的技术深度解析"),
// "Flash Attention：内存与计算的重平衡" -- split the sequence into blocks, run a local softmax in
// on-chip memory with an online softmax so the N x N score matrix is never stored, one thread
// block per (head, query block), partial results accumulated on chip; the KDnuggets page
// ("5 Fun Projects for LLM Inference Engineering"), project 2 -- the gain comes from moving
// less data between HBM and on-chip memory, not from doing less math; the inference-lab page
// ("从零开始的LLM推理优化实验室：从PyTorch基线到Triton内核的完整实践"), "KV缓存实验与长上下文优化" --
// sliding-window attention.
//
// gfx950 design:
//  * A workgroup is 4 waves; a wave owns 32 query rows of one head. The waves of a workgroup
//    are the query heads that share one KV head (GQA) and/or consecutive 32-row chunks, so one
//    K/V tile in LDS serves 128 query rows.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16: A = 32 keys of
//    the K tile (LDS, [key][d] rows), B = Q^T held in registers for the whole kernel. In the
//    accumulator each lane then owns one query column, so the row max / row sum are in-lane
//    reductions plus one exchange between the two 32-lane halves.
//  * P^T (bf16) goes straight from the score accumulator into the B operand of the PV MFMA,
//    O^T += V^T P^T; V is stored transposed in LDS ([d][key]) with the key slots of every
//    16-key group permuted so that each lane's 8 keys are contiguous (one 16-byte LDS read).
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are in flight while
//    the current one is computed; one barrier per tile.
//  * Tiles entirely hidden by the causal mask or the window are never visited; the mask is
//    applied only on tiles that straddle an edge. exp2 with scale*log2(e) folded into one FMA.
#include "common.h"
#include "launch.h"
#include <type_traits>

namespace attn {

constexpr int kPrefillThreads = 256;
constexpr int kBN = 64;  // keys per tile
// The running max lags the true max by at most this much (log2 units), so probabilities stay
// below 2^kRescaleSlack; O and l share the same reference, so o = O / l is unchanged.
constexpr float kRescaleSlack = 8.0f;

// max / sum over lanes l and l ^ 32 (the two halves of a 32x32 accumulator column)
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct PrefillTile {
  static constexpr int KPAD = D + 8;      // K row pitch in LDS (elements)
  static constexpr int VPAD = kBN + 8;    // V^T row pitch in LDS (elements)
  static constexpr int K_ELEMS = kBN * KPAD;
  static constexpr int V_ELEMS = D * VPAD;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int K_CHUNKS = kBN * D / 8;          // 16-byte chunks of a K tile
  static constexpr int K_PER_THREAD = K_CHUNKS / kPrefillThreads;
  static constexpr int V_ITEMS = (kBN / 4) * (D / 8);   // 4 keys x 8 d items of a V tile
};

// Slot of key offset o (0..15) inside its 16-key group of a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_slot(int o) {
  return (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1);
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int S,
    int Hq, int Hkv, int G, int HW, int QW, int n_qblk, int n_hsub, float scale_log2,
    int causal, int window) {
  using T = PrefillTile<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31;  // query column inside the wave's 32 rows
  const int half = lane >> 5;

  // ---- workgroup -> (b, kv head, head sub-group, query block); longest blocks first --------
  int id = blockIdx.x;
  const int qblk_rank = id % n_qblk;
  id /= n_qblk;
  const int hsub = id % n_hsub;
  id /= n_hsub;
  const int g = id % Hkv;
  const int b = id / Hkv;
  const int qblk = causal ? (n_qblk - 1 - qblk_rank) : qblk_rank;

  const int rows = 32 * QW;
  const int q0 = qblk * rows;
  const int head = g * G + hsub * HW + (wave % HW);
  const int q0w = q0 + 32 * (wave / HW);

  // key range of the workgroup and of this wave
  const int q_last = min(S - 1, q0 + rows - 1);
  const int kmin = window > 0 ? max(0, q0 - window + 1) : 0;
  const int kmax = causal ? q_last : S - 1;
  const int jlo = kmin / kBN, jhi = kmax / kBN;
  const bool wave_live = q0w < S;
  const int qw_last = min(S - 1, q0w + 31);
  const int kmin_w = window > 0 ? max(0, q0w - window + 1) : 0;
  const int kmax_w = causal ? qw_last : S - 1;

  // ---- Q^T fragments (B operand), kept in registers --------------------------------------
  constexpr int QSTEPS = D / 16;
  bf16x8 qf[QSTEPS];
  {
    const int qr = q0w + col;
    const uint16_t* qrow = q + (((int64_t)b * S + qr) * Hq + head) * D;
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qr < S) w = *reinterpret_cast<const u32x4*>(qrow + 16 * t + 8 * half);
      qf[t] = __builtin_bit_cast(bf16x8, w);
    }
  }

  constexpr int DB = D / 32;
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = kNegBig, l_run = 0.f;

  // ---- global -> register staging of one K/V tile ---------------------------------------
  const int64_t kv_row_stride = (int64_t)Hkv * D;  // elements between consecutive keys
  const uint16_t* kbase = k + ((int64_t)b * S * Hkv + g) * D;
  const uint16_t* vbase = v + ((int64_t)b * S * Hkv + g) * D;
  u32x4 kst[T::K_PER_THREAD];
  u32x4 vst[4];
  const bool v_thread = tid < T::V_ITEMS;
  const int v_kq = tid / (D / 8), v_dc = tid % (D / 8);

  auto load_tile = [&](int j) {
    const int k0 = j * kBN;
#pragma unroll
    for (int i = 0; i < T::K_PER_THREAD; ++i) {
      const int id2 = tid + kPrefillThreads * i;
      const int key = id2 / (D / 8), dc = id2 % (D / 8);
      u32x4 w = {0u, 0u, 0u, 0u};
      if (k0 + key < S) w = *reinterpret_cast<const u32x4*>(kbase + (k0 + key) * kv_row_stride + 8 * dc);
      kst[i] = w;
    }
    if (v_thread) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * v_kq + r;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key < S) w = *reinterpret_cast<const u32x4*>(vbase + key * kv_row_stride + 8 * v_dc);
        vst[r] = w;
      }
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* ks = smem + stage * T::STAGE;
    uint16_t* vs = ks + T::K_ELEMS;
#pragma unroll
    for (int i = 0; i < T::K_PER_THREAD; ++i) {
      const int id2 = tid + kPrefillThreads * i;
      const int key = id2 / (D / 8), dc = id2 % (D / 8);
      *reinterpret_cast<u32x4*>(ks + key * T::KPAD + 8 * dc) = kst[i];
    }
    if (v_thread) {
      const int kk = 4 * v_kq;  // first key of the quad inside the tile
      const int slot = (kk & ~15) + vt_slot(kk & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 pr;
        pr[0] = __builtin_amdgcn_perm(vst[1][wi], vst[0][wi], sel);
        pr[1] = __builtin_amdgcn_perm(vst[3][wi], vst[2][wi], sel);
        *reinterpret_cast<u32x2*>(vs + (8 * v_dc + e) * T::VPAD + slot) = pr;
      }
    }
  };

  if (jlo <= jhi) {
    load_tile(jlo);
    store_tile(0);
  }
  __syncthreads();

  // One tile step for this wave. MASK selects the edge-tile variant (causal diagonal, window
  // edge or the ragged end of the sequence); interior tiles skip all mask arithmetic.
  auto tile_step = [&](const uint16_t* ks, const uint16_t* vs, int k0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // S^T = K Q^T
    f32x16 sacc[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int t = 0; t < QSTEPS; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (32 * kb + col) * T::KPAD + 16 * t + 8 * half);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], sacc[kb], 0, 0, 0);
      }
    }
    if constexpr (MASK) {
      // register r of block kb holds key offset 32*kb + 8*(r/4) + (r%4) + 4*half of the tile
      const int qp = q0w + col;
      int hi = S - 1 - k0;
      if (causal) hi = min(hi, qp - k0);
      const int lo_off = window > 0 ? qp - window + 1 - k0 : -(1 << 30);
      const int hi4 = hi - 4 * half, lo4 = lo_off - 4 * half;
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
          if (off > hi4 || off < lo4) sacc[kb][r] = -INFINITY;
        }
    }
    // online softmax in the log2 domain; the running max is only moved (and the accumulator
    // rescaled) when some row's max grows by more than kRescaleSlack, so most tiles skip it.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = xhalf_max(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    float rs = 0.f;
    bf16x8 pf[kBN / 16];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(sacc[kb][r], scale_log2, -m_run));
        const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], scale_log2, -m_run));
        rs += p0 + p1;
        const bf16x2 pp = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
        pf[2 * kb + (r >> 3)][r & 7] = pp[0];
        pf[2 * kb + (r >> 3)][(r & 7) + 1] = pp[1];
      }
    l_run += xhalf_sum(rs);
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < kBN / 16; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + (32 * db + col) * T::VPAD + 16 * u + 8 * half);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[u], oacc[db], 0, 0, 0);
      }
  };

  for (int j = jlo; j <= jhi; ++j) {
    const int st = (j - jlo) & 1;
    if (j < jhi) load_tile(j + 1);

    const int k0 = j * kBN;
    const bool relevant = wave_live && k0 <= kmax_w && k0 + kBN - 1 >= kmin_w;
    if (relevant) {
      const uint16_t* ks = smem + st * T::STAGE;
      const uint16_t* vs = ks + T::K_ELEMS;
      const bool full = (!causal || k0 + kBN - 1 <= q0w) &&
                        (window == 0 || qw_last - k0 < window) && (k0 + kBN <= S);
      if (full)
        tile_step(ks, vs, k0, std::false_type{});
      else
        tile_step(ks, vs, k0, std::true_type{});
    }

    if (j < jhi) store_tile(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, bf16 RNE ---------------------------------------------------
  const int qr = q0w + col;
  if (wave_live && qr < S) {
    const float inv = 1.0f / l_run;
    uint16_t* orow = o + (((int64_t)b * S + qr) * Hq + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * half;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    if (lse != nullptr && half == 0)
      lse[((int64_t)b * Hq + head) * S + qr] = (m_run + __log2f(l_run)) * kLn2;
  }
}

int launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;  // heads per workgroup
  const int QW = 4 / HW;                                    // 32-row chunks per head
  const int rows = 32 * QW;
  const int n_qblk = (a.S + rows - 1) / rows;
  const int n_hsub = G / HW;
  const long long nwg = (long long)a.B * a.Hkv * n_hsub * n_qblk;
  const float scale_log2 = a.scale * kLog2e;
  if (a.D == 64) {
    const size_t lds = 2 * PrefillTile<64>::STAGE * sizeof(uint16_t);
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3((unsigned)nwg), dim3(kPrefillThreads), lds,
                       stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, a.S, a.Hq, a.Hkv, G, HW, QW, n_qblk, n_hsub,
                       scale_log2, a.causal, a.window);
  } else {
    const size_t lds = 2 * PrefillTile<128>::STAGE * sizeof(uint16_t);
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3((unsigned)nwg), dim3(kPrefillThreads), lds,
                       stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, a.S, a.Hq, a.Hkv, G, HW, QW, n_qblk, n_hsub,
                       scale_log2, a.causal, a.window);
  }
  return 0;
}

}  // namespace attn
