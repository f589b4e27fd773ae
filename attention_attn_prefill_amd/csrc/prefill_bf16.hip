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
//  * K and V tiles (64 keys at D=64, 32 at D=128) move from global memory straight into LDS with
//    global_load_lds_dwordx4 (no register staging), double-buffered: the next tile's loads are
//    in flight while the current tile is computed; one barrier per tile. Both tiles keep their
//    natural [key][d] rows; 16-byte chunks are XOR-swizzled by key so the MFMA operand reads
//    below are free of LDS bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16: A = 32 keys of
//    the K tile, B = Q^T held in registers for the whole kernel. Each lane then owns one query
//    column, so the row max / row sum are in-lane reductions plus one exchange between the two
//    32-lane halves (v_permlane32_swap).
//  * P^T (bf16) goes straight from the score accumulator into the B operand of the PV MFMA,
//    O^T += V^T P^T. The V^T operand is read from the natural V tile with ds_read_b64_tr_b16
//    (each lane receives 4 consecutive keys of one d), addressed so that its keys line up with
//    the keys the score accumulator put in the same lane.
//  * Tiles hidden by the causal mask or the window from every row of the workgroup are never
//    visited; the mask is applied only on tiles that straddle an edge of the wave's rows (or lie
//    outside them, when another wave of the workgroup needs the tile). exp2 with
//    scale*log2(e) folded into one FMA;
//    the running max moves only when it grows by more than kRescaleSlack.
#include "common.h"
#include "launch.h"
#include "prefill_tile.h"
#include <atomic>
#include <type_traits>

namespace attn {

// Paged mode (chunked prefill): queries are packed rows, sequence b owning rows
// cu_q[b] .. cu_q[b+1]-1, which are the last positions of its ctx[b] keys (bottom-right
// alignment); K/V come from the paged cache through the block table. With k_new / v_new the
// chunk's own K/V rows (packed like the queries) are written into the cache by the same
// launch, and the chunk's keys are read from those rows rather than from the slots being
// written, so no workgroup depends on another's writes.
struct PagedArgs {
  const int32_t* cu_q;
  const int32_t* ctx;
  const int32_t* table;
  int max_blocks, num_blocks;
  const uint16_t* k_new;  // [total_q][Hkv][D] or null
  const uint16_t* v_new;
  uint16_t* k_cache;  // the caches again, for the chunk's slots (written, never read here)
  uint16_t* v_cache;
  // > 0: fixed_q rows per sequence, no cu_q; a row whose position ctx - fixed_q + i is
  // negative sees no key and is written as zeros (multi-row decode semantics)
  int fixed_q;
};

template <int D, bool PAGED>
__global__ __launch_bounds__(kPrefillThreads, D == 128 ? 3 : 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int S,
    int Hq, int Hkv, int G, int HW, int QW, int n_qblk, int n_hsub, float scale_log2,
    int causal, int window, int cpx, int gmajor, PagedArgs pg) {
  using T = PTile<D>;
  constexpr int kBN = T::BN;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query column inside the wave's 32 rows
  const int half = lane >> 5;

  // ---- workgroup -> (b, kv head, head sub-group, query block) -----------------------------
  // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each with its own L2.
  // When the number of (b, kv head, head sub-group) groups is a multiple of 8, group gi runs
  // entirely on XCD gi % 8, so its K/V stream is fetched into one L2 and reused there. An XCD
  // holding several groups interleaves their query blocks when the whole grid is resident at
  // once, and runs the groups one after the other (gmajor) when it is not, so that the keys its
  // resident query blocks need at once are one group's band, not several (long-context window
  // prefill: 2.05 -> 0.74 GB read per call, same time; with the grid resident, interleaving is
  // 4 % faster on the chunked prefill). The query blocks go longest first, dealt to the XCD's
  // CUs in rounds of `cpx` slots whose direction alternates (round r takes ranks rC .. rC+C-1
  // forwards when r is even, backwards when odd). When the whole grid is resident at once, the
  // CU that receives the longest block of one round receives the shortest of the next, so
  // every CU's causal work sums to about the same.
  const int n_groups = gridDim.x / n_qblk;
  int gi, qblk_rank;
  if ((n_groups & 7) == 0) {
    const int xcd = blockIdx.x & 7, slot0 = blockIdx.x >> 3;
    const int round = slot0 / cpx, pos = slot0 % cpx;
    const int len = min(cpx, (int)(gridDim.x >> 3) - round * cpx);  // last round may be short
    const int slot = round * cpx + ((round & 1) ? len - 1 - pos : pos);
    if (gmajor) {
      qblk_rank = slot % n_qblk;
      gi = xcd + 8 * (slot / n_qblk);
    } else {
      const int per_xcd = n_groups >> 3;
      qblk_rank = slot / per_xcd;
      gi = xcd + 8 * (slot % per_xcd);
    }
  } else {
    qblk_rank = blockIdx.x % n_qblk;
    gi = blockIdx.x / n_qblk;
  }
  const int hsub = gi % n_hsub;
  const int g = (gi / n_hsub) % Hkv;
  const int b = gi / (n_hsub * Hkv);
  const int qblk = causal ? (n_qblk - 1 - qblk_rank) : qblk_rank;

  // Sq query rows at positions off + r against Lk keys (contiguous: Sq = Lk = S, off = 0)
  int Sq = S, Lk = S, q_row0 = b * S;
  if constexpr (PAGED) {
    Lk = min(max(pg.ctx[b], 0), pg.max_blocks * 16);
    if (pg.fixed_q > 0) {
      q_row0 = b * pg.fixed_q;
      Sq = pg.fixed_q;
    } else {
      q_row0 = pg.cu_q[b];
      Sq = min(pg.cu_q[b + 1] - q_row0, Lk);  // rows past the context are not computed
    }
  }
  const int off = Lk - Sq;  // negative only with fixed_q rows that precede the sequence
  const int rows = 32 * QW;
  const int q0 = qblk * rows;
  if (q0 >= Sq) return;  // whole workgroup: nothing to do for this sequence
  const int head = g * G + hsub * HW + (wave % HW);
  const int q0w = q0 + 32 * (wave / HW);

  // key range of the workgroup and of this wave (positions)
  const int q_last = min(Sq - 1, q0 + rows - 1);
  const int kmin = window > 0 ? max(0, off + q0 - window + 1) : 0;
  const int kmax = causal ? off + q_last : Lk - 1;
  const int jlo = kmin / kBN, jhi = kmax / kBN;
  const bool wave_live = q0w < Sq;
  const int qw_last = min(Sq - 1, q0w + 31);

  // ---- Q^T fragments (B operand), kept in registers --------------------------------------
  constexpr int QSTEPS = D / 16;
  bf16x8 qf[QSTEPS];
  {
    const int qr = q0w + col;
    const uint16_t* qrow = q + (((int64_t)q_row0 + qr) * Hq + head) * D;
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qr < Sq) w = *reinterpret_cast<const u32x4*>(qrow + 16 * t + 8 * half);
      qf[t] = __builtin_bit_cast(bf16x8, w);
    }
  }

  constexpr int DB = D / 32;
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
    oacc[i] = (f32x16){};
  float m_run = kNegBig, l_run = 0.f;
  float m_thr = kNegBig + kRescaleSlack;  // rescale when a tile's max exceeds this

  // ---- direct global -> LDS tile loads ---------------------------------------------------
  // Wave instruction n (of INSTR per tile) writes LDS bytes [1024n, 1024n + 1024) of the tile;
  // this wave issues n = wave + 4i. Lane l fills LDS row r = n*ROWS_PER_INSTR + l / CHUNKS,
  // swizzled chunk l % CHUNKS, i.e. global chunk (l % CHUNKS) ^ swz(r). The swizzles depend on
  // r only through bits that are the same for every i, so each lane has one fixed chunk.
  const int ld_row0 = wave * T::ROWS_PER_INSTR + lane / T::CHUNKS;
  const int ld_kchunk = (lane % T::CHUNKS) ^ k_swz<D>(ld_row0);
  const int ld_vchunk = (lane % T::CHUNKS) ^ v_swz<D>(ld_row0);
  constexpr int ROW_STEP = 4 * T::ROWS_PER_INSTR;  // rows between this wave's instructions
  const int64_t kv_row_stride = (int64_t)Hkv * D;
  const uint16_t* kbase = k + ((int64_t)b * S * Hkv + g) * D;
  const uint16_t* vbase = v + ((int64_t)b * S * Hkv + g) * D;
  // Contiguous: a load instruction's first row gives a wave-uniform base (SGPRs, advanced by
  // scalar arithmetic per tile) and the lane adds a fixed byte offset (its row within the
  // instruction and its chunk). Paged: one 1 KB load instruction stays inside one 16-key block
  // (16 is a multiple of the rows per instruction), so its block comes from one wave-uniform
  // table lookup; the lane adds its slot and chunk.
  const uint32_t ld_koff = (uint32_t)(((int64_t)ld_row0 * kv_row_stride + 8 * ld_kchunk) * 2);
  const uint32_t ld_voff = (uint32_t)(((int64_t)ld_row0 * kv_row_stride + 8 * ld_vchunk) * 2);
  const int pg_slot_k = (ld_row0 & 15) * D + 8 * ld_kchunk;
  const int pg_slot_v = (ld_row0 & 15) * D + 8 * ld_vchunk;
  const int pg_blk0 = __builtin_amdgcn_readfirstlane(ld_row0 >> 4);
  const int pg_nblk = (Lk + 15) >> 4;
  // contiguous rows: element offset between consecutive tiles and between this wave's rows
  const int64_t tile_stride = (int64_t)kBN * kv_row_stride;
  const int64_t row_step_off = (int64_t)ROW_STEP * kv_row_stride;
  // tile j starts at element offset toff = j * tile_stride of the sequence's K/V (contiguous)
  auto issue_tile = [&](int j, int stage, int64_t toff) {
    const int k0 = j * kBN;
    char* kdst = smem + stage * T::STAGE + wave * 1024;
    char* vdst = kdst + T::TILE;
    if constexpr (PAGED) {
      const int32_t* trow = pg.table + (int64_t)b * pg.max_blocks;
#pragma unroll
      for (int i = 0; i < T::PER_WAVE; ++i) {
        const int lb = (k0 >> 4) + pg_blk0 + i * (ROW_STEP >> 4);
        int pb = lb < pg_nblk ? trow[lb] : 0;  // blocks past the context: any valid block
        if (pb < 0 || pb >= pg.num_blocks) pb = 0;  // unusable entry: never dereferenced
        const int64_t boff = ((int64_t)pb * Hkv + g) * 16 * D;
        if (pg.k_new != nullptr && k0 + kBN > off) {
          // the chunk's own keys (positions off ..) come from its rows; keys past the
          // context read the last row (their scores are masked, their V rows zeroed)
          const uint16_t* ks = k + boff + pg_slot_k;
          const uint16_t* vs = v + boff + pg_slot_v;
          const int key = k0 + ld_row0 + i * ROW_STEP;
          if (key >= off) {
            const int64_t nrow = ((int64_t)(q_row0 + min(key, Lk - 1) - off) * Hkv + g) * D;
            ks = pg.k_new + nrow + 8 * ld_kchunk;
            vs = pg.v_new + nrow + 8 * ld_vchunk;
          }
          lds_dma_16(ks, lds_addr(kdst + i * 4096));
          lds_dma_16(vs, lds_addr(vdst + i * 4096));
        } else {  // the block's base is wave-uniform: SGPR base, fixed lane offsets
          lds_dma_16s(k + boff, 2u * pg_slot_k, lds_addr(kdst + i * 4096));
          lds_dma_16s(v + boff, 2u * pg_slot_v, lds_addr(vdst + i * 4096));
        }
      }
    } else if (k0 + kBN <= S) {
      // uniform row base in SGPRs, fixed per-lane byte offsets (rows ld_row0 + i*ROW_STEP)
#pragma unroll
      for (int i = 0; i < T::PER_WAVE; ++i) {
        const int64_t rbase = toff + i * row_step_off;
        lds_dma_16s(kbase + rbase, ld_koff, lds_addr(kdst + i * 4096));
        lds_dma_16s(vbase + rbase, ld_voff, lds_addr(vdst + i * 4096));
      }
    } else {
#pragma unroll
      for (int i = 0; i < T::PER_WAVE; ++i) {
        const int row = min(k0 + ld_row0 + i * ROW_STEP, S - 1);  // past S: any valid row
        const int64_t roff = (int64_t)row * kv_row_stride;
        lds_dma_16(kbase + roff + 8 * ld_kchunk, lds_addr(kdst + i * 4096));
        lds_dma_16(vbase + roff + 8 * ld_vchunk, lds_addr(vdst + i * 4096));
      }
    }
  };

  // ---- LDS operand addresses (bytes, relative to a stage) --------------------------------
  // K A-operand of step t, block kb: row 32kb + col, chunk (2t + half) ^ k_swz(col).
  int kaddr_t[QSTEPS];
  {
    const int s = k_swz<D>(col);
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) kaddr_t[t] = col * T::ROWB + 16 * ((2 * t + half) ^ s);
  }
  // V^T A-operand via ds_read_b64_tr_b16. Lane group m = lane/16 (h = m/2, dh = m%2), lane i
  // in the group addresses row 16u + 8r + 4h + i/4 and elements 32db + 16dh + 4(i%4) .. +3;
  // it then receives keys 16u + 8r + 4h + 0..3 of d = 32db + 16dh + i, which are the keys the
  // score accumulator holds in elements 4r..4r+3 of this lane's P^T fragment for step u.
  int vaddr_db[DB];
  {
    const int m = lane >> 4, i = lane & 15;
    const int h = m >> 1, dh = m & 1;
    const int row = 4 * h + (i >> 2);  // + 16u + 8r (multiples of 4: swizzle unchanged)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 4 * db + 2 * dh + ((i & 3) >> 1);
      vaddr_db[db] = T::TILE + row * T::ROWB + 16 * (c ^ v_swz<D>(row)) + 8 * (i & 1);
    }
  }

  // One tile step for this wave. `masked` (wave-uniform) applies the causal, window and
  // ragged-end masks; interior tiles skip that arithmetic. There is a single copy of the step
  // in the loop: separate masked/unmasked copies, or skipping the step on some paths, make
  // the compiler merge the O accumulators from several paths into registers that are not the
  // MFMA's tuples, and it then copies all of them every tile.
  auto tile_step = [&](const char* st_base, int k0, bool masked, bool dummy) {
    // S^T = K Q^T; the two 32-key blocks alternate so consecutive MFMAs are independent
    // (a dependent accumulation chain would wait for each result)
    f32x16 sacc[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t)
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st_base + kaddr_t[t] + kb * 32 * T::ROWB);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], sacc[kb], 0, 0, 0);
      }
    if (masked) {
      // register r of block kb holds key offset 32*kb + 8*(r/4) + (r%4) + 4*half of the tile
      const int qp = off + q0w + col;  // query position
      int hi = Lk - 1 - k0;
      if (causal) hi = min(hi, qp - k0);
      if (dummy) hi = -(1 << 30);  // the leading stand-in tile: every score masked
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
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = xhalf_max(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_thr) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      m_thr = m_new + kRescaleSlack;
#pragma unroll
      for (int i = 0; i < DB; ++i)
        oacc[i] *= alpha;
    }
    float rs = 0.f;
    bf16x8 pf[kBN / 16];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(sacc[kb][r], scale_log2, -m_run));
        const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], scale_log2, -m_run));
        const bf16x2 pp = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
        // row sum of the bf16-rounded probabilities, the values the PV MFMA uses
        rs = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, rs, false);
        pf[2 * kb + (r >> 3)][r & 7] = pp[0];
        pf[2 * kb + (r >> 3)][(r & 7) + 1] = pp[1];
      }
    l_run += xhalf_sum(rs);
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < kBN / 16; ++u) {
        const char* p = st_base + vaddr_db[db] + u * 16 * T::ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * T::ROWB));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[u], oacc[db], 0, 0, 0);
      }
  };

  // The tile loop below is unrolled over the two LDS stages, so that each stage's operand
  // addresses are immediates; an odd number of tiles gets one stand-in tile in front (tile
  // jlo - 1, whose keys no row of the workgroup sees, or tile 0 again when jlo = 0), fully
  // masked: it adds nothing and triggers no rescale.
  const int jstart = jlo - ((jhi - jlo + 1) & 1);
  if (jlo <= jhi) issue_tile(max(jstart, 0), 0, (int64_t)max(jstart, 0) * tile_stride);
  int64_t next_toff = (int64_t)(jstart + 1) * tile_stride;  // offset of the tile issued next

  // Tiles jf_lo .. jf_hi are visible whole to every row of this wave (causal limit, window,
  // end of the keys), so they run without per-score masks. Every other tile the workgroup
  // visits is masked: an edge tile, or one outside this wave's key range that another wave
  // needs (every score -inf: it adds nothing and triggers no rescale).
  auto floor_div = [](int a, int n) { return a >= 0 ? a / n : -((n - 1 - a) / n); };
  int jf_lo = 0, jf_hi = -1;
  if (wave_live) {
    jf_hi = floor_div(Lk - kBN, kBN);
    if (causal) jf_hi = min(jf_hi, floor_div(off + q0w - kBN + 1, kBN));
    if (window > 0) jf_lo = max(jf_lo, -floor_div(window - 1 - off - qw_last, kBN));
  }

  if constexpr (PAGED) {
    // The chunk's rows of this workgroup (one head sub-group per KV head writes) go to their
    // cache slots, positions off + i: a bit copy, 16 bytes per thread step. Entries outside
    // [0, num_blocks) are skipped.
    if (pg.k_new != nullptr && hsub == 0) {
      const int n = min(q0 + rows, Sq) - q0;
      const int32_t* trow = pg.table + (int64_t)b * pg.max_blocks;
      for (int c = tid; c < n * T::CHUNKS; c += kPrefillThreads) {
        const int i = q0 + c / T::CHUNKS, ch = c % T::CHUNKS;
        const int p = off + i;
        // the row loads go out with the table load (one round trip, not two): the empty asm
        // passes all three on, so no load is sunk behind the test of the entry
        const int64_t src = ((int64_t)(q_row0 + i) * Hkv + g) * D + 8 * ch;
        u32x4 kw = *reinterpret_cast<const u32x4*>(pg.k_new + src);
        u32x4 vw = *reinterpret_cast<const u32x4*>(pg.v_new + src);
        int pb = trow[p >> 4];
        asm volatile("" : "+v"(pb), "+v"(kw), "+v"(vw));
        if (pb >= 0 && pb < pg.num_blocks) {
          const int64_t dst = (((int64_t)pb * Hkv + g) * 16 + (p & 15)) * D + 8 * ch;
          *reinterpret_cast<u32x4*>(pg.k_cache + dst) = kw;
          *reinterpret_cast<u32x4*>(pg.v_cache + dst) = vw;
        }
      }
    }
  }

  auto body = [&](int j, auto stage) {
    constexpr int st = decltype(stage)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile-j loads have landed
    __syncthreads();                     // ... and everyone's; stage st^1 is no longer read
    if (j < jhi) issue_tile(j + 1, st ^ 1, next_toff);
    next_toff += tile_stride;

    const int k0 = j * kBN;
    if constexpr (PAGED) {
      // Keys no row of the workgroup can see (past the context, left of the window) come
      // from unwritten slots, blocks left of the window or stand-in blocks and may hold
      // anything: their scores are masked, but 0 * NaN in the PV contraction would still be
      // NaN, so their V rows are zeroed (whole rows: the swizzle only permutes chunks).
      if (k0 < kmin || k0 + kBN > Lk) {
        char* vt = smem + st * T::STAGE + T::TILE;
        for (int i = tid; i < kBN * T::CHUNKS; i += kPrefillThreads) {
          const int key = k0 + i / T::CHUNKS;
          if (key < kmin || key >= Lk) *reinterpret_cast<u32x4*>(vt + 16 * i) = (u32x4){0u, 0u, 0u, 0u};
        }
        __syncthreads();
      }
    }
    const bool dummy = j < jlo;
    const bool full = !dummy && j >= jf_lo && j <= jf_hi;
    tile_step(smem + st * T::STAGE, k0, !full, dummy);
  };
  for (int j = jstart; j <= jhi; j += 2) {
    body(j, std::integral_constant<int, 0>{});
    body(j + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = O^T / l, bf16 RNE ---------------------------------------------------
  const int qr = q0w + col;
  if (wave_live && qr < Sq) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;  // a row with no visible key: zeros
    uint16_t* orow = o + (((int64_t)q_row0 + qr) * Hq + head) * D;
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
      lse[PAGED ? ((int64_t)q_row0 + qr) * Hq + head : ((int64_t)b * Hq + head) * S + qr] =
          (m_run + __log2f(l_run)) * kLn2;
  }
}

// the number of workgroups for B sequences of up to S query rows

long long prefill_workgroups(int B, int S, int Hq, int Hkv) {
  int HW, QW;
  prefill_split(Hq, Hkv, HW, QW);
  const long long rows = 32LL * QW;
  return (long long)B * Hkv * (Hq / Hkv / HW) * ((S + rows - 1) / rows);
}

int prefill_threads_per_workgroup() { return kPrefillThreads; }

template <int D, bool PAGED>
static void launch_d(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int S, int Hq, int Hkv, float scale, int causal, int window, PagedArgs pg,
                     hipStream_t stream) {
  const int G = Hq / Hkv;
  int HW, QW;  // heads per workgroup, 32-row chunks per head
  prefill_split(Hq, Hkv, HW, QW);
  const int rows = 32 * QW;
  const int n_qblk = (S + rows - 1) / rows;  // S: rows per sequence (paged: the largest chunk)
  const int n_hsub = G / HW;
  const long long nwg = (long long)B * Hkv * n_hsub * n_qblk;
  const float scale_log2 = scale * kLog2e;
  const size_t lds = 2 * PTile<D>::STAGE;
  // the dynamic-LDS limit is raised to this launch's size once per device (a no-op below the
  // default); if that fails the launch fails and the entry point reports the launch error
  static std::atomic<bool> attr_set[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  if (!attr_set[dev].load(std::memory_order_relaxed))
    attr_set[dev].store(hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, PAGED>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            (int)lds) == hipSuccess,
                        std::memory_order_relaxed);
  // workgroups resident per CU (queried once per device; 1 if the query fails)
  static std::atomic<int> per_cu_cache[kMaxDevices];
  int per_cu = per_cu_cache[dev].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_bf16_kernel<D, PAGED>,
                                                     kPrefillThreads, lds) != hipSuccess ||
        per_cu < 1) {
      (void)hipGetLastError();
      per_cu = 1;
    }
    per_cu_cache[dev].store(per_cu, std::memory_order_relaxed);
  }
  const int cus = device_cus();
  const int gmajor = nwg > (long long)cus * per_cu ? 1 : 0;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, PAGED>), dim3((unsigned)nwg), dim3(kPrefillThreads),
                     lds, stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (uint16_t*)o, lse, S, Hq, Hkv, G, HW, QW, n_qblk, n_hsub, scale_log2, causal,
                     window, cus >= 16 ? cus / 8 : 1, gmajor, pg);
}

int launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const PagedArgs none{nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, 0};
  if (a.D == 64)
    launch_d<64, false>(a.q, a.k, a.v, a.o, a.lse, a.B, a.S, a.Hq, a.Hkv, a.scale, a.causal,
                        a.window, none, stream);
  else
    launch_d<128, false>(a.q, a.k, a.v, a.o, a.lse, a.B, a.S, a.Hq, a.Hkv, a.scale, a.causal,
                         a.window, none, stream);
  return 0;
}

int launch_prefill_paged(const PrefillPagedArgs& a, hipStream_t stream) {
  // one launch: the chunk's K/V rows are written into the cache by the attention kernel
  const PagedArgs pg{a.cu_q,
                     a.ctx,
                     a.table,
                     a.max_blocks_per_seq,
                     a.num_blocks,
                     (const uint16_t*)a.k_new,
                     (const uint16_t*)a.v_new,
                     (uint16_t*)a.k_cache,
                     (uint16_t*)a.v_cache,
                     a.fixed_q};
  if (a.D == 64)
    launch_d<64, true>(a.q, a.k_cache, a.v_cache, a.o, a.lse, a.B, a.max_q_len, a.Hq, a.Hkv,
                       a.scale, a.causal, a.window, pg, stream);
  else
    launch_d<128, true>(a.q, a.k_cache, a.v_cache, a.o, a.lse, a.B, a.max_q_len, a.Hq, a.Hkv,
                        a.scale, a.causal, a.window, pg, stream);
  return 0;
}

}  // namespace attn
