/*
 * attn.h -- C ABI of libattn: fused prefill attention, paged-KV decode attention and KV-cache
 * append for AMD Instinct MI355X (gfx950).
 *
 * Sources (page title, section):
 *  [TI] "从零构建CUDA推理引擎：Tiny-Infer项目的技术深度解析" (Tiny-Infer, a CUDA/C++ engine for
 *       Llama 3.2 1B):
 *       - "Flash Attention：内存与计算的重平衡": attention computed block by block with an online
 *         softmax in on-chip memory, one thread block per (attention head, block of queries),
 *         partial results accumulated on chip, the full score matrix never stored;
 *       - "分页KV缓存：借鉴操作系统的内存管理": the KV cache is cut into fixed-size blocks and a
 *         mapping table sends each logical position to a physical block;
 *       - "推测性解码与INT8量化": the KV cache is stored in INT8 instead of FP16;
 *       - "技术架构与模块设计": a static cache preallocated to the maximum context, with attention
 *         changed to run incrementally (one new token against the cache) for decode.
 *  [IL] "从零开始的LLM推理优化实验室：从PyTorch基线到Triton内核的完整实践",
 *       "KV缓存实验与长上下文优化": static, growing and sliding-window caches.
 *  [TF] "Triton融合算子优化：LLM推理性能提升3倍的工程实践", "3.1 RMSNorm + RoPE 融合": rotary
 *       position embedding applied at the rows' position ids inside a neighbouring
 *       elementwise kernel, so the rows cross HBM once.
 *  [KD] "5 Fun Projects for LLM Inference Engineering" (KDnuggets), project 2 ("write your own
 *       FlashAttention kernel in Triton"): tiling and the online softmax cut HBM<->on-chip traffic;
 *       project 4 (speculative decoding): the target model checks several draft tokens at once.
 *
 * Definition computed by every entry point (fp32 accumulation): for query row i of Sq rows
 * against Lk keys, its position is P = Lk - Sq + i; key j is visible iff (not causal or
 * j <= P) and (window == 0 or P - j < window); s_j = scale * q . k_j;
 * o = sum_j softmax(s)_j v_j over the visible keys. Query head h reads KV head h / (Hq / Hkv).
 *
 * Conventions for every call:
 *  - Every tensor argument is a device pointer owned by the caller; the library allocates no
 *    memory. Its only state is a thread-local last-error string, kernel attributes set once
 *    per device, and the static scratch array of attn_decode_paged_noalloc (part of the code
 *    object) with its per-device address.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL = the default stream) and
 *    returns without synchronising. The result is ready when the stream reaches that point.
 *  - Arguments are validated on the host before any launch; on a nonzero return nothing was
 *    enqueued (except ATTN_ERR_HIP, returned when a launch itself fails).
 *  - bf16 is IEEE bfloat16 stored as 16-bit words; fp16 is IEEE binary16; all tensors are dense,
 *    row-major, with the last dimension contiguous.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  ATTN_ERR_DTYPE = 3,       /* unknown dtype code */
  ATTN_ERR_UNSUPPORTED = 4, /* valid request that the library does not implement */
  ATTN_ERR_WORKSPACE = 5,   /* workspace missing or smaller than attn_decode_workspace_size() */
  ATTN_ERR_HIP = 6          /* a HIP launch failed; attn_last_error() holds the HIP message */
};

/* ATTN_I8 and ATTN_FP8 are KV-cache element types only (codes with fp16 scales); ATTN_FP8 is
 * OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest finite 448,
 * S.1111.111 = NaN, no infinities), stored one code per byte. */
enum attn_dtype { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_I8 = 2, ATTN_FP8 = 3 };

/*
 * attn_prefill -- tiled (FlashAttention-style) prefill attention with an online softmax.
 * [TI] "Flash Attention：内存与计算的重平衡"; [KD] project 2; sliding window: [IL].
 *
 *  q, o : [B][S][Hq][D]  dtype (ATTN_F32 or ATTN_BF16); o gets the same dtype as q, rounded to
 *                        nearest-even from fp32 for bf16.
 *  k, v : [B][S][Hkv][D] same dtype.
 *  lse  : optional fp32 [B][Hq][S], natural-log log-sum-exp of each row's scaled scores; NULL
 *         to skip.
 *  Sq = Lk = S, so query i sits at position i. causal != 0 applies the causal mask;
 *  window = 0 means no window, window > 0 keeps the last `window` keys up to each query.
 *  Requirements: B, S >= 1; Hkv >= 1; Hq a multiple of Hkv; D in {64, 128} (ATTN_ERR_UNSUPPORTED
 *  otherwise); window >= 0; scale finite.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                 int dtype, int B, int S, int Hq, int Hkv, int D,
                 float scale, int causal, int window, void* stream);

/*
 * attn_prefill_paged -- chunked (continued) prefill over a paged KV cache, with the chunk's
 * K/V written into the cache by the same launch. [TI] "分页KV缓存：借鉴操作系统的内存管理" (paged cache) and
 * "Flash Attention：内存与计算的重平衡" (tiled attention with an online softmax); window: [IL].
 *
 *  q, o         : [total_q][Hq][D] bf16, packed: sequence b owns rows cu_q[b] .. cu_q[b+1]-1.
 *  k_new, v_new : [total_q][Hkv][D] bf16, the chunk's keys and values, written (bit copy) to
 *                 positions context_lens[b] - q_len_b .. context_lens[b] - 1 of sequence b
 *                 (q_len_b = cu_q[b+1] - cu_q[b]) by the same launch that computes attention,
 *                 which reads the chunk's own keys from these rows; both NULL when the cache
 *                 already holds them. The slots of those positions must not also hold a key
 *                 that any sequence of the call reads from the cache (a table that maps
 *                 distinct positions to distinct slots guarantees this).
 *  k_cache,
 *  v_cache      : bf16 [num_blocks][Hkv][block_size][D], block_table int32
 *                 [B][max_blocks_per_seq], as in attn_decode_paged.
 *  cu_q         : int32 [B + 1], cu_q[0] = 0, non-decreasing, cu_q[B] = total_q.
 *  context_lens : int32 [B], keys of each sequence after the chunk (q_len_b <= context_lens[b]
 *                 <= max_blocks_per_seq * block_size); row i of sequence b sits at position
 *                 context_lens[b] - q_len_b + i (bottom-right alignment).
 *  lse          : optional fp32 [total_q][Hq] (natural-log log-sum-exp), or NULL.
 *  max_q_len    : host-side bound on every q_len_b, used to size the grid.
 *  Requirements: D in {64, 128}; block_size == 16; Hq % Hkv == 0; total_q >= 0 (0 is a no-op);
 *  causal and window as in attn_prefill; bf16 only. Rows whose chunk is longer than the context
 *  are left unwritten. A live table entry outside [0, num_blocks) is a caller error: it is never
 *  dereferenced (physical block 0 is read in its place, so no access leaves the pools), and
 *  the rows that see its keys get an unspecified result (attn_decode_paged skips such keys
 *  instead; both give a meaningless result for a broken table). Cache
 *  slots that hold no key visible to any row of the chunk (past the context, or left of every
 *  row's window) may hold anything, NaN included, and the table entries of blocks made only
 *  of such slots may hold anything: that content never reaches the result.
 */
int attn_prefill_paged(const void* q, const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, const int32_t* block_table, const int32_t* cu_q,
                       const int32_t* context_lens, void* o, float* lse, int B, int Hq, int Hkv,
                       int D, int block_size, int max_blocks_per_seq, int num_blocks,
                       int max_q_len, int total_q, float scale, int causal, int window,
                       void* stream);

/*
 * attn_decode_workspace_size -- bytes of device workspace attn_decode_paged needs for these
 * sizes (0 when the call runs as a single pass and needs none). split_tokens as below. With
 * more than 16 query heads per KV head the size is that of the virtual KV heads (below),
 * which a bf16 cache on the paged prefill kernel does not use.
 */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_context_len,
                                  int window, int split_tokens);

/*
 * attn_decode_paged -- one new query token per sequence against a paged KV cache.
 * [TI] "分页KV缓存：借鉴操作系统的内存管理" (block table), "技术架构与模块设计" (incremental
 * decode against the cache), "推测性解码与INT8量化" (INT8 cache); sliding window: [IL].
 *
 *  q, o         : [B][Hq][D] bf16. Query b sits at position context_lens[b] - 1. Any finite
 *                 bf16 query is accepted: with an INT8 or FP8 cache the products run on fp16,
 *                 and each query vector is first multiplied by a power of two that brings its
 *                 largest element into [256, 512) (exact), the factor being taken out of the
 *                 score again, so magnitudes beyond fp16's range (>= 65520) or below its
 *                 subnormals lose nothing that the bf16 value holds within 2^-22 of that largest
 *                 element.
 *  k_cache,
 *  v_cache      : [num_blocks][Hkv][block_size][D], bf16 (kv_dtype ATTN_BF16), int8 codes
 *                 (ATTN_I8) or FP8 E4M3 codes (ATTN_FP8; [TF] "3.3 FP8量化支持").
 *                 Logical token t of sequence b lives in slot t % block_size of
 *                 physical block block_table[b][t / block_size].
 *  k_scale,
 *  v_scale      : fp16 [num_blocks][Hkv][block_size], required iff kv_dtype is ATTN_I8 or
 *                 ATTN_FP8, else NULL. The value seen by attention is value(code) * scale
 *                 (INT8: the integer; FP8: the E4M3 value). FP8 NaN codes must not be stored.
 *  block_table  : int32 [B][max_blocks_per_seq]. Entries for blocks that hold no visible
 *                 token (past the context, or wholly left of the window) are never read and
 *                 may hold anything. A live entry outside [0, num_blocks) is not dereferenced:
 *                 its tokens are skipped (the result is then meaningless, but no stray access
 *                 happens).
 *  context_lens : int32 [B], each in [1, min(max_context_len, max_blocks_per_seq*block_size)];
 *                 values outside are clamped to that range on the device (0 or less gives o = 0).
 *  max_context_len : host-side upper bound of context_lens, used to plan the split of the
 *                 KV range across workgroups without reading device memory.
 *  window       : 0 = no window; else only the last `window` positions are attended.
 *  split_tokens : how the KV axis is divided, partials merged by log-sum-exp. 0 = the
 *                 library's choice: with window == 0 and B <= 2048, a persistent grid whose
 *                 waves take equal shares of all (sequence, KV head, block) work, so ragged
 *                 contexts stay balanced; otherwise fixed splits sized from max_context_len.
 *                 Else a positive multiple of block_size, at most 8192
 *                 (ATTN_ERR_UNSUPPORTED above): fixed splits of that many tokens.
 *                 Results are run-to-run identical for a given split_tokens on a given GPU.
 *  workspace    : device buffer of at least attn_decode_workspace_size(...) bytes (may be NULL
 *                 when that size is 0); overwritten by the call; its contents on entry do not
 *                 matter. Two calls in flight at once must not share a workspace.
 *  More than 16 query heads per KV head: virtual KV heads -- each cache head is split into R
 *                 groups of (Hq / Hkv) / R query heads, R the smallest divisor of Hq / Hkv
 *                 that makes a group 16 heads or fewer, and read by the decode kernels once
 *                 per group (R times in all); the results equal those of a cache holding each
 *                 head R times, bit for bit. An INT8 or FP8 cache always takes this path, a
 *                 bf16 cache when R = 2; a bf16 cache with R > 2 is read once by the paged
 *                 prefill kernel instead (as in attn_decode_paged_multi).
 *  Requirements: D in {64, 128}; block_size == 16; Hq % Hkv == 0; q, o, k_cache, v_cache,
 *                 k_scale and v_scale 16-byte aligned (else ATTN_ERR_SHAPE).
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const void* k_scale, const void* v_scale,
                      const int32_t* block_table, const int32_t* context_lens, void* o,
                      int kv_dtype, int B, int Hq, int Hkv, int D,
                      int block_size, int max_blocks_per_seq, int num_blocks,
                      int max_context_len, float scale, int window, int split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. It computes exactly what attn_decode_paged computes with the same
 * arguments (the same kernels; the results are bit-identical) and allocates nothing: the
 * split-KV partials go to a static device array of 32 MiB per GPU, created with the library's
 * code object and held until the process ends. Its address is looked up once per device
 * (hipGetSymbolAddress, with that device current).
 *  - A call whose partials need more than the 32 MiB returns ATTN_ERR_WORKSPACE before any
 *    launch (attn_decode_workspace_size gives the need; e.g. the balanced shape needs about
 *    (B*Hkv + 8*CUs) * (Hq/Hkv) * D * 4 bytes).
 *  - Every call on one GPU shares that GPU's array and overwrites it: calls that may overlap
 *    on one GPU (different streams without ordering between them, or threads) race, and their
 *    results are undefined. Calls ordered on one stream are safe.
 *  - Nothing has to be initialised: the array's contents on entry do not matter.
 * Other arguments and status codes: as attn_decode_paged.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const void* k_scale, const void* v_scale,
                              const int32_t* block_table, const int32_t* context_lens, void* o,
                              int kv_dtype, int B, int Hq, int Hkv, int D,
                              int block_size, int max_blocks_per_seq, int num_blocks,
                              int max_context_len, float scale, int window, int split_tokens,
                              void* stream);

/*
 * attn_decode_multi_workspace_size -- as attn_decode_workspace_size, for attn_decode_paged_multi
 * with q_len query rows per sequence.
 */
size_t attn_decode_multi_workspace_size(int B, int q_len, int Hq, int Hkv, int D,
                                        int max_context_len, int window, int split_tokens);

/*
 * attn_decode_paged_multi -- q_len new query rows per sequence against the paged cache: the
 * verification step of speculative decoding, where the target model scores q_len draft tokens
 * at once. [TI] "推测性解码与INT8量化" (a small draft model proposes tokens, the main model
 * verifies them in parallel); [KD] project 4.
 *
 * Same arguments and rules as attn_decode_paged, except:
 *  q, o         : [B][q_len][Hq][D] bf16. Row r of sequence b sits at position
 *                 context_lens[b] - q_len + r and attends causally: to keys 0 .. that position
 *                 (and, with a window, only the last `window` of them). The q_len draft tokens'
 *                 K/V must already be in the cache (kv_cache_append), so context_lens counts
 *                 them; rows whose position is negative produce zeros.
 *  q_len        : >= 1. Up to (Hq / Hkv) * q_len = 16 query columns per KV head the rows and
 *                 heads share one MFMA tile of the decode kernels, so each K/V byte is read
 *                 once for all of them. Above 16 (e.g. 8 draft tokens at 4 query heads per KV
 *                 head) the decode kernels run on virtual KV heads (as in attn_decode_paged:
 *                 groups of (Hq / Hkv) / R heads with all q_len rows, at most 16 columns, each
 *                 cache head read R times), which needs q_len <= 16 (ATTN_ERR_UNSUPPORTED above
 *                 for an INT8 or FP8 cache). A bf16 cache takes that path when R = 2 (e.g. 5
 *                 to 8 drafts at 4 query heads per KV head); otherwise it is read once by the
 *                 paged prefill kernel (the rows of a sequence as one fixed-size chunk, same row
 *                 positions and zeros; no workspace, split_tokens has no effect, context_lens is
 *                 clamped to the table's capacity only).
 *  workspace    : at least attn_decode_multi_workspace_size(...) bytes (for more than 16
 *                 columns: the virtual KV heads' need, unused on the paged prefill kernel).
 * q_len == 1 computes exactly what attn_decode_paged computes.
 */
int attn_decode_paged_multi(const void* q, const void* k_cache, const void* v_cache,
                            const void* k_scale, const void* v_scale,
                            const int32_t* block_table, const int32_t* context_lens, void* o,
                            int kv_dtype, int B, int q_len, int Hq, int Hkv, int D,
                            int block_size, int max_blocks_per_seq, int num_blocks,
                            int max_context_len, float scale, int window, int split_tokens,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_cache_append -- write T new K/V rows into the paged cache.
 * [TI] "技术架构与模块设计" (cache written as tokens are produced), "分页KV缓存：借鉴操作系统的内存管理"
 * (logical position -> physical block through the table), "推测性解码与INT8量化" (INT8 storage).
 *
 *  k_new, v_new : [T][Hkv][D] bf16.
 *  seq_idx, pos : int32 [T]; row t goes to sequence seq_idx[t] at logical position pos[t], i.e.
 *                 slot pos % block_size of block block_table[seq_idx][pos / block_size].
 *  block_table  : int32 [num_seqs][max_blocks_per_seq].
 *  k_cache, v_cache, k_scale, v_scale : as in attn_decode_paged. cache_dtype ATTN_BF16 copies
 *                 the bits; ATTN_I8 quantizes each (token, KV head) row of D values:
 *                 a = max|x|, scale = fp16(fp32(a) / 127) (IEEE division, round to nearest
 *                 even), code = clamp(rint(x / fp32(scale)), -127, 127) with ties to even; a
 *                 zero scale gives zero codes. ATTN_FP8 ([TF] "3.3 FP8量化支持", dynamic
 *                 per-token scale): scale = fp16(fp32(a) / 448), code = the E4M3 value nearest
 *                 to clamp(x / fp32(scale), -448, 448), ties to even, sign kept (-0 -> 0x80);
 *                 a zero scale gives zero codes.
 *  Rows whose seq_idx is outside [0, num_seqs), whose pos is outside
 *  [0, max_blocks_per_seq*block_size), or whose table entry is outside [0, num_blocks) are not
 *  written. Two rows aimed at the same slot leave one of them, unspecified which.
 *  Requirements: T >= 0 (T == 0 is a no-op); D in {64, 128}; block_size == 16.
 */
int kv_cache_append(const void* k_new, const void* v_new, const int32_t* seq_idx,
                    const int32_t* pos, const int32_t* block_table,
                    void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                    int cache_dtype, int T, int Hkv, int D, int block_size,
                    int num_seqs, int max_blocks_per_seq, int num_blocks, void* stream);

/*
 * kv_cache_append_rope -- kv_cache_append with rotary position embedding fused into the write:
 * each K row is turned at its own position pos[t] before it is stored (and quantized, for an
 * INT8 cache); V rows are stored as in kv_cache_append. [TF] "3.1 RMSNorm + RoPE 融合"; [TI]
 * "技术架构与模块设计" (RoPE among the Llama 3.2 1B operators).
 * RoPE rule (the pages name it without a formula; Llama convention): for i < D/2, element i
 * pairs with element i + D/2 and the pair is rotated by the angle pos * rope_base^(-2i/D):
 *   out_i = x_i cos - x_{i+D/2} sin,  out_{i+D/2} = x_i sin + x_{i+D/2} cos,
 * the angle in fp64 (reduced modulo 2*pi in fp64), sin, cos and the rotation in fp32, the
 * result rounded to bf16 (nearest even) for a bf16 cache. rope_base: finite and > 0 (Llama 3.2 uses 500000, the original
 * RoPE 10000); otherwise ATTN_ERR_SHAPE. Everything else as kv_cache_append.
 */
int kv_cache_append_rope(const void* k_new, const void* v_new, const int32_t* seq_idx,
                         const int32_t* pos, const int32_t* block_table,
                         void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                         int cache_dtype, int T, int Hkv, int D, int block_size,
                         int num_seqs, int max_blocks_per_seq, int num_blocks, float rope_base,
                         void* stream);

/*
 * attn_rope_inplace -- the same rotation applied in place to bf16 rows x [T][H][D] at
 * positions pos[T] (int32): the query side, turned before attention by the rule the cache
 * append used for K. [TF] "3.1 RMSNorm + RoPE 融合".
 * Requirements: T >= 0 (0 = no-op), H >= 1, D in {64, 128}, rope_base finite and > 0.
 */
int attn_rope_inplace(void* x, const int32_t* pos, int T, int H, int D, float rope_base,
                      void* stream);

/* Static string naming a status code. */
const char* attn_status_str(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
