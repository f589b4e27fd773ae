// C ABI of libattn: host-side validation and dispatch. Every check runs before any HIP call,
// so an invalid request returns a status code without touching the device.
#include "../../include/attn.h"
#include "launch.h"

#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return ATTN_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool supported_d(int D) { return D == 64 || D == 128; }

int kv_kind(int dtype) {
  return dtype == ATTN_I8 ? attn::kKvI8 : dtype == ATTN_FP8 ? attn::kKvFp8 : attn::kKvBf16;
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "invalid shape or size";
    case ATTN_ERR_DTYPE: return "invalid dtype";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                 int B, int S, int Hq, int Hkv, int D, float scale, int causal, int window,
                 void* stream) {
  if (!q || !k || !v || !o) return fail(ATTN_ERR_NULL, "q, k, v and o are required");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_DTYPE, "prefill dtype %d", dtype);
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1) return fail(ATTN_ERR_SHAPE, "B, S, Hq, Hkv must be >= 1");
  if (Hq % Hkv != 0) return fail(ATTN_ERR_SHAPE, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
  if (window < 0) return fail(ATTN_ERR_SHAPE, "window %d < 0", window);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  if (!supported_d(D)) return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  if ((long long)B * S * Hq > (1LL << 31) / 2) return fail(ATTN_ERR_SHAPE, "B*S*Hq too large");
  attn::PrefillArgs a{q, k, v, o, lse, B, S, Hq, Hkv, D, scale, causal != 0, window};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16)
    attn::launch_prefill_bf16(a, st);
  else
    attn::launch_prefill_f32(a, st);
  return check_launch("attn_prefill");
}

int attn_prefill_paged(const void* q, const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, const int32_t* block_table, const int32_t* cu_q,
                       const int32_t* context_lens, void* o, float* lse, int B, int Hq, int Hkv,
                       int D, int block_size, int max_blocks_per_seq, int num_blocks,
                       int max_q_len, int total_q, float scale, int causal, int window,
                       void* stream) {
  if (total_q < 0) return fail(ATTN_ERR_SHAPE, "total_q %d < 0", total_q);
  if (B < 1 || Hq < 1 || Hkv < 1 || max_blocks_per_seq < 1 || num_blocks < 1 || max_q_len < 0)
    return fail(ATTN_ERR_SHAPE, "B, Hq, Hkv, max_blocks_per_seq, num_blocks must be >= 1, max_q_len >= 0");
  if (Hq % Hkv != 0) return fail(ATTN_ERR_SHAPE, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
  if (window < 0) return fail(ATTN_ERR_SHAPE, "window %d < 0", window);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  if (!supported_d(D)) return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
  if ((long long)max_blocks_per_seq * block_size > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "max_blocks_per_seq * block_size overflows int32");
  if (B > 65535) return fail(ATTN_ERR_SHAPE, "B must be <= 65535");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(ATTN_ERR_NULL, "k_new and v_new must be both given or both NULL");
  if (total_q == 0 || max_q_len == 0) return ok();
  // the grid is one-dimensional: its thread count must stay below 2^32
  if (attn::prefill_workgroups(B, max_q_len, Hq, Hkv) * attn::prefill_threads_per_workgroup() >=
      (1LL << 32))
    return fail(ATTN_ERR_SHAPE, "B * Hq * max_q_len too large for one launch");
  if (!q || !k_cache || !v_cache || !block_table || !cu_q || !context_lens || !o)
    return fail(ATTN_ERR_NULL, "q, k_cache, v_cache, block_table, cu_q, context_lens and o are required");
  attn::PrefillPagedArgs a{q, k_new, v_new, k_cache, v_cache, block_table, cu_q, context_lens,
                           o, lse, B, Hq, Hkv, D, max_blocks_per_seq, num_blocks, max_q_len,
                           total_q, scale, causal != 0, window, 0};
  attn::launch_prefill_paged(a, reinterpret_cast<hipStream_t>(stream));
  return check_launch("attn_prefill_paged");
}

// query columns ((Hq / Hkv) * q_len) one decode wave holds: one MFMA tile
constexpr int kMaxDecodeCols = 16;

// More columns than that: each cache head serves R virtual KV heads of (Hq / Hkv) / R query
// heads, R the smallest divisor of Hq / Hkv that brings a virtual head's columns to
// kMaxDecodeCols or fewer (the cache head is then read R times). 0: none exists
// (q_len > kMaxDecodeCols). INT8 / FP8 caches always take this path; bf16 caches only at R = 2
// (5 to 8 drafts at 4 query heads per KV head: ~100 against ~118 us on the paged prefill kernel,
// which reads the cache once but fills a quarter of its rows; at R = 4, ~180 us).
static int virtual_kv_rep(int G, int q_len) {
  for (int R = 1; R <= G; ++R)
    if (G % R == 0 && (G / R) * q_len <= kMaxDecodeCols) return R;
  return 0;
}

static size_t decode_workspace(int B, int q_len, int Hq, int Hkv, int D, int max_context_len,
                               int window, int split_tokens) {
  if (B < 1 || q_len < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || max_context_len < 1 || window < 0 ||
      split_tokens < 0)
    return 0;
  // Wider than one tile: the virtual KV heads' size (a bf16 cache on the paged prefill kernel
  // needs none of it), so it holds for either cache.
  const int R = virtual_kv_rep(Hq / Hkv, q_len);
  if (R == 0) return 0;
  return attn::plan_decode(B, q_len, Hq, Hkv * R, D, max_context_len, window, split_tokens)
      .workspace_bytes;
}

size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_context_len, int window,
                                  int split_tokens) {
  return decode_workspace(B, 1, Hq, Hkv, D, max_context_len, window, split_tokens);
}

size_t attn_decode_multi_workspace_size(int B, int q_len, int Hq, int Hkv, int D,
                                        int max_context_len, int window, int split_tokens) {
  return decode_workspace(B, q_len, Hq, Hkv, D, max_context_len, window, split_tokens);
}

static int decode_impl(const char* who, const void* q, const void* k_cache, const void* v_cache,
                       const void* k_scale, const void* v_scale, const int32_t* block_table,
                       const int32_t* context_lens, void* o, int kv_dtype, int B, int q_len,
                       int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                       int num_blocks, int max_context_len, float scale, int window,
                       int split_tokens, void* workspace, size_t workspace_bytes, void* stream,
                       bool static_scratch = false) {
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !o)
    return fail(ATTN_ERR_NULL, "q, k_cache, v_cache, block_table, context_lens and o are required");
  if (kv_dtype != ATTN_BF16 && kv_dtype != ATTN_I8 && kv_dtype != ATTN_FP8)
    return fail(ATTN_ERR_DTYPE, "decode kv_dtype %d", kv_dtype);
  if (kv_dtype != ATTN_BF16 && (!k_scale || !v_scale))
    return fail(ATTN_ERR_NULL, "an int8 / fp8 cache needs k_scale and v_scale");
  if (kv_dtype == ATTN_BF16 && (k_scale || v_scale))
    return fail(ATTN_ERR_SHAPE, "k_scale/v_scale must be NULL for a bf16 cache");
  for (const void* p : {q, k_cache, v_cache, k_scale, v_scale, (const void*)o})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
      return fail(ATTN_ERR_SHAPE, "q, o, the caches and their scales must be 16-byte aligned");
  if (B < 1 || q_len < 1 || Hq < 1 || Hkv < 1 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      max_context_len < 1)
    return fail(ATTN_ERR_SHAPE, "B, q_len, Hq, Hkv, max_blocks_per_seq, num_blocks, max_context_len must be >= 1");
  if (Hq % Hkv != 0) return fail(ATTN_ERR_SHAPE, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
  if (window < 0) return fail(ATTN_ERR_SHAPE, "window %d < 0", window);
  if (split_tokens < 0) return fail(ATTN_ERR_SHAPE, "split_tokens %d < 0", split_tokens);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  if (!supported_d(D)) return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
  if (split_tokens % block_size != 0) return fail(ATTN_ERR_SHAPE, "split_tokens %d is not a multiple of block_size", split_tokens);
  if (split_tokens > attn::kMaxSplitTokens)
    return fail(ATTN_ERR_UNSUPPORTED, "split_tokens %d > %d", split_tokens, attn::kMaxSplitTokens);
  int kv_rep = 1;
  const int rep = Hq / Hkv * q_len > kMaxDecodeCols ? virtual_kv_rep(Hq / Hkv, q_len) : 1;
  if (kv_dtype != ATTN_BF16 || rep == 2) {
    // More query columns per KV head than one decode MFMA tile holds (INT8 / FP8 cache, or bf16
    // at R = 2): virtual KV heads, each cache head read once per virtual head
    kv_rep = rep;
    if (kv_rep == 0)
      return fail(ATTN_ERR_UNSUPPORTED, "q_len %d > %d needs a bf16 cache", q_len, kMaxDecodeCols);
  } else if (Hq / Hkv * q_len > kMaxDecodeCols) {
    // More query columns per KV head than one decode MFMA tile holds, bf16 cache, R != 2: the
    // rows are a fixed-size chunk per sequence, computed by the paged prefill kernel (it reads
    // the cache through the same block table, K/V once per workgroup of query heads).
    if (B > 65535) return fail(ATTN_ERR_SHAPE, "B must be <= 65535");
    if ((long long)max_blocks_per_seq * block_size > 0x7fffffffLL)
      return fail(ATTN_ERR_SHAPE, "max_blocks_per_seq * block_size overflows int32");
    if (attn::prefill_workgroups(B, q_len, Hq, Hkv) * attn::prefill_threads_per_workgroup() >=
        (1LL << 32))
      return fail(ATTN_ERR_SHAPE, "B * Hq * q_len too large for one launch");
    // no k_new / v_new: the kernel only reads the caches (their pointers are non-const in the
    // argument block for the append the paged prefill can fuse)
    attn::PrefillPagedArgs a{q, nullptr, nullptr, const_cast<void*>(k_cache),
                             const_cast<void*>(v_cache), block_table, nullptr, context_lens, o,
                             nullptr, B, Hq, Hkv, D, max_blocks_per_seq, num_blocks, q_len,
                             B * q_len, scale, 1, window, q_len};
    attn::launch_prefill_paged(a, reinterpret_cast<hipStream_t>(stream));
    return check_launch(who);
  }
  if (B > 65535 / q_len || (long long)Hkv * kv_rep > 65535)
    return fail(ATTN_ERR_SHAPE, "B * q_len and Hkv must be <= 65535");
  const int Hkv_v = Hkv * kv_rep;  // virtual KV heads
  attn::DecodePlan plan =
      attn::plan_decode(B, q_len, Hq, Hkv_v, D, max_context_len, window, split_tokens);
  if (static_scratch) {
    // the partials go to this GPU's static scratch array instead of a caller workspace
    if (plan.workspace_bytes > attn::kNoAllocScratchBytes)
      return fail(ATTN_ERR_WORKSPACE,
                  "%s needs %zu bytes of scratch here; the static scratch holds %zu", who,
                  plan.workspace_bytes, attn::kNoAllocScratchBytes);
    const hipError_t e = attn::noalloc_scratch(&workspace);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: scratch address: %s", who, hipGetErrorString(e));
    workspace_bytes = attn::kNoAllocScratchBytes;
  }
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", plan.workspace_bytes,
                workspace ? workspace_bytes : (size_t)0);
  attn::DecodeArgs a{q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, o,
                     kv_kind(kv_dtype), B, q_len, Hq, Hkv_v, D, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, scale, window, plan, workspace, kv_rep};
  attn::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
  return check_launch(who);
}

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const void* k_scale, const void* v_scale, const int32_t* block_table,
                      const int32_t* context_lens, void* o, int kv_dtype, int B, int Hq, int Hkv,
                      int D, int block_size, int max_blocks_per_seq, int num_blocks,
                      int max_context_len, float scale, int window, int split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl("attn_decode_paged", q, k_cache, v_cache, k_scale, v_scale, block_table,
                     context_lens, o, kv_dtype, B, 1, Hq, Hkv, D, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, scale, window, split_tokens, workspace,
                     workspace_bytes, stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const void* k_scale, const void* v_scale,
                              const int32_t* block_table, const int32_t* context_lens, void* o,
                              int kv_dtype, int B, int Hq, int Hkv, int D, int block_size,
                              int max_blocks_per_seq, int num_blocks, int max_context_len,
                              float scale, int window, int split_tokens, void* stream) {
  return decode_impl("attn_decode_paged_noalloc", q, k_cache, v_cache, k_scale, v_scale,
                     block_table, context_lens, o, kv_dtype, B, 1, Hq, Hkv, D, block_size,
                     max_blocks_per_seq, num_blocks, max_context_len, scale, window, split_tokens,
                     nullptr, 0, stream, /*static_scratch=*/true);
}

int attn_decode_paged_multi(const void* q, const void* k_cache, const void* v_cache,
                            const void* k_scale, const void* v_scale,
                            const int32_t* block_table, const int32_t* context_lens, void* o,
                            int kv_dtype, int B, int q_len, int Hq, int Hkv, int D,
                            int block_size, int max_blocks_per_seq, int num_blocks,
                            int max_context_len, float scale, int window, int split_tokens,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl("attn_decode_paged_multi", q, k_cache, v_cache, k_scale, v_scale,
                     block_table, context_lens, o, kv_dtype, B, q_len, Hq, Hkv, D, block_size,
                     max_blocks_per_seq, num_blocks, max_context_len, scale, window, split_tokens,
                     workspace, workspace_bytes, stream);
}

static int append_impl(const char* who, const void* k_new, const void* v_new,
                       const int32_t* seq_idx, const int32_t* pos, const int32_t* block_table,
                       void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                       int cache_dtype, int T, int Hkv, int D, int block_size, int num_seqs,
                       int max_blocks_per_seq, int num_blocks, bool rope, float rope_base,
                       void* stream) {
  if (cache_dtype != ATTN_BF16 && cache_dtype != ATTN_I8 && cache_dtype != ATTN_FP8)
    return fail(ATTN_ERR_DTYPE, "cache dtype %d", cache_dtype);
  if (T < 0) return fail(ATTN_ERR_SHAPE, "T %d < 0", T);
  if (Hkv < 1 || num_seqs < 1 || max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_SHAPE, "Hkv, num_seqs, max_blocks_per_seq, num_blocks must be >= 1");
  if (rope && !(std::isfinite(rope_base) && rope_base > 0.f))
    return fail(ATTN_ERR_SHAPE, "rope_base must be finite and > 0");
  if (!supported_d(D)) return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
  if ((long long)max_blocks_per_seq * block_size > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "max_blocks_per_seq * block_size overflows int32");
  if (T == 0) return ok();
  if (!k_new || !v_new || !seq_idx || !pos || !block_table || !k_cache || !v_cache)
    return fail(ATTN_ERR_NULL, "k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache are required");
  if (cache_dtype != ATTN_BF16 && (!k_scale || !v_scale))
    return fail(ATTN_ERR_NULL, "an int8 / fp8 cache needs k_scale and v_scale");
  attn::AppendArgs a{k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache, k_scale, v_scale,
                     kv_kind(cache_dtype), T, Hkv, D, block_size, num_seqs, max_blocks_per_seq,
                     num_blocks};
  if (rope)
    attn::launch_kv_append_rope(a, (double)rope_base, reinterpret_cast<hipStream_t>(stream));
  else
    attn::launch_kv_append(a, reinterpret_cast<hipStream_t>(stream));
  return check_launch(who);
}

int kv_cache_append(const void* k_new, const void* v_new, const int32_t* seq_idx,
                    const int32_t* pos, const int32_t* block_table, void* k_cache, void* v_cache,
                    void* k_scale, void* v_scale, int cache_dtype, int T, int Hkv, int D,
                    int block_size, int num_seqs, int max_blocks_per_seq, int num_blocks,
                    void* stream) {
  return append_impl("kv_cache_append", k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache,
                     k_scale, v_scale, cache_dtype, T, Hkv, D, block_size, num_seqs,
                     max_blocks_per_seq, num_blocks, false, 0.f, stream);
}

int kv_cache_append_rope(const void* k_new, const void* v_new, const int32_t* seq_idx,
                         const int32_t* pos, const int32_t* block_table, void* k_cache,
                         void* v_cache, void* k_scale, void* v_scale, int cache_dtype, int T,
                         int Hkv, int D, int block_size, int num_seqs, int max_blocks_per_seq,
                         int num_blocks, float rope_base, void* stream) {
  return append_impl("kv_cache_append_rope", k_new, v_new, seq_idx, pos, block_table, k_cache,
                     v_cache, k_scale, v_scale, cache_dtype, T, Hkv, D, block_size, num_seqs,
                     max_blocks_per_seq, num_blocks, true, rope_base, stream);
}

int attn_rope_inplace(void* x, const int32_t* pos, int T, int H, int D, float rope_base,
                      void* stream) {
  if (T < 0 || H < 1) return fail(ATTN_ERR_SHAPE, "T must be >= 0 and H >= 1");
  if (!(std::isfinite(rope_base) && rope_base > 0.f))
    return fail(ATTN_ERR_SHAPE, "rope_base must be finite and > 0");
  if (!supported_d(D)) return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  if (T == 0) return ok();
  if (!x || !pos) return fail(ATTN_ERR_NULL, "x and pos are required");
  attn::launch_rope_rows(x, pos, T, H, D, (double)rope_base, reinterpret_cast<hipStream_t>(stream));
  return check_launch("attn_rope_inplace");
}

}  // extern "C"
