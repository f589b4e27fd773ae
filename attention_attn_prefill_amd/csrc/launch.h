// Internal launcher interface between the C ABI layer (attn_api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, S, Hq, Hkv, D;
  float scale;
  int causal, window;
};

// KV-cache element kinds (bf16 values, INT8 codes, FP8 E4M3 codes; byte kinds carry fp16
// per-(token, KV head) scales)
constexpr int kKvBf16 = 0, kKvI8 = 1, kKvFp8 = 2;

constexpr int kMaxSplitTokens = 8192;  // largest split_tokens a decode call accepts
constexpr int kStreamMaxB = 2048;      // largest batch of the balanced decode shape
constexpr int kMaxDevices = 64;        // devices with per-device launch state (attributes set once)
// Device scratch of attn_decode_paged_noalloc: one static array per GPU, held until the
// process ends.
constexpr size_t kNoAllocScratchBytes = 32u << 20;

struct DecodePlan {
  bool stream;           // balanced persistent shape (else fixed splits)
  int stream_waves_max;  // balanced: most waves a launch may use (sizes the partial slots)
  int split_tokens;      // fixed split: tokens per workgroup along the KV axis (multiple of 16)
  int n_split;           // fixed split: workgroups per (sequence, KV head)
  size_t prefix_off, part_o_off, part_lse_off;  // workspace layout (bytes)
  size_t workspace_bytes;
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const void* k_scale;
  const void* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* o;
  int kv;  // cache element kind: kKvBf16, kKvI8 or kKvFp8
  // Hkv counts virtual KV heads: each of the cache's Hkv / kv_rep heads serves kv_rep of them,
  // Hq / Hkv query heads each (kv_rep = 1: the cache's own heads)
  int B, q_len, Hq, Hkv, D, block_size, max_blocks_per_seq, num_blocks, max_context_len;
  float scale;
  int window;
  DecodePlan plan;
  void* workspace;
  int kv_rep;
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* block_table;
  void* k_cache;
  void* v_cache;
  void* k_scale;
  void* v_scale;
  int kv;  // cache element kind: kKvBf16, kKvI8 or kKvFp8
  int T, Hkv, D, block_size, num_seqs, max_blocks_per_seq, num_blocks;
};

struct PrefillPagedArgs {
  const void* q;       // [total_q][Hq][D] packed query rows
  const void* k_new;   // [total_q][Hkv][D] the chunk's K rows, or null (already in the cache)
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* table;
  const int32_t* cu_q;  // [B + 1], or null with fixed_q > 0
  const int32_t* ctx;   // [B]
  void* o;
  float* lse;  // [total_q][Hq] or null
  int B, Hq, Hkv, D, max_blocks_per_seq, num_blocks, max_q_len, total_q;
  float scale;
  int causal, window;
  // > 0: every sequence has exactly fixed_q rows (rows b*fixed_q ..), row i at position
  // ctx - fixed_q + i even when that is negative (such rows see no key and get zeros): the
  // layout and row semantics of multi-row decode
  int fixed_q;
};

DecodePlan plan_decode(int B, int q_len, int Hq, int Hkv, int D, int max_context_len, int window,
                       int split_tokens);

// Compute units of the current device (256 on MI355X if the query fails).
int device_cus();

int launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
int launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
int launch_decode(const DecodeArgs& a, hipStream_t stream);
int launch_kv_append(const AppendArgs& a, hipStream_t stream);
int launch_kv_append_rope(const AppendArgs& a, double rope_base, hipStream_t stream);
int launch_rope_rows(void* x, const int32_t* pos, int T, int H, int D, double rope_base,
                     hipStream_t stream);
int launch_prefill_paged(const PrefillPagedArgs& a, hipStream_t stream);

// Device address of this GPU's static decode scratch (kNoAllocScratchBytes), looked up once
// per device with that device current.
hipError_t noalloc_scratch(void** ptr);

// Workgroups and threads per workgroup of a bf16 prefill launch over B sequences of up to S
// query rows (the grid is one-dimensional).
long long prefill_workgroups(int B, int S, int Hq, int Hkv);
int prefill_threads_per_workgroup();

}  // namespace attn
