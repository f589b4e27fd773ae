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

constexpr int kMaxSplitTokens = 8192;  // largest split_tokens a decode call accepts

struct DecodePlan {
  int split_tokens;  // tokens per workgroup along the KV axis (multiple of 16)
  int n_split;       // workgroups per (sequence, KV head)
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
  bool int8;
  int B, Hq, Hkv, D, block_size, max_blocks_per_seq, num_blocks, max_context_len;
  float scale;
  int window;
  DecodePlan plan;
  void* workspace;
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
  bool int8;
  int T, Hkv, D, block_size, num_seqs, max_blocks_per_seq, num_blocks;
};

DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int max_context_len, int window,
                       int split_tokens);

int launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
int launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
int launch_decode(const DecodeArgs& a, hipStream_t stream);
int launch_kv_append(const AppendArgs& a, hipStream_t stream);

}  // namespace attn
