// Launchers behind the C ABI (host side).  Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Where element (block, slot offset, kv head, 0) of a cache sits: strides in
// elements.  Block-major slots then heads ([blocks, block_size, heads, dim])
// or block-major heads then slots ([blocks, heads, block_size, dim]).
struct CacheGeom {
  int64_t block, slot, head;
};
inline CacheGeom cache_geom(bool heads_outer, int64_t num_kv_heads, int64_t block_size,
                            int64_t head_dim) {
  if (heads_outer) return {num_kv_heads * block_size * head_dim, head_dim, block_size * head_dim};
  return {block_size * num_kv_heads * head_dim, num_kv_heads * head_dim, head_dim};
}

struct StoreArgs {
  const void* k;
  const void* v;
  int64_t k_tok_stride, k_head_stride, v_tok_stride, v_head_stride;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  int32_t num_tokens, num_kv_heads, head_dim, block_size;
  int32_t elt_bytes;  // 2 (bf16) or 4 (fp32)
  CacheGeom geom;
};
hipError_t launch_store(const StoreArgs& a, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  int64_t q_seq_stride, q_head_stride;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  int64_t block_table_stride;
  const int32_t* context_lens;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size;
  int32_t max_context_len, partition_tokens, num_splits;
  float scale;
  float* ws_acc;  // [B, Hq, S, D]
  float* ws_ml;   // [B, Hq, S, 2]
  bool bf16;
  CacheGeom geom;
  // the fused store (k_new == nullptr: none): row b is sequence b's new token
  const void* k_new;
  const void* v_new;
  int64_t k_tok_stride, k_head_stride, v_tok_stride, v_head_stride;
  const int32_t* slot_mapping;
  // Shared prefixes (prefix_group == nullptr: none).  Sequence b of group
  // prefix_group[b] in [0, num_prefix_groups) skips its splits s <
  // min(min(prefix_tokens[group], max_prefix_tokens) / partition_tokens,
  // (context_lens[b] - 1) / partition_tokens): the shared-prefix pass writes them.
  const int32_t* prefix_group;
  const int32_t* prefix_tokens;
  int32_t num_prefix_groups, max_prefix_tokens;
  // The partition pass's work list (nullptr: none): work_list[0] entries
  // (sequence << 16 | split) from work_list[1] on, one per workgroup column,
  // written by the shared-prefix pass's launch.
  const int32_t* work_list;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// The shared-prefix pass (bf16): the split statistics of every member's splits
// inside its group's prefix, in the layout of the partition pass.
struct PrefixArgs {
  const void* q;
  int64_t q_seq_stride, q_head_stride;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  int64_t block_table_stride;
  const int32_t* context_lens;
  const int32_t* prefix_group;
  const int32_t* prefix_tokens;
  int32_t num_groups, max_prefix_tokens;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size;
  int32_t partition_tokens, num_splits;
  float scale;
  float* ws_acc;
  float* ws_ml;
  CacheGeom geom;
  const StoreArgs* store;  // non-null: this step's K/V store, by extra workgroups of the launch
  int32_t* work_list;      // non-null: the partition pass's work list, by one extra workgroup
  int32_t max_context_len;
};
hipError_t launch_prefix_splits(const PrefixArgs& a, hipStream_t stream);

// Bytes of the decode workspace before the work list (16-byte aligned).
inline size_t decode_ws_stats_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t num_splits,
                                    int64_t head_dim) {
  return (static_cast<size_t>(num_seqs * num_q_heads * num_splits * (head_dim + 2)) *
              sizeof(float) + 15) / 16 * 16;
}

struct ReduceArgs {
  const float* ws_acc;
  const float* ws_ml;
  const int32_t* context_lens;
  int32_t num_seqs, num_q_heads, head_dim, num_splits, partition_tokens;
  void* out;
  int64_t out_seq_stride, out_head_stride;
  bool bf16;
};
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);

// The prefill workspace opens with this many bytes of work-list counters
// (claim counter, entry count, finished workgroups) ahead of the work list.
constexpr size_t kPrefillTicketBytes = 512;

struct PrefillArgs {
  const void* q;
  int64_t q_tok_stride, q_head_stride;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* block_table;
  int64_t block_table_stride;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size;
  int32_t max_seqlen_q, max_seqlen_k, total_q;
  float scale;
  int32_t split_keys, num_splits;  // num_splits == 1: no split, ws_acc / ws_ml unused
  uint32_t* tickets;               // work-list counters and length (kPrefillTicketBytes)
  int2* items;                     // work list written by the plan kernel
  int2* merges;                    // split query tiles, written by the plan kernel
  float* ws_acc;                   // [S, total_q, Hq, D]
  float* ws_ml;                    // [S, total_q, Hq, 2]
  void* out;
  int64_t out_tok_stride, out_head_stride;
  CacheGeom geom;
  const StoreArgs* store;  // non-null: this step's K/V store, in the work-list launch
  bool planned;            // the work list is in the workspace already: no plan launch
  bool plan_only;          // only the plan launch (pa_prefill_plan)
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

struct RopeArgs {
  const void* qkv;
  int64_t qkv_tok_stride;
  const void* q_weight;  // both null: no q/k norm
  const void* k_weight;
  const int32_t* positions;
  const int32_t* slot_mapping;
  int32_t num_tokens, num_q_heads, num_kv_heads, head_dim;
  float eps;
  double theta;
  void* q_out;
  int64_t q_out_tok_stride;
  void* k_cache;
  void* v_cache;
  int32_t block_size;
  int32_t elt_bytes;
  CacheGeom geom;
};
hipError_t launch_norm_rope_store(const RopeArgs& a, hipStream_t stream);

// The fixed device-resident workspace of pa_store_decode_noalloc: each GPU the
// library runs on holds one copy for the rest of the process.
constexpr size_t kDecodeScratchBytes = size_t{64} << 20;
// The current device's copy (its address asked of the runtime once per device).
hipError_t decode_scratch(float** ptr);

// The prefill work list is built by one workgroup that holds a per-sequence
// table in LDS, which bounds the batch.
constexpr int kPrefillPlanMaxSeqs = 4096;

// Query positions per prefill work item for a GQA group size.
inline int prefill_rows_per_tile(int group) { return 32 * (group >= 4 ? 1 : 4 / group); }

}  // namespace pa
