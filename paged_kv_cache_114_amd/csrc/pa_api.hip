// C ABI entry points: host-side argument checks, then the launchers.
// The contract of every function is documented in include/pa.h.

#include "pa.h"

#include "pa_internal.h"

namespace {

constexpr int kVersion = 201;  // 0.2.1
constexpr int64_t kPrefillMaxTableEntries = 8192;  // 32 KB of LDS beside the K/V tile buffers

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_bytes(int32_t dtype) {
  if (dtype == PA_DTYPE_F32) return 4;
  if (dtype == PA_DTYPE_BF16) return 2;
  return 0;
}

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }
bool block_size_ok(int32_t bs) { return is_pow2(bs) && bs >= 8 && bs <= 1024; }
bool group_ok(int32_t hq, int32_t hkv) {
  if (hkv <= 0 || hq <= 0 || hq % hkv != 0) return false;
  const int g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

int launched(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

bool layout_ok(int32_t l) { return l == PA_CACHE_BSHD || l == PA_CACHE_BHSD; }

pa::CacheGeom geom_of(int32_t layout, int32_t num_kv_heads, int32_t block_size,
                      int32_t head_dim) {
  return pa::cache_geom(layout == PA_CACHE_BHSD, num_kv_heads, block_size, head_dim);
}

}  // namespace

extern "C" {

int pa_version(void) { return kVersion; }

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape, dtype or alignment";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int pa_store_kv(const void* k, const void* v, int64_t k_tok_stride, int64_t k_head_stride,
                int64_t v_tok_stride, int64_t v_head_stride, void* k_cache, void* v_cache,
                const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t cache_layout,
                int32_t dtype, hipStream_t stream) {
  const int eb = elt_bytes(dtype);
  if (eb == 0 || !layout_ok(cache_layout)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (k_tok_stride < 0 || k_head_stride < 0 || v_tok_stride < 0 || v_head_stride < 0)
    return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (num_blocks > (INT32_MAX / block_size) + int64_t{1}) return PA_ERR_UNSUPPORTED;  // int32 slots
  if (int64_t{num_tokens} * 2 * num_kv_heads * head_dim >= (int64_t{1} << 31))
    return PA_ERR_UNSUPPORTED;
  pa::StoreArgs a{k, v, k_tok_stride, k_head_stride, v_tok_stride, v_head_stride, k_cache,
                  v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, eb,
                  geom_of(cache_layout, num_kv_heads, block_size, head_dim)};
  return launched(pa::launch_store(a, stream));
}

int pa_qk_norm_rope_store(const void* qkv, int64_t qkv_tok_stride, const void* q_norm_weight,
                          const void* k_norm_weight, const int32_t* positions,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, float eps, double rope_theta,
                          void* q_out, int64_t q_out_tok_stride, void* k_cache, void* v_cache,
                          int32_t block_size, int64_t num_blocks, int32_t cache_layout,
                          int32_t dtype, hipStream_t stream) {
  const int eb = elt_bytes(dtype);
  if (eb == 0 || !layout_ok(cache_layout)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  const int64_t heads = int64_t{num_q_heads} + 2 * int64_t{num_kv_heads};
  if (heads > 65536) return PA_ERR_UNSUPPORTED;
  if (qkv_tok_stride < heads * head_dim || q_out_tok_stride < int64_t{num_q_heads} * head_dim)
    return PA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !(eps <= 3.4e38f)) return PA_ERR_INVALID_ARG;   // NaN or infinite
  if (!(rope_theta > 0.0) || !(rope_theta <= 1.7e308)) return PA_ERR_INVALID_ARG;
  if ((q_norm_weight == nullptr) != (k_norm_weight == nullptr)) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!qkv || !positions || !slot_mapping || !q_out || !k_cache || !v_cache)
    return PA_ERR_INVALID_ARG;
  if (num_blocks > (INT32_MAX / block_size) + int64_t{1}) return PA_ERR_UNSUPPORTED;  // int32 slots
  if (!aligned16(qkv) || !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (qkv_tok_stride * eb) % 16 || (q_out_tok_stride * eb) % 16)
    return PA_ERR_UNSUPPORTED;
  if (q_norm_weight && (!aligned16(q_norm_weight) || !aligned16(k_norm_weight)))
    return PA_ERR_UNSUPPORTED;
  pa::RopeArgs a{qkv, qkv_tok_stride, q_norm_weight, k_norm_weight, positions, slot_mapping,
                 num_tokens, num_q_heads, num_kv_heads, head_dim, eps, rope_theta, q_out,
                 q_out_tok_stride, k_cache, v_cache, block_size, eb,
                 geom_of(cache_layout, num_kv_heads, block_size, head_dim)};
  return launched(pa::launch_norm_rope_store(a, stream));
}

int pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                             int32_t max_context_len, int32_t partition_tokens, size_t* bytes,
                             int32_t* num_splits) {
  if (!bytes || !num_splits) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (partition_tokens <= 0 || partition_tokens % 64 != 0) return PA_ERR_UNSUPPORTED;
  int32_t s = (max_context_len + partition_tokens - 1) / partition_tokens;
  if (s < 1) s = 1;
  *num_splits = s;
  // the split statistics, then pa_decode_shared_prefix's work list (a count and
  // one entry per (sequence, split))
  *bytes = pa::decode_ws_stats_bytes(num_seqs, num_q_heads, s, head_dim) +
           (static_cast<size_t>(num_seqs) * s * sizeof(int32_t) + sizeof(int32_t) + 15) / 16 * 16;
  return PA_OK;
}

namespace {

struct NewRows {  // the fused store of pa_store_decode / pa_store_prefill_varlen (k null: none)
  const void* k;
  const void* v;
  int64_t k_tok_stride, k_head_stride, v_tok_stride, v_head_stride;
  const int32_t* slot_mapping;
};

struct SharedPrefix {  // the groups of pa_decode_shared_prefix (group null: none)
  const int32_t* group;
  const int32_t* tokens;
  int32_t num_groups, max_tokens;
};

int decode_common(const void* q, int64_t q_seq_stride, int64_t q_head_stride,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  int64_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int64_t num_blocks, int32_t cache_layout,
                  int32_t max_context_len, int32_t partition_tokens, float scale,
                  void* workspace, size_t workspace_bytes, int32_t dtype, const NewRows& nr,
                  hipStream_t stream, const SharedPrefix& sp = SharedPrefix{}) {
  const int eb = elt_bytes(dtype);
  if (eb == 0 || !layout_ok(cache_layout)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_context_len < 0 || num_blocks <= 0 || block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (!group_ok(num_q_heads, num_kv_heads)) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
      return PA_ERR_INVALID_ARG;
    return PA_ERR_UNSUPPORTED;
  }
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_blocks > (int64_t{1} << 32) ||
      int64_t{block_size} * num_kv_heads * head_dim > int64_t{UINT32_MAX})
    return PA_ERR_UNSUPPORTED;  // 32-bit block ids and block strides
  if (q_seq_stride < 0 || q_head_stride < 0 || block_table_stride < 0) return PA_ERR_INVALID_ARG;
  if (nr.k && (nr.k_tok_stride < 0 || nr.k_head_stride < 0 || nr.v_tok_stride < 0 ||
               nr.v_head_stride < 0))
    return PA_ERR_INVALID_ARG;
  if (!(scale == scale)) return PA_ERR_INVALID_ARG;  // NaN scale
  size_t need = 0;
  int32_t splits = 0;
  int st = pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                    partition_tokens, &need, &splits);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !workspace)
    return PA_ERR_INVALID_ARG;
  if (nr.k && (!nr.v || !nr.slot_mapping)) return PA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (splits > 65535 || num_seqs > 65535) return PA_ERR_UNSUPPORTED;  // grid limits
  if (!aligned16(q) || (q_seq_stride * eb) % 16 || (q_head_stride * eb) % 16 ||
      !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace))
    return PA_ERR_UNSUPPORTED;
  if (nr.k && (!aligned16(nr.k) || !aligned16(nr.v) || (nr.k_tok_stride * eb) % 16 ||
               (nr.k_head_stride * eb) % 16 || (nr.v_tok_stride * eb) % 16 ||
               (nr.v_head_stride * eb) % 16))
    return PA_ERR_UNSUPPORTED;
  float* ws = static_cast<float*>(workspace);
  const size_t acc_elems = static_cast<size_t>(num_seqs) * num_q_heads * splits * head_dim;
  const pa::CacheGeom geom = geom_of(cache_layout, num_kv_heads, block_size, head_dim);
  // The shared-prefix pass runs only when some group can hold a whole split.
  const bool prefix = sp.group && sp.num_groups > 0 && sp.max_tokens >= partition_tokens;
  int32_t* work_list = reinterpret_cast<int32_t*>(
      static_cast<char*>(workspace) +
      pa::decode_ws_stats_bytes(num_seqs, num_q_heads, splits, head_dim));
  NewRows rows = nr;
  if (prefix) {
    // This step's store runs in the prefix pass's launch (its rows lie past every
    // group's prefix, so it never writes what that pass reads), and the partition
    // pass after it reads the stored rows from the cache.
    const pa::StoreArgs store{nr.k, nr.v, nr.k_tok_stride, nr.k_head_stride, nr.v_tok_stride,
                              nr.v_head_stride, const_cast<void*>(k_cache),
                              const_cast<void*>(v_cache), nr.slot_mapping, num_seqs,
                              num_kv_heads, head_dim, block_size, eb, geom};
    pa::PrefixArgs pa_args{q, q_seq_stride, q_head_stride, k_cache, v_cache, block_table,
                           block_table_stride, context_lens, sp.group, sp.tokens, sp.num_groups,
                           sp.max_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           block_size, partition_tokens, splits, scale, ws, ws + acc_elems,
                           geom, nr.k ? &store : nullptr, work_list, max_context_len};
    const int rc = launched(pa::launch_prefix_splits(pa_args, stream));
    if (rc != PA_OK) return rc;
    rows = NewRows{nullptr, nullptr, 0, 0, 0, 0, nullptr};
  }
  pa::DecodeArgs a{q, q_seq_stride, q_head_stride, k_cache, v_cache, block_table,
                   block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                   head_dim, block_size, max_context_len, partition_tokens, splits, scale, ws,
                   ws + acc_elems, dtype == PA_DTYPE_BF16, geom, rows.k, rows.v,
                   rows.k_tok_stride, rows.k_head_stride, rows.v_tok_stride, rows.v_head_stride,
                   rows.slot_mapping, prefix ? sp.group : nullptr, prefix ? sp.tokens : nullptr,
                   prefix ? sp.num_groups : 0, prefix ? sp.max_tokens : 0,
                   prefix ? work_list : nullptr};
  return launched(pa::launch_decode(a, stream));
}

}  // namespace

int pa_decode(const void* q, int64_t q_seq_stride, int64_t q_head_stride, const void* k_cache,
              const void* v_cache, const int32_t* block_table, int64_t block_table_stride,
              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
              int32_t cache_layout, int32_t max_context_len, int32_t partition_tokens,
              float scale, void* workspace, size_t workspace_bytes, int32_t dtype,
              hipStream_t stream) {
  return decode_common(q, q_seq_stride, q_head_stride, k_cache, v_cache, block_table,
                       block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, cache_layout, max_context_len,
                       partition_tokens, scale, workspace, workspace_bytes, dtype,
                       NewRows{nullptr, nullptr, 0, 0, 0, 0, nullptr}, stream);
}

int pa_store_decode(const void* k_new, const void* v_new, int64_t k_tok_stride,
                    int64_t k_head_stride, int64_t v_tok_stride, int64_t v_head_stride,
                    const int32_t* slot_mapping, const void* q, int64_t q_seq_stride,
                    int64_t q_head_stride, void* k_cache, void* v_cache,
                    const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, int32_t cache_layout, int32_t max_context_len,
                    int32_t partition_tokens, float scale, void* workspace,
                    size_t workspace_bytes, int32_t dtype, hipStream_t stream) {
  if (num_seqs > 0 && max_context_len > 0 && (!k_new || !v_new || !slot_mapping))
    return PA_ERR_INVALID_ARG;
  if (num_blocks > 0 && block_size > 0 && num_blocks > (INT32_MAX / block_size) + int64_t{1})
    return PA_ERR_UNSUPPORTED;  // int32 slots
  return decode_common(q, q_seq_stride, q_head_stride, k_cache, v_cache, block_table,
                       block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, cache_layout, max_context_len,
                       partition_tokens, scale, workspace, workspace_bytes, dtype,
                       NewRows{k_new, v_new, k_tok_stride, k_head_stride, v_tok_stride,
                               v_head_stride, slot_mapping},
                       stream);
}

int pa_decode_shared_prefix(const void* k_new, const void* v_new, int64_t k_tok_stride,
                            int64_t k_head_stride, int64_t v_tok_stride, int64_t v_head_stride,
                            const int32_t* slot_mapping, const void* q, int64_t q_seq_stride,
                            int64_t q_head_stride, void* k_cache, void* v_cache,
                            const int32_t* block_table, int64_t block_table_stride,
                            const int32_t* context_lens, const int32_t* prefix_group,
                            const int32_t* prefix_tokens, int32_t num_groups,
                            int32_t max_prefix_tokens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, int32_t cache_layout, int32_t max_context_len,
                            int32_t partition_tokens, float scale, void* workspace,
                            size_t workspace_bytes, int32_t dtype, hipStream_t stream) {
  if (dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;  // the prefix pass is bf16 MFMA
  if (num_groups < 0 || max_prefix_tokens < 0 || max_prefix_tokens > max_context_len)
    return PA_ERR_INVALID_ARG;
  // the store is all or nothing
  const bool store = k_new || v_new || slot_mapping;
  if (store && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  if (store && num_blocks > 0 && block_size > 0 &&
      num_blocks > (INT32_MAX / block_size) + int64_t{1})
    return PA_ERR_UNSUPPORTED;  // int32 slots
  if (num_groups > 0 && num_seqs > 0 && max_context_len > 0) {
    if (!prefix_group || !prefix_tokens) return PA_ERR_INVALID_ARG;
    if (num_kv_heads > 0 && int64_t{num_groups} * num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  }
  return decode_common(q, q_seq_stride, q_head_stride, k_cache, v_cache, block_table,
                       block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, cache_layout, max_context_len,
                       partition_tokens, scale, workspace, workspace_bytes, dtype,
                       NewRows{k_new, v_new, k_tok_stride, k_head_stride, v_tok_stride,
                               v_head_stride, slot_mapping},
                       stream, SharedPrefix{prefix_group, prefix_tokens, num_groups,
                                            max_prefix_tokens});
}

int pa_store_decode_noalloc(const void* k_new, const void* v_new, int64_t k_tok_stride,
                            int64_t k_head_stride, int64_t v_tok_stride, int64_t v_head_stride,
                            const int32_t* slot_mapping, const void* q, int64_t q_seq_stride,
                            int64_t q_head_stride, void* k_cache, void* v_cache,
                            const int32_t* block_table, int64_t block_table_stride,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, int32_t cache_layout, int32_t max_context_len,
                            int32_t partition_tokens, float scale, void* out,
                            int64_t out_seq_stride, int64_t out_head_stride, int32_t dtype,
                            hipStream_t stream) {
  // The size check comes first: a request larger than the fixed workspace is
  // refused before any pointer is looked at or any runtime call is made.
  size_t need = 0;
  int32_t splits = 0;
  if (num_q_heads <= 0 || head_dim <= 0) return PA_ERR_INVALID_ARG;
  const int st = pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                          partition_tokens, &need, &splits);
  if (st != PA_OK) return st;
  if (need > pa::kDecodeScratchBytes) return PA_ERR_WORKSPACE;
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  // the reduce's own output checks, before the store launch can change the caches
  const int eb = elt_bytes(dtype);
  if (!out || out_seq_stride < 0 || out_head_stride < 0) return PA_ERR_INVALID_ARG;
  if (eb == 0 || !head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
  const int64_t lane_bytes = int64_t{head_dim} / 64 * eb;
  if ((reinterpret_cast<uintptr_t>(out) % lane_bytes) || (out_seq_stride * eb) % lane_bytes ||
      (out_head_stride * eb) % lane_bytes)
    return PA_ERR_UNSUPPORTED;
  float* ws = nullptr;
  if (pa::decode_scratch(&ws) != hipSuccess) return PA_ERR_LAUNCH;
  const int rc = pa_store_decode(k_new, v_new, k_tok_stride, k_head_stride, v_tok_stride,
                                 v_head_stride, slot_mapping, q, q_seq_stride, q_head_stride,
                                 k_cache, v_cache, block_table, block_table_stride, context_lens,
                                 num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                 num_blocks, cache_layout, max_context_len, partition_tokens,
                                 scale, ws, pa::kDecodeScratchBytes, dtype, stream);
  if (rc != PA_OK) return rc;
  return pa_decode_reduce(ws, pa::kDecodeScratchBytes, context_lens, num_seqs, num_q_heads,
                          head_dim, splits, partition_tokens, out, out_seq_stride, out_head_stride,
                          dtype, stream);
}

int pa_decode_reduce(const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t num_splits,
                     int32_t partition_tokens, void* out, int64_t out_seq_stride,
                     int64_t out_head_stride, int32_t dtype, hipStream_t stream) {
  const int eb = elt_bytes(dtype);
  if (eb == 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_heads <= 0 || num_splits <= 0) return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
  if (partition_tokens <= 0 || partition_tokens % 64 != 0) return PA_ERR_UNSUPPORTED;
  if (out_seq_stride < 0 || out_head_stride < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!workspace || !context_lens || !out) return PA_ERR_INVALID_ARG;
  const size_t need =
      static_cast<size_t>(num_seqs) * num_q_heads * num_splits * (head_dim + 2) * sizeof(float);
  if (workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(out) % eb) != 0)
    return PA_ERR_UNSUPPORTED;
  // Each lane writes head_dim / 64 adjacent elements with one store.
  const int64_t lane_bytes = int64_t{head_dim} / 64 * eb;
  if ((reinterpret_cast<uintptr_t>(out) % lane_bytes) || (out_seq_stride * eb) % lane_bytes ||
      (out_head_stride * eb) % lane_bytes)
    return PA_ERR_UNSUPPORTED;
  const float* ws = static_cast<const float*>(workspace);
  const size_t acc_elems = static_cast<size_t>(num_seqs) * num_q_heads * num_splits * head_dim;
  pa::ReduceArgs a{ws, ws + acc_elems, context_lens, num_seqs, num_q_heads, head_dim, num_splits,
                   partition_tokens, out, out_seq_stride, out_head_stride,
                   dtype == PA_DTYPE_BF16};
  return launched(pa::launch_reduce(a, stream));
}

namespace {

// Prefill workspace layout (bytes): [0, kPrefillTicketBytes) the work-list
// counters; the work list (int2 per item, capacity items); then, when tiles
// are split, the split tiles and acc [S, total_q, Hq, D] and ml [S, total_q,
// Hq, 2] floats.
struct PrefillLayout {
  size_t items_off, merges_off, acc_off, ml_off, bytes;
};

PrefillLayout prefill_layout(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t splits) {
  auto round256 = [](size_t x) { return (x + 255) / 256 * 256; };
  const int64_t rows = pa::prefill_rows_per_tile(num_q_heads / num_kv_heads);
  const size_t tiles = static_cast<size_t>((total_q + rows - 1) / rows + num_seqs);
  const size_t capacity = tiles * splits * num_kv_heads;
  PrefillLayout l;
  l.items_off = pa::kPrefillTicketBytes;
  l.merges_off = round256(l.items_off + capacity * 8);
  l.acc_off = round256(l.merges_off + (splits > 1 ? tiles * 8 : 0));
  const size_t slots = splits > 1 ? static_cast<size_t>(splits) * total_q * num_q_heads : 0;
  l.ml_off = round256(l.acc_off + slots * head_dim * sizeof(float));
  l.bytes = round256(l.ml_off + slots * 2 * sizeof(float));
  return l;
}

}  // namespace

int pa_prefill_workspace_size(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen_k,
                              int32_t split_keys, size_t* bytes, int32_t* num_splits) {
  if (!bytes || !num_splits) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || total_q < 0 || head_dim <= 0 || max_seqlen_k < 0 || split_keys < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_INVALID_ARG;
  if (split_keys % 64 != 0) return PA_ERR_UNSUPPORTED;
  const int32_t s = split_keys == 0 ? 1 : (max_seqlen_k + split_keys - 1) / split_keys;
  *num_splits = s > 1 ? s : 1;
  *bytes = prefill_layout(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, *num_splits)
               .bytes;
  return PA_OK;
}

namespace {

int prefill_common(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                   const void* k_cache, const void* v_cache, const int32_t* cu_seqlens_q,
                   const int32_t* cu_seqlens_k, const int32_t* block_table,
                   int64_t block_table_stride, int32_t num_seqs, int32_t total_q,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, int32_t cache_layout,
                   int32_t max_seqlen_q, int32_t max_seqlen_k, float scale, int32_t split_keys,
                   void* workspace, size_t workspace_bytes, void* out, int64_t out_tok_stride,
                   int64_t out_head_stride, int32_t dtype, const NewRows& nr,
                   hipStream_t stream, bool planned = false) {
  const int eb = elt_bytes(dtype);
  if (eb == 0 || !layout_ok(cache_layout)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_blocks <= 0 ||
      block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (max_seqlen_q > max_seqlen_k) return PA_ERR_INVALID_ARG;
  if (!group_ok(num_q_heads, num_kv_heads)) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
      return PA_ERR_INVALID_ARG;
    return PA_ERR_UNSUPPORTED;
  }
  if (dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (q_tok_stride < 0 || q_head_stride < 0 || out_tok_stride < 0 || out_head_stride < 0 ||
      block_table_stride < 0)
    return PA_ERR_INVALID_ARG;
  if (nr.k && (nr.k_tok_stride < 0 || nr.k_head_stride < 0 || nr.v_tok_stride < 0 ||
               nr.v_head_stride < 0))
    return PA_ERR_INVALID_ARG;
  // the tile kernel reads 64 of this step's rows with 32-bit offsets
  if (nr.k && (nr.k_tok_stride > (int64_t{1} << 23) || nr.v_tok_stride > (int64_t{1} << 23)))
    return PA_ERR_UNSUPPORTED;
  if (!(scale > 0.f)) return PA_ERR_INVALID_ARG;  // also rejects NaN
  size_t need = 0;
  int32_t splits = 1;
  const int st = pa_prefill_workspace_size(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                                           max_seqlen_k, split_keys, &need, &splits);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PA_OK;
  if (num_seqs > pa::kPrefillPlanMaxSeqs) return PA_ERR_UNSUPPORTED;
  {  // work items hold the query tile and the key range in 16 bits each
    const int64_t rows = pa::prefill_rows_per_tile(num_q_heads / num_kv_heads);
    if ((max_seqlen_q + rows - 1) / rows > 65535 || splits > 32767) return PA_ERR_UNSUPPORTED;
  }
  if (num_blocks > INT32_MAX / block_size) return PA_ERR_UNSUPPORTED;  // 32-bit slots
  // the sequence's block-table entries are staged in LDS next to two K/V tiles
  if ((max_seqlen_k + int64_t{block_size} - 1) / block_size > kPrefillMaxTableEntries)
    return PA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !cu_seqlens_k || !block_table || !out ||
      !workspace)
    return PA_ERR_INVALID_ARG;
  if (nr.k && (!nr.v || !nr.slot_mapping)) return PA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (q_tok_stride * eb) % 16 || (q_head_stride * eb) % 16 || (out_tok_stride * eb) % 16 ||
      (out_head_stride * eb) % 16)
    return PA_ERR_UNSUPPORTED;
  if (nr.k && (!aligned16(nr.k) || !aligned16(nr.v) || (nr.k_tok_stride * eb) % 16 ||
               (nr.k_head_stride * eb) % 16 || (nr.v_tok_stride * eb) % 16 ||
               (nr.v_head_stride * eb) % 16))
    return PA_ERR_UNSUPPORTED;
  const PrefillLayout lay =
      prefill_layout(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, splits);
  const pa::CacheGeom geom = geom_of(cache_layout, num_kv_heads, block_size, head_dim);
  // the store of this step's rows (one per query row), when asked for
  const pa::StoreArgs store{nr.k, nr.v, nr.k_tok_stride, nr.k_head_stride, nr.v_tok_stride,
                            nr.v_head_stride, const_cast<void*>(k_cache),
                            const_cast<void*>(v_cache), nr.slot_mapping, total_q, num_kv_heads,
                            head_dim, block_size, eb, geom};
  pa::PrefillArgs a{q, q_tok_stride, q_head_stride, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k,
                    block_table, block_table_stride, num_seqs, num_q_heads, num_kv_heads,
                    head_dim, block_size, max_seqlen_q, max_seqlen_k, total_q, scale,
                    split_keys, splits, static_cast<uint32_t*>(workspace),
                    reinterpret_cast<int2*>(static_cast<char*>(workspace) + lay.items_off),
                    reinterpret_cast<int2*>(static_cast<char*>(workspace) + lay.merges_off),
                    reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.acc_off),
                    reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.ml_off),
                    out, out_tok_stride, out_head_stride, geom, nr.k ? &store : nullptr,
                    planned, false};
  return launched(pa::launch_prefill(a, stream));
}

// The shape checks pa_prefill_plan shares with the prefill calls (the ones
// that decide the work list and the workspace); PA_OK or the error.
int plan_checks(int32_t num_seqs, int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                int32_t head_dim, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t split_keys,
                size_t* need, int32_t* splits) {
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return PA_ERR_INVALID_ARG;
  if (max_seqlen_q > max_seqlen_k) return PA_ERR_INVALID_ARG;
  if (!group_ok(num_q_heads, num_kv_heads)) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
      return PA_ERR_INVALID_ARG;
    return PA_ERR_UNSUPPORTED;
  }
  if (!head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
  const int st = pa_prefill_workspace_size(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                                           max_seqlen_k, split_keys, need, splits);
  if (st != PA_OK) return st;
  if (num_seqs > pa::kPrefillPlanMaxSeqs) return PA_ERR_UNSUPPORTED;
  const int64_t rows = pa::prefill_rows_per_tile(num_q_heads / num_kv_heads);
  if ((max_seqlen_q + rows - 1) / rows > 65535 || *splits > 32767) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

}  // namespace

int pa_prefill_varlen(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                      const void* k_cache, const void* v_cache, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, const int32_t* block_table,
                      int64_t block_table_stride, int32_t num_seqs, int32_t total_q,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks, int32_t cache_layout,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, float scale,
                      int32_t split_keys, void* workspace, size_t workspace_bytes, void* out,
                      int64_t out_tok_stride, int64_t out_head_stride, int32_t dtype,
                      hipStream_t stream) {
  return prefill_common(q, q_tok_stride, q_head_stride, k_cache, v_cache, cu_seqlens_q,
                        cu_seqlens_k, block_table, block_table_stride, num_seqs, total_q,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        cache_layout, max_seqlen_q, max_seqlen_k, scale, split_keys, workspace,
                        workspace_bytes, out, out_tok_stride, out_head_stride, dtype,
                        NewRows{nullptr, nullptr, 0, 0, 0, 0, nullptr}, stream);
}

int pa_store_prefill_varlen(const void* k_new, const void* v_new, int64_t k_tok_stride,
                            int64_t k_head_stride, int64_t v_tok_stride, int64_t v_head_stride,
                            const int32_t* slot_mapping, const void* q, int64_t q_tok_stride,
                            int64_t q_head_stride, void* k_cache, void* v_cache,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            const int32_t* block_table, int64_t block_table_stride,
                            int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, int32_t cache_layout, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, float scale, int32_t split_keys,
                            void* workspace, size_t workspace_bytes, void* out,
                            int64_t out_tok_stride, int64_t out_head_stride, int32_t dtype,
                            hipStream_t stream) {
  if (num_seqs > 0 && total_q > 0 && max_seqlen_q > 0 && (!k_new || !v_new || !slot_mapping))
    return PA_ERR_INVALID_ARG;
  return prefill_common(q, q_tok_stride, q_head_stride, k_cache, v_cache, cu_seqlens_q,
                        cu_seqlens_k, block_table, block_table_stride, num_seqs, total_q,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        cache_layout, max_seqlen_q, max_seqlen_k, scale, split_keys, workspace,
                        workspace_bytes, out, out_tok_stride, out_head_stride, dtype,
                        NewRows{k_new, v_new, k_tok_stride, k_head_stride, v_tok_stride,
                                v_head_stride, slot_mapping},
                        stream);
}

int pa_prefill_plan(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                    int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t split_keys,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  int32_t splits = 1;
  const int st = plan_checks(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, max_seqlen_q,
                             max_seqlen_k, split_keys, &need, &splits);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PA_OK;
  if (!cu_seqlens_q || !cu_seqlens_k || !workspace) return PA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_UNSUPPORTED;
  const PrefillLayout lay =
      prefill_layout(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, splits);
  pa::PrefillArgs a{nullptr, 0, 0, nullptr, nullptr, cu_seqlens_q, cu_seqlens_k, nullptr, 0,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, 8, max_seqlen_q, max_seqlen_k,
                    total_q, 1.f, split_keys, splits, static_cast<uint32_t*>(workspace),
                    reinterpret_cast<int2*>(static_cast<char*>(workspace) + lay.items_off),
                    reinterpret_cast<int2*>(static_cast<char*>(workspace) + lay.merges_off),
                    nullptr, nullptr, nullptr, 0, 0, pa::CacheGeom{0, 0, 0}, nullptr, false,
                    true};
  return launched(pa::launch_prefill(a, stream));
}

int pa_prefill_varlen_planned(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                              const void* k_cache, const void* v_cache,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              const int32_t* block_table, int64_t block_table_stride,
                              int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, int32_t cache_layout, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, float scale, int32_t split_keys,
                              void* workspace, size_t workspace_bytes, void* out,
                              int64_t out_tok_stride, int64_t out_head_stride, int32_t dtype,
                              hipStream_t stream) {
  return prefill_common(q, q_tok_stride, q_head_stride, k_cache, v_cache, cu_seqlens_q,
                        cu_seqlens_k, block_table, block_table_stride, num_seqs, total_q,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        cache_layout, max_seqlen_q, max_seqlen_k, scale, split_keys, workspace,
                        workspace_bytes, out, out_tok_stride, out_head_stride, dtype,
                        NewRows{nullptr, nullptr, 0, 0, 0, 0, nullptr}, stream, true);
}

int pa_store_prefill_varlen_planned(
    const void* k_new, const void* v_new, int64_t k_tok_stride, int64_t k_head_stride,
    int64_t v_tok_stride, int64_t v_head_stride, const int32_t* slot_mapping, const void* q,
    int64_t q_tok_stride, int64_t q_head_stride, void* k_cache, void* v_cache,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* block_table,
    int64_t block_table_stride, int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    int32_t cache_layout, int32_t max_seqlen_q, int32_t max_seqlen_k, float scale,
    int32_t split_keys, void* workspace, size_t workspace_bytes, void* out,
    int64_t out_tok_stride, int64_t out_head_stride, int32_t dtype, hipStream_t stream) {
  if (num_seqs > 0 && total_q > 0 && max_seqlen_q > 0 && (!k_new || !v_new || !slot_mapping))
    return PA_ERR_INVALID_ARG;
  return prefill_common(q, q_tok_stride, q_head_stride, k_cache, v_cache, cu_seqlens_q,
                        cu_seqlens_k, block_table, block_table_stride, num_seqs, total_q,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        cache_layout, max_seqlen_q, max_seqlen_k, scale, split_keys, workspace,
                        workspace_bytes, out, out_tok_stride, out_head_stride, dtype,
                        NewRows{k_new, v_new, k_tok_stride, k_head_stride, v_tok_stride,
                                v_head_stride, slot_mapping},
                        stream, true);
}

}  // extern "C"
