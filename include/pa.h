/*
 * pa.h -- C ABI of the MI355X (gfx950) paged KV-cache attention library.
 *
 * The library implements the attention step of a nano-vLLM-style inference
 * engine over a paged KV cache: the per-head q/k norm and rotary embedding
 * that precede the cache, storing this step's K/V rows through a slot
 * mapping, variable-length causal prefill, and batched single-token decode
 * with a split-K (flash-decoding) partition plus a reduce.
 *
 * Sources (web pages describing the method):
 *   [Intro]   "大模型推理入门与 nano-vLLM 源码详解" (duanmeng.github.io)
 *   [Pico #6] "Pico-vLLM 开发日志 #6" on Fain's blog (koas-w.github.io)
 *   [Log-walk] "对着日志读懂 nano-vllm" (juejin.cn)
 *   [Pico #8] "Pico-vLLM 开发日志 #8 更多Triton Kernel和性能优化" (koas-w.github.io)
 *   [Analysis] "nano-vllm 技术分析" (deepseek.csdn.net)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named *_cache, q, k, v, qkv, q_out, *_weight, out, workspace,
 *   slot_mapping, positions, block_table, context_lens, cu_seqlens_* are
 *   DEVICE pointers; every other argument is a host value.  The caller owns
 *   all memory (the library never allocates, frees, synchronises, or reads
 *   device memory from the host).
 *   All work is enqueued on `stream` (may be 0 for the null stream); launch
 *   shapes depend only on host arguments, so calls can be captured in a HIP
 *   graph.
 * - KV cache layout: k_cache, v_cache are contiguous arrays of `dtype`, one
 *   layer's slice of the engine pool, in one of two layouts chosen by
 *   `cache_layout`:
 *     PA_CACHE_BSHD  [num_blocks, block_size, num_kv_heads, head_dim], the
 *                    nano-vLLM pool [Intro §11.5]: a slot's heads are adjacent;
 *     PA_CACHE_BHSD  [num_blocks, num_kv_heads, block_size, head_dim], the
 *                    Pico-vLLM pool [Pico #6]: a head's slots within a block
 *                    are adjacent.
 *   Slot s is block s / block_size, offset s % block_size [Intro §9.2].
 * - dtype: PA_DTYPE_F32 or PA_DTYPE_BF16.  q, k, v, qkv, q_out, the norm
 *   weights, caches and out all share it.  Arithmetic is fp32 throughout; outputs are rounded to `dtype`
 *   (round to nearest even for bf16).
 * - head_dim in {64, 128}; block_size a power of two in [8, 1024];
 *   num_q_heads a multiple of num_kv_heads with a group size
 *   num_q_heads / num_kv_heads in {1, 2, 4, 8}.  Query head h reads kv head
 *   h / group (consecutive query heads share a kv head [Intro §19.6]).
 * - Strides are in elements; the innermost (head_dim) stride is always 1.
 *   Vector loads need 16-byte alignment of device pointers and of
 *   stride * sizeof(dtype); pa_store_kv falls back to element copies when a
 *   source is not aligned, the other entry points reject misalignment.
 * - Device-resident values are not validated: slots, block-table entries,
 *   lengths and cu_seqlens must be in range, else the behaviour is undefined.
 *   Documented sentinels: slot -1 (no write), block-table entries past a
 *   sequence's ceil(len / block_size) blocks (never read, so -1 padding is
 *   legal), context_len 0 (output zeros).
 * - cache_layout: PA_CACHE_BSHD or PA_CACHE_BHSD (anything else:
 *   PA_ERR_UNSUPPORTED); the same value must be used by every call that
 *   touches one cache.
 * - Return value: PA_OK, or a negative PA_ERR_* code.  Argument checks run on
 *   the host before any launch; a failed launch returns PA_ERR_LAUNCH.
 *   pa_strerror() names a code.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shape */
  PA_ERR_UNSUPPORTED = -2, /* head_dim, block_size, group, dtype or alignment */
  PA_ERR_WORKSPACE = -3,   /* workspace too small for the requested split */
  PA_ERR_LAUNCH = -4       /* the HIP runtime reported a launch error */
};

enum pa_dtype { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 };

enum pa_cache_layout { PA_CACHE_BSHD = 0, PA_CACHE_BHSD = 1 };

/* Library version as major * 10000 + minor * 100 + patch. */
int pa_version(void);

/* Static description of a status code. */
const char* pa_strerror(int status);

/*
 * pa_store_kv -- write this step's K and V rows into the paged cache.
 *
 * Defined by [Intro §13.1] and the store of [Pico #6]: for each new token i
 * with s = slot_mapping[i] != -1, copy k[i, h, :] to the row of kv head h at
 * slot s of k_cache (k_cache[s / block_size, s % block_size, h, :] in
 * PA_CACHE_BSHD) for every kv head h, and the same for v.  A slot of -1 is a
 * padding row [Intro §13.5] and writes nothing.  The copy is bitwise (NaN
 * payloads, signed zeros survive).
 *
 *   k, v               [num_tokens, num_kv_heads, head_dim], token strides
 *                      k_tok_stride / v_tok_stride and head strides
 *                      k_head_stride / v_head_stride (elements, may describe a
 *                      view into a fused QKV buffer [Pico #6, pitfall 1]).
 *   k_cache, v_cache   as in the conventions; num_blocks physical blocks, laid
 *                      out as cache_layout says.
 *   slot_mapping       int32 [num_tokens]; unique slots in
 *                      [0, num_blocks * block_size), or -1.
 * num_tokens == 0 is a no-op.  Slots must not repeat within a call (which
 * write wins would be unspecified).
 */
int pa_store_kv(const void* k, const void* v, int64_t k_tok_stride, int64_t k_head_stride,
                int64_t v_tok_stride, int64_t v_head_stride, void* k_cache, void* v_cache,
                const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t cache_layout,
                int32_t dtype, hipStream_t stream);

/*
 * pa_qk_norm_rope_store -- per-head q/k RMSNorm, rotary position embedding,
 * and the store of this step's rotated K and raw V into the paged cache.
 *
 * Defined by [Intro §12.2, §19.3, §19.7], [Analysis §4.2, §4.4] ("nano-vllm
 * 技术分析", deepseek.csdn.net) and the fused RoPE + cache-store kernel of
 * [Pico #8 §1] ("Pico-vLLM 开发日志 #8"): token t's projection row holds
 * num_q_heads Q heads, then num_kv_heads K heads, then num_kv_heads V heads,
 * head_dim features each.  Every Q and K head x becomes
 *   y_i = gamma_i * x_i / sqrt(mean_j(x_j^2) + eps)      (gamma: q_norm_weight
 * for Q heads, k_norm_weight for K heads; both NULL: y = x, the model without
 * q/k norm), then each pair (y_i, y_{i+d/2}), i < d/2, is turned by
 * phi = positions[t] * rope_theta^(-2i/d) radians:
 *   y_i' = y_i cos(phi) - y_{i+d/2} sin(phi),  y_{i+d/2}' = y_i sin(phi) + y_{i+d/2} cos(phi).
 * Rotated Q goes to q_out[t]; rotated K and the V row, copied bit for bit, go
 * to slot s = slot_mapping[t] as pa_store_kv writes them (s = -1: K and V are
 * not written, q_out[t] still is).  Arithmetic is fp32 (the angle and its
 * reduction to one turn are fp64); each result is rounded once to dtype.
 *
 *   qkv             [num_tokens, >= (num_q_heads + 2 * num_kv_heads) * head_dim]
 *                   of dtype, row stride qkv_tok_stride (elements).
 *   q_norm_weight,  [head_dim] of dtype each, or both NULL.
 *   k_norm_weight
 *   positions       int32 [num_tokens], the tokens' logical positions (any value).
 *   slot_mapping    int32 [num_tokens] as for pa_store_kv.
 *   q_out           [num_tokens, num_q_heads, head_dim] of dtype, row stride
 *                   q_out_tok_stride >= num_q_heads * head_dim; it may be the Q
 *                   part of qkv itself (same rows: an in-place update), no other
 *                   overlap.
 *   k_cache, v_cache  as in the conventions.
 * eps must be finite and >= 0, rope_theta finite and > 0.  head_dim 64 or 128;
 * any num_q_heads, num_kv_heads >= 1 (no head reads another here, so the
 * group-size rule does not apply).  Every device pointer and both strides (in
 * bytes) must be 16-byte aligned.  num_tokens == 0 is a no-op.
 */
int pa_qk_norm_rope_store(const void* qkv, int64_t qkv_tok_stride, const void* q_norm_weight,
                          const void* k_norm_weight, const int32_t* positions,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, float eps, double rope_theta,
                          void* q_out, int64_t q_out_tok_stride, void* k_cache, void* v_cache,
                          int32_t block_size, int64_t num_blocks, int32_t cache_layout,
                          int32_t dtype, hipStream_t stream);

/*
 * pa_decode_workspace_size -- host-only helper for pa_decode.
 *
 * A decode of num_seqs sequences whose longest context is max_context_len,
 * cut into splits of partition_tokens logical positions, uses
 * num_splits = max(1, ceil(max_context_len / partition_tokens)) splits and a
 * workspace of
 *
 *   acc [num_seqs, num_q_heads, num_splits, head_dim] float   then
 *   ml  [num_seqs, num_q_heads, num_splits, 2] float          then, from the
 *       next 16-byte boundary,
 *   list [1 + num_seqs * num_splits] int32 (rounded up to 16 bytes)
 *
 * acc is the split's un-normalised output sum_j 2^(t_j - m) v_j, ml holds
 * m = max_j t_j and l = sum_j 2^(t_j - m), where t_j = scale * log2(e) * q.k_j
 * is the score in base-2 units and j runs over the split's readable positions
 * [Intro §9.5, §13.3].  Splits at or past a sequence's context are not written.
 * list is pa_decode_shared_prefix's work list for its partition pass (a count,
 * then the (sequence, split) pairs it computes), rewritten by every such call;
 * no other call reads or writes it.  partition_tokens must be a positive
 * multiple of 64.
 */
int pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                             int32_t max_context_len, int32_t partition_tokens, size_t* bytes,
                             int32_t* num_splits);

/*
 * pa_decode -- split-K partition pass of batched single-token decode.
 *
 * Defined by the decode path of [Intro §9.5, §11.4, §13.2] and the paged
 * decode kernel of [Pico #6]: sequence b has context_lens[b] readable keys,
 * including the token stored this step (so store before decode); query head h
 * of sequence b attends, with weights softmax(scale * q.k_j), over positions
 * 0..context_lens[b]-1 gathered through block_table[b].  This pass writes the
 * per-split statistics described at pa_decode_workspace_size; pa_decode_reduce
 * turns them into the output.
 *
 *   q             [num_seqs, num_q_heads, head_dim], strides q_seq_stride,
 *                 q_head_stride.
 *   block_table   int32 [num_seqs, >= ceil(max_context_len / block_size)]
 *                 with row stride block_table_stride.
 *   context_lens  int32 [num_seqs], each in [0, max_context_len].
 *   workspace     float, at least the size pa_decode_workspace_size gives
 *                 (workspace_bytes is checked).
 */
int pa_decode(const void* q, int64_t q_seq_stride, int64_t q_head_stride, const void* k_cache,
              const void* v_cache, const int32_t* block_table, int64_t block_table_stride,
              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
              int32_t cache_layout, int32_t max_context_len, int32_t partition_tokens,
              float scale, void* workspace, size_t workspace_bytes, int32_t dtype,
              hipStream_t stream);

/*
 * pa_store_decode -- pa_store_kv of one new token per sequence and the
 * pa_decode partition pass, in one launch.
 *
 * The decode step of [Intro §13.1, §13.2] (store this step's K/V, then
 * attend) for the batch where sequence b has exactly one new token, row b of
 * k_new / v_new, at position context_lens[b] - 1 and slot slot_mapping[b]
 * (-1: no store).  A padding row has slot -1 and context_lens[b] = 0; a row
 * with one of the two and not the other is invalid.  When the fused launch
 * would keep fewer waves resident than the grid needs while the plain
 * partition kernel would not, the library stores first in a launch of its
 * own; the results are the same bits either way.  The cache rows at those slots afterwards hold the new K/V exactly as
 * pa_store_kv writes them, and the workspace holds exactly what pa_decode
 * writes after that store (bit for bit); follow with pa_decode_reduce.
 * slot_mapping[b] must be the slot block_table[b] gives position
 * context_lens[b] - 1 (the slot the engine computes for it [Intro §11.4]).
 *
 *   k_new, v_new   [num_seqs, num_kv_heads, head_dim] of dtype, strides
 *                  k_tok_stride / k_head_stride and v_tok_stride /
 *                  v_head_stride (elements, 16-byte aligned rows).
 *   slot_mapping   int32 [num_seqs].
 * Every other argument is as for pa_decode; the caches are written, so they
 * are not const here.
 */
int pa_store_decode(const void* k_new, const void* v_new, int64_t k_tok_stride,
                    int64_t k_head_stride, int64_t v_tok_stride, int64_t v_head_stride,
                    const int32_t* slot_mapping, const void* q, int64_t q_seq_stride,
                    int64_t q_head_stride, void* k_cache, void* v_cache,
                    const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, int32_t cache_layout, int32_t max_context_len,
                    int32_t partition_tokens, float scale, void* workspace,
                    size_t workspace_bytes, int32_t dtype, hipStream_t stream);

/*
 * pa_decode_shared_prefix -- the partition pass of pa_decode (or, with this
 * step's rows, of pa_store_decode) for a batch in which groups of sequences
 * share the physical blocks of a common prefix: the prefix cache of
 * [Intro §10.5], whose sequences that begin with the same prompt point their
 * first block-table entries at the same blocks.
 *
 * Sequence b belongs to group prefix_group[b] (-1: none).  Every member of
 * group g holds the same block ids in the first ceil(T_g / block_size)
 * entries of its block_table row, where T_g = min(prefix_tokens[g],
 * max_prefix_tokens).  For a member with L = context_lens[b] positions, its
 * splits s < min(floor(T_g / partition_tokens), floor((L - 1) /
 * partition_tokens)) -- the splits wholly inside the shared prefix, never the
 * one holding its last position -- are computed for all members of the group
 * together by a bf16 MFMA pass that reads each prefix key once per 32 query
 * rows (all query heads of a kv head, 32 / G members at a time) instead of once
 * per sequence; the partition pass skips them and computes every other split
 * as pa_decode does.  Afterwards the workspace holds the split statistics
 * pa_decode defines (the prefix splits agree with pa_decode's to fp32
 * rounding: P enters the MFMA as a bf16 head plus a bf16 remainder); follow
 * with pa_decode_reduce.
 *
 *   k_new, v_new, slot_mapping   this step's store as in pa_store_decode, or
 *                  all three NULL for none (then the caches are only read).  The
 *                  store runs in the prefix pass's launch, alongside its reads of
 *                  the shared blocks, and the partition pass after it reads the
 *                  stored rows from the cache; so no stored slot may be one the
 *                  prefix pass reads: a member's new token (position L - 1) must
 *                  lie past its group's prefix, L > prefix_tokens[g], and no
 *                  slot_mapping entry may point at a group's first T_g positions
 *                  (a step that does write there stores first, with
 *                  pa_store_kv).
 *   prefix_group   int32 [num_seqs], each -1 or in [0, num_groups).
 *   prefix_tokens  int32 [num_groups], the shared length of each group.
 *   max_prefix_tokens   a bound on prefix_tokens, at most max_context_len
 *                  (larger values are cut to it); it sizes the launch.
 * Members are found on the device, so a group may be any subset of the batch;
 * the pass launches ceil(num_seqs * G / 32) x (num_groups * num_kv_heads) x
 * (max_prefix_tokens / partition_tokens) workgroups, of which those past a
 * group's members or prefix return at once, so it suits batches with a few
 * groups.  The same launch carries this step's store (when asked for) and
 * writes the partition pass's work list to the workspace's tail (see
 * pa_decode_workspace_size): the (sequence, split) pairs that pass computes,
 * full splits first and then the partial ones longest first, which the
 * partition launch then takes in that order.  With num_groups = 0 (or
 * max_prefix_tokens < partition_tokens) this is pa_decode / pa_store_decode.
 * bf16 only (PA_ERR_UNSUPPORTED otherwise); every other argument and the error
 * behaviour are as for pa_store_decode.
 */
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
                            size_t workspace_bytes, int32_t dtype, hipStream_t stream);

/*
 * pa_store_decode_noalloc -- pa_store_decode followed by pa_decode_reduce, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid it).
 *
 * The split workspace is a fixed device array inside the library, 64 MiB on
 * every GPU it runs on, held until the process ends; nothing is allocated or
 * freed by this call.  A request whose workspace (the size
 * pa_decode_workspace_size gives) exceeds 64 MiB returns PA_ERR_WORKSPACE
 * before anything is launched.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from different host
 * threads without ordering) race and give undefined results; calls ordered on
 * one stream do not.  The array needs no clearing between calls (each call
 * writes every split statistic it reads).
 *
 * Arguments are those of pa_store_decode without workspace / workspace_bytes,
 * plus out, out_seq_stride, out_head_stride as for pa_decode_reduce; the
 * results are bit for bit those of pa_store_decode then pa_decode_reduce.
 */
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
                            hipStream_t stream);

/*
 * pa_decode_reduce -- merge the splits written by pa_decode.
 *
 * [Intro §9.5]: with m* = max_s m_s, out = sum_s 2^(m_s - m*) acc_s /
 * sum_s 2^(m_s - m*) l_s over the splits s < ceil(context_lens[b] /
 * partition_tokens) -- never a sum of per-split normalised outputs.  A
 * sequence with context_len 0 gets zeros.
 *
 *   out   [num_seqs, num_q_heads, head_dim] of dtype, strides out_seq_stride,
 *         out_head_stride.
 * num_splits and partition_tokens must be the values pa_decode used.
 */
int pa_decode_reduce(const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t num_splits,
                     int32_t partition_tokens, void* out, int64_t out_seq_stride,
                     int64_t out_head_stride, int32_t dtype, hipStream_t stream);

/*
 * pa_prefill_workspace_size -- host-only helper for pa_prefill_varlen.
 *
 * The prefill runs as a fixed set of workgroups (one per resident slot) that
 * take work items -- (sequence, kv head, query tile, key range) -- from a
 * device-built list ordered largest first, so a batch with one long sequence
 * still keeps every compute unit busy.  A query tile whose keys span
 * more than split_keys positions is cut into ceil(keys / split_keys) key
 * ranges of equal length (whole 64-key tiles, at most split_keys keys each);
 * the ranges' partial results (the flash-decoding split of [Intro §9.5]
 * applied to prefill) meet in a merge pass.  A sequence with one query
 * position (a decode row of a mixed batch) is never cut: its item reads its
 * keys decode-style, split over the workgroup's waves.  With S = ceil(max_seqlen_k /
 * split_keys) (S = 1 when split_keys is 0, the no-split setting) the
 * workspace holds, in order and 256-byte aligned: the work-list counters
 * (512 bytes), the work list ((ceil(total_q / R) + num_seqs) * S *
 * num_kv_heads entries of 8 bytes, R = 32 * max(1, 4 / group) query rows per
 * tile), and when S > 1 the list of split query tiles ((ceil(total_q / R) +
 * num_seqs) entries of 8 bytes) and
 *
 *   acc [S, total_q, num_q_heads, head_dim]   then
 *   ml  [S, total_q, num_q_heads, 2]
 *
 * floats: acc is a range's un-normalised output, ml its (m, l) in base-2
 * units as for decode.  The library rewrites all of it on every call, so it
 * needs no initialisation; a workspace serves one call at a time.
 * split_keys must be 0 or a positive multiple of 64.
 */
int pa_prefill_workspace_size(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen_k,
                              int32_t split_keys, size_t* bytes, int32_t* num_splits);

/*
 * pa_prefill_varlen -- variable-length causal prefill over the paged cache.
 *
 * Defined by [Intro §10.2, §11.2, §13.2, §13.3]: sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (Lq rows) and Lk = cu_seqlens_k[b+1]
 * - cu_seqlens_k[b] keys, read from the paged cache through block_table[b]
 * (store this step's K/V first).  With c = Lk - Lq cached positions, query row
 * i sits at position c + i and attends to positions 0..c+i (a causal mask
 * aligned to the bottom-right).  Scores are scale * q.k in fp32; the softmax
 * runs online in fp32; both matrix products run on bf16 MFMA tiles.  The
 * probabilities enter P.V rounded to nearest bf16 (8 significant bits), except
 * for a block of 32 query rows whose first row sees fewer than 256 keys: there
 * they enter as a truncated bf16 head plus the bf16 remainder (about 16
 * significant bits), because with few keys the weight sits on a few values
 * and bf16 rounding alone can exceed the stated error bound.
 *
 *   q, out        [total_q, num_q_heads, head_dim] (total_q = cu_seqlens_q[num_seqs]),
 *                 strides q_tok_stride / q_head_stride, out_tok_stride /
 *                 out_head_stride.
 *   cu_seqlens_q, cu_seqlens_k  int32 [num_seqs + 1], non-decreasing, 0 first,
 *                 with Lq <= Lk per sequence, Lq <= max_seqlen_q and
 *                 Lk <= max_seqlen_k.
 *   block_table   int32 [num_seqs, >= ceil(max_seqlen_k / block_size)],
 *                 row stride block_table_stride.
 *   split_keys    keys per workgroup for long query tiles (0: never split, a
 *                 positive multiple of 64 otherwise); splitting shortens the
 *                 longest workgroup's key loop when one sequence dominates.
 *   workspace     device buffer of at least the bytes pa_prefill_workspace_size
 *                 gives for the same sizes and split_keys, 16-byte aligned;
 *                 workspace_bytes is checked.
 * scale must be positive.  Supported: dtype bf16 (head_dim 64 or 128),
 * num_seqs <= 4096 and ceil(max_seqlen_k / block_size) <= 8192;
 * PA_DTYPE_F32 returns PA_ERR_UNSUPPORTED.  Enqueues the work-list build, the
 * tile kernel and, when S > 1, the merge.
 */
int pa_prefill_varlen(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                      const void* k_cache, const void* v_cache, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, const int32_t* block_table,
                      int64_t block_table_stride, int32_t num_seqs, int32_t total_q,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks, int32_t cache_layout,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, float scale,
                      int32_t split_keys, void* workspace, size_t workspace_bytes, void* out,
                      int64_t out_tok_stride, int64_t out_head_stride, int32_t dtype,
                      hipStream_t stream);

/*
 * pa_store_prefill_varlen -- pa_store_kv of this step's new rows and
 * pa_prefill_varlen in the prefill's own launches.
 *
 * [Intro §13.1, §13.2]: the prefill step stores the new tokens' K/V, then
 * attends over the paged cache.  The new tokens are the query rows: row i of
 * k_new / v_new is query row i's token and goes to slot slot_mapping[i] (-1:
 * not stored), exactly as pa_store_kv writes it.  The tile kernel reads the
 * keys of this step's positions from k_new / v_new rather than from the cache,
 * and each work item writes the rows of its own query positions to the cache
 * from the tiles it holds, so no pass of its own stores them.  The output and
 * the pool are bit for bit those of pa_store_kv followed by pa_prefill_varlen
 * when each row's slot_mapping entry is the slot its position has in the
 * sequence's block_table (as an engine's metadata always has it); a row
 * stored at another slot, or not at all, is still read from k_new / v_new.
 *
 *   k_new, v_new   [total_q, num_kv_heads, head_dim] of dtype, strides
 *                  k_tok_stride / k_head_stride and v_tok_stride /
 *                  v_head_stride (elements, 16-byte aligned rows; token
 *                  strides of at most 2^23 elements).
 *   slot_mapping   int32 [total_q].
 * Every other argument is as for pa_prefill_varlen; the caches are written,
 * so they are not const here.
 */
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
                            hipStream_t stream);

/*
 * pa_prefill_plan -- build pa_prefill_varlen's work list once for a batch.
 *
 * The work list (the (sequence, kv head, query tile, key range) items in
 * largest-first order) depends only on cu_seqlens_q, cu_seqlens_k, num_seqs,
 * total_q, the head counts and head_dim, max_seqlen_q, max_seqlen_k and
 * split_keys -- the attention metadata an engine prepares once per step and
 * every layer of the step shares [Intro §11.4].  This call writes it into
 * `workspace` (sized by pa_prefill_workspace_size for the same values);
 * pa_prefill_varlen_planned and pa_store_prefill_varlen_planned then run a
 * layer's prefill on it without building it again, for as many calls (layers)
 * as the step has: each call leaves the list ready for the next (the last of
 * its workgroups resets the claim counter).  Calls that use one workspace must
 * be ordered (one stream); the arguments listed above must be the ones the
 * plan was built with, and a workspace holds one plan at a time (a
 * pa_prefill_varlen call on it replaces the plan with its own, for the same
 * metadata an identical one).  Errors as for pa_prefill_varlen.
 */
int pa_prefill_plan(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                    int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t split_keys,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* pa_prefill_varlen on the work list pa_prefill_plan built in `workspace`
 * (same arguments; the outputs are bit for bit those of pa_prefill_varlen). */
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
                              hipStream_t stream);

/* pa_store_prefill_varlen on the work list pa_prefill_plan built in
 * `workspace` (same arguments; outputs and caches bit for bit those of
 * pa_store_prefill_varlen). */
int pa_store_prefill_varlen_planned(
    const void* k_new, const void* v_new, int64_t k_tok_stride, int64_t k_head_stride,
    int64_t v_tok_stride, int64_t v_head_stride, const int32_t* slot_mapping, const void* q,
    int64_t q_tok_stride, int64_t q_head_stride, void* k_cache, void* v_cache,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* block_table,
    int64_t block_table_stride, int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    int32_t cache_layout, int32_t max_seqlen_q, int32_t max_seqlen_k, float scale,
    int32_t split_keys, void* workspace, size_t workspace_bytes, void* out,
    int64_t out_tok_stride, int64_t out_head_stride, int32_t dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
