// Batched single-token decode over the paged KV cache: split-K partition pass
// and the reduce that merges the splits.
//
// What is computed ("大模型推理入门与 nano-vLLM 源码详解" [Intro] §9.5, §11.4,
// §13.3; "Pico-vLLM 开发日志 #6" [Pico #6], its paged decode kernel): for
// sequence b and query head h, softmax(scale * q.k_j) weights over the
// context_lens[b] readable positions j, gathered through block_table[b], times
// v_j.  GQA: query heads g*G .. g*G+G-1 read kv head g [Intro §19.6].
//
// Design for gfx950:
// * One wave owns one (sequence, kv head, split).  The G query heads of the
//   GQA group are all held by that wave, so each K/V byte is read from HBM
//   exactly once and feeds every query head that needs it.
// * A head row (head_dim elements) is spread over kR lanes, 16 bytes each, so
//   one wave load covers 64 / kR tokens with fully used 16-byte lanes; the kR
//   partial dot products are combined with DPP row operations (no LDS).
// * A tile is kU such loads for K and for V.  The loads of the next tile are
//   issued before the current one is consumed (two register sets), so the
//   kU * 2 KiB of the next tile are in flight while a wave computes, and the
//   register budget still fits several waves per SIMD.  The loads are
//   non-temporal: each K/V row is read once per step.
// * The workgroup holds NW waves = NW consecutive kv heads of the same
//   (sequence, split) -- all 8 at Qwen3's shape: together they read each
//   token's whole [num_kv_heads, head_dim] row, and they share one staged
//   copy of the split's block-table entries in LDS.
// * Online softmax in fp32, base-2 (scores pre-multiplied by log2 e and exp2
//   on the hardware transcendental unit); the split statistics (m, l, acc)
//   go to the workspace, and the reduce merges them as [Intro §9.5] requires.
// * Optionally (kStore) the same launch does this step's KV store
//   [Intro §13.1]: sequence b's new token sits at position context_lens[b]-1,
//   in the sequence's last split; that split's waves write the token's K and
//   V rows to slot_mapping[b] and use them from registers in place of the row
//   they load from the cache, so the store needs no ordering against the
//   loads and costs no extra launch.

#include <math.h>

#include <mutex>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

template <typename T, int D, int G>
struct DecodeShape {
  static constexpr int kE = Chunk<T>::kElems;  // elements per lane per load
  static constexpr int kR = D / kE;            // lanes per head row
  static constexpr int kTpl = kWave / kR;      // tokens per wave load
  static constexpr int kU = G >= 4 ? 2 : 4;    // loads per tile, each for K and V
  static constexpr int kTile = kTpl * kU;      // tokens per tile
  static_assert(kR >= 1 && kR <= kWave && (kWave % kR) == 0, "row must fit a wave");
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A K/V row read once per step: a non-temporal load, so the stream of a long
// context neither evicts what other waves reuse nor is kept in L2 or MALL
// after its one use (512 contexts of 4096: 6.2 -> 6.9 TB/s; 64 contexts of
// 128..1024: 4.4 -> 4.9 TB/s).  Blocks that
// many sequences share are meant for pa_decode_shared_prefix's prefix pass,
// which reads them through the caches.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

template <typename T, int D, int G, int NW, bool kStore>
__global__ __launch_bounds__(NW* kWave) void decode_partition_kernel(
    const T* __restrict__ q, int64_t q_seq_stride, int64_t q_head_stride,
    const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int64_t bt_stride,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_kv_heads,
    int32_t bs_log2, int32_t max_ctx, int32_t partition_tokens, int32_t num_splits,
    float scale_log2, float* __restrict__ ws_acc, float* __restrict__ ws_ml, uint32_t block_stride,
    int32_t slot_stride, int64_t head_stride, const T* k_new, const T* v_new, int64_t k_tok_stride,
    int64_t k_head_stride, int64_t v_tok_stride, int64_t v_head_stride,
    const int32_t* slot_mapping, T* k_cache_w, T* v_cache_w,
    const int32_t* __restrict__ prefix_group, const int32_t* __restrict__ prefix_tokens,
    int32_t num_groups, int32_t max_prefix, const int32_t* __restrict__ work_list) {
  using S = DecodeShape<T, D, G>;
  constexpr int kE = S::kE, kR = S::kR, kTpl = S::kTpl, kU = S::kU, kTile = S::kTile;
  extern __shared__ int32_t bt_lds[];

  // Without a work list: workgroups are handed to the 8 XCDs round-robin in
  // launch order, and a sequence's later splits are empty when its context is
  // short.  Rotating the sequence index by the split spreads every split level
  // over all XCDs, so no XCD (with its own L2 and fabric share) ends up with
  // most of the full splits.  The order is split-major and ascending, so that
  // sequences holding the same blocks (a prefix-cache hit) read them at about
  // the same time and share the caches.
  // With a work list (prefix groups declared, whose prefix splits belong to
  // the shared-prefix pass): workgroup column i takes entry i, the list holds
  // only the splits this pass computes, full ones first and then the partial
  // ones longest first, and columns past its end return.  Each entry is
  // computed exactly as without the list.
  int split, b;
  if (work_list) {
    const int i = blockIdx.x + gridDim.x * blockIdx.z;
    if (i >= work_list[0]) return;  // uniform over the workgroup
    const int e = work_list[1 + i];
    b = e >> 16;
    split = e & 0xffff;
    if (b >= num_seqs || split >= num_splits) return;  // never for a list the library wrote
  } else {
    split = blockIdx.z;
    b = (blockIdx.x + num_seqs - split % num_seqs) % num_seqs;
  }
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = blockIdx.y * NW + wave;
  const int row = lane / kR;  // which token of a wave load
  const int col = lane % kR;  // which 16-byte chunk of the head row
  const int num_q_heads = num_kv_heads * G;
  const int t0 = split * partition_tokens;

  // The context length, the split's block-table window and the query are
  // independent loads, issued together: the window is the most a split can
  // touch, clipped to the bt_entries columns every table row has.
  // Every block-table row has the bt_entries columns a max_ctx-token context uses.
  const int bt_entries = (max_ctx + (1 << bs_log2) - 1) >> bs_log2;
  const int first_blk = t0 >> bs_log2;
  const int win = min((partition_tokens >> bs_log2) + 2, bt_entries - first_blk);
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * bt_stride + first_blk;
  for (int i = threadIdx.x; i < win; i += NW * kWave) bt_lds[i] = bt_row[i];
  uint4 q_raw[G];
#pragma unroll
  for (int i = 0; i < G; ++i)
    q_raw[i] = load16(q + static_cast<int64_t>(b) * q_seq_stride +
                      static_cast<int64_t>(g * G + i) * q_head_stride + col * kE);
  // The fused store's inputs are loaded with the rest, whether or not this is
  // the sequence's last split, so no dependent load sits before the tiles.
  int32_t slot = -1;
  uint4 k_new_raw = make_uint4(0, 0, 0, 0), v_new_raw = make_uint4(0, 0, 0, 0);
  if constexpr (kStore) {
    slot = slot_mapping[b];
    k_new_raw = load16(k_new + b * k_tok_stride + g * k_head_stride + col * kE);
    v_new_raw = load16(v_new + b * v_tok_stride + g * v_head_stride + col * kE);
  }
  // A member of a shared-prefix group leaves the splits inside its prefix (all
  // but the one holding its last position) to the shared-prefix pass.
  const int grp = prefix_group ? prefix_group[b] : -1;  // outside [0, num_groups): none
  // A context longer than max_ctx (a caller error) is cut to it, so no split reads
  // past the staged window.
  const int ctx = min(context_lens[b], max_ctx);
  if (t0 >= ctx) return;  // empty split (uniform over the workgroup): nothing written
  if (static_cast<unsigned>(grp) < static_cast<unsigned>(num_groups) &&
      split < min(min(prefix_tokens[grp], max_prefix) / partition_tokens,
                              (ctx - 1) / partition_tokens))
    return;  // written by the shared-prefix pass (uniform)
  const int t1 = min(t0 + partition_tokens, ctx);
  const int bs_mask = (1 << bs_log2) - 1;

  // The fused store: only position ctx - 1 of the last split is affected, and
  // only this split's waves read it; its rows are used from registers where
  // the tile loads would supply them (whatever those loads return is
  // discarded), and written to the cache at the end.
  const int new_pos = kStore && t1 == ctx && slot >= 0 ? ctx - 1 : -1;
  __syncthreads();  // bt_lds ready

  float qf[G][kE];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    Chunk<T>::widen(q_raw[i], qf[i]);
#pragma unroll
    for (int e = 0; e < kE; ++e) qf[i][e] *= scale_log2;
  }

  float m[G], l[G], acc[G][kE];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[i][e] = 0.f;
  }

  const T* kbase = k_cache + g * head_stride + col * kE;
  const T* vbase = v_cache + g * head_stride + col * kE;

  // Loads of tile n+1 are issued before tile n is consumed, so a wave never
  // waits on HBM with nothing else queued.  Rows past t1 read row t1 - 1
  // (cached, finite) and are masked in the scores; the prefetch is never
  // skipped, which keeps the compiler's wait counts exact (a conditional load
  // would make it wait for every outstanding load).
  auto load_tile = [&](int tb, uint4 (&kr)[kU], uint4 (&vr)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = min(tb + u * kTpl + row, t1 - 1);
      // one 32 x 32 -> 64-bit multiply: block ids and the block stride fit 32 bits
      const uint32_t blk = bt_lds[(j >> bs_log2) - first_blk];
      const uint64_t off = static_cast<uint64_t>(blk) * block_stride +
                           static_cast<uint32_t>(j & bs_mask) * static_cast<uint32_t>(slot_stride);
      kr[u] = load16_stream(kbase + off);
      vr[u] = load16_stream(vbase + off);
    }
    // keep the scheduler from sinking these loads into the consume that follows
    __builtin_amdgcn_sched_barrier(0);
  };

  auto consume = [&](int tb, const uint4 (&kr)[kU], const uint4 (&vr)[kU]) {
    float sc[kU][G];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float kf[kE];
      // The fused store's row is taken from registers (a select at use, so the
      // loads of the next tile stay in flight).
      const bool is_new = kStore && min(tb + u * kTpl + row, t1 - 1) == new_pos;
      Chunk<T>::widen(is_new ? k_new_raw : kr[u], kf);
      const bool valid = tb + u * kTpl + row < t1;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < kE; ++e) d = fmaf(qf[i][e], kf[e], d);
        d = group_sum<kR>(d);
        sc[u][i] = valid ? d : -INFINITY;
      }
    }

#pragma unroll
    for (int i = 0; i < G; ++i) {
      float mt = sc[0][i];
#pragma unroll
      for (int u = 1; u < kU; ++u) mt = fmaxf(mt, sc[u][i]);
      mt = across_groups_max<kR>(mt);
      // m_new is finite: the first tile consumed starts at t0 < t1.
      const float m_new = fmaxf(m[i], mt);
      const float alpha = fast_exp2(m[i] - m_new);
      m[i] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        sc[u][i] = fast_exp2(sc[u][i] - m_new);
        psum += sc[u][i];
      }
      l[i] = l[i] * alpha + psum;
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[i][e] *= alpha;
    }

#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float vf[kE];
      const bool is_new = kStore && min(tb + u * kTpl + row, t1 - 1) == new_pos;
      Chunk<T>::widen(is_new ? v_new_raw : vr[u], vf);
#pragma unroll
      for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[i][e] = fmaf(sc[u][i], vf[e], acc[i][e]);
    }
  };

  // Two register sets alternate; the loop is unrolled by two by hand so no
  // set is ever copied.  The body has no exit between a load and the consume
  // that precedes its use (an early exit there lets the compiler sink the load
  // to the next iteration, which removes the overlap).  When the split has an
  // odd number of tiles the last consume sees a tile wholly past t1: every
  // score is -inf, so it adds nothing (m is finite by then).
  uint4 ka[kU], va[kU], kb[kU], vb[kU];
  load_tile(t0, ka, va);
  int tb = t0;
  do {
    load_tile(tb + kTile, kb, vb);
    consume(tb, ka, va);
    load_tile(tb + 2 * kTile, ka, va);
    consume(tb + kTile, kb, vb);
    tb += 2 * kTile;
  } while (tb < t1);

  // Combine the wave's token rows (all share the running maximum m).
#pragma unroll
  for (int i = 0; i < G; ++i) {
    l[i] = across_groups_sum<kR>(l[i]);
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[i][e] = across_groups_sum<kR>(acc[i][e]);
  }
  if (row == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int64_t idx = (static_cast<int64_t>(b) * num_q_heads + g * G + i) * num_splits + split;
      float4* dst = reinterpret_cast<float4*>(ws_acc + idx * D + col * kE);
#pragma unroll
      for (int e = 0; e < kE; e += 4)
        dst[e / 4] = make_float4(acc[i][e], acc[i][e + 1], acc[i][e + 2], acc[i][e + 3]);
      if (col == 0) reinterpret_cast<float2*>(ws_ml)[idx] = make_float2(m[i], l[i]);
    }
  }
  if constexpr (kStore) {
    if (new_pos >= 0 && row == 0) {
      const uint64_t off =
          static_cast<uint64_t>(static_cast<uint32_t>(slot >> bs_log2)) * block_stride +
          static_cast<uint32_t>(slot & bs_mask) * static_cast<uint32_t>(slot_stride) +
          g * head_stride + col * kE;
      *reinterpret_cast<uint4*>(k_cache_w + off) = k_new_raw;
      *reinterpret_cast<uint4*>(v_cache_w + off) = v_new_raw;
    }
  }
}

// One wave per (sequence, query head); each lane owns D / 64 output elements.
template <typename T, int D>
__global__ __launch_bounds__(4 * kWave) void decode_reduce_kernel(
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ context_lens, int32_t num_q_heads, int32_t num_splits,
    int32_t partition_tokens, T* __restrict__ out, int64_t out_seq_stride,
    int64_t out_head_stride) {
  constexpr int kDpl = D / kWave;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int h = blockIdx.x * 4 + wave;
  const int b = blockIdx.y;
  if (h >= num_q_heads) return;
  const int64_t base = (static_cast<int64_t>(b) * num_q_heads + h) * num_splits;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + base;
  const float* acc = ws_acc + base * D + lane * kDpl;

  // The first kPre splits' statistics and partial outputs are loaded together
  // with the context length instead of after it: the workspace holds
  // num_splits slots per row, so these loads stay in bounds, and slots past
  // the row's active splits are loaded but never used.
  constexpr int kPre = 4;
  float2 st[kPre];
  float part[kPre][kDpl];
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < num_splits) {
      st[s] = ml[s];
#pragma unroll
      for (int k = 0; k < kDpl; ++k) part[s][k] = acc[static_cast<int64_t>(s) * D + k];
    }
  const int ctx = context_lens[b];
  const int ns = min(num_splits, (ctx + partition_tokens - 1) / partition_tokens);

  // The next kMid splits are loaded in one batch with the maximum's loads (they
  // do not depend on it), so a row of up to kPre + kMid splits costs two round
  // trips to memory; further splits go kMid at a time.  Splits are combined in
  // ascending order whatever the batching.
  constexpr int kMid = 12;
  float2 st2[kMid];
  float part2[kMid][kDpl];
#pragma unroll
  for (int j = 0; j < kMid; ++j)
    if (kPre + j < ns) {
      st2[j] = ml[kPre + j];
#pragma unroll
      for (int k = 0; k < kDpl; ++k) part2[j][k] = acc[static_cast<int64_t>(kPre + j) * D + k];
    }
  float m_star = -INFINITY;
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < ns) m_star = fmaxf(m_star, st[s].x);
  for (int s = kPre + lane; s < ns; s += kWave) m_star = fmaxf(m_star, ml[s].x);
  m_star = across_groups_max<1>(m_star);

  float o[kDpl], lsum = 0.f;
#pragma unroll
  for (int k = 0; k < kDpl; ++k) o[k] = 0.f;
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < ns) {
      const float w = fast_exp2(st[s].x - m_star);
      lsum = fmaf(w, st[s].y, lsum);
#pragma unroll
      for (int k = 0; k < kDpl; ++k) o[k] = fmaf(w, part[s][k], o[k]);
    }
#pragma unroll
  for (int j = 0; j < kMid; ++j)
    if (kPre + j < ns) {
      const float w = fast_exp2(st2[j].x - m_star);
      lsum = fmaf(w, st2[j].y, lsum);
#pragma unroll
      for (int k = 0; k < kDpl; ++k) o[k] = fmaf(w, part2[j][k], o[k]);
    }
  for (int s0 = kPre + kMid; s0 < ns; s0 += kMid) {
#pragma unroll
    for (int j = 0; j < kMid; ++j)
      if (s0 + j < ns) {
        st2[j] = ml[s0 + j];
#pragma unroll
        for (int k = 0; k < kDpl; ++k) part2[j][k] = acc[static_cast<int64_t>(s0 + j) * D + k];
      }
#pragma unroll
    for (int j = 0; j < kMid; ++j)
      if (s0 + j < ns) {
        const float w = fast_exp2(st2[j].x - m_star);
        lsum = fmaf(w, st2[j].y, lsum);
#pragma unroll
        for (int k = 0; k < kDpl; ++k) o[k] = fmaf(w, part2[j][k], o[k]);
      }
  }
  const float inv = ns > 0 ? 1.f / lsum : 0.f;
  T* dst = out + static_cast<int64_t>(b) * out_seq_stride + static_cast<int64_t>(h) * out_head_stride +
           lane * kDpl;
#pragma unroll
  for (int k = 0; k < kDpl; ++k) {
    const float val = ns > 0 ? o[k] * inv : 0.f;
    if constexpr (sizeof(T) == 2)
      reinterpret_cast<uint16_t*>(dst)[k] = f32_to_bf16_rne(val);
    else
      reinterpret_cast<float*>(dst)[k] = val;
  }
}

template <typename T, int D, int G, int NW, bool kStore>
hipError_t run_partition(const DecodeArgs& a, hipStream_t stream) {
  const int bs_log2 = __builtin_ctz(static_cast<unsigned>(a.block_size));
  const int max_blk = (a.partition_tokens >> bs_log2) + 2;
  dim3 grid(a.num_seqs, a.num_kv_heads / NW, a.num_splits);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, G, NW, kStore>), grid, dim3(NW * kWave),
                     max_blk * sizeof(int32_t), stream, static_cast<const T*>(a.q),
                     a.q_seq_stride, a.q_head_stride, static_cast<const T*>(a.k_cache),
                     static_cast<const T*>(a.v_cache), a.block_table, a.block_table_stride,
                     a.context_lens, a.num_seqs, a.num_kv_heads, bs_log2, a.max_context_len,
                     a.partition_tokens, a.num_splits, a.scale * kLog2e, a.ws_acc, a.ws_ml,
                     static_cast<uint32_t>(a.geom.block), static_cast<int32_t>(a.geom.slot),
                     a.geom.head, static_cast<const T*>(a.k_new), static_cast<const T*>(a.v_new),
                     a.k_tok_stride, a.k_head_stride, a.v_tok_stride, a.v_head_stride,
                     a.slot_mapping, static_cast<T*>(const_cast<void*>(a.k_cache)),
                     static_cast<T*>(const_cast<void*>(a.v_cache)), a.prefix_group,
                     a.prefix_tokens, a.num_prefix_groups, a.max_prefix_tokens, a.work_list);
  return hipGetLastError();
}

template <typename T, int D, int G, bool kStore>
hipError_t pick_nw(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_kv_heads % 8 == 0) return run_partition<T, D, G, 8, kStore>(a, stream);
  if (a.num_kv_heads % 4 == 0) return run_partition<T, D, G, 4, kStore>(a, stream);
  if (a.num_kv_heads % 2 == 0) return run_partition<T, D, G, 2, kStore>(a, stream);
  return run_partition<T, D, G, 1, kStore>(a, stream);
}

// Waves of kernel K resident at once on the current GPU (0 if the query
// fails).  The split window's LDS is a few hundred bytes, far below what
// limits residency, so the answer depends only on the kernel and the device
// and is kept per device.
template <auto kKernel>
int64_t resident_waves(int threads, size_t lds) {
  constexpr int kMaxDevices = 64;
  static int64_t known[kMaxDevices] = {};  // 0: not asked yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices && known[dev] > 0) return known[dev];
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kKernel, threads, lds) != hipSuccess)
    return 0;
  const int64_t waves = int64_t{occ} * cus * (threads / kWave);
  if (dev >= 0 && dev < kMaxDevices) known[dev] = waves;
  return waves;
}

// The fused store costs the partition kernel registers (fewer waves resident:
// at Qwen3's shape one 8-wave workgroup per CU instead of two).  When the grid
// does not fit the GPU at once with them (a long-context batch such as 512
// sequences x 8 kv heads, or a grid of many splits that runs in several
// rounds, where the waves resident set the bytes in flight), the store goes
// first as its own launch and the plain kernel follows; both ways write the
// same bits.
template <typename T, int D, int G, int NW>
hipError_t run_with_store(const DecodeArgs& a, hipStream_t stream) {
  const int64_t waves = int64_t{a.num_seqs} * a.num_kv_heads * a.num_splits;
  const size_t lds = ((a.partition_tokens / a.block_size) + 2) * sizeof(int32_t);
  const int64_t fused = resident_waves<decode_partition_kernel<T, D, G, NW, true>>(NW * kWave, lds);
  const int64_t plain = resident_waves<decode_partition_kernel<T, D, G, NW, false>>(NW * kWave, lds);
  if (waves <= fused || plain <= fused) return run_partition<T, D, G, NW, true>(a, stream);
  const StoreArgs sa{a.k_new, a.v_new, a.k_tok_stride, a.k_head_stride, a.v_tok_stride,
                     a.v_head_stride, const_cast<void*>(a.k_cache),
                     const_cast<void*>(a.v_cache), a.slot_mapping, a.num_seqs, a.num_kv_heads,
                     a.head_dim, a.block_size, static_cast<int32_t>(sizeof(T)), a.geom};
  const hipError_t err = launch_store(sa, stream);
  if (err != hipSuccess) return err;
  return run_partition<T, D, G, NW, false>(a, stream);
}

template <typename T, int D, int G>
hipError_t pick_store(const DecodeArgs& a, hipStream_t stream) {
  if (!a.k_new) return pick_nw<T, D, G, false>(a, stream);
  if (a.num_kv_heads % 8 == 0) return run_with_store<T, D, G, 8>(a, stream);
  if (a.num_kv_heads % 4 == 0) return run_with_store<T, D, G, 4>(a, stream);
  if (a.num_kv_heads % 2 == 0) return run_with_store<T, D, G, 2>(a, stream);
  return run_with_store<T, D, G, 1>(a, stream);
}

template <typename T, int D>
hipError_t pick_group(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return pick_store<T, D, 1>(a, stream);
    case 2: return pick_store<T, D, 2>(a, stream);
    case 4: return pick_store<T, D, 4>(a, stream);
    case 8: return pick_store<T, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t run_reduce(const ReduceArgs& a, hipStream_t stream) {
  dim3 grid((a.num_q_heads + 3) / 4, a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), grid, dim3(4 * kWave), 0, stream, a.ws_acc,
                     a.ws_ml, a.context_lens, a.num_q_heads, a.num_splits, a.partition_tokens,
                     static_cast<T*>(a.out), a.out_seq_stride, a.out_head_stride);
  return hipGetLastError();
}

}  // namespace

// The workspace of pa_store_decode_noalloc: a file-scope device array, one copy
// per GPU.  In host code its name is only a stand-in for the symbol; the device
// address is asked of the runtime (once per device, with that device current)
// and only that address is ever passed to a kernel.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* known[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!known[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    known[dev] = static_cast<float*>(p);
  }
  *ptr = known[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.bf16) return a.head_dim == 128 ? pick_group<bf16_t, 128>(a, stream)
                                       : pick_group<bf16_t, 64>(a, stream);
  return a.head_dim == 128 ? pick_group<float, 128>(a, stream) : pick_group<float, 64>(a, stream);
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream) {
  if (a.bf16) return a.head_dim == 128 ? run_reduce<bf16_t, 128>(a, stream)
                                       : run_reduce<bf16_t, 64>(a, stream);
  return a.head_dim == 128 ? run_reduce<float, 128>(a, stream) : run_reduce<float, 64>(a, stream);
}

}  // namespace pa
