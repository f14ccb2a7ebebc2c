// Variable-length causal prefill over the paged KV cache, bf16 MFMA.
//
// What is computed ("大模型推理入门与 nano-vLLM 源码详解" [Intro] §10.2, §11.2,
// §13.2, §13.3): sequence b owns query rows cu_q[b]..cu_q[b+1]-1 and reads
// Lk = cu_k[b+1]-cu_k[b] keys through its block table; with c = Lk - Lq
// cached positions, query row i (position c + i) attends to keys 0..c+i.
// Each (query, head) output is softmax(scale * q.K^T) V, computed tile by tile
// with a running maximum, exponential sum and un-normalised output that are
// rescaled whenever the maximum grows [Intro §13.3].
//
// Design for gfx950 (wave64, v_mfma_f32_32x32x16_bf16):
// * A workgroup owns one kv head g of one sequence and a tile of query
//   positions; its waves are the G query heads of the GQA group times kRB
//   blocks of 32 rows, so each K/V tile staged in LDS feeds every query head
//   that reads kv head g.
// * Scores are computed transposed, S^T = K Q^T (A operand = K from LDS, B
//   operand = Q^T held in registers for the whole key loop).  In the MFMA
//   accumulator layout each lane then owns ONE query and 16 keys per 32-key
//   block, so the softmax max and sum are in-lane plus one exchange with the
//   partner lane (lane ^ 32).
// * O^T = V^T P^T: the probabilities feed the second MFMA straight from the
//   score registers.  V stays row-major ([key][dim]) in LDS and each V^T
//   operand is read with two ds_read_b64_tr_b16 (gfx950's transposing LDS
//   read), whose per-16-lane transpose hands every lane 4 keys of one dim;
//   the keys are chosen to match the order in which the score accumulator
//   holds P, so no data is permuted anywhere.
// * P enters the P.V MFMA as bf16.  Rows that see at least 256 keys round p
//   to nearest; a wave whose rows see fewer also sends p's remainder (p minus
//   its truncated bf16 head) through the MFMA, so P carries ~16 significant
//   bits: with few keys the weight sits on a few values, and bf16 P alone can
//   miss the 2e-3 absolute bound where they cancel.  The remainder costs half
//   again the P.V work, so only those waves pay it.
// * K/V tiles go from HBM straight into LDS by DMA (global_load_lds, 16 bytes
//   a lane), double-buffered: the next tile streams in while the MFMAs read the
//   current one, with no registers or VALU spent on staging and one barrier
//   per tile.  Rows are XOR-swizzled by 16-byte chunk, with a pattern per
//   tile (K or V) chosen so the operand reads are free of bank conflicts.
// * The sequence's block-table entries are staged in LDS once, so a K/V
//   address never waits on a global load.
// * The output is rescaled only when a tile's maximum score exceeds the
//   reference maximum by more than 8 in base-2 units (lazy rescaling);
//   otherwise the probabilities are taken against the old reference and stay
//   below 2^8.
// * Work items (sequence, query tile, key range, kv head) come from a list
//   built on the device by one workgroup, heaviest first; a fixed set of
//   workgroups, one per resident slot, takes them from a counter.
// * With the step's store (kNew), keys at this step's positions are read from
//   the new K/V rows instead of the cache, and each item writes the rows of
//   its own query positions to the cache from the tiles it holds in LDS.

#include <math.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBN = 64;  // keys per tile
// The work-list counters open the workspace: tickets[0] the claim counter,
// tickets[1] the number of entries, tickets[2] the number of split tiles, and
// in a 256-byte chunk of its own tickets[kTicketExit], the count of
// workgroups that have left.  Every workgroup's last claim and its exit meet
// at the end of the kernel, and atomics on different words of one line
// serialise behind each other.
constexpr int kTicketExit = 64;
static_assert((kTicketExit + 1) * 4 <= kPrefillTicketBytes, "exit counter fits the ticket area");
// Rows whose first position sees fewer keys than this carry the remainder of
// p through P.V (see short_rows).
constexpr int kRestKeys = 256;
// Word 3 of a raw buffer resource: 32-bit data format, no swizzle or stride.
constexpr int kBufferFlags = 0x00020000;
// v_perm_b32 selector: perm(a, b, sel) picks bytes of {a:b} (b = bytes 0-3);
// this one keeps the high halves: b.hi | a.hi << 16.
constexpr uint32_t kPermHigh = 0x07060302u;

template <int D, int G>
struct PrefillShape {
  static constexpr int kRB = G >= 4 ? 1 : 4 / G;     // 32-row blocks per query head
  static constexpr int kWaves = G * kRB;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kBM = 32 * kRB;               // query positions per workgroup
  static constexpr int kSteps = D / 16;              // MFMA k-steps over head_dim
  static constexpr int kDB = D / 32;                 // 32-wide output blocks over head_dim
  static constexpr int kChunks = D / 8;              // 16-byte chunks per K/V row
  static constexpr int kRowsPerDma = 1024 / (2 * D); // rows one wave-wide 1 KB DMA fills
  static constexpr int kDmaPerTile = kBN / kRowsPerDma;
  static constexpr int kDmaPerWave = kDmaPerTile / kWaves;
  static_assert(kDmaPerTile % kWaves == 0, "DMA pieces must split evenly over the waves");
};

template <int B>
struct Buf {};

// Compile-time loop: f(std::integral_constant<int, I>) for I = kBegin .. kEnd - 1.
template <int kBegin, int kEnd, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (kBegin < kEnd) {
    f(std::integral_constant<int, kBegin>{});
    static_for<kBegin + 1, kEnd>(f);
  }
}
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// LDS position of 16-byte chunk c of a K or V row is c ^ swizzle(row).  The
// swizzles are chosen per access pattern so that every 32 lanes the LDS serves
// together hit distinct banks (64 banks of 4 bytes):
// * K is read as 16-byte A operands, one row per lane, 32 consecutive rows:
//   128-element rows use row mod 16; 64-element rows (two per bank line) use
//   (row / 2) mod 8.
// * V is read with ds_read_b64_tr_b16: a 16-lane group reads 4 consecutive
//   keys x 2 chunks x 2 halves, and the two groups of a half-wave differ in
//   chunk bit 1; spreading the 4 keys over chunk bits 2-3 (D=128) or over
//   chunk bit 2 and the bank-line half (D=64) separates all 32 lanes.
template <int D>
__device__ __forceinline__ int k_swizzle(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swizzle(int key) {
  return D == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// This step's K/V rows when the prefill also stores them (kNew): tiles of
// these positions are read from here rather than from the cache, and each
// work item writes the rows of its own query positions into the cache.
struct NewKV {
  const char* k;                // row (token t, kv head g) at k + t * k_tok_b + g * k_head_b
  const char* v;
  int32_t k_tok_b, v_tok_b;     // bytes; 64 rows fit 32-bit offsets (checked on the host)
  int64_t k_head_b, v_head_b;   // bytes
  const int32_t* slot_mapping;  // token -> cache slot, -1: not stored
  uint16_t* k_cache;            // the caches, written
  uint16_t* v_cache;
};

// A decode row of a mixed batch (a sequence with one query position): taken
// decode-style instead of as a 64-row MFMA tile with one live row.  The
// workgroup's waves split the G query heads into groups of at most two and the
// keys into consecutive ranges; a wave holds its heads' queries and reads every
// key of its range once, 16 bytes a lane (a head row over kR lanes, 64 / kR
// keys per load, the loads of the next tile issued before the current one is
// consumed), with an fp32 online softmax in base 2.  The ranges' (m, l, acc)
// meet in LDS and the normalised row is written.  With kNew the last key is
// this step's row, read from the new K/V and written to its slot here.
// `scratch` (at least kRanges * G * D floats) and `ml_scratch` (kRanges * G * 2
// floats) are LDS the item does not otherwise use; every thread of the
// workgroup calls this.
template <int D, int G, int kWaves, bool kNew>
__device__ __forceinline__ void decode_row(
    const uint16_t* __restrict__ q, int64_t q_tok_stride, int64_t q_head_stride,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* bt_lds, int bs_log2, int64_t block_stride, int64_t slot_stride,
    int64_t head_stride, int g, int q_row, int lk, float scale_log2, uint16_t* __restrict__ out,
    int64_t out_tok_stride, int64_t out_head_stride, const NewKV& nk, float* scratch,
    float* ml_scratch) {
  constexpr int kE = 8, kR = D / kE, kTpl = kWave / kR, kU = 2, kTile = kTpl * kU;
  constexpr int kGW = G < 2 ? G : 2;          // query heads per wave
  constexpr int kHG = G / kGW;                // head groups
  constexpr int kRanges = kWaves / kHG;       // key ranges
  static_assert(kRanges >= 1 && kRanges * kHG == kWaves, "waves must cover heads x ranges");
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int row = lane / kR;
  const int col = lane % kR;
  const int hg = wave % kHG;
  const int range = wave / kHG;
  const int n_tiles = (lk + kTile - 1) / kTile;
  const int t0 = (range * n_tiles / kRanges) * kTile;
  const int t1 = min(((range + 1) * n_tiles / kRanges) * kTile, lk);
  const int bs_mask = (1 << bs_log2) - 1;
  const int head0 = g * G + hg * kGW;

  float qf[kGW][kE];
#pragma unroll
  for (int i = 0; i < kGW; ++i) {
    const uint4 raw = load16(q + static_cast<int64_t>(q_row) * q_tok_stride +
                             static_cast<int64_t>(head0 + i) * q_head_stride + col * kE);
    Chunk<bf16_t>::widen(raw, qf[i]);
#pragma unroll
    for (int e = 0; e < kE; ++e) qf[i][e] *= scale_log2;
  }
  // this step's row (kNew): position lk - 1, read from the new K/V
  uint4 k_new_raw = make_uint4(0, 0, 0, 0), v_new_raw = make_uint4(0, 0, 0, 0);
  if constexpr (kNew) {
    k_new_raw = load16(nk.k + static_cast<int64_t>(q_row) * nk.k_tok_b + g * nk.k_head_b +
                       col * kE * 2);
    v_new_raw = load16(nk.v + static_cast<int64_t>(q_row) * nk.v_tok_b + g * nk.v_head_b +
                       col * kE * 2);
  }
  const int new_pos = kNew ? lk - 1 : -1;

  float m[kGW], l[kGW], acc[kGW][kE];
#pragma unroll
  for (int i = 0; i < kGW; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[i][e] = 0.f;
  }
  const uint16_t* kbase = k_cache + g * head_stride + col * kE;
  const uint16_t* vbase = v_cache + g * head_stride + col * kE;
  // Keys past t1 read key t1 - 1 (a readable row) and are masked.
  auto load_tile = [&](int tb, uint4 (&kr)[kU], uint4 (&vr)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = min(tb + u * kTpl + row, t1 - 1);
      const int64_t off = static_cast<int64_t>(bt_lds[j >> bs_log2]) * block_stride +
                          (j & bs_mask) * slot_stride;
      kr[u] = load16(kbase + off);
      vr[u] = load16(vbase + off);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto consume = [&](int tb, const uint4 (&kr)[kU], const uint4 (&vr)[kU]) {
    float sc[kU][kGW];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = tb + u * kTpl + row;
      float kf[kE];
      Chunk<bf16_t>::widen(kNew && min(j, t1 - 1) == new_pos ? k_new_raw : kr[u], kf);
#pragma unroll
      for (int i = 0; i < kGW; ++i) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < kE; ++e) d = fmaf(qf[i][e], kf[e], d);
        d = group_sum<kR>(d);
        sc[u][i] = j < t1 ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int i = 0; i < kGW; ++i) {
      float mt = sc[0][i];
#pragma unroll
      for (int u = 1; u < kU; ++u) mt = fmaxf(mt, sc[u][i]);
      mt = across_groups_max<kR>(mt);
      const float m_new = fmaxf(m[i], mt);  // finite: the first tile starts below t1
      const float alpha = __builtin_amdgcn_exp2f(m[i] - m_new);
      m[i] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        sc[u][i] = __builtin_amdgcn_exp2f(sc[u][i] - m_new);
        psum += sc[u][i];
      }
      l[i] = l[i] * alpha + psum;
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[i][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = tb + u * kTpl + row;
      float vf[kE];
      Chunk<bf16_t>::widen(kNew && min(j, t1 - 1) == new_pos ? v_new_raw : vr[u], vf);
#pragma unroll
      for (int i = 0; i < kGW; ++i)
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[i][e] = fmaf(sc[u][i], vf[e], acc[i][e]);
    }
  };
  if (t0 < t1) {  // uniform over the wave
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
#pragma unroll
    for (int i = 0; i < kGW; ++i) {
      l[i] = across_groups_sum<kR>(l[i]);
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[i][e] = across_groups_sum<kR>(acc[i][e]);
    }
  }
  // Partials of (range, head): acc at scratch[(range * G + head) * D], (m, l) at
  // ml_scratch[(range * G + head) * 2]; an empty range leaves m = -inf, l = 0.
  if (row == 0) {
#pragma unroll
    for (int i = 0; i < kGW; ++i) {
      float* dst = scratch + (range * G + hg * kGW + i) * D + col * kE;
#pragma unroll
      for (int e = 0; e < kE; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(acc[i][e], acc[i][e + 1], acc[i][e + 2], acc[i][e + 3]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < kGW; ++i) {
      ml_scratch[(range * G + hg * kGW + i) * 2] = m[i];
      ml_scratch[(range * G + hg * kGW + i) * 2 + 1] = l[i];
    }
  }
  if constexpr (kNew) {  // this step's row into its slot
    const int slot = nk.slot_mapping[q_row];
    if (wave == 0 && row == 0 && slot >= 0) {
      const int64_t off = static_cast<int64_t>(slot >> bs_log2) * block_stride +
                          (slot & bs_mask) * slot_stride + g * head_stride + col * kE;
      *reinterpret_cast<uint4*>(nk.k_cache + off) = k_new_raw;
      *reinterpret_cast<uint4*>(nk.v_cache + off) = v_new_raw;
    }
  }
  __syncthreads();
  for (int t = tid; t < G * D; t += kWaves * kWave) {
    const int i = t / D, d = t % D;
    float m_star = -INFINITY;
#pragma unroll
    for (int r = 0; r < kRanges; ++r) m_star = fmaxf(m_star, ml_scratch[(r * G + i) * 2]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int r = 0; r < kRanges; ++r) {
      const float mr = ml_scratch[(r * G + i) * 2];
      const float c = mr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mr - m_star);
      lsum = fmaf(c, ml_scratch[(r * G + i) * 2 + 1], lsum);
      o = fmaf(c, scratch[(r * G + i) * D + d], o);
    }
    out[static_cast<int64_t>(q_row) * out_tok_stride +
        static_cast<int64_t>(g * G + i) * out_head_stride + d] = f32_to_bf16_rne(o / lsum);
  }
}

template <int D, int G, bool kNew>
__global__ __launch_bounds__((PrefillShape<D, G>::kThreads), 2) void prefill_kernel(
    const uint16_t* __restrict__ q, int64_t q_tok_stride, int64_t q_head_stride,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    const int32_t* __restrict__ block_table, int64_t bt_stride, int32_t num_kv_heads,
    int32_t bs_log2, int32_t max_seqlen_k, float scale_log2, int32_t split_tiles,
    uint32_t* __restrict__ tickets,
    const int2* __restrict__ items, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    int32_t total_q, uint16_t* __restrict__ out, int64_t out_tok_stride,
    int64_t out_head_stride, int64_t block_stride, int64_t slot_stride, int64_t head_stride,
    NewKV nk) {
  using S = PrefillShape<D, G>;
  // Two K/V tile buffers, row-major [key][dim], each row's 16-byte chunks
  // XOR-swizzled (k_swizzle / v_swizzle) so the MFMA operand reads are free
  // of bank conflicts.
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[kBN * D];
  extern __shared__ int32_t bt_lds[];  // this sequence's block-table entries

  __shared__ int ticket_lds;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int half = lane / 32;
  const int col = lane % 32;

  // DMA piece i of this wave fills tile rows piece * kRowsPerDma .. + kRowsPerDma - 1
  // (piece = wave * kDmaPerWave + i); lane l brings the 16-byte source chunk
  // that the swizzle puts at LDS position l % kChunks of row l / kChunks.
  auto dma_row = [&](int i) { return (wave * S::kDmaPerWave + i) * S::kRowsPerDma + lane / S::kChunks; };
  // K operand (A of S^T = K Q^T): row mb*32 + col, chunk 2s + half.
  int k_off[S::kSteps];
#pragma unroll
  for (int s = 0; s < S::kSteps; ++s)
    k_off[s] = col * D + 8 * ((2 * s + half) ^ k_swizzle<D>(col));  // rows col and col + 32
  // V operand (A of O^T = V^T P^T) via transpose reads: for read t of step ks,
  // lane (half, col) supplies the row of key ks*16 + 8t + 4 half + (col % 16) / 4
  // and dims db*32 + 16 (col / 16) + 4 (col % 4) .. +3; the read hands it the
  // keys ks*16 + 8t + 4 half + e (e = 0..3) of dim db*32 + col.
  // The swizzle of key + 8 equals that of key, so read t = 1 sits 8 rows after
  // read t = 0.
  int v_off[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) {
    const int key = 4 * half + (col % 16) / 4;
    const int j4 = col % 4;
    const int chunk = db * 4 + 2 * (col / 16) + j4 / 2;
    v_off[db] = key * D + 8 * (chunk ^ v_swizzle<D>(key)) + 4 * (j4 % 2);
  }
  const int bs_mask = (1 << bs_log2) - 1;
  // When a block holds at least a tile (64 tokens), the 64 rows of a tile are
  // consecutive slots of one block, so a DMA source is one wave-uniform base
  // plus a per-lane byte offset that is the same for every tile.
  const bool tile_in_block = bs_log2 >= 6;
  // Byte offset of a lane's source within the tile: a uniform part for the
  // piece, (piece * kRowsPerDma) rows, plus a per-lane part.  The V swizzle
  // depends only on row bits below kRowsPerDma, so its lane part is the same
  // for every piece.
  static_assert(S::kRowsPerDma % 4 == 0, "V swizzle must not depend on the piece");
  const int row_bytes = static_cast<int>(slot_stride) * 2;
  uint32_t dma_klane[S::kDmaPerWave];
#pragma unroll
  for (int i = 0; i < S::kDmaPerWave; ++i)
    dma_klane[i] = (lane / S::kChunks) * row_bytes +
                   16 * ((lane % S::kChunks) ^ k_swizzle<D>(dma_row(i)));
  const uint32_t dma_vlane = (lane / S::kChunks) * row_bytes +
                             16 * ((lane % S::kChunks) ^ v_swizzle<D>(lane / S::kChunks));
  // The same per-lane chunks at the row strides of this step's K and V rows.
  uint32_t new_klane[S::kDmaPerWave], new_vlane = 0;
  if constexpr (kNew) {
#pragma unroll
    for (int i = 0; i < S::kDmaPerWave; ++i)
      new_klane[i] = (lane / S::kChunks) * nk.k_tok_b +
                     16 * ((lane % S::kChunks) ^ k_swizzle<D>(dma_row(i)));
    new_vlane = (lane / S::kChunks) * nk.v_tok_b +
                16 * ((lane % S::kChunks) ^ v_swizzle<D>(lane / S::kChunks));
  }

  // Work entries come from the plan heaviest first, the kv heads of one query
  // tile side by side (they read the same K/V rows, so those DRAM pages are
  // open together).  A workgroup's first entry is its own index; after that
  // it takes the next one from a counter as soon as it is free, claimed while
  // it works on its last key tile so the claim's latency is hidden.  The long
  // key loops start first and the short ones fill the gaps around them.
  const int n_entries = static_cast<int>(tickets[1]);
  int next_entry = blockIdx.x;  // meaningful in thread 0 only
  for (;;) {
  if (tid == 0) ticket_lds = next_entry;
  __syncthreads();
  // The entry is the same for the whole workgroup: everything derived from it
  // lives in scalar registers.
  const int entry = __builtin_amdgcn_readfirstlane(ticket_lds);
  if (entry >= n_entries) break;  // uniform: every wave leaves together
  const int2 item = items[entry];
  const int b = item.x & 0xffff;
  const int g = item.x >> 16;
  const int qt = item.y & 0xffff;
  const int split = item.y >> 16;
  const int q_begin = cu_q[b];
  // lengths as the plan kernel reads them: an Lk above max_seqlen_k (or Lq above
  // Lk) is a caller error, cut here so no key past the staged table is read
  const int lk = min(cu_k[b + 1] - cu_k[b], max_seqlen_k);
  const int lq = min(cu_q[b + 1] - q_begin, lk);
  const int ctx0 = lk - lq;                                 // cached positions
  const int wg_q0 = qt * S::kBM;                            // first query row of the tile
  const int wg_last_pos = ctx0 + min(lq, wg_q0 + S::kBM) - 1;
  const int n_kt = wg_last_pos / kBN + 1;
  // A tile that needs more than split_tiles key tiles is cut into
  // ceil(n_kt / split_tiles) key ranges of equal length (to a tile), one item
  // each, so the longest range is as short as the count allows; their partial
  // results meet in the merge kernel.  Split 0 always holds key 0, which every
  // row sees.  A decode row (lq == 1) is one item over all its keys (see
  // decode_row).
  const int n_split = lq == 1 ? 1 : (n_kt + split_tiles - 1) / split_tiles;
  const int range_tiles = (n_kt + n_split - 1) / n_split;
  const int kt_begin = split * range_tiles;
  const int kt_end = min(n_kt, kt_begin + range_tiles);
  const int last_pos = min(kt_end * kBN - 1, wg_last_pos);  // last key this item loads

  const int head = g * G + wave / S::kRB;
  const int w_q0 = wg_q0 + (wave % S::kRB) * 32;            // first query row of the wave
  const int my_row = w_q0 + col;                            // this lane's query row
  const bool row_ok = my_row < lq;
  const int my_pos = ctx0 + my_row;                         // its position in the sequence
  // last position the wave needs; -1 for a wave whose rows all lie past the
  // sequence (a ragged last tile, a decode row's empty row block): it only
  // moves tiles and meets the barriers (mixed batch 63.5 -> 61.1 us)
  const int w_last_pos = w_q0 < lq ? ctx0 + min(lq - 1, w_q0 + 31) : -1;
  // A row that sees fewer than kRestKeys keys can put most of its weight on a
  // few of them, where rounding p to bf16 (relative error up to 2^-9) can move
  // the output by more than the 2e-3 absolute bound when the weighted values
  // cancel; such waves carry p's remainder through P.V as well.  Rows that see
  // more keys take p rounded to nearest bf16, as FlashAttention does.
  const bool short_rows = ctx0 + w_q0 + 1 < kRestKeys;

  // Only keys kt_begin * 64 .. last_pos are ever loaded, so the entries of
  // their blocks are all the workgroup needs.
  const int first_blk = (kt_begin * kBN) >> bs_log2;
  {  // the block-table entries the tile's keys use, staged once
    const int32_t* bt_row = block_table + static_cast<int64_t>(b) * bt_stride + first_blk;
    const int n_bt = (last_pos >> bs_log2) - first_blk + 1;
    for (int i = tid; i < n_bt; i += S::kThreads) bt_lds[i] = bt_row[i];
  }

  // Q^T fragments: lane (half, col) holds dims s*16 + 8*half .. +7 of query row col.
  bf16x8_t qf[S::kSteps];
  {
    const uint16_t* qp = q + static_cast<int64_t>(q_begin + my_row) * q_tok_stride +
                         static_cast<int64_t>(head) * q_head_stride + 8 * half;
#pragma unroll
    for (int s = 0; s < S::kSteps; ++s)
      qf[s] = as_bf16x8(row_ok ? load16(qp + 16 * s) : make_uint4(0, 0, 0, 0));
  }
  // kNew: the item writes the K/V rows of its own positions p0 .. wg_last_pos
  // that lie in its key range, in the iteration whose tile holds them.  Lane
  // (piece i) handles tile row dma_row(i) of every tile -- the row its own DMA
  // brought in -- which is position p0 + ((dma_row(i) - p0) mod 64) + 64 j for
  // j < kPosPerRow; their slots are loaded here, with the query.
  constexpr int kPosPerRow = (S::kBM + kBN - 1) / kBN;
  const int p0 = ctx0 + wg_q0;
  int32_t st_slot[S::kDmaPerWave][kPosPerRow];
  if constexpr (kNew) {
#pragma unroll
    for (int i = 0; i < S::kDmaPerWave; ++i)
#pragma unroll
      for (int j = 0; j < kPosPerRow; ++j) {
        const int pos = p0 + ((dma_row(i) - p0) & (kBN - 1)) + kBN * j;
        st_slot[i][j] = pos <= wg_last_pos ? nk.slot_mapping[q_begin + pos - ctx0] : -1;
      }
  }
  __syncthreads();  // bt_lds ready

  if (lq == 1) {  // a decode row: decode-style over all its keys, then the next item
    if (tid == 0) next_entry = static_cast<int>(gridDim.x + atomicAdd(tickets, 1));
    static_assert(S::kWaves * 2 * D * 4 <= kBN * D * 2, "decode-row partials fit a tile buffer");
    decode_row<D, G, S::kWaves, kNew>(
        q, q_tok_stride, q_head_stride, k_cache, v_cache, bt_lds, bs_log2, block_stride,
        slot_stride, head_stride, g, q_begin, lk, scale_log2, out, out_tok_stride,
        out_head_stride, nk, reinterpret_cast<float*>(k_lds0), reinterpret_cast<float*>(v_lds0));
    continue;  // the loop's barrier keeps the next item's LDS writes behind every read
  }

  // A tile moves from HBM to LDS by DMA (global_load_lds): a wave-wide
  // instruction writes 1 KB of LDS, lane l's 16 bytes at offset 16 l, so each
  // lane fetches the source chunk that the swizzle places at its position.
  // Keys past last_pos are masked (past wg_last_pos they are in the future of
  // every row) or belong to the next split; they are fetched from position
  // last_pos (a readable row), so P.V only ever multiplies finite values.
  // A lane's row within the tile and its source chunks are the same for every
  // tile.
  auto dma = [&](uint16_t* lds, int kt0, auto is_v) {
    constexpr bool kV = decltype(is_v)::value;
    const uint16_t* cache = kV ? v_cache : k_cache;
    if (kNew && kt0 >= ctx0 && kt0 + kBN - 1 <= last_pos) {
      // a whole tile of this step's rows: consecutive rows of the new K or V
      const int32_t tok_b = kV ? nk.v_tok_b : nk.k_tok_b;
      const char* src = (kV ? nk.v : nk.k) + static_cast<int64_t>(q_begin + kt0 - ctx0) * tok_b +
                        g * (kV ? nk.v_head_b : nk.k_head_b);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(src), 0, 0x7fffffff, kBufferFlags);
#pragma unroll
      for (int i = 0; i < S::kDmaPerWave; ++i) {
        const int piece = wave * S::kDmaPerWave + i;
        lds_void_t* dst = (lds_void_t*)(lds + piece * 512);
        const uint32_t voff = kV ? new_vlane : new_klane[i];
        const int soff = piece * S::kRowsPerDma * tok_b;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, soff, 0, 0);
      }
    } else if (tile_in_block && kt0 + kBN - 1 <= last_pos && (!kNew || kt0 + kBN - 1 < ctx0)) {
      const int blk = __builtin_amdgcn_readfirstlane(bt_lds[(kt0 >> bs_log2) - first_blk]);
      const int64_t tile_off =
          blk * block_stride + (kt0 & bs_mask) * slot_stride + g * head_stride;
      // a buffer resource over the tile's first row: scalar base, 32-bit lane offsets
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(cache + tile_off), 0, 0x7fffffff, kBufferFlags);
#pragma unroll
      for (int i = 0; i < S::kDmaPerWave; ++i) {
        const int piece = wave * S::kDmaPerWave + i;
        lds_void_t* dst = (lds_void_t*)(lds + piece * 512);
        const uint32_t voff = kV ? dma_vlane : dma_klane[i];
        const int soff = piece * S::kRowsPerDma * row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, soff, 0, 0);
      }
    } else {
      // Piece by piece: a piece's kRowsPerDma rows lie in one block (block
      // sizes are powers of two of at least 8); rows past last_pos are taken
      // from last_pos, so each piece needs one block-table entry and one
      // uniform base, and a lane only adds its clamped row.  With kNew, lanes
      // whose row is one of this step's (position >= ctx0) read it from the
      // new rows instead, based at the piece's first such row.
#pragma unroll
      for (int i = 0; i < S::kDmaPerWave; ++i) {
        const int piece = wave * S::kDmaPerWave + i;
        const int r0 = min(kt0 + piece * S::kRowsPerDma, last_pos);
        const int lane_row = lane / S::kChunks;
        const int dr = min(lane_row, last_pos - r0);
        lds_void_t* dst = (lds_void_t*)(lds + piece * 512);
        if (kNew && r0 + dr >= ctx0) {
          const int n0 = max(r0, ctx0);
          const int32_t tok_b = kV ? nk.v_tok_b : nk.k_tok_b;
          const char* src = (kV ? nk.v : nk.k) + static_cast<int64_t>(q_begin + n0 - ctx0) * tok_b +
                            g * (kV ? nk.v_head_b : nk.k_head_b);
          const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<char*>(src), 0, 0x7fffffff, kBufferFlags);
          const uint32_t off = (kV ? new_vlane : new_klane[i]) + (r0 + dr - n0 - lane_row) * tok_b;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, off, 0, 0, 0);
        } else {
          const int blk = __builtin_amdgcn_readfirstlane(bt_lds[(r0 >> bs_log2) - first_blk]);
          const int64_t row_off =
              blk * block_stride + (r0 & bs_mask) * slot_stride + g * head_stride;
          const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<uint16_t*>(cache + row_off), 0, 0x7fffffff, kBufferFlags);
          const uint32_t off = (kV ? dma_vlane : dma_klane[i]) + (dr - lane_row) * row_bytes;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, off, 0, 0, 0);
        }
      }
    }
  };

  // kNew: write the rows of this item's positions that the tile in k_src /
  // v_src holds (tile kt) to their slots.  Each lane reads back the 16 bytes
  // its own DMA placed and stores them at the source chunk they came from.
  auto store_tile = [&](const uint16_t* k_src, const uint16_t* v_src, int kt) {
    // Everything lane-dependent is derived here from an opaque copy of the
    // lane index, so the compiler cannot hoist it out of the key loop and hold
    // it in registers for the whole loop (it did: 40 more VGPRs).
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < S::kDmaPerWave; ++i)
#pragma unroll
      for (int j = 0; j < kPosPerRow; ++j) {
        const int piece = wave * S::kDmaPerWave + i;
        const int trow = piece * S::kRowsPerDma + ln / S::kChunks;  // dma_row(i)
        const int pos = p0 + ((trow - p0) & (kBN - 1)) + kBN * j;
        int slot = st_slot[i][j];
        asm volatile("" : "+v"(slot));
        if ((pos >> 6) == kt && slot >= 0) {  // slot -1 also past wg_last_pos
          const uint4 kd = *reinterpret_cast<const uint4*>(k_src + piece * 512 + ln * 8);
          const uint4 vd = *reinterpret_cast<const uint4*>(v_src + piece * 512 + ln * 8);
          const int64_t row = (slot >> bs_log2) * block_stride + (slot & bs_mask) * slot_stride +
                              g * head_stride;
          *reinterpret_cast<uint4*>(nk.k_cache + row +
                                    8 * ((ln % S::kChunks) ^ k_swizzle<D>(trow))) = kd;
          *reinterpret_cast<uint4*>(nk.v_cache + row +
                                    8 * ((ln % S::kChunks) ^ v_swizzle<D>(ln / S::kChunks))) = vd;
        }
        // one row at a time: the tile loop's registers are nearly all taken
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  f32x16_t acc_o[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) acc_o[db] = f32x16_t{};
  // Reference maximum (base-2 scaled units) of this lane's query.  It is raised
  // only when a tile's maximum exceeds it by more than kLazy, so the output is
  // rescaled rarely; meanwhile p = 2^(t - m_ref) stays below 2^kLazy.
  constexpr float kLazy = 8.f;
  float m_ref = -INFINITY;
  float l_run = 0.f;  // this lane's share of the exponential sum

  // S^T = K Q^T for one 64-key tile: two 32-key accumulator chains.  The K
  // operand reads run kLead steps ahead of their MFMAs, in an order the
  // scheduler may not change: left to itself it issued each read right before
  // its MFMA, which then waited the LDS latency (8 prompts of 64..2048: 62.2
  // -> 58.2 us; a chunked-prefill batch with decode rows: 66.6 -> 61.5 us;
  // leads of 3 and 4 were no better).
  auto qk = [&](const uint16_t* kt_lds, f32x16_t (&acc_s)[2]) {
    acc_s[0] = f32x16_t{};
    acc_s[1] = f32x16_t{};
    constexpr int kLead = 2;
    uint4 a0[S::kSteps], a1[S::kSteps];
    static_for<0, S::kSteps + kLead>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < S::kSteps) {
        a0[i] = *reinterpret_cast<const uint4*>(kt_lds + k_off[i]);
        a1[i] = *reinterpret_cast<const uint4*>(kt_lds + k_off[i] + 32 * D);
      }
      if constexpr (i >= kLead) {
        constexpr int s = i - kLead;
        acc_s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0[s]), qf[s], acc_s[0], 0, 0, 0);
        acc_s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1[s]), qf[s], acc_s[1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // One tile: S^T = K Q^T, the causal mask where the tile reaches past the
  // wave's first position, the tile maximum and (rarely) a raised reference
  // maximum; then P and P.V.  Register e of accumulator mb holds the key
  // mb * 32 + 8 (e / 4) + (e % 4) + 4 half of the tile for this lane's query.
  auto compute = [&](const uint16_t* kt_lds, const uint16_t* vt_lds, int kt0, auto with_rest) {
    constexpr bool kRest = decltype(with_rest)::value;
    f32x16_t acc_s[2];
    qk(kt_lds, acc_s);
    // a real branch (most tiles need no mask), not 64 selects on every tile
    if (__builtin_expect(kt0 + kBN - 1 > ctx0 + w_q0, 0)) {
      const int lim = my_pos - kt0 - 4 * half;  // key index (within the tile, sans 4 half) limit
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mb * 32 + 8 * (r / 4) + (r % 4) > lim) acc_s[mb][r] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, acc_s[mb][r]);
    tmax = fmaxf(tmax, lane_xor32(tmax)) * scale_log2;  // scale_log2 > 0
    if (__ballot(tmax > m_ref + kLazy)) {  // wave-uniform: raise the reference
      const float m_new = fmaxf(m_ref, tmax);
      // a row that has seen no key yet (m_ref = m_new = -inf) keeps alpha = 1
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < S::kDB; ++db) acc_o[db] *= alpha;
    }
    // A row of a later split may not have seen a key yet (m_ref = -inf, every
    // score -inf): take its p against 0, which gives 0, instead of NaN.
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;

    // With kRest, p = 2^(t - m_ref) goes in as a bf16 head (truncated) plus a
    // bf16 remainder (~16 significant bits); without, as p rounded to nearest
    // bf16.  Packed two per word in the order the B operand of P.V wants: pair
    // pr holds keys 2 (pr % 8) and 2 (pr % 8) + 1 of accumulator pr / 8, and
    // P.V step ks (keys 16 ks .. 16 ks + 15) takes pairs 4 ks .. 4 ks + 3.
    //
    // The instruction order from here on is fixed by hand: one P.V MFMA per
    // slot, each slot closed by a scheduling fence, with the slot's share of
    // the probability work and the V operand reads for MFMAs a few slots
    // ahead, so the vector ALU forms the probabilities of keys 16 (ks + 1) ..
    // while the matrix cores multiply those of step ks.  Pairs 0-3 (step 0)
    // are formed before the first slot.  Within a step the MFMAs go by pairs
    // of output blocks, head(db), head(db + 1), remainder(db), remainder(db +
    // 1), so each V operand is live for a few slots only; each accumulator
    // still takes the head product before the remainder.
    constexpr int kPer = kRest ? 2 : 1;       // MFMAs per output block and 16 keys
    constexpr int kSlots = 4 * kPer * S::kDB;  // P.V MFMAs of the tile
    constexpr int kDV = 3;                     // slots between a V operand read and its first MFMA
    static_assert(S::kDB % 2 == 0, "output blocks are paired");
    constexpr auto pv_slot = [](int ks, int db) constexpr {
      return kRest ? ks * 2 * S::kDB + 4 * (db / 2) + db % 2 : ks * S::kDB + db;
    };
    // half-pair h: exponentials of pair h / 2 for even h, packing for odd h;
    // -1 = before the first slot
    constexpr auto half_slot = [](int h) constexpr {
      return h < 8 ? -1 : (h - 8) * (3 * kPer * S::kDB) / 24;
    };
    uint32_t w_hi[16], w_lo[16];
    float pe[16][2];
    bf16x8_t va[4][S::kDB];
    float psum = 0.f;
    auto half_pair = [&](auto hc) __attribute__((always_inline)) {
      constexpr int h = decltype(hc)::value;
      constexpr int pr = h / 2, mb = pr / 8, r = 2 * (pr % 8);
      if constexpr (h % 2 == 0) {
        pe[pr][0] = __builtin_amdgcn_exp2f(fmaf(acc_s[mb][r], scale_log2, -m_use));
        pe[pr][1] = __builtin_amdgcn_exp2f(fmaf(acc_s[mb][r + 1], scale_log2, -m_use));
      } else {
        const float p0 = pe[pr][0], p1 = pe[pr][1];
        psum += p0 + p1;
        if constexpr (kRest) {
          const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
          const float r0 = p0 - __uint_as_float(b0 & 0xffff0000u);
          const float r1 = p1 - __uint_as_float(b1 & 0xffff0000u);
          w_hi[pr] = __builtin_amdgcn_perm(b1, b0, kPermHigh);
          w_lo[pr] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), kPermHigh);
        } else {
          w_hi[pr] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t));
        }
      }
    };
    auto slot = [&](auto ic) __attribute__((always_inline)) {
      constexpr int sl = decltype(ic)::value;
      static_for<0, 4>([&](auto ksc) __attribute__((always_inline)) {
        static_for<0, S::kDB>([&](auto dbc) __attribute__((always_inline)) {
          constexpr int ks = decltype(ksc)::value, db = decltype(dbc)::value;
          if constexpr (cmax(pv_slot(ks, db) - kDV, -1) == sl) {
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(vt_lds + ks * 16 * D + v_off[db]));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(vt_lds + ks * 16 * D + 8 * D + v_off[db]));
            va[ks][db] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        });
      });
      if constexpr (sl >= 0) {
        constexpr int ks = sl / (kPer * S::kDB), j = sl % (kPer * S::kDB);
        constexpr int db = kRest ? 2 * (j / 4) + j % 2 : j;
        bf16x8_t pb;
        if constexpr (!kRest || j % 4 < 2)
          pb = as_bf16x8(make_uint4(w_hi[4 * ks], w_hi[4 * ks + 1], w_hi[4 * ks + 2], w_hi[4 * ks + 3]));
        else
          pb = as_bf16x8(make_uint4(w_lo[4 * ks], w_lo[4 * ks + 1], w_lo[4 * ks + 2], w_lo[4 * ks + 3]));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks][db], pb, acc_o[db], 0, 0, 0);
      }
      static_for<0, 32>([&](auto hc) __attribute__((always_inline)) {
        if constexpr (half_slot(decltype(hc)::value) == sl) half_pair(hc);
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<-1, kSlots>(slot);
    l_run += psum;
  };

  // One tile per iteration: start the DMA of the next tile into the other
  // buffer (last read one iteration ago, and every wave has passed the barrier
  // since), multiply the current one, then wait for this wave's DMA and meet
  // at the barrier.  Buffers are chosen at compile time (the loop is unrolled
  // by two) so the compiler can tell the DMA target from the buffer being read.
  auto iteration = [&](int kt, auto buf, auto with_rest) {
    constexpr bool kFirst = std::is_same<decltype(buf), Buf<0>>::value;
    const uint16_t* k_cur = kFirst ? k_lds0 : k_lds1;
    const uint16_t* v_cur = kFirst ? v_lds0 : v_lds1;
    uint16_t* k_nxt = kFirst ? k_lds1 : k_lds0;
    uint16_t* v_nxt = kFirst ? v_lds1 : v_lds0;
    const int kt0 = kt * kBN;
    if (tid == 0 && kt + 1 == kt_end)
      next_entry = static_cast<int>(gridDim.x + atomicAdd(tickets, 1u));
    if (kt + 1 < kt_end) {
      dma(k_nxt, kt0 + kBN, std::false_type{});
      dma(v_nxt, kt0 + kBN, std::true_type{});
    }
    // the stores complete while the tile is multiplied (waited for below)
    if constexpr (kNew)
      if (kt0 <= wg_last_pos && kt0 + kBN > p0) store_tile(k_cur, v_cur, kt);
    if (kt0 <= w_last_pos) compute(k_cur, v_cur, kt0, with_rest);  // else: all in this wave's future
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  dma(k_lds0, kt_begin * kBN, std::false_type{});
  dma(v_lds0, kt_begin * kBN, std::true_type{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // One loop per kind of wave (the waves of a workgroup may run different
  // copies; both meet the same barriers once per tile).
  auto key_loop = [&](auto with_rest) {
    for (int kt = kt_begin; kt < kt_end; kt += 2) {
      iteration(kt, Buf<0>{}, with_rest);
      if (kt + 1 < kt_end) iteration(kt + 1, Buf<1>{}, with_rest);
    }
  };
  if (short_rows)
    key_loop(std::true_type{});
  else
    key_loop(std::false_type{});

  const float l_tot = l_run + lane_xor32(l_run);
  if (n_split > 1) {
  if (row_ok) {
    // Partial result of this key range, against its own reference maximum:
    // acc [split][row][head][D] un-normalised, ml [split][row][head] = (m, l).
    const int64_t slot =
        (static_cast<int64_t>(split) * total_q + q_begin + my_row) * (num_kv_heads * G) + head;
    float* pp = ws_acc + slot * D;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(pp + db * 32 + 8 * r4 + 4 * half) =
            make_float4(acc_o[db][4 * r4], acc_o[db][4 * r4 + 1], acc_o[db][4 * r4 + 2],
                        acc_o[db][4 * r4 + 3]);
    if (half == 0) reinterpret_cast<float2*>(ws_ml)[slot] = make_float2(m_ref, l_tot);
  }
  } else {
  // The wave's 32 x D output tile goes out through LDS so that every store
  // writes whole rows, 16 bytes a lane: written straight from the registers,
  // a lane holds 8 bytes of a row and each store would touch 32 rows 4 KB
  // apart.  The K/V tile buffers are idle once the last tile's barrier has
  // passed; each holds two waves' tiles, row-major with the 16-byte chunk
  // index XOR-swizzled by the row against bank conflicts.  Rows past the
  // sequence's end are staged (whatever they hold) but not stored.
  constexpr int kC = D / 8;  // 16-byte chunks per row
  static_assert(S::kWaves <= 8, "two staged tiles per K/V buffer");
  uint16_t* const buf = wave < 4 ? (wave < 2 ? k_lds0 : k_lds1) : (wave < 6 ? v_lds0 : v_lds1);
  char* const stage = reinterpret_cast<char*>(buf) + (wave % 2) * (32 * D * 2);
  // The lane index is made opaque here so that the staging addresses, which
  // are the same for every item, are computed here instead of being hoisted
  // out of the item loop into registers the tile loop needs.
  int sl = lane;
  asm volatile("" : "+v"(sl));
  const int s_col = sl % 32, s_half = sl / 32;
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < S::kDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int chunk = 4 * db + r4;  // dims db * 32 + 8 * r4 .. + 7
      const uint32_t lo = f32x2_to_bf16x2_rne(acc_o[db][4 * r4 + 0] * inv, acc_o[db][4 * r4 + 1] * inv);
      const uint32_t hi = f32x2_to_bf16x2_rne(acc_o[db][4 * r4 + 2] * inv, acc_o[db][4 * r4 + 3] * inv);
      *reinterpret_cast<uint2*>(stage + s_col * (2 * D) + ((chunk ^ (s_col % kC)) * 16) +
                                8 * s_half) = make_uint2(lo, hi);
    }
  __syncthreads();  // n_split is the workgroup's: every wave is here
  constexpr int kRowsPer = kWave / kC;  // rows one wave-wide read covers
  const int c = sl % kC;
#pragma unroll
  for (int i = 0; i < 32 / kRowsPer; ++i) {
    const int r = i * kRowsPer + sl / kC;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + r * (2 * D) + ((c ^ (r % kC)) * 16));
    if (w_q0 + r < lq)
      *reinterpret_cast<uint4*>(out + static_cast<int64_t>(q_begin + w_q0 + r) * out_tok_stride +
                                static_cast<int64_t>(head) * out_head_stride + c * 8) = v;
  }
  }
  }  // next item
  // The last workgroup to leave resets the claim counter (every other one has
  // made its final claim before it counted itself out), so the work list can
  // serve the next call with the same metadata without being rebuilt.
  if (tid == 0 && atomicAdd(&tickets[kTicketExit], 1u) == gridDim.x - 1) {
    atomicExch(&tickets[0], 0u);
    atomicExch(&tickets[kTicketExit], 0u);
  }
}

// Work list of the prefill kernel, built on the device by one workgroup: one
// entry per (sequence, query tile, key range, kv head), ordered by the number
// of key tiles the entry covers, largest first (a counting sort; the order
// among equal weights is arbitrary and does not change any result), the kv
// heads of one (tile, range) adjacent.  tickets[0] is the claim counter, reset
// here (and by the tile kernel's last workgroup); tickets[1] the number of
// entries; tickets[2] the number of split query tiles, listed in merges[] for
// the merge kernel.
constexpr int kPlanThreads = 1024;
// A decode row's item weighs its key tiles divided by this (its waves split the
// keys and do no MFMA work), for the largest-first order.
constexpr int kDecodeRowShare = 4;
constexpr int kPlanBins = 1024;  // weights >= kPlanBins - 1 share the last bin

// Inclusive prefix sum over the 64 lanes of a wave by DPP moves: shifts right
// by 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside
// the row read 0), then lane 15 added into rows 1 and 3 and lane 31 into rows
// 2 and 3.  Lanes a move does not write get `old`, here 0.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

template <int BM>
__device__ __forceinline__ void plan_body(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int32_t num_seqs,
    int32_t max_seqlen_k, int32_t split_tiles, int32_t num_kv_heads, uint32_t* __restrict__ tickets,
    int2* __restrict__ items, int2* __restrict__ merges) {
  __shared__ int tile_start[kPrefillPlanMaxSeqs + 1];  // first query-tile index per sequence
  __shared__ int n_merges;
  __shared__ int seq_lq[kPrefillPlanMaxSeqs];
  __shared__ int seq_ctx0[kPrefillPlanMaxSeqs];
  __shared__ int bin_count[kPlanBins];
  __shared__ int bin_base[kPlanBins];
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ int wave_sum[kPlanWaves];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  bin_count[tid] = 0;
  if (tid == 0) n_merges = 0;
  static_assert(kPlanBins == kPlanThreads, "one bin per thread");
  static_assert(kPlanWaves <= kWave, "wave totals scanned by one wave");

  // Inclusive scan of x over the block: within each wave, then across the
  // wave totals.  Returns this thread's inclusive prefix; *total receives the
  // block total.
  auto block_scan = [&](int x, int* total) {
    x = wave_inclusive_sum(x);
    if (lane == kWave - 1) wave_sum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      const int v = wave_inclusive_sum(lane < kPlanWaves ? wave_sum[lane] : 0);
      if (lane < kPlanWaves) wave_sum[lane] = v;
    }
    __syncthreads();
    const int excl_waves = wave > 0 ? wave_sum[wave - 1] : 0;
    *total = wave_sum[kPlanWaves - 1];
    __syncthreads();  // wave_sum is reused by the next scan
    return x + excl_waves;
  };

  // 1. per sequence: query rows, cached positions, query tiles and the
  //    exclusive prefix of the tile counts; each thread owns kPer consecutive
  //    sequences
  constexpr int kPer = (kPrefillPlanMaxSeqs + kPlanThreads - 1) / kPlanThreads;
  int n_local[kPer];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = tid * kPer + k;
    n_local[k] = 0;
    if (b < num_seqs) {
      // lengths cut as the tile kernel cuts them
      const int lk = min(cu_k[b + 1] - cu_k[b], max_seqlen_k);
      const int lq = min(cu_q[b + 1] - cu_q[b], lk);
      seq_lq[b] = lq;
      seq_ctx0[b] = lk - lq;
      n_local[k] = (lq + BM - 1) / BM;
    }
    sum += n_local[k];
  }
  int n_tiles = 0;
  int run = block_scan(sum, &n_tiles) - sum;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = tid * kPer + k;
    if (b < num_seqs) tile_start[b] = run;
    run += n_local[k];
  }
  if (tid == 0) tile_start[num_seqs] = n_tiles;
  __syncthreads();

  // Visit every (tile, range): tile i belongs to the last sequence whose first
  // tile is at or before i (sequences without tiles share their successor's
  // start).
  auto for_each_range = [&](auto&& fn) {
    for (int i = tid; i < n_tiles; i += kPlanThreads) {
      int lo = 0, hi = num_seqs - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (tile_start[mid] <= i) lo = mid; else hi = mid - 1;
      }
      const int b = lo;
      const int qt = i - tile_start[b];
      const int n_kt = (seq_ctx0[b] + min(seq_lq[b], (qt + 1) * BM) - 1) / kBN + 1;
      if (seq_lq[b] == 1) {  // a decode row: one item, its keys shared by the waves
        fn(b, qt, 0, 1, min(max(1, n_kt / kDecodeRowShare), kPlanBins - 1));
        continue;
      }
      const int n_split = (n_kt + split_tiles - 1) / split_tiles;
      const int range_tiles = (n_kt + n_split - 1) / n_split;  // equal lengths, to a tile
      for (int sp = 0; sp < n_split; ++sp)
        fn(b, qt, sp, n_split, min(min(range_tiles, n_kt - sp * range_tiles), kPlanBins - 1));
    }
  };

  // 2. ranges per weight
  for_each_range([&](int, int, int, int, int w) { atomicAdd(&bin_count[w], 1); });
  __syncthreads();
  // 3. bin bases for descending weight order, in entries
  const int c = bin_count[kPlanBins - 1 - tid] * num_kv_heads;
  int n_entries = 0;
  bin_base[kPlanBins - 1 - tid] = block_scan(c, &n_entries) - c;
  bin_count[kPlanBins - 1 - tid] = 0;
  __syncthreads();
  // 4. placement: the kv heads of a range take consecutive entries
  for_each_range([&](int b, int qt, int sp, int n_split, int w) {
    const int at = bin_base[w] + atomicAdd(&bin_count[w], num_kv_heads);
    for (int g = 0; g < num_kv_heads; ++g)
      items[at + g] = make_int2(b | (g << 16), qt | (sp << 16));
    if (sp == 0 && n_split > 1) merges[atomicAdd(&n_merges, 1)] = make_int2(b, qt);
  });
  __syncthreads();
  if (tid == 0) {
    tickets[0] = 0u;
    tickets[1] = static_cast<uint32_t>(n_entries);
    tickets[2] = static_cast<uint32_t>(n_merges);
    tickets[kTicketExit] = 0u;  // workgroups of the tile kernel that have left
  }
}

template <int BM>
__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int32_t num_seqs,
    int32_t max_seqlen_k, int32_t split_tiles, int32_t num_kv_heads,
    uint32_t* __restrict__ tickets, int2* __restrict__ items, int2* __restrict__ merges) {
  plan_body<BM>(cu_q, cu_k, num_seqs, max_seqlen_k, split_tiles, num_kv_heads, tickets, items,
                merges);
}

// Merge of the key-range partials of split query tiles ([Intro §9.5]: each
// partial carries its own maximum m_s and sum l_s, so the output is
// sum_s 2^(m_s - m*) acc_s / sum_s 2^(m_s - m*) l_s with m* = max_s m_s).
// A query tile's (row, query head, 4 dims) items are spread over
// kMergeParts workgroups, one item per thread, so the many short dependent
// loads of a merge overlap across waves; consecutive threads take
// consecutive dims, so each partial row is read with coalesced 16-byte loads.
template <int D, int G>
struct MergeShape {
  static constexpr int kChunks = D / 4;                                  // items per (row, head)
  static constexpr int kItems = PrefillShape<D, G>::kBM * G * kChunks;  // per query tile
  static constexpr int kParts = kItems / 256;
  static_assert(kItems % 256 == 0, "a tile's items fill whole workgroups");
};

template <int D, int G>
__global__ __launch_bounds__(256) void prefill_merge_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int32_t num_kv_heads,
    int32_t max_seqlen_k, const uint32_t* __restrict__ tickets, const int2* __restrict__ merges,
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml, int32_t total_q,
    int32_t split_tiles, uint16_t* __restrict__ out, int64_t out_tok_stride,
    int64_t out_head_stride) {
  using S = PrefillShape<D, G>;
  using M = MergeShape<D, G>;
  // Only the split tiles the plan listed are visited: (tile, kv head, part)
  // pieces are strided over a fixed grid.
  const int64_t n_work = static_cast<int64_t>(tickets[2]) * num_kv_heads * M::kParts;
  for (int64_t work = blockIdx.x; work < n_work; work += gridDim.x) {
  const int part = static_cast<int>(work % M::kParts);
  const int g = static_cast<int>((work / M::kParts) % num_kv_heads);
  const int2 tile = merges[work / (static_cast<int64_t>(M::kParts) * num_kv_heads)];
  const int item = part * 256 + threadIdx.x;
  const int b = tile.x;
  const int qt = tile.y;
  const int q_begin = cu_q[b];
  const int lk = min(cu_k[b + 1] - cu_k[b], max_seqlen_k);
  const int lq = min(cu_q[b + 1] - q_begin, lk);
  const int wg_q0 = qt * S::kBM;
  const int wg_last_pos = lk - lq + min(lq, wg_q0 + S::kBM) - 1;
  const int n_split = (wg_last_pos / kBN + split_tiles) / split_tiles;
  const int c = item % M::kChunks;
  const int i = (item / M::kChunks) % G;
  const int r = item / (M::kChunks * G);
  if (wg_q0 + r >= lq) continue;
  const int64_t row = q_begin + wg_q0 + r;
  const int64_t head = g * G + i;
  const int64_t num_q_heads = static_cast<int64_t>(num_kv_heads) * G;
  const int64_t split_stride = static_cast<int64_t>(total_q) * num_q_heads;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + row * num_q_heads + head;
  const float* acc = ws_acc + (row * num_q_heads + head) * D + 4 * c;
  // split 0 holds key 0, which every row sees, so m_star is finite
  float m_star = -INFINITY;
  for (int sp = 0; sp < n_split; ++sp) m_star = fmaxf(m_star, ml[sp * split_stride].x);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float l = 0.f;
  for (int sp = 0; sp < n_split; ++sp) {
    const float2 st = ml[sp * split_stride];
    const float4 v = *reinterpret_cast<const float4*>(acc + sp * split_stride * D);
    const float w = st.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.x - m_star);
    l = fmaf(w, st.y, l);
    o.x = fmaf(w, v.x, o.x);
    o.y = fmaf(w, v.y, o.y);
    o.z = fmaf(w, v.z, o.z);
    o.w = fmaf(w, v.w, o.w);
  }
  const float inv = 1.f / l;
  const uint32_t lo = f32x2_to_bf16x2_rne(o.x * inv, o.y * inv);
  const uint32_t hi = f32x2_to_bf16x2_rne(o.z * inv, o.w * inv);
  *reinterpret_cast<uint2*>(out + row * out_tok_stride + head * out_head_stride + 4 * c) =
      make_uint2(lo, hi);
  }
}

// Workgroups of the tile kernel resident per CU, and in total, on the current
// device.  The answer depends on the kernel, its LDS (the block-table stage,
// sized from max_seqlen_k) and the device; it is asked of the runtime once per
// device and LDS size.
template <int D, int G, bool kNew>
int resident_per_cu(size_t lds) {
  constexpr int kMaxDevices = 64, kMaxLds = 64;
  static int known[kMaxDevices][kMaxLds] = {};  // 0: not asked yet; indexed by lds / 512
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  const size_t li = lds / 512;
  const bool cache = dev >= 0 && dev < kMaxDevices && li < kMaxLds;
  if (cache && known[dev][li] > 0) return known[dev][li];
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, prefill_kernel<D, G, kNew>,
                                                   PrefillShape<D, G>::kThreads, lds) != hipSuccess)
    return 1;
  occ = occ > 0 ? occ : 1;
  if (cache) known[dev][li] = occ;
  return occ;
}

template <int D, int G, bool kNew>
int resident_slots(size_t lds, hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static int cus_known[kMaxDevices] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return 0;
  int cus = dev >= 0 && dev < kMaxDevices ? cus_known[dev] : 0;
  if (cus == 0) {
    *err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (*err != hipSuccess) return 0;
    if (dev >= 0 && dev < kMaxDevices) cus_known[dev] = cus;
  }
  return cus * resident_per_cu<D, G, kNew>(lds);
}

template <int D, int G, bool kNew>
hipError_t run(const PrefillArgs& a, const NewKV& nk, hipStream_t stream) {
  using S = PrefillShape<D, G>;
  const int bs_log2 = __builtin_ctz(static_cast<unsigned>(a.block_size));
  const size_t bt_bytes = static_cast<size_t>((a.max_seqlen_k + a.block_size - 1) >> bs_log2) * 4;
  // split_tiles >= every tile's key-tile count when nothing is split
  const int split_tiles = a.num_splits > 1 ? a.split_keys / kBN : (a.max_seqlen_k + kBN - 1) / kBN;
  hipError_t err = hipSuccess;
  if (!a.planned) {  // else the work list is in the workspace already (pa_prefill_plan)
    hipLaunchKernelGGL((prefill_plan_kernel<S::kBM>), dim3(1), dim3(kPlanThreads), 0, stream,
                       a.cu_seqlens_q, a.cu_seqlens_k, a.num_seqs, a.max_seqlen_k, split_tiles,
                       a.num_kv_heads, a.tickets, a.items, a.merges);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.plan_only) return hipSuccess;
  // one workgroup per resident slot: they stay until the work list is empty
  const int slots = resident_slots<D, G, kNew>(bt_bytes, &err);
  if (err != hipSuccess) return err;
  const int cus = slots / cmax(1, resident_per_cu<D, G, kNew>(bt_bytes));
  hipLaunchKernelGGL((prefill_kernel<D, G, kNew>), dim3(slots), dim3(S::kThreads), bt_bytes,
                     stream, static_cast<const uint16_t*>(a.q), a.q_tok_stride, a.q_head_stride,
                     static_cast<const uint16_t*>(a.k_cache), static_cast<const uint16_t*>(a.v_cache),
                     a.cu_seqlens_q, a.cu_seqlens_k, a.block_table, a.block_table_stride,
                     a.num_kv_heads, bs_log2, a.max_seqlen_k, a.scale * kLog2e, split_tiles,
                     a.tickets, a.items,
                     a.ws_acc, a.ws_ml, a.total_q, static_cast<uint16_t*>(a.out),
                     a.out_tok_stride, a.out_head_stride, a.geom.block, a.geom.slot, a.geom.head,
                     nk);
  err = hipGetLastError();
  if (err != hipSuccess || a.num_splits == 1) return err;
  hipLaunchKernelGGL((prefill_merge_kernel<D, G>), dim3(4 * cus), dim3(256), 0, stream,
                     a.cu_seqlens_q, a.cu_seqlens_k, a.num_kv_heads, a.max_seqlen_k, a.tickets,
                     a.merges,
                     a.ws_acc, a.ws_ml, a.total_q, split_tiles, static_cast<uint16_t*>(a.out),
                     a.out_tok_stride, a.out_head_stride);
  return hipGetLastError();
}

template <int D, int G>
hipError_t run(const PrefillArgs& a, hipStream_t stream) {
  if (!a.store) return run<D, G, false>(a, NewKV{}, stream);
  // This step's rows: the tile kernel reads them from k / v and stores them.
  const StoreArgs& st = *a.store;
  const int64_t kt = st.k_tok_stride * 2, vt = st.v_tok_stride * 2;
  // lane offsets within a 64-row tile of the new rows are 32-bit
  if (kt > (int64_t{1} << 24) || vt > (int64_t{1} << 24)) return hipErrorInvalidValue;
  const NewKV nk{static_cast<const char*>(st.k), static_cast<const char*>(st.v),
                 static_cast<int32_t>(kt), static_cast<int32_t>(vt), st.k_head_stride * 2,
                 st.v_head_stride * 2, st.slot_mapping, static_cast<uint16_t*>(st.k_cache),
                 static_cast<uint16_t*>(st.v_cache)};
  return run<D, G, true>(a, nk, stream);
}

template <int D>
hipError_t pick_group(const PrefillArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return run<D, 1>(a, stream);
    case 2: return run<D, 2>(a, stream);
    case 4: return run<D, 4>(a, stream);
    case 8: return run<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  return a.head_dim == 128 ? pick_group<128>(a, stream) : pick_group<64>(a, stream);
}

}  // namespace pa
