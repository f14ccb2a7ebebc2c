// Split statistics of a shared prefix for batched decode, bf16 MFMA.
//
// What is computed ("大模型推理入门与 nano-vLLM 源码详解" [Intro] §9.5, §10.5,
// §13.3): with the prefix cache, sequences that begin with the same prompt
// hold the same physical blocks at the front of their block tables
// [Intro §10.5].  In a decode step every member of such a group attends over
// those positions with its own query, so the flash-decoding split statistics
// (m, l, acc) of the splits inside the shared prefix [Intro §9.5] are one
// computation per member over the same keys.  This pass computes them for all
// members of a group and all query heads of a kv head together, reading each
// prefix key once per workgroup of 32 query rows instead of once per
// sequence; the partition pass skips those splits and the reduce merges them
// with the rest as usual.
//
// Design for gfx950 (wave64, v_mfma_f32_32x32x16_bf16):
// * A workgroup owns one (group, kv head, split) and 32 query rows: the G
//   query heads of 32 / G members, row r = member (r / G), head (r % G).  Its
//   4 waves take the split's 64-key tiles in turn (wave w: tiles w, w + 4,
//   ...) and meet in LDS at the end, where their statistics are merged as the
//   reduce merges splits.
// * Scores are computed transposed, S^T = K Q^T.  K goes from the cache
//   straight into the A operand (a lane holds 16 bytes of one key's row);
//   Q^T is held in registers for the whole split.  In the accumulator layout a
//   lane owns one query row and 16 keys per 32-key block, so the maximum and
//   the sum are in-lane plus one exchange with lane ^ 32.
// * O^T = V^T P^T.  A V tile goes from the cache into the wave's own LDS
//   region by DMA (global_load_lds, 16 bytes a lane), row-major with its
//   16-byte chunks XOR-swizzled; each V^T operand is read with two
//   ds_read_b64_tr_b16, whose per-16-lane transpose hands a lane 4 keys of one
//   dim in the order in which the score accumulator holds P.
// * P enters P.V as a bf16 head (truncated) plus its bf16 remainder, about 16
//   significant bits, and the running maximum is exact (the output is rescaled
//   whenever it grows), so m is the split's maximum score as the partition
//   pass writes it and the statistics agree with it to fp32 rounding.
// * Members are found on the device: wave 0 scans prefix_group with ballots,
//   so the caller needs no member lists, and the block ids of the prefix come
//   from the group's first member's block-table row.

#include <math.h>

#include <algorithm>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_store_rows.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTile = 64;     // keys per tile
constexpr int kRowsWg = 32;   // query rows per workgroup
constexpr int kWavesWg = 4;   // waves per workgroup
// v_perm_b32 selector keeping the high halves: b.hi | a.hi << 16.
constexpr uint32_t kPermHigh = 0x07060302u;

template <int D>
struct PrefixShape {
  static constexpr int kSteps = D / 16;               // MFMA k-steps over head_dim
  static constexpr int kDB = D / 32;                  // 32-wide output blocks over head_dim
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kRowsPerLoad = kWave / kChunks;
  static constexpr int kLoadsPerTile = kTile / kRowsPerLoad;
  // one wave's LDS: a V tile, later its 32 x (D + 4) fp32 partial output
  static constexpr int kAccStride = D + 4;            // padded against bank conflicts
  static constexpr int kRegionElems =
      (kTile * D > kRowsWg * kAccStride * 2) ? kTile * D : kRowsWg * kAccStride * 2;
  static_assert((kRegionElems * 2) % 256 == 0, "regions must start on a bank line");
};

// LDS position of 16-byte chunk c of V row `key` is c ^ v_swizzle(key): the 32
// lanes a transpose read serves together then hit distinct banks.
template <int D>
__device__ __forceinline__ int v_swizzle(int key) {
  return D == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// The partition pass's work list for this call, built by one workgroup: the
// (sequence, split) pairs that pass computes -- splits [lo, n) of sequence b,
// n = ceil(L / P) for its context L (cut to max_ctx), lo the first split the
// shared-prefix pass does not take (the partition kernel's own skip rule) --
// full splits first, then the partial last splits longest first (32 length
// classes), so the hardware hands out the longest work first and the short
// splits fill the end.  list[0] is the count; entries are b << 16 | split.
// Order within a class follows the atomics and does not matter: every entry
// is computed the same wherever it sits.
__device__ __forceinline__ void build_work_list(
    int32_t* __restrict__ list, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ prefix_group, const int32_t* __restrict__ prefix_tokens,
    int32_t num_seqs, int32_t num_groups, int32_t max_prefix, int32_t max_ctx, int32_t P) {
  constexpr int kClasses = 33;  // 0: full splits; 1..32: partial, longest first
  __shared__ int count[kClasses], offset[kClasses];
  const int tid = threadIdx.x;
  if (tid < kClasses) count[tid] = 0;
  __syncthreads();
  auto range = [&](int b, int& lo, int& n, int& tail) {
    const int ctx = min(context_lens[b], max_ctx);
    n = ctx > 0 ? (ctx + P - 1) / P : 0;
    const int grp = prefix_group[b];
    lo = n > 0 && static_cast<unsigned>(grp) < static_cast<unsigned>(num_groups)
             ? max(min(min(prefix_tokens[grp], max_prefix) / P, (ctx - 1) / P), 0)
             : 0;
    tail = ctx - (n - 1) * P;  // 1 .. P when n > 0
  };
  auto cls = [&](int tail) { return 1 + (P - 1 - tail) * 32 / P; };  // 1 .. 32 for tail < P
  for (int b = tid; b < num_seqs; b += blockDim.x) {
    int lo, n, tail;
    range(b, lo, n, tail);
    if (n <= lo) continue;
    const int full = tail == P ? n - lo : n - 1 - lo;
    if (full > 0) atomicAdd(&count[0], full);
    if (tail < P) atomicAdd(&count[cls(tail)], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int total = 0;
    for (int c = 0; c < kClasses; ++c) {
      offset[c] = total;
      total += count[c];
    }
    list[0] = total;
  }
  __syncthreads();
  for (int b = tid; b < num_seqs; b += blockDim.x) {
    int lo, n, tail;
    range(b, lo, n, tail);
    if (n <= lo) continue;
    const int full = tail == P ? n - lo : n - 1 - lo;
    if (full > 0) {
      const int at = atomicAdd(&offset[0], full);
      for (int k = 0; k < full; ++k) list[1 + at + k] = (b << 16) | (lo + k);
    }
    if (tail < P) list[1 + atomicAdd(&offset[cls(tail)], 1)] = (b << 16) | (n - 1);
  }
}

template <int D, int G>
__global__ __launch_bounds__(kWavesWg * kWave) void prefix_split_kernel(
    const uint16_t* __restrict__ q, int64_t q_seq_stride, int64_t q_head_stride,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int64_t bt_stride,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ prefix_group,
    const int32_t* __restrict__ prefix_tokens, int32_t num_seqs, int32_t num_kv_heads,
    int32_t bs_log2, int32_t max_prefix, int32_t partition_tokens, int32_t num_splits,
    float scale_log2, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    int64_t block_stride, int64_t slot_stride, int64_t head_stride, StoreRows store,
    int32_t store_x, int32_t* __restrict__ work_list, int32_t max_ctx) {
  using S = PrefixShape<D>;
  constexpr int kMembers = kRowsWg / G;  // members per workgroup
  __shared__ __attribute__((aligned(1024))) uint16_t region[kWavesWg][S::kRegionElems];
  __shared__ float m_lds[kWavesWg][kRowsWg];
  __shared__ float l_lds[kWavesWg][kRowsWg];
  __shared__ int member_lds[kMembers];
  __shared__ int leader_lds, count_lds;
  extern __shared__ int32_t bt_lds[];  // the split's block ids, from the leader's row

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int half = lane / 32;
  const int col = lane % 32;
  // The last store_x columns of the grid copy this step's K/V rows into the
  // cache instead (none when store.rows is 0); a stored row is never a slot
  // this pass reads (the new positions lie past every group's prefix).
  // The column before them builds the partition pass's work list (its first
  // workgroup; the others return).
  const int plan_x = work_list ? 1 : 0;
  if (plan_x && static_cast<int>(blockIdx.x) == static_cast<int>(gridDim.x) - store_x - 1) {
    if (blockIdx.y == 0 && blockIdx.z == 0)
      build_work_list(work_list, context_lens, prefix_group, prefix_tokens, num_seqs,
                      static_cast<int>(gridDim.y) / num_kv_heads, max_prefix, max_ctx,
                      partition_tokens);
    return;
  }
  if (static_cast<int>(blockIdx.x) >= static_cast<int>(gridDim.x) - store_x) {
    const int wg = blockIdx.x - (gridDim.x - store_x) + store_x * (blockIdx.y + gridDim.y * blockIdx.z);
    store_rows<uint4>(store, wg * kWavesWg + wave, store_x * gridDim.y * gridDim.z * kWavesWg);
    return;
  }
  const int tile = blockIdx.x;
  const int grp = blockIdx.y / num_kv_heads;
  const int h = blockIdx.y % num_kv_heads;
  const int split = blockIdx.z;
  const int P = partition_tokens;

  // Splits wholly inside the group's prefix; the rest belong to the partition pass.
  const int n_prefix_splits = min(prefix_tokens[grp], max_prefix) / P;
  if (split >= n_prefix_splits) return;  // uniform

  // Members with rank tile * kMembers .. + kMembers - 1 among the sequences of
  // this group, in batch order, and the group's first member (the leader).
  // kScan chunks of 64 sequences per round, their loads issued together.
  if (wave == 0) {
    constexpr int kScan = 4;
    const int r_lo = tile * kMembers;
    int seen = 0, leader = -1;
    for (int c0 = 0; c0 < num_seqs && seen < r_lo + kMembers; c0 += kScan * kWave) {
      int grp_of[kScan];
#pragma unroll
      for (int k = 0; k < kScan; ++k) {
        const int b = c0 + k * kWave + lane;
        grp_of[k] = b < num_seqs ? prefix_group[b] : -1;
      }
#pragma unroll
      for (int k = 0; k < kScan; ++k) {
        const int c = c0 + k * kWave;
        const bool is_member = grp_of[k] == grp;
        const uint64_t mask = __ballot(is_member);
        const int rank = seen + __popcll(mask & ((uint64_t{1} << lane) - 1));
        if (is_member && rank >= r_lo && rank < r_lo + kMembers) member_lds[rank - r_lo] = c + lane;
        if (leader < 0 && mask) leader = c + __builtin_ctzll(mask);
        seen += __popcll(mask);
      }
    }
    if (lane == 0) {
      leader_lds = leader;
      count_lds = min(max(seen - r_lo, 0), kMembers);
    }
  }
  __syncthreads();
  const int n_members = count_lds;
  if (n_members == 0) return;  // uniform: this tile lies past the group's last member
  const int leader = leader_lds;

  const int key_begin = split * P;
  const int first_blk = key_begin >> bs_log2;
  {
    const int n_bt = ((key_begin + P - 1) >> bs_log2) - first_blk + 1;
    const int32_t* row = block_table + static_cast<int64_t>(leader) * bt_stride + first_blk;
    for (int i = tid; i < n_bt; i += kWavesWg * kWave) bt_lds[i] = row[i];
  }

  // Q^T fragments: lane (half, col) holds dims s*16 + 8*half .. +7 of row col.
  const int my_member = col / G;
  const bool row_ok = my_member < n_members;
  bf16x8_t qf[S::kSteps];
  {
    const int b = row_ok ? member_lds[my_member] : 0;
    const uint16_t* qp = q + static_cast<int64_t>(b) * q_seq_stride +
                         static_cast<int64_t>(h * G + col % G) * q_head_stride + 8 * half;
#pragma unroll
    for (int s = 0; s < S::kSteps; ++s)
      qf[s] = as_bf16x8(row_ok ? load16(qp + 16 * s) : make_uint4(0, 0, 0, 0));
  }
  __syncthreads();  // bt_lds ready

  const int bs_mask = (1 << bs_log2) - 1;
  auto row_of = [&](int key) -> int64_t {
    const uint32_t blk = bt_lds[(key >> bs_log2) - first_blk];
    return static_cast<int64_t>(blk) * block_stride + (key & bs_mask) * slot_stride +
           h * head_stride;
  };

  uint16_t* my_region = region[wave];
  // V operand reads: for read t of step ks, lane (half, col) supplies the row
  // of key ks*16 + 8t + 4 half + (col % 16) / 4 and dims db*32 + 16 (col / 16)
  // + 4 (col % 4) .. +3; the read hands it keys ks*16 + 8t + 4 half + e (e =
  // 0..3) of dim db*32 + col.  The swizzle of key + 8 equals that of key.
  int v_off[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) {
    const int key = 4 * half + (col % 16) / 4;
    const int j4 = col % 4;
    const int chunk = db * 4 + 2 * (col / 16) + j4 / 2;
    v_off[db] = key * D + 8 * (chunk ^ v_swizzle<D>(key)) + 4 * (j4 % 2);
  }
  // V DMA: instruction i fills rows i * kRowsPerLoad .. + kRowsPerLoad - 1;
  // lane l brings the source chunk the swizzle places at position l % kChunks
  // of row l / kChunks (the swizzle depends only on row bits below kRowsPerLoad).
  static_assert(S::kRowsPerLoad % 4 == 0, "V swizzle must not depend on the load");
  const int dma_row = lane / S::kChunks;
  const int dma_chunk = (lane % S::kChunks) ^ v_swizzle<D>(dma_row);

  f32x16_t acc_o[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) acc_o[db] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = P / kTile;
  for (int t = wave; t < n_tiles; t += kWavesWg) {
    const int key0 = key_begin + t * kTile;
    // K operands of both 32-key blocks, straight into registers.
    uint4 ka[2][S::kSteps];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint16_t* kp = k_cache + row_of(key0 + kb * 32 + col) + 8 * half;
#pragma unroll
      for (int s = 0; s < S::kSteps; ++s) ka[kb][s] = load16(kp + 16 * s);
    }
    // The V tile into this wave's region (read only by this wave).
#pragma unroll
    for (int i = 0; i < S::kLoadsPerTile; ++i) {
      const uint16_t* src =
          v_cache + row_of(key0 + i * S::kRowsPerLoad + dma_row) + 8 * dma_chunk;
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(my_region + i * 512), 16, 0, 0);
    }

    f32x16_t acc_s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int s = 0; s < S::kSteps; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[kb][s]), qf[s],
                                                           acc_s[kb], 0, 0, 0);
    }

    // Exact running maximum (base-2 units; scale_log2 > 0).
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, acc_s[kb][r]);
    tmax = fmaxf(tmax, lane_xor32(tmax)) * scale_log2;
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) acc_o[db] *= alpha;

    // p as a truncated bf16 head and the bf16 remainder, packed two per word in
    // the order the B operand of P.V wants: pair pr holds keys 2 (pr % 8) and
    // 2 (pr % 8) + 1 of accumulator pr / 8; step ks takes pairs 4 ks .. 4 ks + 3.
    uint32_t w_hi[16], w_lo[16];
    float psum = 0.f;
#pragma unroll
    for (int pr = 0; pr < 16; ++pr) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(acc_s[pr / 8][2 * (pr % 8)], scale_log2, -m_new));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(acc_s[pr / 8][2 * (pr % 8) + 1], scale_log2, -m_new));
      psum += p0 + p1;
      const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
      const float r0 = p0 - __uint_as_float(b0 & 0xffff0000u);
      const float r1 = p1 - __uint_as_float(b1 & 0xffff0000u);
      w_hi[pr] = __builtin_amdgcn_perm(b1, b0, kPermHigh);
      w_lo[pr] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), kPermHigh);
    }
    l_run += psum;

    // this wave's V DMA has landed (also a compiler fence: no LDS read moves above it)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t ph = as_bf16x8(make_uint4(w_hi[4 * ks], w_hi[4 * ks + 1], w_hi[4 * ks + 2],
                                               w_hi[4 * ks + 3]));
      const bf16x8_t pl = as_bf16x8(make_uint4(w_lo[4 * ks], w_lo[4 * ks + 1], w_lo[4 * ks + 2],
                                               w_lo[4 * ks + 3]));
#pragma unroll
      for (int db = 0; db < S::kDB; ++db) {
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(my_region + ks * 16 * D + v_off[db]));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(my_region + ks * 16 * D + 8 * D + v_off[db]));
        const bf16x8_t va =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, ph, acc_o[db], 0, 0, 0);
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pl, acc_o[db], 0, 0, 0);
      }
    }
    // The region is refilled by the next tile's DMA: every read of this one
    // returns first, and no DMA is moved above this point.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  // This wave's partial: row col, dims db*32 + 8 r4 + 4 half .. +3 in
  // acc_o[db][4 r4 ..]; a wave with no tile leaves m = -inf, l = 0, acc = 0.
  const float l_tot = l_run + lane_xor32(l_run);
  float* acc_lds = reinterpret_cast<float*>(my_region);
#pragma unroll
  for (int db = 0; db < S::kDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(acc_lds + col * S::kAccStride + db * 32 + 8 * r4 + 4 * half) =
          make_float4(acc_o[db][4 * r4], acc_o[db][4 * r4 + 1], acc_o[db][4 * r4 + 2],
                      acc_o[db][4 * r4 + 3]);
  if (half == 0) {
    m_lds[wave][col] = m_run;
    l_lds[wave][col] = l_tot;
  }
  __syncthreads();

  // Merge the waves' partials and write the split statistics in the layout of
  // the partition pass: thread t writes dims (t % 8) * D / 8 .. of row t / 8.
  constexpr int kDimsPerThread = D / 8;
  const int row = tid / 8;
  const int d0 = (tid % 8) * kDimsPerThread;
  const int member = row / G;
  if (member >= n_members) return;
  const int b = member_lds[member];
  const int ctx = context_lens[b];
  // A member's own last position is never in a skipped split (it may be this
  // step's token); the partition pass computes the split that holds it.
  const int n_skip = ctx >= 1 ? min(n_prefix_splits, (ctx - 1) / P) : 0;
  if (split >= n_skip) return;
  float m_star = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWavesWg; ++w) m_star = fmaxf(m_star, m_lds[w][row]);
  float c[kWavesWg], l_sum = 0.f;
#pragma unroll
  for (int w = 0; w < kWavesWg; ++w) {
    c[w] = m_lds[w][row] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_lds[w][row] - m_star);
    l_sum = fmaf(c[w], l_lds[w][row], l_sum);
  }
  const int head = h * G + row % G;
  const int64_t idx =
      (static_cast<int64_t>(b) * (num_kv_heads * G) + head) * num_splits + split;
  float* dst = ws_acc + idx * D + d0;
#pragma unroll
  for (int e = 0; e < kDimsPerThread; e += 4) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWavesWg; ++w) {
      const float4 a = *reinterpret_cast<const float4*>(
          reinterpret_cast<const float*>(region[w]) + row * S::kAccStride + d0 + e);
      o.x = fmaf(c[w], a.x, o.x);
      o.y = fmaf(c[w], a.y, o.y);
      o.z = fmaf(c[w], a.z, o.z);
      o.w = fmaf(c[w], a.w, o.w);
    }
    *reinterpret_cast<float4*>(dst + e) = o;
  }
  if (tid % 8 == 0) reinterpret_cast<float2*>(ws_ml)[idx] = make_float2(m_star, l_sum);
}

template <int D, int G>
hipError_t run_prefix(const PrefixArgs& a, hipStream_t stream) {
  const int bs_log2 = __builtin_ctz(static_cast<unsigned>(a.block_size));
  const size_t lds = (static_cast<size_t>(a.partition_tokens / a.block_size) + 2) * sizeof(int32_t);
  const int tiles = (a.num_seqs * G + kRowsWg - 1) / kRowsWg;
  StoreRows store{};  // rows = 0: no store
  int store_x = 0;
  if (a.store) {
    if (!store_rows_16(*a.store, &store)) return hipErrorInvalidValue;
    // extra columns of (groups * kv heads * prefix splits) workgroups, about 4 rows a wave
    const int64_t per_col = int64_t{kWavesWg} * 4 * a.num_groups * a.num_kv_heads *
                            (a.max_prefix_tokens / a.partition_tokens);
    store_x = static_cast<int>(std::min<int64_t>((store.rows + per_col - 1) / per_col, 1024));
    store_x = std::max(store_x, 1);
  }
  dim3 grid(tiles + (a.work_list ? 1 : 0) + store_x, a.num_groups * a.num_kv_heads,
            a.max_prefix_tokens / a.partition_tokens);
  hipLaunchKernelGGL((prefix_split_kernel<D, G>), grid, dim3(kWavesWg * kWave), lds, stream,
                     static_cast<const uint16_t*>(a.q), a.q_seq_stride, a.q_head_stride,
                     static_cast<const uint16_t*>(a.k_cache),
                     static_cast<const uint16_t*>(a.v_cache), a.block_table,
                     a.block_table_stride, a.context_lens, a.prefix_group, a.prefix_tokens,
                     a.num_seqs, a.num_kv_heads, bs_log2, a.max_prefix_tokens,
                     a.partition_tokens, a.num_splits, a.scale * kLog2e, a.ws_acc, a.ws_ml,
                     a.geom.block, a.geom.slot, a.geom.head, store, store_x, a.work_list,
                     a.max_context_len);
  return hipGetLastError();
}

template <int D>
hipError_t pick_prefix_group(const PrefixArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return run_prefix<D, 1>(a, stream);
    case 2: return run_prefix<D, 2>(a, stream);
    case 4: return run_prefix<D, 4>(a, stream);
    case 8: return run_prefix<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefix_splits(const PrefixArgs& a, hipStream_t stream) {
  return a.head_dim == 128 ? pick_prefix_group<128>(a, stream) : pick_prefix_group<64>(a, stream);
}

}  // namespace pa
