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
//   score registers.  V is written to LDS transposed ([dim][key]) and with
//   the keys of each 16-key group permuted to match the order in which the
//   accumulator layout holds them, so every MFMA operand is a single 16-byte
//   LDS read.
// * Each p is split into a bf16 head and a bf16 remainder (p - head) and both
//   go through the P.V MFMA, so P carries ~16 significant bits instead of
//   bf16's 8: with bf16 P alone, rows whose weighted values cancel can miss
//   a 2e-3 absolute error bound.  This costs half again the MFMA work.
// * LDS rows are padded by 16 bytes so the 16-byte reads of 32 consecutive
//   rows fall in distinct banks.
// * K/V tiles are double-buffered in LDS: while the MFMAs read one buffer,
//   the tile after it (fetched from HBM into registers one tile earlier) is
//   written into the other, so each tile costs one barrier.
// * The sequence's block-table entries are staged in LDS once, so a K/V
//   address never waits on a global load.
// * The output is rescaled only when a tile's maximum score exceeds the
//   reference maximum by more than 8 in base-2 units (lazy rescaling);
//   otherwise the probabilities are taken against the old reference and stay
//   below 2^8.
// * Query tiles are dispatched heaviest first: blockIdx.z counts tiles back
//   from the end of each sequence, and the last tiles see the most keys.

#include <math.h>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBN = 64;   // keys per tile
constexpr int kPad = 8;   // bf16 elements of row padding in LDS

template <int D, int G>
struct PrefillShape {
  static constexpr int kRB = G >= 4 ? 1 : 4 / G;     // 32-row blocks per query head
  static constexpr int kWaves = G * kRB;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kBM = 32 * kRB;               // query positions per workgroup
  static constexpr int kSteps = D / 16;              // MFMA k-steps over head_dim
  static constexpr int kDB = D / 32;                 // 32-wide output blocks over head_dim
  static constexpr int kKChunks = kBN * D / 8;       // 16-byte chunks of a K tile
  static constexpr int kKPer = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVGroups = (kBN / 4) * (D / 8);  // (4 keys x 8 dims) groups of a V tile
  static constexpr int kVPer = (kVGroups + kThreads - 1) / kThreads;
  static constexpr int kKRow = D + kPad;             // LDS row of K (elements)
  static constexpr int kVRow = kBN + kPad;           // LDS row of V^T (elements)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// Position, within a group of 16 keys, at which key kk is stored in V^T so that
// lane half h reads, for slots 8h..8h+7, the keys the score accumulator holds.
__device__ __forceinline__ int vt_slot_of_quad(int quad) {  // first slot of keys 4q..4q+3
  return 8 * (quad & 1) + 4 * (quad >> 1);
}

template <int D, int G>
__global__ __launch_bounds__((PrefillShape<D, G>::kThreads), 2) void prefill_kernel(
    const uint16_t* __restrict__ q, int64_t q_tok_stride, int64_t q_head_stride,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    const int32_t* __restrict__ block_table, int64_t bt_stride, int32_t num_kv_heads,
    int32_t bs_log2, float scale_log2, uint16_t* __restrict__ out, int64_t out_tok_stride,
    int64_t out_head_stride) {
  using S = PrefillShape<D, G>;
  // Two K/V tile buffers: one is read by the MFMAs while the other is filled.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kBN * S::kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * S::kVRow];
  extern __shared__ int32_t bt_lds[];  // this sequence's block-table entries

  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int q_begin = cu_q[b];
  const int lq = cu_q[b + 1] - q_begin;
  const int lk = cu_k[b + 1] - cu_k[b];
  const int n_qt = (lq + S::kBM - 1) / S::kBM;
  const int qt = n_qt - 1 - static_cast<int>(blockIdx.z);  // heaviest tiles first
  if (qt < 0) return;
  const int ctx0 = lk - lq;                                 // cached positions
  const int wg_q0 = qt * S::kBM;                            // first query row of the tile
  const int wg_last_pos = ctx0 + min(lq, wg_q0 + S::kBM) - 1;
  const int n_kt = wg_last_pos / kBN + 1;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int half = lane / 32;
  const int col = lane % 32;
  const int head = g * G + wave / S::kRB;
  const int w_q0 = wg_q0 + (wave % S::kRB) * 32;            // first query row of the wave
  const int my_row = w_q0 + col;                            // this lane's query row
  const bool row_ok = my_row < lq;
  const int my_pos = ctx0 + my_row;                         // its position in the sequence
  const int w_last_pos = ctx0 + min(lq - 1, w_q0 + 31);     // last position the wave needs

  // Only keys 0..wg_last_pos are ever loaded (later keys of the last tile are in
  // every row's future and stay zero in LDS), so the entries of blocks
  // 0..wg_last_pos / block_size are all the tile needs.
  {  // the block-table entries the tile's keys use, staged once
    const int32_t* bt_row = block_table + static_cast<int64_t>(b) * bt_stride;
    const int n_bt = (wg_last_pos >> bs_log2) + 1;
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
  __syncthreads();  // bt_lds ready

  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * D;
  const int bs_mask = (1 << bs_log2) - 1;
  auto row_ptr = [&](const uint16_t* cache, int pos) {
    const int64_t blk = bt_lds[pos >> bs_log2];
    return cache + ((blk << bs_log2) + (pos & bs_mask)) * slot_stride + static_cast<int64_t>(g) * D;
  };

  uint4 kreg[S::kKPer];
  uint4 vreg[S::kVPer][4];
  auto fetch = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < S::kKPer; ++i) {
      const int c = tid + i * S::kThreads;
      const int key = c / (D / 8), chunk = c % (D / 8);
      const int pos = kt0 + key;
      kreg[i] = (c < S::kKChunks && pos <= wg_last_pos)
                    ? load16(row_ptr(k_cache, pos) + 8 * chunk)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < S::kVPer; ++i) {
      const int gi = tid + i * S::kThreads;
      const int quad = gi % (kBN / 4), chunk = gi / (kBN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = kt0 + 4 * quad + r;
        vreg[i][r] = (gi < S::kVGroups && pos <= wg_last_pos)
                         ? load16(row_ptr(v_cache, pos) + 8 * chunk)
                         : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < S::kKPer; ++i) {
      const int c = tid + i * S::kThreads;
      if (c < S::kKChunks) {
        const int key = c / (D / 8), chunk = c % (D / 8);
        *reinterpret_cast<uint4*>(&k_lds[buf][key * S::kKRow + 8 * chunk]) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < S::kVPer; ++i) {
      const int gi = tid + i * S::kThreads;
      if (gi < S::kVGroups) {
        const int quad = gi % (kBN / 4), chunk = gi / (kBN / 4);
        const int slot = 16 * (quad / 4) + vt_slot_of_quad(quad % 4);
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[i][0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[i][1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[i][2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[i][3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // dims 2j (low halves) and 2j+1 (high halves)
          const uint2 lo = make_uint2((w0[j] & 0xffffu) | (w1[j] << 16),
                                      (w2[j] & 0xffffu) | (w3[j] << 16));
          const uint2 hi = make_uint2((w0[j] >> 16) | (w1[j] & 0xffff0000u),
                                      (w2[j] >> 16) | (w3[j] & 0xffff0000u));
          const int dim = 8 * chunk + 2 * j;
          *reinterpret_cast<uint2*>(&vt_lds[buf][dim * S::kVRow + slot]) = lo;
          *reinterpret_cast<uint2*>(&vt_lds[buf][(dim + 1) * S::kVRow + slot]) = hi;
        }
      }
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

  fetch(0);
  stage(0);
  __syncthreads();
  if (n_kt > 1) fetch(kBN);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int kt0 = kt * kBN;
    const int buf = kt & 1;
    if (kt0 <= w_last_pos) {  // otherwise the whole tile lies in this wave's future
      f32x16_t acc_s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        acc_s[mb] = f32x16_t{};
        const uint16_t* kp = &k_lds[buf][(mb * 32 + col) * S::kKRow + 8 * half];
#pragma unroll
        for (int s = 0; s < S::kSteps; ++s)
          acc_s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(*reinterpret_cast<const uint4*>(kp + 16 * s)), qf[s], acc_s[mb], 0, 0,
              0);
      }

      // causal mask on tiles that reach past the wave's first position
      if (kt0 + kBN - 1 > ctx0 + w_q0) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + mb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
            if (key > my_pos) acc_s[mb][r] = -INFINITY;
          }
      }

      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, acc_s[mb][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)) * scale_log2;  // scale_log2 > 0
      if (__ballot(tmax > m_ref + kLazy)) {  // wave-uniform: raise the reference
        const float m_new = fmaxf(m_ref, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < S::kDB; ++db) acc_o[db] *= alpha;
      }

      // p = 2^(t - m_ref) as a bf16 head (truncated) plus a bf16 remainder
      float psum = 0.f;
      bf16x8_t pf_hi[4], pf_lo[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(acc_s[mb][r], scale_log2, -m_ref));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(acc_s[mb][r + 1], scale_log2, -m_ref));
          psum += p0 + p1;
          const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
          const float r0 = p0 - __uint_as_float(b0 & 0xffff0000u);
          const float r1 = p1 - __uint_as_float(b1 & 0xffff0000u);
          const uint32_t hi = (b0 >> 16) | (b1 & 0xffff0000u);
          const uint32_t lo = (__float_as_uint(r0) >> 16) | (__float_as_uint(r1) & 0xffff0000u);
          const int ks = 2 * mb + r / 8, e = r % 8;
          pf_hi[ks][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(hi));
          pf_hi[ks][e + 1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(hi >> 16));
          pf_lo[ks][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(lo));
          pf_lo[ks][e + 1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(lo >> 16));
        }
      l_run += psum;

#pragma unroll
      for (int db = 0; db < S::kDB; ++db) {
        const uint16_t* vp = &vt_lds[buf][(db * 32 + col) * S::kVRow + 8 * half];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8_t va = as_bf16x8(*reinterpret_cast<const uint4*>(vp + 16 * ks));
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf_hi[ks], acc_o[db], 0, 0, 0);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf_lo[ks], acc_o[db], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < n_kt) stage(buf ^ 1);  // the other buffer was last read one tile ago
    __syncthreads();
    if (kt + 2 < n_kt) fetch(kt0 + 2 * kBN);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (!row_ok) return;
  const float inv = 1.f / l_tot;
  uint16_t* op = out + static_cast<int64_t>(q_begin + my_row) * out_tok_stride +
                 static_cast<int64_t>(head) * out_head_stride;
#pragma unroll
  for (int db = 0; db < S::kDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dim = db * 32 + 8 * r4 + 4 * half;
      const uint32_t lo = f32_to_bf16_rne(acc_o[db][4 * r4 + 0] * inv) |
                          (static_cast<uint32_t>(f32_to_bf16_rne(acc_o[db][4 * r4 + 1] * inv)) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc_o[db][4 * r4 + 2] * inv) |
                          (static_cast<uint32_t>(f32_to_bf16_rne(acc_o[db][4 * r4 + 3] * inv)) << 16);
      *reinterpret_cast<uint2*>(op + dim) = make_uint2(lo, hi);
    }
}

template <int D, int G>
hipError_t run(const PrefillArgs& a, hipStream_t stream) {
  using S = PrefillShape<D, G>;
  const int bs_log2 = __builtin_ctz(static_cast<unsigned>(a.block_size));
  const int tiles = (a.max_seqlen_q + S::kBM - 1) / S::kBM;
  const size_t bt_bytes = static_cast<size_t>((a.max_seqlen_k + a.block_size - 1) >> bs_log2) * 4;
  dim3 grid(a.num_kv_heads, a.num_seqs, tiles);
  hipLaunchKernelGGL((prefill_kernel<D, G>), grid, dim3(S::kThreads), bt_bytes, stream,
                     static_cast<const uint16_t*>(a.q), a.q_tok_stride, a.q_head_stride,
                     static_cast<const uint16_t*>(a.k_cache), static_cast<const uint16_t*>(a.v_cache),
                     a.cu_seqlens_q, a.cu_seqlens_k, a.block_table, a.block_table_stride,
                     a.num_kv_heads, bs_log2, a.scale * kLog2e, static_cast<uint16_t*>(a.out),
                     a.out_tok_stride, a.out_head_stride);
  return hipGetLastError();
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
