// The KV store's row copy (the body of the store kernel).
//
// [Intro §13.1] ("大模型推理入门与 nano-vLLM 源码详解"): each new token's K and V
// rows for all kv heads are copied into slot slot_mapping[i] of this layer's
// cache; a slot of -1 is a padding row and is skipped.
//
// One wave moves one (token, K or V) row: num_kv_heads * head_dim elements,
// read as W-sized words and written to the slot's head rows (adjacent in the
// slots-then-heads layout, block_size rows apart in the heads-then-slots
// one).  The slot is loaded once per row and is uniform over the wave (a
// padding row is skipped whole).  Lane l takes words l, l + 64, ...; each
// lane issues all of its loads before its first store, so a wave keeps the
// whole row in flight.  A word's head is word >> hw_log2 (head_dim * element
// size / sizeof(W) is a power of two).
#pragma once

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kStoreUnroll = 2;  // words per lane whose loads are issued together
                                 // (a Qwen3 row of 8 heads x 128 bf16 is 2 per lane)
                                 // -- the copy below is written for exactly 2

struct StoreRows {
  const char* k;
  const char* v;
  int64_t k_tok_b, k_head_b, v_tok_b, v_head_b;  // source strides, bytes
  char* k_cache;
  char* v_cache;
  const int32_t* slot_mapping;
  int32_t rows;           // 2 * tokens: row r is token r / 2, K (even) or V (odd)
  int32_t words_per_row;
  int32_t hw_log2;        // log2(words per head)
  int32_t bs_log2;
  int64_t block_b, slot_b, cache_head_b;  // cache strides, bytes
};

// The row-copy description of a store in 16-byte words (false: a shape or an
// alignment the copy cannot take that way).
bool store_rows_16(const StoreArgs& a, StoreRows* r);

// Rows first_row, first_row + row_step, ... of the store, one per wave.
template <typename W>
__device__ __forceinline__ void store_rows(const StoreRows& a, int first_row, int row_step) {
  const int lane = threadIdx.x % kWave;
  const int hw_mask = (1 << a.hw_log2) - 1;
  const int bs_mask = (1 << a.bs_log2) - 1;
  for (int r = first_row; r < a.rows; r += row_step) {
    const int tok = r >> 1;
    const bool is_v = r & 1;
    const int32_t slot = a.slot_mapping[tok];
    if (slot < 0) continue;  // -1: padding row, nothing to write
    const char* src = is_v ? a.v + tok * a.v_tok_b : a.k + tok * a.k_tok_b;
    const int64_t head_b = is_v ? a.v_head_b : a.k_head_b;
    char* dst = (is_v ? a.v_cache : a.k_cache) + (slot >> a.bs_log2) * a.block_b +
                (slot & bs_mask) * a.slot_b;
    auto word = [&](int w) { return min(w, a.words_per_row - 1); };
    auto src_at = [&](int w) {
      return reinterpret_cast<const W*>(src + (w >> a.hw_log2) * head_b +
                                        (w & hw_mask) * static_cast<int64_t>(sizeof(W)));
    };
    auto dst_at = [&](int w) {
      return reinterpret_cast<W*>(dst + (w >> a.hw_log2) * a.cache_head_b +
                                  (w & hw_mask) * static_cast<int64_t>(sizeof(W)));
    };
    for (int w0 = 0; w0 < a.words_per_row; w0 += kStoreUnroll * kWave) {
      // No lane branches: a lane past the row re-reads its last word and writes
      // the same value back, so the loads issue back to back and the wave waits
      // once before its stores.  (Two named words, not an array: inside a large
      // kernel an array here has been left in scratch memory.)
      const int wa = word(w0 + lane), wb = word(w0 + kWave + lane);
      const W va = *src_at(wa);
      const W vb = *src_at(wb);
      *dst_at(wa) = va;
      *dst_at(wb) = vb;
    }
  }
}

}  // namespace pa
