// KV store through slot_mapping.
//
// [Intro §13.1] ("大模型推理入门与 nano-vLLM 源码详解"): each new token's K and V
// rows for all kv heads are copied into slot slot_mapping[i] of this layer's
// cache; a slot of -1 is a padding row and is skipped.  The source may be a
// strided view (token and head strides), the point of [Pico #6, pitfall 1].
//
// One wave moves one (token, K or V) row: num_kv_heads * head_dim elements,
// read as W-sized words and written to the slot's head rows (adjacent in the
// slots-then-heads layout, block_size rows apart in the heads-then-slots
// one).  The slot is loaded once per row and is uniform over the wave (a
// padding row is skipped whole).  Lane l takes words l, l + 64,
// ...; each lane issues all of its loads before its first store, so a wave
// keeps the whole row in flight.  A word's head is word >> hw_log2
// (head_dim * element size / sizeof(W) is a power of two).

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kStoreWaves = 4;  // waves per workgroup
constexpr int kStoreUnroll = 2; // words per lane whose loads are issued together
                                // (a Qwen3 row of 8 heads x 128 bf16 is 2 per lane)

template <typename W>
__global__ __launch_bounds__(kStoreWaves* kWave) void store_kernel(
    const char* __restrict__ k, const char* __restrict__ v, int64_t k_tok_b, int64_t k_head_b,
    int64_t v_tok_b, int64_t v_head_b, char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int32_t rows, int32_t words_per_row,
    int32_t hw_log2, int32_t bs_log2, int64_t block_b, int64_t slot_b, int64_t cache_head_b) {
  const int lane = threadIdx.x % kWave;
  const int hw_mask = (1 << hw_log2) - 1;
  const int bs_mask = (1 << bs_log2) - 1;
  for (int r = blockIdx.x * kStoreWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
       r < rows; r += gridDim.x * kStoreWaves) {
    const int tok = r >> 1;
    const bool is_v = r & 1;
    const int32_t slot = slot_mapping[tok];
    if (slot < 0) continue;  // -1: padding row, nothing to write
    const char* src = is_v ? v + tok * v_tok_b : k + tok * k_tok_b;
    const int64_t head_b = is_v ? v_head_b : k_head_b;
    char* dst =
        (is_v ? v_cache : k_cache) + (slot >> bs_log2) * block_b + (slot & bs_mask) * slot_b;
    for (int w0 = 0; w0 < words_per_row; w0 += kStoreUnroll * kWave) {
      // No lane branches: a lane past the row re-reads its last word and writes
      // the same value back, so the loads issue back to back and the wave waits
      // once before its stores.
      W val[kStoreUnroll];
#pragma unroll
      for (int u = 0; u < kStoreUnroll; ++u) {
        const int w = min(w0 + u * kWave + lane, words_per_row - 1);
        val[u] = *reinterpret_cast<const W*>(src + (w >> hw_log2) * head_b +
                                             (w & hw_mask) * static_cast<int64_t>(sizeof(W)));
      }
#pragma unroll
      for (int u = 0; u < kStoreUnroll; ++u) {
        const int w = min(w0 + u * kWave + lane, words_per_row - 1);
        *reinterpret_cast<W*>(dst + (w >> hw_log2) * cache_head_b +
                              (w & hw_mask) * static_cast<int64_t>(sizeof(W))) = val[u];
      }
    }
  }
}

template <typename W>
hipError_t run(const StoreArgs& a, hipStream_t stream) {
  const int64_t eb = a.elt_bytes;
  const int words_per_head = static_cast<int>(a.head_dim * eb / sizeof(W));
  const int hw_log2 = __builtin_ctz(static_cast<unsigned>(words_per_head));
  if ((1 << hw_log2) != words_per_head) return hipErrorInvalidValue;
  const int words_per_row = a.num_kv_heads * words_per_head;
  const int64_t rows = int64_t{a.num_tokens} * 2;
  if (rows >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const int64_t want = (rows + kStoreWaves - 1) / kStoreWaves;
  const int blocks = static_cast<int>(want < 16384 ? (want > 0 ? want : 1) : 16384);
  hipLaunchKernelGGL(store_kernel<W>, dim3(blocks), dim3(kStoreWaves * kWave), 0, stream,
                     static_cast<const char*>(a.k), static_cast<const char*>(a.v),
                     a.k_tok_stride * eb, a.k_head_stride * eb, a.v_tok_stride * eb,
                     a.v_head_stride * eb, static_cast<char*>(a.k_cache),
                     static_cast<char*>(a.v_cache), a.slot_mapping, static_cast<int32_t>(rows),
                     words_per_row, hw_log2, __builtin_ctz(static_cast<unsigned>(a.block_size)),
                     a.geom.block * eb, a.geom.slot * eb, a.geom.head * eb);
  return hipGetLastError();
}

bool aligned(const void* p, int64_t a, int64_t b, int64_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0 && (a % n) == 0 && (b % n) == 0;
}

}  // namespace

hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  const int64_t eb = a.elt_bytes;
  const int64_t kt = a.k_tok_stride * eb, kh = a.k_head_stride * eb;
  const int64_t vt = a.v_tok_stride * eb, vh = a.v_head_stride * eb;
  // The cache rows are always 16-byte aligned (head_dim * elt is 128 or more bytes
  // and the cache base comes from the allocator); only the sources can force
  // narrower words.
  if (aligned(a.k, kt, kh, 16) && aligned(a.v, vt, vh, 16) &&
      reinterpret_cast<uintptr_t>(a.k_cache) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(a.v_cache) % 16 == 0)
    return run<uint4>(a, stream);
  if (aligned(a.k, kt, kh, 4) && aligned(a.v, vt, vh, 4) &&
      reinterpret_cast<uintptr_t>(a.k_cache) % 4 == 0 &&
      reinterpret_cast<uintptr_t>(a.v_cache) % 4 == 0)
    return run<uint32_t>(a, stream);
  return run<uint16_t>(a, stream);
}

}  // namespace pa
