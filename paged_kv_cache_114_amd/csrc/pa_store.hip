// KV store through slot_mapping.
//
// [Intro §13.1] ("大模型推理入门与 nano-vLLM 源码详解"): each new token's K and V
// rows for all kv heads are copied into slot slot_mapping[i] of this layer's
// cache; a slot of -1 is a padding row and is skipped.  The source may be a
// strided view (token and head strides), the point of [Pico #6, pitfall 1].
//
// Work is flattened over (token, K|V, head, word) so consecutive lanes move
// consecutive 16-byte words of one head row: every wave reads and writes whole
// contiguous segments, which is all an HBM-bound copy needs.

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

template <typename W>
__global__ __launch_bounds__(256) void store_kernel(
    const char* __restrict__ k, const char* __restrict__ v, int64_t k_tok_b, int64_t k_head_b,
    int64_t v_tok_b, int64_t v_head_b, char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, uint32_t total, uint32_t per_tensor,
    uint32_t words_per_head, int64_t row_bytes, int64_t head_bytes) {
  // total = tokens * 2 * per_tensor < 2^31 (checked on the host)
  for (uint32_t item = blockIdx.x * blockDim.x + threadIdx.x; item < total;
       item += gridDim.x * blockDim.x) {
    const uint32_t tok = item / (2 * per_tensor);
    const uint32_t rem = item - tok * 2 * per_tensor;
    const bool is_v = rem >= per_tensor;
    const uint32_t c = is_v ? rem - per_tensor : rem;
    const uint32_t head = c / words_per_head;
    const uint32_t word = c - head * words_per_head;
    const int32_t slot = slot_mapping[tok];
    if (slot < 0) continue;  // -1: padding row, nothing to write
    const char* src = is_v ? v + tok * v_tok_b + head * v_head_b : k + tok * k_tok_b + head * k_head_b;
    char* dst = (is_v ? v_cache : k_cache) + static_cast<int64_t>(slot) * row_bytes + head * head_bytes;
    reinterpret_cast<W*>(dst)[word] = reinterpret_cast<const W*>(src)[word];
  }
}

template <typename W>
hipError_t run(const StoreArgs& a, hipStream_t stream) {
  const int64_t eb = a.elt_bytes;
  const uint32_t words_per_head = static_cast<uint32_t>(a.head_dim * eb / sizeof(W));
  const uint32_t per_tensor = static_cast<uint32_t>(a.num_kv_heads) * words_per_head;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * 2 * per_tensor;
  if (total >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const int64_t want = (total + 255) / 256;
  const int blocks = static_cast<int>(want < 16384 ? (want > 0 ? want : 1) : 16384);
  hipLaunchKernelGGL(store_kernel<W>, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const char*>(a.k), static_cast<const char*>(a.v),
                     a.k_tok_stride * eb, a.k_head_stride * eb, a.v_tok_stride * eb,
                     a.v_head_stride * eb, static_cast<char*>(a.k_cache),
                     static_cast<char*>(a.v_cache), a.slot_mapping, static_cast<uint32_t>(total),
                     per_tensor, words_per_head, static_cast<int64_t>(a.num_kv_heads) * a.head_dim * eb,
                     static_cast<int64_t>(a.head_dim) * eb);
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
