// KV store through slot_mapping (the row copy itself is in pa_store_rows.h).
//
// [Intro §13.1] ("大模型推理入门与 nano-vLLM 源码详解"): each new token's K and V
// rows for all kv heads are copied into slot slot_mapping[i] of this layer's
// cache; a slot of -1 is a padding row and is skipped.  The source may be a
// strided view (token and head strides), the point of [Pico #6, pitfall 1].

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_store_rows.h"

namespace pa {
namespace {

constexpr int kStoreWaves = 4;  // waves per workgroup

template <typename W>
__global__ __launch_bounds__(kStoreWaves* kWave) void store_kernel(StoreRows a) {
  store_rows<W>(a, blockIdx.x * kStoreWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave),
                gridDim.x * kStoreWaves);
}

// The row-copy description of a store (false: a shape the copy cannot take).
template <typename W>
bool store_rows_args(const StoreArgs& a, StoreRows* r) {
  const int64_t eb = a.elt_bytes;
  const int words_per_head = static_cast<int>(a.head_dim * eb / sizeof(W));
  const int hw_log2 = __builtin_ctz(static_cast<unsigned>(words_per_head));
  if ((1 << hw_log2) != words_per_head) return false;
  const int64_t rows = int64_t{a.num_tokens} * 2;
  if (rows >= (int64_t{1} << 31)) return false;
  *r = StoreRows{static_cast<const char*>(a.k), static_cast<const char*>(a.v),
                 a.k_tok_stride * eb, a.k_head_stride * eb, a.v_tok_stride * eb,
                 a.v_head_stride * eb, static_cast<char*>(a.k_cache),
                 static_cast<char*>(a.v_cache), a.slot_mapping, static_cast<int32_t>(rows),
                 a.num_kv_heads * words_per_head, hw_log2,
                 __builtin_ctz(static_cast<unsigned>(a.block_size)), a.geom.block * eb,
                 a.geom.slot * eb, a.geom.head * eb};
  return true;
}

template <typename W>
hipError_t run(const StoreArgs& a, hipStream_t stream) {
  StoreRows r;
  if (!store_rows_args<W>(a, &r)) return hipErrorInvalidValue;
  const int64_t want = (int64_t{r.rows} + kStoreWaves - 1) / kStoreWaves;
  const int blocks = static_cast<int>(want < 16384 ? (want > 0 ? want : 1) : 16384);
  hipLaunchKernelGGL(store_kernel<W>, dim3(blocks), dim3(kStoreWaves * kWave), 0, stream, r);
  return hipGetLastError();
}

bool aligned(const void* p, int64_t a, int64_t b, int64_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0 && (a % n) == 0 && (b % n) == 0;
}

}  // namespace

bool store_rows_16(const StoreArgs& a, StoreRows* r) {
  const int64_t eb = a.elt_bytes;
  return aligned(a.k, a.k_tok_stride * eb, a.k_head_stride * eb, 16) &&
         aligned(a.v, a.v_tok_stride * eb, a.v_head_stride * eb, 16) &&
         reinterpret_cast<uintptr_t>(a.k_cache) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(a.v_cache) % 16 == 0 && store_rows_args<uint4>(a, r);
}

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
