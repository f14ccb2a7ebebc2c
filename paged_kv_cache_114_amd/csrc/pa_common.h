// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;

// log2(e): scores are carried in base-2 units so the softmax uses exp2.
constexpr float kLog2e = 1.4426950408889634f;

// bf16 storage is the upper 16 bits of an IEEE binary32.
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kBytes = 4;
};
template <>
struct Elt<bf16_t> {
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
// Two values at once (lo in the low half): one v_cvt_pk_bf16_f32.  Its bits
// equal the integer rounding (add 0x7fff plus the kept lsb, NaN quieted by
// setting bit 6) on every class of input -- ties, near-ties, denormals,
// infinities, values that round to infinity, NaN payloads -- checked on the
// GPU; the integer form, written out, cost ~10 instructions a value with its
// NaN branch.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return static_cast<uint16_t>(f32x2_to_bf16x2_rne(f, 0.f));
}

// Widen the 16 bytes one lane holds into fp32 values.
template <typename T>
struct Chunk;
template <>
struct Chunk<bf16_t> {
  static constexpr int kElems = 8;
  __device__ __forceinline__ static void widen(const uint4& w, float* f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  }
};
template <>
struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void widen(const uint4& w, float* f) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
};

// DPP lane moves (gfx9 encodings).  Bound control on, all rows and banks on.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, true));
}
constexpr int kDppQuadXor1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of kLanes lanes (kLanes in {1,2,4,8,16,32,64}); every
// lane of a group ends with the group's sum.
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (kLanes >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (kLanes >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (kLanes >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (kLanes >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (kLanes >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (kLanes >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

// The value of lane i ^ 32: one v_permlane32_swap (the two halves of a copy
// traded) and a select, instead of a round trip through the LDS unit.
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// Max across lanes that differ only in the lane bits from kFrom up to the wave.
template <int kFrom>
__device__ __forceinline__ float across_groups_max(float x) {
#pragma unroll
  for (int m = kFrom; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
  return x;
}
template <int kFrom>
__device__ __forceinline__ float across_groups_sum(float x) {
#pragma unroll
  for (int m = kFrom; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace pa
