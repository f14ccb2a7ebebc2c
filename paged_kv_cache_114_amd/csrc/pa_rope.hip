// Per-head q/k RMSNorm, rotary position embedding, and the paged store of the
// rotated K and the untouched V -- the step that produces what the attention
// kernels read.
//
// What is computed ("大模型推理入门与 nano-vLLM 源码详解" §12.2, §19.3, §19.7;
// "nano-vllm 技术分析" §4.2, §4.4; the fused kernel of "Pico-vLLM 开发日志 #8"
// §1): a token's projection row holds Hq query heads, then Hkv key heads, then
// Hkv value heads.  Each Q and K head is normalised over its own features,
// y = gamma * x / sqrt(mean(x^2) + eps), with separate gammas for Q and K (or
// not at all when no gammas are given), and then rotated: feature i pairs with
// feature i + d/2 and the pair turns by p * theta^(-2i/d) radians at the
// token's position p.  Q goes to q_out; K and V go to the token's cache slot.
//
// Layout of the work: a head is spread over d/16 lanes, each holding 8
// features of the first half and the 8 partner features of the second half,
// so every rotation pair sits in one lane and a head's sum of squares is a
// reduction over d/16 neighbouring lanes (DPP moves).  A wave covers 1024/d
// heads per pass (8 for d = 128); Qwen3-0.6B's 32 head slots (16 Q, 8 K, 8 V)
// are four passes.  A wave takes one pass of one token at a time, so even a
// decode batch of a few tokens spreads over many waves; it issues the pass's
// loads, then computes the token's d/2 rotation angles (one per lane, shared
// through LDS) while they are in flight.  Measured against waves that take
// all four passes of a token (and compute its angles once), one pass per wave
// was as fast or faster at every batch size tried (64 to 16384 tokens).
//
// Precision: the pair frequencies are fp64 powers of theta^(-2/d) (computed
// once on the host), the angle p * omega and its reduction to [-pi, pi] are
// fp64, its sine and cosine fp32; norm and rotation run in fp32 and the
// result is rounded once to the storage type.  The pages' implementations
// look up a table of fp32 angles instead; the definition does not round the
// angle, and neither does this.

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kRopeWaves = 4;       // waves per workgroup
constexpr int kHalfElems = 8;       // features per lane in each half of a head
constexpr double kTwoPi = 6.283185307179586;
constexpr double kInvTwoPi = 0.15915494309189535;

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 8 consecutive features held by one lane: one 16-byte word for bf16, two for fp32.
template <typename T>
struct Eight;
template <>
struct Eight<bf16_t> {
  static constexpr int kWords = 1;
  __device__ __forceinline__ static void widen(const uint4* w, float* f) {
    Chunk<bf16_t>::widen(w[0], f);
  }
  __device__ __forceinline__ static void narrow(const float* f, uint4* w) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = __builtin_bit_cast(uint32_t,
                                __builtin_convertvector(f32x2_t{f[2 * i], f[2 * i + 1]}, bf16x2_t));
    w[0] = uint4{u[0], u[1], u[2], u[3]};
  }
};
template <>
struct Eight<float> {
  static constexpr int kWords = 2;
  __device__ __forceinline__ static void widen(const uint4* w, float* f) {
    Chunk<float>::widen(w[0], f);
    Chunk<float>::widen(w[1], f + 4);
  }
  __device__ __forceinline__ static void narrow(const float* f, uint4* w) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      w[i] = uint4{__float_as_uint(f[4 * i]), __float_as_uint(f[4 * i + 1]),
                   __float_as_uint(f[4 * i + 2]), __float_as_uint(f[4 * i + 3])};
  }
};

// A work item is one pass of one token; every item of the token computes the
// token's angles (cheap next to the item's loads).
template <typename T, int D>
__global__ __launch_bounds__(kRopeWaves* kWave) void norm_rope_store_kernel(
    const char* qkv, int64_t qkv_tok_b, const char* __restrict__ q_weight,
    const char* __restrict__ k_weight, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ slot_mapping, int32_t num_items, int32_t passes,
    int32_t num_q_heads, int32_t num_kv_heads, float eps, double freq_ratio, char* q_out,
    int64_t q_out_tok_b, char* k_cache, char* v_cache, int32_t bs_log2, int64_t block_b,
    int64_t slot_b, int64_t cache_head_b) {
  using E = Eight<T>;
  constexpr int kEb = Elt<T>::kBytes;
  constexpr int kPairs = D / 2;
  constexpr int kLanesPerHead = D / (2 * kHalfElems);  // 8 for d = 128
  constexpr int kHeadsPerPass = kWave / kLanesPerHead;
  constexpr int kHeadBytes = D * kEb;
  static_assert(kPairs <= kWave, "one angle per lane");

  __shared__ f32x2_t angle_lds[kRopeWaves][kPairs];

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int part = lane % kLanesPerHead;      // which 8-feature slice of the halves
  const int head_in_pass = lane / kLanesPerHead;
  const int lo_b = part * kHalfElems * kEb;   // byte offset of the slice in a head
  const int hi_b = lo_b + kPairs * kEb;       // ...and of its partners
  const int total_heads = num_q_heads + 2 * num_kv_heads;
  const bool use_norm = q_weight != nullptr;

  // Per-lane constants: the raw norm weights of the lane's 16 features, and
  // the frequency of the pair whose angle this lane computes,
  // omega_j = theta^(-2j/d) = freq_ratio^j, by binary powering in fp64.
  uint4 gq[2][E::kWords], gk[2][E::kWords];
  if (use_norm) {
#pragma unroll
    for (int i = 0; i < E::kWords; ++i) {
      gq[0][i] = load16(q_weight + lo_b + 16 * i);
      gq[1][i] = load16(q_weight + hi_b + 16 * i);
      gk[0][i] = load16(k_weight + lo_b + 16 * i);
      gk[1][i] = load16(k_weight + hi_b + 16 * i);
    }
  }
  double omega = 1.0;
  {
    double f = freq_ratio;
    for (int e = lane % kPairs; e != 0; e >>= 1) {
      if (e & 1) omega *= f;
      f *= f;
    }
  }

  for (int item = blockIdx.x * kRopeWaves + wave; item < num_items;
       item += gridDim.x * kRopeWaves) {
    const int tok = item / passes;
    const int hs = (item - tok * passes) * kHeadsPerPass + head_in_pass;  // this lane's head slot
    const int32_t pos = positions[tok];
    const int32_t slot = slot_mapping[tok];

    // The loads go out first.  A lane whose head slot is past the row re-reads
    // the last head and stores nothing.
    uint4 lo[E::kWords], hi[E::kWords];
    {
      const char* src = qkv + tok * qkv_tok_b + min(hs, total_heads - 1) * kHeadBytes;
#pragma unroll
      for (int i = 0; i < E::kWords; ++i) {
        lo[i] = load16(src + lo_b + 16 * i);
        hi[i] = load16(src + hi_b + 16 * i);
      }
    }

    // The token's angles: lane j < d/2 turns pair j by pos * omega_j, reduced
    // to [-pi, pi] in fp64 before the fp32 sine and cosine.
    if (lane < kPairs) {
      const double phi = static_cast<double>(pos) * omega;
      const double turns = rint(phi * kInvTwoPi);
      const float r = static_cast<float>(fma(-turns, kTwoPi, phi));
      float s, c;
      sincosf(r, &s, &c);
      angle_lds[wave][lane] = f32x2_t{c, s};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float cs[kHalfElems], sn[kHalfElems];
#pragma unroll
    for (int j = 0; j < kHalfElems; ++j) {
      const f32x2_t a = angle_lds[wave][part * kHalfElems + j];
      cs[j] = a.x;
      sn[j] = a.y;
    }

    {
      const bool is_q = hs < num_q_heads;
      const bool is_v = hs >= num_q_heads + num_kv_heads;
      float a[kHalfElems], b[kHalfElems];
      E::widen(lo, a);
      E::widen(hi, b);
      if (!is_v) {  // uniform over a head's lanes, so the reduction sees only its head
        if (use_norm) {
          float ss = 0.f;
#pragma unroll
          for (int j = 0; j < kHalfElems; ++j) ss = fmaf(a[j], a[j], fmaf(b[j], b[j], ss));
          ss = group_sum<kLanesPerHead>(ss);
          const float inv_rms = rsqrtf(ss * (1.0f / D) + eps);
          uint4 wa[E::kWords], wb[E::kWords];
#pragma unroll
          for (int i = 0; i < E::kWords; ++i) {
            wa[i] = is_q ? gq[0][i] : gk[0][i];
            wb[i] = is_q ? gq[1][i] : gk[1][i];
          }
          float ga[kHalfElems], gb[kHalfElems];
          E::widen(wa, ga);
          E::widen(wb, gb);
#pragma unroll
          for (int j = 0; j < kHalfElems; ++j) {
            a[j] *= inv_rms * ga[j];
            b[j] *= inv_rms * gb[j];
          }
        }
#pragma unroll
        for (int j = 0; j < kHalfElems; ++j) {
          const float ra = fmaf(a[j], cs[j], -b[j] * sn[j]);
          const float rb = fmaf(a[j], sn[j], b[j] * cs[j]);
          a[j] = ra;
          b[j] = rb;
        }
      }
      // past the row, or a padding row's K and V: nothing to store
      const bool store = hs < total_heads && (is_q || slot >= 0);
      char* dst;
      if (is_q) {
        dst = q_out + tok * q_out_tok_b + static_cast<int64_t>(hs) * kHeadBytes;
      } else {
        const int kv = is_v ? hs - num_q_heads - num_kv_heads : hs - num_q_heads;
        dst = (is_v ? v_cache : k_cache) + (slot >> bs_log2) * block_b +
              (slot & ((1 << bs_log2) - 1)) * slot_b + kv * cache_head_b;
      }
      uint4 oa[E::kWords], ob[E::kWords];
      if (is_v) {  // V is copied bit for bit
#pragma unroll
        for (int i = 0; i < E::kWords; ++i) {
          oa[i] = lo[i];
          ob[i] = hi[i];
        }
      } else {
        E::narrow(a, oa);
        E::narrow(b, ob);
      }
      if (store) {
#pragma unroll
        for (int i = 0; i < E::kWords; ++i) {
          *reinterpret_cast<uint4*>(dst + lo_b + 16 * i) = oa[i];
          *reinterpret_cast<uint4*>(dst + hi_b + 16 * i) = ob[i];
        }
      }
    }
    // the next item rewrites this wave's angles only after they were read
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

template <typename T, int D>
hipError_t run(const RopeArgs& a, hipStream_t stream) {
  const int64_t eb = Elt<T>::kBytes;
  const int heads_per_pass = kWave / (D / (2 * kHalfElems));
  const int passes = (a.num_q_heads + 2 * a.num_kv_heads + heads_per_pass - 1) / heads_per_pass;
  const int64_t items = int64_t{a.num_tokens} * passes;
  if (items >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const int64_t want = (items + kRopeWaves - 1) / kRopeWaves;
  const int blocks = static_cast<int>(want < 16384 ? want : 16384);
  // theta^(-2/d): the ratio of successive pair frequencies
  const double freq_ratio = pow(a.theta, -2.0 / a.head_dim);
  hipLaunchKernelGGL((norm_rope_store_kernel<T, D>), dim3(blocks), dim3(kRopeWaves * kWave), 0,
                     stream, static_cast<const char*>(a.qkv), a.qkv_tok_stride * eb,
                     static_cast<const char*>(a.q_weight), static_cast<const char*>(a.k_weight),
                     a.positions, a.slot_mapping, static_cast<int32_t>(items), passes,
                     a.num_q_heads, a.num_kv_heads, a.eps, freq_ratio,
                     static_cast<char*>(a.q_out), a.q_out_tok_stride * eb,
                     static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache),
                     __builtin_ctz(static_cast<unsigned>(a.block_size)), a.geom.block * eb,
                     a.geom.slot * eb, a.geom.head * eb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_rope_store(const RopeArgs& a, hipStream_t stream) {
  if (a.elt_bytes == 2)
    return a.head_dim == 128 ? run<bf16_t, 128>(a, stream) : run<bf16_t, 64>(a, stream);
  return a.head_dim == 128 ? run<float, 128>(a, stream) : run<float, 64>(a, stream);
}

}  // namespace pa
