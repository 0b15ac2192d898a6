// Device-side helpers shared by the gfx950 kernels (bf16 conversions, dot
// products, wave reductions, device-coherent loads/stores, greedy keys).
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace qt {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kInvSqrtHd = 0.08838834764831845f;  // 1/sqrt(128)

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// x ~ hi + lo with both parts bfloat16 (x - hi is exact in fp32).
__device__ __forceinline__ void split_bf16(float x, uint16_t* hi, uint16_t* lo, size_t i) {
  const uint16_t h = f2bf(x);
  hi[i] = h;
  lo[i] = f2bf(x - bf2f(h));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot8(const uint4& w, const uint4& x, float c) {
  c = dot2(w.x, x.x, c);
  c = dot2(w.y, x.y, c);
  c = dot2(w.z, x.z, c);
  return dot2(w.w, x.w, c);
}

// Two signed int8 (bytes 2i, 2i+1 of word) -> packed bf16 pair.  |q| <= 127 is
// exact in bfloat16, so taking the high half of the float is exact.
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t word, int i) {
  const float lo = (float)(int)(int8_t)(word >> (16 * i));
  const float hi = (float)(int)(int8_t)(word >> (16 * i + 8));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// Greedy key: order-preserving float bits in the high word, (~index) in the low
// word, so a 64-bit max picks the largest value and, among equal values, the
// lowest index.  -0 is folded onto +0 so that the two compare equal.
__device__ __forceinline__ unsigned long long greedy_key(float v, int idx) {
  v += 0.0f;
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - (uint32_t)idx);
}
__device__ __forceinline__ int key_index(unsigned long long k) {
  return (int)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

template <int V>
struct Log2 {
  static constexpr int value = 1 + Log2<V / 2>::value;
};
template <>
struct Log2<1> {
  static constexpr int value = 0;
};

// Sum V values held by every lane over the 64 lanes of the wave.  After the
// call, lane l holds the total of value index (l >> (6 - log2 V)).  Halving
// exchange: each step sends half of the remaining values to the partner lane.
template <int V>
__device__ __forceinline__ float transpose_reduce(float (&v)[V], int lane) {
  constexpr int P = Log2<V>::value;
#pragma unroll
  for (int s = 0; s < P; ++s) {
    const int h = (V >> s) >> 1;
    const int o = 32 >> s;
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = up ? v[i] : v[i + h];
      const float keep = up ? v[i + h] : v[i];
      v[i] = keep + __shfl_xor(send, o);
    }
  }
  float r = v[0];
#pragma unroll
  for (int o = 32 >> P; o >= 1; o >>= 1) r += __shfl_xor(r, o);
  return r;
}

// Device-coherent (agent-scope) store / load: performed at the point where all
// XCDs see the same data, without cache-wide writeback or invalidation.
__device__ __forceinline__ void dev_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float dev_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

}  // namespace dev
}  // namespace qt
