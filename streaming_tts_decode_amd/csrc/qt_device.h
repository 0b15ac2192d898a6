// Device-side helpers shared by the gfx950 kernels (bf16 / fp16 conversions, dot
// products, wave reductions, device-coherent loads/stores, greedy keys).
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace qt {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// float <-> IEEE half bits (round to nearest even; out of range -> inf).
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Half of v that also notes in `over` a finite v that half cannot hold (|v| >= 65520
// rounds to infinity).  Producers of GEMM inputs write half(x * gain) of residual rows
// before the RMS factor is applied, so a large residual would otherwise become inf
// without a trace; the caller ORs QT_STATUS_FP16_RANGE into the status word.
__device__ __forceinline__ uint16_t f2h_chk(float v, bool& over) {
  const uint16_t h = f2h(v);
  over = over || (((h & 0x7fffu) == 0x7c00u) && !(fabsf(v) == INFINITY));
  return h;
}

// fp16 dot products with fp32 accumulation (v_dot2_f32_f16).
__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}
__device__ __forceinline__ float dot8h(const uint4& w, const uint4& x, float c) {
  c = dot2h(w.x, x.x, c);
  c = dot2h(w.y, x.y, c);
  c = dot2h(w.z, x.z, c);
  return dot2h(w.w, x.w, c);
}

// Two signed int8 (bytes 2i, 2i+1 of word) -> packed fp16 pair (exact: integers
// up to 2048 are exact in fp16, so rounding toward zero changes nothing).
__device__ __forceinline__ uint32_t i8pair_to_f16x2(uint32_t word, int i) {
  const float lo = (float)(int)(int8_t)(word >> (16 * i));
  const float hi = (float)(int)(int8_t)(word >> (16 * i + 8));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
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

// ---- cross-lane reductions (every participating lane must be active)
// DPP row steps within 16-lane rows: quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.  After the four steps every lane of a row holds the
// row's total, with the same bits in every lane (each step adds a lane's value to
// its mirror's, a commutative pair).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return v;
}
template <int CTRL>
__device__ __forceinline__ void max_u64_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t oh = dpp_u32<CTRL>(hi), ol = dpp_u32<CTRL>(lo);
  const bool take = oh > hi || (oh == hi && ol > lo);
  hi = take ? oh : hi;
  lo = take ? ol : lo;
}
__device__ __forceinline__ unsigned long long row_max16_u64(unsigned long long k) {
  uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  max_u64_step<kDppXor1>(hi, lo);
  max_u64_step<kDppXor2>(hi, lo);
  max_u64_step<kDppHalfMirror>(hi, lo);
  max_u64_step<kDppMirror>(hi, lo);
  return ((unsigned long long)hi << 32) | lo;
}

// Sum over lanes l, l^16, l^32 and l^48 with the gfx950 lane-swap instructions;
// all four lanes receive the same total.
__device__ __forceinline__ float sum_q4(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = __int_as_float(p[0]) + __int_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(q[0]) + __int_as_float(q[1]);
}

// Maximum over the same four lanes, all four receiving it.
__device__ __forceinline__ float max_q4(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(q[0]), __int_as_float(q[1]));
}

__device__ __forceinline__ float lane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Wave-wide reductions: row totals, then the four rows combined as uniform values.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = row_max16_u64(v);
  unsigned long long best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    const unsigned long long k = ((unsigned long long)hi << 32) | lo;
    best = k > best ? k : best;
  }
  return best;
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

// Non-temporal 16-byte load, for data read once per frame (streamed weights,
// the Talker KV cache): it then does not displace what later steps re-read.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The inverse frequency of RoPE pair l (dimensions l and l + 64) in revolutions
// per position, theta^(-2l/128) / (2 pi), in double.
__device__ __forceinline__ double rope_inv_rev(int l, float theta_log2) {
  return exp2(-(double)(2 * l) * (double)theta_log2 / 128.0) *
         0.15915494309189533576888376337251;  // 1 / (2 pi)
}

// Per-head RMSNorm + rotate-half RoPE of one 128-vector held by one wave, lane l
// holding elements l (v0) and l + 64 (v1), the two halves of its RoPE pair: the
// norm is one wave reduction and the rotation stays in the lane, so no block
// barrier is needed.  The angle pos * inv_rev is reduced to [0, 1) revolutions
// in double; the hardware sine and cosine take it from there.
__device__ __forceinline__ void norm_rope_pair(float& v0, float& v1, float g0, float g1, float eps,
                                               double inv_rev, int pos) {
  const float f = 1.0f / sqrtf(wave_sum(v0 * v0 + v1 * v1) * (1.0f / 128.0f) + eps);
  v0 = v0 * f * g0;
  v1 = v1 * f * g1;
  double rev = (double)pos * inv_rev;
  rev -= floor(rev);
  const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
  const float r0 = v0 * cs - v1 * sn, r1 = v1 * cs + v0 * sn;
  v0 = r0;
  v1 = r1;
}

}  // namespace dev
}  // namespace qt
