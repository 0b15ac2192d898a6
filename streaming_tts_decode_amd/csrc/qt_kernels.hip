// gfx950 kernels of the lockstep decode frame.
//
// Every kernel here is launched by qt_abi.cpp on the caller's stream; shapes
// are validated on the host before launch (see the launchers at the end).
//
// Data types: weights bf16 or int8 (+ fp32 per-row scale), GEMM activations
// bf16, accumulation fp32, residual streams fp32, KV caches bf16.
#include <math.h>

#include "qt_internal.h"

namespace qt {
namespace {

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

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Epilogue over a block's finished tile: tile[r * tld + m] is the dot product
// of weight row n0 + r with activation row m (before the INT8 scale).
__device__ void gemm_epilogue(const GemmArgs& a, int n0, int rows, const float* tile, int tld) {
  const int M = a.M;
  const int tid = threadIdx.x, nthr = blockDim.x;
  if (a.epi == EPI_SWIGLU) {
    for (int e = tid; e < (rows >> 1) * M; e += nthr) {
      const int pr = e / M, m = e - pr * M;
      const int n = n0 + 2 * pr;
      float g = tile[(2 * pr) * tld + m], u = tile[(2 * pr + 1) * tld + m];
      if (a.scale) {
        g *= a.scale[n];
        u *= a.scale[n + 1];
      }
      split_bf16(silu(g) * u, a.out_bf16, a.out_bf16_lo, (size_t)m * a.out_ld + (n >> 1));
    }
    return;
  }
  for (int e = tid; e < rows * M; e += nthr) {
    const int r = e / M, m = e - r * M;
    const int n = n0 + r;
    float y = tile[r * tld + m];
    if (a.scale) y *= a.scale[n];
    if (a.epi == EPI_STORE) {
      a.out_f32[(size_t)m * a.out_ld + n] = y;
    } else if (a.epi == EPI_RESID) {
      a.out_f32[(size_t)m * a.out_ld + n] += y;
    } else {  // EPI_HEAD
      if (n < a.n_logits)
        a.logits[(size_t)m * a.logits_ld + n] = y;
      else
        a.out_f32[(size_t)m * a.out_ld + (n - a.n_logits)] = y;
    }
  }
  if (a.epi == EPI_HEAD && n0 < a.argmax_range) {
    const int lane = tid & 63, wave = tid >> 6, nw = nthr >> 6;
    for (int m = wave; m < M; m += nw) {
      unsigned long long best = 0;
      bool nan = false;
      for (int r = lane; r < rows; r += 64) {
        const int n = n0 + r;
        if (n >= a.argmax_range) break;
        float y = tile[r * tld + m];
        if (a.scale) y *= a.scale[n];
        if (y != y) {
          nan = true;
          continue;
        }
        const unsigned long long k = greedy_key(y, n);
        best = k > best ? k : best;
      }
      best = wave_max_u64(best);
      if (nan) atomicOr(a.status, QT_STATUS_NAN);
      if (lane == 0 && best) atomicMax(&a.keys[(size_t)m * a.keys_ld], best);
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny GEMM, VALU path (M <= 8 activation rows).
// Block = 4 waves; wave w owns weight rows n0 + w*RW .. +RW and walks the whole
// K range with 16-byte chunks per lane (lane-contiguous, so one wave load is
// 1 KB of one row); activations come from L1/L2.  The RW x MP partial sums are
// reduced across the wave with a halving exchange; no cross-wave reduction.
template <int MP, int RW, bool I8>
__global__ __launch_bounds__(256) void k_gemm_valu(GemmArgs a) {
  constexpr int V = MP * RW;
  constexpr int P = Log2<V>::value;
  __shared__ float tile[4 * RW * MP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = a.row0 + blockIdx.x * 4 * RW;
  const int nw0 = n0 + wave * RW;
  const int M = a.M;
  float acc[RW][MP];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int b = 0; b < MP; ++b) acc[r][b] = 0.0f;

  if (!I8) {
    const int KC = a.K >> 3;  // 8 bf16 per 16-byte chunk
    const uint4* W = reinterpret_cast<const uint4*>(a.W);
#pragma unroll 2
    for (int kc = lane; kc < KC; kc += 64) {
      uint4 x[MP], xl[MP];
#pragma unroll
      for (int b = 0; b < MP; ++b) {
        x[b] = make_uint4(0, 0, 0, 0);
        xl[b] = make_uint4(0, 0, 0, 0);
        if (b < M) {
          x[b] = reinterpret_cast<const uint4*>(a.act + (size_t)b * a.act_ld)[kc];
          if (a.act_lo) xl[b] = reinterpret_cast<const uint4*>(a.act_lo + (size_t)b * a.act_ld)[kc];
        }
      }
      uint4 w[RW];
#pragma unroll
      for (int r = 0; r < RW; ++r) w[r] = W[(size_t)(nw0 + r) * KC + kc];
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int b = 0; b < MP; ++b) acc[r][b] = dot8(w[r], xl[b], dot8(w[r], x[b], acc[r][b]));
    }
  } else {
    const int KC = a.K >> 4;  // 16 int8 per 16-byte chunk
    const uint4* W = reinterpret_cast<const uint4*>(a.W);
#pragma unroll 2
    for (int kc = lane; kc < KC; kc += 64) {
      uint4 x0[MP], x1[MP], l0[MP], l1[MP];
#pragma unroll
      for (int b = 0; b < MP; ++b) {
        x0[b] = x1[b] = l0[b] = l1[b] = make_uint4(0, 0, 0, 0);
        if (b < M) {
          const uint4* p = reinterpret_cast<const uint4*>(a.act + (size_t)b * a.act_ld);
          x0[b] = p[2 * kc];
          x1[b] = p[2 * kc + 1];
          if (a.act_lo) {
            const uint4* pl = reinterpret_cast<const uint4*>(a.act_lo + (size_t)b * a.act_ld);
            l0[b] = pl[2 * kc];
            l1[b] = pl[2 * kc + 1];
          }
        }
      }
      uint4 wq[RW];
#pragma unroll
      for (int r = 0; r < RW; ++r) wq[r] = W[(size_t)(nw0 + r) * KC + kc];
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        uint4 wa, wb;  // 16 int8 -> 16 bf16
        wa.x = i8pair_to_bf16x2(wq[r].x, 0);
        wa.y = i8pair_to_bf16x2(wq[r].x, 1);
        wa.z = i8pair_to_bf16x2(wq[r].y, 0);
        wa.w = i8pair_to_bf16x2(wq[r].y, 1);
        wb.x = i8pair_to_bf16x2(wq[r].z, 0);
        wb.y = i8pair_to_bf16x2(wq[r].z, 1);
        wb.z = i8pair_to_bf16x2(wq[r].w, 0);
        wb.w = i8pair_to_bf16x2(wq[r].w, 1);
#pragma unroll
        for (int b = 0; b < MP; ++b)
          acc[r][b] = dot8(wb, l1[b], dot8(wa, l0[b], dot8(wb, x1[b], dot8(wa, x0[b], acc[r][b]))));
      }
    }
  }

  float flat[V];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int b = 0; b < MP; ++b) flat[r * MP + b] = acc[r][b];
  const float tot = transpose_reduce<V>(flat, lane);
  if ((lane & ((64 >> P) - 1)) == 0) {
    const int idx = lane >> (6 - P);
    tile[(wave * RW + idx / MP) * MP + (idx % MP)] = tot;
  }
  __syncthreads();
  gemm_epilogue(a, n0, 4 * RW, tile, MP);
}

// ---------------------------------------------------------------------------
// Skinny GEMM, MFMA path (8 < M <= 64).  v_mfma_f32_16x16x32_bf16 with the
// weight rows as the A operand (16 rows) and the activation rows as the B
// operand (16 columns per tile, MT tiles).  Lane l feeds row (l & 15) at a
// 32-element K slice starting at 32*(l >> 4) of every 128-element K step, and
// the four MFMAs of the step take its four 8-element pieces; A and B use the
// same K permutation, so the sum over K is unchanged.  The 4 waves of a block
// split K; their accumulators are summed in a fixed order through LDS.
template <int MT, int RT, bool I8>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs a) {
  __shared__ float red[4][RT][MT][64][4];
  __shared__ float tile[RT * 16 * MT * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int n0 = a.row0 + blockIdx.x * RT * 16;
  const int Kw = a.K >> 2;
  const int kbeg = wave * Kw;
  const int M = a.M;
  f32x4 acc[RT][MT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kb = kbeg; kb < kbeg + Kw; kb += 128) {
    bf16x8 bop[MT][4], bol[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + i;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bop[t][s] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        bol[t][s] = bop[t][s];
      }
      if (m < M) {
        const size_t off = (size_t)m * a.act_ld + kb + 32 * q;
        const uint4* p = reinterpret_cast<const uint4*>(a.act + off);
#pragma unroll
        for (int s = 0; s < 4; ++s) bop[t][s] = __builtin_bit_cast(bf16x8, p[s]);
        if (a.act_lo) {
          const uint4* pl = reinterpret_cast<const uint4*>(a.act_lo + off);
#pragma unroll
          for (int s = 0; s < 4; ++s) bol[t][s] = __builtin_bit_cast(bf16x8, pl[s]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int n = n0 + r * 16 + i;
      bf16x8 aop[4];
      if (!I8) {
        const uint4* p = reinterpret_cast<const uint4*>(
            reinterpret_cast<const uint16_t*>(a.W) + (size_t)n * a.K + kb + 32 * q);
#pragma unroll
        for (int s = 0; s < 4; ++s) aop[s] = __builtin_bit_cast(bf16x8, p[s]);
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(
            reinterpret_cast<const int8_t*>(a.W) + (size_t)n * a.K + kb + 32 * q);
        const uint4 w0 = p[0], w1 = p[1];
        const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint4 c;
          c.x = i8pair_to_bf16x2(words[2 * s], 0);
          c.y = i8pair_to_bf16x2(words[2 * s], 1);
          c.z = i8pair_to_bf16x2(words[2 * s + 1], 0);
          c.w = i8pair_to_bf16x2(words[2 * s + 1], 1);
          aop[s] = __builtin_bit_cast(bf16x8, c);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[s], bop[t][s], acc[r][t], 0, 0, 0);
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[s], bol[t][s], acc[r][t], 0, 0, 0);
        }
    }
  }

#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][r][t][lane][j] = acc[r][t][j];
  __syncthreads();
  // D layout of the 16x16 output: lane l, element j holds row 4*(l>>4)+j, column l&15.
  constexpr int TLD = MT * 16;
  for (int e = threadIdx.x; e < RT * MT * 256; e += 256) {
    const int j = e & 3, l = (e >> 2) & 63, t = (e >> 8) % MT, r = (e >> 8) / MT;
    const float s = red[0][r][t][l][j] + red[1][r][t][l][j] + red[2][r][t][l][j] + red[3][r][t][l][j];
    tile[(r * 16 + 4 * (l >> 4) + j) * TLD + t * 16 + (l & 15)] = s;
  }
  __syncthreads();
  gemm_epilogue(a, n0, RT * 16, tile, TLD);
}

// ---------------------------------------------------------------------------
// Row RMSNorm: u = x / sqrt(mean(x^2) + eps) * g as a hi/lo bf16 pair.  One block per row.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, int x_ld, const uint16_t* g,
                                                 int K, float eps, uint16_t* u, uint16_t* u_lo,
                                                 int u_ld) {
  __shared__ float part[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)row * x_ld;
  float ss = 0.f;
  for (int k = tid; k < K; k += 256) ss += xr[k] * xr[k];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)K + eps);
  const size_t base = (size_t)row * u_ld;
  for (int k = tid; k < K; k += 256) split_bf16(xr[k] * inv * bf2f(g[k]), u, u_lo, base + k);
}

// Per-head RMSNorm + rotate-half RoPE of one 128-vector held by 128 threads
// (thread d of the group holds element d).  `buf` is a 128-float LDS slot used
// for the pair exchange; `ss_slot` two floats for the sum of squares of the two
// waves of the group.  Returns the rotated element d.
__device__ __forceinline__ float norm_rope_128(float v, int d, const uint16_t* gain, float eps,
                                               int pos, float theta_log2, float* buf,
                                               float* ss_slot) {
  const int lane = threadIdx.x & 63;
  float ss = wave_sum(v * v);
  if (lane == 0) ss_slot[(d >> 6)] = ss;
  __syncthreads();
  const float tot = ss_slot[0] + ss_slot[1];
  const float nv = v * (1.0f / sqrtf(tot * (1.0f / 128.0f) + eps)) * bf2f(gain[d]);
  buf[d] = nv;
  __syncthreads();
  const int i = d & 63;
  // angle = pos * theta^(-2i/128), reduced mod 2*pi in double before the float sincos
  const double inv_freq = exp2(-(double)(2 * i) * (double)theta_log2 / 128.0);
  double ang = (double)pos * inv_freq;
  const double two_pi = 6.283185307179586476925286766559;
  ang -= two_pi * floor(ang / two_pi);
  float sn, cs;
  sincosf((float)ang, &sn, &cs);
  const float partner = buf[d ^ 64];
  return (d < 64) ? nv * cs - partner * sn : nv * cs + partner * sn;
}

// ---------------------------------------------------------------------------
// Talker decode attention over paged KV.  Grid (split, kv head, session).
// The block for (b, h, s) handles query heads 2h, 2h+1 over positions
// [s*S, min((s+1)*S, p+1)) where p = kv_len[b] is the new token's position.
// The split holding p also normalises/rotates the new key, stores the new key
// and value into their page and uses them from LDS.  Splits write (max, sum,
// unnormalised output) partials; the last block to arrive merges them in split
// order (deterministic), writes the bf16 attention output and resets the
// counter.
__global__ __launch_bounds__(256) void k_attn_paged(AttnPagedArgs a, float theta_log2) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float qs[2][128];
  __shared__ float rb[2][128];
  __shared__ float knew[128], vnew[128];
  __shared__ float sc[2][kMaxPagesPerSplit * kPage];
  __shared__ float red[4][2][128];
  __shared__ float ssq[2][2];
  __shared__ float stat[2][2];
  __shared__ float mstat[2], lstat[2];
  __shared__ int s_last;

  const int cap = a.max_pages * kPage;
  const int p = a.kv_len[b];
  const int j0 = 2 * h;
  const int jj = tid >> 7, d = tid & 127;
  const size_t orow = (size_t)b * a.o_ld + (j0 + jj) * 128 + d;
  if (p < 0 || p >= cap) {
    if (s == 0) a.o[orow] = a.o_lo[orow] = 0;
    return;
  }
  const int S = a.pages_per_split * kPage;
  const int n_active = p / S + 1;
  if (s >= n_active) return;
  const int t0 = s * S, t1 = min(t0 + S, p + 1);
  const bool has_new = (s == n_active - 1);
  const float* qrow = a.qkv + (size_t)b * a.qkv_ld;
  const int q_dim = a.n_q * 128, kv_dim = a.n_kv * 128;

  // q heads j0 (threads 0..127) and j0+1 (128..255)
  {
    const float v = qrow[(j0 + jj) * 128 + d];
    const float r = norm_rope_128(v, d, a.q_norm, a.eps, p, theta_log2, rb[jj], ssq[jj]);
    qs[jj][d] = r * kInvSqrtHd;
  }
  const int* ptab = a.page_table + (size_t)b * a.max_pages;
  if (has_new) {
    // threads 0..127: key of KV head h (normalised and rotated); threads 128..255:
    // value (taken raw; the normalisation both halves run keeps barriers uniform)
    const float raw = qrow[q_dim + (jj ? kv_dim : 0) + h * 128 + d];
    const float kr = norm_rope_128(raw, d, a.k_norm, a.eps, p, theta_log2, rb[jj], ssq[jj]);
    const float kv = jj ? raw : kr;
    const uint16_t bits = f2bf(kv);
    const int pg = ptab[p / kPage];
    if (pg >= 0 && pg < a.num_pages) {
      const size_t off = ((size_t)pg * a.n_kv + h) * (kPage * 128) + (size_t)(p % kPage) * 128 + d;
      (jj == 0 ? a.k_pool : a.v_pool)[off] = bits;
    } else if (d == 0 && jj == 0) {
      atomicOr(a.status, QT_STATUS_BAD_PAGE);
    }
    (jj == 0 ? knew : vnew)[d] = bf2f(bits);
  }
  __syncthreads();

  // scores: thread (pi = tid>>4, c = tid&15) covers position t0+16g+pi, dims 8c..8c+7
  const int pi = tid >> 4, c = tid & 15;
  float q0[8], q1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    q0[e] = qs[0][8 * c + e];
    q1[e] = qs[1][8 * c + e];
  }
  uint4 kk[kMaxPagesPerSplit], vv[kMaxPagesPerSplit];
#pragma unroll
  for (int g = 0; g < kMaxPagesPerSplit; ++g) {
    kk[g] = make_uint4(0, 0, 0, 0);
    vv[g] = make_uint4(0, 0, 0, 0);
    const int t = t0 + g * kPage + pi;
    if (g < a.pages_per_split && t < t1 && t != p) {
      const int pg = ptab[t / kPage];
      if (pg >= 0 && pg < a.num_pages) {
        const size_t off = ((size_t)pg * a.n_kv + h) * (kPage * 128) + (size_t)pi * 128 + 8 * c;
        kk[g] = *reinterpret_cast<const uint4*>(a.k_pool + off);
        vv[g] = *reinterpret_cast<const uint4*>(a.v_pool + off);
      } else if (c == 0) {
        atomicOr(a.status, QT_STATUS_BAD_PAGE);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kMaxPagesPerSplit; ++g) {
    if (g >= a.pages_per_split) break;
    const int t = t0 + g * kPage + pi;
    float kf[8];
    if (t == p) {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = knew[8 * c + e];
    } else {
      kf[0] = bf_lo(kk[g].x); kf[1] = bf_hi(kk[g].x);
      kf[2] = bf_lo(kk[g].y); kf[3] = bf_hi(kk[g].y);
      kf[4] = bf_lo(kk[g].z); kf[5] = bf_hi(kk[g].z);
      kf[6] = bf_lo(kk[g].w); kf[7] = bf_hi(kk[g].w);
    }
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s0 = fmaf(q0[e], kf[e], s0);
      s1 = fmaf(q1[e], kf[e], s1);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      s0 += __shfl_xor(s0, o);
      s1 += __shfl_xor(s1, o);
    }
    if (c == 0) {
      sc[0][g * kPage + pi] = (t < t1) ? s0 : -INFINITY;
      sc[1][g * kPage + pi] = (t < t1) ? s1 : -INFINITY;
    }
  }
  __syncthreads();

  // softmax statistics per head over this split (threads 0..127 head 0, 128..255 head 1)
  const int n = t1 - t0;
  {
    const float v = (d < n) ? sc[jj][d] : -INFINITY;
    const float mx = wave_max(v);
    if (lane == 0) stat[jj][wave & 1] = mx;
    __syncthreads();
    const float m = fmaxf(stat[jj][0], stat[jj][1]);
    const float e = (d < n) ? expf(v - m) : 0.f;
    const float sm = wave_sum(e);
    __syncthreads();
    if (d < n) sc[jj][d] = e;
    if (lane == 0) stat[jj][wave & 1] = sm;
    if (d == 0) mstat[jj] = m;
    __syncthreads();
    if (d == 0) lstat[jj] = stat[jj][0] + stat[jj][1];
  }
  __syncthreads();

  // weighted values
  float a0[8], a1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a0[e] = a1[e] = 0.f;
#pragma unroll
  for (int g = 0; g < kMaxPagesPerSplit; ++g) {
    if (g >= a.pages_per_split) break;
    const int t = t0 + g * kPage + pi;
    if (t < t1) {
      const float w0 = sc[0][g * kPage + pi], w1 = sc[1][g * kPage + pi];
      float vf[8];
      if (t == p) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = vnew[8 * c + e];
      } else {
        vf[0] = bf_lo(vv[g].x); vf[1] = bf_hi(vv[g].x);
        vf[2] = bf_lo(vv[g].y); vf[3] = bf_hi(vv[g].y);
        vf[4] = bf_lo(vv[g].z); vf[5] = bf_hi(vv[g].z);
        vf[6] = bf_lo(vv[g].w); vf[7] = bf_hi(vv[g].w);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a0[e] = fmaf(w0, vf[e], a0[e]);
        a1[e] = fmaf(w1, vf[e], a1[e]);
      }
    }
  }
  // reduce over the 4 positions of the wave (lanes c, c+16, c+32, c+48)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a0[e] += __shfl_xor(a0[e], 16);
    a1[e] += __shfl_xor(a1[e], 16);
    a0[e] += __shfl_xor(a0[e], 32);
    a1[e] += __shfl_xor(a1[e], 32);
  }
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[wave][0][8 * c + e] = a0[e];
      red[wave][1][8 * c + e] = a1[e];
    }
  }
  __syncthreads();
  const float out = red[0][jj][d] + red[1][jj][d] + red[2][jj][d] + red[3][jj][d];
  if (n_active == 1) {
    split_bf16(out / lstat[jj], a.o, a.o_lo, orow);
    return;
  }
  float* pp = a.part + (((size_t)b * a.n_q + j0 + jj) * a.n_splits + s) * 130;
  pp[2 + d] = out;
  if (d == 0) {
    pp[0] = mstat[jj];
    pp[1] = lstat[jj];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&a.counters[(size_t)b * a.n_kv + h], 1u);
    s_last = (prev == (unsigned)(n_active - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* pb = a.part + ((size_t)b * a.n_q + j0 + jj) * a.n_splits * 130;
  float M = -INFINITY;
  for (int ss = 0; ss < n_active; ++ss) M = fmaxf(M, pb[ss * 130]);
  float L = 0.f, O = 0.f;
  for (int ss = 0; ss < n_active; ++ss) {
    const float w = expf(pb[ss * 130] - M);
    L = fmaf(pb[ss * 130 + 1], w, L);
    O = fmaf(pb[ss * 130 + 2 + d], w, O);
  }
  split_bf16(O / L, a.o, a.o_lo, orow);
  if (tid == 0) a.counters[(size_t)b * a.n_kv + h] = 0u;
}

// ---------------------------------------------------------------------------
// Code-predictor attention over its short, preallocated, contiguous cache.
// Grid (kv head, session).  n_new (1 or 2) new positions pos0 .. pos0+n_new-1
// are normalised, rotated, appended, and each attends causally to positions
// 0 .. its own.  At most 16 positions: one thread group of 16 per position.
__global__ __launch_bounds__(256) void k_attn_pred(AttnPredArgs a, float theta_log2) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jj = tid >> 7, d = tid & 127;
  __shared__ float qs[2][2][128];
  __shared__ float kn[2][128], vn[2][128];
  __shared__ float rb[2][128];
  __shared__ float ssq[2][2];
  __shared__ float sc[2][2][16];
  __shared__ float red[4][2][2][128];
  __shared__ float lsum[2][2];
  const int j0 = 2 * h;
  const int q_dim = a.n_q * 128, kv_dim = a.n_kv * 128;
  uint16_t* kbase = a.k_cache + (size_t)b * a.sess_stride;
  uint16_t* vbase = a.v_cache + (size_t)b * a.sess_stride;

  for (int i = 0; i < a.n_new; ++i) {
    const float* row = a.qkv + (size_t)(i * a.B + b) * a.qkv_ld;
    const int pos = a.pos0 + i;
    const float r = norm_rope_128(row[(j0 + jj) * 128 + d], d, a.q_norm, a.eps, pos, theta_log2,
                                  rb[jj], ssq[jj]);
    qs[i][jj][d] = r * kInvSqrtHd;
    __syncthreads();
    const float raw = row[q_dim + (jj ? kv_dim : 0) + h * 128 + d];
    const float kr = norm_rope_128(raw, d, a.k_norm, a.eps, pos, theta_log2, rb[jj], ssq[jj]);
    const float kv = jj ? raw : kr;
    const uint16_t bits = f2bf(kv);
    const size_t off = ((size_t)pos * a.n_kv + h) * 128 + d;
    (jj == 0 ? kbase : vbase)[off] = bits;
    (jj == 0 ? kn[i] : vn[i])[d] = bf2f(bits);
    __syncthreads();
  }

  const int n_pos = a.pos0 + a.n_new;
  const int t = tid >> 4, c = tid & 15;
  float kf[8], vf[8];
  if (t < n_pos) {
    if (t >= a.pos0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kf[e] = kn[t - a.pos0][8 * c + e];
        vf[e] = vn[t - a.pos0][8 * c + e];
      }
    } else {
      const size_t off = ((size_t)t * a.n_kv + h) * 128 + 8 * c;
      const uint4 kq = *reinterpret_cast<const uint4*>(kbase + off);
      const uint4 vq = *reinterpret_cast<const uint4*>(vbase + off);
      kf[0] = bf_lo(kq.x); kf[1] = bf_hi(kq.x); kf[2] = bf_lo(kq.y); kf[3] = bf_hi(kq.y);
      kf[4] = bf_lo(kq.z); kf[5] = bf_hi(kq.z); kf[6] = bf_lo(kq.w); kf[7] = bf_hi(kq.w);
      vf[0] = bf_lo(vq.x); vf[1] = bf_hi(vq.x); vf[2] = bf_lo(vq.y); vf[3] = bf_hi(vq.y);
      vf[4] = bf_lo(vq.z); vf[5] = bf_hi(vq.z); vf[6] = bf_lo(vq.w); vf[7] = bf_hi(vq.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[e] = vf[e] = 0.f;
  }
  // scores for every (new position i, head jj)
  for (int i = 0; i < a.n_new; ++i) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(qs[i][hh][8 * c + e], kf[e], s);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (c == 0) sc[i][hh][t] = (t <= a.pos0 + i) ? s : -INFINITY;
    }
  }
  __syncthreads();
  if (tid < 2 * a.n_new) {
    const int i = tid >> 1, hh = tid & 1;
    float m = -INFINITY;
    for (int u = 0; u <= a.pos0 + i; ++u) m = fmaxf(m, sc[i][hh][u]);
    float l = 0.f;
    for (int u = 0; u < 16; ++u) {
      const float e = (u <= a.pos0 + i) ? expf(sc[i][hh][u] - m) : 0.f;
      sc[i][hh][u] = e;
      l += e;
    }
    lsum[i][hh] = l;
  }
  __syncthreads();
  for (int i = 0; i < a.n_new; ++i) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float w = (t < n_pos) ? sc[i][hh][t] : 0.f;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e] = w * vf[e];
        acc[e] += __shfl_xor(acc[e], 16);
        acc[e] += __shfl_xor(acc[e], 32);
      }
      if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][i][hh][8 * c + e] = acc[e];
      }
    }
  }
  __syncthreads();
  for (int i = 0; i < a.n_new; ++i) {
    const float out = red[0][i][jj][d] + red[1][i][jj][d] + red[2][i][jj][d] + red[3][i][jj][d];
    split_bf16(out / lsum[i][jj], a.o, a.o_lo, (size_t)(i * a.B + b) * a.o_ld + (j0 + jj) * 128 + d);
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_frame_begin(FrameBeginArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  if (a.mode != QT_MODE_PREDICTOR) {
    for (int i = tid; i < a.Ht; i += 256)
      a.x_t[(size_t)b * a.Ht + i] = bf2f(a.talker_in[(size_t)b * a.Ht + i]);
    if (tid == 0) {
      const int p = a.kv_len[b];
      if (p < 0 || p + 1 > a.capacity) atomicOr(a.status, QT_STATUS_KV_OVERFLOW);
    }
  } else {
    for (int i = tid; i < a.Ht; i += 256) a.u[(size_t)b * a.u_ld + i] = a.h_in[(size_t)b * a.Ht + i];
  }
  for (int k = tid; k < a.ncb; k += 256) {
    unsigned long long key = 0;
    if (a.mode == QT_MODE_PREDICTOR && k == 0) key = greedy_key(0.0f, a.tok0_in[b]);
    a.keys[(size_t)b * a.ncb + k] = key;
  }
  if (tid < a.n_kv) a.counters[(size_t)b * a.n_kv + tid] = 0u;
}

__global__ __launch_bounds__(256) void k_embed(EmbedArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  int tok = a.forced ? a.forced[(size_t)b * a.ncb + a.step - 1]
                     : key_index(a.keys[(size_t)b * a.ncb + a.step - 1]);
  if (tok < 0 || tok >= a.vocab) {
    if (tid == 0) atomicOr(a.status, QT_STATUS_BAD_TOKEN);
    tok = 0;
  }
  const uint16_t* src = a.table + (size_t)tok * a.H;
  float* dst = a.x + (size_t)(a.row_off + b) * a.H;
  for (int i = tid; i < a.H; i += 256) dst[i] = bf2f(src[i]);
}

__global__ __launch_bounds__(256) void k_frame_end(FrameEndArgs a) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.B * a.ncb) return;
  const int b = e / a.ncb, k = e - b * a.ncb;
  int tok = key_index(a.keys[e]);
  if (a.mode == QT_MODE_TALKER && k > 0) tok = -1;
  a.tokens[e] = tok;
  if (k == 0 && a.mode != QT_MODE_PREDICTOR) {
    const int p = a.kv_len[b];
    if (p >= 0 && p + 1 <= a.capacity) a.kv_len[b] = p + 1;
  }
}

// ---------------------------------------------------------------------------
// Per-row symmetric INT8: s = max|w| / 127 (IEEE divide), q = clamp(rint(w / s), +-127).
__global__ __launch_bounds__(256) void k_quantize(const uint16_t* w, long long cols, int8_t* q,
                                                  long long q_stride, float* scale,
                                                  long long s_stride) {
  __shared__ float part[4];
  const long long r = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* row = w + r * cols;
  float amax = 0.f;
  for (long long k = tid; k < cols; k += 256) amax = fmaxf(amax, fabsf(bf2f(row[k])));
  amax = wave_max(amax);
  if ((tid & 63) == 0) part[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float sc = __fdiv_rn(amax, 127.0f);
  if (tid == 0) scale[r * s_stride] = sc;
  int8_t* qr = q + r * q_stride;
  for (long long k = tid; k < cols; k += 256) {
    float v = 0.f;
    if (sc != 0.f) {
      v = rintf(__fdiv_rn(bf2f(row[k]), sc));
      v = fminf(fmaxf(v, -127.f), 127.f);
    }
    qr[k] = (int8_t)(int)v;
  }
}

inline int pow2_at_least(int m) {
  int p = 1;
  while (p < m) p <<= 1;
  return p;
}

template <int MP, bool I8>
hipError_t gemm_valu_mp(const GemmArgs& a, hipStream_t s) {
  if (a.nrows >= 4096) {
    hipLaunchKernelGGL((k_gemm_valu<MP, 4, I8>), dim3(a.nrows / 16), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_gemm_valu<MP, 2, I8>), dim3(a.nrows / 8), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int MT, bool I8>
hipError_t gemm_mfma_mt(const GemmArgs& a, hipStream_t s) {
  if (a.nrows >= 4096) {
    hipLaunchKernelGGL((k_gemm_mfma<MT, 2, I8>), dim3(a.nrows / 32), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_gemm_mfma<MT, 1, I8>), dim3(a.nrows / 16), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <bool I8>
hipError_t gemm_dispatch(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 8) {
    switch (pow2_at_least(a.M)) {
      case 1: return gemm_valu_mp<1, I8>(a, s);
      case 2: return gemm_valu_mp<2, I8>(a, s);
      case 4: return gemm_valu_mp<4, I8>(a, s);
      default: return gemm_valu_mp<8, I8>(a, s);
    }
  }
  if (a.M <= 16) return gemm_mfma_mt<1, I8>(a, s);
  if (a.M <= 32) return gemm_mfma_mt<2, I8>(a, s);
  return gemm_mfma_mt<4, I8>(a, s);
}

}  // namespace

// --------------------------------------------------------------------------- launchers
hipError_t launch_rmsnorm(const float* x, int x_ld, const uint16_t* g, int K, float eps,
                          uint16_t* u, uint16_t* u_lo, int u_ld, int M, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(M), dim3(256), 0, s, x, x_ld, g, K, eps, u, u_lo, u_ld);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 64 || a.nrows <= 0 || (a.nrows % 64) || (a.K % 512) ||
      (a.epi == EPI_SWIGLU && (a.row0 & 1)))
    return hipErrorInvalidValue;
  return a.scale ? gemm_dispatch<true>(a, s) : gemm_dispatch<false>(a, s);
}

hipError_t launch_attn_paged(const AttnPagedArgs& a, int B, float theta, hipStream_t s) {
  if (a.pages_per_split < 1 || a.pages_per_split > kMaxPagesPerSplit || a.n_q != 2 * a.n_kv)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_paged, dim3(a.n_splits, a.n_kv, B), dim3(256), 0, s, a,
                     (float)log2((double)theta));
  return hipGetLastError();
}

hipError_t launch_attn_pred(const AttnPredArgs& a, float theta, hipStream_t s) {
  if (a.n_new < 1 || a.n_new > 2 || a.pos0 < 0 || a.pos0 + a.n_new > 16 || a.n_q != 2 * a.n_kv)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_pred, dim3(a.n_kv, a.B), dim3(256), 0, s, a,
                     (float)log2((double)theta));
  return hipGetLastError();
}

hipError_t launch_frame_begin(const FrameBeginArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_frame_begin, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_embed(const EmbedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_frame_end(const FrameEndArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_frame_end, dim3((a.B * a.ncb + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* w, long long rows, long long cols, int8_t* q,
                           long long q_row_stride, float* scale, long long scale_stride,
                           hipStream_t s) {
  if (rows <= 0 || cols <= 0 || rows > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)rows), dim3(256), 0, s, w, cols, q, q_row_stride,
                     scale, scale_stride);
  return hipGetLastError();
}

}  // namespace qt
