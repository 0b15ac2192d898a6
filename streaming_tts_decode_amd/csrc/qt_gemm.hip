// Weight-streaming GEMMs of the decode frame on gfx950:
//   y[m][n] = sum_k W[n][k] * act[m][k]   (times scale[n] for INT8 weights)
// for M = 1..64 activation rows (sessions, or 2 x sessions at predictor step 1).
//
// Every weight byte is read once per call for all M rows, and a block issues all
// of its weight and activation loads of a step group before any arithmetic, so
// a call costs about one memory round trip (these GEMMs are latency-bound at small
// batch).  No block waits on another block.
//  * VALU (M <= 2): a 4-wave block owns 4 weight rows, one per wave; lanes walk K
//    in 16-byte chunks (one wave load = 1 KB of a row); v_dot2_f32_bf16.
//  * MFMA (M >= 3): v_mfma_f32_16x16x32_bf16 with weight rows as the A operand.
//    An 8-wave block owns 16 weight rows; wave w takes the 128-wide K steps
//    w, w+8, ... two at a time, and the waves' 16x16 accumulator tiles are summed
//    in a fixed order through LDS.  Within a step, lane (i, q) (i = lane & 15,
//    q = lane >> 4) feeds row i with elements [32s + 8q, +8) to the s-th MFMA, so
//    the four lanes of a row read 64 contiguous bytes per load instruction; the
//    activation operand uses the same mapping.
//
// Activations are a bf16 hi/lo pair (hi + lo carries ~16 bits of the fp32 value).
// RMSNorm is split between producer and consumer: the GEMM (or kernel) that
// writes a residual row v also writes hi/lo(v * gain) and the row block's sum of
// squares; the consuming GEMM multiplies its outputs by 1/rms from those sums.
#include <stdio.h>

#include "qt_device.h"
#include "qt_internal.h"

namespace qt {
namespace {
using namespace dev;

// Registers for prefetched sum-of-squares slots, per wave.
constexpr int kSsRegs = 16;

// Issue the sum-of-squares loads of rows m = first + step*j before the main loads,
// so that waiting on them later does not wait on the main loads.
__device__ __forceinline__ void ss_prefetch(const GemmArgs& a, int first, int step,
                                            float (&r)[kSsRegs], int& per_lane) {
  const int lane = threadIdx.x & 63;
  per_lane = (a.ss_in_slots + 63) / 64;
  int idx = 0;
#pragma unroll
  for (int j = 0; j < kSsRegs; ++j) r[j] = 0.f;
  for (int m = first; m < a.M; m += step)
    for (int s = 0; s < per_lane && idx < kSsRegs; ++s, ++idx) {
      const int slot = lane + 64 * s;
      r[idx] = slot < a.ss_in_slots ? a.ss_in[(size_t)slot * a.ss_in_ld + m] : 0.f;
    }
}

// Finish the inverse RMS of the prefetched rows into s_inv (slots that did not fit
// in the registers are summed directly).
__device__ __forceinline__ void ss_finish(const GemmArgs& a, int first, int step,
                                          const float (&r)[kSsRegs], int per_lane, float* s_inv) {
  const int lane = threadIdx.x & 63;
  int idx = 0;
  for (int m = first; m < a.M; m += step) {
    float ss = 0.f;
    for (int s = 0; s < per_lane; ++s, ++idx) {
      if (idx < kSsRegs) {
        ss += r[idx];
      } else {
        const int slot = lane + 64 * s;
        if (slot < a.ss_in_slots) ss += a.ss_in[(size_t)slot * a.ss_in_ld + m];
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) s_inv[m] = 1.0f / sqrtf(ss / (float)a.K + a.norm_eps);
  }
}

// Epilogue over the final tile: tile[r * tld + m] is row n0 + r, activation row m
// (before the INT8 scale and the RMSNorm factor).
__device__ void gemm_epilogue(const GemmArgs& a, int rpb, int n0, float* tile, int tld,
                              const float* s_inv) {
  const int M = a.M;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nw = nthr >> 6;
  if (a.scale || a.ss_in) {
    for (int e = tid; e < rpb * M; e += nthr) {
      const int r = e / M, m = e - r * M;
      float y = tile[r * tld + m];
      if (a.scale) y *= a.scale[n0 + r];
      if (a.ss_in) y *= s_inv[m];
      tile[r * tld + m] = y;
    }
    __syncthreads();
  }
  if (a.epi == EPI_SWIGLU) {
    for (int e = tid; e < (rpb >> 1) * M; e += nthr) {
      const int pr = e / M, m = e - pr * M;
      const int n = n0 + 2 * pr;
      const float g = tile[(2 * pr) * tld + m], u = tile[(2 * pr + 1) * tld + m];
      split_bf16(silu(g) * u, a.out_bf16, a.out_bf16_lo, (size_t)m * a.out_ld + (n >> 1));
    }
    return;
  }
  // first output row of residual / projection values (-1: none in this GEMM)
  const int base = a.epi == EPI_RESID ? 0 : (a.epi == EPI_HEAD ? a.n_logits : -1);
  for (int e = tid; e < rpb * M; e += nthr) {
    const int r = e / M, m = e - r * M;
    const int n = n0 + r;
    float v = tile[r * tld + m];
    if (a.epi == EPI_STORE) {
      a.out_f32[(size_t)m * a.out_ld + n] = v;
      continue;
    }
    if (a.epi == EPI_RESID) {
      float* p = a.out_f32 + (size_t)m * a.out_ld + n;
      v += *p;
      *p = v;
    } else if (n < a.n_logits) {  // EPI_HEAD logits
      a.logits[(size_t)m * a.logits_ld + n] = v;
      continue;
    } else {  // EPI_HEAD projection rows
      a.out_f32[(size_t)m * a.out_ld + (n - a.n_logits)] = v;
    }
    tile[r * tld + m] = v;
    if (a.u_gain) {
      const int c = n - base;
      split_bf16(v * bf2f(a.u_gain[c]), a.u_hi, a.u_lo, (size_t)m * a.u_ld + c);
    }
  }
  if (a.epi == EPI_HEAD && n0 < a.argmax_range) {
    for (int m = wave; m < M; m += nw) {
      unsigned long long best = 0;
      bool nan = false;
      for (int r = lane; r < rpb; r += 64) {
        const int n = n0 + r;
        if (n >= a.argmax_range) break;
        const float y = tile[r * tld + m];
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
  if (!a.ss_out || base < 0 || n0 < base) return;
  const int slot = (n0 - base) / rpb;
  __syncthreads();
  for (int m = wave; m < M; m += nw) {
    float ss = 0.f;
    for (int r = lane; r < rpb; r += 64) {
      const float v = tile[r * tld + m];
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) a.ss_out[(size_t)slot * a.ss_out_ld + m] = ss;
  }
}

// ------------------------------------------------------------------ VALU path
// Block = 4 waves, one weight row each; lane l loads chunks l, l+64, ... (NI per
// lane) of the row and of every activation row before any arithmetic.
template <int MP, int NI, bool I8>
__global__ __launch_bounds__(256) void k_gemm_valu(GemmArgs a) {
  constexpr int EPC = I8 ? 16 : 8;  // weight elements per 16-byte chunk
  constexpr int G = EPC / 8;        // 8-element activation groups per chunk
  __shared__ float tile[4 * MP];
  __shared__ float s_inv[MP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = a.row0 + blockIdx.x * 4;
  const int n = n0 + wave;
  const int M = a.M;
  const int KC = a.K / EPC;
  const uint4* W = reinterpret_cast<const uint4*>(a.W);

  float ssr[kSsRegs];
  int ss_per_lane = 0;
  if (a.ss_in && wave < MP) ss_prefetch(a, wave, 4, ssr, ss_per_lane);

  uint4 w[NI];
  uint4 xh[NI][G][MP], xl[NI][G][MP];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    w[i] = c < KC ? W[(size_t)n * KC + c] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int k = c * EPC + 8 * g;
#pragma unroll
      for (int b = 0; b < MP; ++b) {
        xh[i][g][b] = xl[i][g][b] = make_uint4(0, 0, 0, 0);
        if (c < KC && b < M) {
          xh[i][g][b] = *reinterpret_cast<const uint4*>(a.act + (size_t)b * a.act_ld + k);
          if (a.act_lo) xl[i][g][b] = *reinterpret_cast<const uint4*>(a.act_lo + (size_t)b * a.act_ld + k);
        }
      }
    }
  }

  float acc[MP];
#pragma unroll
  for (int b = 0; b < MP; ++b) acc[b] = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (!I8) {
#pragma unroll
      for (int b = 0; b < MP; ++b) acc[b] = dot8(w[i], xl[i][0][b], dot8(w[i], xh[i][0][b], acc[b]));
    } else {
      uint4 wa, wb;
      wa.x = i8pair_to_bf16x2(w[i].x, 0);
      wa.y = i8pair_to_bf16x2(w[i].x, 1);
      wa.z = i8pair_to_bf16x2(w[i].y, 0);
      wa.w = i8pair_to_bf16x2(w[i].y, 1);
      wb.x = i8pair_to_bf16x2(w[i].z, 0);
      wb.y = i8pair_to_bf16x2(w[i].z, 1);
      wb.z = i8pair_to_bf16x2(w[i].w, 0);
      wb.w = i8pair_to_bf16x2(w[i].w, 1);
#pragma unroll
      for (int b = 0; b < MP; ++b) {
        float t = dot8(wa, xh[i][0][b], acc[b]);
        t = dot8(wa, xl[i][0][b], t);
        t = dot8(wb, xh[i][G - 1][b], t);
        acc[b] = dot8(wb, xl[i][G - 1][b], t);
      }
    }
  }
  constexpr int P = Log2<MP>::value;
  const float tot = transpose_reduce<MP>(acc, lane);
  if ((lane & ((64 >> P) - 1)) == 0) tile[wave * MP + (lane >> (6 - P))] = tot;
  if (a.ss_in && wave < MP) ss_finish(a, wave, 4, ssr, ss_per_lane, s_inv);
  __syncthreads();
  gemm_epilogue(a, 4, n0, tile, MP, s_inv);
}

// ------------------------------------------------------------------ MFMA path
constexpr int kMfmaWaves = 8;

template <int MT, int SPW, bool I8>
__global__ __launch_bounds__(512) void k_gemm_mfma(GemmArgs a) {
  constexpr int TLD = 64;  // tile columns (activation rows)
  constexpr int NW = kMfmaWaves;
  __shared__ float red[NW][16 * TLD];
  __shared__ float tile[16 * TLD];
  __shared__ float s_inv[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int n0 = a.row0 + blockIdx.x * 16;
  const int n = n0 + i;
  const int M = a.M;
  const int nsteps = a.K / 128;

  float ssr[kSsRegs];
  int ss_per_lane = 0;
  if (a.ss_in) ss_prefetch(a, wave, NW, ssr, ss_per_lane);

  const int passes = (M + 16 * MT - 1) / (16 * MT);
  for (int pass = 0; pass < passes; ++pass) {
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int st0 = wave; st0 < nsteps; st0 += NW * SPW) {
      // ---- issue every load of this group of steps
      uint4 wr[SPW][4];
      uint4 bh[SPW][MT][4], bl[SPW][MT][4];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int st = st0 + NW * j;
        const bool ok = st < nsteps;
        const int kb = st * 128 + 8 * q;  // piece s of this lane: [kb + 32 s, +8)
        if (!I8) {
          const uint16_t* p = reinterpret_cast<const uint16_t*>(a.W) + (size_t)n * a.K + kb;
#pragma unroll
          for (int s = 0; s < 4; ++s)
            wr[j][s] = ok ? *reinterpret_cast<const uint4*>(p + 32 * s) : make_uint4(0, 0, 0, 0);
        } else {
          const int8_t* p = reinterpret_cast<const int8_t*>(a.W) + (size_t)n * a.K + kb;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint2 v = ok ? *reinterpret_cast<const uint2*>(p + 32 * s) : make_uint2(0, 0);
            wr[j][s] = make_uint4(v.x, v.y, 0, 0);
          }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int m = (pass * MT + t) * 16 + i;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            uint4 h = make_uint4(0, 0, 0, 0), l = make_uint4(0, 0, 0, 0);
            if (ok && m < M) {
              const size_t off = (size_t)m * a.act_ld + kb + 32 * s;
              h = *reinterpret_cast<const uint4*>(a.act + off);
              if (a.act_lo) l = *reinterpret_cast<const uint4*>(a.act_lo + off);
            }
            bh[j][t][s] = h;
            bl[j][t][s] = l;
          }
        }
      }
      // ---- multiply
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8 aop;
          if (!I8) {
            aop = __builtin_bit_cast(bf16x8, wr[j][s]);
          } else {
            uint4 c;
            c.x = i8pair_to_bf16x2(wr[j][s].x, 0);
            c.y = i8pair_to_bf16x2(wr[j][s].x, 1);
            c.z = i8pair_to_bf16x2(wr[j][s].y, 0);
            c.w = i8pair_to_bf16x2(wr[j][s].y, 1);
            aop = __builtin_bit_cast(bf16x8, c);
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, __builtin_bit_cast(bf16x8, bh[j][t][s]), acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, __builtin_bit_cast(bf16x8, bl[j][t][s]), acc[t], 0, 0, 0);
          }
        }
      }
    }
    // D layout of a 16x16 tile: lane l, element j -> weight row 4*(l>>4)+j, activation column l&15
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][(4 * q + j) * TLD + (pass * MT + t) * 16 + i] = acc[t][j];
  }
  if (a.ss_in) ss_finish(a, wave, NW, ssr, ss_per_lane, s_inv);
  __syncthreads();
  for (int e = tid; e < 16 * M; e += NW * 64) {
    const int r = e / M, m = e - r * M;
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) s += red[v][r * TLD + m];
    tile[r * TLD + m] = s;
  }
  __syncthreads();
  gemm_epilogue(a, 16, n0, tile, TLD, s_inv);
}

// NI = 16-byte chunks per lane over K (up to K = 6144: 12 bf16, 6 int8).
template <int MP, bool I8>
hipError_t valu_ni(const GemmArgs& a, int ni, hipStream_t s) {
  const dim3 grid(a.nrows / 4);
  switch (ni) {
    case 1: launch_kernel((k_gemm_valu<MP, 1, I8>), grid, dim3(256), s, a); break;
    case 2: launch_kernel((k_gemm_valu<MP, 2, I8>), grid, dim3(256), s, a); break;
    case 3: launch_kernel((k_gemm_valu<MP, 3, I8>), grid, dim3(256), s, a); break;
    case 4: launch_kernel((k_gemm_valu<MP, 4, I8>), grid, dim3(256), s, a); break;
    default:
      if constexpr (I8) {
        launch_kernel((k_gemm_valu<MP, 6, I8>), grid, dim3(256), s, a);
      } else {
        if (ni <= 6)
          launch_kernel((k_gemm_valu<MP, 6, I8>), grid, dim3(256), s, a);
        else
          launch_kernel((k_gemm_valu<MP, 12, I8>), grid, dim3(256), s, a);
      }
      break;
  }
  return hipGetLastError();
}

template <bool I8>
hipError_t gemm_dispatch(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
  if (p.mfma) {
    const dim3 grid(a.nrows / 16), block(64 * kMfmaWaves);
    if (p.mt == 1)
      launch_kernel((k_gemm_mfma<1, 2, I8>), grid, block, s, a);
    else
      launch_kernel((k_gemm_mfma<2, 2, I8>), grid, block, s, a);
    return hipGetLastError();
  }
  return p.mp == 1 ? valu_ni<1, I8>(a, p.ni, s) : valu_ni<2, I8>(a, p.ni, s);
}

}  // namespace

// Launch shape for nrows weight rows, K columns, M activation rows.
GemmPlan plan_gemm(int nrows, int K, int M, bool i8) {
  GemmPlan p{};
  if (M >= 3) {
    p.mfma = true;
    p.mt = M <= 16 ? 1 : 2;
    p.nw = kMfmaWaves;
    p.rows_per_block = 16;
  } else {
    p.mfma = false;
    p.mp = M == 1 ? 1 : 2;
    p.rw = 1;
    const int chunks = (K / (i8 ? 16 : 8) + 63) / 64;  // 16-byte chunks per lane
    p.ni = chunks <= 4 ? chunks : (chunks <= 6 ? 6 : 12);
    p.rows_per_block = 4;
  }
  p.row_blocks = nrows / p.rows_per_block;
  return p;
}

void gemm_kernel_name(const GemmArgs& a, char* buf, int len) {
  const bool i8 = a.scale != nullptr;
  const GemmPlan p = plan_gemm(a.nrows, a.K, a.M, i8);
  if (p.mfma)
    snprintf(buf, len, "k_gemm_mfma<%d,2,%s>", p.mt, i8 ? "true" : "false");
  else
    snprintf(buf, len, "k_gemm_valu<%d,%d,%s>", p.mp, p.ni, i8 ? "true" : "false");
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 64 || a.nrows <= 0 || (a.nrows % 64) || (a.K % 512) ||
      (a.epi == EPI_SWIGLU && (a.row0 & 1)))
    return hipErrorInvalidValue;
  const bool i8 = a.scale != nullptr;
  const GemmPlan p = plan_gemm(a.nrows, a.K, a.M, i8);
  if (!p.mfma && (a.K / (i8 ? 16 : 8) + 63) / 64 > (i8 ? 6 : 12)) return hipErrorInvalidValue;
  if (a.ss_in && a.ss_in_slots < 1) return hipErrorInvalidValue;
  return i8 ? gemm_dispatch<true>(a, p, s) : gemm_dispatch<false>(a, p, s);
}

}  // namespace qt
