// Weight-streaming GEMMs of the decode frame on gfx950:
//   y[m][n] = sum_k W[n][k] * act[m][k]   (times scale[n] for INT8 weights)
// for M = 1..64 activation rows (sessions, or 2 x sessions at predictor step 1).
//
// Every weight byte is read once per call for all M rows.  A block owns 16
// weight rows over the whole of K; its waves take the K steps round-robin
// (wave w: steps w, w+NW, ...), G steps per load group, and issue all loads of a
// group before any arithmetic.  The waves' partial sums are added in a fixed
// order through LDS, so results do not depend on timing, and no block waits on
// another block.
//
// Memory layouts (see qt_internal.h) make every load a contiguous piece:
//  * weights are packed in 1 KB tiles holding exactly the 16x32 A operand of a
//    v_mfma_f32_16x16x32_bf16 (bf16) or of two of them (int8), so one wave load
//    instruction reads 1 KB of contiguous memory;
//  * activations are "chunked", [K/8][rows][8], so the 16 rows of an 8-wide K
//    chunk that one MFMA B operand needs are 256 contiguous bytes.
// Lane (i, q) (i = lane & 15, q = lane >> 4) holds weight row i, K elements
// [8q, 8q+8) of each 32-wide step.
//  * MFMA form (M >= 3): the activation rows are the 16-column B operand tiles.
//  * VALU form (M <= 2): each lane forms v_dot2_f32_bf16 products of its weight
//    piece with the (broadcast) activation piece of the same K range; the four
//    lanes of a row are summed with cross-lane adds.
//
// Activations are a bf16 hi/lo pair (hi + lo carries ~16 bits of the fp32 value),
// each multiplied by the weights.  RMSNorm is split between producer and consumer:
// the GEMM (or kernel) that writes a residual row v also writes hi/lo(v * gain)
// and the 16-row block's sum of squares; the consuming GEMM multiplies its
// outputs by 1/rms from those sums.
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

// Eight values to chunked hi/lo bf16 pieces (16 bytes each).
__device__ __forceinline__ void split8(const float (&v)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint16_t h0 = f2bf(v[2 * p]), h1 = f2bf(v[2 * p + 1]);
    const uint16_t l0 = f2bf(v[2 * p] - bf2f(h0)), l1 = f2bf(v[2 * p + 1] - bf2f(h1));
    h[p] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[p] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Operands of the epilogue that live in memory, loaded at kernel start so that
// their latency overlaps the main loads: the residual values this thread adds to
// (elements e = tid + k*nthr of the 16 x M tile, e -> (m = e/16, r = e%16)), the
// INT8 scale of row n0 + tid%16 and the next norm's gains of the block's columns.
constexpr int kMaxResid = 2;  // 16 * 64 tile elements over >= 512 threads
struct EpiPrefetch {
  float x[kMaxResid];
  float scale;
  float gain;  // column c0 + tid (tid < 16)
};

__device__ __forceinline__ void epi_prefetch(const GemmArgs& a, int n0, EpiPrefetch& p) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int M = a.M;
#pragma unroll
  for (int k = 0; k < kMaxResid; ++k) {
    const int e = tid + k * nthr;
    p.x[k] = (a.epi == EPI_RESID && e < kGemmRows * M)
                 ? a.out_f32[(size_t)(e >> 4) * a.out_ld + n0 + (e & 15)]
                 : 0.f;
  }
  p.scale = a.scale ? a.scale[n0 + (tid & 15)] : 1.f;
  const int base = a.epi == EPI_RESID ? 0 : a.n_logits;
  p.gain = (a.u_gain && (a.epi == EPI_RESID || a.epi == EPI_HEAD) && n0 >= base && tid < kGemmRows)
               ? bf2f(a.u_gain[n0 - base + tid])
               : 0.f;
}

// Epilogue over the block's tile: tile[r * tld + m] is weight row n0 + r (r < 16),
// activation row m, before the INT8 scale and the RMSNorm factor.  s_gain: LDS
// copy of the prefetched gains.
__device__ void gemm_epilogue(const GemmArgs& a, int n0, float* tile, int tld,
                              const float* s_inv, const EpiPrefetch& pf, const float* s_gain) {
  constexpr int R = kGemmRows;
  const int M = a.M;
  const int tid = threadIdx.x, nthr = blockDim.x;
  if (a.scale || a.ss_in) {
    for (int e = tid; e < R * M; e += nthr) {
      const int m = e >> 4, r = e & 15;
      float y = tile[r * tld + m] * pf.scale;
      if (a.ss_in) y *= s_inv[m];
      tile[r * tld + m] = y;
    }
    __syncthreads();
  }
  if (a.epi == EPI_STORE) {
    for (int e = tid; e < R * M; e += nthr) {
      const int m = e >> 4, r = e & 15;
      a.out_f32[(size_t)m * a.out_ld + n0 + r] = tile[r * tld + m];
    }
    return;
  }
  if (a.epi == EPI_SWIGLU) {
    // rows 2p (gate) and 2p+1 (up) -> output column n0/2 + p: one 8-wide chunk per m
    for (int m = tid; m < M; m += nthr) {
      float v[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) v[p] = silu(tile[(2 * p) * tld + m]) * tile[(2 * p + 1) * tld + m];
      uint4 hi, lo;
      split8(v, hi, lo);
      const size_t o = chunked(m, n0 >> 1, a.u_ld);
      *reinterpret_cast<uint4*>(a.u_hi + o) = hi;
      *reinterpret_cast<uint4*>(a.u_lo + o) = lo;
    }
    return;
  }
  if (a.epi == EPI_HEAD && n0 < a.n_logits) {
    for (int e = tid; e < R * M; e += nthr) {
      const int m = e >> 4, r = e & 15;
      a.logits[(size_t)m * a.logits_ld + n0 + r] = tile[r * tld + m];
    }
    if (n0 < a.argmax_range) {
      // greedy-key candidate of these 16 rows (lowest index wins ties; NaN flagged)
      for (int m = tid; m < M; m += nthr) {
        unsigned long long best = 0;
        bool nan = false;
        for (int r = 0; r < R && n0 + r < a.argmax_range; ++r) {
          const float y = tile[r * tld + m];
          if (y != y) {
            nan = true;
            continue;
          }
          const unsigned long long k = greedy_key(y, n0 + r);
          best = k > best ? k : best;
        }
        a.cand[(size_t)m * a.cand_ld + n0 / kKeyBlock] = best;
        if (nan) atomicOr(a.status, QT_STATUS_NAN);
      }
    }
    return;
  }
  // residual rows (EPI_RESID: x += y) or projection rows (EPI_HEAD: x = y)
  const int base = a.epi == EPI_RESID ? 0 : a.n_logits;
  const int c0 = n0 - base;
#pragma unroll
  for (int k = 0; k < kMaxResid; ++k) {
    const int e = tid + k * nthr;
    if (e >= R * M) break;
    const int m = e >> 4, r = e & 15;
    float v = tile[r * tld + m];
    if (a.epi == EPI_RESID) v += pf.x[k];
    a.out_f32[(size_t)m * a.out_ld + c0 + r] = v;
    tile[r * tld + m] = v;
  }
  if (!a.u_gain) return;
  __syncthreads();
  // the next norm's input (two 8-wide chunks) and this block's sum of squares
  for (int m = tid; m < M; m += nthr) {
    float ss = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = tile[(8 * h + j) * tld + m];
        ss = fmaf(x, x, ss);
        v[j] = x * s_gain[8 * h + j];
      }
      uint4 hi, lo;
      split8(v, hi, lo);
      const size_t o = chunked(m, c0 + 8 * h, a.u_ld);
      *reinterpret_cast<uint4*>(a.u_hi + o) = hi;
      *reinterpret_cast<uint4*>(a.u_lo + o) = lo;
    }
    a.ss_out[(size_t)(c0 / R) * a.ss_out_ld + m] = ss;
  }
}

// Eight int8 weights (bytes 8*sb .. 8*sb+7 of w) as a bf16x8 operand (exact).
__device__ __forceinline__ uint4 i8_to_bf16x8(const uint4& w, int sb) {
  const uint32_t a = sb ? w.z : w.x, b = sb ? w.w : w.y;
  return make_uint4(i8pair_to_bf16x2(a, 0), i8pair_to_bf16x2(a, 1), i8pair_to_bf16x2(b, 0),
                    i8pair_to_bf16x2(b, 1));
}

// One block: weight rows [n0, n0+16) over all of K.  NW waves, MT 16-row MFMA
// activation tiles (MT == 0: VALU form for M <= 2), G K steps per load group.
template <int NW, int MT, int G, bool I8>
__global__ __launch_bounds__(NW * 64) void k_gemm(GemmArgs a) {
  constexpr int TLD = MT ? 16 * MT : 2;  // tile columns (activation rows)
  constexpr int SUB = I8 ? 2 : 1;        // 32-wide MFMA K substeps per packed K step
  constexpr int MV = MT ? 16 * MT : 2;   // activation rows held per lane group
  __shared__ float red[NW][kGemmRows * TLD];
  __shared__ float s_inv[64];
  __shared__ float s_gain[kGemmRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int rt = (a.row0 >> 4) + blockIdx.x;
  const int n0 = rt * kGemmRows;
  const int M = a.M, ld = a.act_ld;
  const int ksteps = a.K / (32 * SUB);
  const uint4* W = reinterpret_cast<const uint4*>(a.W) + (size_t)rt * ksteps * 64 + lane;
  const uint4* H = reinterpret_cast<const uint4*>(a.act);
  const uint4* L = reinterpret_cast<const uint4*>(a.act_lo);
  const bool has_lo = a.act_lo != nullptr;

  float ssr[kSsRegs];
  int ss_per_lane = 0;
  if (a.ss_in) ss_prefetch(a, wave, NW, ssr, ss_per_lane);
  EpiPrefetch pf;
  epi_prefetch(a, n0, pf);

  // activation row m of chunk c: 16 bytes at H[c * ld + m]
  if constexpr (MT > 0) {
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = wave; j0 < ksteps; j0 += NW * G) {
      uint4 w[G], h[G][SUB][MT], l[G][SUB][MT];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int j = j0 + NW * g;
        const bool ok = j < ksteps;
        w[g] = ok ? W[(size_t)j * 64] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          const size_t c = (size_t)(j * SUB + sb) * 4 + q;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const int m = 16 * t + i;
            const bool in = ok && m < M;
            h[g][sb][t] = in ? H[c * ld + m] : make_uint4(0, 0, 0, 0);
            l[g][sb][t] = in && has_lo ? L[c * ld + m] : make_uint4(0, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          const bf16x8 A = __builtin_bit_cast(bf16x8, I8 ? i8_to_bf16x8(w[g], sb) : w[g]);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                A, __builtin_bit_cast(bf16x8, h[g][sb][t]), acc[t], 0, 0, 0);
            if (has_lo)
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  A, __builtin_bit_cast(bf16x8, l[g][sb][t]), acc[t], 0, 0, 0);
          }
        }
      }
    }
    // D layout of a 16x16 tile: lane l, element e -> weight row 4*(l>>4)+e, column l&15
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][(4 * q + e) * TLD + 16 * t + i] = acc[t][e];
  } else {
    float acc[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) acc[m] = 0.f;
    for (int j0 = wave; j0 < ksteps; j0 += NW * G) {
      uint4 w[G], h[G][SUB][MV], l[G][SUB][MV];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int j = j0 + NW * g;
        const bool ok = j < ksteps;
        w[g] = ok ? W[(size_t)j * 64] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          const size_t c = (size_t)(j * SUB + sb) * 4 + q;
#pragma unroll
          for (int m = 0; m < MV; ++m) {
            const bool in = ok && m < M;
            h[g][sb][m] = in ? H[c * ld + m] : make_uint4(0, 0, 0, 0);
            l[g][sb][m] = in && has_lo ? L[c * ld + m] : make_uint4(0, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          const uint4 A = I8 ? i8_to_bf16x8(w[g], sb) : w[g];
#pragma unroll
          for (int m = 0; m < MV; ++m) acc[m] = dot8(A, l[g][sb][m], dot8(A, h[g][sb][m], acc[m]));
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      float v = acc[m];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (q == 0) red[wave][i * TLD + m] = v;
    }
  }
  if (a.ss_in) ss_finish(a, wave, NW, ssr, ss_per_lane, s_inv);
  if (tid < kGemmRows) s_gain[tid] = pf.gain;
  __syncthreads();
  for (int e = tid; e < kGemmRows * M; e += NW * 64) {
    const int m = e >> 4, r = e & 15;
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) s += red[v][r * TLD + m];
    red[0][r * TLD + m] = s;
  }
  __syncthreads();
  gemm_epilogue(a, n0, red[0], TLD, s_inv, pf, s_gain);
}

template <bool I8>
hipError_t gemm_dispatch(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
  const dim3 grid(p.row_blocks), block(64 * p.nw);
  switch (p.mt) {
    case 0: launch_kernel((k_gemm<16, 0, 2, I8>), grid, block, s, a); break;
    case 1: launch_kernel((k_gemm<8, 1, 2, I8>), grid, block, s, a); break;
    case 2: launch_kernel((k_gemm<8, 2, 2, I8>), grid, block, s, a); break;
    default: launch_kernel((k_gemm<8, 4, 1, I8>), grid, block, s, a); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ packing
// Source rows [rows][K] bf16 -> rows row0 + r*step of a tiled [N][K] matrix.
__global__ __launch_bounds__(256) void k_pack_tiled(const uint16_t* src, int rows, int K,
                                                    uint16_t* dst, int row0, int step) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;  // one 8-wide chunk
  const int kc = K >> 3;
  if (e >= (long long)rows * kc) return;
  const int r = (int)(e / kc), k = (int)(e - (long long)r * kc) << 3;
  const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)r * K + k);
  *reinterpret_cast<uint4*>(dst + tiled_bf16(row0 + r * step, k, K)) = v;
}

// Rows row0 + r*step of a tiled int8 [N][K] matrix -> row-major [rows][K].
__global__ __launch_bounds__(256) void k_untile_i8(const int8_t* tiled, int rows, int K, int row0,
                                                   int step, int8_t* out) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int kc = K >> 3;
  if (e >= (long long)rows * kc) return;
  const int r = (int)(e / kc), k = (int)(e - (long long)r * kc) << 3;
  const uint2 v = *reinterpret_cast<const uint2*>(tiled + tiled_i8(row0 + r * step, k, K));
  *reinterpret_cast<uint2*>(out + (size_t)r * K + k) = v;
}

}  // namespace

// Launch shape for nrows weight rows, K columns, M activation rows.
GemmPlan plan_gemm(int nrows, int K, int M, bool i8) {
  (void)K;
  (void)i8;
  GemmPlan p{};
  if (M <= 2) {
    p.nw = 16, p.mt = 0, p.g = 2;
  } else if (M <= 16) {
    p.nw = 8, p.mt = 1, p.g = 2;
  } else if (M <= 32) {
    p.nw = 8, p.mt = 2, p.g = 2;
  } else {
    p.nw = 8, p.mt = 4, p.g = 1;
  }
  p.rows_per_block = kGemmRows;
  p.row_blocks = nrows / kGemmRows;
  return p;
}

void gemm_kernel_name(const GemmArgs& a, char* buf, int len) {
  const bool i8 = a.scale != nullptr;
  const GemmPlan p = plan_gemm(a.nrows, a.K, a.M, i8);
  snprintf(buf, len, "k_gemm<%d,%d,%d,%s>", p.nw, p.mt, p.g, i8 ? "true" : "false");
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 64 || a.nrows <= 0 || (a.nrows % kGemmRows) || (a.row0 % kGemmRows) ||
      a.row0 + a.nrows > a.N || a.K <= 0 || (a.K % 64) || a.act_ld < a.M)
    return hipErrorInvalidValue;
  if (a.ss_in && a.ss_in_slots < 1) return hipErrorInvalidValue;
  if (a.epi == EPI_HEAD && ((a.n_logits % kGemmRows) || (a.argmax_range > a.n_logits)))
    return hipErrorInvalidValue;
  if ((a.epi == EPI_RESID || a.epi == EPI_HEAD) && a.u_gain && !a.ss_out) return hipErrorInvalidValue;
  const bool i8 = a.scale != nullptr;
  const GemmPlan p = plan_gemm(a.nrows, a.K, a.M, i8);
  return i8 ? gemm_dispatch<true>(a, p, s) : gemm_dispatch<false>(a, p, s);
}

hipError_t launch_pack_tiled(const uint16_t* src, int rows, int K, uint16_t* dst, int row0,
                             int step, hipStream_t s) {
  if (rows <= 0 || K <= 0 || (K % 32) || row0 < 0 || step < 1) return hipErrorInvalidValue;
  const long long n = (long long)rows * (K / 8);
  launch_kernel(k_pack_tiled, dim3((unsigned)((n + 255) / 256)), dim3(256), s, src, rows, K, dst,
                row0, step);
  return hipGetLastError();
}

hipError_t launch_untile_i8(const int8_t* tiled, int rows, int K, int row0, int step, int8_t* out,
                            hipStream_t s) {
  if (rows <= 0 || K <= 0 || (K % 64) || row0 < 0 || step < 1) return hipErrorInvalidValue;
  const long long n = (long long)rows * (K / 8);
  launch_kernel(k_untile_i8, dim3((unsigned)((n + 255) / 256)), dim3(256), s, tiled, rows, K, row0,
                step, out);
  return hipGetLastError();
}

}  // namespace qt
