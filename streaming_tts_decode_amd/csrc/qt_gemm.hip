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
//    v_mfma_f32_16x16x32_f16 (half) or of two of them (int8), so one wave load
//    instruction reads 1 KB of contiguous memory;
//  * activations are "chunked", [K/8][rows][8], so the 16 rows of an 8-wide K
//    chunk that one MFMA B operand needs are 256 contiguous bytes.
// Lane (i, q) (i = lane & 15, q = lane >> 4) holds weight row i, K elements
// [8q, 8q+8) of each 32-wide step.
//  * MFMA form (M >= 3): the activation rows are the 16-column B operand tiles.
//  * VALU form (M <= 2): each lane forms v_dot2_f32_f16 products of its weight
//    piece with the (broadcast) activation piece of the same K range; the four
//    lanes of a row are summed with cross-lane adds.
//
// Activations and packed weights are IEEE half, accumulation fp32.  RMSNorm is
// split between producer and consumer: the GEMM (or kernel) that writes a
// residual row v also writes half(v * gain) and the 16-row block's sum of
// squares; the consuming GEMM multiplies its outputs by 1/rms from those sums.
#include <stdio.h>

#include "qt_device.h"
#include "qt_internal.h"

namespace qt {
namespace {
using namespace dev;

// ---- RMSNorm statistics of the input rows (consumer side)
// The producer of x left per-16-column sums of squares in ss_in[slot][m]
// (slot < ss_in_slots).  Thread t of the block handles row m = t % MP and slots
// g, g + G, ... with g = t / MP, G = NTHR / MP, where MP is the block's padded
// row count: a constant, so the mapping costs no division (rows m >= M load
// nothing).  The loads are coalesced over m and issued before the main loads;
// after the main loop the G partials of a row are added in a fixed order.
template <int MP, int NTHR>
struct SsPrefetch {
  static constexpr int G = NTHR / MP;
  static constexpr int PER = (128 + G - 1) / G;  // slots per thread held in registers
  float v[PER];
};

template <int MP, int NTHR>
__device__ __forceinline__ void ss_prefetch(const GemmArgs& a, SsPrefetch<MP, NTHR>& p) {
  using S = SsPrefetch<MP, NTHR>;
  const int tid = threadIdx.x, g = tid / MP, m = tid % MP;
  const bool on = m < a.M;
#pragma unroll
  for (int k = 0; k < S::PER; ++k) {
    const int slot = g + k * S::G;
    p.v[k] = (on && slot < a.ss_in_slots) ? a.ss_in[(size_t)slot * a.ss_in_ld + m] : 0.f;
  }
}

// Partial of this thread (slots beyond the registered ones are loaded now).
template <int MP, int NTHR>
__device__ __forceinline__ float ss_partial(const GemmArgs& a, const SsPrefetch<MP, NTHR>& p) {
  using S = SsPrefetch<MP, NTHR>;
  const int tid = threadIdx.x, g = tid / MP, m = tid % MP;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < S::PER; ++k) s += p.v[k];
  if (m < a.M)
    for (int slot = g + S::PER * S::G; slot < a.ss_in_slots; slot += S::G)
      s += a.ss_in[(size_t)slot * a.ss_in_ld + m];
  return s;
}

// 16-byte weight load: non-temporal for matrices streamed once per frame, a
// plain (cached) load for matrices that later steps of the frame read again
// (the predictor's layers fit in the memory-side cache and stay there).
template <bool KEEP>
__device__ __forceinline__ uint4 load_w(const uint4* p) {
  return KEEP ? *p : load_nt(p);
}

// Operands of the epilogue that live in memory, loaded at kernel start so that
// their latency overlaps the main loads.  Epilogue thread mapping: element
// e = tid + k*nthr of the 16 x M tile is row r = e % 16, activation row m = e / 16
// (so r = tid % 16 for every k): the residual value it adds to, the INT8 scale of
// its row and the next norm's gain of its column.
constexpr int kMaxElem = 2;  // 16 * 64 tile elements over >= 512 threads
struct EpiPrefetch {
  float x[kMaxElem];
  float scale;
  uint32_t gain_bits;  // raw bfloat16: converted at use, so no wait is forced here
};

__device__ __forceinline__ void epi_prefetch(const GemmArgs& a, int nthr, int n0, int rows,
                                             EpiPrefetch& p) {
  const int tid = threadIdx.x;
  const int M = a.M, r = tid & 15;
#pragma unroll
  for (int k = 0; k < kMaxElem; ++k) {
    const int e = tid + k * nthr;
    p.x[k] = (a.epi == EPI_RESID && e < kGemmRows * M)
                 ? a.out_f32[(size_t)(e >> 4) * a.out_ld + n0 + r]
                 : 0.f;
  }
  p.scale = a.scale ? a.scale[n0 + tid % rows] : 1.f;  // row tid % rows of the block
  const int base = a.epi == EPI_RESID ? 0 : a.n_logits;
  p.gain_bits = (a.u_gain && (a.epi == EPI_RESID || a.epi == EPI_HEAD) && n0 >= base)
                    ? (uint32_t)a.u_gain[n0 - base + r]
                    : 0u;
}

// Epilogue, one thread per output element.  y(r, m): the block's finished value
// of weight row n0 + r for activation row m (waves summed in order, INT8 scale and
// RMSNorm factor applied).  s_scale: the 16 rows' scales (for SwiGLU, whose
// threads need two rows).  TLD: row stride of the partial tiles in LDS, odd so
// that the 16 rows a thread group reads fall in distinct banks.
// s_ssp: the statistics partials ([SG][MV], summed here per row when SG <= 32, so
// that no second barrier is needed); s_inv: the rows' norm factors otherwise.
template <int NW, int TLD, int R, int MV, int SG>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, int n0,
                                              const float (*red)[kGemmRows * R * TLD],
                                              const float* s_inv, const float* s_ssp,
                                              const float* s_scale, const EpiPrefetch& pf) {
  const int M = a.M;
  const int tid = threadIdx.x;
  constexpr int nthr = NW * 64;
  auto inv_row = [&](int m) -> float {
    if (!a.ss_in) return 1.f;
    if constexpr (SG <= 32) {
      float ss = 0.f;
#pragma unroll
      for (int g = 0; g < SG; ++g) ss += s_ssp[g * MV + m];
      return 1.0f / sqrtf(ss / (float)a.K + a.norm_eps);
    } else {
      return s_inv[m];
    }
  };
  auto y = [&](int r, int m, float inv) -> float {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w][r * TLD + m];
    if (a.scale) v *= s_scale[r];
    if (a.ss_in) v *= inv;
    return v;
  };
  bool over = false;  // a half input out of range (QT_STATUS_FP16_RANGE)
  if (a.epi == EPI_SWIGLU) {
    // rows 2p (gate) and 2p+1 (up) of the block's 16R -> output column n0/2 + p
    for (int e = tid; e < 8 * R * M; e += nthr) {
      const int m = e / (8 * R), p = e - m * (8 * R);
      const float inv = inv_row(m);
      const float v = silu(y(2 * p, m, inv)) * y(2 * p + 1, m, inv);
      a.u[chunked(m, (n0 >> 1) + p, a.u_ld)] = f2h_chk(v, over);
    }
    if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
    return;
  }
  const bool logits = a.epi == EPI_HEAD && n0 < a.n_logits;
  const int base = a.epi == EPI_RESID ? 0 : a.n_logits;
  const int c0 = n0 - base;
#pragma unroll
  for (int k = 0; k < kMaxElem; ++k) {
    const int e = tid + k * nthr;
    if (e >= kGemmRows * M) break;  // whole 16-lane groups leave together
    const int m = e >> 4, r = e & 15;
    float v = y(r, m, inv_row(m));
    if (a.epi == EPI_STORE) {
      a.out_f32[(size_t)m * a.out_ld + n0 + r] = v;
    } else if (logits) {
      a.logits[(size_t)m * a.logits_ld + n0 + r] = v;
      if (n0 < a.argmax_range) {
        // greedy-key candidate of the 16 rows (lowest index wins ties; NaN flagged)
        const bool valid = n0 + r < a.argmax_range;
        const bool nan = valid && v != v;
        unsigned long long key = (valid && !nan) ? greedy_key(v, n0 + r) : 0ull;
        key = row_max16_u64(key);
        if (nan) atomicOr(a.status, QT_STATUS_NAN);
        if (r == 0) a.cand[(size_t)m * a.cand_ld + n0 / kKeyBlock] = key;
      }
    } else {
      // residual rows (EPI_RESID: x += y) or projection rows (EPI_HEAD: x = y), then
      // the next norm's input and the 16 columns' sum of squares
      if (a.epi == EPI_RESID) v += pf.x[k];
      a.out_f32[(size_t)m * a.out_ld + c0 + r] = v;
      if (a.u_gain) {
        // the conversion stays here: folded into the prefetch's branch it would make
        // the kernel wait for that load before its main loop
        uint32_t gb = pf.gain_bits;
        asm volatile("" : "+v"(gb));
        a.u[chunked(m, c0 + r, a.u_ld)] = f2h_chk(v * bf2f((uint16_t)gb), over);
        const float ss = row_sum16(v * v);
        if (r == 0) a.ss_out[(size_t)(c0 / kGemmRows) * a.ss_out_ld + m] = ss;
      }
    }
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
}

// Eight int8 weights (bytes 8*sb .. 8*sb+7 of w) as a half x 8 operand (exact).
__device__ __forceinline__ uint4 i8_to_f16x8(const uint4& w, int sb) {
  const uint32_t a = sb ? w.z : w.x, b = sb ? w.w : w.y;
  return make_uint4(i8pair_to_f16x2(a, 0), i8pair_to_f16x2(a, 1), i8pair_to_f16x2(b, 0),
                    i8pair_to_f16x2(b, 1));
}

// Every kernel argument is a scalar load, and the compiler issues each one where
// its value is first needed, often inside a branch: the prologue became a chain
// of five or six dependent round trips before the first weight load.  Taking
// every field through an empty asm at entry issues the loads together and waits
// for them once.
__device__ __forceinline__ void fetch_args(const GemmArgs& a, int msplit) {
  asm volatile("" ::"s"(a.W), "s"(a.scale), "s"(a.act), "s"(a.ss_in), "s"(a.out_f32),
               "s"(a.logits), "s"(a.cand), "s"(a.status), "s"(a.u_gain), "s"(a.u),
               "s"(a.ss_out), "s"(msplit));
  asm volatile("" ::"s"(a.N), "s"(a.K), "s"(a.row0), "s"(a.nrows), "s"(a.act_ld), "s"(a.M),
               "s"(a.ss_in_ld), "s"(a.ss_in_slots), "s"(a.norm_eps), "s"(a.epi), "s"(a.out_ld),
               "s"(a.logits_ld), "s"(a.n_logits), "s"(a.argmax_range), "s"(a.cand_ld),
               "s"(a.u_ld), "s"(a.ss_out_ld), "s"(a.keep_w));
}

// One block: weight rows [n0, n0+16) over all of K.  NW waves, MT 16-row MFMA
// activation tiles (MT == 0: VALU form for M <= 2), G K steps per load group.
template <int NW, int MT, int G, bool I8, bool KEEP, int R>
__global__ __launch_bounds__(NW * 64) void k_gemm(GemmArgs args_in, int msplit) {
  const GemmArgs& args = args_in;
  fetch_args(args, msplit);
  constexpr int TLD = (MT ? 16 * MT : 2) + 1;  // tile row stride: activation rows + 1 (odd)
  constexpr int SUB = I8 ? 2 : 1;        // 32-wide MFMA K substeps per packed K step
  constexpr int MV = MT ? 16 * MT : 2;   // activation rows held per lane group
  __shared__ float red[NW][kGemmRows * R * TLD];
  __shared__ float s_ssp[NW * 64];
  __shared__ float s_inv[64];
  __shared__ float s_scale[kGemmRows * R];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  // block -> (weight tile, activation-row part).  With msplit > 1, blocks b and
  // b + 8, b + 16, ... (the same XCD under round-robin dispatch) share a tile.
  int rtl = blockIdx.x, mh = 0;
  if (msplit > 1) {  // (a power of two)
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3, sh = __builtin_ctz(msplit);
    mh = slot & (msplit - 1);
    rtl = (slot >> sh) * 8 + x;
  }
  // this block's rows m0 .. m0 + M-1 of the activations, as a shifted view
  GemmArgs a = args;
  {
    const int m0 = mh * (MT ? 16 * MT : 2);
    a.M = min(args.M - m0, MT ? 16 * MT : 2);
    const size_t c8 = (size_t)m0 * 8;
    a.act += c8;
    if (a.ss_in) a.ss_in += m0;
    a.out_f32 += (size_t)m0 * a.out_ld;
    if (a.logits) a.logits += (size_t)m0 * a.logits_ld;
    if (a.cand) a.cand += (size_t)m0 * a.cand_ld;
    if (a.u) a.u += c8;
    if (a.ss_out) a.ss_out += m0;
  }
  if (a.M <= 0) return;  // (plan_gemm never makes an empty part; whole block leaves)
  const int rt = (a.row0 >> 4) + rtl * R;  // first of the block's R row tiles
  const int n0 = rt * kGemmRows;
  const int M = a.M, ld = a.act_ld;
  const int ksteps = a.K / (32 * SUB);
  const uint4* W = reinterpret_cast<const uint4*>(a.W) + (size_t)rt * ksteps * 64 + lane;
  const uint4* H = reinterpret_cast<const uint4*>(a.act);

  SsPrefetch<MV, NW * 64> ssp;
  if (a.ss_in) ss_prefetch(a, ssp);
  EpiPrefetch pf;
  epi_prefetch(a, NW * 64, n0, kGemmRows * R, pf);

  // activation row m of chunk c: 16 bytes at H[c * ld + m]
  if constexpr (MT > 0) {
    f32x4 acc[R][MT];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[rr][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = wave; j0 < ksteps; j0 += NW * G) {
      uint4 w[G][R], h[G][SUB][MT];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int j = j0 + NW * g;
        const bool ok = j < ksteps;
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
          w[g][rr] = ok ? load_w<KEEP>(W + ((size_t)rr * ksteps + j) * 64) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          const size_t c = (size_t)(j * SUB + sb) * 4 + q;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const int m = 16 * t + i;
            h[g][sb][t] = ok && m < M ? H[c * ld + m] : make_uint4(0, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
#pragma unroll
          for (int rr = 0; rr < R; ++rr) {
            const f16x8 A = __builtin_bit_cast(f16x8, I8 ? i8_to_f16x8(w[g][rr], sb) : w[g][rr]);
#pragma unroll
            for (int t = 0; t < MT; ++t)
              acc[rr][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  A, __builtin_bit_cast(f16x8, h[g][sb][t]), acc[rr][t], 0, 0, 0);
          }
        }
      }
    }
    // D layout of a 16x16 tile: lane l, element e -> weight row 4*(l>>4)+e, column l&15
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[wave][(16 * rr + 4 * q + e) * TLD + 16 * t + i] = acc[rr][t][e];
  } else {
    float acc[R][MV];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int m = 0; m < MV; ++m) acc[rr][m] = 0.f;
    for (int j0 = wave; j0 < ksteps; j0 += NW * G) {
      uint4 w[G][R], h[G][SUB][MV];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int j = j0 + NW * g;
        const bool ok = j < ksteps;
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
          w[g][rr] = ok ? load_w<KEEP>(W + ((size_t)rr * ksteps + j) * 64) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          const size_t c = (size_t)(j * SUB + sb) * 4 + q;
#pragma unroll
          for (int m = 0; m < MV; ++m)
            h[g][sb][m] = ok && m < M ? H[c * ld + m] : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
#pragma unroll
          for (int rr = 0; rr < R; ++rr) {
            const uint4 A = I8 ? i8_to_f16x8(w[g][rr], sb) : w[g][rr];
#pragma unroll
            for (int m = 0; m < MV; ++m) acc[rr][m] = dot8h(A, h[g][sb][m], acc[rr][m]);
          }
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        const float v = sum_q4(acc[rr][m]);
        if (q == 0) red[wave][(16 * rr + i) * TLD + m] = v;
      }
  }
  if (a.ss_in) s_ssp[tid] = ss_partial(a, ssp);
  if (tid < kGemmRows * R) s_scale[tid] = pf.scale;
  __syncthreads();
  // row m's SG statistics partials are summed in a fixed order: few of them (many
  // rows) by every epilogue thread of the row itself, else by a wave (tree sum
  // over its lanes) before a second barrier
  constexpr int SG = SsPrefetch<MV, NW * 64>::G;
  if constexpr (SG > 32) {
    if (a.ss_in) {
      for (int m = wave; m < M; m += NW) {
        float ss = 0.f;
        for (int g = lane; g < SG; g += 64) ss += s_ssp[g * MV + m];
        ss = wave_sum(ss);
        if (lane == 0) s_inv[m] = 1.0f / sqrtf(ss / (float)a.K + a.norm_eps);
      }
      __syncthreads();
    }
  }
  gemm_epilogue<NW, TLD, R, MV, SG>(a, n0, red, s_inv, s_ssp, s_scale, pf);
}

template <bool I8, bool KEEP>
hipError_t gemm_dispatch(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
  const dim3 grid(p.row_blocks * p.msplit), block(64 * p.nw);
  const int ms = p.msplit;
  // (the group sizes here and in plan_gemm agree)
  if (p.tiles == 3) {  // (streamed matrices only)
    if constexpr (KEEP) {
      return hipErrorInvalidConfiguration;
    } else {
      switch (p.mt) {
        case 0: launch_kernel((k_gemm<16, 0, 2, I8, false, 3>), grid, block, s, a, ms); break;
        case 1: launch_kernel((k_gemm<8, 1, 4, I8, false, 3>), grid, block, s, a, ms); break;
        case 2: launch_kernel((k_gemm<8, 2, 2, I8, false, 3>), grid, block, s, a, ms); break;
        default: return hipErrorInvalidConfiguration;
      }
      return hipGetLastError();
    }
  }
  switch (p.mt) {
    case 0: launch_kernel((k_gemm<16, 0, 2, I8, KEEP, 1>), grid, block, s, a, ms); break;
    case 1: launch_kernel((k_gemm<8, 1, 8, I8, KEEP, 1>), grid, block, s, a, ms); break;
    case 2: launch_kernel((k_gemm<8, 2, KEEP ? 4 : 2, I8, KEEP, 1>), grid, block, s, a, ms); break;
    default: launch_kernel((k_gemm<8, 4, KEEP ? 2 : 1, I8, KEEP, 1>), grid, block, s, a, ms); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ many-row GEMM
// The same products for M in the hundreds or thousands (a prompt's rows): a block
// computes 128 weight rows x 128 activation rows, each of its four waves a 64 x 64
// quarter as 4 x 4 tiles of v_mfma_f32_16x16x32_f16, reading the weight tiles and
// the chunked activations straight into operand registers (the next K step's
// loads are in flight during this step's products).  Blocks that share weight rows
// run on one XCD (rows_tile), so a weight tile is fetched from memory about once
// and the other row blocks find it in that XCD's L2.  Outputs match the epilogues above:
// EPI_STORE, EPI_RESID (x += y; half(x * gain) and per-16-row sums of squares)
// and EPI_SWIGLU (rows 2p, 2p+1 -> column p), with the INT8 scale and the RMSNorm
// factor 1/sqrt(sum ss / K + eps) of each activation row.
// TN x TM: 16-row weight tiles x 16-row activation tiles per wave (4 x 4, or
// smaller when the big tiles would leave CUs idle); the block's four waves cover
// 2 TN x 2 TM tiles.
// Tile of this block in the many-row forms.  The dispatcher deals consecutive
// blocks round-robin over the eight XCDs, each with its own L2, so blocks whose ids
// agree mod 8 run on one XCD (whichever XCD the first block went to).  Each such
// class takes a contiguous range of tiles, activation blocks fastest: the blocks
// that share a weight tile then share one L2, and a weight tile is fetched from
// memory once rather than once per activation block.  Handing the tiles out in
// launch order instead fetched the gate/up matrix of a 1024-row prompt about 7.5
// times per launch (memory-side counters: 405 MB against 69 MB with this order).
__device__ __forceinline__ void rows_tile(int& mblk, int& nblk) {
  const int nM = gridDim.x, G = gridDim.x * gridDim.y;
  const int id = blockIdx.x + blockIdx.y * nM;
  const int k = id & 7, slot = id >> 3, base = G >> 3, rem = G & 7;
  const int t = k * base + (k < rem ? k : rem) + slot;  // a bijection of [0, G)
  nblk = t / nM;
  mblk = t - nblk * nM;
}

// Norm factors of a block's BM activation rows mb .. mb + BM - 1, the consumer side
// of an RMSNorm: s_inv[r] = 1 / sqrt(sum of row mb + r's ss_in slots / K + eps), or 1
// without a norm.  The slots are [slots][ss_in_ld] floats.  Each of the NT threads
// takes four consecutive rows of every G-th slot (G = NT / (BM / 4)), U slots per
// batch, and issues a batch's loads before adding any, so the sums cost one memory
// round trip per batch rather than one per slot; the G partials are then added in
// order through LDS.  `mid` runs between the first batch's loads and their use
// (the caller's first operand copies, which then fly with them).  Rows past M read
// row M - 1 and count nothing.  Ends with a plain barrier, which waits for no
// memory operation other than the LDS writes of the partials.
template <int BM, int NT, int U, typename Mid>
__device__ __forceinline__ void norm_factors(const GemmArgs& a, int mb, float* s_inv,
                                             float (*s_part)[BM], Mid mid) {
  constexpr int TPS = BM / 4, G = NT / TPS;
  static_assert(NT % TPS == 0, "row groups must divide over the threads");
  const int tid = threadIdx.x;
  if (!a.ss_in) {
    for (int r = tid; r < BM; r += NT) s_inv[r] = 1.f;
    mid();
    return;
  }
  const int g = tid / TPS, c = tid - g * TPS;
  const int m = mb + 4 * c, S = a.ss_in_slots;
  const int mm = min(m, a.M - 4);  // (M is a multiple of 16)
  const bool live = m < a.M;
  float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
  auto batch = [&](float4 (&v)[U], int s0) {
#pragma unroll
    for (int k = 0; k < U; ++k) {  // (slots past the end re-read the last one)
      const int sl = min(s0 + k * G, S - 1);
      v[k] = *reinterpret_cast<const float4*>(a.ss_in + (size_t)sl * a.ss_in_ld + mm);
    }
  };
  auto add = [&](const float4 (&v)[U], int s0) {
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (live && s0 + k * G < S) {
        part.x += v[k].x;
        part.y += v[k].y;
        part.z += v[k].z;
        part.w += v[k].w;
      }
  };
  {
    float4 v[U];
    batch(v, g);
    mid();
    add(v, g);
  }
  for (int s0 = g + U * G; s0 < S; s0 += U * G) {
    float4 v[U];
    batch(v, s0);
    add(v, s0);
  }
  *reinterpret_cast<float4*>(&s_part[g][4 * c]) = part;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  for (int r = tid; r < BM; r += NT) {
    float ss = 0.f;
    for (int q = 0; q < G; ++q) ss += s_part[q][r];
    s_inv[r] = 1.0f / sqrtf(ss / (float)a.K + a.norm_eps);  // (rows past M: unused)
  }
}

template <bool I8, int TN, int TM>
__global__ __launch_bounds__(256) void k_gemm_rows(GemmArgs a) {
  constexpr int SUB = I8 ? 2 : 1;
  constexpr int BM = 32 * TM;  // activation rows per block
  __shared__ float s_inv[BM];
  __shared__ __attribute__((aligned(16))) float s_part[256 / (BM / 4)][BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  int mblk, nblk;
  rows_tile(mblk, nblk);
  const int mb = BM * mblk;
  const int n0 = a.row0 + 32 * TN * nblk + 16 * TN * (wave & 1);
  const int m0 = mb + 16 * TM * (wave >> 1);
  const int M = a.M, ld = a.act_ld;
  const int ksteps = a.K / (32 * SUB);
  norm_factors<BM, 256, 8>(a, mb, s_inv, s_part, [] {});
  const uint4* W = reinterpret_cast<const uint4*>(a.W) + (size_t)(n0 >> 4) * ksteps * 64 + lane;
  const uint4* Hq = reinterpret_cast<const uint4*>(a.act) + (size_t)q * ld;
  bool mrow[TM];
  int hrow[TM];  // rows past M read row M - 1 (their products are never stored)
#pragma unroll
  for (int u = 0; u < TM; ++u) {
    mrow[u] = m0 + 16 * u + i < M;
    hrow[u] = min(m0 + 16 * u + i, M - 1);
  }
  f32x4 acc[TN][TM];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int u = 0; u < TM; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Two register slots: step j + 1's loads are issued before step j's products.
  // Every load is unconditional (the step past the end re-reads the last one), and
  // the slots are used in place rather than copied, so the compiler can count the
  // loads in flight and wait only for step j's: a load under a condition, or a copy
  // of a register still being loaded, made it wait for all of them, which left
  // each step a full memory round trip.
  uint4 rw[2][TN], rh[2][SUB][TM];
  auto load = [&](int j, uint4 (&w)[TN], uint4 (&h)[SUB][TM]) {
#pragma unroll
    for (int t = 0; t < TN; ++t) w[t] = W[((size_t)t * ksteps + j) * 64];
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      const uint4* Hc = Hq + (size_t)((j * SUB + sb) * 4) * ld;
#pragma unroll
      for (int u = 0; u < TM; ++u) h[sb][u] = Hc[hrow[u]];
    }
  };
  auto step = [&](const uint4 (&w)[TN], const uint4 (&h)[SUB][TM]) {
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const f16x8 A = __builtin_bit_cast(f16x8, I8 ? i8_to_f16x8(w[t], sb) : w[t]);
#pragma unroll
        for (int u = 0; u < TM; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              A, __builtin_bit_cast(f16x8, h[sb][u]), acc[t][u], 0, 0, 0);
      }
  };
  load(0, rw[0], rh[0]);
  if constexpr (!I8) {
    for (int j = 0; j < ksteps; j += 2) {
      load(min(j + 1, ksteps - 1), rw[1], rh[1]);
      __builtin_amdgcn_sched_barrier(0);
      step(rw[0], rh[0]);
      __builtin_amdgcn_sched_barrier(0);
      load(min(j + 2, ksteps - 1), rw[0], rh[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (j + 1 < ksteps) step(rw[1], rh[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // (INT8: the two slots of converted operands would need too many registers;
    // the next step's raw loads are copied into place instead)
    for (int j = 0; j < ksteps; ++j) {
      if (j + 1 < ksteps) load(j + 1, rw[1], rh[1]);
      step(rw[0], rh[0]);
#pragma unroll
      for (int t = 0; t < TN; ++t) rw[0][t] = rw[1][t];
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int u = 0; u < TM; ++u) rh[0][sb][u] = rh[1][sb][u];
    }
  }
  __syncthreads();
  // accumulator (t, u), lane (i, q), element e: weight row n0 + 16t + 4q + e,
  // activation row m0 + 16u + i
  bool over = false;
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int nb = n0 + 16 * t + 4 * q;
    float sc[4] = {1.f, 1.f, 1.f, 1.f};
    if (a.scale)
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = a.scale[nb + e];
#pragma unroll
    for (int u = 0; u < TM; ++u) {
      const int m = m0 + 16 * u + i;
      if (!mrow[u]) continue;  // (the four lanes of a row leave together)
      const float inv = s_inv[m - mb];
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[t][u][e] * sc[e] * inv;
      if (a.epi == EPI_STORE) {
        *reinterpret_cast<float4*>(a.out_f32 + (size_t)m * a.out_ld + nb) =
            make_float4(v[0], v[1], v[2], v[3]);
      } else if (a.epi == EPI_SWIGLU) {
        const uint32_t pk = (uint32_t)f2h_chk(silu(v[0]) * v[1], over) |
                            ((uint32_t)f2h_chk(silu(v[2]) * v[3], over) << 16);
        *reinterpret_cast<uint32_t*>(a.u + chunked(m, nb >> 1, a.u_ld)) = pk;
      } else {  // EPI_RESID
        float* xp = a.out_f32 + (size_t)m * a.out_ld + nb;
        const float4 x0 = *reinterpret_cast<const float4*>(xp);
        const float x[4] = {x0.x + v[0], x0.y + v[1], x0.z + v[2], x0.w + v[3]};
        *reinterpret_cast<float4*>(xp) = make_float4(x[0], x[1], x[2], x[3]);
        if (a.u_gain) {
          uint32_t h2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e)
            h2[e] = (uint32_t)f2h_chk(x[2 * e] * bf2f(a.u_gain[nb + 2 * e]), over) |
                    ((uint32_t)f2h_chk(x[2 * e + 1] * bf2f(a.u_gain[nb + 2 * e + 1]), over) << 16);
          *reinterpret_cast<uint2*>(a.u + chunked(m, nb, a.u_ld)) = make_uint2(h2[0], h2[1]);
          float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
          ss += __shfl_xor(ss, 16);
          ss += __shfl_xor(ss, 32);
          if (q == 0) a.ss_out[(size_t)((n0 + 16 * t) >> 4) * a.ss_out_ld + m] = ss;
        }
      }
    }
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
}

constexpr int kCUs = 256;    // compute units of a gfx950 (MI355X)
constexpr int kPipeKU = 2;  // K steps of 32 per stage of the copy-pipelined form

// 16-byte LDS read at a byte offset, hidden from the compiler's wait insertion
// (which would otherwise wait for every copy in flight before any LDS read); the
// caller waits with lds_wait before using the values.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 lds_read16(uint32_t off) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(off));
  return v;
}

// Pipelined form for half weights: the block's operands for a stage of KU
// 32-wide K steps (per step its 2 TN weight tiles in lane order and its
// activation rows of the step's 4 chunks) are copied global -> LDS by the load
// unit itself (global_load_lds, 16 bytes per lane at the wave's LDS base +
// 16 x lane), NS stages in flight.  Before a stage is used, each wave waits until
// at most the younger stages' copies are outstanding, and one barrier both
// publishes the stage and frees the buffer the next copies overwrite; all of the
// stage's operand reads are issued before one wait.  Activation rows past M are
// copied from row M - 1 (their products are never stored).
template <int TN, int TM, int NS, int KU>
__global__ __launch_bounds__(256) void k_gemm_rows_pipe(GemmArgs a) {
  constexpr int BM = 32 * TM;
  constexpr int WT = 2 * TN;                   // weight tiles per K step
  constexpr int AP = 4 * (BM / 64);            // 64-row activation pieces per K step
  constexpr int PER = KU * (WT + AP) / 4;      // copies per wave per stage
  constexpr int STEP = WT * 64 + 4 * BM;       // uint4 per K step
  constexpr int STAGE = KU * STEP;             // uint4 per stage (KU K steps)
  static_assert((KU * (WT + AP)) % 4 == 0, "copies must divide over the four waves");
  __shared__ uint4 lds[NS * STAGE];
  __shared__ float s_inv[BM];
  __shared__ __attribute__((aligned(16))) float s_part[256 / (BM / 4)][BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  int mblk, nblk;
  rows_tile(mblk, nblk);
  const int mb = BM * mblk;
  const int nb0 = a.row0 + 32 * TN * nblk;
  const int wn = 16 * TN * (wave & 1), wm = 16 * TM * (wave >> 1);
  const int n0 = nb0 + wn, m0 = mb + wm;
  const int M = a.M, ld = a.act_ld;
  const int ksteps = a.K / 32;
  const int nst = ksteps / KU;  // stages (the launcher checks that KU divides the K steps)
  norm_factors<BM, 256, 8>(a, mb, s_inv, s_part, [] {});
  const uint4* W = reinterpret_cast<const uint4*>(a.W) + (size_t)(nb0 >> 4) * ksteps * 64;
  const uint4* H = reinterpret_cast<const uint4*>(a.act);
  // copy stage g (K steps g*KU .. g*KU+KU-1) into buffer buf: piece p of the stage
  // is K step kk = p / (WT + AP), within it weight tile x < WT or activation piece
  auto issue = [&](int g, int buf) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int p = wave + 4 * r;  // (wave-uniform)
      const int kk = p / (WT + AP), x = p % (WT + AP);
      const int j = g * KU + kk;
      const uint4* src;
      uint4* dst;
      if (x < WT) {
        src = W + ((size_t)x * ksteps + j) * 64 + lane;
        dst = lds + buf * STAGE + kk * STEP + x * 64;
      } else {
        const int y = x - WT, c = y / (BM / 64), h = y % (BM / 64);
        int row = mb + 64 * h + lane;
        row = row < M ? row : M - 1;
        src = H + (size_t)(4 * j + c) * ld + row;
        dst = lds + buf * STAGE + kk * STEP + WT * 64 + c * BM + 64 * h;
      }
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
    }
  };
  f32x4 acc[TN][TM];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int u = 0; u < TM; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nst) issue(st, st);
  // s_inv is in LDS before the first barrier (a full one, with its fence)
  __syncthreads();
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;  // byte offset of the array in LDS
  for (int g = 0; g < nst; ++g) {
    if (g + NS - 2 < nst) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER * (NS - 2)) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // every wave's copies of stage g have landed
    if (g + NS - 1 < nst) issue(g + NS - 1, (g + NS - 1) % NS);
    u32x4 av[KU][TN], bv[KU][TM];
#pragma unroll
    for (int kk = 0; kk < KU; ++kk) {
      const uint32_t sw = lds0 + (uint32_t)((g % NS) * STAGE + kk * STEP) * 16;
      const uint32_t sa = sw + WT * 64 * 16;
#pragma unroll
      for (int t = 0; t < TN; ++t) av[kk][t] = lds_read16(sw + (((wave & 1) * TN + t) * 64 + lane) * 16);
#pragma unroll
      for (int u = 0; u < TM; ++u) bv[kk][u] = lds_read16(sa + (q * BM + wm + 16 * u + i) * 16);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < KU; ++kk) {
#pragma unroll
      for (int t = 0; t < TN; ++t) asm volatile("" : "+v"(av[kk][t]));
#pragma unroll
      for (int u = 0; u < TM; ++u) asm volatile("" : "+v"(bv[kk][u]));
    }
#pragma unroll
    for (int kk = 0; kk < KU; ++kk)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int u = 0; u < TM; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(f16x8, av[kk][t]), __builtin_bit_cast(f16x8, bv[kk][u]), acc[t][u], 0, 0, 0);
  }
  bool mrow[TM];
#pragma unroll
  for (int u = 0; u < TM; ++u) mrow[u] = m0 + 16 * u + i < M;
  bool over = false;
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int nb = n0 + 16 * t + 4 * q;
    float sc[4] = {1.f, 1.f, 1.f, 1.f};
    if (a.scale)
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = a.scale[nb + e];
#pragma unroll
    for (int u = 0; u < TM; ++u) {
      const int m = m0 + 16 * u + i;
      if (!mrow[u]) continue;  // (the four lanes of a row leave together)
      const float inv = s_inv[m - mb];
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[t][u][e] * sc[e] * inv;
      if (a.epi == EPI_STORE) {
        *reinterpret_cast<float4*>(a.out_f32 + (size_t)m * a.out_ld + nb) =
            make_float4(v[0], v[1], v[2], v[3]);
      } else if (a.epi == EPI_SWIGLU) {
        const uint32_t pk = (uint32_t)f2h_chk(silu(v[0]) * v[1], over) |
                            ((uint32_t)f2h_chk(silu(v[2]) * v[3], over) << 16);
        *reinterpret_cast<uint32_t*>(a.u + chunked(m, nb >> 1, a.u_ld)) = pk;
      } else {  // EPI_RESID
        float* xp = a.out_f32 + (size_t)m * a.out_ld + nb;
        const float4 x0 = *reinterpret_cast<const float4*>(xp);
        const float x[4] = {x0.x + v[0], x0.y + v[1], x0.z + v[2], x0.w + v[3]};
        *reinterpret_cast<float4*>(xp) = make_float4(x[0], x[1], x[2], x[3]);
        if (a.u_gain) {
          uint32_t h2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e)
            h2[e] = (uint32_t)f2h_chk(x[2 * e] * bf2f(a.u_gain[nb + 2 * e]), over) |
                    ((uint32_t)f2h_chk(x[2 * e + 1] * bf2f(a.u_gain[nb + 2 * e + 1]), over) << 16);
          *reinterpret_cast<uint2*>(a.u + chunked(m, nb, a.u_ld)) = make_uint2(h2[0], h2[1]);
          float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
          ss += __shfl_xor(ss, 16);
          ss += __shfl_xor(ss, 32);
          if (q == 0) a.ss_out[(size_t)((n0 + 16 * t) >> 4) * a.ss_out_ld + m] = ss;
        }
      }
    }
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
}

// Large-tile form for many activation rows (the prompt prefill), on the 32 x 32 x 16
// matrix instruction.  Each wave owns a (32 TM activation rows) x (32 TN weight
// rows) tile as TN x TM accumulators of 32 x 32; WGM x WGN waves make a block of
// BM = 32 TM WGM rows by BN = 32 TN WGN weight rows.  Every operand byte is
// copied once per block from global memory into LDS by the load unit
// (global_load_lds, 16 bytes per lane at the wave's LDS base + 16 x lane), KS
// 32-wide K steps per stage, NS stages in the ring; each wave then reads its
// fragments from LDS.  KS > 1 splits the K steps over KS groups of waves (group g
// takes step KS s + g of stage s), whose partial sums are added at the end.  Per K
// step the LDS holds the BN/16 weight tiles as packed (1 KB each, lane order of
// the 16-row tile) and the activations as 4 chunks of BM rows x 16 bytes.
//
// Fragment reads are conflict-free: for the weights, lane l takes row l & 31 of
// the 32-row block (tile (l >> 4) & 1 of the two, row l & 15 in it) at chunk
// 2h + (l >> 5) of the K step's half h, so each 16 lanes read 256 contiguous
// bytes; for the activations lanes 0-31 and 32-63 each read 512 contiguous bytes.
// Accumulator element e of lane l is weight row 8(e >> 2) + 4(l >> 5) + (e & 3) and
// activation row l & 31 of the 32 x 32 tile, so a lane holds four consecutive
// weight rows per group: the SwiGLU pairs (even, odd) and the 16-row sums of
// squares (two groups and the lane 32 apart) stay within reach.
template <int TM, int TN, int WGM, int WGN, int NS, int KS>
__global__ __launch_bounds__(64 * WGM * WGN * KS) void k_gemm_mx(GemmArgs a, PrefillQkArgs qk, float theta_log2) {
  constexpr int NL = WGM * WGN;                     // waves per K group
  constexpr int NW = NL * KS;
  constexpr int BM = 32 * TM * WGM, BN = 32 * TN * WGN;
  constexpr int WT = BN / 16, AP = BM / 16;         // 1 KB pieces per K step
  constexpr int P = KS * (WT + AP);                 // pieces per stage
  constexpr int PHI = (P + NW - 1) / NW, PLO = P / NW, NHI = P % NW;  // copies per wave
  constexpr int STEP = 64 * (BN + BM);              // bytes per K step
  constexpr int STAGE = KS * STEP;
  static_assert(BM % 64 == 0, "activation pieces are 64 rows");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NS * STAGE];
  __shared__ float s_inv[BM];
  __shared__ __attribute__((aligned(16))) float s_part[64 * NW / (BM / 4)][BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = wave / NL, wl = wave - kg * NL;  // K group, wave within it
  const int wx = wl % WGN, wy = wl / WGN;
  int mblk, nblk;
  rows_tile(mblk, nblk);
  const int mb = BM * mblk;
  const int nb0 = a.row0 + BN * nblk;
  const int M = a.M, ld = a.act_ld;
  const int ksteps = a.K / 32, nst = ksteps / KS;  // (the launcher checks that 2 KS divides ksteps)
  const uint4* W = reinterpret_cast<const uint4*>(a.W) + (size_t)(nb0 >> 4) * ksteps * 64;
  const uint4* H = reinterpret_cast<const uint4*>(a.act);
  // copy stage s (K steps KS s .. KS s + KS - 1) into ring slot s % NS: piece p is
  // K step KS s + p / (WT + AP), within it x = p % (WT + AP): weight tile x < WT,
  // else the activation rows 64 h .. 64 h + 63 of chunk c (rows past M re-read row
  // M - 1; their products are never stored)
  auto copy_one = [&](int s, int r) {  // this wave's r-th piece of stage s
    const int p = wave + NW * r;         // (wave-uniform)
    if (r < PLO || p < P) {
      const int kk = p / (WT + AP), x = p % (WT + AP), j = KS * s + kk;
      uint8_t* base = lds + (s % NS) * STAGE + kk * STEP;
      const uint4* src;
      uint8_t* dst;
      if (x < WT) {
        src = W + ((size_t)x * ksteps + j) * 64 + lane;
        dst = base + x * 1024;
      } else {
        const int y = x - WT, c = y / (BM / 64), h = y % (BM / 64);
        const int row = min(mb + 64 * h + lane, M - 1);
        src = H + (size_t)(4 * j + c) * ld + row;
        dst = base + WT * 1024 + (c * BM + 64 * h) * 16;
      }
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
    }
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int r = 0; r < PHI; ++r) copy_one(s, r);
  };
  f32x16 acc[TN][TM];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int u = 0; u < TM; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][u][e] = 0.f;
  // this lane's fragment offsets within a K step, for half 0 (half 1: + 32 bytes
  // for the weights' chunk pair, + 2 BM x 16 for the activations')
  uint32_t offw[TN], offa[TM];
#pragma unroll
  for (int t = 0; t < TN; ++t)
    offw[t] = (uint32_t)(((32 * TN * wx + 32 * t) / 16 + ((lane >> 4) & 1)) * 1024 +
                         ((lane >> 5) * 16 + (lane & 15)) * 16);
#pragma unroll
  for (int u = 0; u < TM; ++u)
    offa[u] = (uint32_t)(WT * 1024 + ((lane >> 5) * BM + 32 * TM * wy + 32 * u + (lane & 31)) * 16);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  // fragment r of this wave's K step of stage s: r < 2 TN the weights' (half
  // r / TN, tile r % TN), then the activations' (half, tile) in the same order
  auto read_one = [&](int s, int r, u32x4 (&wv)[2][TN], u32x4 (&av)[2][TM]) {
    const uint32_t sb = lds0 + (uint32_t)((s % NS) * STAGE + kg * STEP);
    if (r < 2 * TN) {
      const int h = r / TN, t = r % TN;
      wv[h][t] = lds_read16(sb + offw[t] + 32 * 16 * h);
    } else {
      const int h = (r - 2 * TN) / TM, u = (r - 2 * TN) % TM;
      av[h][u] = lds_read16(sb + offa[u] + 2 * BM * 16 * h);
    }
  };
  auto read = [&](int s, u32x4 (&wv)[2][TN], u32x4 (&av)[2][TM]) {
#pragma unroll
    for (int r = 0; r < 2 * (TN + TM); ++r) read_one(s, r, wv, av);
  };
  // Stage s: K group g takes its K step KS s + g (KS > 1: two or more waves per
  // SIMD, so that one wave's waits overlap another's products).  A wave's fragments
  // of stage s were read during stage s - 1.  Once they are in (and so this wave is
  // done with slot s % NS) and this wave's copies of stage s + 1 have landed, one
  // barrier lets the slot be refilled with stage s + NS and stage s + 1 be read.
  // Those reads and copies are placed between stage s's products, one group after
  // each product (the reads with the first half, so that they are in before the
  // next stage; the copies with the second half), fenced so that the scheduler
  // keeps that order.
  constexpr int NMF = 2 * TN * TM, HALF = NMF / 2, NRD = 2 * (TN + TM);
  auto body = [&](int s, u32x4 (&wv)[2][TN], u32x4 (&av)[2][TM], u32x4 (&wn)[2][TN],
                  u32x4 (&an)[2][TM]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int t = 0; t < TN; ++t) asm volatile("" : "+v"(wv[h][t]));
#pragma unroll
      for (int u = 0; u < TM; ++u) asm volatile("" : "+v"(av[h][u]));
    }
    if (s + NS - 1 < nst) {  // younger issued stages than s + 1: NS - 2 of them
      if (NHI == 0 || wave < NHI) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PHI * (NS - 2)) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PLO * (NS - 2)) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    const bool more_reads = s + 1 < nst, more_copies = s + NS < nst;
#pragma unroll
    for (int f = 0; f < NMF; ++f) {
      const int h = f / (TN * TM), t = (f / TM) % TN, u = f % TM;
      acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          __builtin_bit_cast(f16x8, wv[h][t]), __builtin_bit_cast(f16x8, av[h][u]), acc[t][u], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < NRD; ++r)
        if (r * HALF / NRD == f && more_reads) read_one(s + 1, r, wn, an);
#pragma unroll
      for (int c = 0; c < PHI; ++c)
        if (HALF + c * (NMF - HALF) / PHI == f && more_copies) copy_one(s + NS, c);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the ring's first NS stages are copied while the norm sums are in flight
  norm_factors<BM, 64 * NW, 16>(a, mb, s_inv, s_part, [&] {
#pragma unroll
    for (int st = 0; st < NS; ++st)
      if (st < nst) issue(st);
  });
  // stage 0 in (younger issued stages: min(NS, nst) - 1 of them), s_inv written
  if (NS <= nst) {
    if (NHI == 0 || wave < NHI) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(PHI * (NS - 1)) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(PLO * (NS - 1)) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  u32x4 w0[2][TN], a0[2][TM], w1[2][TN], a1[2][TM];
  read(0, w0, a0);
  for (int s = 0; s < nst; s += 2) {  // (nst is even)
    body(s, w0, a0, w1, a1);
    body(s + 1, w1, a1, w0, a0);
  }
  // ---- epilogue.  The ring is free once every wave is past its last step; it
  // stages the block's outputs so that they leave as whole rows (f32 rows for a
  // store or a residual) or whole 16-byte chunk rows (half outputs) rather than as
  // the accumulators' scattered 16-byte pieces.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (KS > 1) {
    // the K groups' partial sums: groups g > 0 leave theirs in LDS, group 0 adds
    // them in group order
    constexpr int NA = TN * TM * 16;
    float* red = reinterpret_cast<float*>(lds);  // [KS - 1][NL][NA][64]
    static_assert((KS - 1) * NL * NA * 64 * 4 <= NS * STAGE, "partials fit the ring");
    if (kg > 0) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int u = 0; u < TM; ++u)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            red[(((kg - 1) * NL + wl) * NA + (t * TM + u) * 16 + e) * 64 + lane] = acc[t][u][e];
    }
    __syncthreads();
    if (kg == 0) {
      for (int g2 = 1; g2 < KS; ++g2)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int u = 0; u < TM; ++u)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              acc[t][u][e] += red[(((g2 - 1) * NL + wl) * NA + (t * TM + u) * 16 + e) * 64 + lane];
    }
    __syncthreads();
  }
  bool over = false;
  constexpr int NT = 64 * NW, VLD = BN + 4, C4 = BN / 4;
  constexpr bool stage_u = (BN / 16) * BM * 16 <= NS * STAGE;              // SwiGLU halves
  constexpr bool stage_v = BM * VLD * 4 + BM * BN * 2 <= NS * STAGE;      // f32 tile + halves
  // accumulator (t, u), lane l, group g: activation row r, weight rows nl .. nl + 3
  // (local to the block); K group 0 holds the sums
  auto for_each_group = [&](auto&& f) {
    if (kg != 0) return;
#pragma unroll
    for (int u = 0; u < TM; ++u) {
      const int r = 32 * TM * wy + 32 * u + (lane & 31);
      const float inv = s_inv[r];
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = 32 * TN * wx + 32 * t + 8 * g + 4 * (lane >> 5);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[t][u][4 * g + e] * inv;
          f(r, nl, v);
        }
    }
  };
  if (a.epi == EPI_SWIGLU && stage_u) {
    // SwiGLU of each (gate, up) pair -> output column nl / 2, staged as chunk rows
    // [BN / 16 chunks][BM rows][8 halves]; then copied out 64 rows x 16 bytes at a time
    uint32_t* ut = reinterpret_cast<uint32_t*>(lds);
    for_each_group([&](int r, int nl, const float (&v)[4]) {
      const int oc = nl >> 1;
      ut[((oc >> 3) * BM + r) * 4 + ((oc & 7) >> 1)] =
          (uint32_t)f2h_chk(silu(v[0]) * v[1], over) | ((uint32_t)f2h_chk(silu(v[2]) * v[3], over) << 16);
    });
    __syncthreads();
    for (int p = wave; p < (BN / 16) * (BM / 64); p += NW) {  // (wave-uniform)
      const int c = p / (BM / 64), r = 64 * (p % (BM / 64)) + lane, m = mb + r;
      const uint4 val = *reinterpret_cast<const uint4*>(ut + (c * BM + r) * 4);
      if (m < M) *reinterpret_cast<uint4*>(a.u + chunked(m, (nb0 >> 1) + 8 * c, a.u_ld)) = val;
    }
  } else if (a.epi != EPI_SWIGLU && stage_v) {
    // f32 tile [BM][BN + 4] (the padding keeps the lanes' 16-byte writes apart)
    float* vt = reinterpret_cast<float*>(lds);
    // q/k pass in the epilogue: a tile of 128 columns is one head (see below); each
    // row's position and, for k and v, its page are looked up once, while the tile
    // is staged, into int2 s_row[BM] after the tile: (rotation position, page or
    // -1 none, -2 past the table, -3 bad page)
    const bool fused = a.epi == EPI_STORE && BN == 128 && qk.qkv;
    const int q_dim = qk.n_q * 128, kv_dim = qk.n_kv * 128, col0 = nb0;
    const int kind = col0 < q_dim ? 0 : (col0 < q_dim + kv_dim ? 1 : 2);  // q, k, v
    int2* s_row = reinterpret_cast<int2*>(lds + BM * VLD * 4);
    int row_sq = -1, row_pos = 0;
    if (fused && tid < BM) {
      const int m = min(mb + tid, M - 1);
      row_sq = qk.rowinfo[2 * m];
      row_pos = qk.rowinfo[2 * m + 1];
    }
    for_each_group([&](int r, int nl, const float (&v)[4]) {
      *reinterpret_cast<float4*>(vt + r * VLD + nl) = make_float4(v[0], v[1], v[2], v[3]);
    });
    if (fused && tid < BM) {
      int pg = -1;
      if (kind > 0 && row_sq >= 0) {
        if (row_pos >= qk.max_pages * kPage) {
          pg = -2;
        } else {
          pg = qk.page_table[(size_t)row_sq * qk.max_pages + row_pos / kPage];
          if (pg < 0 || pg >= qk.num_pages) pg = -3;
        }
      }
      s_row[tid] = make_int2(row_sq >= 0 ? row_pos : 0, pg);
    }
    __syncthreads();
    // thread i: row i / C4, columns 4 (i % C4) .. + 3; a wave covers whole rows
    if (fused) {
      // The tile is one head of the prompt's q, k or v for BM rows: each wave takes
      // whole rows, lane l elements l and l + 64, and applies what the separate
      // q/k pass would (same arithmetic, same order): q and k are normalised and
      // rotated; q goes back into qkv scaled by 1/sqrt(128), k and v to their pages.
      static_assert(BM * VLD * 4 + BM * 8 <= NS * STAGE || BN != 128, "row table fits");
      const int h = (col0 - q_dim - (kind == 2 ? kv_dim : 0)) >> 7;
      const uint16_t* gain = kind == 0 ? qk.q_norm : qk.k_norm;
      const float g0 = bf2f(gain[lane]), g1 = bf2f(gain[lane + 64]);
      const double inv_rev = rope_inv_rev(lane, theta_log2);
      uint16_t* dst = kind == 1 ? qk.k_pool : qk.v_pool;
      constexpr int RR = 4;  // rows per pass: independent reductions and rotations
      for (int r0 = wave * RR; r0 < BM; r0 += NW * RR) {
        float v0[RR], v1[RR];
        int2 ri[RR];
#pragma unroll
        for (int k = 0; k < RR; ++k) {  // (rows past BM are read clamped, never written)
          const int r = min(r0 + k, BM - 1);
          v0[k] = vt[r * VLD + lane];
          v1[k] = vt[r * VLD + lane + 64];
          ri[k] = s_row[r];
        }
        if (kind < 2)
#pragma unroll
          for (int k = 0; k < RR; ++k) norm_rope_pair(v0[k], v1[k], g0, g1, qk.eps, inv_rev, ri[k].x);
#pragma unroll
        for (int k = 0; k < RR; ++k) {
          const int m = mb + r0 + k;
          if (m >= M || r0 + k >= BM) break;  // (wave-uniform)
          if (kind == 0) {
            float* row = qk.qkv + (size_t)m * qk.qkv_ld + col0;
            row[lane] = v0[k] * kInvSqrtHd;
            row[lane + 64] = v1[k] * kInvSqrtHd;
            continue;
          }
          const int pg = ri[k].y;
          if (pg < 0) {  // -1: a row past every sequence
            if (kind == 1 && lane == 0 && pg == -2) atomicOr(qk.status, QT_STATUS_KV_OVERFLOW);
            if (kind == 1 && lane == 0 && pg == -3) atomicOr(qk.status, QT_STATUS_BAD_PAGE);
            continue;
          }
          const size_t off = ((size_t)pg * qk.n_kv + h) * (kPage * 128) + (size_t)(ri[k].x % kPage) * 128;
          dst[off + lane] = f2bf(v0[k]);
          dst[off + lane + 64] = f2bf(v1[k]);
        }
      }
    } else if (a.epi == EPI_STORE) {
      for (int i = tid; i < BM * C4; i += NT) {
        const int r = i / C4, c4 = i - r * C4, m = mb + r;
        if (m < M)
          *reinterpret_cast<float4*>(a.out_f32 + (size_t)m * a.out_ld + nb0 + 4 * c4) =
              *reinterpret_cast<const float4*>(vt + r * VLD + 4 * c4);
      }
    } else {  // EPI_RESID: x += v; u = half(x * gain) staged as chunk rows; 16-column sums
      uint2* ut = reinterpret_cast<uint2*>(lds + BM * VLD * 4);  // [BN / 8][BM][2]
      // every trip's residual and gains are loaded before any is stored back (a
      // store to x between them would keep the compiler from issuing the next
      // trip's load early: one memory round trip per trip)
      constexpr int IT = BM * C4 / NT;  // trips per thread (every lane runs every trip)
      float4 xo[IT];
      uint2 gn[IT];
#pragma unroll
      for (int k = 0; k < IT; ++k) {
        const int i = tid + k * NT, r = i / C4, c4 = i - r * C4, m = min(mb + r, M - 1);
        const int n = nb0 + 4 * c4;
        xo[k] = *reinterpret_cast<const float4*>(a.out_f32 + (size_t)m * a.out_ld + n);
        gn[k] = a.u_gain ? *reinterpret_cast<const uint2*>(a.u_gain + n) : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int k = 0; k < IT; ++k) {
        const int i = tid + k * NT;
        const int r = i / C4, c4 = i - r * C4, m = mb + r, n = nb0 + 4 * c4;
        const bool live = m < M;
        const float4 v = *reinterpret_cast<const float4*>(vt + r * VLD + 4 * c4);
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (live) {
          x[0] = xo[k].x + v.x;
          x[1] = xo[k].y + v.y;
          x[2] = xo[k].z + v.z;
          x[3] = xo[k].w + v.w;
          *reinterpret_cast<float4*>(a.out_f32 + (size_t)m * a.out_ld + n) = make_float4(x[0], x[1], x[2], x[3]);
        }
        if (a.u_gain) {
          const float g[4] = {bf_lo(gn[k].x), bf_hi(gn[k].x), bf_lo(gn[k].y), bf_hi(gn[k].y)};
          uint32_t h2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e)
            h2[e] = (uint32_t)f2h_chk(x[2 * e] * g[2 * e], over) |
                    ((uint32_t)f2h_chk(x[2 * e + 1] * g[2 * e + 1], over) << 16);
          ut[((c4 >> 1) * BM + r) * 2 + (c4 & 1)] = make_uint2(h2[0], h2[1]);
          // the 16 columns of a sum are four consecutive lanes
          float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
          ss += __shfl_xor(ss, 1);
          ss += __shfl_xor(ss, 2);
          if (live && (c4 & 3) == 0) a.ss_out[(size_t)(n >> 4) * a.ss_out_ld + m] = ss;
        }
      }
      if (a.u_gain) {
        __syncthreads();
        for (int p = wave; p < (BN / 8) * (BM / 64); p += NW) {  // (wave-uniform)
          const int c = p / (BM / 64), r = 64 * (p % (BM / 64)) + lane, m = mb + r;
          const uint4 val = *reinterpret_cast<const uint4*>(ut + (c * BM + r) * 2);
          if (m < M) *reinterpret_cast<uint4*>(a.u + chunked(m, nb0 + 8 * c, a.u_ld)) = val;
        }
      }
    }
  } else {
    // (tiles too large to stage: the accumulators' pieces go out directly)
    if (kg == 0)
#pragma unroll
    for (int u = 0; u < TM; ++u) {
      const int r = 32 * TM * wy + 32 * u + (lane & 31);
      const int m = mb + r;
      if (m >= M) continue;  // (lanes l and l ^ 32 hold the same row and leave together)
      const float inv = s_inv[r];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int nt = nb0 + 32 * TN * wx + 32 * t;  // first weight row of the 32 x 32 tile
#pragma unroll
        for (int s = 0; s < 2; ++s) {  // 16-row halves of the tile
          float ss = 0.f;
#pragma unroll
          for (int g = 2 * s; g < 2 * s + 2; ++g) {
            const int nb = nt + 8 * g + 4 * (lane >> 5);
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[t][u][4 * g + e] * inv;
            if (a.epi == EPI_STORE) {
              *reinterpret_cast<float4*>(a.out_f32 + (size_t)m * a.out_ld + nb) =
                  make_float4(v[0], v[1], v[2], v[3]);
            } else if (a.epi == EPI_SWIGLU) {
              const uint32_t pk = (uint32_t)f2h_chk(silu(v[0]) * v[1], over) |
                                  ((uint32_t)f2h_chk(silu(v[2]) * v[3], over) << 16);
              *reinterpret_cast<uint32_t*>(a.u + chunked(m, nb >> 1, a.u_ld)) = pk;
            } else {  // EPI_RESID
              float* xp = a.out_f32 + (size_t)m * a.out_ld + nb;
              const float4 x0 = *reinterpret_cast<const float4*>(xp);
              const float x[4] = {x0.x + v[0], x0.y + v[1], x0.z + v[2], x0.w + v[3]};
              *reinterpret_cast<float4*>(xp) = make_float4(x[0], x[1], x[2], x[3]);
              if (a.u_gain) {
                uint32_t h2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e)
                  h2[e] = (uint32_t)f2h_chk(x[2 * e] * bf2f(a.u_gain[nb + 2 * e]), over) |
                          ((uint32_t)f2h_chk(x[2 * e + 1] * bf2f(a.u_gain[nb + 2 * e + 1]), over) << 16);
                *reinterpret_cast<uint2*>(a.u + chunked(m, nb, a.u_ld)) = make_uint2(h2[0], h2[1]);
                ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
              }
            }
          }
          if (a.epi == EPI_RESID && a.u_gain) {
            ss += __shfl_xor(ss, 32);
            if (lane < 32) a.ss_out[(size_t)((nt + 16 * s) >> 4) * a.ss_out_ld + m] = ss;
          }
        }
      }
    }
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
}

// ------------------------------------------------------------------ packing
// Source rows [rows][K] bf16 -> half rows row0 + r*step of a tiled [N][K] matrix.
// A finite bf16 weight beyond the half range (|w| > 65504) sets *range_flag.
__global__ __launch_bounds__(256) void k_pack_tiled(const uint16_t* src, int rows, int K,
                                                    uint16_t* dst, int row0, int step,
                                                    uint32_t* range_flag) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;  // one 8-wide chunk
  const int kc = K >> 3;
  if (e >= (long long)rows * kc) return;
  const int r = (int)(e / kc), k = (int)(e - (long long)r * kc) << 3;
  const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)r * K + k);
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
  bool over = false;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = (uint32_t)f2h_chk(bf_lo(in[j]), over) | ((uint32_t)f2h_chk(bf_hi(in[j]), over) << 16);
  *reinterpret_cast<uint4*>(dst + tiled_bf16(row0 + r * step, k, K)) = make_uint4(o[0], o[1], o[2], o[3]);
  if (over) atomicOr(range_flag, 1u);
}

// Rows row0 + r*step of a tiled INT8-quantised [N][K] matrix -> row-major int8
// [rows][K], from int8 tiles or from half tiles holding the integer values.
__global__ __launch_bounds__(256) void k_untile_i8(const void* tiled, int half_src, int rows, int K,
                                                   int row0, int step, int8_t* out) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int kc = K >> 3;
  if (e >= (long long)rows * kc) return;
  const int r = (int)(e / kc), k = (int)(e - (long long)r * kc) << 3;
  uint2 v;
  if (half_src) {
    const uint4 h = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(tiled) +
                                                    tiled_bf16(row0 + r * step, k, K));
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
    uint32_t b[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = (int)h2f((uint16_t)(hw[j >> 1] >> (16 * (j & 1))));
      b[j >> 2] |= ((uint32_t)q & 0xffu) << (8 * (j & 3));
    }
    v = make_uint2(b[0], b[1]);
  } else {
    v = *reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(tiled) +
                                        tiled_i8(row0 + r * step, k, K));
  }
  *reinterpret_cast<uint2*>(out + (size_t)r * K + k) = v;
}

}  // namespace

// Launch shape for nrows weight rows, K columns, M activation rows.  Small weight
// matrices with many activation rows split the rows over 2 or 4 blocks per tile,
// aiming at >= 256 blocks.
GemmPlan plan_gemm(int nrows, int K, int M, bool i8, bool keep, bool swiglu) {
  (void)K;
  (void)i8;
  GemmPlan p{};
  p.rows_per_block = kGemmRows;
  p.row_blocks = nrows / kGemmRows;
  p.msplit = 1;
  p.tiles = 1;
  // A streamed SwiGLU matrix with three times more row tiles than CUs: three
  // tiles per block, so every block re-reads the activations a third as often
  // and keeps three tiles' weight loads in flight (at most two 16-row
  // activation tiles: the Talker's own batch).
  if (swiglu && !keep && p.row_blocks >= 768 && p.row_blocks % 3 == 0 && M <= 32) {
    p.tiles = 3;
    p.row_blocks /= 3;
  }
  if (M <= 2) {
    p.nw = 16, p.mt = 0, p.g = 2;
    return p;
  }
  const int tiles = (M + 15) / 16;
  if (tiles > 1 && p.row_blocks % 8 == 0 && p.tiles == 1)
    while (p.msplit * 2 <= tiles && p.row_blocks * p.msplit < 256) p.msplit *= 2;
  const int mt = (tiles + p.msplit - 1) / p.msplit;
  p.nw = 8;
  p.mt = mt <= 1 ? 1 : (mt <= 2 ? 2 : 4);
  // K steps per load group (measured on the frame): larger groups keep more
  // bytes in flight, until the registers they take cost a block per CU, which
  // the streamed Talker matrices with two activation tiles feel.  One activation
  // tile: 8 (C3 -1.3% against 4; the 3-tile streamed form keeps 4)
  p.g = p.mt == 1 ? (p.tiles == 3 ? 4 : 8) : (p.mt == 2 ? (keep ? 4 : 2) : (keep ? 2 : 1));
  return p;
}

void gemm_kernel_name(const GemmArgs& a, char* buf, int len) {
  const bool i8 = a.w8 != 0;
  const GemmPlan p = plan_gemm(a.nrows, a.K, a.M, i8, a.keep_w != 0, a.epi == EPI_SWIGLU);
  snprintf(buf, len, "k_gemm<%d,%d,%d,%s,%s,%d>", p.nw, p.mt, p.g, i8 ? "true" : "false",
           a.keep_w ? "true" : "false", p.tiles);
}

hipError_t launch_gemm_rows(const GemmArgs& a, hipStream_t s, const PrefillQkArgs* qk, float theta,
                             bool* qk_done) {
  if (qk_done) *qk_done = false;
  const PrefillQkArgs none{};
  if (a.M < 1 || a.nrows <= 0 || (a.nrows % 128) || (a.row0 % kGemmRows) ||
      a.row0 + a.nrows > a.N || a.K <= 0 || (a.K % 64) || a.act_ld < a.M || (a.M % 16))
    return hipErrorInvalidValue;
  if (a.epi != EPI_STORE && a.epi != EPI_RESID && a.epi != EPI_SWIGLU) return hipErrorInvalidValue;
  if (a.ss_in && a.ss_in_slots < 1) return hipErrorInvalidValue;
  if (a.epi == EPI_RESID && a.u_gain && !a.ss_out) return hipErrorInvalidValue;
  // 128 x 128 blocks unless they leave fewer than two blocks per CU: then 64 weight
  // rows, then 64 x 64
  const bool i8 = a.w8 != 0;
  // Many rows: the large-tile LDS form, on the first shape whose blocks fill every
  // CU at least once
  if (!i8 && !a.scale) {
    const long long m256 = (a.M + 255) / 256, m128 = (a.M + 127) / 128;
    if (a.nrows % 192 == 0 && m256 * (a.nrows / 192) >= kCUs) {
      launch_kernel((k_gemm_mx<2, 2, 4, 3, 5, 1>), dim3((unsigned)m256, a.nrows / 192), dim3(768), s, a, none,
                    0.f);
      return hipGetLastError();
    }
    // (the 4-wave tiles take their K steps in two groups of waves: stages of two
    // steps, so K must be a multiple of 128)
    if (a.K % 128 == 0 && m128 * (a.nrows / 128) >= kCUs) {
      // 128-column tiles of a QKV projection are whole heads: the q/k pass is done
      // in the epilogue (whole matrix, rows as the pass expects, 2 q heads per kv head)
      const bool fuse = qk && a.epi == EPI_STORE && a.row0 == 0 && qk->qkv == a.out_f32 &&
                        qk->qkv_ld == a.out_ld && qk->R == a.M && qk->n_q == 2 * qk->n_kv &&
                        a.nrows == (qk->n_q + 2 * qk->n_kv) * 128;
      launch_kernel((k_gemm_mx<2, 2, 2, 2, 4, 2>), dim3((unsigned)m128, a.nrows / 128), dim3(512), s, a,
                    fuse ? *qk : none, fuse ? (float)log2((double)theta) : 0.f);
      if (qk_done) *qk_done = fuse;
      return hipGetLastError();
    }
    if (a.K % 256 == 0 && m128 * (a.nrows / 64) >= kCUs) {
      launch_kernel((k_gemm_mx<2, 2, 2, 1, 3, 4>), dim3((unsigned)m128, a.nrows / 64), dim3(512), s, a, none,
                    0.f);
      return hipGetLastError();
    }
    if (a.K % 128 == 0 && m128 * (a.nrows / 64) >= kCUs) {
      launch_kernel((k_gemm_mx<2, 1, 2, 2, 5, 2>), dim3((unsigned)m128, a.nrows / 64), dim3(512), s, a, none,
                    0.f);
      return hipGetLastError();
    }
  }
  const long long big = (long long)((a.M + 127) / 128) * (a.nrows / 128);
  const long long mid = (long long)((a.M + 127) / 128) * (a.nrows / 64);
  // (measured at 1024 rows: the direct form for 128 x 128 and 64 x 128 blocks, the
  // copy-pipelined form for 64 x 64, with stages of two K steps, four in flight;
  // splitting K in halves for twice the blocks gained nothing for the QKV shape)
  if (big >= 512) {
    const dim3 grid((a.M + 127) / 128, a.nrows / 128);
    if (i8) launch_kernel((k_gemm_rows<true, 4, 4>), grid, dim3(256), s, a);
    else launch_kernel((k_gemm_rows<false, 4, 4>), grid, dim3(256), s, a);
  } else if (mid >= 512) {
    const dim3 grid((a.M + 127) / 128, a.nrows / 64);
    if (i8) launch_kernel((k_gemm_rows<true, 2, 4>), grid, dim3(256), s, a);
    else launch_kernel((k_gemm_rows<false, 2, 4>), grid, dim3(256), s, a);
  } else {
    const dim3 grid((a.M + 63) / 64, a.nrows / 64);
    if (i8) launch_kernel((k_gemm_rows<true, 2, 2>), grid, dim3(256), s, a);
    else launch_kernel((k_gemm_rows_pipe<2, 2, 4, kPipeKU>), grid, dim3(256), s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 64 || a.nrows <= 0 || (a.nrows % kGemmRows) || (a.row0 % kGemmRows) ||
      a.row0 + a.nrows > a.N || a.K <= 0 || (a.K % 64) || a.act_ld < a.M)
    return hipErrorInvalidValue;
  if (a.ss_in && a.ss_in_slots < 1) return hipErrorInvalidValue;
  if (a.epi == EPI_HEAD && ((a.n_logits % kGemmRows) || (a.argmax_range > a.n_logits)))
    return hipErrorInvalidValue;
  if ((a.epi == EPI_RESID || a.epi == EPI_HEAD) && a.u_gain && !a.ss_out) return hipErrorInvalidValue;
  const bool i8 = a.w8 != 0;
  const GemmPlan p = plan_gemm(a.nrows, a.K, a.M, i8, a.keep_w != 0, a.epi == EPI_SWIGLU);
  if (a.keep_w) return i8 ? gemm_dispatch<true, true>(a, p, s) : gemm_dispatch<false, true>(a, p, s);
  return i8 ? gemm_dispatch<true, false>(a, p, s) : gemm_dispatch<false, false>(a, p, s);
}

hipError_t launch_pack_tiled(const uint16_t* src, int rows, int K, uint16_t* dst, int row0,
                             int step, uint32_t* range_flag, hipStream_t s) {
  if (rows <= 0 || K <= 0 || (K % 32) || row0 < 0 || step < 1 || !range_flag)
    return hipErrorInvalidValue;
  const long long n = (long long)rows * (K / 8);
  launch_kernel(k_pack_tiled, dim3((unsigned)((n + 255) / 256)), dim3(256), s, src, rows, K, dst,
                row0, step, range_flag);
  return hipGetLastError();
}

hipError_t launch_untile_i8(const void* tiled, bool half_src, int rows, int K, int row0, int step,
                            int8_t* out, hipStream_t s) {
  if (rows <= 0 || K <= 0 || (K % 64) || row0 < 0 || step < 1) return hipErrorInvalidValue;
  const long long n = (long long)rows * (K / 8);
  launch_kernel(k_untile_i8, dim3((unsigned)((n + 255) / 256)), dim3(256), s, tiled,
                half_src ? 1 : 0, rows, K, row0, step, out);
  return hipGetLastError();
}

}  // namespace qt
