// The code predictor of a frame as one persistent launch on gfx950.
//
// The predictor's 15 steps are a chain of about 400 dependent operations (per step
// an embedding gather, five decoder layers of QKV / attention / output projection
// / gate-up / down, and a head), each too small to fill the chip: as separate
// kernels every one pays a kernel boundary.  Here 256 blocks, one per CU, run the
// whole chain and synchronise among themselves.  The work is laid out so that most
// boundaries stay inside one XCD (32 CUs sharing an L2), where a barrier costs about
// 1 us, and only two per layer span the chip:
//
//   XCD x (x = 0..7) owns KV head x and query heads 2x, 2x+1:
//     QKV      its 512 rows of the fused [q; k; v] matrix          (XCD barrier)
//     attention of those heads for every session                  (XCD barrier)
//     O        the K-slice [256x, 256x+256) of the output projection: a partial
//              sum over its heads, for all 1024 output rows       (grid barrier)
//     residual x += the eight partials (in XCD order), RMSNorm input (XCD barrier)
//     gate/up  its FFN columns [384x, 384x+384), SwiGLU            (XCD barrier)
//     down     the matching K-slice of the down projection: a partial for all
//              1024 rows                                           (grid barrier)
//     residual x += the eight partials, next norm's input          (XCD barrier)
//   step head: rows [256x, 256x+256) of the step's codec head, greedy keys per
//              16 rows                                             (grid barrier)
//   next step: greedy token (or the forced one), embedding row     (XCD barrier)
//
// Every XCD keeps its own copy of the residual rows; all eight copies are computed
// with the same operations in the same order, so they are equal.  Sums over the
// eight partials, over the waves of a block and over the 32 column slices of a
// norm are taken in a fixed order: results do not depend on timing.
//
// Memory coherence: data that only the blocks of one XCD exchange is written with
// plain stores (they land in the XCD's L2) and read with device-scope loads, which
// bypass the CU's L1; data that crosses XCDs (the partial sums and the greedy keys)
// is written with device-scope stores and read with device-scope loads.  A block
// waits for its own stores before it arrives at a barrier.  Barrier counters are
// device-scope atomics; every wait is bounded, and a wait that expires raises an
// abort flag that releases every later wait and sets QT_STATUS_SYNC.
#include "qt_device.h"
#include "qt_internal.h"

namespace qt {
namespace {
using namespace dev;

constexpr int PH = 1024;   // predictor hidden
constexpr int PF = 3072;   // FFN width
constexpr int PV = 2048;   // code vocabulary (rows of a step head)
constexpr int NX = 8;      // XCDs = KV heads
constexpr int NR = 32;     // blocks per XCD
constexpr int NW = 8;      // waves per block
constexpr int NT = NW * 64;
constexpr int RED_LD = 65;            // row stride of the partial tiles in LDS (64 rows + 1)
constexpr int kSpin = 1 << 20;        // polls before a barrier wait gives up
constexpr size_t kLds = 96 * 1024;    // dynamic LDS per block: one block per CU

// sync words (unsigned index; each counter in its own 256-byte line)
constexpr int SY_ARRIVE = 0;          // + 64 x: grid-barrier arrivals of XCD x
constexpr int SY_TOP = 64 * 8;        // XCDs complete
constexpr int SY_REL = 64 * 9;        // + 64 x: release generation for XCD x
constexpr int SY_XBAR = 64 * 17;      // + 64 x: XCD-barrier arrivals of XCD x
constexpr int SY_ABORT = 64 * 25;
constexpr int SY_RANK = 64 * 26;      // + 64 x: blocks that found themselves on XCD x
constexpr int SY_ALL = 64 * 34;       // blocks started
static_assert(SY_ALL + 64 <= (int)kPredSyncWords, "sync area");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kDev = 16;  // cache-policy bit sc1: device scope (bypasses the CU's L1)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}
// device-scope loads at a byte offset from a buffer base
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDev);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ldf4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDev);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}
__device__ __forceinline__ float ldf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kDev));
}
__device__ __forceinline__ unsigned long long ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kDev);
  return ((unsigned long long)v.y << 32) | v.x;
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_sync(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 15u;
}

// ---- barriers (one lane of the block runs them between two block barriers)
struct Sync {
  unsigned* w;
  uint32_t* status;
  int x;
  unsigned grid_gen, xcd_gen;
};

__device__ __forceinline__ void abort_all(Sync& s) {
  __hip_atomic_store(&s.w[SY_ABORT], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  atomicOr(s.status, QT_STATUS_SYNC);
}

// Wait until *p >= target; false if the wait expired or another block aborted.
__device__ bool spin_ge(Sync& s, const unsigned* p, unsigned target, bool rmw) {
  for (int it = 0; it < kSpin; ++it) {
    const unsigned v = rmw ? __hip_atomic_fetch_add(const_cast<unsigned*>(p), 0u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                           : ld_sync(p);
    if (v >= target) return true;
    if (ld_sync(&s.w[SY_ABORT])) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  abort_all(s);
  return false;
}

// All blocks: arrivals counted per XCD, the last of an XCD counts the XCD in, the
// last XCD releases every XCD's word.
__device__ void grid_wait(Sync& s) {
  const unsigned gen = ++s.grid_gen;
  const unsigned prev = __hip_atomic_fetch_add(&s.w[SY_ARRIVE + 64 * s.x], 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
  if (prev + 1 == NR * gen) {
    const unsigned t = __hip_atomic_fetch_add(&s.w[SY_TOP], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (t + 1 == NX * gen)
      for (int q = 0; q < NX; ++q)
        __hip_atomic_store(&s.w[SY_REL + 64 * q], gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  spin_ge(s, &s.w[SY_REL + 64 * s.x], gen, false);
}

// The 32 blocks of this XCD.
__device__ void xcd_wait(Sync& s) {
  const unsigned gen = ++s.xcd_gen;
  unsigned* c = &s.w[SY_XBAR + 64 * s.x];
  __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  spin_ge(s, c, NR * gen, true);
}

// Roles: a block's XCD is the hardware's XCC id (the dispatcher deals blocks round-
// robin over the XCDs, but from wherever the previous kernel left off), its rank
// among that XCD's blocks is its arrival order there.  Once all 256 blocks have
// arrived, every XCD must hold exactly 32 of them; otherwise (or if they never all
// arrive) the launch gives up.  Returns false if this block must leave.
__device__ bool take_role(Sync& s, int* x_out, int* r_out) {
  __shared__ int s_x, s_r, s_ok;
  if (threadIdx.x == 0) {
    const unsigned x = xcc_id();
    bool ok = x < (unsigned)NX && gridDim.x == kPredBlocks;
    unsigned r = 0;
    if (ok) {
      r = __hip_atomic_fetch_add(&s.w[SY_RANK + 64 * x], 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&s.w[SY_ALL], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s.x = (int)x;
      ok = spin_ge(s, &s.w[SY_ALL], kPredBlocks, false);
      for (int q = 0; ok && q < NX; ++q) ok = ld_sync(&s.w[SY_RANK + 64 * q]) == (unsigned)NR;
    }
    if (!ok) abort_all(s);
    s_x = ok ? (int)x : 0;
    s_r = ok ? (int)r : 0;
    s_ok = ok;
  }
  __syncthreads();
  *x_out = s_x;
  *r_out = s_r;
  return s_ok != 0;
}

// Stage boundary: every wave's stores are complete, then one lane synchronises.
template <bool GRID>
__device__ __forceinline__ void boundary(Sync& s) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (GRID) grid_wait(s);
    else xcd_wait(s);
  }
  __syncthreads();
}

// ---- per-block view of the buffers
struct Ctx {
  int x, r, B, M, ldm, step, layer;
  float eps;
  float* xl;         // this XCD's residual rows [ldm][1024]
  uint16_t* ul;      // this XCD's next-GEMM input, chunked [128][ldm][8]
  float* sl;         // this XCD's sums of squares [32][ldm]
  float* ql;         // [ldm][512]
  uint16_t* ol;      // chunked [32][ldm][8]
  uint16_t* fl;      // chunked [48][ldm][8]
};

// ---- residual rows: x (+)= ..., then the next norm's half input and the sums of
// squares of this block's 32 columns.  Thread (m, c4): row m, columns 32r + 4c4 ..+3.
__device__ __forceinline__ void put_row4(const Ctx& c, int m, int col, const float (&v)[4],
                                         const uint16_t* gain, uint32_t* status) {
  *reinterpret_cast<float4*>(c.xl + (size_t)m * PH + col) = make_float4(v[0], v[1], v[2], v[3]);
  const uint2 g = *reinterpret_cast<const uint2*>(gain + col);
  bool over = false;
  const uint32_t h0 = (uint32_t)f2h_chk(v[0] * bf_lo(g.x), over) |
                      ((uint32_t)f2h_chk(v[1] * bf_hi(g.x), over) << 16);
  const uint32_t h1 = (uint32_t)f2h_chk(v[2] * bf_lo(g.y), over) |
                      ((uint32_t)f2h_chk(v[3] * bf_hi(g.y), over) << 16);
  *reinterpret_cast<uint2*>(c.ul + chunked(m, col, c.ldm)) = make_uint2(h0, h1);
  if (over) atomicOr(status, QT_STATUS_FP16_RANGE);
}

__device__ __forceinline__ void put_ss(const Ctx& c, int m, bool on, const float (&v)[4]) {
  float ss = on ? (v[0] * v[0] + v[1] * v[1]) + (v[2] * v[2] + v[3] * v[3]) : 0.f;
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 4);
  if (on && (threadIdx.x & 7) == 0) c.sl[(size_t)c.r * c.ldm + m] = ss;
}

// x += sum over the eight XCDs' partials (part: [8][ldm][1024], device-scope).
__device__ void stage_reduce(const Ctx& c, const float* part, const uint16_t* gain,
                             uint32_t* status) {
  const int tid = threadIdx.x, m = tid >> 3, col = 32 * c.r + 4 * (tid & 7);
  const bool on = m < c.M;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (on) {
    const __amdgpu_buffer_rsrc_t rx = rsrc(c.xl), rp = rsrc(part);
    float4 p[NX + 1];
    p[0] = ldf4(rx, (uint32_t)(((size_t)m * PH + col) * 4));
#pragma unroll
    for (int j = 0; j < NX; ++j) p[j + 1] = ldf4(rp, (uint32_t)((((size_t)j * c.ldm + m) * PH + col) * 4));
    v[0] = p[0].x, v[1] = p[0].y, v[2] = p[0].z, v[3] = p[0].w;
#pragma unroll
    for (int j = 1; j <= NX; ++j) {
      v[0] += p[j].x;
      v[1] += p[j].y;
      v[2] += p[j].z;
      v[3] += p[j].w;
    }
    put_row4(c, m, col, v, gain, status);
  }
  put_ss(c, m, on, v);
}

// The step's input rows: the greedy (or forced) token of the previous codebook's
// embedding row; at step 1 also the projection rows [0, B) left by the Talker.
__device__ void stage_embed(const Ctx& c, const PredPersistArgs& a, uint32_t* status) {
  const int tid = threadIdx.x, m = tid >> 3, sub = tid & 7, col = 32 * c.r + 4 * sub;
  const bool on = m < c.M;
  const int k = c.step;
  const bool proj = k == 1 && m < c.B;
  const int b = k == 1 ? m - c.B : m;
  // greedy key of codebook k-1: eight lanes of the row take 16 candidates each
  unsigned long long best = 0ull;
  if (on && !proj && !a.forced) {
    const __amdgpu_buffer_rsrc_t rc = rsrc(a.cand);
    const size_t base = ((size_t)(k - 1) * c.B + b) * a.cand_ld;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      unsigned long long kv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[e] = ld8(rc, (uint32_t)((base + 16 * sub + 8 * h + e) * 8));
#pragma unroll
      for (int e = 0; e < 8; ++e) best = kv[e] > best ? kv[e] : best;
    }
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    const unsigned long long ob = ((unsigned long long)(uint32_t)__shfl_xor((int)(best >> 32), o) << 32) |
                                  (uint32_t)__shfl_xor((int)(uint32_t)best, o);
    best = ob > best ? ob : best;
  }
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (on) {
    if (proj) {
      const float4 p = *reinterpret_cast<const float4*>(a.x_p + (size_t)m * PH + col);
      v[0] = p.x, v[1] = p.y, v[2] = p.z, v[3] = p.w;
    } else {
      int tok = a.forced ? a.forced[(size_t)b * a.ncb + k - 1] : key_index(best);
      if (tok < 0 || tok >= PV) {
        if (sub == 0 && c.x == 0 && c.r == 0) atomicOr(status, QT_STATUS_BAD_TOKEN);
        tok = 0;
      }
      const uint2 e = *reinterpret_cast<const uint2*>(a.embed[k - 1] + (size_t)tok * PH + col);
      v[0] = bf_lo(e.x), v[1] = bf_hi(e.x), v[2] = bf_lo(e.y), v[3] = bf_hi(e.y);
    }
    put_row4(c, m, col, v, a.g_in[0], status);
  }
  put_ss(c, m, on, v);
}

// ---- GEMM over this block's weight tiles.  y[m][n] = sum_k W[n][k] act[m][k] over the
// stage's K range: K steps kg0 .. kg0 + nk - 1 of the packed matrix (ks_full steps per
// row tile), whose activations are chunks 0 .. of `act` (chunked, ldm rows, local K).
// Wave w takes K steps w, w + 8, ...; its partial tiles go to LDS and the epilogue sums
// the eight waves in order.
struct Gemm {
  const void* W;
  const float* scale;
  int ks_full, kg0, nk;
  int nt, rt[2];        // row tiles of this block (global tile index) and their count
  const uint16_t* act;
  int row0;             // first activation row used (M rows)
  bool norm;            // multiply by 1 / rms of the rows (sums of squares in ss_loc)
};

template <bool I8>
__device__ __forceinline__ uint4 i8_half8(const uint4& w, int sb) {
  const uint32_t lo = sb ? w.z : w.x, hi = sb ? w.w : w.y;
  return make_uint4(i8pair_to_f16x2(lo, 0), i8pair_to_f16x2(lo, 1), i8pair_to_f16x2(hi, 0),
                    i8pair_to_f16x2(hi, 1));
}

// The rows' norm factors: eight lanes per row add four slots each, then the eight
// partials in a fixed order (lane-swap tree).
__device__ __forceinline__ void norm_factors(const Ctx& c, int row0, float* s_inv) {
  const int tid = threadIdx.x, m = tid >> 3, s8 = tid & 7;
  float ss = 0.f;
  if (m < c.M) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(c.sl);
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = ldf(rs, (uint32_t)(((size_t)(4 * s8 + e) * c.ldm + row0 + m) * 4));
    ss = (p[0] + p[1]) + (p[2] + p[3]);
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 4);
  if (m < c.M && s8 == 0) s_inv[m] = 1.0f / sqrtf(ss / (float)PH + c.eps);
}

// Runs the products; leaves per-wave partial tiles in red ([wave][tile][16][RED_LD])
// and the rows' norm factors in s_inv, then a block barrier.  MTX: 16-row activation
// tiles at most (the step's rows M <= 16 MTX).
template <bool I8, int MTX>
__device__ void gemm_core(const Ctx& c, const Gemm& g, float* red, float* s_inv) {
  constexpr int SUB = I8 ? 2 : 1;
  constexpr int JM = I8 ? 2 : 4;  // K steps per wave at most (K <= 1024 per stage)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int M = c.M, mt = (M + 15) >> 4;
  // every load of the block is issued before any arithmetic: this wave's weight
  // pieces and activation pieces, and the rows' sums of squares
  const uint4* W = reinterpret_cast<const uint4*>(g.W) + lane;
  uint4 w[2][JM];
  uint4 h[JM][SUB][MTX];
  const __amdgpu_buffer_rsrc_t ra = rsrc(g.act);
#pragma unroll
  for (int s = 0; s < JM; ++s) {
    const int j = wave + NW * s;
    if (j < g.nk) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (t < g.nt) w[t][s] = W[((size_t)g.rt[t] * g.ks_full + g.kg0 + j) * 64];
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) {
        const int ch = (j * SUB + sb) * 4 + q;
#pragma unroll
        for (int u = 0; u < MTX; ++u) {
          const int m = 16 * u + i;
          h[s][sb][u] = (u < mt && m < M)
                            ? ld16(ra, (uint32_t)((((size_t)ch * c.ldm) + g.row0 + m) * 16))
                            : make_uint4(0, 0, 0, 0);
        }
      }
    }
  }
  if (g.norm) norm_factors(c, g.row0, s_inv);
  f32x4 acc[2][MTX];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < MTX; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < JM; ++s) {
    if (wave + NW * s < g.nk) {
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (t < g.nt) {
            const f16x8 A = __builtin_bit_cast(f16x8, I8 ? i8_half8<I8>(w[t][s], sb) : w[t][s]);
#pragma unroll
            for (int u = 0; u < MTX; ++u)
              if (u < mt)
                acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    A, __builtin_bit_cast(f16x8, h[s][sb][u]), acc[t][u], 0, 0, 0);
          }
        }
    }
  }
  // accumulator (t, u), lane (i, q), element e: weight row 4q + e, activation row 16u + i
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (t < g.nt)
#pragma unroll
      for (int u = 0; u < MTX; ++u)
        if (u < mt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            red[((wave * 2 + t) * 16 + 4 * q + e) * RED_LD + 16 * u + i] = acc[t][u][e];
  __syncthreads();
}

// The block's finished value of weight row 16 rt[t] + r16 for activation row m.
template <bool I8>
__device__ __forceinline__ float gemm_value(const Gemm& g, const float* red, const float* s_inv,
                                           int t, int r16, int m) {
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) v += red[((w * 2 + t) * 16 + r16) * RED_LD + m];
  if (g.scale) v *= g.scale[16 * g.rt[t] + r16];  // INT8-quantised (int8 or half values)
  if (g.norm) v *= s_inv[m];
  return v;
}

// ---- attention of KV head x (query heads 2x, 2x+1) for session b over the
// frame-local predictor cache: the new positions pos0 .. pos0 + n_new - 1 are
// normalised, rotated, appended and attend causally to positions 0 .. own.  Waves
// 0..3 take one new vector each (query heads, key, value), lane l holding dimensions
// l and l + 64 (the RoPE pair); thread group t = tid / 16 < 16 then holds cached
// position t, dimensions 8 (tid % 16) .. +7.
struct AttnSmem {
  float qs[2][2][128];
  float kn[2][128], vn[2][128];
  float sc[2][2][16];
  float red[4][2][2][128];
  float lsum[2][2];
};

__device__ void stage_attn(const Ctx& c, const PredPersistArgs& a, AttnSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = c.r;
  const bool active = b < c.B;
  const int n_new = c.step == 1 ? 2 : 1, pos0 = c.step == 1 ? 0 : c.step;
  const int l = c.layer;
  const size_t lay = ((size_t)l * a.ncb * NX) * 128;
  uint16_t* kbase = a.kc + (size_t)b * a.sess_stride + lay;
  uint16_t* vbase = a.vc + (size_t)b * a.sess_stride + lay;
  const int t = tid >> 4, cc = tid & 15;
  // one round trip: every cached position of this head and the new vectors
  uint4 kq = make_uint4(0, 0, 0, 0), vq = make_uint4(0, 0, 0, 0);
  float x0[2] = {0.f, 0.f}, x1[2] = {0.f, 0.f};
  float g0 = 0.f, g1 = 0.f;
  if (active && wave < 4) {
    if (t < pos0) {
      const size_t off = ((size_t)t * NX + c.x) * 128 + 8 * cc;
      kq = ld16(rsrc(kbase), (uint32_t)(off * 2));
      vq = ld16(rsrc(vbase), (uint32_t)(off * 2));
    }
    const int col = wave < 2 ? wave * 128 : (wave == 2 ? 256 : 384);
    const __amdgpu_buffer_rsrc_t rq = rsrc(c.ql);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i < n_new) {
        const size_t row = (size_t)(i * c.B + b) * 512 + col;
        x0[i] = ldf(rq, (uint32_t)((row + lane) * 4));
        x1[i] = ldf(rq, (uint32_t)((row + lane + 64) * 4));
      }
    }
    const uint16_t* gain = wave < 2 ? a.g_q[l] : a.g_k[l];
    g0 = bf2f(gain[lane]);
    g1 = bf2f(gain[lane + 64]);
  }
  if (active && wave < 4) {
    const double inv_rev = rope_inv_rev(lane, a.theta_log2);
    for (int i = 0; i < n_new; ++i) {
      const int pos = pos0 + i;
      float v0 = x0[i], v1 = x1[i];
      if (wave < 3) norm_rope_pair(v0, v1, g0, g1, c.eps, inv_rev, pos);
      if (wave < 2) {
        sm.qs[i][wave][lane] = v0 * kInvSqrtHd;
        sm.qs[i][wave][lane + 64] = v1 * kInvSqrtHd;
      } else {
        const uint16_t b0 = f2bf(v0), b1 = f2bf(v1);
        const size_t off = ((size_t)pos * NX + c.x) * 128;
        uint16_t* dst = wave == 2 ? kbase : vbase;
        dst[off + lane] = b0;
        dst[off + lane + 64] = b1;
        float* nb = wave == 2 ? sm.kn[i] : sm.vn[i];
        nb[lane] = bf2f(b0);
        nb[lane + 64] = bf2f(b1);
      }
    }
  }
  __syncthreads();
  const int n_pos = pos0 + n_new;
  float kf[8], vf[8];
  if (t < n_pos && t >= pos0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = sm.kn[t - pos0][8 * cc + e];
      vf[e] = sm.vn[t - pos0][8 * cc + e];
    }
  } else if (t < n_pos) {
    kf[0] = bf_lo(kq.x); kf[1] = bf_hi(kq.x); kf[2] = bf_lo(kq.y); kf[3] = bf_hi(kq.y);
    kf[4] = bf_lo(kq.z); kf[5] = bf_hi(kq.z); kf[6] = bf_lo(kq.w); kf[7] = bf_hi(kq.w);
    vf[0] = bf_lo(vq.x); vf[1] = bf_hi(vq.x); vf[2] = bf_lo(vq.y); vf[3] = bf_hi(vq.y);
    vf[4] = bf_lo(vq.z); vf[5] = bf_hi(vq.z); vf[6] = bf_lo(vq.w); vf[7] = bf_hi(vq.w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[e] = vf[e] = 0.f;
  }
  if (active && wave < 4) {
    for (int i = 0; i < n_new; ++i) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float sdot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sdot = fmaf(sm.qs[i][hh][8 * cc + e], kf[e], sdot);
        sdot = row_sum16(sdot);
        if (cc == 0) sm.sc[i][hh][t] = (t <= pos0 + i) ? sdot : -INFINITY;
      }
    }
  }
  __syncthreads();
  if (active && wave == 0) {
    const int i = lane >> 5, hh = (lane >> 4) & 1, u = lane & 15;
    if (i < n_new) {
      const bool in = u <= pos0 + i;
      const float v = in ? sm.sc[i][hh][u] : -INFINITY;
      const float mx = row_max16(v);
      const float e = in ? expf(v - mx) : 0.f;
      const float lsum = row_sum16(e);
      sm.sc[i][hh][u] = e;
      if (u == 0) sm.lsum[i][hh] = lsum;
    }
  }
  __syncthreads();
  if (active && wave < 4) {
    for (int i = 0; i < n_new; ++i) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float wgt = (t < n_pos) ? sm.sc[i][hh][t] : 0.f;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = sum_q4(wgt * vf[e]);
        if (lane < 16) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sm.red[wave][i][hh][8 * cc + e] = acc[e];
        }
      }
    }
  }
  __syncthreads();
  if (active && tid < 256) {
    const int jj = tid >> 7, d = tid & 127;
    bool over = false;
    for (int i = 0; i < n_new; ++i) {
      const float out = sm.red[0][i][jj][d] + sm.red[1][i][jj][d] + sm.red[2][i][jj][d] +
                        sm.red[3][i][jj][d];
      c.ol[chunked(i * c.B + b, jj * 128 + d, c.ldm)] = f2h_chk(out / sm.lsum[i][jj], over);
    }
    if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
  }
}

// ---------------------------------------------------------------------------
template <bool I8, int MTX>
__global__ __launch_bounds__(NT) void k_pred_persist(PredPersistArgs a) {
  extern __shared__ __align__(16) char smem[];
  float* red = reinterpret_cast<float*>(smem);
  float* s_inv = red + NW * 2 * 16 * RED_LD;
  AttnSmem& asm_ = *reinterpret_cast<AttnSmem*>(smem);
  constexpr int KS = I8 ? 64 : 32;  // K per packed step
  const int tid = threadIdx.x;
  Sync sy;
  sy.w = a.sync;
  sy.status = a.status;
  sy.grid_gen = sy.xcd_gen = 0;
  int bx, br;
  if (!take_role(sy, &bx, &br)) return;  // (uniform per block; every block leaves)
  sy.x = bx;

  Ctx c;
  c.x = bx;
  c.r = br;
  c.B = a.B;
  c.ldm = a.ldm;
  c.eps = a.eps;
  c.xl = a.x_loc + (size_t)c.x * a.ldm * PH;
  c.ul = a.u_loc + (size_t)c.x * (PH / 8) * a.ldm * 8;
  c.sl = a.ss_loc + (size_t)c.x * NR * a.ldm;
  c.ql = a.qkv_loc + (size_t)c.x * a.ldm * 512;
  c.ol = a.o_loc + (size_t)c.x * 32 * a.ldm * 8;
  c.fl = a.f_loc + (size_t)c.x * 48 * a.ldm * 8;
  const int x = c.x, r = c.r;

  for (int k = 1; k <= a.n_steps; ++k) {
    c.step = k;
    c.M = k == 1 ? 2 * a.B : a.B;
    c.layer = 0;
    stage_embed(c, a, a.status);
    boundary<false>(sy);
    for (int l = 0; l < a.layers; ++l) {
      c.layer = l;
      if (l > 0) {
        stage_reduce(c, a.p_d, a.g_in[l], a.status);
        boundary<false>(sy);
      }
      {  // QKV rows of head x: q 2x, 2x+1 (tiles 16x ..), key x (128 + 8x ..), value x (192 + 8x ..)
        Gemm g{};
        g.W = a.w_qkv[l];
        g.scale = a.s_qkv[l];
        g.ks_full = PH / KS;
        g.kg0 = 0;
        g.nk = PH / KS;
        g.nt = 1;
        g.rt[0] = r < 16 ? 16 * x + r : (r < 24 ? 128 + 8 * x + (r - 16) : 192 + 8 * x + (r - 24));
        g.act = c.ul;
        g.row0 = 0;
        g.norm = true;
        gemm_core<I8, MTX>(c, g, red, s_inv);
        for (int e = tid; e < 16 * c.M; e += NT) {
          const int r16 = e & 15, m = e >> 4;
          c.ql[(size_t)m * 512 + 16 * r + r16] = gemm_value<I8>(g, red, s_inv, 0, r16, m);
        }
      }
      boundary<false>(sy);
      stage_attn(c, a, asm_);
      boundary<false>(sy);
      {  // output projection, K-slice of heads 2x, 2x+1: partial sums of all 1024 rows
        Gemm g{};
        g.W = a.w_o[l];
        g.scale = a.s_o[l];
        g.ks_full = 2048 / KS;
        g.kg0 = x * (256 / KS);
        g.nk = 256 / KS;
        g.nt = 2;
        g.rt[0] = r;
        g.rt[1] = r + 32;
        g.act = c.ol;
        g.row0 = 0;
        g.norm = false;
        gemm_core<I8, MTX>(c, g, red, s_inv);
        float* po = a.p_o + (size_t)x * a.ldm * PH;
        for (int e = tid; e < 2 * 16 * c.M; e += NT) {
          const int r16 = e & 15, m = (e >> 4) % c.M, t = (e >> 4) / c.M;
          st_dev(po + (size_t)m * PH + 16 * g.rt[t] + r16, gemm_value<I8>(g, red, s_inv, t, r16, m));
        }
      }
      boundary<true>(sy);
      stage_reduce(c, a.p_o, a.g_post[l], a.status);
      boundary<false>(sy);
      {  // gate/up rows of FFN columns [384x, 384x + 384): 48 tiles, SwiGLU
        Gemm g{};
        g.W = a.w_gu[l];
        g.scale = a.s_gu[l];
        g.ks_full = PH / KS;
        g.kg0 = 0;
        g.nk = PH / KS;
        g.nt = r < 16 ? 2 : 1;
        g.rt[0] = 48 * x + r;
        g.rt[1] = 48 * x + r + 32;
        g.act = c.ul;
        g.row0 = 0;
        g.norm = true;
        gemm_core<I8, MTX>(c, g, red, s_inv);
        // rows 2p (gate) and 2p + 1 (up) of a tile -> local FFN column 8 (tile - 48x) + p
        bool over = false;
        for (int e = tid; e < g.nt * 8 * c.M; e += NT) {
          const int p = e & 7, m = (e >> 3) % c.M, t = (e >> 3) / c.M;
          const float gt = gemm_value<I8>(g, red, s_inv, t, 2 * p, m);
          const float up = gemm_value<I8>(g, red, s_inv, t, 2 * p + 1, m);
          c.fl[chunked(m, 8 * (g.rt[t] - 48 * x) + p, c.ldm)] = f2h_chk(silu(gt) * up, over);
        }
        if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
      }
      boundary<false>(sy);
      {  // down projection, K-slice of FFN columns [384x, 384x + 384): partials of all rows
        Gemm g{};
        g.W = a.w_dn[l];
        g.scale = a.s_dn[l];
        g.ks_full = PF / KS;
        g.kg0 = x * (384 / KS);
        g.nk = 384 / KS;
        g.nt = 2;
        g.rt[0] = r;
        g.rt[1] = r + 32;
        g.act = c.fl;
        g.row0 = 0;
        g.norm = false;
        gemm_core<I8, MTX>(c, g, red, s_inv);
        float* pd = a.p_d + (size_t)x * a.ldm * PH;
        for (int e = tid; e < 2 * 16 * c.M; e += NT) {
          const int r16 = e & 15, m = (e >> 4) % c.M, t = (e >> 4) / c.M;
          st_dev(pd + (size_t)m * PH + 16 * g.rt[t] + r16, gemm_value<I8>(g, red, s_inv, t, r16, m));
        }
      }
      boundary<true>(sy);
    }
    stage_reduce(c, a.p_d, a.g_final, a.status);
    boundary<false>(sy);
    {  // the step's head, rows [256x, 256x + 256), at the last position's rows
      const int row0 = k == 1 ? a.B : 0;
      if (r < 16) {
        Gemm g{};
        g.W = a.w_head[k - 1];
        g.scale = a.s_head[k - 1];
        g.ks_full = PH / KS;
        g.kg0 = 0;
        g.nk = PH / KS;
        g.nt = 1;
        g.rt[0] = 16 * x + r;
        g.act = c.ul;
        g.row0 = row0;
        g.norm = true;
        Ctx ch = c;
        ch.M = a.B;
        gemm_core<I8, MTX>(ch, g, red, s_inv);
        const int nrow = 16 * g.rt[0];
        for (int e = tid; e < 16 * a.B; e += NT) {  // (whole 16-lane groups)
          const int r16 = e & 15, b = e >> 4;
          const float v = gemm_value<I8>(g, red, s_inv, 0, r16, b);
          a.logits[((size_t)b * (a.ncb - 1) + (k - 1)) * PV + nrow + r16] = v;
          const bool nan = v != v;
          unsigned long long key = nan ? 0ull : greedy_key(v, nrow + r16);
          key = row_max16_u64(key);
          if (nan) atomicOr(a.status, QT_STATUS_NAN);
          if (r16 == 0) st_dev(a.cand + ((size_t)k * a.B + b) * a.cand_ld + g.rt[0], key);
        }
      }
    }
    boundary<true>(sy);
  }
}

// The predictor's tiles are halves in both weight modes (INT8 mode holds its
// quantised values as halves), so only the half form is instantiated.
template <int MTX>
hipError_t prepare_one(int cus) {
  const void* k = (const void*)k_pred_persist<false, MTX>;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e != hipSuccess) return e;
  // every block waits on all the others at each stage: all of them must be
  // resident at once, which the occupancy of this launch shape has to allow
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, NT, kLds);
  if (e != hipSuccess) return e;
  return (long long)per_cu * cus >= kPredBlocks ? hipSuccess : hipErrorInvalidConfiguration;
}

template <int MTX>
hipError_t pred_launch(const PredPersistArgs& a, hipStream_t s) {
  const dim3 grid(kPredBlocks), block(NT);
  if (g_launch_events.start)
    hipExtLaunchKernelGGL(k_pred_persist<false, MTX>, grid, block, kLds, s, g_launch_events.start,
                          g_launch_events.stop, 0, a);
  else
    hipLaunchKernelGGL((k_pred_persist<false, MTX>), grid, block, kLds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t prepare_pred_persist(int cus) {
  hipError_t e = prepare_one<1>(cus);
  if (e == hipSuccess) e = prepare_one<2>(cus);
  if (e == hipSuccess) e = prepare_one<4>(cus);
  return e;
}

hipError_t launch_pred_persist(const PredPersistArgs& a, hipStream_t s) {
  if (a.B < 1 || a.B > 32 || a.ldm < 2 * a.B || a.layers < 1 || a.layers > kPredMaxLayers ||
      a.n_steps < 1 || a.n_steps > kPredMaxSteps || a.ncb != a.n_steps + 1 || a.cand_ld < PV / 16)
    return hipErrorInvalidValue;
  // 16-row activation tiles of the largest step (step 1 carries 2B rows)
  if (a.B <= 8) return pred_launch<1>(a, s);
  if (a.B <= 16) return pred_launch<2>(a, s);
  return pred_launch<4>(a, s);
}

}  // namespace qt
