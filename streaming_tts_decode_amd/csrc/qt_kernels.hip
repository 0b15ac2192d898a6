// gfx950 kernels of the lockstep decode frame.
//
// Every kernel here is launched by qt_abi.cpp on the caller's stream; shapes
// are validated on the host before launch (see the launchers at the end).
//
// Data types: GEMM weights packed as IEEE half (from the bf16 source weights) or
// int8 (+ fp32 per-row scale), GEMM activations half, accumulation fp32, residual
// streams fp32, embeddings, norm gains and KV caches bf16.
#include <math.h>

#include "qt_device.h"
#include "qt_internal.h"

namespace qt {
namespace {

using namespace dev;

// Merge of query head j's n_active split partials of session b, output dimension d:
// 16 splits per round trip, every thread loading the splits' (max, sum) and its
// own dimension of their outputs at once (indices past the last split repeat it
// and are masked), then folding them into a running (max, sum, output) in split
// order.  COHERENT: partials written in the same launch by other blocks (device-
// coherent loads); else written by an earlier launch.
template <bool COHERENT>
__device__ __forceinline__ void merge_splits(const AttnPagedArgs& a, int b, int j, int d, int n_active,
                                             size_t orow) {
  const float* pb = a.part + ((size_t)b * a.n_q + j) * a.n_splits * 130;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < n_active; c0 += 16) {
    float mv[16], lv[16], ov[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float* ps = pb + (size_t)min(c0 + k, n_active - 1) * 130;
      mv[k] = COHERENT ? dev_load(ps) : ps[0];
      lv[k] = COHERENT ? dev_load(ps + 1) : ps[1];
      ov[k] = COHERENT ? dev_load(ps + 2 + d) : ps[2 + d];
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (c0 + k < n_active) Mc = fmaxf(Mc, mv[k]);
    const float r = expf(M - Mc);  // 0 on the first chunk (M = -inf, Mc finite)
    L *= r;
    O *= r;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (c0 + k < n_active) {
        const float w = expf(mv[k] - Mc);
        L = fmaf(lv[k], w, L);
        O = fmaf(ov[k], w, O);
      }
    }
    M = Mc;
  }
  bool over = false;
  a.o[orow] = f2h_chk(O / L, over);
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
}

// ---------------------------------------------------------------------------
// Talker decode attention over paged KV.  Grid (kv head, session, split): the
// eight KV heads of one page are adjacent 4 KB pieces of it, and with the head
// index fastest their blocks are dispatched together, so each page is read from
// DRAM while its rows are open (measured: a quarter less time than with the
// split index fastest).  Splits past a session's cache come last.
// The block for (b, h, s) handles query heads 2h, 2h+1 over positions
// [s*S, min((s+1)*S, p+1)) where p = kv_len[b] is the new token's position.
// The split holding p also normalises/rotates the new key, stores the new key
// and value into their page and uses them from LDS.  Splits write (max, sum,
// unnormalised output) partials; the last block to arrive merges them in split
// order (deterministic), writes the (half) attention output and resets the
// counter.
//
// Memory round trips are kept to two before the arithmetic: the cache length,
// this split's page-table entries and the raw q / k / v values are loaded
// together; then all of the split's K/V loads are issued, and the q and k
// normalisation and rotation run while they are in flight.
//
// SEP (batches of kAttnMergeMinBatch sessions or more): splits store their
// partials with plain stores and exit, and k_attn_merge merges them in the next
// launch, with the same arithmetic.  A block then ends without waiting for its
// stores and an atomic (two round trips); with four rounds of blocks per launch
// that shortens the launch by more than the extra launch costs.
template <int PPS, bool SEP>
__global__ __launch_bounds__(256) void k_attn_paged(AttnPagedArgs a, float theta_log2) {
  const int h = blockIdx.x, b = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float qs[2][128];
  __shared__ float knew[128], vnew[128];
  __shared__ float sc[2][PPS * kPage];
  __shared__ float red[4][2][128];
  __shared__ float mstat[2], lstat[2];
  __shared__ int s_last;

  const int cap = a.max_pages * kPage;
  const int j0 = 2 * h;
  const int jj = tid >> 7, d = tid & 127;
  const float* qrow = a.qkv + (size_t)b * a.qkv_ld;
  const int q_dim = a.n_q * 128, kv_dim = a.n_kv * 128;
  const int* ptab = a.page_table + (size_t)b * a.max_pages;

  // ---- round trip 1: nothing here depends on the cache length
  const int p = a.kv_len[b];
  int pg[PPS];  // (entries past the table's end are read as its last and never used)
#pragma unroll
  for (int g = 0; g < PPS; ++g) {
    const int pidx = s * PPS + g;
    pg[g] = ptab[pidx < a.max_pages ? pidx : a.max_pages - 1];
  }
  // this wave's vector (waves 0, 1: query heads j0, j0+1; wave 2: the new key;
  // wave 3: the new value), lane l holding dimensions l and l + 64, and its gain
  const int col = wave < 2 ? (j0 + wave) * 128 : q_dim + (wave == 3 ? kv_dim : 0) + h * 128;
  const float x0 = qrow[col + lane], x1 = qrow[col + lane + 64];
  const uint16_t* gain = wave < 2 ? a.q_norm : a.k_norm;
  const uint16_t g0_bits = gain[lane], g1_bits = gain[lane + 64];

  const size_t orow = chunked(b, (j0 + jj) * 128 + d, a.o_ld);
  if (p < 0 || p >= cap) {
    if (s == 0) a.o[orow] = 0;
    return;
  }
  const int S = PPS * kPage;
  const int n_active = p / S + 1;
  if (s >= n_active) return;
  const int t0 = s * S, t1 = min(t0 + S, p + 1);
  const bool has_new = (s == n_active - 1);
  const int pgn = ptab[p / kPage];  // page of the new token (loaded ahead of the K/V)

  // ---- round trip 2: the split's K/V; thread (pi = tid>>4, c = tid&15) covers
  // positions t0 + 16g + pi, dims 8c..8c+7
  const int pi = tid >> 4, c = tid & 15;
  // All keys are requested before any value, so that the scores and the softmax
  // can start while the values are still arriving.  Every load is issued (lanes
  // with nothing to read take page 0 and bit g of `okm` stays clear), so the
  // compiler can count the loads in flight and wait only for the ones it needs.
  // Non-temporal: the cache is streamed once per frame and should not displace
  // the predictor weights that every step re-reads.
  uint4 kk[PPS], vv[PPS];
  size_t koff[PPS];
  uint32_t okm = 0;
  bool bad = false;
#pragma unroll
  for (int g = 0; g < PPS; ++g) {
    const int t = t0 + g * kPage + pi;
    const bool in = t < t1 && t != p;  // (t < t1 implies a page inside the table)
    const bool valid = pg[g] >= 0 && pg[g] < a.num_pages;
    bad = bad || (in && !valid);
    const bool ok = in && valid;
    okm |= ok ? (1u << g) : 0u;
    koff[g] = ((size_t)(ok ? pg[g] : 0) * a.n_kv + h) * (kPage * 128) + (size_t)pi * 128 + 8 * c;
    kk[g] = load_nt(reinterpret_cast<const uint4*>(a.k_pool + koff[g]));
  }
#pragma unroll
  for (int g = 0; g < PPS; ++g)
    vv[g] = load_nt(reinterpret_cast<const uint4*>(a.v_pool + koff[g]));
  if (bad && c == 0) atomicOr(a.status, QT_STATUS_BAD_PAGE);

  // q heads, and in the split holding p the new key and value, while the K/V
  // loads fly: one vector per wave, no block barrier until all are in LDS
  if (wave < 2 || has_new) {
    float v0 = x0, v1 = x1;
    if (wave < 3)  // the value is taken raw
      norm_rope_pair(v0, v1, bf2f(g0_bits), bf2f(g1_bits), a.eps, rope_inv_rev(lane, theta_log2), p);
    if (wave < 2) {
      qs[wave][lane] = v0 * kInvSqrtHd;
      qs[wave][lane + 64] = v1 * kInvSqrtHd;
    } else {
      const uint16_t b0 = f2bf(v0), b1 = f2bf(v1);
      if (pgn >= 0 && pgn < a.num_pages) {
        const size_t off = ((size_t)pgn * a.n_kv + h) * (kPage * 128) + (size_t)(p % kPage) * 128;
        uint16_t* dst = wave == 2 ? a.k_pool : a.v_pool;
        dst[off + lane] = b0;
        dst[off + lane + 64] = b1;
      } else if (wave == 2 && lane == 0) {
        atomicOr(a.status, QT_STATUS_BAD_PAGE);
      }
      float* nb = wave == 2 ? knew : vnew;
      nb[lane] = bf2f(b0);
      nb[lane + 64] = bf2f(b1);
    }
  }
  __syncthreads();

  float q0[8], q1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    q0[e] = qs[0][8 * c + e];
    q1[e] = qs[1][8 * c + e];
  }
#pragma unroll
  for (int g = 0; g < PPS; ++g) {
    const int t = t0 + g * kPage + pi;
    float kf[8];
    if (t == p) {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = knew[8 * c + e];
    } else {
      if (!((okm >> g) & 1u)) kk[g] = make_uint4(0, 0, 0, 0);  // bad page: zeros
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
    s0 = row_sum16(s0);
    s1 = row_sum16(s1);
    if (c == 0) {
      sc[0][g * kPage + pi] = (t < t1) ? s0 : -INFINITY;
      sc[1][g * kPage + pi] = (t < t1) ? s1 : -INFINITY;
    }
  }
  __syncthreads();

  // softmax statistics per head over this split: wave w < 2 takes head w, lane l
  // its positions l and l + 64 (wave reductions only, one barrier)
  const int n = t1 - t0;
  if (wave < 2) {
    const int u0 = lane, u1 = lane + 64;
    const float v0 = u0 < n ? sc[wave][u0] : -INFINITY;
    const float v1 = u1 < n ? sc[wave][u1] : -INFINITY;
    const float m = wave_max(fmaxf(v0, v1));
    const float e0 = u0 < n ? expf(v0 - m) : 0.f, e1 = u1 < n ? expf(v1 - m) : 0.f;
    const float sm = wave_sum(e0 + e1);
    if (u0 < n) sc[wave][u0] = e0;
    if (u1 < n) sc[wave][u1] = e1;
    if (lane == 0) {
      mstat[wave] = m;
      lstat[wave] = sm;
    }
  }
  __syncthreads();

  // weighted values
  float a0[8], a1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a0[e] = a1[e] = 0.f;
#pragma unroll
  for (int g = 0; g < PPS; ++g) {
    const int t = t0 + g * kPage + pi;
    if (t < t1) {
      const float w0 = sc[0][g * kPage + pi], w1 = sc[1][g * kPage + pi];
      float vf[8];
      if (t == p) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = vnew[8 * c + e];
      } else {
        if (!((okm >> g) & 1u)) vv[g] = make_uint4(0, 0, 0, 0);  // bad page: zeros
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
    a0[e] = sum_q4(a0[e]);
    a1[e] = sum_q4(a1[e]);
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
    bool over = false;
    a.o[orow] = f2h_chk(out / lstat[jj], over);
    if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
    return;
  }
  float* pp = a.part + (((size_t)b * a.n_q + j0 + jj) * a.n_splits + s) * 130;
  if (SEP) {  // merged by k_attn_merge, after this launch
    pp[2 + d] = out;
    if (d == 0) {
      pp[0] = mstat[jj];
      pp[1] = lstat[jj];
    }
    return;
  }
  // Publish this split's partial with device-coherent stores, wait until they
  // are performed, then count the split in.  The last split to arrive reads all
  // partials with device-coherent loads.  (A full agent-scope fence here would
  // write back and invalidate the whole L2 of the XCD once per block.)
  dev_store(pp + 2 + d, out);
  if (d == 0) {
    dev_store(pp, mstat[jj]);
    dev_store(pp + 1, lstat[jj]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned* cnt = &a.counters[(size_t)b * a.n_kv + h];
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (unsigned)(n_active - 1));
  }
  __syncthreads();
  if (!s_last) return;
  merge_splits<true>(a, b, j0 + jj, d, n_active, orow);
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The split partials of k_attn_paged<PPS, true>, merged: grid (KV head, session),
// thread (jj, d) for query head 2h + jj, dimension d.  Sessions with one split (the
// output is already written) or an out-of-range position (zeros written) are left.
__global__ __launch_bounds__(256) void k_attn_merge(AttnPagedArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int jj = tid >> 7, d = tid & 127;
  const int p = a.kv_len[b];
  if (p < 0 || p >= a.max_pages * kPage) return;
  const int n_active = p / (a.pages_per_split * kPage) + 1;
  if (n_active == 1) return;
  merge_splits<false>(a, b, 2 * h + jj, d, n_active, chunked(b, (2 * h + jj) * 128 + d, a.o_ld));
}

// ---------------------------------------------------------------------------
// Code-predictor attention over its short, preallocated, contiguous cache.
// Grid (kv head, session).  n_new (1 or 2) new positions pos0 .. pos0+n_new-1
// are normalised, rotated, appended, and each attends causally to positions
// 0 .. its own.  At most 16 positions: one thread group of 16 per position.
// The new vectors go one per wave (waves 0, 1: query heads 2h, 2h+1; wave 2: the
// key; wave 3: the value), lane l holding dimensions l and l + 64, the two halves
// of each RoPE pair: the norm is one wave reduction and the rotation stays in the
// lane, with no block barrier.  The softmax of all (new position, head) rows is
// one wave's work, a row of 16 lanes per row.
__global__ __launch_bounds__(256) void k_attn_pred(AttnPredArgs a, float theta_log2) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jj = tid >> 7, d = tid & 127;
  __shared__ float qs[2][2][128];
  __shared__ float kn[2][128], vn[2][128];
  __shared__ float sc[2][2][16];
  __shared__ float red[4][2][2][128];
  __shared__ float lsum[2][2];
  const int j0 = 2 * h;
  const int q_dim = a.n_q * 128, kv_dim = a.n_kv * 128;
  uint16_t* kbase = a.k_cache + (size_t)b * a.sess_stride;
  uint16_t* vbase = a.v_cache + (size_t)b * a.sess_stride;

  // one round trip: every cached position (thread group t = tid>>4 holds position
  // t, dims 8c..8c+7), this wave's vector of every new position and its gain
  const int t = tid >> 4, c = tid & 15;
  uint4 kq = make_uint4(0, 0, 0, 0), vq = make_uint4(0, 0, 0, 0);
  if (t < a.pos0) {
    const size_t off = ((size_t)t * a.n_kv + h) * 128 + 8 * c;
    kq = *reinterpret_cast<const uint4*>(kbase + off);
    vq = *reinterpret_cast<const uint4*>(vbase + off);
  }
  const int col = wave < 2 ? (j0 + wave) * 128 : q_dim + (wave == 3 ? kv_dim : 0) + h * 128;
  float x0[2] = {0.f, 0.f}, x1[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i < a.n_new) {
      const float* row = a.qkv + (size_t)(i * a.B + b) * a.qkv_ld + col;
      x0[i] = row[lane];
      x1[i] = row[lane + 64];
    }
  }
  const uint16_t* gain = wave < 2 ? a.q_norm : a.k_norm;
  const float g0 = bf2f(gain[lane]), g1 = bf2f(gain[lane + 64]);
  const double inv_rev = rope_inv_rev(lane, theta_log2);
  for (int i = 0; i < a.n_new; ++i) {
    const int pos = a.pos0 + i;
    float v0 = x0[i], v1 = x1[i];
    // q heads and the key: RMSNorm with the gain, then RoPE (the value is taken raw)
    if (wave < 3) norm_rope_pair(v0, v1, g0, g1, a.eps, inv_rev, pos);
    if (wave < 2) {
      qs[i][wave][lane] = v0 * kInvSqrtHd;
      qs[i][wave][lane + 64] = v1 * kInvSqrtHd;
    } else {
      const uint16_t b0 = f2bf(v0), b1 = f2bf(v1);
      const size_t off = ((size_t)pos * a.n_kv + h) * 128;
      uint16_t* dst = wave == 2 ? kbase : vbase;
      dst[off + lane] = b0;
      dst[off + lane + 64] = b1;
      float* nb = wave == 2 ? kn[i] : vn[i];
      nb[lane] = bf2f(b0);
      nb[lane + 64] = bf2f(b1);
    }
  }
  __syncthreads();

  const int n_pos = a.pos0 + a.n_new;
  float kf[8], vf[8];
  if (t < n_pos) {
    if (t >= a.pos0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kf[e] = kn[t - a.pos0][8 * c + e];
        vf[e] = vn[t - a.pos0][8 * c + e];
      }
    } else {
      kf[0] = bf_lo(kq.x); kf[1] = bf_hi(kq.x); kf[2] = bf_lo(kq.y); kf[3] = bf_hi(kq.y);
      kf[4] = bf_lo(kq.z); kf[5] = bf_hi(kq.z); kf[6] = bf_lo(kq.w); kf[7] = bf_hi(kq.w);
      vf[0] = bf_lo(vq.x); vf[1] = bf_hi(vq.x); vf[2] = bf_lo(vq.y); vf[3] = bf_hi(vq.y);
      vf[4] = bf_lo(vq.z); vf[5] = bf_hi(vq.z); vf[6] = bf_lo(vq.w); vf[7] = bf_hi(vq.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[e] = vf[e] = 0.f;
  }
  // scores for every (new position i, head hh)
  for (int i = 0; i < a.n_new; ++i) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(qs[i][hh][8 * c + e], kf[e], s);
      s = row_sum16(s);
      if (c == 0) sc[i][hh][t] = (t <= a.pos0 + i) ? s : -INFINITY;
    }
  }
  __syncthreads();
  // softmax: wave 0, lane (i, hh, u) = (lane >> 5, (lane >> 4) & 1, lane & 15)
  if (wave == 0) {
    const int i = lane >> 5, hh = (lane >> 4) & 1, u = lane & 15;
    if (i < a.n_new) {  // (rows of 16 lanes: uniform within each row)
      const bool in = u <= a.pos0 + i;
      const float v = in ? sc[i][hh][u] : -INFINITY;
      const float m = row_max16(v);
      const float e = in ? expf(v - m) : 0.f;
      const float l = row_sum16(e);
      sc[i][hh][u] = e;
      if (u == 0) lsum[i][hh] = l;
    }
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
        acc[e] = sum_q4(acc[e]);
      }
      if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][i][hh][8 * c + e] = acc[e];
      }
    }
  }
  __syncthreads();
  bool over = false;
  for (int i = 0; i < a.n_new; ++i) {
    const float out = red[0][i][jj][d] + red[1][i][jj][d] + red[2][i][jj][d] + red[3][i][jj][d];
    a.o[chunked(i * a.B + b, (j0 + jj) * 128 + d, a.o_ld)] = f2h_chk(out / lsum[i][jj], over);
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
}

// ---------------------------------------------------------------------------
// Frame entry: Talker input rows to fp32 with their sums of squares and the first
// norm's half input (predictor mode: the given post-norm hidden as the projection
// input), capacity check, codebook-0 candidates of predictor mode, attention
// counters cleared.
__global__ __launch_bounds__(256) void k_frame_begin(FrameBeginArgs a) {
  __shared__ float part[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  bool over = false;
  if (a.mode != QT_MODE_PREDICTOR) {
    float ss = 0.f;
    for (int i = tid; i < a.Ht; i += 256) {
      const size_t e = (size_t)b * a.Ht + i;
      const float v = bf2f(a.talker_in[e]);
      a.x_t[e] = v;
      a.u[chunked(b, i, a.B)] = f2h_chk(v * bf2f(a.gain[i]), over);
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) {
      a.ss_t[b] = part[0] + part[1] + part[2] + part[3];
      const int p = a.kv_len[b];
      if (p < 0 || p + 1 > a.capacity) atomicOr(a.status, QT_STATUS_KV_OVERFLOW);
    }
  } else {
    for (int i = tid; i < a.Ht; i += 256)
      a.u[chunked(b, i, a.B)] = f2h_chk(bf2f(a.h_in[(size_t)b * a.Ht + i]), over);
    unsigned long long* c0 = a.cand + (size_t)b * a.cand_ld;
    for (int k = tid; k < a.cand_ld; k += 256) c0[k] = k == 0 ? greedy_key(0.0f, a.tok0_in[b]) : 0ull;
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
  if (tid < a.n_kv) a.counters[(size_t)b * a.n_kv + tid] = 0u;
  if (a.pred_sync && b == 0)
    for (unsigned i = tid; i < kPredSyncWords; i += 256) a.pred_sync[i] = 0u;
}

// Best of n greedy-key candidates, reduced by the 64 lanes of a wave.
__device__ __forceinline__ unsigned long long best_key_wave(const unsigned long long* c, int n) {
  const int lane = threadIdx.x & 63;
  unsigned long long best = 0;
  for (int k = lane; k < n; k += 64) best = c[k] > best ? c[k] : best;
  return wave_max_u64(best);
}

// ---------------------------------------------------------------------------
// Token draws (qt_sampling).  Philox4x64-10 as defined by Salmon, Moraes, Dror and
// Shaw (SC 2011): per round, words 0 and 2 are multiplied by two 64-bit constants
// and the new words are (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)); the key advances by the Weyl increments (golden ratio, sqrt 3 - 1).
// Only the first output word of a block is used.
__device__ __forceinline__ uint64_t philox4x64_word0(uint64_t c0, uint64_t c1, uint64_t k0) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t c2 = 0, c3 = 0, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return c0;
}

// Float -> unsigned key with the same order (larger float, larger key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int kSampleSlots = 16;  // row entries per thread: rows up to 4096 entries

struct SampleSmem {
  uint32_t hist[256];
  float cval[QT_SAMPLER_MAX_TOP_K];
  int cidx[QT_SAMPLER_MAX_TOP_K];
  int eq[kSampleSlots][4];
  uint32_t digit;
  int above;
  int n_cand;
  int token;
};

// One draw over row[0, V) by the 256 threads of a block (every thread returns the
// token).  1. penalty and temperature; 2. the top_k-th largest score by a 4-pass
// radix select over order keys (8 bits per pass), entries equal to it ranked by
// index; 3. the candidates sorted by one wave (bitonic, (score desc, index asc));
// 4. weights, running sums (wave scan), the top-p cut and the draw.
__device__ int sample_row(const float* row, int V, float temperature, float top_p,
                          float penalty, int top_k, const uint32_t* seen, float u,
                          SampleSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ne = (V + 255) >> 8;
  uint32_t key[kSampleSlots];
#pragma unroll
  for (int e = 0; e < kSampleSlots; ++e) {
    const int i = tid + 256 * e;
    key[e] = 0u;  // below every score: entries past V and NaN scores
    if (e < ne && i < V) {
      float x = row[i];
      if (seen && ((seen[i >> 5] >> (i & 31)) & 1u)) x = x > 0.f ? x / penalty : x * penalty;
      const float z = x / temperature;
      if (z == z) key[e] = order_key(z);
    }
  }
  const int k = top_k < V ? top_k : V;
  uint32_t prefix = 0, pmask = 0;
  int kr = k;
  if (tid == 0) sm.n_cand = 0;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    sm.hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kSampleSlots; ++e)
      if (e < ne && (key[e] & pmask) == prefix) atomicAdd(&sm.hist[(key[e] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 4l..4l+3; "above" counts the keys in higher bins
      const uint32_t h0 = sm.hist[4 * lane], h1 = sm.hist[4 * lane + 1];
      const uint32_t h2 = sm.hist[4 * lane + 2], h3 = sm.hist[4 * lane + 3];
      const uint32_t own = h0 + h1 + h2 + h3;
      uint32_t suf = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_down(suf, off);
        if (lane + off < 64) suf += t;
      }
      uint32_t above = suf - own;
      const uint32_t hs[4] = {h3, h2, h1, h0};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < (uint32_t)kr && (uint32_t)kr <= above + hs[q]) {
          sm.digit = 4 * lane + 3 - q;
          sm.above = (int)above;
        }
        above += hs[q];
      }
    }
    __syncthreads();
    prefix |= sm.digit << shift;
    pmask |= 255u << shift;
    kr -= sm.above;
  }
  // candidates: every key above the threshold, and the kr lowest-index keys equal to it
  int rank_base = 0;
  {
    uint64_t masks[kSampleSlots];
#pragma unroll
    for (int e = 0; e < kSampleSlots; ++e) {
      masks[e] = __ballot(e < ne && key[e] == prefix);
      if (lane == 0 && e < ne) sm.eq[e][wave] = __popcll(masks[e]);
    }
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int e = 0; e < kSampleSlots; ++e) {
      if (e < ne) {
        const int i = tid + 256 * e;
        bool take = key[e] > prefix;
        if (key[e] == prefix) {
          int rank = rank_base + __popcll(masks[e] & below);
          for (int w = 0; w < wave; ++w) rank += sm.eq[e][w];
          take = rank < kr;
        }
        if (take) {
          const int slot = atomicAdd(&sm.n_cand, 1);
          sm.cval[slot] = key[e] ? key_value(key[e]) : -INFINITY;
          sm.cidx[slot] = i;
        }
        rank_base += sm.eq[e][0] + sm.eq[e][1] + sm.eq[e][2] + sm.eq[e][3];
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    float v = lane < k ? sm.cval[lane] : -INFINITY;
    int idx = lane < k ? sm.cidx[lane] : 0x7fffffff;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const float ov = __shfl_xor(v, stride);
        const int oi = __shfl_xor(idx, stride);
        const bool desc = (lane & size) == 0 || size == 64;
        const bool lower = (lane & stride) == 0;
        const bool greater = v > ov || (v == ov && idx < oi);
        if (greater != (lower == desc)) {
          v = ov;
          idx = oi;
        }
      }
    }
    const float vmax = __shfl(v, 0);
    float w = 0.f;
    if (lane < k) w = vmax == -INFINITY ? (lane == 0 ? 1.f : 0.f) : expf(v - vmax);
    float cum = w;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(cum, off);
      if (lane >= off) cum += t;
    }
    const float total = __shfl(cum, k - 1);
    int m = __popcll(__ballot(lane < k && cum < top_p * total)) + 1;
    m = m < k ? m : k;
    const float r = u * __shfl(cum, m - 1);
    const uint64_t hit = __ballot(lane < m && cum > r);
    const int j = hit ? __ffsll((unsigned long long)hit) - 1 : m - 1;
    const int tok = __shfl(idx, j);
    if (lane == 0) sm.token = (tok >= 0 && tok < V) ? tok : 0;
  }
  __syncthreads();
  return sm.token;
}

// Session b's draw of `row` with its parameters and random stream; thread 0 writes
// the token to *tok_out and, for codebook 0, adds it to the seen set.
__device__ int sample_session(const SamplerArgs& s, const SampleRow& row, int b,
                              int32_t* tok_out, uint32_t* status, SampleSmem& sm) {
  const qt_sampler_params p = s.params[2 * b + row.group];
  const uint64_t seed = s.seed[b];
  const uint32_t ctr = (uint32_t)s.counter[b];
  float T = p.temperature, tp = p.top_p, pen = p.repetition_penalty;
  int tk = p.top_k;
  const bool ok = T > 0.f && T < INFINITY && tp > 0.f && tp <= 1.f && pen >= 1.f &&
                  pen < INFINITY && tk >= 1 && tk <= QT_SAMPLER_MAX_TOP_K;
  if (!ok) {
    if (threadIdx.x == 0) atomicOr(status, QT_STATUS_BAD_SAMPLER);
    T = 1.f, tp = 1.f, pen = 1.f, tk = 1;
  }
  const uint64_t x = philox4x64_word0(ctr, (uint64_t)row.codebook, seed);
  const float u = (float)(uint32_t)(x >> 40) * 0x1p-24f;
  uint32_t* seen = (row.group == 0 && s.seen0) ? s.seen0 + (size_t)b * s.seen_ld : nullptr;
  const int tok = sample_row(row.logits + (size_t)b * row.ld, row.V, T, tp, pen, tk, seen, u, sm);
  if (threadIdx.x == 0) {
    *tok_out = tok;
    if (seen) seen[tok >> 5] |= 1u << (tok & 31);
  }
  return tok;
}

// qt_sample: row r drawn with its own parameters, seed and counter.
__global__ __launch_bounds__(256) void k_sample_rows(SampleRowsArgs a) {
  __shared__ SampleSmem sm;
  const int r = blockIdx.x;
  SamplerArgs s{};
  s.params = a.params + r;  // the draw reads params[2 b + group] with b = 0, group = 0
  s.seed = a.seed + r;
  s.counter = a.counter + r;
  s.seen0 = a.seen ? a.seen + (size_t)r * a.seen_ld : nullptr;
  s.seen_ld = a.seen_ld;
  SampleRow row{a.logits + (size_t)r * a.ld, 0, a.V, 0, a.codebook};
  sample_session(s, row, 0, a.tokens + r, a.status, sm);
}

// Predictor step input: row E_step[token] (token = forced, or the previous step's
// greedy token) to fp32, with its sum of squares and the first norm's half input.
__global__ __launch_bounds__(256) void k_embed(EmbedArgs a) {
  __shared__ float part[4];
  __shared__ int s_tok;
  __shared__ SampleSmem sm;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (a.sample) {
    const int drawn = sample_session(a.smp, a.row, b, a.tokens + (size_t)b * a.ncb + a.row.codebook,
                                     a.status, sm);
    if (tid == 0) s_tok = a.forced ? a.forced[(size_t)b * a.ncb + a.step - 1] : drawn;
  } else if (a.forced) {
    if (tid == 0) s_tok = a.forced[(size_t)b * a.ncb + a.step - 1];
  } else if (tid < 64) {
    const unsigned long long k =
        best_key_wave(a.cand + ((size_t)(a.step - 1) * a.B + b) * a.cand_ld, a.n_cand);
    if (tid == 0) s_tok = key_index(k);
  }
  __syncthreads();
  int tok = s_tok;
  if (tok < 0 || tok >= a.vocab) {
    if (tid == 0) atomicOr(a.status, QT_STATUS_BAD_TOKEN);
    tok = 0;
  }
  const uint16_t* src = a.table + (size_t)tok * a.H;
  const int m = a.row_off + b;
  float* dst = a.x + (size_t)m * a.H;
  float ss = 0.f;
  bool over = false;
  for (int i = tid; i < a.H; i += 256) {
    const float v = bf2f(src[i]);
    dst[i] = v;
    a.u[chunked(m, i, a.u_ld)] = f2h_chk(v * bf2f(a.gain[i]), over);
    ss = fmaf(v, v, ss);
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  for (int sl = tid; sl < a.ss_slots; sl += 256)
    a.ss[(size_t)sl * a.ss_ld + m] = sl == 0 ? part[0] + part[1] + part[2] + part[3] : 0.f;
}

// Frame exit, one block per session: each codebook's candidates reduced to its
// greedy token, and the session's cache length advanced.
__global__ __launch_bounds__(256) void k_frame_end(FrameEndArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  if (a.sample) {
    // the predictor's draws were written by the embedding gathers; this block draws
    // the last one (codebook 0 in Talker mode), then advances the cache length
    __shared__ SampleSmem sm;
    if (a.mode == QT_MODE_PREDICTOR && wave == 0) {
      const unsigned long long best = best_key_wave(a.cand + (size_t)b * a.cand_ld, a.n_cand0);
      if (tid == 0) a.tokens[(size_t)b * a.ncb] = key_index(best);
    }
    if (a.mode == QT_MODE_TALKER && tid >= 1 && tid < a.ncb) a.tokens[(size_t)b * a.ncb + tid] = -1;
    sample_session(a.smp, a.row, b, a.tokens + (size_t)b * a.ncb + a.row.codebook, a.status, sm);
    if (tid == 0 && a.mode != QT_MODE_PREDICTOR) {
      const int p = a.kv_len[b];
      if (p >= 0 && p + 1 <= a.capacity) a.kv_len[b] = p + 1;
    }
    return;
  }
  for (int k = wave; k < a.ncb; k += 4) {
    const unsigned long long best = best_key_wave(
        a.cand + ((size_t)k * a.B + b) * a.cand_ld, k == 0 ? a.n_cand0 : a.n_cand);
    if ((tid & 63) == 0) {
      int tok = key_index(best);
      if (a.mode == QT_MODE_TALKER && k > 0) tok = -1;
      a.tokens[(size_t)b * a.ncb + k] = tok;
    }
  }
  if (tid == 0 && a.mode != QT_MODE_PREDICTOR) {
    const int p = a.kv_len[b];
    if (p >= 0 && p + 1 <= a.capacity) a.kv_len[b] = p + 1;
  }
}

// ---------------------------------------------------------------------------
// Per-row symmetric INT8: s = max|w| / 127 (IEEE divide), q = clamp(rint(w / s), +-127).
// With q_half the integers go to half tiles instead (exact: |q| <= 127).
__global__ __launch_bounds__(256) void k_quantize(const uint16_t* w, long long cols, int8_t* q,
                                                  uint16_t* q_half, long long q_stride,
                                                  float* scale, long long s_stride, int tiled_K,
                                                  long long row0) {
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
  for (long long k = tid; k < cols; k += 256) {
    float v = 0.f;
    if (sc != 0.f) {
      v = rintf(__fdiv_rn(bf2f(row[k]), sc));
      v = fminf(fmaxf(v, -127.f), 127.f);
    }
    if (q_half) {
      q_half[tiled_bf16((int)(row0 + r * q_stride), (int)k, tiled_K)] = f2h(v);
    } else {
      const size_t o = tiled_K ? tiled_i8((int)(row0 + r * q_stride), (int)k, tiled_K)
                               : (size_t)(r * q_stride + k);
      q[o] = (int8_t)(int)v;
    }
  }
}

// ---------------------------------------------------------------------------
// Scheduler helpers, one block per batch slot.
// Setup: the slot's cache length, page-table row, Talker input row and forced tokens.
// On a session's first frame its row comes from the host mirror written at open
// (read at system scope, so no stale cache line is used); a page appended this
// frame is also stored into the session's device row.  Padding slots get length 0,
// the padding page and a zero input.
// Collect: the slot's outputs copied to its session's result rows and, where asked,
// the end-of-speech decision: the entry wins the codebook-0 choice (lowest index
// wins ties) -> the frame number goes to the device flag and the host buffer.
__global__ __launch_bounds__(256) void k_sched_setup(SchedSetupArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int sess = a.slot_session[b];
  int32_t* row = a.page_table + (size_t)b * a.max_pages;
  uint4* in_row = reinterpret_cast<uint4*>(a.talker_in + (size_t)b * a.H);
  if (sess < 0) {
    for (int i = tid; i < a.max_pages; i += 256) row[i] = a.pad_page;
    for (int i = tid; i < a.H / 8; i += 256) in_row[i] = make_uint4(0, 0, 0, 0);
    if (a.forced)
      for (int i = tid; i < a.ncb; i += 256) a.forced[(size_t)b * a.ncb + i] = 0;
    if (a.params) {
      for (int i = tid; i < a.seen_ld; i += 256) a.seen[(size_t)b * a.seen_ld + i] = 0u;
      if (tid < 2) a.params[2 * b + tid] = qt_sampler_params{1.f, 1.f, 1.f, 1};
      if (tid == 2) a.seed[b] = 0;
    }
    if (tid == 0) a.kv_len[b] = 0;
    return;
  }
  int32_t* dev_row = a.sess_pages + (size_t)sess * a.max_pages;
  const int first = a.slot_first[b];
  for (int i = tid; i < a.max_pages; i += 256) {
    int32_t v;
    if (i == a.new_index[b]) {
      v = a.new_page[b];
    } else if (first >= 0) {
      v = i < first ? __hip_atomic_load(a.host_pages + (size_t)sess * a.max_pages + i,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
                    : a.pad_page;
    } else {
      v = dev_row[i];
    }
    row[i] = v;
    if (first >= 0 || i == a.new_index[b]) dev_row[i] = v;
  }
  const uint4* in = reinterpret_cast<const uint4*>(a.in_ptr[b]);
  for (int i = tid; i < a.H / 8; i += 256) in_row[i] = in[i];
  if (a.forced) {
    const int32_t* f = a.forced_ptr[b];
    for (int i = tid; i < a.ncb; i += 256) a.forced[(size_t)b * a.ncb + i] = f ? f[i] : 0;
  }
  if (a.params) {
    uint32_t* dst = a.seen + (size_t)b * a.seen_ld;
    const uint32_t* src = a.sess_seen + (size_t)sess * a.seen_ld;
    for (int i = tid; i < a.seen_ld; i += 256) dst[i] = first >= 0 ? 0u : src[i];
    if (tid < 2) a.params[2 * b + tid] = a.slot_params[b][tid];
    if (tid == 2) a.seed[b] = a.slot_seed[b];
  }
  if (tid == 0) {
    a.kv_len[b] = a.slot_len[b];
    if (first >= 0) a.flags[sess] = 0;
  }
}

// Grid (slot, part): the slot's rows are copied by kSchedCollectParts blocks.
constexpr int kSchedCollectParts = 16;

__global__ __launch_bounds__(256) void k_sched_collect(SchedCollectArgs a) {
  const int b = blockIdx.x, part = blockIdx.y, tid = threadIdx.x;
  const int sess = a.slot_session[b];
  if (sess < 0) return;
  const int t = part * 256 + tid, stride = kSchedCollectParts * 256;
  const float4* l0 = reinterpret_cast<const float4*>(a.logits0 + (size_t)b * a.talker_vocab);
  float4* r0 = reinterpret_cast<float4*>(a.res_logits0 + (size_t)sess * a.talker_vocab);
  for (int i = t; i < a.talker_vocab / 4; i += stride) r0[i] = l0[i];
  const float4* lp = reinterpret_cast<const float4*>(a.logits_pred + (size_t)b * a.pred_elems);
  float4* rp = reinterpret_cast<float4*>(a.res_pred + (size_t)sess * a.pred_elems);
  for (int i = t; i < a.pred_elems / 4; i += stride) rp[i] = lp[i];
  if (part != 0) return;
  for (int i = tid; i < a.ncb; i += 256)
    a.res_tokens[(size_t)sess * a.ncb + i] = a.tokens[(size_t)b * a.ncb + i];
  if (a.sampled)
    for (int i = tid; i < a.seen_ld; i += 256)
      a.sess_seen[(size_t)sess * a.seen_ld + i] = a.seen[(size_t)b * a.seen_ld + i];
  const bool check = a.eos_index >= 0 && a.slot_check[b] > 0 && a.flags[sess] == 0;
  __shared__ int s_greedy;
  if (a.sampled && check) {
    // the greedy codebook-0 choice (lowest index wins ties; NaN never chosen)
    __shared__ unsigned long long best[4];
    const float* lg = a.logits0 + (size_t)b * a.talker_vocab;
    unsigned long long k = 0ull;
    for (int v = tid; v < a.cb0_range; v += 256) {
      const float x = lg[v];
      const unsigned long long c = x == x ? greedy_key(x, v) : 0ull;
      k = c > k ? c : k;
    }
    k = wave_max_u64(k);
    if ((tid & 63) == 0) best[tid >> 6] = k;
    __syncthreads();
    if (tid == 0) {
      unsigned long long m = best[0];
      for (int w = 1; w < 4; ++w) m = best[w] > m ? best[w] : m;
      s_greedy = key_index(m);
    }
    __syncthreads();
  }
  if (tid == 0 && check) {
    const float* lg = a.logits0 + (size_t)b * a.talker_vocab;
    const int t0 = a.sampled ? s_greedy : a.tokens[(size_t)b * a.ncb];
    const int e = a.eos_index;
    bool end = false;
    if (t0 >= 0 && t0 < a.cb0_range)
      end = e == t0 || (e < t0 ? lg[e] >= lg[t0] : lg[e] > lg[t0]);
    if (end) {
      a.flags[sess] = a.slot_check[b];
      __hip_atomic_store(a.host_flags + sess, a.slot_check[b], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// ---------------------------------------------------------------------------
// Prompt prefill.  Entry, one block per row: the row's sequence and position
// (sequences are packed in order; rows past the last one are padding, set to
// zero), the residual x, the first norm's half input and its sum of squares.
__global__ __launch_bounds__(256) void k_prefill_begin(PrefillBeginArgs a) {
  __shared__ float part[4];
  __shared__ int s_seq;
  const int r = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) {
    int seq = -1, pos = 0;
    for (int q = 0; q < a.max_seqs; ++q) {
      const int lo = a.seq_start[q], hi = a.seq_start[q + 1];
      if (lo <= r && r < hi) {
        seq = q;
        pos = r - lo;
        break;
      }
    }
    s_seq = seq;
    a.rowinfo[2 * r] = seq;
    a.rowinfo[2 * r + 1] = pos;
  }
  __syncthreads();
  const bool live = s_seq >= 0;
  float ss = 0.f;
  bool over = false;
  for (int i = tid; i < a.H; i += 256) {
    const float v = live ? bf2f(a.embeds[(size_t)r * a.H + i]) : 0.f;
    a.x[(size_t)r * a.H + i] = v;
    a.u[chunked(r, i, a.R)] = f2h_chk(v * bf2f(a.gain[i]), over);
    ss = fmaf(v, v, ss);
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) a.ss[r] = part[0] + part[1] + part[2] + part[3];
}

// Per (kQkRows rows, KV head h): query heads 2h, 2h+1 and key head h normalised and
// rotated at each row's position (the same arithmetic as a decode step), one vector
// per wave (waves 0, 1: the query heads; wave 2: the key; wave 3: the value), lane l
// holding dimensions l and l + 64; q is stored back scaled by 1/sqrt(128), the key
// (bf16) and the raw value go to the page slot.  All of the block's rows are loaded
// before any is used, and the rotation's frequency is computed once per lane.
constexpr int kQkRows = 4;
__global__ __launch_bounds__(256) void k_prefill_qk(PrefillQkArgs a, float theta_log2) {
  const int r0 = blockIdx.x * kQkRows, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q_dim = a.n_q * 128, kv_dim = a.n_kv * 128;
  const int col = wave < 2 ? (2 * h + wave) * 128 : q_dim + (wave == 3 ? kv_dim : 0) + h * 128;
  int seq[kQkRows], pos[kQkRows];
  float v0[kQkRows], v1[kQkRows];
#pragma unroll
  for (int rr = 0; rr < kQkRows; ++rr) {
    const int r = r0 + rr;
    const bool in = r < a.R;
    const float* row = a.qkv + (size_t)(in ? r : 0) * a.qkv_ld;
    seq[rr] = in ? a.rowinfo[2 * r] : -1;
    pos[rr] = in ? a.rowinfo[2 * r + 1] : 0;
    v0[rr] = row[col + lane];
    v1[rr] = row[col + lane + 64];
  }
  const uint16_t* gain = wave < 2 ? a.q_norm : a.k_norm;
  const float g0 = bf2f(gain[lane]), g1 = bf2f(gain[lane + 64]);
  const double inv_rev = rope_inv_rev(lane, theta_log2);
#pragma unroll
  for (int rr = 0; rr < kQkRows; ++rr) {
    const int p = seq[rr] >= 0 ? pos[rr] : 0;
    if (wave < 3)  // the value is taken raw
      norm_rope_pair(v0[rr], v1[rr], g0, g1, a.eps, inv_rev, p);
  }
  if (wave < 2) {
#pragma unroll
    for (int rr = 0; rr < kQkRows; ++rr) {
      if (r0 + rr >= a.R) break;
      float* row = a.qkv + (size_t)(r0 + rr) * a.qkv_ld;
      row[col + lane] = v0[rr] * kInvSqrtHd;
      row[col + lane + 64] = v1[rr] * kInvSqrtHd;
    }
    return;
  }
  uint16_t* dst = wave == 2 ? a.k_pool : a.v_pool;
#pragma unroll
  for (int rr = 0; rr < kQkRows; ++rr) {
    const int sq = seq[rr], p = pos[rr];
    if (sq < 0) continue;  // (also rows past R)
    if (p >= a.max_pages * kPage) {
      if (wave == 2 && lane == 0) atomicOr(a.status, QT_STATUS_KV_OVERFLOW);
      continue;
    }
    const int pg = a.page_table[(size_t)sq * a.max_pages + p / kPage];
    if (pg < 0 || pg >= a.num_pages) {
      if (wave == 2 && lane == 0) atomicOr(a.status, QT_STATUS_BAD_PAGE);
      continue;
    }
    const size_t off = ((size_t)pg * a.n_kv + h) * (kPage * 128) + (size_t)(p % kPage) * 128;
    dst[off + lane] = f2bf(v0[rr]);
    dst[off + lane + 64] = f2bf(v1[rr]);
  }
}

// Causal attention over packed sequences on the matrix cores.  Block (64-row
// tile, KV head h, split z), eight waves: wave w serves rows 16(w/2) .. +15 of the
// tile for query head 2h + w%2, so every staged key block serves 128 query rows.
// For each sequence present in the tile, keys come in blocks of KB (64: four
// pages), blocks z, z + n_splits, ... to this split, staged through LDS: K as half
// [key][dim], V as half [dim][key'] with the keys of each 32-key group in the
// order the products below take them.  The sequence's page indices are staged in LDS first
// (a prompt has fewer than 4096 positions, so at most 256 pages), and the K/V
// pieces of the next kPfRing key blocks are always in flight: each is requested
// unconditionally (a block past the split's last re-reads the last; positions past
// the tile's rows or on a bad page are zeroed when staged), so that no wait for a
// page index or for a later block holds up the current one.  The split writes its
// unnormalised output, max and sum per (row, head); k_prefill_attn_merge combines
// the splits in order.
// The products are taken transposed, so that a lane holds one query row: lane l
// (i = l & 15, g = l >> 4) owns row i of the wave's 16.  Per block of keys:
//   S^T = K Q^T  (v_mfma_f32_16x16x32_f16, K from LDS as the A operand, the
//                 row's Q as B; KB/16 key tiles x 4 dim steps): lane l holds the
//                 scores of its row for keys 16 t + 4g + e (e < 4);
//   online softmax in the lane: max and sum over its KB/4 scores, then over the
//                 four lanes of the row (lane swaps), one rescale factor per lane;
//   O^T += V^T P^T, one step per 32-key group: the lane's 8 probabilities of the
//                 group, as halves, are the B operand directly (MFMA K index
//                 8g + j <-> key 4g + j, 16 + 4g + j - 4 of the group), V^T staged
//                 in that key order is A; O^T's lane l holds row i, dims
//                 16 nb + 4g + e.
constexpr int kKsLd = 136;  // half elements per staged key row (bank spread)
constexpr int kAttnRows = 64;
constexpr int kPfMaxPages = QT_PREFILL_MAX_ROWS / kPage;
constexpr int kPfRing = 2;  // key blocks in flight
constexpr int kPfKeys = 64;  // keys per staged block

// column of key k (0..31) of a 32-key group in the staged V^T: the order the
// products take them
__device__ __forceinline__ int vt_col(int k) {
  return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3);
}

template <int KB>
__global__ __launch_bounds__(512) void k_prefill_attn(PrefillAttnArgs a) {
  constexpr int NG = KB / 32;       // 32-key groups per block (one P.V step each)
  constexpr int VLD = KB + 8;       // half elements per staged dim row of V^T
  __shared__ __align__(16) _Float16 Ks[KB * kKsLd];
  __shared__ __align__(16) _Float16 Vt[128 * VLD];
  __shared__ int t_seq[kAttnRows], t_pos[kAttnRows];
  __shared__ int s_pg[kPfMaxPages];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, qg = lane >> 4, rg = wave >> 1;
  const int h = blockIdx.y, r0 = kAttnRows * blockIdx.x, qh = 2 * h + (wave & 1);
  const int z = blockIdx.z, nz = a.n_splits;
  if (tid < kAttnRows) {
    const int r = r0 + tid;
    t_seq[tid] = r < a.R ? a.rowinfo[2 * r] : -1;
    t_pos[tid] = r < a.R ? a.rowinfo[2 * r + 1] : 0;
  }
  // Q^T operand: row 16 rg + i of the tile, dims [32 ks + 8 qg, +8), already scaled
  // by 1/sqrt(128), times log2(e): scores, maxima and the partials' max are in
  // base-2 units, so every exponential is one exp2
  f16x8 qf[4];
  {
    const int r = r0 + 16 * rg + i;
    const float* qp = a.qkv + (size_t)(r < a.R ? r : 0) * a.qkv_ld + qh * 128 + 8 * qg;
    constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float4 x0 = *reinterpret_cast<const float4*>(qp + 32 * ks);
      const float4 x1 = *reinterpret_cast<const float4*>(qp + 32 * ks + 4);
      qf[ks] = f16x8{(_Float16)(x0.x * kLog2e), (_Float16)(x0.y * kLog2e), (_Float16)(x0.z * kLog2e),
                     (_Float16)(x0.w * kLog2e), (_Float16)(x1.x * kLog2e), (_Float16)(x1.y * kLog2e),
                     (_Float16)(x1.z * kLog2e), (_Float16)(x1.w * kLog2e)};
    }
  }
  __syncthreads();
  const int row_seq = t_seq[16 * rg + i], row_pos = t_pos[16 * rg + i];
  f32x4 O[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) O[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  int seq_lo = 0x7fffffff, seq_hi = -1;
  for (int r = 0; r < kAttnRows; ++r)
    if (t_seq[r] >= 0) {
      seq_lo = t_seq[r] < seq_lo ? t_seq[r] : seq_lo;
      seq_hi = t_seq[r] > seq_hi ? t_seq[r] : seq_hi;
    }
  const size_t head_off = (size_t)h * (kPage * 128);
  const size_t page_elems = (size_t)a.n_kv * (kPage * 128);
  // staging pieces of 16 bytes, NG of each per thread: K piece (key (tid >> 4) +
  // 32 p, dims 8 (tid & 15)), V piece (key (tid & 31) + 32 p, dims 8 (tid >> 5))
  const int kkey = tid >> 4, kd8 = tid & 15, vkey = tid & 31, vd8 = tid >> 5;
  const int vcol = vt_col(vkey);
  for (int seq = seq_lo; seq <= seq_hi; ++seq) {
    int pmax = -1;
    for (int r = 0; r < kAttnRows; ++r)
      if (t_seq[r] == seq && t_pos[r] > pmax) pmax = t_pos[r];
    if (pmax < 0) continue;
    const int nblk = pmax / KB + 1;
    if (z >= nblk) continue;
    const int cnt = (nblk - z + nz - 1) / nz;  // key blocks z, z + nz, ... of this split
    const int npg = min(min(nblk * (KB / kPage), a.max_pages), kPfMaxPages);
    __syncthreads();  // the previous sequence's page indices are no longer read
    for (int pi = tid; pi < npg; pi += 512) {
      const int pg = a.page_table[(size_t)seq * a.max_pages + pi];
      s_pg[pi] = (pg >= 0 && pg < a.num_pages) ? pg : -1;
    }
    __syncthreads();
    // element offset of the piece (key, d8) of the split's key block n (clamped to
    // its last), and whether it holds a live key
    auto piece = [&](int n, int key, int d8, bool& live) -> size_t {
      const int kpos = KB * (z + nz * min(n, cnt - 1)) + key, pi = kpos >> 4;
      const int pg = pi < npg ? s_pg[pi] : -1;
      live = n < cnt && kpos <= pmax && pg >= 0;
      return (size_t)(pg >= 0 ? pg : 0) * page_elems + head_off + (size_t)(kpos & 15) * 128 + 8 * d8;
    };
    uint4 kr[kPfRing][NG], vr[kPfRing][NG];
    bool klive[kPfRing][NG], vlive[kPfRing][NG];
    auto request = [&](int d, int n) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        kr[d][g] = *reinterpret_cast<const uint4*>(a.k_pool + piece(n, kkey + 32 * g, kd8, klive[d][g]));
        vr[d][g] = *reinterpret_cast<const uint4*>(a.v_pool + piece(n, vkey + 32 * g, vd8, vlive[d][g]));
      }
    };
#pragma unroll
    for (int d = 0; d < kPfRing; ++d) request(d, d);
    const bool row_live = row_seq == seq;
    for (int n0 = 0; n0 < cnt; n0 += kPfRing) {
#pragma unroll
      for (int d = 0; d < kPfRing; ++d) {
        const int n = n0 + d, kb = z + nz * n;
        __syncthreads();  // the previous block of keys is consumed
        if (n < cnt) {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const uint4 kq = klive[d][g] ? kr[d][g] : make_uint4(0, 0, 0, 0);
            const uint4 vq = vlive[d][g] ? vr[d][g] : make_uint4(0, 0, 0, 0);
            const uint32_t kw[4] = {kq.x, kq.y, kq.z, kq.w};
            const uint32_t vw[4] = {vq.x, vq.y, vq.z, vq.w};
            f16x8 kh;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              kh[2 * w] = (_Float16)bf_lo(kw[w]);
              kh[2 * w + 1] = (_Float16)bf_hi(kw[w]);
              Vt[(8 * vd8 + 2 * w) * VLD + 32 * g + vcol] = (_Float16)bf_lo(vw[w]);
              Vt[(8 * vd8 + 2 * w + 1) * VLD + 32 * g + vcol] = (_Float16)bf_hi(vw[w]);
            }
            *reinterpret_cast<f16x8*>(Ks + (kkey + 32 * g) * kKsLd + 8 * kd8) = kh;
          }
        }
        __syncthreads();
        request(d, n + kPfRing);  // the ring slot is free: key block n + kPfRing
        if (n >= cnt) continue;
        // S^T for the block's 2 NG key tiles: lane l holds its row's scores for
        // keys KB kb + 16 t + 4g + e
        f32x4 S[2 * NG];
#pragma unroll
        for (int t = 0; t < 2 * NG; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int t = 0; t < 2 * NG; ++t) {
            const f16x8 ka = *reinterpret_cast<const f16x8*>(Ks + (16 * t + i) * kKsLd + 32 * ks + 8 * qg);
            S[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[ks], S[t], 0, 0, 0);
          }
        float sc[8 * NG];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2 * NG; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = KB * kb + 16 * t + 4 * qg + e;
            sc[4 * t + e] = (row_live && k <= row_pos) ? S[t][e] : -INFINITY;
            mx = fmaxf(mx, sc[4 * t + e]);
          }
        const float mn = fmaxf(m, max_q4(mx));
        const float scale = mn == -INFINITY ? 1.f : exp2f(m - mn);
        float rs = 0.f;
        f16x8 pb[NG];  // 32-key group g: MFMA K index 8 qg + j <-> tile 2g + (j >> 2), e = j & 3
#pragma unroll
        for (int j = 0; j < 8 * NG; ++j) {
          const float p = sc[j] == -INFINITY ? 0.f : exp2f(sc[j] - mn);
          rs += p;
          pb[j >> 3][j & 7] = (_Float16)p;
        }
        l = l * scale + sum_q4(rs);
        m = mn;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) O[nb][e] *= scale;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const f16x8 va = *reinterpret_cast<const f16x8*>(Vt + (16 * nb + i) * VLD + 32 * g + 8 * qg);
            O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[g], O[nb], 0, 0, 0);
          }
        }
      }
    }
  }
  // O^T: lane l holds row 16 rg + i, dims 16 nb + 4g + e; the four lanes of a row
  // hold the same max and sum
  const int row = r0 + 16 * rg + i;
  if (row < a.R) {
    float* pp = a.part + ((size_t)(row * a.n_q + qh) * nz + z) * 130;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) pp[16 * nb + 4 * qg + e] = O[nb][e];  // (partials: 520-byte rows)
    if (qg == 0) {
      pp[128] = m;
      pp[129] = l;
    }
  }
}

// Split merge, block (16-row tile, KV head h): thread t serves (row t/16, query
// head 2h + (t/8)%2), dims 16(t%8) .. +15; splits combined in order with weights
// exp(m_z - max_z m), the half output written chunked for the o projection.
__global__ __launch_bounds__(256) void k_prefill_attn_merge(PrefillAttnArgs a) {
  const int tid = threadIdx.x, h = blockIdx.y, r0 = 16 * blockIdx.x;
  const int pair = tid >> 3, sub = tid & 7, row = r0 + (pair >> 1), qh = 2 * h + (pair & 1);
  const int nz = a.n_splits;
  const float* pp = a.part + (size_t)(row * a.n_q + qh) * nz * 130;
  float M = -INFINITY;
  for (int z = 0; z < nz; ++z) M = fmaxf(M, pp[z * 130 + 128]);
  float acc[16], L = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  for (int z = 0; z < nz; ++z) {
    const float mz = pp[z * 130 + 128];
    const float w = mz == -INFINITY ? 0.f : exp2f(mz - M);  // (maxima in base-2 units)
    L = fmaf(w, pp[z * 130 + 129], L);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = fmaf(w, pp[z * 130 + 16 * sub + e], acc[e]);
  }
  const float inv = (a.rowinfo[2 * row] >= 0 && L > 0.f) ? 1.f / L : 0.f;
  uint32_t packed[8];
  bool over = false;
#pragma unroll
  for (int w = 0; w < 8; ++w)
    packed[w] = (uint32_t)f2h_chk(acc[2 * w] * inv, over) |
                ((uint32_t)f2h_chk(acc[2 * w + 1] * inv, over) << 16);
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
  const int col = qh * 128 + 16 * sub;
  *reinterpret_cast<uint4*>(a.o + chunked(row, col, a.R)) =
      make_uint4(packed[0], packed[1], packed[2], packed[3]);
  *reinterpret_cast<uint4*>(a.o + chunked(row, col + 8, a.R)) =
      make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

// One block per sequence: its length into kv_len, and from its last row the head's
// input (half x * final gain, sum of squares) and the final-normed hidden state.
__global__ __launch_bounds__(256) void k_prefill_last(PrefillLastArgs a) {
  __shared__ float part[4];
  const int q = blockIdx.x, tid = threadIdx.x;
  const int lo = a.seq_start[q], hi = a.seq_start[q + 1];
  const int len = (hi > lo && hi <= a.R) ? hi - lo : 0;
  const float* x = a.x + (size_t)(len ? hi - 1 : 0) * a.H;
  float ss = 0.f;
  bool over = false;
  for (int i = tid; i < a.H; i += 256) {
    const float v = len ? x[i] : 0.f;
    a.u[chunked(q, i, a.max_seqs)] = f2h_chk(v * bf2f(a.gain[i]), over);
    ss = fmaf(v, v, ss);
  }
  if (over) atomicOr(a.status, QT_STATUS_FP16_RANGE);
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  if (tid == 0) {
    a.ss[q] = tot;
    a.kv_len[q] = len;
  }
  if (a.h_last) {
    const float inv = 1.0f / sqrtf(tot / (float)a.H + a.eps);
    for (int i = tid; i < a.H; i += 256)
      a.h_last[(size_t)q * a.H + i] = f2bf(len ? x[i] * inv * bf2f(a.gain[i]) : 0.f);
  }
}

// Greedy codebook-0 token of each sequence's last row from the head's keys.
__global__ __launch_bounds__(64) void k_prefill_end(PrefillEndArgs a) {
  const int q = blockIdx.x;
  const unsigned long long best = best_key_wave(a.cand + (size_t)q * a.cand_ld, a.n_cand);
  if (threadIdx.x == 0) a.tok0[q] = key_index(best);
}

}  // namespace

// --------------------------------------------------------------------------- launchers
template <bool SEP>
void launch_attn_paged_t(const AttnPagedArgs& a, dim3 grid, float tl, hipStream_t s) {
  switch (a.pages_per_split) {
    case 1: launch_kernel(k_attn_paged<1, SEP>, grid, dim3(256), s, a, tl); break;
    case 2: launch_kernel(k_attn_paged<2, SEP>, grid, dim3(256), s, a, tl); break;
    case 3: launch_kernel(k_attn_paged<3, SEP>, grid, dim3(256), s, a, tl); break;
    case 4: launch_kernel(k_attn_paged<4, SEP>, grid, dim3(256), s, a, tl); break;
    case 5: launch_kernel(k_attn_paged<5, SEP>, grid, dim3(256), s, a, tl); break;
    case 6: launch_kernel(k_attn_paged<6, SEP>, grid, dim3(256), s, a, tl); break;
    case 7: launch_kernel(k_attn_paged<7, SEP>, grid, dim3(256), s, a, tl); break;
    default: launch_kernel(k_attn_paged<8, SEP>, grid, dim3(256), s, a, tl); break;
  }
}

hipError_t launch_attn_paged(const AttnPagedArgs& a, int B, float theta, hipStream_t s) {
  if (a.pages_per_split < 1 || a.pages_per_split > kMaxPagesPerSplit || a.n_q != 2 * a.n_kv)
    return hipErrorInvalidValue;
  const dim3 grid(a.n_kv, B, a.n_splits);
  const float tl = (float)log2((double)theta);
  if (attn_merge_separate(B))
    launch_attn_paged_t<true>(a, grid, tl, s);
  else
    launch_attn_paged_t<false>(a, grid, tl, s);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnPagedArgs& a, int B, hipStream_t s) {
  if (a.pages_per_split < 1 || a.pages_per_split > kMaxPagesPerSplit || a.n_q != 2 * a.n_kv)
    return hipErrorInvalidValue;
  launch_kernel(k_attn_merge, dim3(a.n_kv, B), dim3(256), s, a);
  return hipGetLastError();
}

hipError_t launch_attn_pred(const AttnPredArgs& a, float theta, hipStream_t s) {
  if (a.n_new < 1 || a.n_new > 2 || a.pos0 < 0 || a.pos0 + a.n_new > 16 || a.n_q != 2 * a.n_kv)
    return hipErrorInvalidValue;
  launch_kernel(k_attn_pred, dim3(a.n_kv, a.B), dim3(256), s, a,
                     (float)log2((double)theta));
  return hipGetLastError();
}

hipError_t launch_frame_begin(const FrameBeginArgs& a, hipStream_t s) {
  launch_kernel(k_frame_begin, dim3(a.B), dim3(256), s, a);
  return hipGetLastError();
}

hipError_t launch_embed(const EmbedArgs& a, hipStream_t s) {
  launch_kernel(k_embed, dim3(a.B), dim3(256), s, a);
  return hipGetLastError();
}

hipError_t launch_frame_end(const FrameEndArgs& a, hipStream_t s) {
  launch_kernel(k_frame_end, dim3(a.B), dim3(256), s, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* w, long long rows, long long cols, int8_t* q,
                           uint16_t* q_half, long long q_row_stride, float* scale,
                           long long scale_stride, int tiled_K, long long row0, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || rows > 0x7fffffffLL) return hipErrorInvalidValue;
  if (tiled_K && (cols != tiled_K || tiled_K % 64 || row0 < 0)) return hipErrorInvalidValue;
  if (q_half && !tiled_K) return hipErrorInvalidValue;
  launch_kernel(k_quantize, dim3((unsigned)rows), dim3(256), s, w, cols, q, q_half, q_row_stride,
                     scale, scale_stride, tiled_K, row0);
  return hipGetLastError();
}

}  // namespace qt

namespace qt {
hipError_t launch_sched_setup(const SchedSetupArgs& a, hipStream_t s) {
  if (a.B < 1 || a.B > kSchedMaxBatch || (a.H % 8)) return hipErrorInvalidValue;
  launch_kernel(k_sched_setup, dim3(a.B), dim3(256), s, a);
  return hipGetLastError();
}
hipError_t launch_sched_collect(const SchedCollectArgs& a, hipStream_t s) {
  if (a.B < 1 || a.B > kSchedMaxBatch || (a.talker_vocab % 4) || (a.pred_elems % 4) ||
      a.eos_index < -1 || a.eos_index >= a.talker_vocab)
    return hipErrorInvalidValue;
  launch_kernel(k_sched_collect, dim3(a.B, kSchedCollectParts), dim3(256), s, a);
  return hipGetLastError();
}
}  // namespace qt

namespace qt {
hipError_t launch_prefill_begin(const PrefillBeginArgs& a, hipStream_t s) {
  if (a.R < 1 || a.max_seqs < 1) return hipErrorInvalidValue;
  launch_kernel(k_prefill_begin, dim3(a.R), dim3(256), s, a);
  return hipGetLastError();
}
hipError_t launch_prefill_qk(const PrefillQkArgs& a, int R, float theta, hipStream_t s) {
  if (R < 1 || a.n_q != 2 * a.n_kv) return hipErrorInvalidValue;
  if (a.R != R) return hipErrorInvalidValue;
  launch_kernel(k_prefill_qk, dim3((R + kQkRows - 1) / kQkRows, a.n_kv), dim3(256), s, a,
                (float)log2((double)theta));
  return hipGetLastError();
}
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s) {
  if (a.R < 16 || (a.R % 16) || a.n_q != 2 * a.n_kv) return hipErrorInvalidValue;
  if (a.n_splits < 1 || a.n_splits > 64) return hipErrorInvalidValue;
  launch_kernel(k_prefill_attn<kPfKeys>, dim3((a.R + kAttnRows - 1) / kAttnRows, a.n_kv, a.n_splits),
                dim3(512), s, a);
  launch_kernel(k_prefill_attn_merge, dim3(a.R / 16, a.n_kv), dim3(256), s, a);
  return hipGetLastError();
}
hipError_t launch_prefill_last(const PrefillLastArgs& a, hipStream_t s) {
  launch_kernel(k_prefill_last, dim3(a.max_seqs), dim3(256), s, a);
  return hipGetLastError();
}
hipError_t launch_prefill_end(const PrefillEndArgs& a, hipStream_t s) {
  launch_kernel(k_prefill_end, dim3(a.max_seqs), dim3(64), s, a);
  return hipGetLastError();
}
}  // namespace qt

namespace qt {
hipError_t launch_sample_rows(const SampleRowsArgs& a, hipStream_t s) {
  if (a.rows < 1 || a.V < 1 || a.V > 256 * kSampleSlots) return hipErrorInvalidValue;
  launch_kernel(k_sample_rows, dim3(a.rows), dim3(256), s, a);
  return hipGetLastError();
}
}  // namespace qt
