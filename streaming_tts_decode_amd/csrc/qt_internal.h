// Internal interface between the C ABI layer (qt_abi.cpp) and the gfx950
// kernels (qt_kernels.hip).  Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "qt.h"

namespace qt {

constexpr int kHeadDim = 128;   // head dimension the attention kernels are written for
constexpr int kPage = 16;       // Talker KV page size in positions
constexpr int kMaxPagesPerSplit = 8;

// Activations that feed a GEMM are carried as two bfloat16 arrays, hi = bf16(x)
// and lo = bf16(x - hi), so that hi + lo keeps ~16 significant bits of the fp32
// value; each weight operand is multiplied by both.  Weights stay bf16 / int8.
//
// GEMM epilogues.  y[m][n] = sum_k W[n][k] * act[m][k] (times scale[n] in INT8 mode).
enum Epi : int {
  EPI_STORE = 0,   // out_f32[m*out_ld + n] = y
  EPI_RESID = 1,   // out_f32[m*out_ld + n] += y
  EPI_SWIGLU = 2,  // rows interleaved (gate n, up n) at (2n, 2n+1):
                   // out_bf16[m*out_ld + n] = bf16(silu(gate) * up)
  EPI_HEAD = 3,    // n < n_logits: logits[m*logits_ld + n] = y, greedy key over n < argmax_range;
                   // n >= n_logits: out_f32[m*out_ld + n - n_logits] = y (projection rows)
};

struct GemmArgs {
  const void* W;          // bf16 [N][K] or int8 [N][K]
  const float* scale;     // [N] when INT8, else nullptr
  int N, K;               // full matrix
  int row0, nrows;        // rows [row0, row0+nrows) are computed
  const uint16_t* act;    // bf16 [M][act_ld]: high part of the activations
  const uint16_t* act_lo; // bf16 [M][act_ld]: low part, or nullptr
  int act_ld, M;
  // Consumer of an RMSNorm: the activations are x * gain (left by the producer of
  // x), so every output is multiplied by inv[m] = 1/sqrt(sum_s ss_in[s*ss_in_ld+m]/K
  // + eps), the producer's per-row-block sums of squares.  ss_in == nullptr: none.
  const float* ss_in;
  int ss_in_ld, ss_in_slots;
  float norm_eps;
  int epi;
  float* out_f32;
  int out_ld;
  uint16_t* out_bf16;     // EPI_SWIGLU: high part
  uint16_t* out_bf16_lo;  // EPI_SWIGLU: low part
  float* logits;
  int logits_ld, n_logits, argmax_range;
  unsigned long long* keys;  // greedy keys, one per m, stride keys_ld
  int keys_ld;
  uint32_t* status;
  // Producer of an RMSNorm input (EPI_RESID rows, EPI_HEAD projection rows): for
  // every written value v at output column c, u_hi/u_lo[m*u_ld + c] = hi/lo of
  // v * u_gain[c] (the next norm's gain), and per row block the sum of squares of
  // the block's values in ss_out[slot*ss_out_ld + m].  u_gain == nullptr: none.
  const uint16_t* u_gain;
  uint16_t* u_hi;
  uint16_t* u_lo;
  int u_ld;
  float* ss_out;
  int ss_out_ld;
};

// Timing events attached to the next kernel launch on this thread (tracing only):
// when set, the launch goes through hipExtLaunchKernelGGL, which stamps `start` and
// `stop` with the kernel's own begin and end.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;

template <typename Kernel, typename... Args>
inline void launch_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  if (g_launch_events.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, g_launch_events.start, g_launch_events.stop,
                          0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// Launch shape chosen for one GEMM (see plan_gemm).
struct GemmPlan {
  bool mfma;
  int mt, mp, rw, ni, rt, nw;
  int rows_per_block, row_blocks;
};

struct AttnPagedArgs {
  const float* qkv;       // [B][qkv_ld] raw q | k | v projections
  int qkv_ld, n_q, n_kv;
  const uint16_t* q_norm;
  const uint16_t* k_norm;
  float eps;
  uint16_t* k_pool;       // this layer's pages: [num_pages][n_kv][page][128] bf16
  uint16_t* v_pool;
  int num_pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* kv_len;  // [B]
  int pages_per_split, n_splits;
  float* part;            // [B][n_q][n_splits][128 + 2]
  unsigned* counters;     // [B][n_kv]
  uint16_t* o;            // [B][o_ld] bf16 high part of the attention output
  uint16_t* o_lo;         // low part
  int o_ld;
  uint32_t* status;
};

struct AttnPredArgs {
  const float* qkv;       // [n_new*B][qkv_ld]; row i*B + b holds new position pos0+i of session b
  int qkv_ld, n_q, n_kv, B;
  const uint16_t* q_norm;
  const uint16_t* k_norm;
  float eps;
  uint16_t* k_cache;      // this layer: [B][layer_stride] with positions [n_pos][n_kv][128]
  uint16_t* v_cache;
  long long sess_stride;  // elements between sessions
  int pos0, n_new;
  uint16_t* o;            // [n_new*B][o_ld] high part
  uint16_t* o_lo;         // low part
  int o_ld;
};

struct FrameBeginArgs {
  int mode, B, Ht, ncb, n_kv, capacity;
  float eps;
  const uint16_t* talker_in;
  const int32_t* tok0_in;
  const int32_t* kv_len;
  float* x_t;              // [B][Ht] f32
  float* ss_t;             // [B]: sum of squares of the talker input rows (one slot)
  const uint16_t* gain;    // [Ht]: gain of the first Talker norm
  uint16_t* u_hi;          // [B][Ht]: hi/lo of x * gain
  uint16_t* u_lo;
  unsigned long long* keys;  // [B][ncb]
  unsigned* counters;        // [B][n_kv] attention counters, zeroed
  uint32_t* status;
};

struct EmbedArgs {
  int B, H, vocab, ncb, step;   // step k >= 1 embeds the token of codebook k-1
  float eps;
  const uint16_t* table;        // [vocab][H]
  const unsigned long long* keys;
  const int32_t* forced;        // [B][ncb] or nullptr
  float* x;                     // [rows][H]
  float* ss;                    // sums of squares: slot 0 of the written rows, other slots zero
  int ss_ld, ss_slots;
  const uint16_t* gain;         // [H]: gain of the first predictor norm
  uint16_t* u_hi;               // [rows][H]: hi/lo of x * gain
  uint16_t* u_lo;
  int row_off;
  uint32_t* status;
};

struct FrameEndArgs {
  int mode, B, ncb, capacity;
  const unsigned long long* keys;
  int32_t* tokens;  // [B][ncb]
  int32_t* kv_len;
};

// launchers (enqueue only; shapes are validated by the caller)
GemmPlan plan_gemm(int nrows, int K, int M, bool i8);
// Kernel symbol (with template arguments) that launch_gemm picks for these arguments.
void gemm_kernel_name(const GemmArgs& a, char* buf, int len);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
hipError_t launch_attn_paged(const AttnPagedArgs& a, int B, float theta, hipStream_t s);
hipError_t launch_attn_pred(const AttnPredArgs& a, float theta, hipStream_t s);
hipError_t launch_frame_begin(const FrameBeginArgs& a, hipStream_t s);
hipError_t launch_embed(const EmbedArgs& a, hipStream_t s);
hipError_t launch_frame_end(const FrameEndArgs& a, hipStream_t s);
hipError_t launch_quantize(const uint16_t* w, long long rows, long long cols, int8_t* q,
                           long long q_row_stride, float* scale, long long scale_stride,
                           hipStream_t s);

}  // namespace qt
