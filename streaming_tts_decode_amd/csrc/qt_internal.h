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
// From this many sessions on, the Talker attention's split partials are merged by
// a launch of their own (k_attn_merge) instead of by the last split to arrive.
constexpr int kAttnMergeMinBatch = 16;
inline bool attn_merge_separate(int B) { return B >= kAttnMergeMinBatch; }

// Activations that feed a GEMM are IEEE half (11-bit significand: about eight
// times finer than bfloat16, which the 28-layer stack amplifies past the logit
// tolerance), and the GEMM weights are packed as half too so that both MFMA
// operands share the type: converting a bfloat16 weight to half is exact for
// |w| >= 2^-14 and within 2^-25 below.  INT8 weights become exact halves in
// registers.  Accumulation is fp32; residual streams are fp32.
//
// Layouts (all chosen so that every GEMM load and store moves whole 16-byte
// pieces of contiguous memory):
//  * packed weights, half: W[n][k] of an [N][K] matrix sits in 1 KB tiles
//    [N/16][K/32][64 lanes][8]; lane q*16+i of tile (n/16, k/32) holds
//    W[16*(n/16)+i][32*(k/32) + 8q .. +8], the A operand of one
//    16x16x32 MFMA.  tiled_bf16() gives the element offset (2-byte elements).
//  * packed weights, int8: 1 KB tiles [N/16][K/64][64][16 bytes]; lane q*16+i
//    holds W[16*(n/16)+i][64j + 8q .. +8] in bytes 0..7 and
//    W[..][64j + 32 + 8q .. +8] in bytes 8..15 (j = k/64).  tiled_i8().
//  * activations ("chunked"): element (m, k) of a [rows][K] activation is at
//    ((k/8)*ld + m)*8 + k%8, i.e. [K/8][ld][8]; ld is the buffer's row count.
//    Sixteen consecutive rows of one 8-column chunk are 256 contiguous bytes.
__host__ __device__ inline size_t tiled_bf16(int n, int k, int K) {
  return ((((size_t)(n >> 4) * (K >> 5) + (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (n & 15)) << 3) +
         (k & 7);
}
__host__ __device__ inline size_t tiled_i8(int n, int k, int K) {
  return ((((size_t)(n >> 4) * (K >> 6) + (k >> 6)) * 64 + ((k >> 3) & 3) * 16 + (n & 15)) << 4) +
         (((k >> 5) & 1) << 3) + (k & 7);
}
__host__ __device__ inline size_t chunked(int m, int k, int ld) {
  return (((size_t)(k >> 3) * ld + m) << 3) + (k & 7);
}

constexpr int kGemmRows = 16;   // weight rows per GEMM block (one MFMA A tile)
constexpr int kKeyBlock = 16;   // logits rows per greedy-key candidate

// GEMM epilogues.  y[m][n] = sum_k W[n][k] * act[m][k] (times scale[n] in INT8 mode).
enum Epi : int {
  EPI_STORE = 0,   // out_f32[m*out_ld + n] = y
  EPI_RESID = 1,   // out_f32[m*out_ld + n] += y
  EPI_SWIGLU = 2,  // rows interleaved (gate n, up n) at (2n, 2n+1):
                   // u (chunked, no gain) column n = silu(gate) * up
  EPI_HEAD = 3,    // n < n_logits: logits[m*logits_ld + n] = y, greedy-key candidates over
                   // n < argmax_range; n >= n_logits: out_f32[m*out_ld + n - n_logits] = y
                   // (projection rows)
};

struct GemmArgs {
  const void* W;          // packed tiles (see above) of a half or int8 [N][K] matrix
  const float* scale;     // [N] per-row scales of an INT8-quantised matrix, else nullptr
  int w8;                 // 1: W holds int8 tiles; 0: half tiles (in INT8 mode, the
                          // quantised values of a cache-resident matrix as exact halves)
  int keep_w;             // 1: the matrix is read again within the frame (predictor
                          // steps), so its loads go through the caches; 0: streamed
  int N, K;               // full matrix
  int row0, nrows;        // rows [row0, row0+nrows) are computed (multiples of 16)
  const uint16_t* act;    // chunked half [K/8][act_ld][8] activations
  int act_ld, M;          // rows 0..M-1 of the chunked array are used
  // Consumer of an RMSNorm: the activations are x * gain (left by the producer of
  // x), so every output is multiplied by inv[m] = 1/sqrt(sum_s ss_in[s*ss_in_ld+m]/K
  // + eps), the producer's per-row-block sums of squares.  ss_in == nullptr: none.
  const float* ss_in;
  int ss_in_ld, ss_in_slots;
  float norm_eps;
  int epi;
  float* out_f32;         // row-major f32 [M][out_ld]
  int out_ld;
  float* logits;
  int logits_ld, n_logits, argmax_range;
  // greedy-key candidates: cand[m*cand_ld + n/16] = best key of rows n..n+15
  unsigned long long* cand;
  int cand_ld;
  uint32_t* status;
  // Chunked half output: EPI_SWIGLU writes the SwiGLU activations here; a producer
  // of an RMSNorm input (EPI_RESID rows, EPI_HEAD projection rows) writes
  // v * u_gain[c] for every value v at output column c, and per 16-row block the
  // sum of squares of the block's values in ss_out[slot*ss_out_ld + m].
  const uint16_t* u_gain;
  uint16_t* u;
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

// Launch shape chosen for one GEMM (see plan_gemm): 16 weight rows (one tile, or
// three for large SwiGLU matrices) per block, nw
// waves splitting K; mt > 0: MFMA over mt 16-row activation tiles, mt == 0: VALU
// dot products (M <= 2); g = K steps per load group.  msplit > 1: the activation
// rows are split over msplit blocks per weight tile (more blocks for GEMMs with
// few weight rows); the blocks sharing a tile run on one XCD, so the tile is read
// from HBM once.
struct GemmPlan {
  int nw, mt, g, msplit;
  int rows_per_block;  // rows per sum-of-squares slot of a producing epilogue (16)
  int row_blocks;      // blocks along the weight rows
  int tiles;           // 16-row weight tiles per block (1, or 3 for large SwiGLU matrices)
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
  uint16_t* o;            // chunked half [q_dim/8][o_ld][8]: the attention output
  int o_ld;               // rows of the chunked output (>= B)
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
  uint16_t* o;            // chunked half [q_dim/8][o_ld][8]; row i*B + b: position pos0+i of session b
  int o_ld;               // rows of the chunked output (>= n_new*B)
  uint32_t* status;
};

struct FrameBeginArgs {
  int mode, B, Ht, ncb, n_kv, capacity;
  unsigned* pred_sync;      // sync counters of the persistent predictor, cleared (or nullptr)
  float eps;
  const uint16_t* talker_in;
  const int32_t* tok0_in;
  const int32_t* kv_len;
  const uint16_t* h_in;     // [B][Ht] bf16 post-norm hidden (predictor mode)
  float* x_t;              // [B][Ht] f32
  float* ss_t;             // [B]: sum of squares of the talker input rows (one slot)
  const uint16_t* gain;    // [Ht]: gain of the first Talker norm
  uint16_t* u;             // chunked half [Ht/8][B][8]: x * gain (predictor mode: h_in)
  unsigned long long* cand;  // [ncb][B][cand_ld] greedy-key candidates
  int cand_ld;
  unsigned* counters;        // [B][n_kv] attention counters, zeroed
  uint32_t* status;
};

// Drawing codec tokens instead of taking the argmax (qt_sampling in qt.h).
struct SamplerArgs {
  const qt_sampler_params* params;  // [B][2]; nullptr: greedy
  const uint64_t* seed;             // [B]
  const int32_t* counter;           // [B]
  uint32_t* seen0;                  // [B][seen_ld] or nullptr
  int seen_ld;
};

// The row a draw reads: session b's logits at logits + b * ld, entries [0, V).
struct SampleRow {
  const float* logits;
  long long ld;
  int V;
  int group;     // 0: codebook 0 (params [b][0], penalty, seen update); 1: predictor
  int codebook;  // Philox counter word 1 and the tokens column written
};

struct EmbedArgs {
  int B, H, vocab, ncb, step;   // step k >= 1 embeds the token of codebook k-1
  float eps;
  const uint16_t* table;        // [vocab][H]
  const unsigned long long* cand;  // candidates of codebook step-1: [B][cand_ld], n_cand used
  int cand_ld, n_cand;
  const int32_t* forced;        // [B][ncb] or nullptr
  float* x;                     // [rows][H]
  float* ss;                    // sums of squares: slot 0 of the written rows, other slots zero
  int ss_ld, ss_slots;
  const uint16_t* gain;         // [H]: gain of the first predictor norm
  uint16_t* u;                  // chunked half [H/8][u_ld][8]: x * gain
  int u_ld;
  int row_off;
  uint32_t* status;
  int sample;                   // 1: draw codebook step-1 from `row` instead of the argmax keys
  SamplerArgs smp;
  SampleRow row;
  int32_t* tokens;              // [B][ncb]: the drawn token is written to column step-1
};

struct FrameEndArgs {
  int mode, B, ncb, capacity;
  const unsigned long long* cand;  // [ncb][B][cand_ld]
  int cand_ld, n_cand0, n_cand;    // candidates of codebook 0 / of the others
  int32_t* tokens;  // [B][ncb]
  int32_t* kv_len;
  int sample;       // 1: the frame draws tokens; this kernel draws `row` (the last draw)
  SamplerArgs smp;
  SampleRow row;
  uint32_t* status;
};

// Prompt prefill (qt_prefill): rows of packed sequences; rowinfo[2r] = sequence
// of row r (-1: padding), rowinfo[2r+1] = its position.
struct PrefillBeginArgs {
  int R, H, max_seqs;
  const int32_t* seq_start;
  const uint16_t* embeds;   // [R][H] bf16
  const uint16_t* gain;     // first input norm
  float* x;                 // [R][H]
  uint16_t* u;              // chunked half [H/8][R][8]
  float* ss;                // slot 0: [R]
  int32_t* rowinfo;         // [R][2]
  uint32_t* status;
};

struct PrefillQkArgs {
  float* qkv;               // [R][qkv_ld]: q is replaced by its normalised, rotated, scaled form
  int R;                    // rows
  int qkv_ld, n_q, n_kv;
  const uint16_t* q_norm;
  const uint16_t* k_norm;
  float eps;
  uint16_t* k_pool;         // this layer's pages
  uint16_t* v_pool;
  int num_pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* rowinfo;
  uint32_t* status;
};

struct PrefillAttnArgs {
  const float* qkv;
  int qkv_ld, n_q, n_kv, R;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int num_pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* rowinfo;
  uint16_t* o;              // chunked half [q_dim/8][R][8]
  float* part;              // [R][n_q][n_splits][128 + 2]: split outputs, max and sum
  int n_splits;             // key blocks of a tile are dealt round-robin over the splits
  uint32_t* status;
};

struct PrefillLastArgs {
  int max_seqs, H, R;
  const int32_t* seq_start;
  const float* x;
  const uint16_t* gain;     // final norm
  float eps;
  uint16_t* u;              // chunked half [H/8][max_seqs][8]
  float* ss;                // [max_seqs]
  uint16_t* h_last;         // [max_seqs][H] bf16 or nullptr
  int32_t* kv_len;
  uint32_t* status;
};

struct PrefillEndArgs {
  int max_seqs, cand_ld, n_cand;
  const unsigned long long* cand;
  int32_t* tok0;
};

// qt_sample: one block per row.
struct SampleRowsArgs {
  int rows, V, codebook, seen_ld;
  long long ld;
  const float* logits;
  const qt_sampler_params* params;  // [rows]
  const uint64_t* seed;
  const int32_t* counter;
  uint32_t* seen;                   // [rows][seen_ld] or nullptr
  int32_t* tokens;
  uint32_t* status;
};
hipError_t launch_sample_rows(const SampleRowsArgs& a, hipStream_t s);

hipError_t launch_prefill_begin(const PrefillBeginArgs& a, hipStream_t s);
hipError_t launch_prefill_qk(const PrefillQkArgs& a, int R, float theta, hipStream_t s);
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s);
hipError_t launch_prefill_last(const PrefillLastArgs& a, hipStream_t s);
hipError_t launch_prefill_end(const PrefillEndArgs& a, hipStream_t s);

// Scheduler helpers (qt_sched.cpp): per-group batch tables in, per-session results out.
constexpr int kSchedMaxBatch = 32;

struct SchedSetupArgs {
  int B, H, ncb, max_pages, pad_page;
  const int32_t* host_pages;     // pinned host [max_sessions][max_pages]: rows at open
  int32_t* sess_pages;           // device [max_sessions][max_pages]
  int32_t* kv_len;               // batch [B]
  int32_t* page_table;           // batch [B][max_pages]
  uint16_t* talker_in;           // batch [B][H]
  int32_t* forced;               // batch [B][ncb] (nullptr: the group is not teacher-forced)
  int32_t* flags;                // device [max_sessions]: frame that ended the session, or 0
  int32_t slot_session[kSchedMaxBatch];  // -1: padding slot
  int32_t slot_len[kSchedMaxBatch];      // cached positions before this frame
  int32_t slot_first[kSchedMaxBatch];    // pages held at open if this is the first frame, else -1
  int32_t new_index[kSchedMaxBatch];     // page appended this frame at this row index, or -1
  int32_t new_page[kSchedMaxBatch];
  const uint16_t* in_ptr[kSchedMaxBatch];
  const int32_t* forced_ptr[kSchedMaxBatch];
  // sampling groups: per-slot parameters and seed into the batch tables, and the
  // session's seen set (cleared on its first frame) into the batch seen table
  qt_sampler_params* params;     // batch [B][2], or nullptr
  uint64_t* seed;                // batch [B]
  uint32_t* seen;                // batch [B][seen_ld]
  uint32_t* sess_seen;           // [max_sessions][seen_ld]
  int seen_ld;
  qt_sampler_params slot_params[kSchedMaxBatch][2];
  uint64_t slot_seed[kSchedMaxBatch];
};

struct SchedCollectArgs {
  int B, talker_vocab, cb0_range, pred_elems, ncb, eos_index;
  const float* logits0;          // batch outputs
  const float* logits_pred;
  const int32_t* tokens;
  float* res_logits0;            // per session
  float* res_pred;
  int32_t* res_tokens;
  int32_t* flags;                // device [max_sessions]
  int32_t* host_flags;           // pinned host [max_sessions]
  int32_t slot_session[kSchedMaxBatch];
  int32_t slot_check[kSchedMaxBatch];    // frame number to record at end of speech, or 0
  // sampling groups: tokens[b][0] is a draw, so the end-of-speech test takes the
  // greedy choice from logits0 itself; the batch seen rows go back to the sessions
  int sampled;
  const uint32_t* seen;          // batch [B][seen_ld]
  uint32_t* sess_seen;           // [max_sessions][seen_ld]
  int seen_ld;
};

hipError_t launch_sched_setup(const SchedSetupArgs& a, hipStream_t s);
hipError_t launch_sched_collect(const SchedCollectArgs& a, hipStream_t s);

// Persistent code predictor (qt_pred.hip): every predictor step of a frame in one
// launch of 256 blocks, one per CU, 32 on each of the eight XCDs (a block reads its
// XCD from the hardware; the launch stops with QT_STATUS_SYNC if the blocks are not
// all resident or not 32 per XCD).  XCD x owns KV
// head x (its QKV rows and attention), the K-slice [256x, 256x + 256) of the output
// projection, FFN columns [384x, 384x + 384) (its gate/up rows and the matching
// K-slice of down) and head rows [256x, 256x + 256).  Shapes: predictor hidden 1024,
// 16 query / 8 KV heads of 128, FFN 3072, code vocabulary 2048, B <= 32.
constexpr int kPredMaxLayers = 8;
constexpr int kPredMaxSteps = 15;
constexpr int kPredBlocks = 256;
constexpr unsigned kPredSyncWords = 64 * 40;  // sync counters, one 256-byte line each

struct PredPersistArgs {
  int B, layers, n_steps, ncb, ldm;  // ldm: rows of the per-XCD buffers (>= 2B)
  float eps, theta_log2;
  const void* w_qkv[kPredMaxLayers];
  const void* w_o[kPredMaxLayers];
  const void* w_gu[kPredMaxLayers];
  const void* w_dn[kPredMaxLayers];
  const float* s_qkv[kPredMaxLayers];  // INT8 row scales (nullptr in bf16 mode)
  const float* s_o[kPredMaxLayers];
  const float* s_gu[kPredMaxLayers];
  const float* s_dn[kPredMaxLayers];
  const uint16_t* g_in[kPredMaxLayers];
  const uint16_t* g_q[kPredMaxLayers];
  const uint16_t* g_k[kPredMaxLayers];
  const uint16_t* g_post[kPredMaxLayers];
  const uint16_t* g_final;
  const void* w_head[kPredMaxSteps];
  const float* s_head[kPredMaxSteps];
  const uint16_t* embed[kPredMaxSteps];  // [2048][1024] bf16
  const float* x_p;               // [B][1024]: projection rows left by the Talker's head GEMM
  unsigned long long* cand;       // [ncb][B][cand_ld] greedy keys (codebook 0 from the head GEMM)
  int cand_ld;
  const int32_t* forced;          // [B][ncb] or nullptr
  float* logits;                  // [B][ncb-1][2048]
  uint32_t* status;
  uint16_t* kc;                   // predictor cache [B][layers][ncb][8][128] bf16
  uint16_t* vc;
  long long sess_stride;          // elements per session of the cache
  // workspace: per-XCD buffers and the cross-XCD partial sums
  float* x_loc;                   // [8][ldm][1024] residual rows
  uint16_t* u_loc;                // [8][128][ldm][8] half: next GEMM's normalised input
  float* ss_loc;                  // [8][32][ldm] sums of squares per 32-column slice
  float* qkv_loc;                 // [8][ldm][512]: q heads 2x, 2x+1, key x, value x
  uint16_t* o_loc;                // [8][32][ldm][8] half: attention output of heads 2x, 2x+1
  uint16_t* f_loc;                // [8][48][ldm][8] half: SwiGLU output, FFN slice x
  float* p_o;                     // [8][ldm][1024] output-projection partial of XCD x
  float* p_d;                     // [8][ldm][1024] down-projection partial of XCD x
  unsigned* sync;                 // kPredSyncWords, zero at launch (k_frame_begin clears it)
};
hipError_t launch_pred_persist(const PredPersistArgs& a, hipStream_t s);
// Per process and device, before the first launch (not under stream capture): the
// kernel's 96 KB of dynamic LDS (which also keeps it to one block per CU), and a
// check that the occupancy of that shape lets all kPredBlocks blocks be resident
// on `cus` CUs at once (hipErrorInvalidConfiguration if not).
hipError_t prepare_pred_persist(int cus);

// Configuration of a loaded model, and the thread-local error text behind
// qt_last_error() (qt_abi.cpp).
const qt_model_cfg* model_cfg(const qt_model* m);
qt_status report(qt_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// launchers (enqueue only; shapes are validated by the caller)
GemmPlan plan_gemm(int nrows, int K, int M, bool i8, bool keep, bool swiglu = false);
// Kernel symbol (with template arguments) that launch_gemm picks for these arguments.
void gemm_kernel_name(const GemmArgs& a, char* buf, int len);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// Many activation rows (M a multiple of 16; nrows a multiple of 128): EPI_STORE,
// EPI_RESID and EPI_SWIGLU, one 16-row statistics slot per 16 weight rows.
// qk: the prompt's q/k pass that follows a QKV projection; when the projection's
// tiles are whole heads the pass is done in its epilogue and *qk_done is set, else
// the caller launches it.
hipError_t launch_gemm_rows(const GemmArgs& a, hipStream_t s, const PrefillQkArgs* qk = nullptr,
                            float theta = 0.f, bool* qk_done = nullptr);
hipError_t launch_attn_paged(const AttnPagedArgs& a, int B, float theta, hipStream_t s);
// after launch_attn_paged when attn_merge_separate(B)
hipError_t launch_attn_merge(const AttnPagedArgs& a, int B, hipStream_t s);
hipError_t launch_attn_pred(const AttnPredArgs& a, float theta, hipStream_t s);
hipError_t launch_frame_begin(const FrameBeginArgs& a, hipStream_t s);
hipError_t launch_embed(const EmbedArgs& a, hipStream_t s);
hipError_t launch_frame_end(const FrameEndArgs& a, hipStream_t s);
// Pack bf16 source rows [rows][K] as half rows row0 + i*step of a tiled [N][K] matrix;
// a finite weight beyond the half range sets *range_flag (device word).
hipError_t launch_pack_tiled(const uint16_t* src, int rows, int K, uint16_t* dst, int row0, int step,
                             uint32_t* range_flag, hipStream_t s);
// Copy rows row0 + i*step (i < rows) of a tiled INT8-quantised [N][K] matrix out
// row-major as int8: from int8 tiles, or (half_src) from half tiles holding the values.
hipError_t launch_untile_i8(const void* tiled, bool half_src, int rows, int K, int row0, int step,
                            int8_t* out, hipStream_t s);
// INT8 quantizer.  tiled_K == 0: q row r at q + r*q_row_stride; tiled_K > 0: source row r
// becomes row row0 + r*q_row_stride of a tiled [N][tiled_K] matrix: int8 tiles at q, or,
// when q_half is given, half tiles at q_half holding the same integer values.
hipError_t launch_quantize(const uint16_t* w, long long rows, long long cols, int8_t* q,
                           uint16_t* q_half, long long q_row_stride, float* scale,
                           long long scale_stride, int tiled_K, long long row0, hipStream_t s);

}  // namespace qt
