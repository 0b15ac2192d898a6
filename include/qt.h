/*
 * qt.h -- C ABI of the MI355X (gfx950) lockstep decode-frame library (libqt.so).
 *
 * One call decodes one codec frame for every active session of a
 * Qwen3-TTS-style speech model: a Talker decoder step that emits codebook 0,
 * the Talker-to-predictor projection, then the code-predictor steps that emit
 * codebooks 1 .. n_codebooks-1.  Every shared weight matrix is streamed once
 * per use for the whole batch, and all per-session state (KV pages, lengths,
 * tokens) stays in caller-owned buffers.
 *
 * Sources for the operations (the pages define what is computed, not these
 * signatures):
 *  - "Qwen3-TTS Native v0.3.0" release notes, What changed: one batched call per
 *    frame runs the talker and the 15-step code predictor for every active
 *    session, each shared weight read once per frame, per-session KV and state
 *    kept request-local; the whole frame captured once per session tuple and
 *    replayed as a graph; opt-in INT8 weight-only decode, per-output-channel
 *    symmetric, quantized at engine load from the BF16 weights.
 *  - qwen.lukaloehr.com llms.txt: the token is handed from talker to predictor
 *    device to device.
 *  - M* "Qwen3-TTS PR 5": Graph section (paged KV, RoPE positions as Talker
 *    resources); What changed (Talker 2048 -> predictor 1024 projection; weight
 *    loading checks coverage in both directions); Parity section (teacher-forced
 *    logits).
 *  - decomputer.nl article on Qwen3-TTS serving, sections 3 and 5: the code
 *    predictor always runs 15 steps per frame on a preallocated KV cache; no
 *    needless CPU-GPU synchronisation.
 *
 * Conventions
 *  - Every pointer documented "device" is a HIP device pointer on the current
 *    device; "host" pointers are ordinary host memory.  The library never
 *    allocates device memory: the caller passes every buffer (packed weights,
 *    workspace, KV pages, inputs, outputs).
 *  - bf16 tensors are raw bfloat16 bit patterns (uint16), row-major.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls that take a
 *    stream only enqueue work on it and never synchronise the host.
 *  - Errors: every function returns a qt_status; host-detectable problems are
 *    reported before anything is enqueued.  qt_last_error() gives a
 *    thread-local description of the most recent failure.  Conditions only the
 *    device can see (a session whose cache is full, a page id out of range, a
 *    token out of range, a NaN logit) OR a bit into the caller's `status` word
 *    and skip that session's writes; the host reads the word whenever it likes.
 *  - Handles (qt_model, qt_graph) are opaque host objects owned by the caller
 *    and released with the matching destroy call.  A qt_model refers to the
 *    caller's packed-weight buffer, which must outlive it.
 */
#ifndef QT_H
#define QT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QT_ABI_VERSION 3

typedef enum {
  QT_OK = 0,
  QT_E_INVALID_ARG = 1,       /* null pointer, non-positive size, bad enum value */
  QT_E_SHAPE = 2,             /* a dimension the kernels do not support, or a tensor shape mismatch */
  QT_E_DTYPE = 3,             /* a tensor of the wrong element type */
  QT_E_MISSING_TENSOR = 4,    /* qt_load_weights: an expected weight is absent */
  QT_E_UNEXPECTED_TENSOR = 5, /* qt_load_weights: an unknown or duplicated weight name */
  QT_E_CAPACITY = 6,          /* a buffer smaller than required, or a batch above the workspace's */
  QT_E_STATE = 7,             /* the handle is not usable for this call */
  QT_E_HIP = 8,               /* a HIP runtime call failed; see qt_last_error() */
  QT_E_UNSUPPORTED = 9        /* a valid request the library does not implement */
} qt_status;

typedef enum { QT_BF16 = 0, QT_F32 = 1, QT_I8 = 2, QT_I32 = 3 } qt_dtype;

typedef enum {
  QT_MODE_FULL = 0,      /* Talker step + projection + all predictor steps */
  QT_MODE_TALKER = 1,    /* Talker step and codebook 0 only */
  QT_MODE_PREDICTOR = 2  /* projection + predictor steps from a given hidden state and token */
} qt_mode;

/* Bits OR-ed into qt_frame_outputs.status by the device. */
#define QT_STATUS_KV_OVERFLOW 1u /* kv_len[b] + 1 > max_pages * page_size: session b skipped */
#define QT_STATUS_BAD_PAGE 2u    /* a page id outside [0, num_pages): that page is read as zeros */
#define QT_STATUS_BAD_TOKEN 4u   /* a forced / input token outside the code vocabulary: 0 used */
#define QT_STATUS_NAN 8u         /* a NaN logit was produced */
#define QT_STATUS_BAD_SAMPLER 16u /* sampler parameters out of range: that draw was greedy */
#define QT_STATUS_FP16_RANGE 32u  /* a GEMM input held a finite value beyond the IEEE half range
                                     (|v| >= 65520): it became +-inf.  GEMM inputs are half(x * gain)
                                     of the residual rows (before the RMS factor), the SwiGLU
                                     output and the attention output */
#define QT_STATUS_SYNC 64u        /* the one-launch code predictor could not synchronise its blocks
                                     (they were not all resident, or not on the expected XCDs):
                                     that frame's predictor outputs are not valid */

/* One decoder stack (Qwen3-style: pre-norm, q/k RMSNorm, rotate-half RoPE,
 * grouped-query attention, SwiGLU).  The library supports head_dim = 128,
 * n_q_heads = 2 * n_kv_heads, hidden, n_q_heads*head_dim and ffn multiples
 * of 512. */
typedef struct {
  int32_t layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn;
  float rope_theta, rms_eps;
} qt_decoder_cfg;

typedef struct {
  qt_decoder_cfg talker, predictor;
  int32_t talker_vocab; /* rows of the Talker codec head (3072) */
  int32_t code_vocab;   /* rows of each predictor embedding and head (2048) */
  int32_t cb0_range;    /* codebook-0 argmax runs over [0, cb0_range) (2048) */
  int32_t n_codebooks;  /* 1 Talker codebook + (n_codebooks - 1) predictor steps, 2..16 */
  int32_t page_size;    /* Talker KV page size in positions; the library supports 16 */
} qt_model_cfg;

/* A named source tensor for qt_load_weights: device pointer, bf16, [rows, cols];
 * vectors (norm gains) are rows = 1, cols = n. */
typedef struct {
  const char* name;
  const void* data;
  int32_t dtype;
  int64_t rows, cols;
} qt_tensor;

typedef struct qt_model qt_model;
typedef struct qt_graph qt_graph;

typedef struct {
  int32_t batch;             /* B >= 1 active sessions */
  int32_t* kv_len;           /* device int32 [B]: Talker positions already cached per session;
                                the frame appends at position kv_len[b] and then adds 1
                                (FULL and TALKER modes) */
  const int32_t* page_table; /* device int32 [B][max_pages]: page id of positions
                                [i*page_size, (i+1)*page_size) of session b */
  int32_t max_pages;         /* row length of page_table; capacity = max_pages * page_size */
} qt_sessions;

typedef struct {
  void* k_pages;     /* device bf16 [talker layers][num_pages][n_kv][page_size][head_dim] */
  void* v_pages;     /* same layout; cached keys are stored after q/k-norm and RoPE */
  int32_t num_pages;
} qt_kv_caches;

/* ------------------------------------------------------------------ sampling
 * Codec tokens drawn instead of taken greedily ("Qwen3-TTS PR 5", Graph: two
 * samplers, the codebook-0 one with a repetition penalty; "Qwen3-TTS Native v0.3.0",
 * What changed: sampling state, seen-token histories and random states stay per
 * request, and seeded runs repeat exactly).  For one row of logits x over the
 * draw range (codebook 0: [0, cb0_range) of logits0; predictor step k: its
 * code_vocab logits), in float32:
 *   1. codebook 0 only: an entry already in the session's seen set becomes
 *      x / penalty if x > 0, else x * penalty;
 *   2. z = x / temperature (a NaN z is never drawn);
 *   3. the top_k largest z, ties to the lower index, ordered by (z descending,
 *      index ascending), with weights w_j = exp(z_j - z_0);
 *   4. the shortest prefix whose weight sum reaches top_p times the top_k total
 *      is kept (at least one entry);
 *   5. with r = u * (kept total), the token is the first kept entry whose running
 *      weight sum exceeds r.
 * u is the top 24 bits of word 0 of Philox4x64-10 (Salmon et al., SC 2011) with
 * key (seed[b], 0) and counter ((uint32) counter[b], codebook, 0, 0), times 2^-24.
 * Drawn tokens are what `tokens` reports; with `forced`, the predictor still
 * embeds the forced tokens.  Codebook 0's drawn token is added to the seen set. */
#define QT_SAMPLER_MAX_TOP_K 64

typedef struct {
  float temperature;        /* > 0 */
  float top_p;              /* (0, 1] */
  float repetition_penalty; /* >= 1, codebook 0 only (1: none) */
  int32_t top_k;            /* 1 .. QT_SAMPLER_MAX_TOP_K */
} qt_sampler_params;

typedef struct {
  const qt_sampler_params* params; /* device [B][2]: [b][0] codebook 0, [b][1] the predictor's codebooks */
  const uint64_t* seed;            /* device [B]: per-session Philox key */
  const int32_t* counter;          /* device [B]: per-session draw counter, e.g. kv_len (read before
                                      the frame advances kv_len) */
  uint32_t* seen0;                 /* device [B][(cb0_range + 31) / 32] bit sets of codebook-0 tokens
                                      already emitted, or NULL (no penalty, no update) */
} qt_sampling;

/* Draw one token per row of caller-given logits with the frame's sampler (the
 * same steps 1-5 and Philox draw as above), e.g. for logits computed elsewhere.
 * logits: device f32 [rows][ld], entries [0, V) drawn over, V <= 4096;
 * params: device [rows]; seed, counter: device [rows]; codebook: the Philox
 * counter's second word; seen: device [rows][(V + 31) / 32] bit sets or NULL (the
 * penalty applies to their entries, and each row's draw is added); tokens: device
 * int32 [rows]; status: device uint32 [1] (QT_STATUS_BAD_SAMPLER for a row whose
 * parameters are out of range: that row is drawn greedily).  Enqueued on `stream`. */
qt_status qt_sample(const float* logits, int32_t rows, int32_t ld, int32_t V,
                    const qt_sampler_params* params, const uint64_t* seed, const int32_t* counter,
                    int32_t codebook, uint32_t* seen, int32_t* tokens, uint32_t* status,
                    void* stream);

typedef struct {
  int32_t mode;            /* qt_mode */
  const void* talker_in;   /* device bf16 [B][talker hidden]: the Talker input (FULL, TALKER) */
  const void* h_in;        /* device bf16 [B][talker hidden]: the post-norm Talker hidden (PREDICTOR) */
  const int32_t* tok0_in;  /* device int32 [B]: codebook-0 tokens (PREDICTOR) */
  const int32_t* forced;   /* device int32 [B][n_codebooks] or NULL: teacher forcing; predictor
                              step k embeds forced[b][k-1] instead of the frame's own token */
  const qt_sampling* sampling; /* host descriptor or NULL (greedy); its arrays are device memory */
} qt_frame_inputs;

typedef struct {
  float* logits0;      /* device f32 [B][talker_vocab] (FULL, TALKER) */
  float* logits_pred;  /* device f32 [B][n_codebooks-1][code_vocab] (FULL, PREDICTOR) */
  int32_t* tokens;     /* device int32 [B][n_codebooks]: the frame's tokens, greedy (lowest index
                          wins ties) or drawn (qt_sampling); TALKER fills column 0, PREDICTOR
                          copies tok0_in into it */
  uint32_t* status;    /* device uint32 [1]: QT_STATUS_* bits are OR-ed in; the caller clears it */
} qt_frame_outputs;

/* Text of the last failure on this thread ("" if none). */
const char* qt_last_error(void);
int32_t qt_abi_version(void);

/* Check that the configuration is one the kernels support.  QT_E_SHAPE otherwise.
 * (This and the two sizing calls below are the library's own memory plan; the pages
 * describe the engine, not its buffers.) */
qt_status qt_validate_cfg(const qt_model_cfg* cfg);

/* Bytes of the packed-weight buffer for this configuration (int8_mode 0: bf16, 1: INT8). */
qt_status qt_packed_bytes(const qt_model_cfg* cfg, int32_t int8_mode, uint64_t* bytes);

/* Bytes of the per-call workspace for up to max_batch sessions and page tables of
 * max_pages entries. */
qt_status qt_workspace_bytes(const qt_model_cfg* cfg, int32_t max_batch, int32_t max_pages,
                             uint64_t* bytes);

/* Load the weights ("Qwen3-TTS PR 5", What changed: weight loading checks coverage
 * in both directions; "Qwen3-TTS Native v0.3.0", What changed: INT8 weight-only decode
 * is chosen when the engine loads and is quantized from the BF16 weights).
 * Validate and pack the model weights into the caller's device buffer `packed`
 * (at least qt_packed_bytes bytes, 256-byte aligned).  `tensors` (host array of
 * n_tensors entries) must name every expected weight exactly once with the
 * expected shape and dtype bf16, and nothing else (checked in both directions:
 * QT_E_MISSING_TENSOR / QT_E_UNEXPECTED_TENSOR / QT_E_SHAPE / QT_E_DTYPE).
 * Names: talker.layers.{l}.{input_norm,q_proj,k_proj,v_proj,q_norm,k_norm,o_proj,
 * post_norm,gate_proj,up_proj,down_proj}, talker.final_norm, talker.codec_head,
 * projection, predictor.layers.{l}.{...same...}, predictor.final_norm,
 * predictor.codec_embed.{i}, predictor.lm_head.{i} for i < n_codebooks-1.
 * int8_mode 1 quantizes every decode GEMM weight (attention, FFN, projection, codec
 * head and predictor heads) with qt_quantize_int8's arithmetic; embeddings and norm
 * gains stay bf16.  The Talker's quantized matrices (and the codec head with the
 * projection) are stored as int8, the code predictor's as the same integers in half
 * (exact: |q| <= 127), since its matrices stay cached across its steps and its
 * launches are bound by latency rather than bytes; the products are the same.  The
 * prompt prefill stays BF16 (same passage): in INT8 mode the Talker's matrices keep
 * an unquantised half copy that only qt_prefill reads.
 * Packing is enqueued on `stream`; the source tensors may be
 * freed once it has completed.  *out receives a handle for qt_frame_decode.
 * Range: in bf16 mode the GEMM weights are packed as IEEE half (exact for
 * |w| >= 2^-14, within 2^-25 below), so a weight matrix holding a finite entry with
 * |w| > 65504 is refused with QT_E_UNSUPPORTED naming it; to find out, the call waits
 * for the packing to finish on `stream`.  INT8 mode takes any finite weights for
 * decoding; a Talker weight beyond the half range then makes qt_prefill and
 * qt_prefill_graph_create return QT_E_UNSUPPORTED naming it.  At decode time the
 * GEMM inputs are half too: a residual row value x with
 * |x * gain| >= 65520 sets QT_STATUS_FP16_RANGE (see the status bits). */
qt_status qt_load_weights(const qt_model_cfg* cfg, const qt_tensor* tensors, int32_t n_tensors,
                          int32_t int8_mode, void* packed, uint64_t packed_bytes, void* stream,
                          qt_model** out);

/* Per-output-channel symmetric INT8 ("Qwen3-TTS Native v0.3.0", What changed):
 * for each row r of the device bf16 [rows, cols] matrix w,
 *   scale[r] = f32(max_k |w[r][k]|) / 127   (IEEE float32 divide),
 *   q[r][k]  = clamp(round_half_even(f32(w[r][k]) / scale[r]), -127, 127)
 * with an all-zero row giving scale 0 and q 0.  q (device int8 [rows, cols]) and
 * scale (device f32 [rows]) are written on `stream`. */
qt_status qt_quantize_int8(const void* w_bf16, int64_t rows, int64_t cols, int8_t* q,
                           float* scale, void* stream);

/* Copy the packed INT8 form of the named decode weight back out in its source row
 * order: q (device int8 [rows, cols]) and scale (device f32 [rows]).  For checking
 * that the weights a model decodes with are the quantizer's output.  QT_E_STATE if
 * the model was loaded in bf16 mode. */
qt_status qt_model_export_int8(const qt_model* model, const char* name, int8_t* q, float* scale,
                               void* stream);

/* One lockstep frame ("Qwen3-TTS Native v0.3.0", What changed: one batched call runs
 * the Talker step and the 15-step code predictor for every active session, every
 * shared weight read once per frame, per-session state kept request-local;
 * decomputer.nl article, parts 3 and 5: the predictor always runs its fixed steps on
 * a preallocated cache, and the decode loop avoids CPU-GPU synchronisation;
 * qwen.lukaloehr.com llms.txt: the codebook-0 token goes from Talker to predictor on
 * the device).  The predictor runs as a chain of launches; with QT_PREDICTOR=persistent
 * in the environment when the model is loaded, greedy and teacher-forced frames of a
 * model whose predictor has the full-size shapes (hidden 1024, 16 / 8 heads, FFN 3072,
 * vocabulary 2048) run every predictor step in one launch on a 256-CU device
 * (QT_KERNEL_PREDICTOR).  Both compute the same definition.
 * Decode one frame for all sessions (see qt_mode).  Enqueues every kernel of the frame
 * on `stream` and returns without synchronising.  `workspace` is a device buffer of at
 * least qt_workspace_bytes(cfg, B, max_pages) bytes; the caller must not touch it while
 * a frame that uses it is in flight, and concurrent frames need separate workspaces.
 * Outputs are overwritten; kv_len is advanced on the device. */
qt_status qt_frame_decode(qt_model* model, const qt_sessions* sessions, const qt_kv_caches* kv,
                          const qt_frame_inputs* in, const qt_frame_outputs* out, void* workspace,
                          uint64_t workspace_bytes, void* stream);

/* The same frame as qt_frame_decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the per-frame scratch is a static array of QT_NOALLOC_SCRATCH_BYTES
 * bytes inside the library, one per GPU, held until the process ends, instead of a
 * caller workspace.  Nothing is allocated or freed by this call.  A batch whose
 * workspace (qt_workspace_bytes(cfg, batch, max_pages)) exceeds that size is refused
 * with QT_E_CAPACITY before anything is enqueued: 32 sessions with page tables of up
 * to 256 pages (4096 positions) fit.  Every call on one GPU shares that GPU's array:
 * calls whose frames overlap on the device (other streams, or other threads) race
 * and give wrong results; calls enqueued in order on one stream do not.  The frame
 * clears what it needs cleared itself, so nothing from an earlier call leaks in.
 * Arguments, outputs and errors are otherwise those of qt_frame_decode. */
#define QT_NOALLOC_SCRATCH_BYTES (48u << 20)
qt_status qt_frame_decode_noalloc(qt_model* model, const qt_sessions* sessions,
                                  const qt_kv_caches* kv, const qt_frame_inputs* in,
                                  const qt_frame_outputs* out, void* stream);

/* Frames as graphs ("Qwen3-TTS Native v0.3.0", What changed: the frame is captured
 * once per session tuple and replayed; decomputer.nl article, part 5: graphs for a
 * fixed set of batch sizes).
 * Capture the same frame as qt_frame_decode into a HIP graph and instantiate it.  The
 * graph bakes in every pointer and the batch size: the caller keeps all buffers alive
 * and at the same addresses until qt_graph_destroy, and changes per-frame data only by
 * rewriting buffer contents (inputs, forced tokens, kv_len). */
qt_status qt_frame_graph_create(qt_model* model, const qt_sessions* sessions,
                                const qt_kv_caches* kv, const qt_frame_inputs* in,
                                const qt_frame_outputs* out, void* workspace,
                                uint64_t workspace_bytes, qt_graph** out_graph);

/* Replay a captured frame or prefill on `stream` (enqueue only). */
qt_status qt_frame_graph_launch(qt_graph* graph, void* stream);

void qt_graph_destroy(qt_graph* graph);
void qt_model_destroy(qt_model* model);

/* ------------------------------------------------------------------ prefill
 * The Talker over prompt positions, before the decode loop ("Qwen3-TTS PR 5", What
 * changed: the Talker prefill replays a packed graph over token buckets 32..1024).
 * Several sequences are packed into one call: sequence s holds rows
 * [seq_start[s], seq_start[s+1]) of `embeds`, its positions 0, 1, ... from an
 * empty cache, and every row runs the same decoder layers as a decode step
 * (q/k-norm before RoPE, grouped-query attention causal within its sequence).
 * The keys and values of every position go to the sequence's pages, so decode
 * frames can follow with kv_len = the sequence length.  At each sequence's last
 * row the codec head gives logits0 (and its greedy codebook-0 token), and the
 * final-normed hidden state is what a PREDICTOR-mode frame takes as h_in.
 * Rows past seq_start[max_seqs] are padding: they write no keys or values.  A
 * graph captured for one `rows` (a bucket) serves every packing of at most that
 * many rows, since the boundaries are read from device memory. */
#define QT_PREFILL_MAX_SEQS 32
#define QT_PREFILL_MAX_ROWS 4096

typedef struct {
  int32_t rows;              /* R: rows of the call, a multiple of 16; above 64, a multiple of 64;
                                at most QT_PREFILL_MAX_ROWS */
  int32_t max_seqs;          /* 1..QT_PREFILL_MAX_SEQS */
  const int32_t* seq_start;  /* device int32 [max_seqs + 1], non-decreasing, seq_start[0] = 0,
                                seq_start[max_seqs] <= rows */
  const void* embeds;        /* device bf16 [rows][talker hidden]: the Talker input of each row */
  const int32_t* page_table; /* device int32 [max_seqs][max_pages]: page of positions
                                [i*page_size, (i+1)*page_size) of sequence s */
  int32_t max_pages;
  int32_t* kv_len;           /* device int32 [max_seqs]: set to each sequence's length */
  float* logits0;            /* device f32 [max_seqs][talker_vocab]: codec head at the last row
                                (all zero for an empty sequence) */
  int32_t* tok0;             /* device int32 [max_seqs] or NULL: greedy codebook-0 token there */
  void* h_last;              /* device bf16 [max_seqs][talker hidden] or NULL: final-normed hidden */
  uint32_t* status;          /* device uint32 [1]: QT_STATUS_* bits are OR-ed in */
} qt_prefill_args;

/* Bytes of the prefill workspace for `rows` rows and max_seqs sequences. */
qt_status qt_prefill_workspace_bytes(const qt_model_cfg* cfg, int32_t rows, int32_t max_seqs,
                                     uint64_t* bytes);

/* Enqueue a prefill on `stream` (no host synchronisation).  `workspace`: at least
 * qt_prefill_workspace_bytes, 256-byte aligned, not shared with a call in flight.
 * A sequence longer than max_pages * page_size sets QT_STATUS_KV_OVERFLOW and its
 * positions past the capacity are not stored.  The Talker runs on its unquantised
 * weights in both modes ("Qwen3-TTS Native v0.3.0", What changed: prefill stays
 * BF16); QT_E_UNSUPPORTED if an INT8-mode model holds a Talker weight beyond the
 * half range (see qt_load_weights). */
qt_status qt_prefill(qt_model* model, const qt_prefill_args* args, const qt_kv_caches* kv,
                     void* workspace, uint64_t workspace_bytes, void* stream);

/* Capture the same prefill into a graph (see qt_frame_graph_create for ownership). */
qt_status qt_prefill_graph_create(qt_model* model, const qt_prefill_args* args,
                                  const qt_kv_caches* kv, void* workspace,
                                  uint64_t workspace_bytes, qt_graph** out_graph);

/* ------------------------------------------------------------------ tracing
 * Per-kernel timing of one frame, for measuring each kernel against the memory
 * roofline.  A frame is launched as a sequence of kernels; qt_frame_trace enqueues
 * exactly the kernels qt_frame_decode enqueues, with the same arguments, each
 * through hipExtLaunchKernel with a start and a stop event that the runtime stamps
 * with that kernel's own begin and end (dispatch gaps between kernels are not in
 * the intervals).  The frame's results are the same as qt_frame_decode's. */
typedef enum {
  QT_KERNEL_FRAME_BEGIN = 0, /* k_frame_begin: per-session entry state */
  QT_KERNEL_GEMM = 1,        /* k_gemm_valu / k_gemm_mfma: one weight matrix over m rows */
  QT_KERNEL_ATTN_PAGED = 2,  /* k_attn_paged: Talker q/k-norm, RoPE, KV append, paged attention */
  QT_KERNEL_ATTN_PRED = 3,   /* k_attn_pred: the same over the predictor's frame-local KV */
  QT_KERNEL_EMBED = 4,       /* k_embed: codebook-embedding gather of a predictor step */
  QT_KERNEL_FRAME_END = 5,   /* k_frame_end: tokens out, kv_len advance */
  QT_KERNEL_PREDICTOR = 6,   /* k_pred_persist: every code-predictor step of the frame in one
                                launch (QT_PREDICTOR=persistent; see qt_frame_decode); by
                                default the predictor runs as QT_KERNEL_EMBED / GEMM /
                                ATTN_PRED launches */
  QT_KERNEL_ATTN_MERGE = 7   /* k_attn_merge: the Talker attention's split partials merged in
                                split order, after each QT_KERNEL_ATTN_PAGED launch of a frame
                                of 16 sessions or more (below 16, the last split to finish
                                merges them inside k_attn_paged) */
} qt_kernel_kind;

typedef struct {
  int32_t kind;     /* qt_kernel_kind */
  int32_t step;     /* 0: Talker or frame entry/exit; k in 1..n_codebooks-1: predictor step k */
  int32_t layer;    /* decoder layer of the launch, -1 if none */
  int32_t m;        /* GEMM: activation rows; other kernels: sessions */
  int32_t n, k;     /* GEMM: weight rows and columns streamed (W is [n, k]); else 0 */
  int32_t int8;     /* GEMM weight storage: 0 half (bf16 mode); 1 int8 tiles + f32 row
                       scales; 2 INT8-quantised values held as half tiles + f32 row
                       scales (the code predictor's matrices in INT8 mode) */
  int32_t n_logits; /* GEMM: f32 logits written per row (head GEMMs), else 0 */
  char name[40];    /* kernel symbol with its template arguments, e.g. "k_gemm_mfma<2,2,false>" */
} qt_launch_info;

typedef struct qt_trace qt_trace;

/* Create a trace handle holding timing events for up to max_launches launches. */
qt_status qt_trace_create(int32_t max_launches, qt_trace** out);

/* Number of kernel launches one frame of this mode and batch (1..32 sessions) makes:
 * *n receives it.  From 16 sessions on, each Talker layer adds a QT_KERNEL_ATTN_MERGE
 * launch.  QT_E_INVALID_ARG for a NULL pointer, a mode outside qt_mode or a batch
 * outside 1..32; a cfg that qt_model_create would refuse is refused the same way. */
qt_status qt_frame_launch_count(const qt_model_cfg* cfg, int32_t mode, int32_t batch, int32_t* n);

/* Enqueue one frame exactly as qt_frame_decode (same arguments and checks) with the
 * trace's events recorded around its launches.  QT_E_CAPACITY, before anything is
 * enqueued, if the frame has more launches than the trace holds. */
qt_status qt_frame_trace(qt_model* model, const qt_sessions* sessions, const qt_kv_caches* kv,
                         const qt_frame_inputs* in, const qt_frame_outputs* out, void* workspace,
                         uint64_t workspace_bytes, void* stream, qt_trace* trace);

/* Wait for the last traced frame to finish and read it back: info[i] (host array) and
 * ms[i] = milliseconds from begin to end of launch i, for i < *n.  QT_E_CAPACITY
 * if max < the number of launches; QT_E_STATE if no frame has been traced. */
qt_status qt_trace_read(qt_trace* trace, qt_launch_info* info, float* ms, int32_t max,
                        int32_t* n);

void qt_trace_destroy(qt_trace* trace);

#ifdef __cplusplus
}
#endif
#endif
