/*
 * CPU oracle for the lockstep Qwen3-TTS-style decode frame.
 *
 * TEST INFRASTRUCTURE ONLY.  This code is the slow, plain reference that the
 * HIP path is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Arithmetic: float64 throughout, bfloat16 weights widened exactly.  The one
 * exception is the INT8 quantizer, whose definition (per-output-channel
 * symmetric, scale = max|w| / 127, round half to even, clamp to +-127;
 * "Qwen3-TTS Native v0.3.0", What changed, INT8 decode bullet) is evaluated
 * in IEEE float32 exactly as written, because its result must be reproduced
 * bit for bit.
 *
 * Layouts: every matrix is row-major [out, in] (y = W x).  The oracle's KV
 * cache is contiguous per session: [layers][capacity][n_kv][head_dim] float64.
 */
#ifndef QT_ORACLE_H
#define QT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t layers, hidden, n_q, n_kv, head_dim, ffn;
  double rope_theta, eps;
} orc_dims;

/* y = W x.  bf16 mode: w != NULL.  INT8 mode: q, s != NULL, y_n = s_n sum_k q_nk x_k. */
typedef struct {
  const uint16_t* w;
  const int8_t* q;
  const float* s;
  int32_t rows, cols;
} orc_mat;

typedef struct {
  const uint16_t *in_norm, *q_norm, *k_norm, *post_norm;
  orc_mat q, k, v, o, gate, up, down;
} orc_layer;

typedef struct {
  orc_dims dims;
  const orc_layer* layers;
  const uint16_t* final_norm;
} orc_stack;

typedef struct {
  orc_stack talker, predictor;
  orc_mat codec_head, projection;
  const orc_mat* lm_heads;          /* [n_codebooks - 1] */
  const uint16_t* const* embeds;    /* [n_codebooks - 1], each [code_vocab][predictor hidden] */
  int32_t talker_vocab, code_vocab, cb0_range, n_codebooks;
} orc_model;

enum { ORC_MODE_FULL = 0, ORC_MODE_TALKER = 1, ORC_MODE_PREDICTOR = 2 };

/* ---- pieces (exposed for the closed-form pins) ---- */
double orc_bf16_to_f64(uint16_t h);
void orc_rmsnorm(const double* x, const uint16_t* g, int32_t n, double eps, double* y);
void orc_rope(double* v, int32_t head_dim, int64_t pos, double theta);
double orc_silu(double z);
void orc_linear(const orc_mat* m, const double* x, double* y);
/* one query head over n_pos cached positions; K/V rows are `stride` doubles apart */
void orc_attend(const double* q, const double* K, const double* V, int32_t n_pos,
                int64_t stride, int32_t head_dim, double* out);
/* grouped-query attention: q [n_q][hd]; K,V [n_pos][n_kv][hd]; out [n_q][hd] */
void orc_gqa(const double* q, const double* K, const double* V, int32_t n_pos,
             int32_t n_q, int32_t n_kv, int32_t head_dim, double* out);
/* argmax over v[0..n); ties go to the lowest index; -1 if any NaN is present */
int32_t orc_argmax(const double* v, int32_t n);
/* per-row symmetric INT8; returns the number of rows processed */
int64_t orc_quantize_int8(const uint16_t* w, int64_t rows, int64_t cols, int8_t* q, float* s);

/* Run a decoder stack on n_new consecutive positions pos0 .. pos0+n_new-1 of one
 * session.  x: [n_new][hidden] inputs, overwritten with the final-normed outputs.
 * kc/vc: the session cache [layers][capacity][n_kv][head_dim]; positions < pos0
 * must hold the earlier keys/values; the new ones are written.  Returns 0, or -1
 * if pos0 + n_new > capacity. */
int32_t orc_stack_forward(const orc_stack* st, double* x, int32_t n_new, int32_t pos0,
                          double* kc, double* vc, int32_t capacity);

/* OpenMP thread count of the oracle's loops (for timing only; results do not
 * depend on it). */
int32_t orc_max_threads(void);
void orc_set_threads(int32_t n);

/* One decode frame for one session.
 *   mode FULL:      talker_in -> Talker at position *len -> logits0, tok0 ->
 *                   projection -> predictor steps 1..n_codebooks-1.
 *   mode TALKER:    only the Talker step, logits0 and tok0.
 *   mode PREDICTOR: h_in (the post-norm Talker hidden, [talker hidden]) and tok0_in
 *                   feed the projection and the predictor steps.
 * forced: NULL, or [n_codebooks] tokens; when given, the predictor's embedding
 *   lookups use forced[k-1] in place of the frame's own tok_{k-1}.
 * Outputs: logits0 [talker_vocab] (FULL/TALKER), logits_pred [(n_cb-1)][code_vocab]
 *   (FULL/PREDICTOR), tokens [n_cb] (own argmaxes; PREDICTOR copies tok0_in to [0]),
 *   h_out [talker hidden] (optional, FULL/TALKER: the post-norm Talker output).
 * *len is advanced by one in FULL/TALKER mode.  Returns 0 or a negative error. */
int32_t orc_frame(const orc_model* m, int32_t mode, const double* talker_in,
                  const double* h_in, int32_t tok0_in, double* kc, double* vc,
                  int32_t capacity, int32_t* len, const int32_t* forced,
                  double* logits0, double* logits_pred, int32_t* tokens, double* h_out);

#ifdef __cplusplus
}
#endif
#endif
