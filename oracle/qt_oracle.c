/*
 * CPU oracle for the lockstep Qwen3-TTS-style decode frame -- plain C99 + OpenMP.
 *
 * TEST INFRASTRUCTURE ONLY (see qt_oracle.h).  Every function is the plain
 * definition of its step, written so that it can be checked against the pages
 * by eye: no blocking, no fusion, no reordering beyond the definition.
 * OpenMP only splits independent output rows / heads across threads; every
 * dot product is one sequential float64 sum in index order, so results do
 * not depend on the thread count.
 *
 * What the frame is (sources):
 *  - "Qwen3-TTS Native v0.3.0" release notes, What changed: one call runs the
 *    Talker step and the 15-step code predictor for every active session.
 *  - decomputer.nl article on Qwen3-TTS serving, section "Hoe we Qwen3-TTS hebben
 *    geoptimaliseerd": the Talker predicts codebook 0, the Code Predictor the
 *    remaining 15 codebooks; section 3: always exactly 15 steps per frame with
 *    a preallocated predictor KV cache.
 *  - M* "Qwen3-TTS PR 5", What changed vs the 0.6B port: the Talker-to-predictor
 *    projection 2048 -> 1024; Graph section: paged KV and RoPE positions.
 * The pages do not spell out the layer; this follows the plain Qwen3-style
 * decoder layer: pre-norm RMSNorm, per-head RMSNorm on q and k before
 * rotate-half RoPE, grouped-query attention with scale 1/sqrt(head_dim), no
 * biases, SwiGLU feed-forward, residual adds, a final RMSNorm per stack.
 */
#include "qt_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Thread count of the OpenMP loops, for timing the oracle (results do not depend
 * on it: every dot product is summed by one thread in index order). */
int32_t orc_max_threads(void) { return (int32_t)omp_get_max_threads(); }
void orc_set_threads(int32_t n) { omp_set_num_threads(n > 0 ? n : 1); }

double orc_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* RMSNorm: y = x / sqrt(mean(x^2) + eps) * g.  y may alias x. */
void orc_rmsnorm(const double* x, const uint16_t* g, int32_t n, double eps, double* y) {
  double ss = 0.0;
  for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
  const double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int32_t i = 0; i < n; ++i) y[i] = x[i] * inv * orc_bf16_to_f64(g[i]);
}

/* Rotate-half RoPE at integer position pos: pair (i, i + d/2) turns by the
 * angle pos * theta^(-2i/d).  ("RoPE positions" are a Talker resource in the
 * M* page's Graph section; the frequency base 1e6 is the workload's.) */
void orc_rope(double* v, int32_t d, int64_t pos, double theta) {
  const int32_t half = d / 2;
  for (int32_t i = 0; i < half; ++i) {
    const double inv_freq = pow(theta, -(2.0 * (double)i) / (double)d);
    const double a = (double)pos * inv_freq;
    const double c = cos(a), s = sin(a);
    const double x1 = v[i], x2 = v[i + half];
    v[i] = x1 * c - x2 * s;
    v[i + half] = x2 * c + x1 * s;
  }
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* y = W x for a row-major [rows, cols] matrix.  INT8 mode: y_r = s_r * sum_k q_rk x_k
 * ("Qwen3-TTS Native v0.3.0", What changed: per-output-channel symmetric INT8). */
void orc_linear(const orc_mat* m, const double* x, double* y) {
  const int32_t rows = m->rows, cols = m->cols;
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < rows; ++r) {
    double acc = 0.0;
    if (m->q) {
      const int8_t* row = m->q + (int64_t)r * cols;
      for (int32_t k = 0; k < cols; ++k) acc += (double)row[k] * x[k];
      y[r] = (double)m->s[r] * acc;
    } else {
      const uint16_t* row = m->w + (int64_t)r * cols;
      for (int32_t k = 0; k < cols; ++k) acc += orc_bf16_to_f64(row[k]) * x[k];
      y[r] = acc;
    }
  }
}

/* softmax(q . K[t] / sqrt(d)) weighted sum of V[t] over t = 0 .. n_pos-1. */
void orc_attend(const double* q, const double* K, const double* V, int32_t n_pos,
                int64_t stride, int32_t d, double* out) {
  for (int32_t i = 0; i < d; ++i) out[i] = 0.0;
  if (n_pos <= 0) return;
  double* s = (double*)malloc(sizeof(double) * (size_t)n_pos);
  const double scale = 1.0 / sqrt((double)d);
  double mx = -INFINITY;
  for (int32_t t = 0; t < n_pos; ++t) {
    double dot = 0.0;
    for (int32_t i = 0; i < d; ++i) dot += q[i] * K[(int64_t)t * stride + i];
    s[t] = dot * scale;
    if (s[t] > mx) mx = s[t];
  }
  double den = 0.0;
  for (int32_t t = 0; t < n_pos; ++t) {
    s[t] = exp(s[t] - mx);
    den += s[t];
  }
  for (int32_t t = 0; t < n_pos; ++t) {
    const double p = s[t] / den;
    for (int32_t i = 0; i < d; ++i) out[i] += p * V[(int64_t)t * stride + i];
  }
  free(s);
}

/* Grouped-query attention: query head j reads KV head floor(j / (n_q / n_kv)). */
void orc_gqa(const double* q, const double* K, const double* V, int32_t n_pos,
             int32_t n_q, int32_t n_kv, int32_t d, double* out) {
  const int32_t group = n_q / n_kv;
  const int64_t stride = (int64_t)n_kv * d;
#pragma omp parallel for schedule(static)
  for (int32_t j = 0; j < n_q; ++j) {
    const int32_t h = j / group;
    orc_attend(q + (int64_t)j * d, K + (int64_t)h * d, V + (int64_t)h * d, n_pos, stride, d,
               out + (int64_t)j * d);
  }
}

int32_t orc_argmax(const double* v, int32_t n) {
  int32_t best = -1;
  for (int32_t i = 0; i < n; ++i) {
    if (isnan(v[i])) return -1;
    if (best < 0 || v[i] > v[best]) best = i;
  }
  return best;
}

/* Per-output-channel symmetric INT8 ("Qwen3-TTS Native v0.3.0", What changed):
 * s = f32(max_k |w_k|) / 127 in IEEE float32; q_k = clamp(rint(w_k / s), -127, 127)
 * with an IEEE float32 divide and round-half-to-even; an all-zero row gives s = 0, q = 0. */
int64_t orc_quantize_int8(const uint16_t* w, int64_t rows, int64_t cols, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* row = w + r * cols;
    float amax = 0.0f;
    for (int64_t k = 0; k < cols; ++k) {
      const float a = fabsf(bf16_to_f32(row[k]));
      if (a > amax) amax = a;
    }
    const float sc = amax / 127.0f;
    s[r] = sc;
    for (int64_t k = 0; k < cols; ++k) {
      float rq = 0.0f;
      if (sc != 0.0f) {
        const float t = bf16_to_f32(row[k]) / sc;
        rq = nearbyintf(t); /* default rounding mode: to nearest, ties to even */
        if (rq > 127.0f) rq = 127.0f;
        if (rq < -127.0f) rq = -127.0f;
      }
      q[r * cols + k] = (int8_t)rq;
    }
  }
  return rows;
}

int32_t orc_stack_forward(const orc_stack* st, double* x, int32_t n_new, int32_t pos0,
                          double* kc, double* vc, int32_t cap) {
  const orc_dims* d = &st->dims;
  if (n_new <= 0 || pos0 < 0 || pos0 + n_new > cap) return -1;
  const int32_t H = d->hidden, hd = d->head_dim, nq = d->n_q, nkv = d->n_kv, F = d->ffn;
  const int32_t qd = nq * hd, kvd = nkv * hd;
  const double eps = d->eps;
  double* u = (double*)malloc(sizeof(double) * (size_t)(H > F ? H : F));
  double* q = (double*)malloc(sizeof(double) * (size_t)n_new * qd);
  double* k = (double*)malloc(sizeof(double) * (size_t)kvd);
  double* v = (double*)malloc(sizeof(double) * (size_t)kvd);
  double* o = (double*)malloc(sizeof(double) * (size_t)n_new * qd);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)H);
  double* g = (double*)malloc(sizeof(double) * (size_t)F);
  double* up = (double*)malloc(sizeof(double) * (size_t)F);
  const int64_t lstride = (int64_t)cap * kvd;

  for (int32_t l = 0; l < d->layers; ++l) {
    const orc_layer* L = &st->layers[l];
    double* Kl = kc + (int64_t)l * lstride;
    double* Vl = vc + (int64_t)l * lstride;
    /* projections; per-head q/k RMSNorm then RoPE; append k, v at the position */
    for (int32_t i = 0; i < n_new; ++i) {
      const int32_t pos = pos0 + i;
      double* qi = q + (int64_t)i * qd;
      orc_rmsnorm(x + (int64_t)i * H, L->in_norm, H, eps, u);
      orc_linear(&L->q, u, qi);
      orc_linear(&L->k, u, k);
      orc_linear(&L->v, u, v);
      for (int32_t j = 0; j < nq; ++j) {
        orc_rmsnorm(qi + j * hd, L->q_norm, hd, eps, qi + j * hd);
        orc_rope(qi + j * hd, hd, pos, d->rope_theta);
      }
      for (int32_t h = 0; h < nkv; ++h) {
        orc_rmsnorm(k + h * hd, L->k_norm, hd, eps, k + h * hd);
        orc_rope(k + h * hd, hd, pos, d->rope_theta);
      }
      memcpy(Kl + (int64_t)pos * kvd, k, sizeof(double) * (size_t)kvd);
      memcpy(Vl + (int64_t)pos * kvd, v, sizeof(double) * (size_t)kvd);
    }
    /* causal attention: the new position pos0+i sees cache positions 0 .. pos0+i */
    for (int32_t i = 0; i < n_new; ++i)
      orc_gqa(q + (int64_t)i * qd, Kl, Vl, pos0 + i + 1, nq, nkv, hd, o + (int64_t)i * qd);
    /* output projection + residual, SwiGLU feed-forward + residual */
    for (int32_t i = 0; i < n_new; ++i) {
      double* xi = x + (int64_t)i * H;
      orc_linear(&L->o, o + (int64_t)i * qd, tmp);
      for (int32_t r = 0; r < H; ++r) xi[r] += tmp[r];
      orc_rmsnorm(xi, L->post_norm, H, eps, u);
      orc_linear(&L->gate, u, g);
      orc_linear(&L->up, u, up);
      for (int32_t f = 0; f < F; ++f) g[f] = orc_silu(g[f]) * up[f];
      orc_linear(&L->down, g, tmp);
      for (int32_t r = 0; r < H; ++r) xi[r] += tmp[r];
    }
  }
  for (int32_t i = 0; i < n_new; ++i)
    orc_rmsnorm(x + (int64_t)i * H, st->final_norm, H, eps, x + (int64_t)i * H);

  free(u); free(q); free(k); free(v); free(o); free(tmp); free(g); free(up);
  return 0;
}

static void embed_row(const uint16_t* table, int32_t cols, int32_t tok, double* out) {
  const uint16_t* row = table + (int64_t)tok * cols;
  for (int32_t c = 0; c < cols; ++c) out[c] = orc_bf16_to_f64(row[c]);
}

int32_t orc_frame(const orc_model* m, int32_t mode, const double* talker_in,
                  const double* h_in, int32_t tok0_in, double* kc, double* vc,
                  int32_t capacity, int32_t* len, const int32_t* forced,
                  double* logits0, double* logits_pred, int32_t* tokens, double* h_out) {
  const int32_t Ht = m->talker.dims.hidden, Hp = m->predictor.dims.hidden;
  const int32_t ncb = m->n_codebooks, Vc = m->code_vocab;
  int32_t rc = 0;
  double* h = (double*)malloc(sizeof(double) * (size_t)Ht);
  double* xp = (double*)malloc(sizeof(double) * (size_t)2 * Hp);
  const int32_t pl = m->predictor.dims.layers;
  const int64_t pkv = (int64_t)pl * ncb * m->predictor.dims.n_kv * m->predictor.dims.head_dim;
  double* pk = (double*)calloc((size_t)pkv, sizeof(double));
  double* pv = (double*)calloc((size_t)pkv, sizeof(double));
  int32_t tok0;

  if (mode == ORC_MODE_FULL || mode == ORC_MODE_TALKER) {
    /* Talker step at position *len, codec head, codebook-0 argmax over [0, cb0_range) */
    memcpy(h, talker_in, sizeof(double) * (size_t)Ht);
    if (orc_stack_forward(&m->talker, h, 1, *len, kc, vc, capacity)) { rc = -1; goto done; }
    *len += 1;
    orc_linear(&m->codec_head, h, logits0);
    tok0 = orc_argmax(logits0, m->cb0_range);
    if (tok0 < 0) { rc = -2; goto done; }
    tokens[0] = tok0;
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)Ht);
    if (mode == ORC_MODE_TALKER) goto done;
  } else {
    memcpy(h, h_in, sizeof(double) * (size_t)Ht);
    tok0 = tok0_in;
    tokens[0] = tok0_in;
  }

  /* predictor step 1: position 0 holds the projected Talker hidden, position 1
   * the codebook-0 token's embedding; head 1 reads position 1 */
  orc_linear(&m->projection, h, xp);
  {
    const int32_t prev = forced ? forced[0] : tok0;
    if (prev < 0 || prev >= Vc) { rc = -3; goto done; }
    embed_row(m->embeds[0], Hp, prev, xp + Hp);
  }
  if (orc_stack_forward(&m->predictor, xp, 2, 0, pk, pv, ncb)) { rc = -1; goto done; }
  orc_linear(&m->lm_heads[0], xp + Hp, logits_pred);
  tokens[1] = orc_argmax(logits_pred, Vc);
  if (tokens[1] < 0) { rc = -2; goto done; }
  /* predictor steps k = 2 .. ncb-1: position k holds E_k[tok_{k-1}] */
  for (int32_t k = 2; k < ncb; ++k) {
    const int32_t prev = forced ? forced[k - 1] : tokens[k - 1];
    if (prev < 0 || prev >= Vc) { rc = -3; goto done; }
    embed_row(m->embeds[k - 1], Hp, prev, xp);
    if (orc_stack_forward(&m->predictor, xp, 1, k, pk, pv, ncb)) { rc = -1; goto done; }
    double* lg = logits_pred + (int64_t)(k - 1) * Vc;
    orc_linear(&m->lm_heads[k - 1], xp, lg);
    tokens[k] = orc_argmax(lg, Vc);
    if (tokens[k] < 0) { rc = -2; goto done; }
  }
done:
  free(h); free(xp); free(pk); free(pv);
  return rc;
}
