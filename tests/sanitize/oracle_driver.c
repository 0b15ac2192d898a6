/* Drives the CPU oracle through full, Talker-only and predictor-only frames of a
 * tiny model (two layers per stack, ragged cache lengths), in bf16 and INT8 weight
 * modes, for the address / undefined-behaviour sanitizer build of the tests.  The
 * weights are filler values from a fixed xorshift sequence: only memory and
 * arithmetic safety is checked here, not the results. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qt_oracle.h"

static uint32_t rng_state = 0x9e3779b9u;
static uint32_t next_u32(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return rng_state;
}
/* a bf16 bit pattern of a value in (-scale, scale) */
static uint16_t filler(float scale) {
  const float u = ((float)(next_u32() >> 8) / 16777216.0f) * 2.0f - 1.0f;
  float v = u * scale;
  uint32_t b;
  memcpy(&b, &v, 4);
  return (uint16_t)(b >> 16);
}
static uint16_t* vec(int n, float scale, float offset) {
  uint16_t* p = (uint16_t*)malloc((size_t)n * 2);
  for (int i = 0; i < n; ++i) {
    float v = offset + ((float)(next_u32() >> 8) / 16777216.0f - 0.5f) * scale;
    uint32_t b;
    memcpy(&b, &v, 4);
    p[i] = (uint16_t)(b >> 16);
  }
  return p;
}

typedef struct {
  orc_mat m;
  int8_t* q;
  float* s;
} mat_t;

static void make_mat(mat_t* t, int rows, int cols, int int8) {
  uint16_t* w = (uint16_t*)malloc((size_t)rows * cols * 2);
  for (int64_t i = 0; i < (int64_t)rows * cols; ++i) w[i] = filler(0.2f);
  t->m.rows = rows;
  t->m.cols = cols;
  t->m.w = w;
  t->m.q = NULL;
  t->m.s = NULL;
  t->q = NULL;
  t->s = NULL;
  if (int8) {
    t->q = (int8_t*)malloc((size_t)rows * cols);
    t->s = (float*)malloc((size_t)rows * 4);
    if (orc_quantize_int8(w, rows, cols, t->q, t->s) != rows) exit(3);
    t->m.w = NULL;
    t->m.q = t->q;
    t->m.s = t->s;
    free(w);
  }
}

static void make_stack(orc_stack* st, orc_layer* L, orc_dims d, int int8, mat_t* store) {
  const int qd = d.n_q * d.head_dim, kvd = d.n_kv * d.head_dim;
  for (int l = 0; l < d.layers; ++l) {
    mat_t* m = store + 7 * l;
    make_mat(&m[0], qd, d.hidden, int8);
    make_mat(&m[1], kvd, d.hidden, int8);
    make_mat(&m[2], kvd, d.hidden, int8);
    make_mat(&m[3], d.hidden, qd, int8);
    make_mat(&m[4], d.ffn, d.hidden, int8);
    make_mat(&m[5], d.ffn, d.hidden, int8);
    make_mat(&m[6], d.hidden, d.ffn, int8);
    L[l].in_norm = vec(d.hidden, 0.2f, 1.0f);
    L[l].q_norm = vec(d.head_dim, 0.2f, 1.0f);
    L[l].k_norm = vec(d.head_dim, 0.2f, 1.0f);
    L[l].post_norm = vec(d.hidden, 0.2f, 1.0f);
    L[l].q = m[0].m;
    L[l].k = m[1].m;
    L[l].v = m[2].m;
    L[l].o = m[3].m;
    L[l].gate = m[4].m;
    L[l].up = m[5].m;
    L[l].down = m[6].m;
  }
  st->dims = d;
  st->layers = L;
  st->final_norm = vec(d.hidden, 0.2f, 1.0f);
}

static double run(int int8) {
  const orc_dims td = {2, 64, 4, 2, 16, 96, 1.0e6, 1.0e-6};
  const orc_dims pd = {2, 32, 4, 2, 16, 48, 1.0e6, 1.0e-6};
  const int talker_vocab = 40, code_vocab = 32, cb0 = 32, ncb = 4;
  orc_layer tl[2], pl[2];
  mat_t tm[14], pm[14], head, proj, heads[3];
  orc_mat lm[3];
  const uint16_t* emb[3];
  orc_model M;
  make_stack(&M.talker, tl, td, int8, tm);
  make_stack(&M.predictor, pl, pd, int8, pm);
  make_mat(&head, talker_vocab, td.hidden, int8);
  make_mat(&proj, pd.hidden, td.hidden, int8);
  for (int i = 0; i < ncb - 1; ++i) {
    make_mat(&heads[i], code_vocab, pd.hidden, int8);
    lm[i] = heads[i].m;
    emb[i] = vec(code_vocab * pd.hidden, 1.0f, 0.0f);
  }
  M.codec_head = head.m;
  M.projection = proj.m;
  M.lm_heads = lm;
  M.embeds = emb;
  M.talker_vocab = talker_vocab;
  M.code_vocab = code_vocab;
  M.cb0_range = cb0;
  M.n_codebooks = ncb;

  double check = 0.0;
  const int lens[3] = {0, 5, 13}, frames = 3, cap = 16;
  const size_t kv_elems = (size_t)td.layers * cap * td.n_kv * td.head_dim;
  double* x = (double*)malloc(sizeof(double) * td.hidden);
  double* l0 = (double*)malloc(sizeof(double) * talker_vocab);
  double* lp = (double*)malloc(sizeof(double) * (ncb - 1) * code_vocab);
  double* h = (double*)malloc(sizeof(double) * td.hidden);
  int32_t tok[4];
  for (int s = 0; s < 3; ++s) {
    double* kc = (double*)calloc(kv_elems, sizeof(double));
    double* vc = (double*)calloc(kv_elems, sizeof(double));
    for (size_t i = 0; i < (size_t)td.layers * lens[s] * td.n_kv * td.head_dim; ++i) {
      kc[i] = (double)(int32_t)next_u32() / 2147483648.0;
      vc[i] = (double)(int32_t)next_u32() / 2147483648.0;
    }
    int32_t len = lens[s];
    for (int f = 0; f < frames; ++f) {
      for (int i = 0; i < td.hidden; ++i) x[i] = (double)(int32_t)next_u32() / 2147483648.0;
      const int mode = (f == 1) ? ORC_MODE_TALKER : ORC_MODE_FULL;
      if (orc_frame(&M, mode, x, NULL, 0, kc, vc, cap, &len, NULL, l0, lp, tok, h) != 0) exit(4);
      for (int i = 0; i < talker_vocab; ++i) check += l0[i];
    }
    if (len != lens[s] + frames) exit(5);
    /* predictor-only frame from the last hidden state and a forced table */
    int32_t forced[4] = {1, 2, 3, 4};
    if (orc_frame(&M, ORC_MODE_PREDICTOR, NULL, h, 7, NULL, NULL, 0, &len, forced, l0, lp, tok, NULL) != 0)
      exit(6);
    for (int i = 0; i < (ncb - 1) * code_vocab; ++i) check += lp[i];
    free(kc);
    free(vc);
  }
  free(x);
  free(l0);
  free(lp);
  free(h);
  for (int i = 0; i < 14; ++i) {
    free((void*)tm[i].m.w); free(tm[i].q); free(tm[i].s);
    free((void*)pm[i].m.w); free(pm[i].q); free(pm[i].s);
  }
  for (int l = 0; l < 2; ++l) {
    free((void*)tl[l].in_norm); free((void*)tl[l].q_norm); free((void*)tl[l].k_norm);
    free((void*)tl[l].post_norm);
    free((void*)pl[l].in_norm); free((void*)pl[l].q_norm); free((void*)pl[l].k_norm);
    free((void*)pl[l].post_norm);
  }
  free((void*)M.talker.final_norm);
  free((void*)M.predictor.final_norm);
  free((void*)head.m.w); free(head.q); free(head.s);
  free((void*)proj.m.w); free(proj.q); free(proj.s);
  for (int i = 0; i < ncb - 1; ++i) {
    free((void*)heads[i].m.w); free(heads[i].q); free(heads[i].s);
    free((void*)emb[i]);
  }
  return check;
}

int main(void) {
  const double a = run(0), b = run(1);
  if (!isfinite(a) || !isfinite(b)) return 7;
  printf("oracle driver ok %.6g %.6g\n", a, b);
  return 0;
}
