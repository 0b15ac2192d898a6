// C ABI of the lockstep decode-frame library: argument validation, weight
// packing, workspace layout, the per-frame kernel sequence and its HIP graph.
// The kernels themselves live in qt_kernels.hip.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "qt.h"
#include "qt_internal.h"

using namespace qt;

namespace qt {
thread_local LaunchEvents g_launch_events;
}

namespace {

thread_local std::string g_err;

qt_status fail(qt_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

qt_status ok() { return QT_OK; }

// Launches of one frame of B sessions: entry, per Talker layer QKV / attention
// (+ the split merge from kAttnMergeMinBatch sessions on) / o / gate-up / down, the
// head GEMM, per predictor step the gather, 5-kernel layers and the step head, and
// the exit kernel.
int frame_launches(const qt_model_cfg& c, int mode, int B) {
  int n = 3;  // entry, head GEMM, exit
  if (mode != QT_MODE_PREDICTOR) n += (attn_merge_separate(B) ? 6 : 5) * c.talker.layers;
  if (mode != QT_MODE_TALKER) n += (c.n_codebooks - 1) * (2 + 5 * c.predictor.layers);
  return n;
}

#define QT_HIP(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(QT_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));            \
  } while (0)

constexpr size_t kAlign = 256;
constexpr int kMaxBatch = 32;  // predictor step 1 carries 2B rows; the GEMMs take up to 64

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// ------------------------------------------------------------------ packed layout
}  // namespace

struct qt_trace {
  std::vector<hipEvent_t> ev;  // start and stop of every launch
  std::vector<qt_launch_info> info;
  int n = -1;                  // launches of the last traced frame
};

namespace {

struct MatSlot {
  size_t w = 0, s = 0;  // byte offsets of the weight rows and (INT8) the scales
  int N = 0, K = 0;
  bool w8 = false;      // int8 tiles (else half tiles)
  size_t wh = 0;        // half tiles of the unquantised weights, for the prompt prefill
};
struct LayerSlots {
  size_t in_norm = 0, q_norm = 0, k_norm = 0, post_norm = 0;
  MatSlot qkv, o, gu, down;  // gu: gate and up rows interleaved (gate n at 2n, up n at 2n+1)
};
struct Plan {
  std::vector<LayerSlots> tl, pl;
  size_t t_final = 0, p_final = 0;
  MatSlot t_head;  // codec head rows [0, talker_vocab) then projection rows
  std::vector<size_t> embeds;
  std::vector<MatSlot> heads;
  size_t range_flags = 0;  // one word per source GEMM weight: set if it exceeds the half range
  int n_mats = 0;
  size_t total = 0;
};

struct Planner {
  size_t off = 0;
  bool i8 = false;
  size_t vec(int n) {
    size_t o = off;
    off = align_up(off + (size_t)n * 2);
    return o;
  }
  // INT8 mode quantises every decode GEMM weight; `narrow` stores the values as
  // int8 tiles (the Talker's matrices, streamed from HBM every frame, where the
  // bytes are the cost), otherwise as exact halves (the code predictor's, which
  // stay in the memory-side cache across its 15 steps and whose launches are
  // latency-bound: there unpacking int8 costs time and saving bytes gains none).
  MatSlot mat(int N, int K, bool narrow) {
    MatSlot m;
    m.N = N;
    m.K = K;
    m.w = off;
    m.w8 = i8 && narrow;
    off = align_up(off + (size_t)N * K * (m.w8 ? 1 : 2));
    if (i8) {
      m.s = off;
      off = align_up(off + (size_t)N * 4);
    }
    // The prompt prefill runs on the bf16 weights in INT8 mode too ("Qwen3-TTS
    // Native v0.3.0", What changed): the Talker's matrices keep a half copy for it.
    m.wh = m.w;
    if (m.w8) {
      m.wh = off;
      off = align_up(off + (size_t)N * K * 2);
    }
    return m;
  }
};

Plan make_plan(const qt_model_cfg& c, bool i8) {
  Planner P;
  P.i8 = i8;
  Plan plan;
  auto layers = [&](const qt_decoder_cfg& d, std::vector<LayerSlots>& v, bool narrow) {
    const int qd = d.n_q_heads * d.head_dim, kvd = d.n_kv_heads * d.head_dim;
    for (int l = 0; l < d.layers; ++l) {
      LayerSlots L;
      L.in_norm = P.vec(d.hidden);
      L.q_norm = P.vec(d.head_dim);
      L.k_norm = P.vec(d.head_dim);
      L.post_norm = P.vec(d.hidden);
      L.qkv = P.mat(qd + 2 * kvd, d.hidden, narrow);
      L.o = P.mat(d.hidden, qd, narrow);
      L.gu = P.mat(2 * d.ffn, d.hidden, narrow);
      L.down = P.mat(d.hidden, d.ffn, narrow);
      v.push_back(L);
    }
  };
  layers(c.talker, plan.tl, true);
  plan.t_final = P.vec(c.talker.hidden);
  plan.t_head = P.mat(c.talker_vocab + c.predictor.hidden, c.talker.hidden, true);
  layers(c.predictor, plan.pl, false);
  plan.p_final = P.vec(c.predictor.hidden);
  for (int i = 0; i < c.n_codebooks - 1; ++i) {
    plan.embeds.push_back(P.vec(c.code_vocab * c.predictor.hidden));
    plan.heads.push_back(P.mat(c.code_vocab, c.predictor.hidden, false));
  }
  // q, k, v, o, gate, up, down per layer; codec head, projection, one head per step
  plan.n_mats = 7 * (c.talker.layers + c.predictor.layers) + 2 + (c.n_codebooks - 1);
  plan.range_flags = P.off;
  P.off = align_up(P.off + (size_t)plan.n_mats * 4);
  plan.total = P.off;
  return plan;
}

// Where each source tensor goes in the packed buffer.
enum Kind { K_VEC, K_MAT, K_EMBED };
struct Dest {
  Kind kind;
  int64_t rows, cols;
  size_t vec_off = 0;      // K_VEC / K_EMBED
  const MatSlot* mat = nullptr;
  int row0 = 0, step = 1;  // K_MAT: source row i -> packed row row0 + i*step
};

std::map<std::string, Dest> make_dests(const qt_model_cfg& c, const Plan& plan) {
  std::map<std::string, Dest> m;
  auto vec = [&](const std::string& n, int len, size_t off) {
    Dest d{K_VEC, 1, len};
    d.vec_off = off;
    m[n] = d;
  };
  auto mat = [&](const std::string& n, int64_t rows, int64_t cols, const MatSlot* s, int row0,
                 int step) {
    Dest d{K_MAT, rows, cols};
    d.mat = s;
    d.row0 = row0;
    d.step = step;
    m[n] = d;
  };
  auto layers = [&](const char* prefix, const qt_decoder_cfg& d, const std::vector<LayerSlots>& v) {
    const int qd = d.n_q_heads * d.head_dim, kvd = d.n_kv_heads * d.head_dim;
    for (int l = 0; l < d.layers; ++l) {
      const std::string p = std::string(prefix) + ".layers." + std::to_string(l) + ".";
      const LayerSlots& L = v[l];
      vec(p + "input_norm", d.hidden, L.in_norm);
      vec(p + "q_norm", d.head_dim, L.q_norm);
      vec(p + "k_norm", d.head_dim, L.k_norm);
      vec(p + "post_norm", d.hidden, L.post_norm);
      mat(p + "q_proj", qd, d.hidden, &L.qkv, 0, 1);
      mat(p + "k_proj", kvd, d.hidden, &L.qkv, qd, 1);
      mat(p + "v_proj", kvd, d.hidden, &L.qkv, qd + kvd, 1);
      mat(p + "o_proj", d.hidden, qd, &L.o, 0, 1);
      mat(p + "gate_proj", d.ffn, d.hidden, &L.gu, 0, 2);
      mat(p + "up_proj", d.ffn, d.hidden, &L.gu, 1, 2);
      mat(p + "down_proj", d.hidden, d.ffn, &L.down, 0, 1);
    }
  };
  layers("talker", c.talker, plan.tl);
  vec("talker.final_norm", c.talker.hidden, plan.t_final);
  mat("talker.codec_head", c.talker_vocab, c.talker.hidden, &plan.t_head, 0, 1);
  mat("projection", c.predictor.hidden, c.talker.hidden, &plan.t_head, c.talker_vocab, 1);
  layers("predictor", c.predictor, plan.pl);
  vec("predictor.final_norm", c.predictor.hidden, plan.p_final);
  for (int i = 0; i < c.n_codebooks - 1; ++i) {
    Dest e{K_EMBED, c.code_vocab, c.predictor.hidden};
    e.vec_off = plan.embeds[i];
    m["predictor.codec_embed." + std::to_string(i)] = e;
    mat("predictor.lm_head." + std::to_string(i), c.code_vocab, c.predictor.hidden,
        &plan.heads[i], 0, 1);
  }
  return m;
}

qt_status check_decoder(const qt_decoder_cfg& d, const char* which) {
  if (d.layers < 1 || d.layers > 256)
    return fail(QT_E_SHAPE, "%s.layers = %d: expected 1..256", which, d.layers);
  if (d.head_dim != kHeadDim)
    return fail(QT_E_SHAPE, "%s.head_dim = %d: the library supports 128", which, d.head_dim);
  if (d.n_kv_heads < 1 || d.n_q_heads != 2 * d.n_kv_heads)
    return fail(QT_E_SHAPE, "%s: n_q_heads (%d) must be 2 * n_kv_heads (%d)", which, d.n_q_heads,
                d.n_kv_heads);
  if (d.hidden < 512 || d.hidden % 512 || d.hidden > 16384)
    return fail(QT_E_SHAPE, "%s.hidden = %d: expected a multiple of 512 up to 16384", which, d.hidden);
  if ((d.n_q_heads * d.head_dim) % 512)
    return fail(QT_E_SHAPE, "%s: n_q_heads * head_dim must be a multiple of 512", which);
  if (d.ffn < 512 || d.ffn % 512 || d.ffn > 32768)
    return fail(QT_E_SHAPE, "%s.ffn = %d: expected a multiple of 512 up to 32768", which, d.ffn);
  if (!(d.rms_eps > 0.f) || !(d.rope_theta > 1.f))
    return fail(QT_E_SHAPE, "%s: rms_eps must be > 0 and rope_theta > 1", which);
  return ok();
}

qt_status check_cfg(const qt_model_cfg* c) {
  if (!c) return fail(QT_E_INVALID_ARG, "cfg is NULL");
  qt_status st = check_decoder(c->talker, "talker");
  if (st) return st;
  if ((st = check_decoder(c->predictor, "predictor"))) return st;
  if (c->talker_vocab < 64 || c->talker_vocab % 64)
    return fail(QT_E_SHAPE, "talker_vocab = %d: expected a positive multiple of 64", c->talker_vocab);
  if (c->code_vocab < 64 || c->code_vocab % 64)
    return fail(QT_E_SHAPE, "code_vocab = %d: expected a positive multiple of 64", c->code_vocab);
  if (c->cb0_range < 1 || c->cb0_range > c->talker_vocab || c->cb0_range > c->code_vocab)
    return fail(QT_E_SHAPE, "cb0_range = %d: expected 1..min(talker_vocab, code_vocab)", c->cb0_range);
  if (c->n_codebooks < 2 || c->n_codebooks > 16)
    return fail(QT_E_SHAPE, "n_codebooks = %d: expected 2..16", c->n_codebooks);
  if (c->page_size != kPage)
    return fail(QT_E_SHAPE, "page_size = %d: the library supports 16", c->page_size);
  return ok();
}

// ------------------------------------------------------------------ workspace layout
struct Ws {
  size_t x_t, x_p, ss_t, ss_p, ut, up, qkv, o, ffn, pk, pv, part, cnt,
      cand, total;
  // the one-launch predictor (pp_ldm > 0): per-XCD rows, partial sums, sync words
  size_t pp_x, pp_u, pp_ss, pp_qkv, pp_o, pp_f, pp_po, pp_pd, pp_sync;
  int pp_ldm;
  int qkv_ld, o_ld, f_ld;
  int cand_ld;        // greedy-key candidates per (codebook, session)
  long long pk_sess;  // elements per session in the predictor cache
};

int key_blocks(int range) { return (range + kKeyBlock - 1) / kKeyBlock; }

// Split-KV shape of the Talker attention: about 1024 blocks over the page table,
// 4 to 8 pages each (fewer pages per split leave the last block of a session-head
// too many partials to merge: at B = 1, 4 pages per split took 8.3 us a layer,
// 1 page 12.2).  The workspace holds partials for the most splits any batch size
// can take (4 pages each), so a workspace sized for B sessions serves every
// smaller batch too.
constexpr int kMinPagesPerSplit = 4;
struct AttnSplit {
  int pps, n_splits;
};
AttnSplit attn_split(int B, int n_kv, int max_pages) {
  const int raw = (B * n_kv * max_pages + 1023) / 1024;
  AttnSplit s;
  s.pps = raw < kMinPagesPerSplit ? kMinPagesPerSplit : (raw > kMaxPagesPerSplit ? kMaxPagesPerSplit : raw);
  s.n_splits = (max_pages + s.pps - 1) / s.pps;
  return s;
}

// Whether a model's predictor has the shapes the one-launch predictor is written
// for (qt_pred.hip): hidden 1024, 16 query / 8 KV heads of 128, FFN 3072, code
// vocabulary 2048, at most kPredMaxLayers layers and kPredMaxSteps steps.
bool pred_persist_shapes(const qt_model_cfg& c) {
  const qt_decoder_cfg& p = c.predictor;
  return p.hidden == 1024 && p.n_q_heads == 16 && p.n_kv_heads == 8 && p.head_dim == kHeadDim &&
         p.ffn == 3072 && c.code_vocab == 2048 && p.layers <= kPredMaxLayers &&
         c.n_codebooks - 1 <= kPredMaxSteps;
}

// Residual rows carry sums of squares per producing 16-row block, so hidden/16
// slots per row.  Activation buffers are chunked [cols/8][rows][8] with rows = B
// (Talker) or 2B (predictor, whose step 1 carries two positions per session).
Ws make_ws(const qt_model_cfg& c, int B, int max_pages) {
  const qt_decoder_cfg &t = c.talker, &p = c.predictor;
  Ws w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const int M = 2 * B;
  const int tq = (t.n_q_heads + 2 * t.n_kv_heads) * t.head_dim;
  const int pq = (p.n_q_heads + 2 * p.n_kv_heads) * p.head_dim;
  w.qkv_ld = tq > pq ? tq : pq;
  w.o_ld = t.n_q_heads * t.head_dim > p.n_q_heads * p.head_dim ? t.n_q_heads * t.head_dim
                                                                 : p.n_q_heads * p.head_dim;
  w.f_ld = t.ffn > p.ffn ? t.ffn : p.ffn;
  w.x_t = take((size_t)B * t.hidden * 4);
  w.x_p = take((size_t)M * p.hidden * 4);
  w.ss_t = take((size_t)(t.hidden / kGemmRows) * B * 4);
  w.ss_p = take((size_t)(p.hidden / kGemmRows) * M * 4);
  w.ut = take((size_t)B * t.hidden * 2);
  w.up = take((size_t)M * p.hidden * 2);
  w.qkv = take((size_t)M * w.qkv_ld * 4);
  w.o = take((size_t)M * w.o_ld * 2);
  w.ffn = take((size_t)M * w.f_ld * 2);
  w.pk_sess = (long long)p.layers * c.n_codebooks * p.n_kv_heads * p.head_dim;
  w.pk = take((size_t)B * w.pk_sess * 2);
  w.pv = take((size_t)B * w.pk_sess * 2);
  const int max_splits = (max_pages + kMinPagesPerSplit - 1) / kMinPagesPerSplit;
  w.part = take((size_t)B * t.n_q_heads * (size_t)max_splits * (kHeadDim + 2) * 4);
  w.cnt = take((size_t)B * t.n_kv_heads * 4);
  w.cand_ld = key_blocks(c.cb0_range) > key_blocks(c.code_vocab) ? key_blocks(c.cb0_range)
                                                                  : key_blocks(c.code_vocab);
  w.cand = take((size_t)c.n_codebooks * B * w.cand_ld * 8);
  w.pp_ldm = 0;
  if (pred_persist_shapes(c)) {
    const int ldm = (2 * B + 15) / 16 * 16;
    const size_t H = 1024, X = 8;
    w.pp_ldm = ldm;
    w.pp_x = take(X * ldm * H * 4);
    w.pp_u = take(X * ldm * H * 2);
    w.pp_ss = take(X * 32 * ldm * 4);
    w.pp_qkv = take(X * ldm * 512 * 4);
    w.pp_o = take(X * ldm * 256 * 2);
    w.pp_f = take(X * ldm * 384 * 2);
    w.pp_po = take(X * ldm * H * 4);
    w.pp_pd = take(X * ldm * H * 4);
    w.pp_sync = take((size_t)kPredSyncWords * 4);
  }
  w.total = off;
  return w;
}

}  // namespace

// ------------------------------------------------------------------ model handle
struct qt_model {
  qt_model_cfg cfg;
  int i8;
  std::string prefill_refusal;  // INT8 mode: a Talker weight the prefill's half copy cannot hold
  int pred_persist;  // frames may run the predictor as one launch (shapes, 256 CUs)
  Plan plan;
  std::map<std::string, Dest> dests;
  char* base;  // packed buffer (device)
  uint64_t bytes;
};

struct qt_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

const uint16_t* vp(const qt_model* m, size_t off) { return (const uint16_t*)(m->base + off); }

// GEMM over a packed matrix with chunked half activations of act_ld rows.  The
// prompt prefill (prefill = true) takes the unquantised half copy in INT8 mode.
GemmArgs gemm_act(const qt_model* m, const MatSlot& s, const uint16_t* act, int act_ld, int M,
                  uint32_t* status, bool prefill = false) {
  GemmArgs a{};
  const bool q = m->i8 && !prefill;
  a.W = m->base + (prefill ? s.wh : s.w);
  a.scale = q ? (const float*)(m->base + s.s) : nullptr;
  a.w8 = q && s.w8 ? 1 : 0;
  a.N = s.N;
  a.K = s.K;
  a.row0 = 0;
  a.nrows = s.N;
  a.act = act;
  a.act_ld = act_ld;
  a.M = M;
  a.status = status;
  return a;
}

// GEMM whose input is an RMSNorm: u = half(x * gain) as left by the producer of x,
// whose sums of squares sit in `slots` slots of ss (stride ss_ld).
GemmArgs gemm_norm(const qt_model* m, const MatSlot& s, const uint16_t* u, int u_ld,
                   const float* ss, int ss_ld, int slots, float eps, int M, uint32_t* status,
                   bool prefill = false) {
  GemmArgs a = gemm_act(m, s, u, u_ld, M, status, prefill);
  a.ss_in = ss;
  a.ss_in_ld = ss_ld;
  a.ss_in_slots = slots;
  a.norm_eps = eps;
  return a;
}

#define QT_LAUNCH(expr)                                                                \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(QT_E_HIP, "launch %s failed: %s", #expr, hipGetErrorString(e_));     \
  } while (0)

qt_status check_frame_args(const qt_model* m, const qt_sessions* ss, const qt_kv_caches* kv,
                           const qt_frame_inputs* in, const qt_frame_outputs* out, void* ws,
                           uint64_t ws_bytes) {
  if (!m) return fail(QT_E_INVALID_ARG, "model is NULL");
  if (!ss || !kv || !in || !out) return fail(QT_E_INVALID_ARG, "a descriptor is NULL");
  if (!ws) return fail(QT_E_INVALID_ARG, "workspace is NULL");
  if (in->mode < QT_MODE_FULL || in->mode > QT_MODE_PREDICTOR)
    return fail(QT_E_INVALID_ARG, "mode = %d is not a qt_mode", in->mode);
  if (ss->batch < 1) return fail(QT_E_INVALID_ARG, "batch = %d: expected >= 1", ss->batch);
  if (ss->batch > kMaxBatch)
    return fail(QT_E_UNSUPPORTED, "batch = %d: the library decodes at most %d sessions per call",
                ss->batch, kMaxBatch);
  if (!out->tokens || !out->status) return fail(QT_E_INVALID_ARG, "outputs.tokens/status is NULL");
  const bool talker = in->mode != QT_MODE_PREDICTOR;
  if (talker) {
    if (!in->talker_in) return fail(QT_E_INVALID_ARG, "inputs.talker_in is NULL");
    if (!out->logits0) return fail(QT_E_INVALID_ARG, "outputs.logits0 is NULL");
    if (!ss->kv_len || !ss->page_table) return fail(QT_E_INVALID_ARG, "sessions.kv_len/page_table is NULL");
    if (ss->max_pages < 1) return fail(QT_E_INVALID_ARG, "sessions.max_pages = %d", ss->max_pages);
    if (!kv->k_pages || !kv->v_pages) return fail(QT_E_INVALID_ARG, "kv pages are NULL");
    if (kv->num_pages < 1) return fail(QT_E_INVALID_ARG, "kv.num_pages = %d", kv->num_pages);
    if (((uintptr_t)kv->k_pages | (uintptr_t)kv->v_pages) & 15)
      return fail(QT_E_INVALID_ARG, "kv pages must be 16-byte aligned");
  } else {
    if (!in->h_in || !in->tok0_in) return fail(QT_E_INVALID_ARG, "inputs.h_in/tok0_in is NULL");
  }
  if (in->mode != QT_MODE_TALKER && !out->logits_pred)
    return fail(QT_E_INVALID_ARG, "outputs.logits_pred is NULL");
  if (in->sampling) {
    const qt_sampling& sp = *in->sampling;
    if (!sp.params || !sp.seed || !sp.counter)
      return fail(QT_E_INVALID_ARG, "sampling.params/seed/counter is NULL");
    if (((uintptr_t)sp.params & 15) || ((uintptr_t)sp.seed & 7) || ((uintptr_t)sp.counter & 3) ||
        ((uintptr_t)sp.seen0 & 3))
      return fail(QT_E_INVALID_ARG, "sampling arrays are not aligned to their element size");
    if (m->cfg.cb0_range > 4096 || m->cfg.code_vocab > 4096)
      return fail(QT_E_UNSUPPORTED, "sampling draws over at most 4096 entries per row");
    if (in->mode == QT_MODE_TALKER && !out->logits0)
      return fail(QT_E_INVALID_ARG, "outputs.logits0 is NULL");
  }
  if ((uintptr_t)ws & (kAlign - 1)) return fail(QT_E_INVALID_ARG, "workspace must be 256-byte aligned");
  const int mp = talker ? ss->max_pages : 1;
  const Ws w = make_ws(m->cfg, ss->batch, mp);
  if (ws_bytes < w.total)
    return fail(QT_E_CAPACITY, "workspace has %llu bytes, this call needs %llu",
                (unsigned long long)ws_bytes, (unsigned long long)w.total);
  return ok();
}

SamplerArgs sampler_args(const qt_model_cfg& c, const qt_sampling& sp) {
  SamplerArgs a{};
  a.params = sp.params;
  a.seed = sp.seed;
  a.counter = sp.counter;
  a.seen0 = sp.seen0;
  a.seen_ld = (c.cb0_range + 31) / 32;
  return a;
}

// Enqueue one frame.  Arguments are validated by the caller.
//
// Per Talker layer: [QKV GEMM on RMSNorm(x)] -> [paged attention: q/k-norm, RoPE,
// KV append, split-KV merge] -> [o-proj GEMM, x += ; RMS statistics of x] ->
// [gate/up GEMM on RMSNorm(x), SwiGLU] -> [down GEMM, x += ; RMS statistics].
// Then the codec head (+ projection rows into the predictor's residual), and
// per predictor step: [embedding gather] -> 5 such layers -> [step head].
qt_status enqueue_frame(const qt_model* m, const qt_sessions* ss, const qt_kv_caches* kv,
                        const qt_frame_inputs* in, const qt_frame_outputs* out, void* wsp,
                        hipStream_t st, qt_trace* tr = nullptr) {
  const qt_model_cfg& c = m->cfg;
  const qt_decoder_cfg &T = c.talker, &Pd = c.predictor;
  const int B = ss->batch, ncb = c.n_codebooks, mode = in->mode;
  const bool talker = mode != QT_MODE_PREDICTOR;
  const int max_pages = talker ? ss->max_pages : 1;
  const Ws w = make_ws(c, B, max_pages);
  char* ws = (char*)wsp;
  float* x_t = (float*)(ws + w.x_t);
  float* x_p = (float*)(ws + w.x_p);
  float* ss_t = (float*)(ws + w.ss_t);
  float* ss_p = (float*)(ws + w.ss_p);
  uint16_t* ut = (uint16_t*)(ws + w.ut);
  uint16_t* up = (uint16_t*)(ws + w.up);
  float* qkv = (float*)(ws + w.qkv);
  uint16_t* o = (uint16_t*)(ws + w.o);
  uint16_t* ffn = (uint16_t*)(ws + w.ffn);
  unsigned long long* cand = (unsigned long long*)(ws + w.cand);
  const int cand_ld = w.cand_ld;
  const int ld_t = B, ld_p = 2 * B;  // rows of the chunked activation buffers
  unsigned* cnt = (unsigned*)(ws + w.cnt);
  const int capacity = max_pages * kPage;

  // Tracing: the next launch carries start/stop events stamped by the kernel itself.
  int cur_step = 0, cur_layer = -1;
  struct EventsOff {
    ~EventsOff() { g_launch_events = LaunchEvents{}; }
  } events_off;
  if (tr) tr->n = 0;
  auto mark = [&](int kind, const char* name, int rows, const GemmArgs* g) -> qt_status {
    if (!tr) return ok();
    if (tr->n >= (int)tr->info.size())
      return fail(QT_E_CAPACITY, "trace holds %d launches", (int)tr->info.size());
    qt_launch_info& li = tr->info[tr->n];
    memset(&li, 0, sizeof li);
    li.kind = kind;
    li.step = cur_step;
    li.layer = cur_layer;
    li.m = rows;
    if (g) {
      li.n = g->nrows;
      li.k = g->K;
      li.int8 = g->scale == nullptr ? 0 : (g->w8 ? 1 : 2);
      if (g->epi == EPI_HEAD) {
        const int hi = g->row0 + g->nrows < g->n_logits ? g->row0 + g->nrows : g->n_logits;
        li.n_logits = hi > g->row0 ? hi - g->row0 : 0;
      }
      gemm_kernel_name(*g, li.name, (int)sizeof li.name);
    } else {
      snprintf(li.name, sizeof li.name, "%s", name);
    }
    g_launch_events.start = tr->ev[2 * tr->n];
    g_launch_events.stop = tr->ev[2 * tr->n + 1];
    ++tr->n;
    return ok();
  };
#define QT_MARK(...)                    \
  do {                                  \
    qt_status m_ = mark(__VA_ARGS__);   \
    if (m_) return m_;                  \
  } while (0)

  FrameBeginArgs fb{};
  fb.mode = mode;
  fb.B = B;
  fb.Ht = T.hidden;
  fb.ncb = ncb;
  fb.n_kv = T.n_kv_heads;
  fb.capacity = capacity;
  fb.eps = T.rms_eps;
  fb.talker_in = (const uint16_t*)in->talker_in;
  fb.tok0_in = in->tok0_in;
  fb.kv_len = ss->kv_len;
  fb.x_t = x_t;
  fb.ss_t = ss_t;
  fb.gain = vp(m, m->plan.tl[0].in_norm);
  fb.u = ut;
  fb.h_in = (const uint16_t*)in->h_in;
  fb.cand = cand;
  fb.cand_ld = cand_ld;
  fb.counters = cnt;
  fb.status = out->status;
  // the one-launch predictor: greedy or teacher-forced frames of a supported model
  const bool pp = m->pred_persist && mode != QT_MODE_TALKER && !in->sampling && w.pp_ldm > 0;
  fb.pred_sync = pp ? (unsigned*)(ws + w.pp_sync) : nullptr;
  QT_MARK(QT_KERNEL_FRAME_BEGIN, "k_frame_begin", B, nullptr);
  QT_LAUNCH(launch_frame_begin(fb, st));

  // predictor matrices are read once per step: keep them in the caches
  bool keep_w = false;
  auto run = [&](GemmArgs& g) -> qt_status {
    g.keep_w = keep_w ? 1 : 0;
    QT_MARK(QT_KERNEL_GEMM, nullptr, g.M, &g);
    QT_LAUNCH(launch_gemm(g, st));
    return ok();
  };
  // A GEMM that writes residual / projection rows v also writes u = half(v * gain)
  // for the next RMSNorm and one sum-of-squares slot per row block; returns the
  // number of rows per block.
  auto produce = [&](GemmArgs& g, const uint16_t* gain, uint16_t* u, int u_ld, float* ss,
                     int ss_ld) -> int {
    g.u_gain = gain;
    g.u = u;
    g.u_ld = u_ld;
    g.ss_out = ss;
    g.ss_out_ld = ss_ld;
    return plan_gemm(g.nrows, g.K, g.M, g.w8 != 0, keep_w).rows_per_block;
  };

  // One decoder layer over M rows of residual x (row stride = hidden).  u: the
  // normalised-input buffer of the stack; ld: rows of the stack's chunked
  // activation buffers; ss / ss_ld: sums of squares of x; *slots: how many slots
  // the last producer of x left; next_gain: gain of the norm that follows the layer.
  auto layer = [&](const qt_decoder_cfg& d, const LayerSlots& L, float* x, uint16_t* u, int ld,
                   float* ss, int ss_ld, int* slots, const uint16_t* next_gain, int M,
                   auto&& attention) -> qt_status {
    qt_status r;
    GemmArgs g = gemm_norm(m, L.qkv, u, ld, ss, ss_ld, *slots, d.rms_eps, M, out->status);
    g.epi = EPI_STORE;
    g.out_f32 = qkv;
    g.out_ld = w.qkv_ld;
    if ((r = run(g))) return r;
    if ((r = attention())) return r;
    g = gemm_act(m, L.o, o, ld, M, out->status);
    g.epi = EPI_RESID;
    g.out_f32 = x;
    g.out_ld = d.hidden;
    *slots = d.hidden / produce(g, vp(m, L.post_norm), u, ld, ss, ss_ld);
    if ((r = run(g))) return r;
    g = gemm_norm(m, L.gu, u, ld, ss, ss_ld, *slots, d.rms_eps, M, out->status);
    g.epi = EPI_SWIGLU;
    g.u = ffn;
    g.u_ld = ld;
    if ((r = run(g))) return r;
    g = gemm_act(m, L.down, ffn, ld, M, out->status);
    g.epi = EPI_RESID;
    g.out_f32 = x;
    g.out_ld = d.hidden;
    *slots = d.hidden / produce(g, next_gain, u, ld, ss, ss_ld);
    return run(g);
  };
  int t_slots = 1, p_slots = 1;
  const int ss_t_ld = B, ss_p_ld = 2 * B;

  // predictor mode: the entry kernel copies h_in into ut (no lo part, no norm)
  GemmArgs head = gemm_act(m, m->plan.t_head, ut, ld_t, B, out->status);

  if (talker) {
    const AttnSplit split = attn_split(B, T.n_kv_heads, max_pages);
    const int pps = split.pps, n_splits = split.n_splits;
    const size_t layer_elems = (size_t)kv->num_pages * T.n_kv_heads * kPage * kHeadDim;
    for (int l = 0; l < T.layers; ++l) {
      cur_layer = l;
      const LayerSlots& L = m->plan.tl[l];
      const uint16_t* next_gain =
          vp(m, l + 1 < T.layers ? m->plan.tl[l + 1].in_norm : m->plan.t_final);
      qt_status s = layer(T, L, x_t, ut, ld_t, ss_t, ss_t_ld, &t_slots, next_gain, B,
                          [&]() -> qt_status {
        AttnPagedArgs a{};
        a.qkv = qkv;
        a.qkv_ld = w.qkv_ld;
        a.n_q = T.n_q_heads;
        a.n_kv = T.n_kv_heads;
        a.q_norm = vp(m, L.q_norm);
        a.k_norm = vp(m, L.k_norm);
        a.eps = T.rms_eps;
        a.k_pool = (uint16_t*)kv->k_pages + (size_t)l * layer_elems;
        a.v_pool = (uint16_t*)kv->v_pages + (size_t)l * layer_elems;
        a.num_pages = kv->num_pages;
        a.page_table = ss->page_table;
        a.max_pages = max_pages;
        a.kv_len = ss->kv_len;
        a.pages_per_split = pps;
        a.n_splits = n_splits;
        a.part = (float*)(ws + w.part);
        a.counters = cnt;
        a.o = o;
        a.o_ld = ld_t;
        a.status = out->status;
        QT_MARK(QT_KERNEL_ATTN_PAGED, "k_attn_paged", B, nullptr);
        QT_LAUNCH(launch_attn_paged(a, B, T.rope_theta, st));
        if (attn_merge_separate(B)) {
          QT_MARK(QT_KERNEL_ATTN_MERGE, "k_attn_merge", B, nullptr);
          QT_LAUNCH(launch_attn_merge(a, B, st));
        }
        return ok();
      });
      if (s) return s;
    }
    cur_layer = -1;
    head = gemm_norm(m, m->plan.t_head, ut, ld_t, ss_t, ss_t_ld, t_slots, T.rms_eps, B,
                     out->status);
    head.nrows = mode == QT_MODE_TALKER ? c.talker_vocab : c.talker_vocab + Pd.hidden;
  } else {
    // projection only, from the caller's bf16 post-norm Talker hidden state
    head.row0 = c.talker_vocab;
    head.nrows = Pd.hidden;
  }
  head.epi = EPI_HEAD;
  head.logits = out->logits0;
  head.logits_ld = c.talker_vocab;
  head.n_logits = c.talker_vocab;
  head.argmax_range = c.cb0_range;
  head.cand = cand;  // codebook 0: [B][cand_ld]
  head.cand_ld = cand_ld;
  head.out_f32 = x_p;  // projection rows land in predictor rows [0, B)
  head.out_ld = Pd.hidden;
  if (mode != QT_MODE_TALKER)
    p_slots = Pd.hidden / produce(head, vp(m, m->plan.pl[0].in_norm), up, ld_p, ss_p, ss_p_ld);
  {
    qt_status s = run(head);
    if (s) return s;
  }

  if (pp) {
    PredPersistArgs a{};
    a.B = B;
    a.layers = Pd.layers;
    a.n_steps = ncb - 1;
    a.ncb = ncb;
    a.ldm = w.pp_ldm;
    a.eps = Pd.rms_eps;
    a.theta_log2 = (float)log2((double)Pd.rope_theta);
    for (int l = 0; l < Pd.layers; ++l) {
      const LayerSlots& L = m->plan.pl[l];
      a.w_qkv[l] = m->base + L.qkv.w;
      a.w_o[l] = m->base + L.o.w;
      a.w_gu[l] = m->base + L.gu.w;
      a.w_dn[l] = m->base + L.down.w;
      if (m->i8) {
        a.s_qkv[l] = (const float*)(m->base + L.qkv.s);
        a.s_o[l] = (const float*)(m->base + L.o.s);
        a.s_gu[l] = (const float*)(m->base + L.gu.s);
        a.s_dn[l] = (const float*)(m->base + L.down.s);
      }
      a.g_in[l] = vp(m, L.in_norm);
      a.g_q[l] = vp(m, L.q_norm);
      a.g_k[l] = vp(m, L.k_norm);
      a.g_post[l] = vp(m, L.post_norm);
    }
    a.g_final = vp(m, m->plan.p_final);
    for (int k = 0; k < ncb - 1; ++k) {
      a.w_head[k] = m->base + m->plan.heads[k].w;
      a.s_head[k] = m->i8 ? (const float*)(m->base + m->plan.heads[k].s) : nullptr;
      a.embed[k] = vp(m, m->plan.embeds[k]);
    }
    a.x_p = x_p;
    a.cand = cand;
    a.cand_ld = cand_ld;
    a.forced = in->forced;
    a.logits = out->logits_pred;
    a.status = out->status;
    a.kc = (uint16_t*)(ws + w.pk);
    a.vc = (uint16_t*)(ws + w.pv);
    a.sess_stride = w.pk_sess;
    a.x_loc = (float*)(ws + w.pp_x);
    a.u_loc = (uint16_t*)(ws + w.pp_u);
    a.ss_loc = (float*)(ws + w.pp_ss);
    a.qkv_loc = (float*)(ws + w.pp_qkv);
    a.o_loc = (uint16_t*)(ws + w.pp_o);
    a.f_loc = (uint16_t*)(ws + w.pp_f);
    a.p_o = (float*)(ws + w.pp_po);
    a.p_d = (float*)(ws + w.pp_pd);
    a.sync = (unsigned*)(ws + w.pp_sync);
    cur_step = 1;
    cur_layer = -1;
    QT_MARK(QT_KERNEL_PREDICTOR, "k_pred_persist", B, nullptr);
    QT_LAUNCH(launch_pred_persist(a, st));
  } else if (mode != QT_MODE_TALKER) {
    keep_w = true;
    for (int k = 1; k < ncb; ++k) {
      const int M = (k == 1) ? 2 * B : B;
      const int emb_row = (k == 1) ? B : 0;
      EmbedArgs e{};
      e.B = B;
      e.H = Pd.hidden;
      e.vocab = c.code_vocab;
      e.ncb = ncb;
      e.step = k;
      e.eps = Pd.rms_eps;
      e.table = vp(m, m->plan.embeds[k - 1]);
      e.cand = cand;
      e.cand_ld = cand_ld;
      e.n_cand = key_blocks(k == 1 ? c.cb0_range : c.code_vocab);
      e.forced = in->forced;
      e.x = x_p;
      e.ss = ss_p;
      e.ss_ld = ss_p_ld;
      if (k > 1) p_slots = 1;  // rows [0, B) are all new
      e.ss_slots = p_slots;
      e.gain = vp(m, m->plan.pl[0].in_norm);
      e.u = up;
      e.u_ld = ld_p;
      e.row_off = emb_row;
      e.status = out->status;
      e.tokens = out->tokens;
      if (in->sampling && !(k == 1 && mode == QT_MODE_PREDICTOR)) {
        e.sample = 1;
        e.smp = sampler_args(c, *in->sampling);
        e.row = k == 1 ? SampleRow{out->logits0, c.talker_vocab, c.cb0_range, 0, 0}
                       : SampleRow{out->logits_pred + (size_t)(k - 2) * c.code_vocab,
                                   (long long)(ncb - 1) * c.code_vocab, c.code_vocab, 1, k - 1};
      }
      cur_step = k;
      cur_layer = -1;
      QT_MARK(QT_KERNEL_EMBED, "k_embed", B, nullptr);
      QT_LAUNCH(launch_embed(e, st));
      for (int l = 0; l < Pd.layers; ++l) {
        cur_layer = l;
        const LayerSlots& L = m->plan.pl[l];
        const uint16_t* next_gain =
            vp(m, l + 1 < Pd.layers ? m->plan.pl[l + 1].in_norm : m->plan.p_final);
        qt_status s = layer(Pd, L, x_p, up, ld_p, ss_p, ss_p_ld, &p_slots, next_gain, M,
                            [&]() -> qt_status {
          AttnPredArgs a{};
          a.qkv = qkv;
          a.qkv_ld = w.qkv_ld;
          a.n_q = Pd.n_q_heads;
          a.n_kv = Pd.n_kv_heads;
          a.B = B;
          a.q_norm = vp(m, L.q_norm);
          a.k_norm = vp(m, L.k_norm);
          a.eps = Pd.rms_eps;
          const size_t lay = (size_t)l * ncb * Pd.n_kv_heads * kHeadDim;
          a.k_cache = (uint16_t*)(ws + w.pk) + lay;
          a.v_cache = (uint16_t*)(ws + w.pv) + lay;
          a.sess_stride = w.pk_sess;
          a.pos0 = (k == 1) ? 0 : k;
          a.n_new = (k == 1) ? 2 : 1;
          a.o = o;
          a.o_ld = ld_p;
          a.status = out->status;
          QT_MARK(QT_KERNEL_ATTN_PRED, "k_attn_pred", B, nullptr);
          QT_LAUNCH(launch_attn_pred(a, Pd.rope_theta, st));
          return ok();
        });
        if (s) return s;
      }
      cur_layer = -1;
      // the step's head reads the last position: rows [emb_row, emb_row + B)
      GemmArgs g = gemm_norm(m, m->plan.heads[k - 1], up + (size_t)emb_row * 8, ld_p,
                             ss_p + emb_row, ss_p_ld, p_slots, Pd.rms_eps, B, out->status);
      g.epi = EPI_HEAD;
      g.logits = out->logits_pred + (size_t)(k - 1) * c.code_vocab;
      g.logits_ld = (ncb - 1) * c.code_vocab;
      g.n_logits = c.code_vocab;
      g.argmax_range = c.code_vocab;
      g.cand = cand + (size_t)k * B * cand_ld;
      g.cand_ld = cand_ld;
      qt_status s = run(g);
      if (s) return s;
    }
  }

  FrameEndArgs fe{};
  fe.mode = mode;
  fe.B = B;
  fe.ncb = ncb;
  fe.capacity = capacity;
  fe.cand = cand;
  fe.cand_ld = cand_ld;
  fe.n_cand0 = key_blocks(c.cb0_range);
  fe.n_cand = key_blocks(c.code_vocab);
  fe.tokens = out->tokens;
  fe.kv_len = ss->kv_len;
  fe.status = out->status;
  if (in->sampling) {
    fe.sample = 1;
    fe.smp = sampler_args(c, *in->sampling);
    fe.row = mode == QT_MODE_TALKER
                 ? SampleRow{out->logits0, c.talker_vocab, c.cb0_range, 0, 0}
                 : SampleRow{out->logits_pred + (size_t)(ncb - 2) * c.code_vocab,
                             (long long)(ncb - 1) * c.code_vocab, c.code_vocab, 1, ncb - 1};
  }
  cur_step = 0;
  cur_layer = -1;
  QT_MARK(QT_KERNEL_FRAME_END, "k_frame_end", B, nullptr);
  QT_LAUNCH(launch_frame_end(fe, st));
  return ok();
#undef QT_MARK
}

// Capture what `enqueue` puts on a fresh stream into an instantiated graph.
template <typename F>
qt_status capture_graph(qt_graph** out_graph, F&& enqueue) {
  hipStream_t cs;
  QT_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return fail(QT_E_HIP, "hipStreamBeginCapture failed: %s", hipGetErrorString(e));
  }
  qt_status st = enqueue(cs);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);
  if (st) {
    if (g) (void)hipGraphDestroy(g);
    return st;
  }
  if (e != hipSuccess) return fail(QT_E_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
  hipGraphExec_t ex;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(QT_E_HIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
  }
  qt_graph* gr = new qt_graph();
  gr->graph = g;
  gr->exec = ex;
  *out_graph = gr;
  return ok();
}

// ------------------------------------------------------------------ prompt prefill
struct PrefillWs {
  size_t x, ss, u, qkv, o, ffn, rowinfo, ul, ssl, cand, part, total;
  int qkv_ld, cand_ld;
};

// Key splits of the prefill attention: a 64-row tile's blocks of 32 keys are
// dealt over this many blocks (at 1024 rows the last tile's 32 key blocks become
// 16 per split).  Measured on 1 x 1024 and 4 x 256 prompts: 2 splits 7.84 / 7.23
// ms, 1 split 8.67 / 7.35, 4 splits 8.05 / 7.44, 8 splits 8.51 / 7.98 (with two
// key blocks in flight, longer loops cost less than more partials to merge).
constexpr int kPrefillSplits = 2;

PrefillWs make_prefill_ws(const qt_model_cfg& c, int R, int S) {
  const qt_decoder_cfg& t = c.talker;
  PrefillWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  w.qkv_ld = (t.n_q_heads + 2 * t.n_kv_heads) * t.head_dim;
  w.cand_ld = key_blocks(c.cb0_range);
  w.x = take((size_t)R * t.hidden * 4);
  w.ss = take((size_t)(t.hidden / kGemmRows) * R * 4);
  w.u = take((size_t)R * t.hidden * 2);
  w.qkv = take((size_t)R * w.qkv_ld * 4);
  w.o = take((size_t)R * t.n_q_heads * t.head_dim * 2);
  w.ffn = take((size_t)R * t.ffn * 2);
  w.rowinfo = take((size_t)R * 2 * 4);
  w.ul = take((size_t)S * t.hidden * 2);
  w.ssl = take((size_t)S * 4);
  w.cand = take((size_t)S * w.cand_ld * 8);
  w.part = take((size_t)R * t.n_q_heads * kPrefillSplits * (kHeadDim + 2) * 4);
  w.total = off;
  return w;
}

qt_status check_prefill_rows(int R, int S) {
  if (R < 16 || R > QT_PREFILL_MAX_ROWS || (R % 16) || (R > 64 && (R % 64)))
    return fail(QT_E_SHAPE, "rows = %d: expected a multiple of 16 (of 64 above 64), at most %d", R,
                QT_PREFILL_MAX_ROWS);
  if (S < 1 || S > QT_PREFILL_MAX_SEQS)
    return fail(QT_E_INVALID_ARG, "max_seqs = %d: expected 1..%d", S, QT_PREFILL_MAX_SEQS);
  return ok();
}

qt_status check_prefill_args(const qt_model* m, const qt_prefill_args* a, const qt_kv_caches* kv,
                             void* ws, uint64_t ws_bytes) {
  if (!m || !a || !kv) return fail(QT_E_INVALID_ARG, "model, args or kv is NULL");
  qt_status st = check_prefill_rows(a->rows, a->max_seqs);
  if (st) return st;
  if (!a->seq_start || !a->embeds || !a->page_table || !a->kv_len || !a->logits0 || !a->status)
    return fail(QT_E_INVALID_ARG, "a prefill array is NULL");
  if (a->max_pages < 1) return fail(QT_E_INVALID_ARG, "max_pages = %d", a->max_pages);
  if (!kv->k_pages || !kv->v_pages || kv->num_pages < 1)
    return fail(QT_E_INVALID_ARG, "kv pages are NULL or empty");
  if (((uintptr_t)kv->k_pages | (uintptr_t)kv->v_pages) & 15)
    return fail(QT_E_INVALID_ARG, "kv pages must be 16-byte aligned");
  if (!ws) return fail(QT_E_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)ws & (kAlign - 1)) return fail(QT_E_INVALID_ARG, "workspace must be 256-byte aligned");
  const PrefillWs w = make_prefill_ws(m->cfg, a->rows, a->max_seqs);
  if (ws_bytes < w.total)
    return fail(QT_E_CAPACITY, "workspace has %llu bytes, this prefill needs %llu",
                (unsigned long long)ws_bytes, (unsigned long long)w.total);
  return ok();
}

// Enqueue a prefill.  Per Talker layer: the four projections as many-row GEMMs
// over all rows, [q/k-norm, RoPE, K/V to pages] and [causal attention].
// Then the last row of each sequence: final norm, codec head, greedy token.
qt_status enqueue_prefill(const qt_model* m, const qt_prefill_args* a, const qt_kv_caches* kv,
                          void* wsp, hipStream_t st) {
  if (!m->prefill_refusal.empty())
    return fail(QT_E_UNSUPPORTED,
                "weight '%s' holds values beyond the IEEE half range (|w| > 65504): the prompt "
                "prefill runs on the unquantised weights as halves, also in INT8 mode",
                m->prefill_refusal.c_str());
  const qt_model_cfg& c = m->cfg;
  const qt_decoder_cfg& T = c.talker;
  const int R = a->rows, S = a->max_seqs;
  const PrefillWs w = make_prefill_ws(c, R, S);
  char* ws = (char*)wsp;
  float* x = (float*)(ws + w.x);
  float* ss = (float*)(ws + w.ss);
  uint16_t* u = (uint16_t*)(ws + w.u);
  float* qkv = (float*)(ws + w.qkv);
  uint16_t* o = (uint16_t*)(ws + w.o);
  uint16_t* ffn = (uint16_t*)(ws + w.ffn);
  int32_t* rowinfo = (int32_t*)(ws + w.rowinfo);

  PrefillBeginArgs b{};
  b.R = R;
  b.H = T.hidden;
  b.max_seqs = S;
  b.seq_start = a->seq_start;
  b.embeds = (const uint16_t*)a->embeds;
  b.gain = vp(m, m->plan.tl[0].in_norm);
  b.x = x;
  b.u = u;
  b.ss = ss;
  b.rowinfo = rowinfo;
  b.status = a->status;
  QT_LAUNCH(launch_prefill_begin(b, st));

  auto run = [&](GemmArgs& g) -> qt_status {
    QT_LAUNCH(launch_gemm_rows(g, st));
    return ok();
  };
  const size_t layer_elems = (size_t)kv->num_pages * T.n_kv_heads * kPage * kHeadDim;
  const int resid_slots = T.hidden / kGemmRows;  // one per 16 weight rows of a residual GEMM
  int slots = 1;
  for (int l = 0; l < T.layers; ++l) {
    const LayerSlots& L = m->plan.tl[l];
    const uint16_t* next_gain =
        vp(m, l + 1 < T.layers ? m->plan.tl[l + 1].in_norm : m->plan.t_final);
    qt_status r;
    GemmArgs g = gemm_norm(m, L.qkv, u, R, ss, R, slots, T.rms_eps, R, a->status, true);
    g.epi = EPI_STORE;
    g.out_f32 = qkv;
    g.out_ld = w.qkv_ld;
    PrefillQkArgs q{};
    q.qkv = qkv;
    q.R = R;
    q.qkv_ld = w.qkv_ld;
    q.n_q = T.n_q_heads;
    q.n_kv = T.n_kv_heads;
    q.q_norm = vp(m, L.q_norm);
    q.k_norm = vp(m, L.k_norm);
    q.eps = T.rms_eps;
    q.k_pool = (uint16_t*)kv->k_pages + (size_t)l * layer_elems;
    q.v_pool = (uint16_t*)kv->v_pages + (size_t)l * layer_elems;
    q.num_pages = kv->num_pages;
    q.page_table = a->page_table;
    q.max_pages = a->max_pages;
    q.rowinfo = rowinfo;
    q.status = a->status;
    bool qk_done = false;  // (the projection's epilogue does the q/k pass when it can)
    QT_LAUNCH(launch_gemm_rows(g, st, &q, T.rope_theta, &qk_done));
    if (!qk_done) QT_LAUNCH(launch_prefill_qk(q, R, T.rope_theta, st));
    PrefillAttnArgs at{};
    at.qkv = qkv;
    at.qkv_ld = w.qkv_ld;
    at.n_q = T.n_q_heads;
    at.n_kv = T.n_kv_heads;
    at.R = R;
    at.k_pool = q.k_pool;
    at.v_pool = q.v_pool;
    at.num_pages = kv->num_pages;
    at.page_table = a->page_table;
    at.max_pages = a->max_pages;
    at.rowinfo = rowinfo;
    at.o = o;
    at.part = (float*)(ws + w.part);
    at.n_splits = kPrefillSplits;
    at.status = a->status;
    QT_LAUNCH(launch_prefill_attn(at, st));
    g = gemm_act(m, L.o, o, R, R, a->status, true);
    g.epi = EPI_RESID;
    g.out_f32 = x;
    g.out_ld = T.hidden;
    g.u_gain = vp(m, L.post_norm);
    g.u = u;
    g.u_ld = R;
    g.ss_out = ss;
    g.ss_out_ld = R;
    if ((r = run(g))) return r;
    g = gemm_norm(m, L.gu, u, R, ss, R, resid_slots, T.rms_eps, R, a->status, true);
    g.epi = EPI_SWIGLU;
    g.u = ffn;
    g.u_ld = R;
    if ((r = run(g))) return r;
    g = gemm_act(m, L.down, ffn, R, R, a->status, true);
    g.epi = EPI_RESID;
    g.out_f32 = x;
    g.out_ld = T.hidden;
    g.u_gain = next_gain;
    g.u = u;
    g.u_ld = R;
    g.ss_out = ss;
    g.ss_out_ld = R;
    if ((r = run(g))) return r;
    slots = resid_slots;
  }

  PrefillLastArgs pl{};
  pl.max_seqs = S;
  pl.H = T.hidden;
  pl.R = R;
  pl.seq_start = a->seq_start;
  pl.x = x;
  pl.gain = vp(m, m->plan.t_final);
  pl.eps = T.rms_eps;
  pl.u = (uint16_t*)(ws + w.ul);
  pl.ss = (float*)(ws + w.ssl);
  pl.h_last = (uint16_t*)a->h_last;
  pl.kv_len = a->kv_len;
  pl.status = a->status;
  QT_LAUNCH(launch_prefill_last(pl, st));
  GemmArgs head =
      gemm_norm(m, m->plan.t_head, pl.u, S, pl.ss, S, 1, T.rms_eps, S, a->status, true);
  head.nrows = c.talker_vocab;
  head.epi = EPI_HEAD;
  head.logits = a->logits0;
  head.logits_ld = c.talker_vocab;
  head.n_logits = c.talker_vocab;
  head.argmax_range = c.cb0_range;
  head.cand = (unsigned long long*)(ws + w.cand);
  head.cand_ld = w.cand_ld;
  head.keep_w = 0;
  QT_LAUNCH(launch_gemm(head, st));
  if (a->tok0) {
    PrefillEndArgs pe{};
    pe.max_seqs = S;
    pe.cand_ld = w.cand_ld;
    pe.n_cand = key_blocks(c.cb0_range);
    pe.cand = head.cand;
    pe.tok0 = a->tok0;
    QT_LAUNCH(launch_prefill_end(pe, st));
  }
  return ok();
}

}  // namespace

namespace qt {
const qt_model_cfg* model_cfg(const qt_model* m) { return &m->cfg; }

qt_status report(qt_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
}  // namespace qt

// ------------------------------------------------------------------ allocation-free frames
// qt_frame_decode_noalloc runs the frame in this file-scope device array instead of
// a caller workspace.  Every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  In host code `scratch` only names a host-side
// stand-in: its device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is ever passed on.
constexpr size_t kNoallocScratchBytes = QT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

qt_status noalloc_scratch(void** out) {
  int dev = -1;
  QT_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QT_E_UNSUPPORTED, "device %d: the allocation-free frame supports devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QT_E_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                  hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return ok();
}
}  // namespace

// ------------------------------------------------------------------ exported
extern "C" {

const char* qt_last_error(void) { return g_err.c_str(); }

int32_t qt_abi_version(void) { return QT_ABI_VERSION; }

qt_status qt_validate_cfg(const qt_model_cfg* cfg) { return check_cfg(cfg); }

qt_status qt_packed_bytes(const qt_model_cfg* cfg, int32_t int8_mode, uint64_t* bytes) {
  qt_status st = check_cfg(cfg);
  if (st) return st;
  if (!bytes) return fail(QT_E_INVALID_ARG, "bytes is NULL");
  if (int8_mode != 0 && int8_mode != 1) return fail(QT_E_INVALID_ARG, "int8_mode must be 0 or 1");
  *bytes = make_plan(*cfg, int8_mode == 1).total;
  return ok();
}

qt_status qt_workspace_bytes(const qt_model_cfg* cfg, int32_t max_batch, int32_t max_pages,
                             uint64_t* bytes) {
  qt_status st = check_cfg(cfg);
  if (st) return st;
  if (!bytes) return fail(QT_E_INVALID_ARG, "bytes is NULL");
  if (max_batch < 1 || max_pages < 1)
    return fail(QT_E_INVALID_ARG, "max_batch and max_pages must be >= 1");
  if (max_batch > kMaxBatch)
    return fail(QT_E_UNSUPPORTED, "max_batch = %d: the library decodes at most %d sessions per call",
                max_batch, kMaxBatch);
  *bytes = make_ws(*cfg, max_batch, max_pages).total;
  return ok();
}

qt_status qt_load_weights(const qt_model_cfg* cfg, const qt_tensor* tensors, int32_t n_tensors,
                          int32_t int8_mode, void* packed, uint64_t packed_bytes, void* stream,
                          qt_model** out) {
  qt_status st = check_cfg(cfg);
  if (st) return st;
  if (!out) return fail(QT_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!tensors || n_tensors < 1) return fail(QT_E_INVALID_ARG, "tensors is NULL or empty");
  if (!packed) return fail(QT_E_INVALID_ARG, "packed buffer is NULL");
  if ((uintptr_t)packed & (kAlign - 1)) return fail(QT_E_INVALID_ARG, "packed buffer must be 256-byte aligned");
  if (int8_mode != 0 && int8_mode != 1) return fail(QT_E_INVALID_ARG, "int8_mode must be 0 or 1");
  const bool i8 = int8_mode == 1;
  Plan plan = make_plan(*cfg, i8);
  if (packed_bytes < plan.total)
    return fail(QT_E_CAPACITY, "packed buffer has %llu bytes, needs %llu",
                (unsigned long long)packed_bytes, (unsigned long long)plan.total);
  qt_model* m = new qt_model();
  m->cfg = *cfg;
  m->i8 = i8;
  m->plan = plan;
  m->dests = make_dests(*cfg, m->plan);
  m->base = (char*)packed;
  m->bytes = packed_bytes;
  // The one-launch predictor (qt_pred.hip) is chosen with QT_PREDICTOR=persistent in
  // the environment when the model is loaded; it needs its 256 blocks resident
  // together, one per CU of a 256-CU device.  By default the predictor runs as a
  // chain of launches, which measured faster (its barriers cost what the kernel
  // boundaries they replace cost, and it has more dependent stages).
  {
    int dev = 0, cus = 0;
    const char* env = getenv("QT_PREDICTOR");
    const bool persistent = env && strcmp(env, "persistent") == 0;
    m->pred_persist = 0;
    if (persistent && pred_persist_shapes(*cfg) && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus == kPredBlocks && prepare_pred_persist(cus) == hipSuccess)
      m->pred_persist = 1;
  }

  // coverage in both directions, shapes and dtypes, before any copy is enqueued
  std::map<std::string, const qt_tensor*> seen;
  for (int i = 0; i < n_tensors; ++i) {
    const qt_tensor& t = tensors[i];
    if (!t.name) {
      delete m;
      return fail(QT_E_INVALID_ARG, "tensor %d has no name", i);
    }
    auto it = m->dests.find(t.name);
    if (it == m->dests.end()) {
      delete m;
      return fail(QT_E_UNEXPECTED_TENSOR, "unexpected tensor '%s'", t.name);
    }
    if (seen.count(t.name)) {
      delete m;
      return fail(QT_E_UNEXPECTED_TENSOR, "tensor '%s' given twice", t.name);
    }
    seen[t.name] = &t;
    if (t.dtype != QT_BF16) {
      delete m;
      return fail(QT_E_DTYPE, "tensor '%s' has dtype %d, expected bf16", t.name, t.dtype);
    }
    if (t.rows != it->second.rows || t.cols != it->second.cols) {
      // (the expected shape lives in the model's table: read it before the model goes)
      const long long er = (long long)it->second.rows, ec = (long long)it->second.cols;
      delete m;
      return fail(QT_E_SHAPE, "tensor '%s' is [%lld, %lld], expected [%lld, %lld]", t.name,
                  (long long)t.rows, (long long)t.cols, er, ec);
    }
    if (!t.data) {
      delete m;
      return fail(QT_E_INVALID_ARG, "tensor '%s' has no data", t.name);
    }
  }
  for (const auto& kvp : m->dests) {
    if (!seen.count(kvp.first)) {
      std::string name = kvp.first;
      delete m;
      return fail(QT_E_MISSING_TENSOR, "missing tensor '%s'", name.c_str());
    }
  }

  hipStream_t s = (hipStream_t)stream;
  // bf16 mode packs the GEMM weights as IEEE half: one flag per source matrix records
  // a finite weight beyond the half range, read back once packing has finished
  uint32_t* range_flags = (uint32_t*)(m->base + m->plan.range_flags);
  std::vector<std::string> mat_names;
  {
    const hipError_t e = hipMemsetAsync(range_flags, 0, (size_t)m->plan.n_mats * 4, s);
    if (e != hipSuccess) {
      delete m;
      return fail(QT_E_HIP, "clearing the range flags failed: %s", hipGetErrorString(e));
    }
  }
  for (const auto& kvp : seen) {
    const Dest& d = m->dests[kvp.first];
    const qt_tensor& t = *kvp.second;
    hipError_t e = hipSuccess;
    if (d.kind == K_VEC || d.kind == K_EMBED) {
      e = hipMemcpyAsync(m->base + d.vec_off, t.data, (size_t)t.rows * t.cols * 2,
                         hipMemcpyDeviceToDevice, s);
    } else if (!i8) {
      if ((int)mat_names.size() >= m->plan.n_mats) {
        delete m;
        return fail(QT_E_STATE, "more GEMM weights than the plan counts");
      }
      e = launch_pack_tiled((const uint16_t*)t.data, (int)d.rows, (int)d.cols,
                            (uint16_t*)(m->base + d.mat->w), d.row0, d.step,
                            range_flags + mat_names.size(), s);
      mat_names.push_back(kvp.first);
    } else {
      float* sc = (float*)(m->base + d.mat->s) + d.row0;
      int8_t* q8 = d.mat->w8 ? (int8_t*)(m->base + d.mat->w) : nullptr;
      uint16_t* qh = d.mat->w8 ? nullptr : (uint16_t*)(m->base + d.mat->w);
      e = launch_quantize((const uint16_t*)t.data, d.rows, d.cols, q8, qh, d.step, sc, d.step,
                          (int)d.cols, d.row0, s);
      if (e == hipSuccess && d.mat->w8) {  // the prefill's half copy
        if ((int)mat_names.size() >= m->plan.n_mats) {
          delete m;
          return fail(QT_E_STATE, "more GEMM weights than the plan counts");
        }
        e = launch_pack_tiled((const uint16_t*)t.data, (int)d.rows, (int)d.cols,
                              (uint16_t*)(m->base + d.mat->wh), d.row0, d.step,
                              range_flags + mat_names.size(), s);
        mat_names.push_back(kvp.first);
      }
    }
    if (e != hipSuccess) {
      delete m;
      return fail(QT_E_HIP, "packing '%s' failed: %s", kvp.first.c_str(), hipGetErrorString(e));
    }
  }
  {
    std::vector<uint32_t> flags(mat_names.size(), 0u);
    hipError_t e = flags.empty() ? hipSuccess
                                 : hipMemcpyAsync(flags.data(), range_flags, flags.size() * 4,
                                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      delete m;
      return fail(QT_E_HIP, "reading the range flags failed: %s", hipGetErrorString(e));
    }
    for (size_t i = 0; i < flags.size(); ++i)
      if (flags[i]) {
        if (i8) {  // decoding takes it (every row scaled); the prompt prefill refuses
          if (m->prefill_refusal.empty()) m->prefill_refusal = mat_names[i];
          continue;
        }
        std::string name = mat_names[i];
        delete m;
        return fail(QT_E_UNSUPPORTED,
                    "weight '%s' holds values beyond the IEEE half range (|w| > 65504): the "
                    "GEMMs take half operands (INT8 mode scales every row and accepts it)",
                    name.c_str());
      }
  }
  *out = m;
  return ok();
}

qt_status qt_quantize_int8(const void* w_bf16, int64_t rows, int64_t cols, int8_t* q, float* scale,
                           void* stream) {
  if (!w_bf16 || !q || !scale) return fail(QT_E_INVALID_ARG, "a pointer is NULL");
  if (rows < 1 || cols < 1) return fail(QT_E_INVALID_ARG, "rows and cols must be >= 1");
  if (rows > 0x7fffffffLL) return fail(QT_E_SHAPE, "rows = %lld: at most 2^31-1", (long long)rows);
  QT_HIP(launch_quantize((const uint16_t*)w_bf16, rows, cols, q, nullptr, cols, scale, 1, 0, 0,
                         (hipStream_t)stream));
  return ok();
}

qt_status qt_model_export_int8(const qt_model* m, const char* name, int8_t* q, float* scale,
                               void* stream) {
  if (!m || !name || !q || !scale) return fail(QT_E_INVALID_ARG, "a pointer is NULL");
  if (!m->i8) return fail(QT_E_STATE, "model was loaded in bf16 mode");
  auto it = m->dests.find(name);
  if (it == m->dests.end() || it->second.kind != K_MAT)
    return fail(QT_E_INVALID_ARG, "'%s' is not a decode GEMM weight", name);
  const Dest& d = it->second;
  hipStream_t s = (hipStream_t)stream;
  QT_HIP(launch_untile_i8(m->base + d.mat->w, !d.mat->w8, (int)d.rows, (int)d.cols, d.row0,
                          d.step, q, s));
  QT_HIP(hipMemcpy2DAsync(scale, 4, m->base + d.mat->s + (size_t)d.row0 * 4, (size_t)4 * d.step, 4,
                          (size_t)d.rows, hipMemcpyDeviceToDevice, s));
  return ok();
}

qt_status qt_frame_decode(qt_model* model, const qt_sessions* sessions, const qt_kv_caches* kv,
                          const qt_frame_inputs* in, const qt_frame_outputs* out, void* workspace,
                          uint64_t workspace_bytes, void* stream) {
  qt_status st = check_frame_args(model, sessions, kv, in, out, workspace, workspace_bytes);
  if (st) return st;
  return enqueue_frame(model, sessions, kv, in, out, workspace, (hipStream_t)stream);
}

qt_status qt_frame_decode_noalloc(qt_model* model, const qt_sessions* sessions,
                                  const qt_kv_caches* kv, const qt_frame_inputs* in,
                                  const qt_frame_outputs* out, void* stream) {
  void* ws = nullptr;
  qt_status st = noalloc_scratch(&ws);
  if (st) return st;
  if (model && sessions && in && sessions->batch >= 1 && sessions->batch <= kMaxBatch &&
      in->mode >= QT_MODE_FULL && in->mode <= QT_MODE_PREDICTOR) {
    const int mp = in->mode != QT_MODE_PREDICTOR ? sessions->max_pages : 1;
    if (mp >= 1) {
      const size_t need = make_ws(model->cfg, sessions->batch, mp).total;
      if (need > kNoallocScratchBytes)
        return fail(QT_E_CAPACITY,
                    "qt_frame_decode_noalloc: %d sessions with %d-page tables need %llu bytes of "
                    "scratch; the library's static scratch holds %llu (qt_frame_decode takes a "
                    "caller workspace of any size)",
                    sessions->batch, mp, (unsigned long long)need,
                    (unsigned long long)kNoallocScratchBytes);
    }
  }
  st = check_frame_args(model, sessions, kv, in, out, ws, kNoallocScratchBytes);
  if (st) return st;
  return enqueue_frame(model, sessions, kv, in, out, ws, (hipStream_t)stream);
}

qt_status qt_frame_graph_create(qt_model* model, const qt_sessions* sessions, const qt_kv_caches* kv,
                                const qt_frame_inputs* in, const qt_frame_outputs* out,
                                void* workspace, uint64_t workspace_bytes, qt_graph** out_graph) {
  if (!out_graph) return fail(QT_E_INVALID_ARG, "out_graph is NULL");
  *out_graph = nullptr;
  qt_status st = check_frame_args(model, sessions, kv, in, out, workspace, workspace_bytes);
  if (st) return st;
  return capture_graph(out_graph, [&](hipStream_t cs) {
    return enqueue_frame(model, sessions, kv, in, out, workspace, cs);
  });
}


qt_status qt_sample(const float* logits, int32_t rows, int32_t ld, int32_t V,
                    const qt_sampler_params* params, const uint64_t* seed, const int32_t* counter,
                    int32_t codebook, uint32_t* seen, int32_t* tokens, uint32_t* status,
                    void* stream) {
  if (!logits || !params || !seed || !counter || !tokens || !status)
    return fail(QT_E_INVALID_ARG, "a qt_sample array is NULL");
  if (rows < 1 || V < 1 || ld < V) return fail(QT_E_INVALID_ARG, "rows = %d, V = %d, ld = %d", rows, V, ld);
  if (V > 4096) return fail(QT_E_UNSUPPORTED, "V = %d: draws cover at most 4096 entries", V);
  if (codebook < 0) return fail(QT_E_INVALID_ARG, "codebook = %d", codebook);
  SampleRowsArgs a{};
  a.rows = rows;
  a.V = V;
  a.ld = ld;
  a.codebook = codebook;
  a.seen_ld = (V + 31) / 32;
  a.logits = logits;
  a.params = params;
  a.seed = seed;
  a.counter = counter;
  a.seen = seen;
  a.tokens = tokens;
  a.status = status;
  QT_LAUNCH(launch_sample_rows(a, (hipStream_t)stream));
  return ok();
}

qt_status qt_prefill_workspace_bytes(const qt_model_cfg* cfg, int32_t rows, int32_t max_seqs,
                                     uint64_t* bytes) {
  qt_status st = check_cfg(cfg);
  if (st) return st;
  if (!bytes) return fail(QT_E_INVALID_ARG, "bytes is NULL");
  if ((st = check_prefill_rows(rows, max_seqs))) return st;
  *bytes = make_prefill_ws(*cfg, rows, max_seqs).total;
  return ok();
}

qt_status qt_prefill(qt_model* model, const qt_prefill_args* args, const qt_kv_caches* kv,
                     void* workspace, uint64_t workspace_bytes, void* stream) {
  qt_status st = check_prefill_args(model, args, kv, workspace, workspace_bytes);
  if (st) return st;
  return enqueue_prefill(model, args, kv, workspace, (hipStream_t)stream);
}

qt_status qt_prefill_graph_create(qt_model* model, const qt_prefill_args* args,
                                  const qt_kv_caches* kv, void* workspace,
                                  uint64_t workspace_bytes, qt_graph** out_graph) {
  if (!out_graph) return fail(QT_E_INVALID_ARG, "out_graph is NULL");
  *out_graph = nullptr;
  qt_status st = check_prefill_args(model, args, kv, workspace, workspace_bytes);
  if (st) return st;
  return capture_graph(out_graph, [&](hipStream_t cs) {
    return enqueue_prefill(model, args, kv, workspace, cs);
  });
}

qt_status qt_frame_graph_launch(qt_graph* graph, void* stream) {
  if (!graph) return fail(QT_E_INVALID_ARG, "graph is NULL");
  QT_HIP(hipGraphLaunch(graph->exec, (hipStream_t)stream));
  return ok();
}

void qt_graph_destroy(qt_graph* graph) {
  if (!graph) return;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
}

void qt_model_destroy(qt_model* model) { delete model; }

qt_status qt_trace_create(int32_t max_launches, qt_trace** out) {
  if (!out) return fail(QT_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(QT_E_INVALID_ARG, "max_launches = %d", max_launches);
  qt_trace* t = new qt_trace();
  t->info.resize(max_launches);
  for (int i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t e;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      qt_trace_destroy(t);
      return fail(QT_E_HIP, "hipEventCreate failed: %s", hipGetErrorString(r));
    }
    t->ev.push_back(e);
  }
  *out = t;
  return ok();
}

qt_status qt_frame_launch_count(const qt_model_cfg* cfg, int32_t mode, int32_t batch, int32_t* n) {
  qt_status st = check_cfg(cfg);
  if (st) return st;
  if (!n) return fail(QT_E_INVALID_ARG, "n is NULL");
  if (mode < QT_MODE_FULL || mode > QT_MODE_PREDICTOR)
    return fail(QT_E_INVALID_ARG, "mode = %d is not a qt_mode", mode);
  if (batch < 1 || batch > kMaxBatch)
    return fail(QT_E_INVALID_ARG, "batch = %d: expected 1..%d", batch, kMaxBatch);
  *n = frame_launches(*cfg, mode, batch);
  return ok();
}

qt_status qt_frame_trace(qt_model* model, const qt_sessions* sessions, const qt_kv_caches* kv,
                         const qt_frame_inputs* in, const qt_frame_outputs* out, void* workspace,
                         uint64_t workspace_bytes, void* stream, qt_trace* trace) {
  if (!trace) return fail(QT_E_INVALID_ARG, "trace is NULL");
  qt_status st = check_frame_args(model, sessions, kv, in, out, workspace, workspace_bytes);
  if (st) return st;
  const int need = frame_launches(model->cfg, in->mode, sessions->batch);
  if (need > (int)trace->info.size())
    return fail(QT_E_CAPACITY, "the frame makes %d launches, the trace holds %d", need,
                (int)trace->info.size());
  trace->n = -1;
  st = enqueue_frame(model, sessions, kv, in, out, workspace, (hipStream_t)stream, trace);
  if (st) trace->n = -1;
  return st;
}

qt_status qt_trace_read(qt_trace* trace, qt_launch_info* info, float* ms, int32_t max,
                        int32_t* n) {
  if (!trace || !info || !ms || !n) return fail(QT_E_INVALID_ARG, "a pointer is NULL");
  if (trace->n < 0) return fail(QT_E_STATE, "no frame has been traced");
  if (max < trace->n) return fail(QT_E_CAPACITY, "%d launches, room for %d", trace->n, max);
  if (trace->n > 0) QT_HIP(hipEventSynchronize(trace->ev[2 * trace->n - 1]));
  for (int i = 0; i < trace->n; ++i) {
    info[i] = trace->info[i];
    QT_HIP(hipEventElapsedTime(&ms[i], trace->ev[2 * i], trace->ev[2 * i + 1]));
  }
  *n = trace->n;
  return ok();
}

void qt_trace_destroy(qt_trace* trace) {
  if (!trace) return;
  for (hipEvent_t e : trace->ev) (void)hipEventDestroy(e);
  delete trace;
}

}  // extern "C"
