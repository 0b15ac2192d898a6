// Host lockstep scheduler around the decode frame: session table, page free list,
// grouping into captured batch sizes, and the per-group setup / graph replay /
// collect sequence.  The behaviour is specified in qt_sched.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "qt.h"
#include "qt_internal.h"
#include "qt_sched.h"

using namespace qt;

namespace {

constexpr size_t kAlign = 256;
constexpr int kRing = 64;  // step events kept; a step waits only for the one kRing back

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

#define SCHED_HIP(expr)                                                                \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return report(QT_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));          \
  } while (0)

// Byte offsets of the scheduler's part of the device buffer (Bm = largest bucket).
struct Layout {
  size_t ws, ws_bytes, kv_len, page_table, talker_in, forced, logits0, logits_pred, tokens,
      status, sess_pages, flags, res_l0, res_lp, res_tok, params, seed, seen, sess_seen, total;
  int seen_ld;
  size_t host_flags, host_pages, host_total;
};

qt_status check_sched_cfg(const qt_model_cfg* mc, const qt_sched_cfg* c) {
  if (!mc || !c) return report(QT_E_INVALID_ARG, "a configuration is NULL");
  qt_status st = qt_validate_cfg(mc);
  if (st) return st;
  if (c->n_buckets < 1 || c->n_buckets > QT_SCHED_MAX_BUCKETS)
    return report(QT_E_INVALID_ARG, "n_buckets = %d: expected 1..%d", c->n_buckets,
                  QT_SCHED_MAX_BUCKETS);
  for (int i = 0; i < c->n_buckets; ++i) {
    const int b = c->buckets[i];
    if (b < 1 || b > QT_SCHED_MAX_BATCH)
      return report(QT_E_INVALID_ARG, "buckets[%d] = %d: expected 1..%d", i, b, QT_SCHED_MAX_BATCH);
    if (i > 0 && b <= c->buckets[i - 1])
      return report(QT_E_INVALID_ARG, "buckets must be strictly ascending (buckets[%d] = %d)", i, b);
  }
  if (c->max_sessions < 1 || c->max_sessions > QT_SCHED_MAX_SESSIONS)
    return report(QT_E_INVALID_ARG, "max_sessions = %d: expected 1..%d", c->max_sessions,
                  QT_SCHED_MAX_SESSIONS);
  if (c->max_pages < 1) return report(QT_E_INVALID_ARG, "max_pages = %d", c->max_pages);
  if (c->eos_index < -1 || c->eos_index >= mc->talker_vocab)
    return report(QT_E_INVALID_ARG, "eos_index = %d: expected -1 or 0..%d", c->eos_index,
                  mc->talker_vocab - 1);
  return QT_OK;
}

qt_status make_layout(const qt_model_cfg& m, const qt_sched_cfg& c, Layout* L) {
  const int Bm = c.buckets[c.n_buckets - 1];
  const size_t S = (size_t)c.max_sessions, mp = (size_t)c.max_pages;
  const size_t pred = (size_t)(m.n_codebooks - 1) * m.code_vocab;
  uint64_t ws = 0;
  qt_status st = qt_workspace_bytes(&m, Bm, c.max_pages, &ws);
  if (st) return st;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L->ws_bytes = ws;
  L->ws = take(ws);
  L->kv_len = take((size_t)Bm * 4);
  L->page_table = take((size_t)Bm * mp * 4);
  L->talker_in = take((size_t)Bm * m.talker.hidden * 2);
  L->forced = take((size_t)Bm * m.n_codebooks * 4);
  L->logits0 = take((size_t)Bm * m.talker_vocab * 4);
  L->logits_pred = take((size_t)Bm * pred * 4);
  L->tokens = take((size_t)Bm * m.n_codebooks * 4);
  L->status = take(4);
  L->sess_pages = take(S * mp * 4);
  L->flags = take(S * 4);
  L->res_l0 = take(S * m.talker_vocab * 4);
  L->res_lp = take(S * pred * 4);
  L->res_tok = take(S * m.n_codebooks * 4);
  L->seen_ld = (m.cb0_range + 31) / 32;
  L->params = take((size_t)Bm * 2 * sizeof(qt_sampler_params));
  L->seed = take((size_t)Bm * 8);
  L->seen = take((size_t)Bm * L->seen_ld * 4);
  L->sess_seen = take(S * L->seen_ld * 4);
  L->total = off;
  L->host_flags = 0;
  L->host_pages = align_up(S * 4);
  L->host_total = L->host_pages + S * mp * 4;
  return QT_OK;
}

enum SessState { S_FREE = 0, S_OPEN = 1, S_RELEASING = 2 };

struct Session {
  int state = S_FREE;
  int length = 0;      // cached positions once every decoded frame has run
  int frames = 0;      // frames decoded (stepped)
  int min_frames = 1, max_frames = 1;
  bool queued = false;
  const void* in = nullptr;
  const int32_t* forced = nullptr;
  long long last_seq = 0;  // step that last decoded it (0: none)
  std::vector<int32_t> pages;
  bool sampling = false;
  qt_sampler_params params[2] = {};
  uint64_t seed = 0;
};

}  // namespace

struct qt_sched {
  qt_model* model;
  qt_model_cfg mc;
  qt_sched_cfg cfg;
  qt_kv_caches kv;
  Layout L;
  char* dev;
  int32_t* host_flags;      // host view of the pinned buffer
  int32_t* host_pages;
  int32_t* host_pages_dev;  // device view of the same memory
  int32_t* host_flags_dev;
  hipStream_t stream;
  int pad_page;
  qt_graph* graphs[QT_SCHED_MAX_BUCKETS][2][2];  // [bucket][forced][sampling]
  std::vector<Session> sess;
  std::vector<int32_t> free_pages;  // stack: popped from the back
  std::vector<int32_t> free_ids;
  hipEvent_t ev[kRing];
  long long seq_issued, seq_done;
};

namespace {

qt_status check_session(qt_sched* s, int32_t id) {
  if (!s) return report(QT_E_INVALID_ARG, "scheduler is NULL");
  if (id < 0 || id >= s->cfg.max_sessions)
    return report(QT_E_INVALID_ARG, "session %d out of range [0, %d)", id, s->cfg.max_sessions);
  if (s->sess[id].state != S_OPEN) return report(QT_E_STATE, "session %d is not open", id);
  return QT_OK;
}

// Pages go back in reverse so that the stack hands them out again in ascending
// order: a session's consecutive pages keep its attention reads local in HBM.
void release(qt_sched* s, int id) {
  Session& q = s->sess[id];
  for (auto it = q.pages.rbegin(); it != q.pages.rend(); ++it) s->free_pages.push_back(*it);
  q = Session();
  s->free_ids.push_back(id);
}

// Mark finished steps (events complete in step order on the one stream) and release
// the sessions closed since whose last frame has run.
void reap(qt_sched* s) {
  while (s->seq_done < s->seq_issued) {
    const long long next = s->seq_done + 1;
    if (hipEventQuery(s->ev[next % kRing]) != hipSuccess) break;
    s->seq_done = next;
  }
  for (int id = 0; id < s->cfg.max_sessions; ++id)
    if (s->sess[id].state == S_RELEASING && s->sess[id].last_seq <= s->seq_done) release(s, id);
}

int end_frame_of(const qt_sched* s, int id) {
  return __atomic_load_n(s->host_flags + id, __ATOMIC_ACQUIRE);
}

bool ended(const qt_sched* s, int id) {
  const Session& q = s->sess[id];
  return end_frame_of(s, id) > 0 || q.frames + (q.queued ? 1 : 0) >= q.max_frames;
}

qt_status plan_groups(const int32_t* cls, int n, const int32_t* buckets, int nb, int32_t* group_of,
                      int32_t* group_bucket, int32_t* n_groups) {
  const int bmax = buckets[nb - 1];
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cls[a] < cls[b]; });
  int g = 0;
  for (int i = 0; i < n;) {
    int j = i;
    while (j < n && cls[order[j]] == cls[order[i]]) ++j;
    // class [i, j): full groups of the largest size, then the remainder
    for (int k = i; k < j; k += bmax) {
      const int size = std::min(bmax, j - k);
      int b = 0;
      while (buckets[b] < size) ++b;
      for (int t = k; t < k + size; ++t) group_of[order[t]] = g;
      group_bucket[g++] = buckets[b];
    }
    i = j;
  }
  *n_groups = g;
  return QT_OK;
}

int bucket_index(const qt_sched* s, int size) {
  for (int i = 0; i < s->cfg.n_buckets; ++i)
    if (s->cfg.buckets[i] == size) return i;
  return -1;
}

// Capture (once) the frame of batch size buckets[bi], teacher-forced or not, drawing
// tokens or not, over the scheduler's batch tables.
qt_status ensure_graph(qt_sched* s, int bi, int forced, int sampled) {
  if (s->graphs[bi][forced][sampled]) return QT_OK;
  const Layout& L = s->L;
  qt_sessions ss{};
  ss.batch = s->cfg.buckets[bi];
  ss.kv_len = (int32_t*)(s->dev + L.kv_len);
  ss.page_table = (const int32_t*)(s->dev + L.page_table);
  ss.max_pages = s->cfg.max_pages;
  qt_frame_inputs in{};
  in.mode = QT_MODE_FULL;
  in.talker_in = s->dev + L.talker_in;
  in.forced = forced ? (const int32_t*)(s->dev + L.forced) : nullptr;
  qt_frame_outputs out{};
  out.logits0 = (float*)(s->dev + L.logits0);
  out.logits_pred = (float*)(s->dev + L.logits_pred);
  out.tokens = (int32_t*)(s->dev + L.tokens);
  out.status = (uint32_t*)(s->dev + L.status);
  qt_sampling smp{};
  if (sampled) {
    smp.params = (const qt_sampler_params*)(s->dev + L.params);
    smp.seed = (const uint64_t*)(s->dev + L.seed);
    smp.counter = ss.kv_len;  // each slot's cache length before the frame
    smp.seen0 = (uint32_t*)(s->dev + L.seen);
    in.sampling = &smp;
  }
  return qt_frame_graph_create(s->model, &ss, &s->kv, &in, &out, s->dev + L.ws, L.ws_bytes,
                               &s->graphs[bi][forced][sampled]);
}

bool params_ok(const qt_sampler_params& p) {
  return p.temperature > 0.f && p.temperature < INFINITY && p.top_p > 0.f && p.top_p <= 1.f &&
         p.repetition_penalty >= 1.f && p.repetition_penalty < INFINITY && p.top_k >= 1 &&
         p.top_k <= QT_SAMPLER_MAX_TOP_K;
}

}  // namespace

extern "C" {

qt_status qt_sched_bytes(const qt_model_cfg* model_cfg, const qt_sched_cfg* cfg,
                         uint64_t* device_bytes, uint64_t* host_bytes) {
  qt_status st = check_sched_cfg(model_cfg, cfg);
  if (st) return st;
  if (!device_bytes || !host_bytes) return report(QT_E_INVALID_ARG, "an output is NULL");
  Layout L;
  st = make_layout(*model_cfg, *cfg, &L);
  if (st) return st;
  *device_bytes = L.total;
  *host_bytes = L.host_total;
  return QT_OK;
}

qt_status qt_sched_create(qt_model* model, const qt_sched_cfg* cfg, const qt_kv_caches* kv,
                          void* device_buf, uint64_t device_bytes, void* host_buf,
                          uint64_t host_bytes, void* stream, qt_sched** out) {
  if (!out) return report(QT_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!model || !kv || !device_buf || !host_buf)
    return report(QT_E_INVALID_ARG, "model, kv, device_buf or host_buf is NULL");
  const qt_model_cfg& mc = *model_cfg(model);
  qt_status st = check_sched_cfg(&mc, cfg);
  if (st) return st;
  if (!kv->k_pages || !kv->v_pages) return report(QT_E_INVALID_ARG, "kv pages are NULL");
  if (kv->num_pages < 2)
    return report(QT_E_INVALID_ARG, "kv.num_pages = %d: expected >= 2 (one is the padding page)",
                  kv->num_pages);
  if ((uintptr_t)device_buf & (kAlign - 1))
    return report(QT_E_INVALID_ARG, "device_buf must be 256-byte aligned");
  if ((uintptr_t)host_buf & 15) return report(QT_E_INVALID_ARG, "host_buf must be 16-byte aligned");
  Layout L;
  st = make_layout(mc, *cfg, &L);
  if (st) return st;
  if (device_bytes < L.total || host_bytes < L.host_total)
    return report(QT_E_CAPACITY, "buffers of %llu / %llu bytes, the scheduler needs %llu / %llu",
                  (unsigned long long)device_bytes, (unsigned long long)host_bytes,
                  (unsigned long long)L.total, (unsigned long long)L.host_total);
  void* host_dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&host_dev, host_buf, 0);
  if (e != hipSuccess || !host_dev)
    return report(QT_E_INVALID_ARG, "host_buf is not pinned, device-mapped memory: %s",
                  hipGetErrorString(e));

  qt_sched* s = new qt_sched();
  s->model = model;
  s->mc = mc;
  s->cfg = *cfg;
  s->kv = *kv;
  s->L = L;
  s->dev = (char*)device_buf;
  s->host_flags = (int32_t*)((char*)host_buf + L.host_flags);
  s->host_pages = (int32_t*)((char*)host_buf + L.host_pages);
  s->host_flags_dev = (int32_t*)((char*)host_dev + L.host_flags);
  s->host_pages_dev = (int32_t*)((char*)host_dev + L.host_pages);
  s->stream = (hipStream_t)stream;
  s->pad_page = kv->num_pages - 1;
  memset(s->graphs, 0, sizeof s->graphs);
  s->sess.resize(cfg->max_sessions);
  for (int id = cfg->max_sessions - 1; id >= 0; --id) s->free_ids.push_back(id);
  for (int p = kv->num_pages - 2; p >= 0; --p) s->free_pages.push_back(p);
  s->seq_issued = s->seq_done = 0;
  int made = 0;
  for (; made < kRing; ++made)
    if (hipEventCreateWithFlags(&s->ev[made], hipEventDisableTiming) != hipSuccess) break;
  if (made < kRing) {
    for (int i = 0; i < made; ++i) (void)hipEventDestroy(s->ev[i]);
    delete s;
    return report(QT_E_HIP, "hipEventCreateWithFlags failed");
  }
  memset(host_buf, 0, L.host_total);
  e = hipMemsetAsync(s->dev + L.status, 0, 4, s->stream);
  if (e != hipSuccess) {
    for (int i = 0; i < kRing; ++i) (void)hipEventDestroy(s->ev[i]);
    delete s;
    return report(QT_E_HIP, "hipMemsetAsync failed: %s", hipGetErrorString(e));
  }
  *out = s;
  return QT_OK;
}

qt_status qt_sched_open(qt_sched* s, int32_t length, int32_t min_frames, int32_t max_frames,
                        int32_t* pages, int32_t* session) {
  if (!s || !session) return report(QT_E_INVALID_ARG, "scheduler or session is NULL");
  const int ps = s->mc.page_size;
  if (length < 0 || (long long)length >= (long long)s->cfg.max_pages * ps)
    return report(QT_E_INVALID_ARG, "length = %d: expected 0 <= length < %d", length,
                  s->cfg.max_pages * ps);
  if (min_frames < 1 || max_frames < 1)
    return report(QT_E_INVALID_ARG, "min_frames = %d, max_frames = %d: expected >= 1", min_frames,
                  max_frames);
  const int need = (length + ps - 1) / ps;
  if (need > 0 && !pages) return report(QT_E_INVALID_ARG, "pages is NULL");
  reap(s);
  if (s->free_ids.empty())
    return report(QT_E_CAPACITY, "%d sessions are open or still in flight", s->cfg.max_sessions);
  if ((int)s->free_pages.size() < need)
    return report(QT_E_CAPACITY, "%d pages needed, %d free", need, (int)s->free_pages.size());
  const int id = s->free_ids.back();
  s->free_ids.pop_back();
  Session& q = s->sess[id];
  q = Session();
  q.state = S_OPEN;
  q.length = length;
  q.min_frames = min_frames;
  q.max_frames = max_frames;
  int32_t* row = s->host_pages + (size_t)id * s->cfg.max_pages;
  for (int i = 0; i < need; ++i) {
    q.pages.push_back(s->free_pages.back());
    s->free_pages.pop_back();
    pages[i] = q.pages.back();
    row[i] = q.pages.back();
  }
  __atomic_store_n(s->host_flags + id, 0, __ATOMIC_RELEASE);
  *session = id;
  return QT_OK;
}

qt_status qt_sched_set_sampling(qt_sched* s, int32_t session, const qt_sampler_params* params,
                                uint64_t seed) {
  qt_status st = check_session(s, session);
  if (st) return st;
  Session& q = s->sess[session];
  if (!params) {
    q.sampling = false;
    return QT_OK;
  }
  for (int g = 0; g < 2; ++g)
    if (!params_ok(params[g]))
      return report(QT_E_INVALID_ARG,
                    "sampler params[%d] out of range (temperature > 0, 0 < top_p <= 1, penalty >= 1, "
                    "top_k 1..%d)", g, QT_SAMPLER_MAX_TOP_K);
  q.sampling = true;
  q.params[0] = params[0];
  q.params[1] = params[1];
  q.seed = seed;
  return QT_OK;
}

qt_status qt_sched_submit(qt_sched* s, int32_t session, const void* talker_in,
                          const int32_t* forced) {
  qt_status st = check_session(s, session);
  if (st) return st;
  if (!talker_in) return report(QT_E_INVALID_ARG, "talker_in is NULL");
  if ((uintptr_t)talker_in & 15) return report(QT_E_INVALID_ARG, "talker_in must be 16-byte aligned");
  Session& q = s->sess[session];
  if (q.queued) return report(QT_E_STATE, "session %d already has a frame queued", session);
  if (ended(s, session)) return report(QT_E_STATE, "session %d has ended", session);
  q.queued = true;
  q.in = talker_in;
  q.forced = forced;
  return QT_OK;
}

qt_status qt_sched_step(qt_sched* s, int32_t* n_groups) {
  if (!s) return report(QT_E_INVALID_ARG, "scheduler is NULL");
  if (n_groups) *n_groups = 0;
  reap(s);
  const int ps = s->mc.page_size, mp = s->cfg.max_pages;
  std::vector<int32_t> ready, cls;
  int new_pages = 0;
  for (int id = 0; id < s->cfg.max_sessions; ++id) {
    const Session& q = s->sess[id];
    if (q.state != S_OPEN || !q.queued) continue;
    if (q.length + 1 > mp * ps)
      return report(QT_E_CAPACITY, "session %d: %d positions fill its %d pages", id, q.length, mp);
    if (q.length == (int)q.pages.size() * ps) ++new_pages;
    ready.push_back(id);
    cls.push_back((q.frames == 0 ? 0 : 4) + (q.forced ? 2 : 0) + (q.sampling ? 1 : 0));
  }
  if (ready.empty()) return QT_OK;
  if (new_pages > (int)s->free_pages.size())
    return report(QT_E_CAPACITY, "%d new pages needed, %d free", new_pages,
                  (int)s->free_pages.size());
  const int n = (int)ready.size();
  std::vector<int32_t> group_of(n), group_bucket(n);
  int32_t ng = 0;
  plan_groups(cls.data(), n, s->cfg.buckets, s->cfg.n_buckets, group_of.data(),
              group_bucket.data(), &ng);
  for (int g = 0; g < ng; ++g) {
    int c = 0;
    for (int i = 0; i < n; ++i)
      if (group_of[i] == g) c = cls[i];
    qt_status st = ensure_graph(s, bucket_index(s, group_bucket[g]), (c >> 1) & 1, c & 1);
    if (st) return st;
  }

  // Every check has passed: the ring slot of this step must be free before work goes in.
  const long long seq = s->seq_issued + 1;
  if (seq - kRing > s->seq_done) {
    SCHED_HIP(hipEventSynchronize(s->ev[seq % kRing]));
    reap(s);
  }
  const Layout& L = s->L;
  for (int g = 0; g < ng; ++g) {
    const int B = group_bucket[g];
    SchedSetupArgs a{};
    a.B = B;
    a.H = s->mc.talker.hidden;
    a.ncb = s->mc.n_codebooks;
    a.max_pages = mp;
    a.pad_page = s->pad_page;
    a.host_pages = s->host_pages_dev;
    a.sess_pages = (int32_t*)(s->dev + L.sess_pages);
    a.kv_len = (int32_t*)(s->dev + L.kv_len);
    a.page_table = (int32_t*)(s->dev + L.page_table);
    a.talker_in = (uint16_t*)(s->dev + L.talker_in);
    a.flags = (int32_t*)(s->dev + L.flags);
    SchedCollectArgs c{};
    c.B = B;
    c.talker_vocab = s->mc.talker_vocab;
    c.cb0_range = s->mc.cb0_range;
    c.pred_elems = (s->mc.n_codebooks - 1) * s->mc.code_vocab;
    c.ncb = s->mc.n_codebooks;
    c.eos_index = s->cfg.eos_index;
    c.logits0 = (const float*)(s->dev + L.logits0);
    c.logits_pred = (const float*)(s->dev + L.logits_pred);
    c.tokens = (const int32_t*)(s->dev + L.tokens);
    c.res_logits0 = (float*)(s->dev + L.res_l0);
    c.res_pred = (float*)(s->dev + L.res_lp);
    c.res_tokens = (int32_t*)(s->dev + L.res_tok);
    c.flags = (int32_t*)(s->dev + L.flags);
    c.host_flags = s->host_flags_dev;
    for (int b = 0; b < B; ++b) {
      a.slot_session[b] = -1;
      a.slot_first[b] = -1;
      a.new_index[b] = -1;
      c.slot_session[b] = -1;
    }
    int forced = 0, sampled = 0, slot = 0;
    for (int i = 0; i < n; ++i) {
      if (group_of[i] != g) continue;
      const int id = ready[i];
      Session& q = s->sess[id];
      const int b = slot++;
      forced = (cls[i] >> 1) & 1;
      sampled = cls[i] & 1;
      a.slot_params[b][0] = q.params[0];
      a.slot_params[b][1] = q.params[1];
      a.slot_seed[b] = q.seed;
      a.slot_session[b] = id;
      a.slot_len[b] = q.length;
      a.slot_first[b] = q.frames == 0 ? (int)q.pages.size() : -1;
      if (q.length == (int)q.pages.size() * ps) {
        a.new_index[b] = (int)q.pages.size();
        a.new_page[b] = s->free_pages.back();
        s->free_pages.pop_back();
        q.pages.push_back(a.new_page[b]);
      }
      a.in_ptr[b] = (const uint16_t*)q.in;
      a.forced_ptr[b] = q.forced;
      c.slot_session[b] = id;
      const int frame = q.frames + 1;
      c.slot_check[b] = frame >= q.min_frames ? frame : 0;
    }
    a.forced = forced ? (int32_t*)(s->dev + L.forced) : nullptr;
    a.seen_ld = L.seen_ld;
    a.sess_seen = (uint32_t*)(s->dev + L.sess_seen);
    if (sampled) {
      a.params = (qt_sampler_params*)(s->dev + L.params);
      a.seed = (uint64_t*)(s->dev + L.seed);
      a.seen = (uint32_t*)(s->dev + L.seen);
    }
    c.sampled = sampled;
    c.seen = (const uint32_t*)(s->dev + L.seen);
    c.sess_seen = (uint32_t*)(s->dev + L.sess_seen);
    c.seen_ld = L.seen_ld;
    SCHED_HIP(launch_sched_setup(a, s->stream));
    qt_status st = qt_frame_graph_launch(s->graphs[bucket_index(s, B)][forced][sampled], s->stream);
    if (st) return st;
    SCHED_HIP(launch_sched_collect(c, s->stream));
  }
  SCHED_HIP(hipEventRecord(s->ev[seq % kRing], s->stream));
  s->seq_issued = seq;
  for (int i = 0; i < n; ++i) {
    Session& q = s->sess[ready[i]];
    q.length += 1;
    q.frames += 1;
    q.queued = false;
    q.in = nullptr;
    q.forced = nullptr;
    q.last_seq = seq;
  }
  if (n_groups) *n_groups = ng;
  return QT_OK;
}

qt_status qt_sched_outputs(qt_sched* s, int32_t session, const float** logits0,
                           const float** logits_pred, const int32_t** tokens, int32_t* frames) {
  qt_status st = check_session(s, session);
  if (st) return st;
  const Layout& L = s->L;
  const size_t pred = (size_t)(s->mc.n_codebooks - 1) * s->mc.code_vocab;
  if (logits0) *logits0 = (const float*)(s->dev + L.res_l0) + (size_t)session * s->mc.talker_vocab;
  if (logits_pred) *logits_pred = (const float*)(s->dev + L.res_lp) + (size_t)session * pred;
  if (tokens) *tokens = (const int32_t*)(s->dev + L.res_tok) + (size_t)session * s->mc.n_codebooks;
  if (frames) *frames = s->sess[session].frames;
  return QT_OK;
}

qt_status qt_sched_state(qt_sched* s, int32_t session, int32_t* state, int32_t* end_frame) {
  if (!s || !state) return report(QT_E_INVALID_ARG, "scheduler or state is NULL");
  if (session < 0 || session >= s->cfg.max_sessions)
    return report(QT_E_INVALID_ARG, "session %d out of range [0, %d)", session,
                  s->cfg.max_sessions);
  const Session& q = s->sess[session];
  int st = QT_SESSION_FREE, ef = 0;
  if (q.state == S_OPEN) {
    const int eos = end_frame_of(s, session);
    if (eos > 0) {
      st = QT_SESSION_ENDED_EOS;
      ef = eos;
    } else if (q.frames + (q.queued ? 1 : 0) >= q.max_frames) {
      st = QT_SESSION_ENDED_MAX;
      ef = q.max_frames;
    } else {
      st = QT_SESSION_RUNNING;
    }
  }
  *state = st;
  if (end_frame) *end_frame = ef;
  return QT_OK;
}

qt_status qt_sched_length(qt_sched* s, int32_t session, int32_t* length) {
  qt_status st = check_session(s, session);
  if (st) return st;
  if (!length) return report(QT_E_INVALID_ARG, "length is NULL");
  *length = s->sess[session].length;
  return QT_OK;
}

qt_status qt_sched_status_word(qt_sched* s, uint32_t** status) {
  if (!s || !status) return report(QT_E_INVALID_ARG, "scheduler or status is NULL");
  *status = (uint32_t*)(s->dev + s->L.status);
  return QT_OK;
}

qt_status qt_sched_free_pages(qt_sched* s, int32_t* n) {
  if (!s || !n) return report(QT_E_INVALID_ARG, "scheduler or n is NULL");
  reap(s);
  *n = (int32_t)s->free_pages.size();
  return QT_OK;
}

qt_status qt_sched_close(qt_sched* s, int32_t session) {
  qt_status st = check_session(s, session);
  if (st) return st;
  Session& q = s->sess[session];
  q.queued = false;
  q.state = S_RELEASING;
  reap(s);
  return QT_OK;
}

qt_status qt_sched_plan(const int32_t* cls, int32_t n, const int32_t* buckets, int32_t n_buckets,
                        int32_t* group_of, int32_t* group_bucket, int32_t* n_groups) {
  if (!buckets || !n_groups) return report(QT_E_INVALID_ARG, "buckets or n_groups is NULL");
  if (n < 0) return report(QT_E_INVALID_ARG, "n = %d", n);
  if (n > 0 && (!cls || !group_of || !group_bucket))
    return report(QT_E_INVALID_ARG, "cls, group_of or group_bucket is NULL");
  if (n_buckets < 1 || n_buckets > QT_SCHED_MAX_BUCKETS)
    return report(QT_E_INVALID_ARG, "n_buckets = %d", n_buckets);
  for (int i = 0; i < n_buckets; ++i)
    if (buckets[i] < 1 || buckets[i] > QT_SCHED_MAX_BATCH || (i > 0 && buckets[i] <= buckets[i - 1]))
      return report(QT_E_INVALID_ARG, "buckets must be strictly ascending in 1..%d",
                    QT_SCHED_MAX_BATCH);
  for (int i = 0; i < n; ++i)
    if (cls[i] < 0) return report(QT_E_INVALID_ARG, "cls[%d] = %d", i, cls[i]);
  return plan_groups(cls, n, buckets, n_buckets, group_of, group_bucket, n_groups);
}

void qt_sched_destroy(qt_sched* s) {
  if (!s) return;
  if (s->seq_issued > s->seq_done) (void)hipEventSynchronize(s->ev[s->seq_issued % kRing]);
  for (auto& row : s->graphs)
    for (auto& pair : row)
      for (qt_graph* g : pair) qt_graph_destroy(g);
  for (hipEvent_t e : s->ev) (void)hipEventDestroy(e);
  delete s;
}

}  // extern "C"
