// Drives the host-side code of libqt (configuration checks, buffer sizing, weight-
// table validation, the scheduler's grouping rule, argument errors) without a GPU,
// for the address / undefined-behaviour sanitizer build of the tests.  Every call
// here returns before anything is enqueued.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "qt.h"
#include "qt_sched.h"

#define EXPECT(c)                                               \
  do {                                                          \
    if (!(c)) {                                                 \
      fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__);  \
      exit(1);                                                  \
    }                                                           \
  } while (0)

static qt_model_cfg full_cfg() {
  qt_model_cfg c;
  memset(&c, 0, sizeof c);
  c.talker = qt_decoder_cfg{28, 2048, 16, 8, 128, 6144, 1e6f, 1e-6f};
  c.predictor = qt_decoder_cfg{5, 1024, 16, 8, 128, 3072, 1e6f, 1e-6f};
  c.talker_vocab = 3072;
  c.code_vocab = 2048;
  c.cb0_range = 2048;
  c.n_codebooks = 16;
  c.page_size = 16;
  return c;
}

int main() {
  qt_model_cfg c = full_cfg();
  EXPECT(qt_validate_cfg(&c) == QT_OK);
  EXPECT(qt_validate_cfg(nullptr) == QT_E_INVALID_ARG);
  qt_model_cfg bad = c;
  bad.talker.head_dim = 64;
  EXPECT(qt_validate_cfg(&bad) == QT_E_SHAPE);
  EXPECT(strlen(qt_last_error()) > 0);
  bad = c;
  bad.n_codebooks = 17;
  EXPECT(qt_validate_cfg(&bad) == QT_E_SHAPE);

  uint64_t bytes = 0, b8 = 0, ws1 = 0, ws32 = 0;
  EXPECT(qt_packed_bytes(&c, 0, &bytes) == QT_OK && bytes > 0);
  // (INT8 mode holds the int8 decode weights and, for the prompt prefill, a half copy)
  EXPECT(qt_packed_bytes(&c, 1, &b8) == QT_OK && b8 > bytes);
  EXPECT(qt_packed_bytes(&c, 2, &b8) == QT_E_INVALID_ARG);
  EXPECT(qt_workspace_bytes(&c, 1, 130, &ws1) == QT_OK);
  EXPECT(qt_workspace_bytes(&c, 32, 130, &ws32) == QT_OK && ws32 > ws1);
  EXPECT(qt_workspace_bytes(&c, 33, 130, &ws32) == QT_E_UNSUPPORTED);
  for (int rows = 16; rows <= 4096; rows *= 2) {
    uint64_t pf = 0;
    EXPECT(qt_prefill_workspace_bytes(&c, rows, 4, &pf) == QT_OK && pf > 0);
  }
  uint64_t pf = 0;
  EXPECT(qt_prefill_workspace_bytes(&c, 100, 4, &pf) == QT_E_SHAPE);
  int32_t n = 0;
  EXPECT(qt_frame_launch_count(&c, QT_MODE_FULL, 1, &n) == QT_OK && n == 548);
  EXPECT(qt_frame_launch_count(&c, QT_MODE_FULL, 32, &n) == QT_OK && n == 576);
  EXPECT(qt_frame_launch_count(&c, QT_MODE_FULL, 33, &n) == QT_E_INVALID_ARG);

  // weight table: a missing tensor, an unknown name and a wrong shape are refused
  // before any device work (the data pointers are never dereferenced)
  std::vector<qt_tensor> t;
  std::vector<std::string> names;
  char dummy[16];
  names.push_back("talker.layers.0.q_proj");
  names.push_back("no.such.weight");
  for (auto& s : names) t.push_back(qt_tensor{s.c_str(), dummy, QT_BF16, 2048, 2048});
  qt_model* m = nullptr;
  alignas(256) static char packed[256];
  EXPECT(qt_load_weights(&c, t.data(), 1, 0, packed, sizeof packed, nullptr, &m) == QT_E_CAPACITY);
  EXPECT(qt_load_weights(&c, t.data(), 2, 0, (void*)0x100000, bytes, nullptr, &m) ==
         QT_E_UNEXPECTED_TENSOR);
  EXPECT(m == nullptr);
  EXPECT(qt_load_weights(&c, t.data(), 1, 0, (void*)0x100000, bytes, nullptr, &m) ==
         QT_E_MISSING_TENSOR);
  t[0].rows = 7;
  EXPECT(qt_load_weights(&c, t.data(), 1, 0, (void*)0x100000, bytes, nullptr, &m) == QT_E_SHAPE);

  // frame calls with missing descriptors
  EXPECT(qt_frame_decode(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
         QT_E_INVALID_ARG);
  EXPECT(qt_frame_decode_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != QT_OK);
  EXPECT(qt_sample(nullptr, 1, 1, 1, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr,
                   nullptr) == QT_E_INVALID_ARG);

  // scheduler sizing and grouping
  qt_sched_cfg sc;
  memset(&sc, 0, sizeof sc);
  sc.n_buckets = 3;
  sc.buckets[0] = 1;
  sc.buckets[1] = 4;
  sc.buckets[2] = 32;
  sc.max_sessions = 64;
  sc.max_pages = 130;
  sc.eos_index = -1;
  uint64_t db = 0, hb = 0;
  EXPECT(qt_sched_bytes(&c, &sc, &db, &hb) == QT_OK && db > 0 && hb > 0);
  sc.buckets[1] = 1;  // not ascending
  EXPECT(qt_sched_bytes(&c, &sc, &db, &hb) != QT_OK);
  const int32_t buckets[3] = {1, 4, 32};
  for (int ready = 0; ready <= 80; ++ready) {
    std::vector<int32_t> cls(ready), group_of(ready > 0 ? ready : 1), group_bucket(ready > 0 ? ready : 1);
    for (int i = 0; i < ready; ++i) cls[i] = (i * 7) % 3;
    int32_t ng = -1;
    EXPECT(qt_sched_plan(cls.data(), ready, buckets, 3, group_of.data(), group_bucket.data(), &ng) ==
           QT_OK);
    int32_t seats = 0;
    for (int g = 0; g < ng; ++g) seats += group_bucket[g];
    EXPECT(seats >= ready);
    for (int i = 0; i < ready; ++i) EXPECT(group_of[i] >= 0 && group_of[i] < ng);
  }
  EXPECT(qt_sched_plan(nullptr, 3, buckets, 3, nullptr, nullptr, nullptr) != QT_OK);
  printf("abi driver ok\n");
  return 0;
}
