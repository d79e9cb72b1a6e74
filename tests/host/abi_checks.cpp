// Host-side checks of libclefhead's C ABI with no GPU: batch validation and
// planning for valid batches (padded, varlen, fp16 flag) and every error
// code, the weight enumeration, the test hooks, and the failure paths of
// clef_head_create that return before or at the first device call.  Built
// with AddressSanitizer on the host code (tests/test_host_asan.py), so any
// out-of-bounds access, use after free or leak in these paths fails the run.
#include <cstdio>
#include <cstring>
#include <vector>

#include "clef_head.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond,        \
                  clef_head_last_error());                             \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

struct Batch {
  // two records of lengths 40 and 25 padded to 48; record 0: a noul and a choice(3)
  // question, record 1: a score(2) question
  std::vector<uint8_t> mask;
  std::vector<int32_t> cu{0, 40, 65}, qoff{0, 2, 3}, qtype{0, 1, 2}, qspan{2, 6, 10, 14, 3, 9};
  std::vector<int32_t> ooff{0, 2, 5, 7}, ospan{6, 8, 8, 10, 14, 16, 16, 19, 19, 22, 9, 11, 11, 12};
  std::vector<int32_t> ids;
  int dummy = 0;
  clef_head_batch b{};
  explicit Batch(int layout) {
    mask.assign(2 * 48, 0);
    for (int t = 0; t < 40; ++t) mask[t] = 1;
    for (int t = 0; t < 25; ++t) mask[48 + t] = 1;
    for (int k = 0; k < 7; ++k)
      for (int t = ospan[2 * k]; t < ospan[2 * k + 1]; ++t) ids.push_back((7 * t + k) % 100);
    b.layout = layout;
    b.num_records = 2;
    b.max_len = 48;
    b.hidden = &dummy;
    b.key_mask = mask.data();
    b.cu_seqlens = cu.data();
    b.num_questions = 3;
    b.num_options = 7;
    b.q_offsets = qoff.data();
    b.q_type = qtype.data();
    b.q_span = qspan.data();
    b.o_offsets = ooff.data();
    b.o_span = ospan.data();
    b.o_ids = ids.data();
  }
};

int main() {
  clef_head_config cfg{};
  cfg.hidden_size = 4096; cfg.width = 1024; cfg.heads = 16; cfg.routing_layers = 2; cfg.layers = 4;
  cfg.feedforward = 4096; cfg.vocab_size = 100; cfg.num_types = 3; cfg.ln_eps = 1e-5f;

  // weight enumeration, all variants
  for (int cross = 0; cross < 2; ++cross)
    for (int prec = 0; prec < 2; ++prec) {
      clef_head_config c = cfg;
      c.field_cross_attention = cross;
      c.precision = prec;
      const int32_t n = clef_head_weight_count(&c);
      EXPECT(n == 119 + (cross ? 4 * 10 : 0));   // 2 + 6 x 2 + 3 + 6 stacks x 16 + 4 + 2 (+ 4 x 10)
      char name[64];
      int64_t numel = 0;
      int32_t dt = 0;
      for (int i = 0; i < n; ++i) EXPECT(clef_head_weight_info(&c, i, name, sizeof name, &numel, &dt) == CLEF_OK);
      EXPECT(clef_head_weight_info(&c, n, name, sizeof name, &numel, &dt) == CLEF_E_ARG);
      EXPECT(clef_head_weight_info(&c, 0, name, 2, &numel, &dt) == CLEF_E_ARG);
    }
  {
    clef_head_config c = cfg;
    c.width = 512;
    EXPECT(clef_head_weight_count(&c) == -1);
    c = cfg;
    c.precision = 7;
    EXPECT(clef_head_weight_count(&c) == -1);
    EXPECT(clef_head_weight_count(nullptr) == -1);
  }

  // valid batches
  for (int layout : {CLEF_PADDED, CLEF_VARLEN, CLEF_PADDED | CLEF_HIDDEN_F16, CLEF_VARLEN | CLEF_HIDDEN_F16}) {
    Batch B(layout);
    int64_t rows = 0;
    EXPECT(clef_head_check_batch(&cfg, &B.b, &rows) == CLEF_OK);
    EXPECT(rows == 65);
    std::vector<int32_t> span((3 + 7 + 2) * 2, -1);
    EXPECT(clef_head_span_rows(&cfg, &B.b, span.data()) == CLEF_OK);
    EXPECT(span[0] == 2 && span[1] == 6 && span[2 * 2] == 40 + 3 && span[2 * 10] == 39 && span[2 * 11] == 64);
  }

  // every error code of the validation
  auto expect_code = [&](int code, void (*edit)(Batch&), int layout) {
    Batch B(layout);
    edit(B);
    EXPECT(clef_head_check_batch(&cfg, &B.b, nullptr) == code);
    EXPECT(std::strlen(clef_head_last_error()) > 0);
  };
  expect_code(CLEF_E_ARG, [](Batch& B) { B.b.q_offsets = nullptr; }, CLEF_PADDED);
  expect_code(CLEF_E_ARG, [](Batch& B) { B.b.hidden = nullptr; }, CLEF_PADDED);
  expect_code(CLEF_E_ARG, [](Batch& B) { B.b.key_mask = nullptr; }, CLEF_PADDED);
  expect_code(CLEF_E_ARG, [](Batch& B) { B.b.cu_seqlens = nullptr; }, CLEF_VARLEN);
  expect_code(CLEF_E_ARG, [](Batch& B) { B.b.layout = 5; }, CLEF_PADDED);
  expect_code(CLEF_E_ARG, [](Batch& B) { B.b.num_records = 0; }, CLEF_PADDED);
  expect_code(CLEF_E_LENGTH, [](Batch& B) { B.mask[45] = 1; }, CLEF_PADDED);
  expect_code(CLEF_E_LENGTH, [](Batch& B) { for (int t = 0; t < 48; ++t) B.mask[48 + t] = 0; }, CLEF_PADDED);
  expect_code(CLEF_E_LENGTH, [](Batch& B) { B.cu[2] = 40; }, CLEF_VARLEN);
  expect_code(CLEF_E_LENGTH, [](Batch& B) { B.cu[0] = 1; }, CLEF_VARLEN);
  expect_code(CLEF_E_SPAN, [](Batch& B) { B.qspan[1] = B.qspan[0]; }, CLEF_PADDED);
  expect_code(CLEF_E_SPAN, [](Batch& B) { B.qspan[5] = 26; }, CLEF_PADDED);
  expect_code(CLEF_E_SPAN, [](Batch& B) { B.ospan[0] = -1; }, CLEF_VARLEN);
  expect_code(CLEF_E_ID, [](Batch& B) { B.ids[3] = 100; }, CLEF_PADDED);
  expect_code(CLEF_E_ID, [](Batch& B) { B.ids.back() = -1; }, CLEF_VARLEN);
  expect_code(CLEF_E_SCHEMA, [](Batch& B) { B.qtype[1] = 3; }, CLEF_PADDED);
  expect_code(CLEF_E_SCHEMA, [](Batch& B) { B.qoff[2] = 2; }, CLEF_PADDED);
  expect_code(CLEF_E_SCHEMA, [](Batch& B) { B.ooff[1] = 3; B.ooff[2] = 5; }, CLEF_PADDED);   // noul with 3 options
  expect_code(CLEF_E_SCHEMA, [](Batch& B) { B.ooff[3] = 6; }, CLEF_PADDED);
  {
    // more options in one question than the per-question kernels hold
    Batch B(CLEF_VARLEN);
    B.cu = {0, 2000};
    B.b.num_records = 1;
    B.qoff = {0, 1};
    B.qtype = {1};
    B.qspan = {0, 1};
    B.ooff = {0, 1025};
    B.ospan.clear();
    B.ids.clear();
    for (int k = 0; k < 1025; ++k) {
      B.ospan.push_back(1 + k);
      B.ospan.push_back(2 + k);
      B.ids.push_back(k % 100);
    }
    B.b.cu_seqlens = B.cu.data();
    B.b.num_questions = 1;
    B.b.num_options = 1025;
    B.b.q_offsets = B.qoff.data();
    B.b.q_type = B.qtype.data();
    B.b.q_span = B.qspan.data();
    B.b.o_offsets = B.ooff.data();
    B.b.o_span = B.ospan.data();
    B.b.o_ids = B.ids.data();
    EXPECT(clef_head_check_batch(&cfg, &B.b, nullptr) == CLEF_E_UNSUPPORTED);
  }
  EXPECT(clef_head_check_batch(&cfg, nullptr, nullptr) == CLEF_E_ARG);
  {
    Batch B(CLEF_PADDED);
    EXPECT(clef_head_span_rows(&cfg, &B.b, nullptr) == CLEF_E_ARG);
  }

  // test hooks
  EXPECT(clef_head_debug_set(CLEF_DEBUG_ALLOC_LIMIT, -1) == CLEF_E_ARG);
  EXPECT(clef_head_debug_set(99, 0) == CLEF_E_ARG);
  EXPECT(clef_head_debug_set(CLEF_DEBUG_ALLOC_LIMIT, 0) == CLEF_OK);
  EXPECT(clef_head_debug_set(CLEF_DEBUG_POISON, 0) == CLEF_OK);

  // create: argument errors, then a valid call that fails at the device (no GPU here)
  clef_head* h = reinterpret_cast<clef_head*>(&cfg);
  int table = 0;
  EXPECT(clef_head_create(&cfg, nullptr, 0, &table, nullptr) == CLEF_E_ARG);
  EXPECT(clef_head_create(nullptr, nullptr, 0, &table, &h) == CLEF_E_ARG && h == nullptr);
  {
    clef_head_config c = cfg;
    c.heads = 8;
    EXPECT(clef_head_create(&c, nullptr, 0, &table, &h) == CLEF_E_UNSUPPORTED && h == nullptr);
  }
  EXPECT(clef_head_create(&cfg, nullptr, 0, nullptr, &h) == CLEF_E_ARG && h == nullptr);
  const int rc = clef_head_create(&cfg, nullptr, 0, &table, &h);
  EXPECT((rc == CLEF_E_HIP || rc == CLEF_E_ARG) && h == nullptr);
  clef_head_destroy(nullptr);
  EXPECT(clef_head_forward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == CLEF_E_ARG);
  EXPECT(clef_head_stream_cancel(nullptr) == CLEF_E_ARG);

  std::printf("%s: %d failures\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}
