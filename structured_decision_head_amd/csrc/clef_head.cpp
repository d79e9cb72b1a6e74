// libclefhead host side: the C ABI, input validation, batch planning (packed
// tables for the kernels), weight repacking, workspace management and the
// launch sequence of the JointSchemaHead forward pass.
//
// Steps (clef-4bit page §三 steps 1-4; CoreML conversion metadata of
// clef-flash, "decision.head" and "softmax"):
//   1. LayerNorm statistics of every valid hidden row; span means of the
//      LayerNorm-ed rows (questions, option contexts) and the last row
//      (global); lexical gather-mean of lm_head rows and the cosine prior.
//   2. memory = W_m LayerNorm(hidden) + b_m; per routing layer K, V of memory.
//   3. option queries u = W_c c + W_l e + W_qo q (+ biases); 2 routing layers
//      (pre-LN cross-attention over the record's memory + pre-LN GELU FFN).
//   4. field vectors (question base + option-weighted summary + global +
//      type embedding); 4 pre-LN self-attention + FFN layers across fields.
//   5. logits = prior + sigmoid(gate) (joint_scale cos(u, f) + MLP[f, u, f*u,
//      |f-u|]); softmax and argmax per question.
#include "clef_head.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <type_traits>
#include <unordered_map>
#include <vector>

#include "kernels.hpp"

using namespace clef;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// Test hooks (clef_head_debug_set): a cap on every single device or pinned
// allocation, and NaN-poisoning of newly allocated working memory.
std::atomic<int64_t> g_alloc_limit{0};
std::atomic<int> g_poison{0};

bool over_limit(size_t bytes) {
  const int64_t lim = g_alloc_limit.load();
  return lim > 0 && (int64_t)bytes > lim;
}

hipError_t dev_malloc(void** p, size_t bytes) {
  *p = nullptr;
  if (over_limit(bytes)) return hipErrorOutOfMemory;
  return hipMalloc(p, bytes);
}

hipError_t pinned_malloc(void** p, size_t bytes) {
  *p = nullptr;
  if (over_limit(bytes)) return hipErrorOutOfMemory;
  return hipHostMalloc(p, bytes, hipHostMallocDefault);
}

#define HIPCHK(x)                                                                              \
  do {                                                                                         \
    hipError_t e_ = (x);                                                                       \
    if (e_ != hipSuccess) return fail(CLEF_E_HIP, "%s failed: %s", #x, hipGetErrorString(e_)); \
  } while (0)

constexpr int D = 1024, F = 4096, NH = 16;
constexpr int TILE = 256;     // row tile of the packed row space
// Routing attention splits each record's keys into chunks, one wave per
// (record, head, chunk, 32-query block).  The chunk is the largest power of
// two from 128 to 1024 keys that still yields kAttnMinWaves waves: longer
// chunks mean fewer flash-decode partials to write and merge, which matters
// when a record has many query blocks; beyond 1024 keys the longest records'
// waves form a tail.
constexpr int kAttnMinWaves = 1024;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

float bf16_to_f(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t f_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// configuration and weight names
// ---------------------------------------------------------------------------
struct WSpec {
  std::string name;
  int64_t numel;
  int32_t dtype;
};

std::vector<WSpec> weight_list(const clef_head_config& c) {
  const int64_t H = c.hidden_size, d = c.width, f = c.feedforward;
  std::vector<WSpec> s;
  auto add = [&](const std::string& n, int64_t numel, int32_t dt = CLEF_BF16) { s.push_back({n, numel, dt}); };
  add("ln_in.w", H);
  add("ln_in.b", H);
  for (const char* n : {"mem", "q_base", "q_opt", "opt_ctx", "opt_lex", "glob"}) {
    add(std::string(n) + ".w", d * H);
    add(std::string(n) + ".b", d);
  }
  add("type_emb", int64_t(c.num_types) * d);
  add("summary.w", d);
  add("summary.b", 1);
  std::vector<std::string> stacks;
  for (int r = 0; r < c.routing_layers; ++r) stacks.push_back("route." + std::to_string(r));
  for (int l = 0; l < c.layers; ++l) stacks.push_back("field." + std::to_string(l));
  for (auto& p : stacks) {
    add(p + ".ln1.w", d);
    add(p + ".ln1.b", d);
    for (const char* m : {"q", "k", "v", "o"}) {
      add(p + "." + m + ".w", d * d);
      add(p + "." + m + ".b", d);
    }
    add(p + ".ln2.w", d);
    add(p + ".ln2.b", d);
    add(p + ".ffn1.w", f * d);
    add(p + ".ffn1.b", f);
    add(p + ".ffn2.w", d * f);
    add(p + ".ffn2.b", d);
  }
  add("score.w1", d * 4 * d);
  add("score.b1", d);
  add("score.w2", d);
  add("score.b2", 1);
  add("gate_logit", 1, CLEF_F32);
  add("joint_scale", 1, CLEF_F32);
  if (c.field_cross_attention)   // decoder-layer field variant: appended after everything else
    for (int l = 0; l < c.layers; ++l) {
      const std::string p = "field." + std::to_string(l);
      add(p + ".xln.w", d);
      add(p + ".xln.b", d);
      for (const char* m : {"xq", "xk", "xv", "xo"}) {
        add(p + "." + m + ".w", d * d);
        add(p + "." + m + ".b", d);
      }
    }
  return s;
}

int check_config(const clef_head_config* c) {
  if (!c) return fail(CLEF_E_ARG, "config is NULL");
  if (c->hidden_size <= 0 || c->width <= 0 || c->heads <= 0 || c->feedforward <= 0 || c->vocab_size <= 0 ||
      c->num_types <= 0 || c->routing_layers < 0 || c->layers < 0 || !(c->ln_eps > 0.f))
    return fail(CLEF_E_ARG, "config has a non-positive size or epsilon");
  if (c->field_cross_attention != 0 && c->field_cross_attention != 1)
    return fail(CLEF_E_ARG, "field_cross_attention must be 0 or 1 (got %d)", c->field_cross_attention);
  if (c->precision != CLEF_PRECISION_BF16 && c->precision != CLEF_PRECISION_F32)
    return fail(CLEF_E_ARG, "precision must be CLEF_PRECISION_BF16 or CLEF_PRECISION_F32 (got %d)", c->precision);
  if (c->width != D || c->heads != NH || c->feedforward != F)
    return fail(CLEF_E_UNSUPPORTED, "kernels are built for width 1024, 16 heads, feedforward 4096 (got %d, %d, %d)",
                c->width, c->heads, c->feedforward);
  if (c->hidden_size % 512 != 0 || c->hidden_size > 8192)
    return fail(CLEF_E_UNSUPPORTED, "hidden_size must be a multiple of 512 up to 8192 (got %d)", c->hidden_size);
  if (c->num_types < 3) return fail(CLEF_E_ARG, "num_types must cover noul, choice and score (>= 3)");
  if (c->routing_layers > 64 || c->layers > 64) return fail(CLEF_E_UNSUPPORTED, "more than 64 layers in a stack");
  return CLEF_OK;
}

// ---------------------------------------------------------------------------
// batch plan
// ---------------------------------------------------------------------------
struct Plan {
  int B = 0, NQ = 0, NO = 0, nact = 0;
  int64_t T = 0, Tpad = 0, Ptot = 0, nids = 0;
  int ntiles = 0, npool = 0, nitems = 0, kchunk = 128;
  bool f16 = false;           // hidden rows are fp16 (CLEF_HIDDEN_F16), else bf16
  std::vector<int32_t> tab;   // all int32 tables, back to back
  size_t off_rec = 0, off_tiles = 0, off_kvtiles = 0, off_pool = 0, off_lex = 0, off_ids = 0, off_optq = 0,
         off_optrec = 0, off_qrec = 0, off_qtype = 0, off_ooff = 0, off_items = 0;
  // decoder-layer field variant: cross-attention work of the fields over the memory rows
  int64_t Ptot_f = 0;
  int nfitems = 0;
  size_t off_frec = 0, off_fitems = 0;
  std::vector<int32_t> span_rows;   // [NQ + NO + B][2] packed-row ranges (for clef_head_span_rows)
};

int build_plan(const clef_head_config& c, const clef_head_batch* b, Plan& p, bool tables) {
  if (!b) return fail(CLEF_E_ARG, "batch is NULL");
  const int layout = b->layout & ~CLEF_HIDDEN_F16;
  if (layout != CLEF_PADDED && layout != CLEF_VARLEN) return fail(CLEF_E_ARG, "unknown layout %d", b->layout);
  p.f16 = (b->layout & CLEF_HIDDEN_F16) != 0;
  const int B = b->num_records;
  if (B < 1) return fail(CLEF_E_ARG, "num_records must be >= 1");
  if (b->num_questions < 0 || b->num_options < 0) return fail(CLEF_E_ARG, "negative question / option count");
  if (!b->q_offsets) return fail(CLEF_E_ARG, "q_offsets is NULL");
  const int NQ = b->num_questions, NO = b->num_options;
  if (NQ > 0 && (!b->q_type || !b->q_span || !b->o_offsets)) return fail(CLEF_E_ARG, "question tables are NULL");
  if (NO > 0 && (!b->o_span || !b->o_ids)) return fail(CLEF_E_ARG, "option tables are NULL");

  // record lengths and first hidden rows
  std::vector<int64_t> len(B), src0(B);
  if (layout == CLEF_PADDED) {
    if (b->max_len < 1) return fail(CLEF_E_LENGTH, "max_len must be >= 1");
    if (!b->key_mask) return fail(CLEF_E_ARG, "key_mask is NULL");
    for (int r = 0; r < B; ++r) {
      const uint8_t* m = b->key_mask + (size_t)r * b->max_len;
      int n = 0;
      while (n < b->max_len && m[n]) ++n;
      for (int t = n; t < b->max_len; ++t)
        if (m[t]) return fail(CLEF_E_LENGTH, "key_mask row %d is not a prefix mask", r);
      if (n < 1) return fail(CLEF_E_LENGTH, "record %d has no valid token", r);
      len[r] = n;
      src0[r] = (int64_t)r * b->max_len;
    }
  } else {
    if (!b->cu_seqlens) return fail(CLEF_E_ARG, "cu_seqlens is NULL");
    if (b->cu_seqlens[0] != 0) return fail(CLEF_E_LENGTH, "cu_seqlens[0] must be 0");
    for (int r = 0; r < B; ++r) {
      const int64_t n = (int64_t)b->cu_seqlens[r + 1] - b->cu_seqlens[r];
      if (n < 1) return fail(CLEF_E_LENGTH, "record %d has length %lld", r, (long long)n);
      len[r] = n;
      src0[r] = b->cu_seqlens[r];
    }
  }
  if (!b->hidden) return fail(CLEF_E_ARG, "hidden is NULL");

  // questions and options
  if (b->q_offsets[0] != 0 || b->q_offsets[B] != NQ)
    return fail(CLEF_E_SCHEMA, "q_offsets must start at 0 and end at num_questions");
  for (int r = 0; r < B; ++r)
    if (b->q_offsets[r + 1] < b->q_offsets[r]) return fail(CLEF_E_SCHEMA, "q_offsets decreases at record %d", r);
  if (NQ > 0 && (b->o_offsets[0] != 0 || b->o_offsets[NQ] != NO))
    return fail(CLEF_E_SCHEMA, "o_offsets must start at 0 and end at num_options");
  if (NQ == 0 && NO != 0) return fail(CLEF_E_SCHEMA, "options without questions");
  int64_t nids = 0;
  for (int r = 0; r < B; ++r) {
    for (int q = b->q_offsets[r]; q < b->q_offsets[r + 1]; ++q) {
      const int t = b->q_type[q];
      if (t < 0 || t > 2) return fail(CLEF_E_SCHEMA, "question %d has type %d (0 noul, 1 choice, 2 score)", q, t);
      const int s = b->q_span[2 * q], e = b->q_span[2 * q + 1];
      if (!(0 <= s && s < e && e <= len[r]))
        return fail(CLEF_E_SPAN, "question %d span [%d, %d) outside record %d of length %lld", q, s, e, r,
                    (long long)len[r]);
      const int no = b->o_offsets[q + 1] - b->o_offsets[q];
      if (no < 1) return fail(CLEF_E_SCHEMA, "question %d has no options", q);
      if (t == 0 && no != 2) return fail(CLEF_E_SCHEMA, "noul question %d has %d options (needs true, false)", q, no);
      if (no > kMaxOptions) return fail(CLEF_E_UNSUPPORTED, "question %d has more than %d options", q, kMaxOptions);
      for (int k = b->o_offsets[q]; k < b->o_offsets[q + 1]; ++k) {
        const int os = b->o_span[2 * k], oe = b->o_span[2 * k + 1];
        if (!(0 <= os && os < oe && oe <= len[r]))
          return fail(CLEF_E_SPAN, "option %d span [%d, %d) outside record %d of length %lld", k, os, oe, r,
                      (long long)len[r]);
        for (int i = 0; i < oe - os; ++i) {
          const int id = b->o_ids[nids + i];
          if (id < 0 || id >= c.vocab_size)
            return fail(CLEF_E_ID, "option %d token id %d outside [0, %d)", k, id, c.vocab_size);
        }
        nids += oe - os;
      }
    }
  }

  p.B = B;
  p.NQ = NQ;
  p.NO = NO;
  p.nids = nids;
  int64_t T = 0;
  for (int r = 0; r < B; ++r) T += len[r];
  p.T = T;

  // pooled row ranges in packed row space (independent of the device layout)
  {
    p.span_rows.assign((size_t)(NQ + NO + B) * 2, 0);
    int64_t base = 0;
    for (int r = 0; r < B; ++r) {
      for (int q = b->q_offsets[r]; q < b->q_offsets[r + 1]; ++q) {
        p.span_rows[2 * q] = int32_t(base + b->q_span[2 * q]);
        p.span_rows[2 * q + 1] = int32_t(base + b->q_span[2 * q + 1]);
        for (int k = b->o_offsets[q]; k < b->o_offsets[q + 1]; ++k) {
          p.span_rows[2 * (NQ + k)] = int32_t(base + b->o_span[2 * k]);
          p.span_rows[2 * (NQ + k) + 1] = int32_t(base + b->o_span[2 * k + 1]);
        }
      }
      p.span_rows[2 * (NQ + NO + r)] = int32_t(base + len[r] - 1);
      p.span_rows[2 * (NQ + NO + r) + 1] = int32_t(base + len[r]);
      base += len[r];
    }
  }
  if (!tables || NQ == 0) return CLEF_OK;

  // active records (with questions), their padded row bases and chunking
  std::vector<int32_t> rec, tiles, kvtiles, pool, lex, ids, optq, optrec, qrec, qtype, ooff, items, frec, fitems;
  std::vector<int> act_of(B, -1);
  int64_t kv0 = 0, pbase = 0, pbase_f = 0;
  int nact = 0;
  auto attn_waves = [&](int64_t ch) {
    int64_t w = 0;
    for (int r = 0; r < B; ++r) {
      const int q0 = b->q_offsets[r], nq = b->q_offsets[r + 1] - q0;
      if (nq == 0) continue;
      const int no = b->o_offsets[q0 + nq] - b->o_offsets[q0];
      w += ceil_div(len[r], ch) * ceil_div(no, 32);
    }
    return w * NH;
  };
  int KCH = 128;
  while (KCH < 1024 && attn_waves(2 * KCH) >= kAttnMinWaves) KCH *= 2;
  p.kchunk = KCH;
  for (int r = 0; r < B; ++r) {
    const int q0 = b->q_offsets[r], nq = b->q_offsets[r + 1] - q0;
    if (nq == 0) continue;
    const int o0 = b->o_offsets[q0], no = b->o_offsets[q0 + nq] - o0;
    const int nc = (int)ceil_div(len[r], KCH);
    act_of[r] = nact;
    rec.insert(rec.end(), {int32_t(kv0), int32_t(len[r]), o0, no, int32_t(pbase), nc, q0, nq});
    for (int64_t t0 = 0; t0 < len[r]; t0 += TILE) {
      tiles.insert(tiles.end(), {int32_t(src0[r] + t0), int32_t(kv0 + t0), int32_t(std::min<int64_t>(TILE, len[r] - t0)), nact});
      kvtiles.insert(kvtiles.end(), {int32_t(kv0 + t0), int32_t(kv0 + t0), TILE, nact});
    }
    for (int ch = 0; ch < nc; ++ch)
      for (int qb = 0; qb < no; qb += 32) items.insert(items.end(), {nact, ch, qb, 0});
    if (c.field_cross_attention) {   // the record's fields as the queries of the same attention kernels
      frec.insert(frec.end(), {int32_t(kv0), int32_t(len[r]), q0, nq, int32_t(pbase_f), nc, q0, nq});
      for (int ch = 0; ch < nc; ++ch)
        for (int qb = 0; qb < nq; qb += 32) fitems.insert(fitems.end(), {nact, ch, qb, 0});
      pbase_f += (int64_t)nq * nc;
    }
    kv0 += ceil_div(len[r], TILE) * TILE;
    pbase += (int64_t)no * nc;
    ++nact;
  }
  p.Ptot_f = pbase_f;
  p.nfitems = (int)fitems.size() / 4;
  if (kv0 > INT32_MAX / 2 || pbase * 64 * NH > INT64_C(1) << 40)
    return fail(CLEF_E_UNSUPPORTED, "batch too large for 32-bit row indices");
  p.nact = nact;
  p.Tpad = kv0;
  p.Ptot = pbase;
  p.ntiles = (int)tiles.size() / 4;
  p.nitems = (int)items.size() / 4;

  // pooling entries: questions, then options, then global rows; lexical entries per option
  std::vector<int32_t> opool;
  int64_t idoff = 0;
  for (int r = 0; r < B; ++r) {
    const int a = act_of[r];
    if (a < 0) continue;
    const int64_t kvb = rec[8 * a];
    for (int q = b->q_offsets[r]; q < b->q_offsets[r + 1]; ++q) {
      const int s = b->q_span[2 * q], e = b->q_span[2 * q + 1];
      pool.insert(pool.end(), {int32_t(src0[r] + s), e - s, int32_t(kvb + s), q});
      qrec.push_back(a);
      qtype.push_back(b->q_type[q]);
      for (int k = b->o_offsets[q]; k < b->o_offsets[q + 1]; ++k) {
        const int os = b->o_span[2 * k], oe = b->o_span[2 * k + 1];
        optq.push_back(q);
        optrec.push_back(a);
        opool.insert(opool.end(), {int32_t(src0[r] + os), oe - os, int32_t(kvb + os), NQ + k});
        lex.insert(lex.end(), {int32_t(idoff), oe - os, q, NQ + NO + a});
        idoff += oe - os;
      }
    }
  }
  pool.insert(pool.end(), opool.begin(), opool.end());
  for (int r = 0; r < B; ++r) {
    const int a = act_of[r];
    if (a < 0) continue;
    const int64_t kvb = rec[8 * a];
    pool.insert(pool.end(), {int32_t(src0[r] + len[r] - 1), 1, int32_t(kvb + len[r] - 1), NQ + NO + a});
  }
  ids.assign(b->o_ids, b->o_ids + nids);
  ooff.assign(b->o_offsets, b->o_offsets + NQ + 1);
  p.npool = (int)pool.size() / 4;

  auto put = [&](const std::vector<int32_t>& v) {
    // keep every table 16-byte aligned (int4 loads)
    while (p.tab.size() % 4) p.tab.push_back(0);
    const size_t off = p.tab.size();
    p.tab.insert(p.tab.end(), v.begin(), v.end());
    return off;
  };
  p.tab.clear();
  p.off_rec = put(rec);
  p.off_tiles = put(tiles);
  p.off_kvtiles = put(kvtiles);
  p.off_pool = put(pool);
  p.off_lex = put(lex);
  p.off_ids = put(ids);
  p.off_optq = put(optq);
  p.off_optrec = put(optrec);
  p.off_qrec = put(qrec);
  p.off_qtype = put(qtype);
  p.off_ooff = put(ooff);
  p.off_items = put(items);
  p.off_frec = put(frec);
  p.off_fitems = put(fitems);
  while (p.tab.size() % 4) p.tab.push_back(0);
  return CLEF_OK;
}

// ---------------------------------------------------------------------------
// device weights
// ---------------------------------------------------------------------------
struct Layer {
  const float *ln1g, *ln1b, *ln2g, *ln2b, *bq, *bo, *b1, *b2, *bqkv;
  const bf16_t *Wq, *Wo, *W1, *W2, *Wqkv;
  // decoder-layer field variant: cross-attention norm, query and output maps
  const float *xlng = nullptr, *xlnb = nullptr, *bxq = nullptr, *bxo = nullptr;
  const bf16_t *Wxq = nullptr, *Wxo = nullptr;
};

struct Weights {
  const float *lnin_g, *lnin_b, *cmem, *dmem, *cmem16, *ba7, *bqq, *bg, *temb, *sw, *bkv, *bs1, *ws2;
  const bf16_t *Wmem, *Wmem16, *Wa7, *Wqq, *Wg, *Wkv, *Ws1;   // Wmem16 holds fp16 bits
  const bf16_t* Wfkv = nullptr;   // decoder-layer field variant: cross K/V of every field layer, stacked
  const float* bfkv = nullptr;
  // precision mode fp32: the memory projection unfolded (LayerNorm applied to the rows) with its own bias,
  // and the stacked K/V projections, in the small GEMMs' fragment order (batches of few row tiles); for the
  // big GEMMs the memory weight also as rows repeated three times, [W | W | W] (against the three bf16
  // terms of each normalised fp16 row), and folded, as the three bf16 terms of fp32(W diag(gamma)) with
  // its row sums (against bf16 rows read three times); the K/V product reads Wkv / Wfkv three times
  const float* bmem = nullptr;
  const bf16_t *Wmem_fr = nullptr, *Wkv_fr = nullptr, *Wfkv_fr = nullptr;
  const bf16_t* Wmem3 = nullptr;    // [W | W | W] (fp32 head, fp16 hidden rows)
  const bf16_t* Wmem3f = nullptr;   // three bf16 terms of fp32(W diag(gamma)) (fp32 head, bf16 hidden rows)
  const float* cmem32 = nullptr;    // row sums of fp32(W diag(gamma))
  std::vector<Layer> route, field;
  float sb, bs2, gate_logit, gate, lam;
};

}  // namespace

// What the heads made from one clef_head_create share besides the weights: the
// side stream and the order of their big-GEMM phases.  A head waits for the
// previous head's K/V GEMM before its memory GEMM starts and marks its own K/V
// GEMM done, so with several batches in flight the (MFMA-bound) big GEMMs of
// one batch run beside the (latency-bound) small-GEMM chains of the others
// instead of all batches doing their GEMMs at once.
struct HeadGroup {
  std::mutex mu;
  hipEvent_t gemm_done = nullptr;
  bool recorded = false;
  ~HeadGroup() {
    if (gemm_done) (void)hipEventDestroy(gemm_done);
  }
};

struct clef_head {
  clef_head_config cfg;
  int device = 0;
  const bf16_t* table = nullptr;
  std::shared_ptr<void> dweights;        // the weight blob, shared by heads made with clef_head_create_sharing
  Weights w;
  // workspace
  void* ws = nullptr;
  size_t ws_bytes = 0;
  void* pinned = nullptr;
  size_t pinned_bytes = 0;
  hipEvent_t staged = nullptr;
  // second stream for the work independent of the big GEMMs; heads made with
  // clef_head_create_sharing use their source's, so that several heads in
  // flight take one extra hardware queue between them, not one each
  std::shared_ptr<std::remove_pointer_t<hipStream_t>> side;
  std::shared_ptr<HeadGroup> group;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool staged_pending = false;
  // end of the handle's last piece of GPU work (forward or streamed chunk): the
  // next one waits for it, and buffers are only freed or regrown after it
  hipEvent_t done = nullptr;
  bool done_recorded = false;
  // trace
  bool trace = false;
  void* tr = nullptr;
  size_t tr_bytes = 0;
  hipStream_t last_stream = nullptr;
  int last_NQ = 0, last_NO = 0, last_B = 0;
  int64_t last_Tpad = 0;
  // workspace pointers of the last forward (for traces)
  float *pooled = nullptr, *ebar = nullptr, *prior = nullptr;
  bf16_t* mem = nullptr;
  float *tr_u = nullptr, *tr_f0 = nullptr, *tr_f = nullptr, *tr_jcos = nullptr, *tr_mlp = nullptr;
  // the index tables the last traced forward uploaded (read back from the device)
  const int32_t* tr_tab = nullptr;
  size_t tr_off_pool = 0, tr_off_lex = 0, tr_off_ids = 0;
  int64_t tr_npool = 0, tr_nlex = 0, tr_nids = 0;
  // allocation-free forwards: the plan's tables, kept until the next such call
  std::vector<int32_t> noalloc_tab;
  // stage timing
  bool prof = false;
  std::vector<hipEvent_t> ev;
  double stage_ms[CLEF_NUM_STAGES] = {};
  int64_t prof_calls = 0;
  // streamed ingest (clef_head_stream_*): the batch's rows arrive in chunks
  struct Stream {
    bool active = false;
    std::vector<int32_t> tab;                  // the plan's tables (end must describe the same batch)
    std::vector<int64_t> cu;                   // first staging row of each record
    std::vector<int32_t> len, received;        // valid rows and rows received per record
    std::vector<std::vector<int>> rec_tiles;   // plan tile indices of each record, in row order
    int64_t ntiles = 0, Tpad = 0;
    size_t off_tiles = 0, off_kvtiles = 0;     // int32 offsets of the tile tables in tab
    size_t ws_tab = 0, ws_stats = 0, ws_mem = 0, ws_kv = 0, ws_bigpart = 0;   // workspace offsets
    int split_mem = 1, split_kv = 1, split_fkv = 1;
    size_t ws_fkv = 0;
    bool f16 = false, gemms = false, cross = false;
    void* rows = nullptr;                      // staging rows [T, H], 16-bit elements
    size_t rows_bytes = 0;
  } strm;
};

namespace {

struct Blob {
  std::vector<uint8_t> host;
  size_t add(const void* src, size_t bytes) {
    const size_t off = align256(host.size());
    host.resize(off + bytes);
    if (src) memcpy(host.data() + off, src, bytes);
    return off;
  }
  size_t add_f32(const std::vector<float>& v) { return add(v.data(), v.size() * 4); }
};

// Weights of the small GEMMs are stored in MFMA fragment order: the [N, K]
// matrix is cut into 16 x 32 blocks (16 output columns, 32 K positions),
// blocks of one 16-column strip follow each other along K, and inside a block
// lane l of a wave finds its 16-byte B fragment (column l % 16, K positions
// 8 (l / 16) .. +8) at element 8 l.  A wave then reads a whole block with one
// fully coalesced 1 KB load instead of touching 16 rows per load.
std::vector<uint16_t> fragment_order(const uint16_t* src, int N, int K) {
  std::vector<uint16_t> out((size_t)N * K);
  const int kb = K / 32;
  for (int n = 0; n < N; ++n)
    for (int k8 = 0; k8 < K / 8; ++k8) {   // 8 consecutive K positions stay together
      const size_t blk = (size_t)(n / 16) * kb + k8 / 4;
      const int lane = (n % 16) + 16 * (k8 % 4);
      memcpy(&out[blk * 512 + lane * 8], src + (size_t)n * K + k8 * 8, 16);
    }
  return out;
}

struct NamedW {
  const void* p;
  int64_t n;
  int32_t dt;
};

int build_weights(clef_head* h, const clef_head_weight* w, int32_t nw) {
  const clef_head_config& c = h->cfg;
  const int H = c.hidden_size;
  std::unordered_map<std::string, NamedW> m;
  if (nw < 0 || (nw > 0 && !w)) return fail(CLEF_E_ARG, "weights array is NULL");
  for (int i = 0; i < nw; ++i) {
    if (!w[i].name || !w[i].host_data) return fail(CLEF_E_ARG, "weight %d has a NULL name or data", i);
    if (m.count(w[i].name)) return fail(CLEF_E_ARG, "weight %s given twice", w[i].name);
    m[w[i].name] = {w[i].host_data, w[i].numel, w[i].dtype};
  }
  const auto specs = weight_list(c);
  for (auto& s : specs) {
    auto it = m.find(s.name);
    if (it == m.end()) return fail(CLEF_E_ARG, "missing weight %s", s.name.c_str());
    if (it->second.n != s.numel || it->second.dt != s.dtype)
      return fail(CLEF_E_ARG, "weight %s has %lld elements of dtype %d, expected %lld of dtype %d", s.name.c_str(),
                  (long long)it->second.n, it->second.dt, (long long)s.numel, s.dtype);
  }
  if (m.size() != specs.size()) return fail(CLEF_E_ARG, "unexpected extra weights (%zu given, %zu expected)", m.size(), specs.size());

  auto bf = [&](const std::string& n) { return static_cast<const uint16_t*>(m[n].p); };
  auto tof = [&](const std::string& n) {
    const auto& e = m[n];
    std::vector<float> v(e.n);
    const uint16_t* s = static_cast<const uint16_t*>(e.p);
    for (int64_t i = 0; i < e.n; ++i) v[i] = bf16_to_f(s[i]);
    return v;
  };
  auto scalar = [&](const std::string& n) { return *static_cast<const float*>(m[n].p); };

  Blob blob;
  struct Fix { size_t off; const void** dst; };
  std::vector<std::pair<size_t, const void**>> fix;
  auto put_bf = [&](const uint16_t* src, size_t n, const bf16_t** dst) { fix.push_back({blob.add(src, n * 2), (const void**)dst}); };
  auto put_f = [&](const std::vector<float>& v, const float** dst) { fix.push_back({blob.add_f32(v), (const void**)dst}); };
  auto put_frag = [&](const uint16_t* src, int N, int K, const bf16_t** dst) {
    const std::vector<uint16_t> v = fragment_order(src, N, K);
    put_bf(v.data(), v.size(), dst);
  };
  // [N][K] rows repeated three times along K: [N][3 K] = [W | W | W]
  auto put_rep3 = [&](const uint16_t* src, int N, int K, const bf16_t** dst) {
    std::vector<uint16_t> v((size_t)N * 3 * K);
    for (int n = 0; n < N; ++n)
      for (int p = 0; p < 3; ++p) memcpy(&v[((size_t)n * 3 + p) * K], src + (size_t)n * K, (size_t)K * 2);
    put_bf(v.data(), v.size(), dst);
  };

  Weights& W = h->w;
  // input LayerNorm (pooling) and the memory projection with the LayerNorm folded in
  const std::vector<float> g = tof("ln_in.w"), be = tof("ln_in.b");
  put_f(g, &W.lnin_g);
  put_f(be, &W.lnin_b);
  {
    const uint16_t* Wm = bf("mem.w");
    const std::vector<float> bm = tof("mem.b");
    std::vector<uint16_t> Wp((size_t)D * H), Wp16((size_t)D * H);
    std::vector<float> cm(D), cm16(D), dm(D);
    for (int j = 0; j < D; ++j) {
      double cs = 0, cs16 = 0, ds = bm[j];
      for (int k = 0; k < H; ++k) {
        const float wv = bf16_to_f(Wm[(size_t)j * H + k]);
        const uint16_t wp = f_to_bf16(wv * g[k]);
        Wp[(size_t)j * H + k] = wp;
        cs += bf16_to_f(wp);
        // fp16 copy for fp16 hidden rows (round to nearest even)
        const _Float16 wh = (_Float16)(wv * g[k]);
        Wp16[(size_t)j * H + k] = __builtin_bit_cast(uint16_t, wh);
        cs16 += (double)(float)wh;
        ds += (double)wv * be[k];
      }
      cm[j] = (float)cs;
      cm16[j] = (float)cs16;
      dm[j] = (float)ds;
    }
    put_bf(Wp.data(), Wp.size(), &W.Wmem);
    put_f(cm, &W.cmem);
    if (c.precision == CLEF_PRECISION_F32) {
      put_frag(Wm, D, H, &W.Wmem_fr);
      put_rep3(Wm, D, H, &W.Wmem3);
      put_f(bm, &W.bmem);
      // the folded weight in fp32, as three exact bf16 terms side by side, and its row sums
      std::vector<uint16_t> Wt((size_t)D * 3 * H);
      std::vector<float> cm32(D);
      for (int j = 0; j < D; ++j) {
        double cs = 0;
        for (int k = 0; k < H; ++k) {
          const float wv = bf16_to_f(Wm[(size_t)j * H + k]) * g[k];
          cs += wv;
          float r = wv;
          for (int t = 0; t < 3; ++t) {
            const uint16_t b = f_to_bf16(r);
            Wt[((size_t)j * 3 + t) * H + k] = b;
            r -= bf16_to_f(b);
          }
        }
        cm32[j] = (float)cs;
      }
      put_bf(Wt.data(), Wt.size(), &W.Wmem3f);
      put_f(cm32, &W.cmem32);
    }
    put_bf(Wp16.data(), Wp16.size(), &W.Wmem16);
    put_f(cm16, &W.cmem16);
    put_f(dm, &W.dmem);
  }
  // option-query projection: [W_c | W_l] along K with the three biases summed; the
  // question term W_qo q depends only on the question, so it is computed once per
  // question, stacked under the field base projection: [W_q ; W_qo] (bias [b_q ; 0])
  {
    std::vector<uint16_t> Wa((size_t)D * 2 * H);
    const uint16_t* a = bf("opt_ctx.w");
    const uint16_t* l = bf("opt_lex.w");
    for (int j = 0; j < D; ++j) {
      memcpy(&Wa[(size_t)j * 2 * H], a + (size_t)j * H, H * 2);
      memcpy(&Wa[(size_t)j * 2 * H + H], l + (size_t)j * H, H * 2);
    }
    put_frag(Wa.data(), D, 2 * H, &W.Wa7);
    const auto b1 = tof("opt_ctx.b"), b2 = tof("opt_lex.b"), b3 = tof("q_opt.b");
    std::vector<float> bs(D);
    for (int j = 0; j < D; ++j) bs[j] = (float)((double)b1[j] + b2[j] + b3[j]);
    put_f(bs, &W.ba7);
    std::vector<uint16_t> Wq((size_t)2 * D * H);
    memcpy(Wq.data(), bf("q_base.w"), (size_t)D * H * 2);
    memcpy(Wq.data() + (size_t)D * H, bf("q_opt.w"), (size_t)D * H * 2);
    put_frag(Wq.data(), 2 * D, H, &W.Wqq);
    std::vector<float> bq(2 * D, 0.f);
    const auto bb = tof("q_base.b");
    std::copy(bb.begin(), bb.end(), bq.begin());
    put_f(bq, &W.bqq);
  }
  put_frag(bf("glob.w"), D, H, &W.Wg);
  put_f(tof("glob.b"), &W.bg);
  put_f(tof("type_emb"), &W.temb);
  put_f(tof("summary.w"), &W.sw);
  W.sb = bf16_to_f(bf("summary.b")[0]);

  const int NR = c.routing_layers, NL = c.layers;
  // K/V of every routing layer stacked: [K_0; V_0; K_1; V_1; ...] rows
  {
    std::vector<uint16_t> Wkv((size_t)NR * 2 * D * D);
    std::vector<float> bkv((size_t)NR * 2 * D);
    for (int r = 0; r < NR; ++r) {
      const std::string p = "route." + std::to_string(r);
      memcpy(&Wkv[(size_t)(2 * r) * D * D], bf(p + ".k.w"), (size_t)D * D * 2);
      memcpy(&Wkv[(size_t)(2 * r + 1) * D * D], bf(p + ".v.w"), (size_t)D * D * 2);
      const auto bk = tof(p + ".k.b"), bv = tof(p + ".v.b");
      std::copy(bk.begin(), bk.end(), bkv.begin() + (size_t)(2 * r) * D);
      std::copy(bv.begin(), bv.end(), bkv.begin() + (size_t)(2 * r + 1) * D);
    }
    if (NR > 0) {
      put_bf(Wkv.data(), Wkv.size(), &W.Wkv);
      put_f(bkv, &W.bkv);
      if (c.precision == CLEF_PRECISION_F32) put_frag(Wkv.data(), NR * 2 * D, D, &W.Wkv_fr);
    } else {
      W.Wkv = nullptr;
      W.bkv = nullptr;
    }
  }
  W.route.resize(NR);
  W.field.resize(NL);
  for (int s = 0; s < NR + NL; ++s) {
    const bool route = s < NR;
    const std::string p = route ? "route." + std::to_string(s) : "field." + std::to_string(s - NR);
    Layer& L = route ? W.route[s] : W.field[s - NR];
    put_f(tof(p + ".ln1.w"), &L.ln1g);
    put_f(tof(p + ".ln1.b"), &L.ln1b);
    put_f(tof(p + ".ln2.w"), &L.ln2g);
    put_f(tof(p + ".ln2.b"), &L.ln2b);
    if (route) {
      put_frag(bf(p + ".q.w"), D, D, &L.Wq);
      put_f(tof(p + ".q.b"), &L.bq);
      L.Wqkv = nullptr;
      L.bqkv = nullptr;
    } else {
      std::vector<uint16_t> Wqkv((size_t)3 * D * D);
      std::vector<float> bqkv((size_t)3 * D);
      int i = 0;
      for (const char* mname : {"q", "k", "v"}) {
        memcpy(&Wqkv[(size_t)i * D * D], bf(p + "." + mname + ".w"), (size_t)D * D * 2);
        const auto bb = tof(p + "." + mname + ".b");
        std::copy(bb.begin(), bb.end(), bqkv.begin() + (size_t)i * D);
        ++i;
      }
      put_frag(Wqkv.data(), 3 * D, D, &L.Wqkv);
      put_f(bqkv, &L.bqkv);
      L.Wq = nullptr;
      L.bq = nullptr;
    }
    put_frag(bf(p + ".o.w"), D, D, &L.Wo);
    put_f(tof(p + ".o.b"), &L.bo);
    put_frag(bf(p + ".ffn1.w"), F, D, &L.W1);
    put_f(tof(p + ".ffn1.b"), &L.b1);
    put_frag(bf(p + ".ffn2.w"), D, F, &L.W2);
    put_f(tof(p + ".ffn2.b"), &L.b2);
  }
  if (c.field_cross_attention && NL > 0) {
    // cross K/V of every field layer stacked like the routing ones: [K_0; V_0; K_1; V_1; ...]
    std::vector<uint16_t> Wf((size_t)NL * 2 * D * D);
    std::vector<float> bfv((size_t)NL * 2 * D);
    for (int l = 0; l < NL; ++l) {
      const std::string p = "field." + std::to_string(l);
      memcpy(&Wf[(size_t)(2 * l) * D * D], bf(p + ".xk.w"), (size_t)D * D * 2);
      memcpy(&Wf[(size_t)(2 * l + 1) * D * D], bf(p + ".xv.w"), (size_t)D * D * 2);
      const auto bk = tof(p + ".xk.b"), bv = tof(p + ".xv.b");
      std::copy(bk.begin(), bk.end(), bfv.begin() + (size_t)(2 * l) * D);
      std::copy(bv.begin(), bv.end(), bfv.begin() + (size_t)(2 * l + 1) * D);
      Layer& L = W.field[l];
      put_f(tof(p + ".xln.w"), &L.xlng);
      put_f(tof(p + ".xln.b"), &L.xlnb);
      put_frag(bf(p + ".xq.w"), D, D, &L.Wxq);
      put_f(tof(p + ".xq.b"), &L.bxq);
      put_frag(bf(p + ".xo.w"), D, D, &L.Wxo);
      put_f(tof(p + ".xo.b"), &L.bxo);
    }
    put_bf(Wf.data(), Wf.size(), &W.Wfkv);
    put_f(bfv, &W.bfkv);
    if (c.precision == CLEF_PRECISION_F32) put_frag(Wf.data(), NL * 2 * D, D, &W.Wfkv_fr);
  }
  put_frag(bf("score.w1"), D, 4 * D, &W.Ws1);
  put_f(tof("score.b1"), &W.bs1);
  put_f(tof("score.w2"), &W.ws2);
  W.bs2 = bf16_to_f(bf("score.b2")[0]);
  W.gate_logit = scalar("gate_logit");
  W.lam = scalar("joint_scale");
  {
    // logistic gate; e^x / (1 + e^x) for x < 0 takes no exponent of a large positive argument
    const double gl = W.gate_logit;
    const double gs = gl >= 0.0 ? 1.0 / (1.0 + std::exp(-gl)) : std::exp(gl) / (1.0 + std::exp(gl));
    W.gate = (float)gs;
  }

  void* d = nullptr;
  if (dev_malloc(&d, blob.host.size()) != hipSuccess)
    return fail(CLEF_E_NOMEM, "hipMalloc of %zu bytes of weights failed", blob.host.size());
  if (hipMemcpy(d, blob.host.data(), blob.host.size(), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(d);
    return fail(CLEF_E_HIP, "copying weights to the device failed");
  }
  const int dev = h->device;
  h->dweights = std::shared_ptr<void>(d, [dev](void* q) {
    int cur = dev;
    (void)hipGetDevice(&cur);
    if (cur != dev) (void)hipSetDevice(dev);
    (void)hipFree(q);
    if (cur != dev) (void)hipSetDevice(cur);
  });
  for (auto& f : fix) *f.second = static_cast<const uint8_t*>(d) + f.first;
  return CLEF_OK;
}

// workspace layout for one plan
struct WsLayout {
  size_t tab, stats, pooled, ebar, prior, mem, kv, fkv, bigpart, xplanes, mplanes, u, ustats, qbuf, attn, hbuf, qv,
      qo, gp, f, fstats, fattn, opart, pm, pl, po, part, total;
};

// fp32 head: whole-K big GEMMs over the activations' three bf16 terms once the
// batch has enough row tiles to fill the chip without splitting K (the memory
// product's 4 column tiles then give more than 64 workgroups); fewer tiles run
// on the split-K small GEMMs.
bool f32_big_gemms(int ntiles) { return ntiles > 16; }

WsLayout ws_layout(const clef_head_config& c, const Plan& p) {
  const size_t H = c.hidden_size, NQ = p.NQ, NO = p.NO, Tp = p.Tpad, NR = c.routing_layers;
  WsLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t r = o; o = align256(o + bytes); return r; };
  L.tab = take(p.tab.size() * 4);
  L.stats = take(Tp * 8);
  L.pooled = take((NQ + NO + p.nact) * H * 4);
  L.ebar = take(NO * H * 4);
  L.prior = take(NO * 4);
  // memory rows and K/V: bf16, or fp32 in the fp32 precision mode
  const bool f32 = c.precision == CLEF_PRECISION_F32;
  const size_t el = f32 ? 4 : 2;
  L.mem = take(Tp * D * el);
  L.kv = take(NR * 2 * NH * Tp * 64 * el);
  const size_t NLx = c.field_cross_attention ? (size_t)c.layers : 0;   // field layers with cross-attention
  L.fkv = take(NLx * 2 * NH * Tp * 64 * el);
  // split-K partial sums of the big GEMMs (few row tiles only; the memory and
  // K/V GEMMs run one after the other on one stream and share the region)
  if (f32) {   // the small-GEMM kernel over the packed rows
    size_t fl = 0;
    if (Tp > 0) {
      fl = sgemm_shape((int)Tp, D, (int)H).part_floats;
      if (NR > 0) fl = std::max(fl, sgemm_shape((int)Tp, (int)NR * 2 * D, D).part_floats);
      if (NLx > 0) fl = std::max(fl, sgemm_shape((int)Tp, (int)NLx * 2 * D, D).part_floats);
    }
    L.bigpart = take(fl * 4);
    if (f32_big_gemms(p.ntiles)) {
      if (p.f16) L.xplanes = take(Tp * 3 * H * 2);   // LayerNorm-ed fp16 rows, three bf16 terms
      L.mplanes = take(Tp * 3 * D * 2);   // memory rows, three bf16 terms
    }
  } else {
    const size_t sm = big_gemm_split(p.ntiles, D / 256, (int)H), skv = big_gemm_split(p.ntiles, (int)NR * 8, D);
    const size_t sf = big_gemm_split(p.ntiles, (int)NLx * 8, D);
    size_t bytes = std::max(sm > 1 ? sm * Tp * D * 4 : 0, (NR > 0 && skv > 1) ? skv * Tp * NR * 2 * D * 4 : 0);
    bytes = std::max(bytes, (NLx > 0 && sf > 1) ? sf * Tp * NLx * 2 * D * 4 : 0);
    L.bigpart = take(bytes);
  }
  L.u = take(NO * D * 4);
  L.ustats = take(NO * 8);
  L.qbuf = take(NO * D * 4);
  L.attn = take(NO * D * 4);
  L.hbuf = take(std::max(NO, NQ) * F * 4);
  L.qv = take(NQ * D * 4);
  L.qo = take(NQ * D * 4);
  L.gp = take((size_t)p.nact * D * 4);
  L.f = take(NQ * D * 4);
  L.fstats = take(NQ * 8);
  L.fattn = take(NQ * D * 4);
  L.opart = take((size_t)NH * ceil_div(NQ, kSgemmRows) * kSgemmRows * D * 4);   // per-head slices of attn W_o^T
  const size_t Pmax = (size_t)std::max(p.Ptot, p.Ptot_f);   // routing and field cross-attention partials
  L.pm = take(NH * Pmax * 4);
  L.pl = take(NH * Pmax * 4);
  L.po = take(NH * Pmax * 64 * 4);
  size_t part = 0;
  const int shapes[][3] = {{p.NO, D, 2 * (int)H}, {p.NQ, 2 * D, (int)H}, {p.nact, D, (int)H}, {p.NO, D, D},
                           {p.NO, F, D},        {p.NO, D, F},        {p.NQ, 3 * D, D},     {p.NQ, D, D},
                           {p.NQ, F, D},        {p.NQ, D, F},        {p.NO, D, 4 * D}};
  for (auto& s : shapes) {
    if (s[0] == 0) continue;
    const SgemmShape g = sgemm_shape(s[0], s[1], s[2], s[1] == D);
    part = std::max(part, g.part_floats);
  }
  // products whose slices are summed by their consumer (field QKV, scoring hidden layer)
  const int pshapes[][3] = {{p.NQ, 3 * D, D}, {p.NO, D, 4 * D}};
  for (auto& s : pshapes) {
    if (s[0] == 0) continue;
    const SgemmShape g = sgemm_shape(s[0], s[1], s[2], false, true);
    part = std::max(part, (size_t)g.nsplit * g.mtiles * kSgemmRows * s[1]);
  }
  L.part = take(part * 4);
  L.total = o;
  return L;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* clef_head_last_error(void) { return g_err.c_str(); }

int32_t clef_head_weight_count(const clef_head_config* cfg) {
  if (check_config(cfg) != CLEF_OK) return -1;
  return (int32_t)weight_list(*cfg).size();
}

int clef_head_weight_info(const clef_head_config* cfg, int32_t i, char* name, int32_t name_cap, int64_t* numel,
                          int32_t* dtype) {
  int rc = check_config(cfg);
  if (rc) return rc;
  const auto s = weight_list(*cfg);
  if (i < 0 || i >= (int32_t)s.size()) return fail(CLEF_E_ARG, "weight index %d out of range", i);
  if (name) {
    if (name_cap < (int32_t)s[i].name.size() + 1) return fail(CLEF_E_ARG, "name buffer too small");
    memcpy(name, s[i].name.c_str(), s[i].name.size() + 1);
  }
  if (numel) *numel = s[i].numel;
  if (dtype) *dtype = s[i].dtype;
  return CLEF_OK;
}

int clef_head_check_batch(const clef_head_config* cfg, const clef_head_batch* batch, int64_t* num_rows) {
  int rc = check_config(cfg);
  if (rc) return rc;
  Plan p;
  rc = build_plan(*cfg, batch, p, false);
  if (rc) return rc;
  if (num_rows) *num_rows = p.T;
  return CLEF_OK;
}

int clef_head_span_rows(const clef_head_config* cfg, const clef_head_batch* batch, int32_t* rows) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!rows) return fail(CLEF_E_ARG, "rows is NULL");
  Plan p;
  rc = build_plan(*cfg, batch, p, false);
  if (rc) return rc;
  memcpy(rows, p.span_rows.data(), p.span_rows.size() * 4);
  return CLEF_OK;
}

namespace {

// Events of a handle and, unless it already has them, its side stream and
// group; created on the current device.
bool create_streams(clef_head* h) {
  if (hipEventCreateWithFlags(&h->staged, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->done, hipEventDisableTiming) != hipSuccess)
    return false;
  if (!h->group) {
    auto g = std::make_shared<HeadGroup>();
    if (hipEventCreateWithFlags(&g->gemm_done, hipEventDisableTiming) != hipSuccess) return false;
    h->group = g;
  }
  if (h->side) return true;
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return false;
  h->side.reset(s, [](hipStream_t q) {
    (void)hipStreamSynchronize(q);
    (void)hipStreamDestroy(q);
  });
  return true;
}

}  // namespace

int clef_head_create(const clef_head_config* cfg, const clef_head_weight* weights, int32_t num_weights,
                     const void* lexical_table, clef_head** out) {
  if (!out) return fail(CLEF_E_ARG, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!lexical_table) return fail(CLEF_E_ARG, "lexical_table is NULL");
  clef_head* h = new clef_head();
  h->cfg = *cfg;
  h->table = static_cast<const bf16_t*>(lexical_table);
  int num_cu = 0;
  if (hipGetDevice(&h->device) != hipSuccess ||
      hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess ||
      num_cu <= 0) {
    delete h;
    return fail(CLEF_E_HIP, "no HIP device");
  }
  rc = build_weights(h, weights, num_weights);
  if (rc) {
    delete h;
    return rc;
  }
  if (!create_streams(h)) {
    clef_head_destroy(h);
    return fail(CLEF_E_HIP, "creating events / the side stream failed");
  }
  *out = h;
  return CLEF_OK;
}

int clef_head_create_sharing(const clef_head* src, clef_head** out) {
  if (!out) return fail(CLEF_E_ARG, "out is NULL");
  *out = nullptr;
  if (!src || !src->dweights) return fail(CLEF_E_ARG, "source handle is NULL");
  int dev_prev = src->device;
  if (hipGetDevice(&dev_prev) != hipSuccess) return fail(CLEF_E_HIP, "no HIP device");
  if (dev_prev != src->device && hipSetDevice(src->device) != hipSuccess)
    return fail(CLEF_E_HIP, "cannot select the source handle's device");
  clef_head* h = new clef_head();
  h->cfg = src->cfg;
  h->device = src->device;
  h->table = src->table;
  h->w = src->w;
  h->dweights = src->dweights;
  h->side = src->side;
  h->group = src->group;
  const bool ok = create_streams(h);
  if (!ok) clef_head_destroy(h);
  if (dev_prev != src->device) (void)hipSetDevice(dev_prev);
  if (!ok) return fail(CLEF_E_HIP, "creating events / the side stream failed");
  *out = h;
  return CLEF_OK;
}

void clef_head_destroy(clef_head* h) {
  if (!h) return;
  if (h->done) {
    if (h->done_recorded) (void)hipEventSynchronize(h->done);   // the handle's last work still reads its buffers
    (void)hipEventDestroy(h->done);
  }
  for (auto e : h->ev) (void)hipEventDestroy(e);
  if (h->side) (void)hipStreamSynchronize(h->side.get());   // this head's side work; the stream goes with its last user
  h->side.reset();
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  if (h->staged) {
    if (h->staged_pending) (void)hipEventSynchronize(h->staged);
    (void)hipEventDestroy(h->staged);
  }
  if (h->ws) (void)hipFree(h->ws);
  if (h->strm.rows) (void)hipFree(h->strm.rows);
  if (h->tr) (void)hipFree(h->tr);
  if (h->pinned) (void)hipHostFree(h->pinned);
  h->dweights.reset();
  delete h;
}

int clef_head_debug_set(int32_t what, int64_t value) {
  if (what == CLEF_DEBUG_ALLOC_LIMIT) {
    if (value < 0) return fail(CLEF_E_ARG, "allocation limit must be >= 0");
    g_alloc_limit.store(value);
    return CLEF_OK;
  }
  if (what == CLEF_DEBUG_POISON) {
    g_poison.store(value != 0 ? 1 : 0);
    return CLEF_OK;
  }
  return fail(CLEF_E_ARG, "unknown debug setting %d", what);
}

int clef_head_set_profiling(clef_head* h, int32_t enable) {
  if (!h) return fail(CLEF_E_ARG, "handle is NULL");
  h->prof = enable != 0;
  for (double& x : h->stage_ms) x = 0.0;
  h->prof_calls = 0;
  return CLEF_OK;
}

int clef_head_stage_times(clef_head* h, double* ms, int64_t* forwards) {
  if (!h || !ms) return fail(CLEF_E_ARG, "NULL argument");
  for (int i = 0; i < CLEF_NUM_STAGES; ++i) ms[i] = h->stage_ms[i];
  if (forwards) *forwards = h->prof_calls;
  return CLEF_OK;
}

int clef_head_set_trace(clef_head* h, int32_t enable) {
  if (!h) return fail(CLEF_E_ARG, "handle is NULL");
  h->trace = enable != 0;
  return CLEF_OK;
}

int clef_head_trace(clef_head* h, int32_t which, void* host_dst, int64_t bytes) {
  if (!h || !host_dst) return fail(CLEF_E_ARG, "NULL argument");
  if (!h->trace || !h->pooled) return fail(CLEF_E_ARG, "tracing was not enabled for the last forward");
  HIPCHK(hipStreamSynchronize(h->last_stream));
  const size_t H = h->cfg.hidden_size, NQ = h->last_NQ, NO = h->last_NO, B = h->last_B;
  const void* src = nullptr;
  size_t n = 0;
  const int NR = h->cfg.routing_layers;
  if (which == CLEF_TRACE_POOLED) { src = h->pooled; n = (NQ + NO + B) * H * 4; }
  else if (which == CLEF_TRACE_LEXICAL) { src = h->ebar; n = NO * H * 4; }
  else if (which == CLEF_TRACE_PRIOR) { src = h->prior; n = NO * 4; }
  else if (which == CLEF_TRACE_MEMORY) {
    src = h->mem;
    n = (size_t)h->last_Tpad * D * (h->cfg.precision == CLEF_PRECISION_F32 ? 4 : 2);
  }
  else if (which == CLEF_TRACE_F0) { src = h->tr_f0; n = NQ * D * 4; }
  else if (which == CLEF_TRACE_F) { src = h->tr_f; n = NQ * D * 4; }
  else if (which == CLEF_TRACE_JCOS) { src = h->tr_jcos; n = NO * 4; }
  else if (which == CLEF_TRACE_MLP) { src = h->tr_mlp; n = NO * 4; }
  else if (which == CLEF_TRACE_POOL_TABLE) { src = h->tr_tab + h->tr_off_pool; n = (size_t)h->tr_npool * 16; }
  else if (which == CLEF_TRACE_LEX_TABLE) { src = h->tr_tab + h->tr_off_lex; n = (size_t)h->tr_nlex * 16; }
  else if (which == CLEF_TRACE_IDS) { src = h->tr_tab + h->tr_off_ids; n = (size_t)h->tr_nids * 4; }
  else if (which >= CLEF_TRACE_U && which <= CLEF_TRACE_U + NR) {
    src = h->tr_u + (size_t)(which - CLEF_TRACE_U) * NO * D;
    n = NO * D * 4;
  } else
    return fail(CLEF_E_ARG, "unknown trace id %d", which);
  if ((size_t)bytes != n) return fail(CLEF_E_ARG, "trace %d holds %zu bytes, %lld requested", which, n, (long long)bytes);
  if (!src) return fail(CLEF_E_ARG, "trace %d was not recorded (joint branch skipped?)", which);
  HIPCHK(hipMemcpy(host_dst, src, n, hipMemcpyDeviceToHost));
  return CLEF_OK;
}

// Grow the workspace and the pinned staging to fit the plan, then upload its
// tables on st (the caller's device is current).
static int stage_plan(clef_head* h, const Plan& p, const WsLayout& L, hipStream_t st) {
  if (L.total > h->ws_bytes) {
    if (h->staged_pending) HIPCHK(hipEventSynchronize(h->staged));
    if (h->done_recorded) HIPCHK(hipEventSynchronize(h->done));   // the old workspace's last reader
    if (h->ws) (void)hipFree(h->ws);
    h->ws = nullptr;
    h->ws_bytes = 0;
    const size_t want = L.total + L.total / 4;
    if (dev_malloc(&h->ws, want) != hipSuccess) return fail(CLEF_E_NOMEM, "workspace hipMalloc of %zu bytes failed", want);
    h->ws_bytes = want;
    if (g_poison.load()) launch_fill_u32(st, h->ws, want, 0xffffffffu);
  }
  const size_t tab_bytes = p.tab.size() * 4;
  if (h->staged_pending) HIPCHK(hipEventSynchronize(h->staged));
  if (tab_bytes > h->pinned_bytes) {
    if (h->pinned) (void)hipHostFree(h->pinned);
    h->pinned = nullptr;
    h->pinned_bytes = 0;
    const size_t want = tab_bytes + tab_bytes / 2 + 4096;
    if (pinned_malloc(&h->pinned, want) != hipSuccess)
      return fail(CLEF_E_NOMEM, "pinned staging of %zu bytes failed", want);
    h->pinned_bytes = want;
  }
  memcpy(h->pinned, p.tab.data(), tab_bytes);
  HIPCHK(hipMemcpyAsync(static_cast<uint8_t*>(h->ws) + L.tab, h->pinned, tab_bytes, hipMemcpyHostToDevice, st));
  HIPCHK(hipEventRecord(h->staged, st));
  h->staged_pending = true;
  return CLEF_OK;
}

// Allocation-free staging: the workspace is the static per-device scratch and
// the tables are copied from ordinary (pageable) host memory, which the HIP
// runtime reads before the copy call returns; the handle keeps its own copy
// of them until the next call all the same.
static int stage_plan_noalloc(clef_head* h, const Plan& p, const WsLayout& L, void* ws, hipStream_t st) {
  if (L.total > kNoallocScratchBytes)
    return fail(CLEF_E_UNSUPPORTED,
                "the batch needs %zu bytes of workspace; the allocation-free entry point holds at most %zu "
                "(use clef_head_forward for larger batches)",
                L.total, (size_t)kNoallocScratchBytes);
  if (g_poison.load()) launch_fill_u32(st, ws, L.total, 0xffffffffu);
  h->noalloc_tab = p.tab;
  HIPCHK(hipMemcpyAsync(static_cast<uint8_t*>(ws) + L.tab, h->noalloc_tab.data(), h->noalloc_tab.size() * 4,
                        hipMemcpyHostToDevice, st));
  return CLEF_OK;
}

// streamed: the row statistics, memory and K/V rows of every tile were
// computed while the rows streamed in (clef_head_stream_rows); only the rest runs.
// noalloc: run in the static scratch and allocate nothing (clef_head_forward_noalloc).
static int forward_impl(clef_head* h, const clef_head_batch* batch, float* logits, float* probs, int32_t* argmax,
                        const clef_head_answers* answers, void* hip_stream, bool streamed = false,
                        bool noalloc = false) {
  if (!h) return fail(CLEF_E_ARG, "handle is NULL");
  if (h->strm.active && !streamed)
    return fail(CLEF_E_ARG, "a streamed batch is in progress on this handle (clef_head_stream_end first)");
  const clef_head_config& c = h->cfg;
  Plan p;
  int rc = build_plan(c, batch, p, true);
  if (rc) return rc;
  if (p.NQ == 0) return CLEF_OK;
  if (!logits || !probs || !argmax) return fail(CLEF_E_ARG, "output buffer is NULL");
  int dev_prev = 0;
  HIPCHK(hipGetDevice(&dev_prev));
  if (dev_prev != h->device) HIPCHK(hipSetDevice(h->device));
  struct Restore {
    int d, p;
    ~Restore() { if (d != p) (void)hipSetDevice(p); }
  } restore{h->device, dev_prev};
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  // the workspace is the handle's: its previous work, on whatever stream, comes first
  if (h->done_recorded) HIPCHK(hipStreamWaitEvent(st, h->done, 0));

  const WsLayout L = ws_layout(c, p);
  if (streamed && L.total > h->ws_bytes) return fail(CLEF_E_ARG, "streamed batch does not fit the staged workspace");
  void* wsbase = nullptr;
  if (noalloc) {
    if (h->trace || h->prof)
      return fail(CLEF_E_ARG, "the allocation-free entry point runs with tracing and stage timing off");
    HIPCHK(noalloc_scratch(h->device, &wsbase));
    const int rc2 = stage_plan_noalloc(h, p, L, wsbase, st);
    if (rc2) return rc2;
  } else {
    const int rc2 = stage_plan(h, p, L, st);
    if (rc2) return rc2;
    wsbase = h->ws;
  }
  const int NR = c.routing_layers, NL = c.layers, NQ = p.NQ, NO = p.NO;
  const size_t H = c.hidden_size;
  if (h->trace) {
    const size_t need = align256((size_t)(NR + 1) * NO * D * 4) + 2 * align256((size_t)NQ * D * 4) + 2 * align256((size_t)NO * 4);
    if (need > h->tr_bytes) {
      if (h->done_recorded) HIPCHK(hipEventSynchronize(h->done));
      if (h->tr) (void)hipFree(h->tr);
      h->tr = nullptr;
      h->tr_bytes = 0;
      if (dev_malloc(&h->tr, need) != hipSuccess) return fail(CLEF_E_NOMEM, "trace hipMalloc failed");
      h->tr_bytes = need;
      if (g_poison.load()) launch_fill_u32(st, h->tr, need, 0xffffffffu);
    }
    uint8_t* t = static_cast<uint8_t*>(h->tr);
    h->tr_u = reinterpret_cast<float*>(t);
    t += align256((size_t)(NR + 1) * NO * D * 4);
    h->tr_f0 = reinterpret_cast<float*>(t);
    t += align256((size_t)NQ * D * 4);
    h->tr_f = reinterpret_cast<float*>(t);
    t += align256((size_t)NQ * D * 4);
    h->tr_jcos = reinterpret_cast<float*>(t);
    t += align256((size_t)NO * 4);
    h->tr_mlp = reinterpret_cast<float*>(t);
  }

  uint8_t* ws = static_cast<uint8_t*>(wsbase);
  int32_t* dtab = reinterpret_cast<int32_t*>(ws + L.tab);

  const int* rec = dtab + p.off_rec;
  const int4* tiles = reinterpret_cast<const int4*>(dtab + p.off_tiles);
  const int4* kvtiles = reinterpret_cast<const int4*>(dtab + p.off_kvtiles);
  const int4* pool = reinterpret_cast<const int4*>(dtab + p.off_pool);
  const int4* lex = reinterpret_cast<const int4*>(dtab + p.off_lex);
  const int* ids = dtab + p.off_ids;
  const int* optq = dtab + p.off_optq;
  const int* optrec = dtab + p.off_optrec;
  const int* qrec = dtab + p.off_qrec;
  const int* qtype = dtab + p.off_qtype;
  const AnswerOut ans = answers ? AnswerOut{answers->value, answers->confidence, answers->value_4dp,
                                            answers->confidence_4dp, answers->probs_4dp}
                                : AnswerOut{nullptr, nullptr, nullptr, nullptr, nullptr};
  const int* ooff = dtab + p.off_ooff;
  const int4* items = reinterpret_cast<const int4*>(dtab + p.off_items);
  const int* frec = dtab + p.off_frec;
  const int4* fitems = reinterpret_cast<const int4*>(dtab + p.off_fitems);

  float2* stats = reinterpret_cast<float2*>(ws + L.stats);
  float* pooled = reinterpret_cast<float*>(ws + L.pooled);
  float* ebar = reinterpret_cast<float*>(ws + L.ebar);
  float* prior = reinterpret_cast<float*>(ws + L.prior);
  bf16_t* mem = reinterpret_cast<bf16_t*>(ws + L.mem);
  bf16_t* kv = reinterpret_cast<bf16_t*>(ws + L.kv);
  bf16_t* fkv = reinterpret_cast<bf16_t*>(ws + L.fkv);
  float* bigpart = reinterpret_cast<float*>(ws + L.bigpart);
  float* u = reinterpret_cast<float*>(ws + L.u);
  float2* ustats = reinterpret_cast<float2*>(ws + L.ustats);
  float* qbuf = reinterpret_cast<float*>(ws + L.qbuf);
  float* attn = reinterpret_cast<float*>(ws + L.attn);
  float* hbuf = reinterpret_cast<float*>(ws + L.hbuf);
  float* qv = reinterpret_cast<float*>(ws + L.qv);
  float* qo = reinterpret_cast<float*>(ws + L.qo);
  float* gp = reinterpret_cast<float*>(ws + L.gp);
  float* f = reinterpret_cast<float*>(ws + L.f);
  float2* fstats = reinterpret_cast<float2*>(ws + L.fstats);
  float* fattn = reinterpret_cast<float*>(ws + L.fattn);
  float* opart = reinterpret_cast<float*>(ws + L.opart);
  float* pm = reinterpret_cast<float*>(ws + L.pm);
  float* pl = reinterpret_cast<float*>(ws + L.pl);
  float* po = reinterpret_cast<float*>(ws + L.po);
  float* part = reinterpret_cast<float*>(ws + L.part);
  const bf16_t* X = static_cast<const bf16_t*>(batch->hidden);
  const Weights& W = h->w;
  const float eps = c.ln_eps;
  const bool joint = W.gate != 0.0f;
  const bool cross = c.field_cross_attention && NL > 0;   // decoder-layer field variant
  // precision mode fp32: memory rows and K/V in fp32, every small GEMM's activations as 3 exact bf16 terms
  const bool f32 = c.precision == CLEF_PRECISION_F32;
  const int NT = f32 ? 3 : 2;
  float* mem32 = reinterpret_cast<float*>(ws + L.mem);
  float* kv32 = reinterpret_cast<float*>(ws + L.kv);
  float* fkv32 = reinterpret_cast<float*>(ws + L.fkv);

  // stage timing: an event at every stage boundary, on the forward's stream
  std::vector<int> marks;
  auto mark = [&](int stage) -> int {
    if (!h->prof) return CLEF_OK;
    if (h->ev.size() <= marks.size()) {
      hipEvent_t e;
      HIPCHK(hipEventCreate(&e));
      h->ev.push_back(e);
    }
    HIPCHK(hipEventRecord(h->ev[marks.size()], st));
    marks.push_back(stage);
    return CLEF_OK;
  };
#define MARK(s) do { int rc_ = mark(s); if (rc_) return rc_; } while (0)
  MARK(-1);

  // The option-query chain (pooling, lexical prior, query / question / global
  // projections, the first routing layer's query projection) does not depend on
  // the memory and K/V GEMMs: it runs on a second stream, forked after the row
  // statistics and joined before the first routing attention, so its small
  // kernels fill the CUs the big GEMMs leave idle.  Stage timing runs serially.
  const bool fork = !h->prof;
  hipStream_t s2 = fork ? h->side.get() : st;

  // step 1: row statistics, pooled vectors, lexical vectors and prior
  if (!streamed) launch_rowstats(st, X, (int)H, p.f16, tiles, p.ntiles, stats, eps);
  MARK(CLEF_STAGE_ROWSTATS);
  if (fork) {
    HIPCHK(hipEventRecord(h->ev_fork, st));
    HIPCHK(hipStreamWaitEvent(s2, h->ev_fork, 0));
  }
  launch_pool(s2, X, (int)H, p.f16, pool, p.npool, stats, W.lnin_g, W.lnin_b, pooled);
  MARK(CLEF_STAGE_POOL);
  launch_lex_prior(s2, h->table, (int)H, lex, NO, ids, pooled, ebar, prior);
  MARK(CLEF_STAGE_LEXICAL);

  if (joint) {
    // step 2: memory and K/V of every routing layer (main stream), after the
    // big GEMMs of the group's previous forward
    if ((NR > 0 || cross) && !streamed) {
      HeadGroup& g = *h->group;
      if (fork) {
        std::lock_guard<std::mutex> lk(g.mu);
        if (g.recorded) HIPCHK(hipStreamWaitEvent(st, g.gemm_done, 0));
      }
      if (f32 && f32_big_gemms(p.ntiles)) {
        // memory rows: bf16 hidden rows (exact) read three times against the three bf16 terms of the folded
        // weight, LayerNorm in the epilogue; fp16 hidden rows normalised into three bf16 terms times
        // [W | W | W].  Then their three-term memory rows times Wkv read three times, into head-major fp32
        // planes
        bf16_t* xplanes = reinterpret_cast<bf16_t*>(ws + L.xplanes);
        bf16_t* mplanes = reinterpret_cast<bf16_t*>(ws + L.mplanes);
        float* mrows = h->trace ? mem32 : nullptr;   // the fp32 rows are read by the memory trace only
        if (p.f16) {
          launch_ln_split3(st, X, (int)H, p.f16, tiles, p.ntiles, stats, W.lnin_g, W.lnin_b, xplanes);
          launch_gemm_mem32(st, xplanes, (int)H, kvtiles, p.ntiles, W.Wmem3, W.bmem, mrows, mplanes);
        } else {
          launch_gemm_mem32_folded(st, X, (int)H, tiles, p.ntiles, W.Wmem3f, stats, W.cmem32, W.dmem, mrows,
                                   mplanes);
        }
        MARK(CLEF_STAGE_MEMORY_GEMM);
        if (NR > 0) launch_gemm_kv32(st, mplanes, kvtiles, p.ntiles, W.Wkv, W.bkv, NR, kv32, p.Tpad);
        if (cross) launch_gemm_kv32(st, mplanes, kvtiles, p.ntiles, W.Wfkv, W.bfkv, NL, fkv32, p.Tpad);
        MARK(CLEF_STAGE_KV_GEMM);
      } else if (f32) {
        // normalised rows times the unfolded memory weight, then K/V into head-major fp32 planes
        const int Tp = (int)p.Tpad;
        if (p.f16)
          launch_sgemm(st, LdHid<true>{X, (int)H, tiles, stats, W.lnin_g, W.lnin_b}, EpStore{mem32, D, W.bmem},
                       W.Wmem_fr, Tp, D, (int)H, bigpart, nullptr, 0.f, 3, 0);
        else
          launch_sgemm(st, LdHid<false>{X, (int)H, tiles, stats, W.lnin_g, W.lnin_b}, EpStore{mem32, D, W.bmem},
                       W.Wmem_fr, Tp, D, (int)H, bigpart, nullptr, 0.f, 3, 0);
        MARK(CLEF_STAGE_MEMORY_GEMM);
        if (NR > 0)
          launch_sgemm(st, LdRows{mem32, D, nullptr}, EpHeads{kv32, p.Tpad, W.bkv}, W.Wkv_fr, Tp, NR * 2 * D, D,
                       bigpart, nullptr, 0.f, 3, 0);
        if (cross)
          launch_sgemm(st, LdRows{mem32, D, nullptr}, EpHeads{fkv32, p.Tpad, W.bfkv}, W.Wfkv_fr, Tp, NL * 2 * D,
                       D, bigpart, nullptr, 0.f, 3, 0);
        MARK(CLEF_STAGE_KV_GEMM);
      } else {
        launch_gemm_mem(st, X, (int)H, p.f16, tiles, p.ntiles, p.f16 ? W.Wmem16 : W.Wmem, stats,
                        p.f16 ? W.cmem16 : W.cmem, W.dmem, mem, bigpart, p.Tpad);
        MARK(CLEF_STAGE_MEMORY_GEMM);
        launch_gemm_kv(st, mem, kvtiles, p.ntiles, W.Wkv, W.bkv, NR, kv, p.Tpad, bigpart);
        if (cross) launch_gemm_kv(st, mem, kvtiles, p.ntiles, W.Wfkv, W.bfkv, NL, fkv, p.Tpad, bigpart);
        MARK(CLEF_STAGE_KV_GEMM);
      }
      if (fork) {
        std::lock_guard<std::mutex> lk(g.mu);
        HIPCHK(hipEventRecord(g.gemm_done, st));
        g.recorded = true;
      }
    }
    // step 3: option queries (with the first routing LayerNorm statistics), question base and global projections
    launch_sgemm(s2, LdRows{pooled, (int)H, nullptr}, EpSplit2{qv, qo, W.bqq}, W.Wqq, NQ, 2 * D, (int)H, part,
                 nullptr, 0.f, NT);
    launch_sgemm(s2, LdSeg2{pooled + (size_t)NQ * H, ebar, (int)H}, EpAddRow{u, W.ba7, qo, optq}, W.Wa7, NO, D,
                 2 * (int)H, part, ustats, eps, NT);
    launch_sgemm(s2, LdRows{pooled + (size_t)(NQ + NO) * H, (int)H, nullptr}, EpStore{gp, D, W.bg}, W.Wg, p.nact, D,
                 (int)H, part, nullptr, 0.f, NT);
    MARK(CLEF_STAGE_QUERY_PROJ);
    if (h->trace) HIPCHK(hipMemcpyAsync(h->tr_u, u, (size_t)NO * D * 4, hipMemcpyDeviceToDevice, s2));
    if (NR > 0) {
      const Layer& Ly = W.route[0];
      launch_sgemm(s2, LdLN{u, D, ustats, Ly.ln1g, Ly.ln1b}, EpStore{qbuf, D, Ly.bq}, Ly.Wq, NO, D, D, part,
                   nullptr, 0.f, NT);
      MARK(CLEF_STAGE_ROUTE_DENSE);
    }
  }
  if (fork) {
    HIPCHK(hipEventRecord(h->ev_join, s2));
    HIPCHK(hipStreamWaitEvent(st, h->ev_join, 0));
  }

  SgemmShape gs{};   // scoring hidden-layer slices (joint branch only)
  gs.nsplit = 1;
  if (joint) {
    for (int r = 0; r < NR; ++r) {
      const Layer& Ly = W.route[r];
      const size_t plane = (size_t)NH * p.Tpad * 64;   // elements of one layer's K (or V), all heads
      if (r > 0) {
        launch_sgemm(st, LdLN{u, D, ustats, Ly.ln1g, Ly.ln1b}, EpStore{qbuf, D, Ly.bq}, Ly.Wq, NO, D, D, part,
                     nullptr, 0.f, NT);
        MARK(CLEF_STAGE_ROUTE_DENSE);
      }
      if (f32)
        launch_route_attn32(st, qbuf, kv32 + (2 * r) * plane, kv32 + (2 * r + 1) * plane, p.Tpad, items, p.nitems,
                            rec, pm, pl, po, p.Ptot, p.kchunk);
      else
        launch_route_attn(st, qbuf, kv + (2 * r) * plane, kv + (2 * r + 1) * plane, p.Tpad, items, p.nitems, rec,
                          pm, pl, po, p.Ptot, p.kchunk);
      launch_route_combine(st, pm, pl, po, p.Ptot, optrec, rec, NO, attn);
      MARK(CLEF_STAGE_ROUTE_ATTN);
      launch_sgemm(st, LdRows{attn, D, nullptr}, EpResid{u, D, Ly.bo}, Ly.Wo, NO, D, D, part, ustats, eps, NT);
      launch_sgemm(st, LdLN{u, D, ustats, Ly.ln2g, Ly.ln2b}, EpGelu{hbuf, F, Ly.b1}, Ly.W1, NO, F, D, part, nullptr,
                   0.f, NT);
      launch_sgemm(st, LdRows{hbuf, F, nullptr}, EpResid{u, D, Ly.b2}, Ly.W2, NO, D, F, part,
                   r + 1 < NR ? ustats : nullptr, eps, NT);
      MARK(CLEF_STAGE_ROUTE_DENSE);
      if (h->trace)
        HIPCHK(hipMemcpyAsync(h->tr_u + (size_t)(r + 1) * NO * D, u, (size_t)NO * D * 4, hipMemcpyDeviceToDevice, st));
    }
    // step 4: field vectors (with the first field LayerNorm statistics) and the field transformer
    launch_field_agg(st, u, ooff, W.sw, W.sb, qv, gp, qrec, qtype, W.temb, NQ, f, fstats, eps);
    if (h->trace) HIPCHK(hipMemcpyAsync(h->tr_f0, f, (size_t)NQ * D * 4, hipMemcpyDeviceToDevice, st));
    for (int l = 0; l < NL; ++l) {
      const Layer& Ly = W.field[l];
      const SgemmShape gq =
          launch_sgemm_partial(st, LdLN{f, D, fstats, Ly.ln1g, Ly.ln1b}, Ly.Wqkv, NQ, 3 * D, D, part, NT);
      const size_t Mq = (size_t)ceil_div(NQ, kSgemmRows) * kSgemmRows;
      launch_field_attn(st, part, gq.nsplit, (size_t)gq.mtiles * kSgemmRows * 3 * D, Ly.bqkv, rec, p.nact, Ly.Wo,
                        opart, Mq * D, NT);
      launch_splitk_reduce(st, opart, NH, Mq, NQ, D, EpResid{f, D, Ly.bo}, fstats, eps);
      if (cross) {
        // cross-attention of the fields over the record's memory rows (the routing attention kernels with
        // the fields as queries), pre-LN, residual
        const size_t plane = (size_t)NH * p.Tpad * 64;
        launch_sgemm(st, LdLN{f, D, fstats, Ly.xlng, Ly.xlnb}, EpStore{qbuf, D, Ly.bxq}, Ly.Wxq, NQ, D, D, part,
                     nullptr, 0.f, NT);
        if (f32)
          launch_route_attn32(st, qbuf, fkv32 + (2 * l) * plane, fkv32 + (2 * l + 1) * plane, p.Tpad, fitems,
                              p.nfitems, frec, pm, pl, po, p.Ptot_f, p.kchunk);
        else
          launch_route_attn(st, qbuf, fkv + (2 * l) * plane, fkv + (2 * l + 1) * plane, p.Tpad, fitems, p.nfitems,
                            frec, pm, pl, po, p.Ptot_f, p.kchunk);
        launch_route_combine(st, pm, pl, po, p.Ptot_f, qrec, frec, NQ, fattn);
        launch_sgemm(st, LdRows{fattn, D, nullptr}, EpResid{f, D, Ly.bxo}, Ly.Wxo, NQ, D, D, part, fstats, eps, NT);
      }
      launch_sgemm(st, LdLN{f, D, fstats, Ly.ln2g, Ly.ln2b}, EpGelu{hbuf, F, Ly.b1}, Ly.W1, NQ, F, D, part, nullptr,
                   0.f, NT);
      launch_sgemm(st, LdRows{hbuf, F, nullptr}, EpResid{f, D, Ly.b2}, Ly.W2, NQ, D, F, part,
                   l + 1 < NL ? fstats : nullptr, eps, NT);
    }
    MARK(CLEF_STAGE_FIELD);
    if (h->trace) HIPCHK(hipMemcpyAsync(h->tr_f, f, (size_t)NQ * D * 4, hipMemcpyDeviceToDevice, st));
    // step 5: residual-MLP hidden layer over [f, u, f*u, |f-u|]
    gs = launch_sgemm_partial(st, LdZ{f, u, optq}, W.Ws1, NO, D, 4 * D, part, NT);
  }
  launch_score(st, u, f, part, gs.nsplit, (size_t)gs.mtiles * kSgemmRows * D, W.bs1, W.ws2, W.bs2, prior, W.gate,
               W.lam, joint ? 1 : 0, ooff, NQ, logits, probs, argmax,
               h->trace && joint ? h->tr_jcos : nullptr, h->trace && joint ? h->tr_mlp : nullptr, qtype, ans);
  MARK(CLEF_STAGE_SCORE);
#undef MARK
  HIPCHK(hipGetLastError());
  HIPCHK(hipEventRecord(h->done, st));
  h->done_recorded = true;
  if (h->prof) {
    HIPCHK(hipEventSynchronize(h->ev[marks.size() - 1]));
    for (size_t i = 1; i < marks.size(); ++i) {
      float ms = 0.f;
      HIPCHK(hipEventElapsedTime(&ms, h->ev[i - 1], h->ev[i]));
      h->stage_ms[marks[i]] += ms;
    }
    ++h->prof_calls;
  }

  h->last_stream = st;
  h->last_NQ = NQ;
  h->last_NO = NO;
  h->last_B = p.nact;
  h->last_Tpad = p.Tpad;
  h->pooled = noalloc ? nullptr : pooled;   // no snapshots of the shared scratch
  h->tr_tab = dtab;
  h->tr_off_pool = p.off_pool;
  h->tr_off_lex = p.off_lex;
  h->tr_off_ids = p.off_ids;
  h->tr_npool = p.npool;
  h->tr_nlex = NO;
  h->tr_nids = p.nids;
  h->ebar = ebar;
  h->prior = prior;
  h->mem = (joint && NR > 0) ? mem : nullptr;
  if (!h->trace || !joint) {
    h->tr_u = h->tr_f0 = h->tr_f = h->tr_jcos = h->tr_mlp = nullptr;
  }
  return CLEF_OK;
}

int clef_head_forward(clef_head* h, const clef_head_batch* batch, float* logits, float* probs, int32_t* argmax,
                      void* hip_stream) {
  return forward_impl(h, batch, logits, probs, argmax, nullptr, hip_stream);
}

int clef_head_forward_answers(clef_head* h, const clef_head_batch* batch, float* logits, float* probs,
                              int32_t* argmax, const clef_head_answers* answers, void* hip_stream) {
  if (!answers) return fail(CLEF_E_ARG, "answers is NULL");
  return forward_impl(h, batch, logits, probs, argmax, answers, hip_stream);
}

int clef_head_forward_noalloc(clef_head* h, const clef_head_batch* batch, float* logits, float* probs,
                              int32_t* argmax, void* hip_stream) {
  return forward_impl(h, batch, logits, probs, argmax, nullptr, hip_stream, false, true);
}

// ---------------------------------------------------------------------------
// Streamed ingest.  The batch is planned exactly as clef_head_forward plans its
// varlen form; rows are copied into handle-owned staging rows as they arrive,
// and each 256-row tile's row statistics, memory rows and K/V rows are
// computed as soon as the tile's last row is in, with the same kernels and the
// same K split as the whole-batch launch, so the result is bit-identical to
// clef_head_forward over the same rows.
// ---------------------------------------------------------------------------
static int stream_plan(clef_head* h, const clef_head_batch* batch, Plan& p) {
  if (!batch) return fail(CLEF_E_ARG, "batch is NULL");
  if ((batch->layout & ~CLEF_HIDDEN_F16) != CLEF_VARLEN)
    return fail(CLEF_E_ARG, "a streamed batch uses the CLEF_VARLEN layout (cu_seqlens)");
  clef_head_batch b = *batch;
  b.hidden = h->strm.rows ? h->strm.rows : reinterpret_cast<const void*>(&h->strm);   // placeholder until staged
  return build_plan(h->cfg, &b, p, true);
}

int clef_head_stream_begin(clef_head* h, const clef_head_batch* batch, void* hip_stream) {
  if (!h) return fail(CLEF_E_ARG, "handle is NULL");
  if (h->strm.active) return fail(CLEF_E_ARG, "a streamed batch is already in progress on this handle");
  if (h->cfg.precision == CLEF_PRECISION_F32)
    return fail(CLEF_E_UNSUPPORTED, "streamed ingest runs in the bf16 precision mode only");
  Plan p;
  int rc = stream_plan(h, batch, p);
  if (rc) return rc;
  int dev_prev = 0;
  HIPCHK(hipGetDevice(&dev_prev));
  if (dev_prev != h->device) HIPCHK(hipSetDevice(h->device));
  struct Restore {
    int d, p;
    ~Restore() { if (d != p) (void)hipSetDevice(p); }
  } restore{h->device, dev_prev};
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  auto& S = h->strm;
  const int B = batch->num_records;
  const size_t H = h->cfg.hidden_size;
  const size_t need = (size_t)std::max<int64_t>(batch->cu_seqlens[B], 1) * H * 2;
  if (need > S.rows_bytes) {
    if (h->done_recorded) HIPCHK(hipEventSynchronize(h->done));
    if (S.rows) (void)hipFree(S.rows);
    S.rows = nullptr;
    S.rows_bytes = 0;
    if (dev_malloc(&S.rows, need) != hipSuccess) return fail(CLEF_E_NOMEM, "staging rows hipMalloc of %zu bytes failed", need);
    S.rows_bytes = need;
    if (g_poison.load()) launch_fill_u32(st, S.rows, need, 0xffffffffu);
  }
  const WsLayout L = ws_layout(h->cfg, p);
  rc = stage_plan(h, p, L, st);
  if (rc) return rc;
  S.tab = p.tab;
  S.cu.assign(batch->cu_seqlens, batch->cu_seqlens + B + 1);
  S.len.resize(B);
  for (int r = 0; r < B; ++r) S.len[r] = (int32_t)(S.cu[r + 1] - S.cu[r]);
  S.received.assign(B, 0);
  S.rec_tiles.assign(B, {});
  const int4* tl = reinterpret_cast<const int4*>(p.tab.data() + p.off_tiles);
  for (int i = 0, r = 0; i < p.ntiles; ++i) {   // tiles run in record order; .x is the first staging row
    while (tl[i].x >= S.cu[r + 1]) ++r;
    S.rec_tiles[r].push_back(i);
  }
  S.ntiles = p.ntiles;
  S.off_tiles = p.off_tiles;
  S.off_kvtiles = p.off_kvtiles;
  S.ws_tab = L.tab;
  S.ws_stats = L.stats;
  S.ws_mem = L.mem;
  S.ws_kv = L.kv;
  S.ws_bigpart = L.bigpart;
  S.Tpad = p.Tpad;
  S.f16 = p.f16;
  S.cross = h->cfg.field_cross_attention && h->cfg.layers > 0;
  S.gemms = h->w.gate != 0.0f && (h->cfg.routing_layers > 0 || S.cross);
  S.split_mem = big_gemm_split(p.ntiles, D / 256, (int)H);
  S.split_kv = big_gemm_split(p.ntiles, h->cfg.routing_layers * 8, D);
  S.split_fkv = big_gemm_split(p.ntiles, (S.cross ? h->cfg.layers : 0) * 8, D);
  S.ws_fkv = L.fkv;
  S.active = true;
  return CLEF_OK;
}

int clef_head_stream_rows(clef_head* h, int32_t record, int32_t row0, int32_t nrows, const void* rows,
                          void* hip_stream) {
  if (!h) return fail(CLEF_E_ARG, "handle is NULL");
  auto& S = h->strm;
  if (!S.active) return fail(CLEF_E_ARG, "no streamed batch in progress (clef_head_stream_begin first)");
  if (record < 0 || record >= (int32_t)S.len.size()) return fail(CLEF_E_ARG, "record %d out of range", record);
  if (nrows < 1 || !rows) return fail(CLEF_E_ARG, "empty chunk or NULL rows");
  if (row0 != S.received[record])
    return fail(CLEF_E_ARG, "record %d: chunk starts at row %d, %d rows received so far (rows arrive in order)", record,
                row0, S.received[record]);
  if ((int64_t)row0 + nrows > S.len[record])
    return fail(CLEF_E_LENGTH, "record %d: rows [%d, %d) past its length %d", record, row0, row0 + nrows,
                S.len[record]);
  int dev_prev = 0;
  HIPCHK(hipGetDevice(&dev_prev));
  if (dev_prev != h->device) HIPCHK(hipSetDevice(h->device));
  struct Restore {
    int d, p;
    ~Restore() { if (d != p) (void)hipSetDevice(p); }
  } restore{h->device, dev_prev};
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (h->done_recorded) HIPCHK(hipStreamWaitEvent(st, h->done, 0));
  const size_t H = h->cfg.hidden_size;
  const auto& tl = S.rec_tiles[record];
  if (!tl.empty()) {   // records without questions take no tiles: their rows are never read
    bf16_t* X = static_cast<bf16_t*>(S.rows);
    HIPCHK(hipMemcpyAsync(X + (size_t)(S.cu[record] + row0) * H, rows, (size_t)nrows * H * 2,
                          hipMemcpyDeviceToDevice, st));
  }
  const int32_t before = S.received[record];
  S.received[record] += nrows;
  // tiles of this record completed by the chunk: tile j holds rows [256 j, min(256 (j + 1), n))
  if (tl.empty()) {
    HIPCHK(hipEventRecord(h->done, st));
    h->done_recorded = true;
    return CLEF_OK;
  }
  const int n = S.len[record];
  uint8_t* ws = static_cast<uint8_t*>(h->ws);
  const int4* htiles = reinterpret_cast<const int4*>(S.tab.data() + S.off_tiles);
  const int4* dtiles = reinterpret_cast<const int4*>(ws + S.ws_tab + S.off_tiles * 4);
  const int4* dkvtiles = reinterpret_cast<const int4*>(ws + S.ws_tab + S.off_kvtiles * 4);
  float2* stats = reinterpret_cast<float2*>(ws + S.ws_stats);
  bf16_t* mem = reinterpret_cast<bf16_t*>(ws + S.ws_mem);
  bf16_t* kv = reinterpret_cast<bf16_t*>(ws + S.ws_kv);
  float* bigpart = reinterpret_cast<float*>(ws + S.ws_bigpart);
  const bf16_t* X = static_cast<const bf16_t*>(S.rows);
  const Weights& W = h->w;
  for (int j = before / 256; j < (int)tl.size(); ++j) {
    const int end = std::min(256 * (j + 1), n);
    if (S.received[record] < end) break;
    if (before >= end) continue;   // completed by an earlier chunk
    const int i = tl[j];
    const long long prow = htiles[i].y;
    launch_rowstats(st, X, (int)H, S.f16, dtiles + i, 1, stats, h->cfg.ln_eps);
    if (S.gemms) {
      launch_gemm_mem(st, X, (int)H, S.f16, dtiles + i, 1, S.f16 ? W.Wmem16 : W.Wmem, stats,
                      S.f16 ? W.cmem16 : W.cmem, W.dmem, mem, bigpart, S.Tpad, S.split_mem, prow);
      launch_gemm_kv(st, mem, dkvtiles + i, 1, W.Wkv, W.bkv, h->cfg.routing_layers, kv, S.Tpad, bigpart, S.split_kv,
                     prow);
      if (S.cross)
        launch_gemm_kv(st, mem, dkvtiles + i, 1, W.Wfkv, W.bfkv, h->cfg.layers,
                       reinterpret_cast<bf16_t*>(ws + S.ws_fkv), S.Tpad, bigpart, S.split_fkv, prow);
    }
  }
  HIPCHK(hipGetLastError());
  HIPCHK(hipEventRecord(h->done, st));
  h->done_recorded = true;
  return CLEF_OK;
}

int clef_head_stream_end(clef_head* h, const clef_head_batch* batch, float* logits, float* probs, int32_t* argmax,
                         const clef_head_answers* answers, void* hip_stream) {
  if (!h) return fail(CLEF_E_ARG, "handle is NULL");
  auto& S = h->strm;
  if (!S.active) return fail(CLEF_E_ARG, "no streamed batch in progress (clef_head_stream_begin first)");
  for (size_t r = 0; r < S.len.size(); ++r)
    if (S.received[r] != S.len[r])
      return fail(CLEF_E_LENGTH, "record %zu: %d of %d rows received", r, S.received[r], S.len[r]);
  Plan p;
  int rc = stream_plan(h, batch, p);
  if (rc) return rc;
  if (p.tab != S.tab) return fail(CLEF_E_ARG, "the batch differs from the one clef_head_stream_begin planned");
  clef_head_batch b = *batch;
  b.hidden = S.rows;
  rc = forward_impl(h, &b, logits, probs, argmax, answers, hip_stream, true);
  if (rc == CLEF_OK) S.active = false;
  return rc;
}

int clef_head_stream_cancel(clef_head* h) {
  if (!h) return fail(CLEF_E_ARG, "handle is NULL");
  h->strm.active = false;
  return CLEF_OK;
}

}  // extern "C"
