// Internal launch interface between the host library and the gfx950 kernels.
#pragma once
#include "common.hpp"

namespace clef {

constexpr int kMaxOptions = 1024;   // options of one question (LDS arrays in the per-question kernels)

// Static scratch of the allocation-free entry point: its size, and the device
// address of the array on `device` (which must be the current device; looked
// up on the first call per device).
constexpr size_t kNoallocScratchBytes = size_t(256) << 20;
hipError_t noalloc_scratch(int device, void** out);

// Position of key k (0..31) inside a 32-key V block: the eight keys one lane
// feeds to a V^T P^T MFMA step sit in 16 contiguous bytes.
DEV int vblock_pos(int k) { return (k & 16) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3); }

// fp32 head: K and V of one head are planes of Tpad keys x 64 dims, stored in
// blocks of 32 keys (2048 floats) in the order of the fp32 routing attention's
// v_mfma_f32_32x32x2_f32 fragments, so that each fragment load of a wave reads
// 1 KB of contiguous memory.  K (A operand of S^T = K Q^T, call i covers dims
// 2 i and 2 i + 1): lane l reads dims d with d % 2 = l / 32 of key l % 32, in
// float4 groups of consecutive d / 2.  V (A operand of O^T = V^T P^T, call i
// covers keys 8 (i / 4) + (i % 4) and that + 4, the order of the score
// accumulators): lane l reads dim 32 dt + l % 32 at keys with (k / 4) % 2 = l / 32.
DEV size_t k32_off(int key, int d) {
  const int idx = d >> 1;
  return (size_t)(key >> 5) * 2048 + ((((idx >> 2) * 2 + (d & 1)) * 32 + (key & 31)) << 2) + (idx & 3);
}
DEV size_t v32_off(int key, int d) {
  const int k = key & 31;
  return (size_t)(key >> 5) * 2048 + (((((d >> 5) * 4 + (k >> 3)) * 2 + ((k >> 2) & 1)) * 32 + (d & 31)) << 2) + (k & 3);
}

// Fill `bytes` (a multiple of 4) at p with the 32-bit pattern v (a kernel, so
// that it can sit in a captured graph; used to poison fresh working memory).
void launch_fill_u32(hipStream_t, void* p, size_t bytes, uint32_t v);

// ---------------------------------------------------------------------------
// row kernels
// ---------------------------------------------------------------------------
// X holds 16-bit hidden elements: bf16, or fp16 when f16 is set.
// tiles: int4 (first hidden row, first packed row, valid rows <= 256, record)
void launch_rowstats(hipStream_t, const bf16_t* X, int H, bool f16, const int4* tiles, int ntiles, float2* stats,
                     float eps);
// fp32 head: LayerNorm-ed rows of every tile's valid rows as three bf16 terms,
// planes[t.y + r][p * H + k]
void launch_ln_split3(hipStream_t, const bf16_t* X, int H, bool f16, const int4* tiles, int ntiles,
                      const float2* stats, const float* gamma, const float* beta, bf16_t* planes);
// entries: int4 (first hidden row, length, first stats row, output slot)
void launch_pool(hipStream_t, const bf16_t* X, int H, bool f16, const int4* ent, int nent, const float2* stats,
                 const float* gamma, const float* beta, float* out);
// entries: int4 (first id, count, question slot, global slot)
void launch_lex_prior(hipStream_t, const bf16_t* E, int H, const int4* ent, int nent, const int* ids,
                      const float* pooled, float* ebar, float* prior);

// ---------------------------------------------------------------------------
// big GEMMs (rows of the packed row space)
// ---------------------------------------------------------------------------
// Number of K slices (1 = no split) for a big GEMM of ntiles row tiles x ntn
// 256-column tiles over depth K: a batch of few row tiles leaves most CUs
// idle, so its K is split until about 256 workgroups run (at most 8 slices,
// each at least 256 deep).  The slices' fp32 partial sums need
// split * Tpad * N floats of workspace.
int big_gemm_split(int ntiles, int ntn, int K);
// f16: hidden and Wm are fp16 (fp16 MFMA), else both bf16.  part: split-K
// workspace (null: never split); Tpad: rows of the packed row space (the
// partial sums of slice s start at row s * Tpad).  split > 0 forces that
// many slices (a launch over some of a batch's tiles that must sum like the
// whole batch's launch); row0: first packed row of the launch's tiles, which
// must be consecutive.
void launch_gemm_mem(hipStream_t, const bf16_t* hidden, int H, bool f16, const int4* tiles, int ntiles,
                     const bf16_t* Wm, const float2* stats, const float* c, const float* d, bf16_t* mem,
                     float* part, long long Tpad, int split = 0, long long row0 = 0);
// fp32 head: the memory product over the LayerNorm-ed rows' three bf16 terms
// (xplanes [rows][3 H], rows in the packed row space, tiles with first A row =
// first packed row) against Wm3 = [W | W | W] ([1024][3 H]); writes fp32 rows
// mem [rows][1024] (skipped when mem is null) and their three bf16 terms
// mplanes [rows][3 x 1024].  The
// K/V product over mplanes against the stacked Wkv ([N][1024], read once per
// term) writes fp32 head-major planes ([layer][K|V][head][Tpad][64], 32-row
// blocks in k32_off / v32_off order).  Whole-K launches.
void launch_gemm_mem32(hipStream_t, const bf16_t* xplanes, int H, const int4* tiles, int ntiles, const bf16_t* Wm3,
                       const float* bias, float* mem, bf16_t* mplanes);
void launch_gemm_kv32(hipStream_t, const bf16_t* mplanes, const int4* tiles, int ntiles, const bf16_t* Wkv,
                      const float* bias, int n_layers, float* kv, long long Tpad);
// fp32 head over bf16 hidden rows (exact in bf16): the raw rows (tiles as in
// launch_gemm_mem) read three times against Wt3 = the three bf16 terms of
// fp32(W diag(gamma)) ([1024][3 H]), LayerNorm folded in the epilogue
// (m = rstd (acc - mu c) + d, c_j the sum of row j's fp32 weights); writes mem
// and mplanes as launch_gemm_mem32 does.
void launch_gemm_mem32_folded(hipStream_t, const bf16_t* hidden, int H, const int4* tiles, int ntiles,
                              const bf16_t* Wt3, const float2* stats, const float* c, const float* d, float* mem,
                              bf16_t* mplanes);
void launch_gemm_kv(hipStream_t, const bf16_t* mem, const int4* tiles, int ntiles, const bf16_t* Wkv,
                    const float* bkv, int n_layers, bf16_t* kv, long long Tpad, float* part, int split = 0,
                    long long row0 = 0);

// ---------------------------------------------------------------------------
// small GEMMs: C[M, N] = A[M, K] W[N, K]^T, A formed by a loader, C by an epilogue
// ---------------------------------------------------------------------------
// A loaders: row() resolves, once per row before the K loop, whatever a row
// needs that does not depend on k (its address, gathered index, statistics);
// fetch() issues the global loads of 8 consecutive A elements (that row,
// columns k..k+7) into a Raw value; cst() issues the loads of any per-column
// constants of those 8 columns (the same for every row a thread handles);
// finish() turns them into floats.  Splitting the steps lets the GEMM keep
// the next chunk's loads in flight while it multiplies the current one, with
// no load left to wait for in finish() and no dependent load in fetch().
DEV void f4x2(float4 a, float4 b, float* x) {
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

struct LdRows {          // A[m] = src[rows ? rows[m] : m]
  const float* src;
  int ld;
  const int* rows;
  struct Raw { float4 a, b; };
  struct Cst {};
  struct Row { const float* p; };
  DEV Row row(int m) const { return Row{src + (size_t)(rows ? rows[m] : m) * ld}; }
  DEV Raw fetch(const Row& w, int k) const {
    const float* p = w.p + k;
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  DEV Cst cst(int) const { return {}; }
  DEV void finish(const Raw& r, const Cst&, int, int, float* x) const { f4x2(r.a, r.b, x); }
};

struct LdLN {            // A[m] = LayerNorm(src[m]) with precomputed (mu, rstd)
  const float* src;
  int ld;
  const float2* stats;
  const float* g;
  const float* b;
  struct Raw { float4 a, c; float2 s; };
  struct Cst { float4 g0, g1, b0, b1; };   // gamma and beta of the 8 columns
  struct Row { const float* p; float2 s; };
  DEV Row row(int m) const { return Row{src + (size_t)m * ld, stats[m]}; }
  DEV Raw fetch(const Row& w, int k) const {
    const float* p = w.p + k;
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4), w.s};
  }
  DEV Cst cst(int k) const {
    return Cst{*reinterpret_cast<const float4*>(g + k), *reinterpret_cast<const float4*>(g + k + 4),
               *reinterpret_cast<const float4*>(b + k), *reinterpret_cast<const float4*>(b + k + 4)};
  }
  DEV void finish(const Raw& r, const Cst& c, int, int, float* x) const {
    float v[8], gg[8], bb[8];
    f4x2(r.a, r.c, v);
    f4x2(c.g0, c.g1, gg);
    f4x2(c.b0, c.b1, bb);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (v[i] - r.s.x) * r.s.y * gg[i] + bb[i];
  }
};

// A[m] = LayerNorm(hidden row of packed row m) (precision mode fp32: the
// memory projection multiplies normalised rows, with nothing folded into the
// weights).  The packed row space is cut into 256-row tiles, tiles[m / 256] =
// (first hidden row, first packed row, valid rows, record); rows past a tile's
// valid count are never read and enter as zeros (their statistics are (0, 0)).
template <bool F16>
struct LdHid {
  const bf16_t* X;
  int H;
  const int4* tiles;
  const float2* stats;
  const float* g;
  const float* b;
  struct Raw { uint4 v; float2 s; };
  struct Cst { float4 g0, g1, b0, b1; };
  struct Row { const bf16_t* p; float2 s; };   // p null: a padding row (zeros)
  DEV Row row(int m) const {
    const int4 t = tiles[m >> 8];
    const int r = m & 255;
    return Row{r < t.z ? X + (size_t)(t.x + r) * H : nullptr, stats[m]};
  }
  DEV Raw fetch(const Row& w, int k) const {
    Raw raw;
    raw.s = w.s;
    raw.v = w.p ? *reinterpret_cast<const uint4*>(w.p + k) : make_uint4(0u, 0u, 0u, 0u);
    return raw;
  }
  DEV Cst cst(int k) const {
    return Cst{*reinterpret_cast<const float4*>(g + k), *reinterpret_cast<const float4*>(g + k + 4),
               *reinterpret_cast<const float4*>(b + k), *reinterpret_cast<const float4*>(b + k + 4)};
  }
  DEV void finish(const Raw& r, const Cst& c, int, int, float* x) const {
    float v[8], gg[8], bb[8];
    unpack8_hidden<F16>(r.v, v);
    f4x2(c.g0, c.g1, gg);
    f4x2(c.b0, c.b1, bb);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (v[i] - r.s.x) * r.s.y * gg[i] + bb[i];
  }
};

struct LdSeg2 {          // A[m] = [p0[m] | p1[m]], each H wide
  const float* p0;
  const float* p1;
  int H;
  struct Raw { float4 a, b; };
  struct Cst {};
  struct Row { size_t off; };
  DEV Row row(int m) const { return Row{(size_t)m * H}; }
  DEV Raw fetch(const Row& w, int k) const {
    const float* p = k < H ? p0 + w.off + k : p1 + w.off + (k - H);
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  DEV Cst cst(int) const { return {}; }
  DEV void finish(const Raw& r, const Cst&, int, int, float* x) const { f4x2(r.a, r.b, x); }
};

struct LdZ {             // A[m] = [f | u | f*u | |f-u|], f = F[fq[m]], u = U[m], each 1024 wide
  const float* F;
  const float* U;
  const int* fq;
  struct Raw { float4 f0, f1, u0, u1; };
  struct Cst {};
  struct Row { const float* f; const float* u; };
  DEV Cst cst(int) const { return {}; }
  DEV Row row(int m) const { return Row{F + (size_t)fq[m] * 1024, U + (size_t)m * 1024}; }
  // only the operands of k's segment (the same for a whole 128-deep chunk)
  DEV Raw fetch(const Row& w, int k) const {
    const int seg = k >> 10, c = k & 1023;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    Raw r{z, z, z, z};
    if (seg != 1) {
      r.f0 = *reinterpret_cast<const float4*>(w.f + c);
      r.f1 = *reinterpret_cast<const float4*>(w.f + c + 4);
    }
    if (seg != 0) {
      r.u0 = *reinterpret_cast<const float4*>(w.u + c);
      r.u1 = *reinterpret_cast<const float4*>(w.u + c + 4);
    }
    return r;
  }
  DEV void finish(const Raw& r, const Cst&, int, int k, float* x) const {
    const int seg = k >> 10;
    float f[8], u[8];
    f4x2(r.f0, r.f1, f);
    f4x2(r.u0, r.u1, u);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      x[i] = seg == 0 ? f[i] : seg == 1 ? u[i] : seg == 2 ? f[i] * u[i] : fabsf(f[i] - u[i]);
  }
};

// Epilogues store one output and return the stored value.  The reduction pass
// uses the 4-wide form: pre4() issues the loads an epilogue needs for 4
// consecutive outputs (bias, residual, gathered row) next to the slice loads,
// apply4() finishes them with one 16-byte store.
DEV float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
DEV float4 add_f4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
DEV void st_f4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

struct EpStore {         // C = acc + bias
  float* C;
  int ldc;
  const float* bias;
  DEV float operator()(int m, int n, float v) const {
    const float r = v + bias[n];
    C[(size_t)m * ldc + n] = r;
    return r;
  }
  struct Pre { float4 b; };
  DEV Pre pre4(int, int n) const { return Pre{ld_f4(bias + n)}; }
  DEV float4 apply4(int m, int n, float4 v, const Pre& p) const {
    const float4 r = add_f4(v, p.b);
    st_f4(C + (size_t)m * ldc + n, r);
    return r;
  }
};

struct EpGelu {          // C = GELU(acc + bias)
  float* C;
  int ldc;
  const float* bias;
  DEV float operator()(int m, int n, float v) const {
    const float r = gelu_erf(v + bias[n]);
    C[(size_t)m * ldc + n] = r;
    return r;
  }
  struct Pre { float4 b; };
  DEV Pre pre4(int, int n) const { return Pre{ld_f4(bias + n)}; }
  DEV float4 apply4(int m, int n, float4 v, const Pre& p) const {
    const float4 r = make_float4(gelu_erf(v.x + p.b.x), gelu_erf(v.y + p.b.y), gelu_erf(v.z + p.b.z),
                                 gelu_erf(v.w + p.b.w));
    st_f4(C + (size_t)m * ldc + n, r);
    return r;
  }
};

struct EpAddRow {        // C = acc + bias + add[idx[m]] (a per-row gathered term), width 1024
  float* C;
  const float* bias;
  const float* add;
  const int* idx;
  DEV float operator()(int m, int n, float v) const {
    const float r = v + bias[n] + add[(size_t)idx[m] * 1024 + n];
    C[(size_t)m * 1024 + n] = r;
    return r;
  }
  struct Pre { float4 b, a; };
  DEV Pre pre4(int m, int n) const { return Pre{ld_f4(bias + n), ld_f4(add + (size_t)idx[m] * 1024 + n)}; }
  DEV float4 apply4(int m, int n, float4 v, const Pre& p) const {
    const float4 r = make_float4(v.x + p.b.x + p.a.x, v.y + p.b.y + p.a.y, v.z + p.b.z + p.a.z,
                                 v.w + p.b.w + p.a.w);
    st_f4(C + (size_t)m * 1024 + n, r);
    return r;
  }
};

struct EpSplit2 {        // columns [0, 1024) -> C0, [1024, 2048) -> C1, plus bias
  float* C0;
  float* C1;
  const float* bias;
  DEV float operator()(int m, int n, float v) const {
    const float r = v + bias[n];
    if (n < 1024) C0[(size_t)m * 1024 + n] = r; else C1[(size_t)m * 1024 + (n - 1024)] = r;
    return r;
  }
  struct Pre { float4 b; };
  DEV Pre pre4(int, int n) const { return Pre{ld_f4(bias + n)}; }
  DEV float4 apply4(int m, int n, float4 v, const Pre& p) const {   // the 4 columns never straddle 1024
    const float4 r = add_f4(v, p.b);
    st_f4(n < 1024 ? C0 + (size_t)m * 1024 + n : C1 + (size_t)m * 1024 + (n - 1024), r);
    return r;
  }
};

struct EpResid {         // C += acc + bias (residual stream)
  float* C;
  int ldc;
  const float* bias;
  DEV float operator()(int m, int n, float v) const {
    float* p = C + (size_t)m * ldc + n;
    const float r = *p + (v + bias[n]);
    *p = r;
    return r;
  }
  struct Pre { float4 b, c; };
  DEV Pre pre4(int m, int n) const { return Pre{ld_f4(bias + n), ld_f4(C + (size_t)m * ldc + n)}; }
  DEV float4 apply4(int m, int n, float4 v, const Pre& p) const {
    const float4 r = make_float4(p.c.x + (v.x + p.b.x), p.c.y + (v.y + p.b.y), p.c.z + (v.z + p.b.z),
                                 p.c.w + (v.w + p.b.w));
    st_f4(C + (size_t)m * ldc + n, r);
    return r;
  }
};

struct EpHeads {         // C = acc + bias into head-major planes: columns [64 p, 64 p + 64) -> plane p of Tpad rows
  float* C;              // columns stacked [K_0 | V_0 | K_1 | V_1 | ...], 1024 each; planes in k32_off / v32_off order
  long long Tpad;
  const float* bias;
  DEV float* at(int m, int n) const {
    const int d = n & 63;
    return C + (size_t)(n >> 6) * Tpad * 64 + (((n >> 10) & 1) ? v32_off(m, d) : k32_off(m, d));
  }
  DEV float operator()(int m, int n, float v) const {
    const float r = v + bias[n];
    *at(m, n) = r;
    return r;
  }
  struct Pre { float4 b; };
  DEV Pre pre4(int, int n) const { return Pre{ld_f4(bias + n)}; }
  DEV float4 apply4(int m, int n, float4 v, const Pre& p) const {   // the 4 columns never straddle a plane
    const float4 r = add_f4(v, p.b);
    *at(m, n) = r.x;
    *at(m, n + 1) = r.y;
    *at(m, n + 2) = r.z;
    *at(m, n + 3) = r.w;
    return r;
  }
};

struct EpPart {          // C = acc (one raw split-K slice; the consumer adds the bias)
  float* C;
  int ldc;
  DEV float operator()(int m, int n, float v) const {
    C[(size_t)m * ldc + n] = v;
    return v;
  }
};

constexpr int kMaxSplit = 16;   // most K slices a small GEMM is split into
constexpr int kSgemmRows = 64;  // rows per small-GEMM tile (slice row stride is a multiple)

// Sum of the split-K slices of 4 consecutive outputs, in slice order, plus bias
// (the same order the reduction kernel uses).
DEV float4 sum_slices4(const float* p, int nsplit, size_t stride, const float* bias) {
  float4 t[kMaxSplit];
#pragma unroll
  for (int q = 0; q < kMaxSplit; ++q)
    if (q < nsplit) t[q] = *reinterpret_cast<const float4*>(p + (size_t)q * stride);
  float4 s = t[0];
#pragma unroll
  for (int q = 1; q < kMaxSplit; ++q)
    if (q < nsplit) { s.x += t[q].x; s.y += t[q].y; s.z += t[q].z; s.w += t[q].w; }
  const float4 b = *reinterpret_cast<const float4*>(bias);
  return make_float4(s.x + b.x, s.y + b.y, s.z + b.z, s.w + b.w);
}

struct SgemmShape {
  int mtiles, ntiles, kchunk, nsplit;
  int wr;                 // waves along rows: tile width 128 / wr columns
  size_t part_floats;
};
// need_reduce: always split K (>= 2 slices) so that a reduction pass runs;
// consumer_sums: the slices are summed by the consuming kernel (no reduction pass)
SgemmShape sgemm_shape(int M, int N, int K, bool need_reduce = false, bool consumer_sums = false);

// stats != nullptr (N must be 1024): the reduction pass also writes the
// LayerNorm statistics (mean, 1/sqrt(var + eps)) of every finished output row.
// nt: bf16 terms per fp32 activation (2: about 16 significant bits; 3: exact,
// the fp32 precision mode).  order: tile walk (0: row tiles of one column tile
// consecutive; 1: column tiles of one row tile consecutive).
template <class Ld, class Epi>
void launch_sgemm(hipStream_t, const Ld&, const Epi&, const bf16_t* W, int M, int N, int K, float* part,
                  float2* stats = nullptr, float eps = 0.f, int nt = 2, int order = 0);

// No reduction pass: slice q of A W^T (without bias) is left at
// part + (q * mtiles * kSgemmRows + m) * N + n for the consumer to sum.
template <class Ld>
SgemmShape launch_sgemm_partial(hipStream_t, const Ld&, const bf16_t* W, int M, int N, int K, float* part,
                                int nt = 2);

// The reduction pass alone, over nsplit slices part + (q * Mp + m) * N + n
// that another kernel wrote (summed in slice order, then the epilogue; stats
// as in launch_sgemm, N = 1024).
template <class Epi>
void launch_splitk_reduce(hipStream_t, const float* part, int nsplit, size_t Mp, int M, int N, const Epi&,
                          float2* stats, float eps);

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
// rec: 8 ints per active record: kv0, n, o0, no, pbase, nc, q0, nq
// items: int4 (active record, key chunk, first query of a 32-query block, 0);
// chunk: keys per chunk, a multiple of 64
void launch_route_attn(hipStream_t, const float* Q, const bf16_t* Kl, const bf16_t* Vl, long long Tpad,
                       const int4* items, int nitems, const int* rec, float* pm, float* pl, float* po,
                       long long Ptot, int chunk);
// fp32 form (precision mode fp32): the same items, partials and scaling, over
// fp32 K and V held in head-major planes of Tpad rows x 64 floats (head j of
// the layer at Kl + j * Tpad * 64, elements at k32_off / v32_off), fp32
// operands and accumulation throughout (v_mfma_f32_32x32x2_f32).
void launch_route_attn32(hipStream_t, const float* Q, const float* Kl, const float* Vl, long long Tpad,
                         const int4* items, int nitems, const int* rec, float* pm, float* pl, float* po,
                         long long Ptot, int chunk);
void launch_route_combine(hipStream_t, const float* pm, const float* pl, const float* po, long long Ptot,
                          const int* opt_rec, const int* rec, int NO, float* out);
// QKV: split-K slices (nsplit, slice stride in floats, row width 3072) + bias.
// Writes, per head j, split-K slice j of attn W_o^T at P + j * pstride +
// row * 1024 (rows of every record's fields; Wo in the small GEMMs' fragment
// order, K = 1024; nt bf16 terms per activation as in launch_sgemm).
void launch_field_attn(hipStream_t, const float* qkv_part, int nsplit, size_t stride, const float* bqkv,
                       const int* rec, int nrec, const bf16_t* Wo, float* P, size_t pstride, int nt = 2);

// ---------------------------------------------------------------------------
// aggregation and scoring
// ---------------------------------------------------------------------------
void launch_field_agg(hipStream_t, const float* U, const int* o_off, const float* sw, float sb, const float* qv,
                      const float* gp, const int* q_rec, const int* q_type, const float* temb, int NQ, float* F,
                      float2* fstats, float eps);
// Answer outputs of the scoring kernel, each optional (null = not written):
// value / confidence fp32 [NQ], their 4-decimal copies, 4-decimal probs [NO].
struct AnswerOut {
  float* value;
  float* confidence;
  float* value_4dp;
  float* confidence_4dp;
  float* probs_4dp;
};
// hpart: split-K slices of W1 z (nsplit, slice stride in floats), b1 its bias
void launch_score(hipStream_t, const float* U, const float* F, const float* hpart, int nsplit, size_t hstride,
                  const float* b1, const float* w2, float b2, const float* prior, float gate, float lam, int joint,
                  const int* o_off, int NQ, float* logits, float* probs, int* amax, float* jcos, float* mlp,
                  const int* q_type, const AnswerOut& ans);

}  // namespace clef
