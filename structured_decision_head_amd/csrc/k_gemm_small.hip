// Small-M GEMMs of the head: option-query projections, the routing layers'
// Q / O / FFN maps, the field layers' QKV / O / FFN maps and the residual-MLP
// first layer.  M is the number of options or questions (5 to ~1100), N and K
// are 1024..15360; these are weight streams, so the work is split along K
// until the grid fills the chip and the partial sums are reduced by the last
// second kernel that adds the slices in a fixed order (deterministic).
//
// Precision: activations are fp32; each 8-element group is split into NT bf16
// terms (NT = 2: hi = bf16(x), lo = bf16(x - hi), about 16 significant bits of
// x; NT = 3: a third term bf16(x - hi - lo) makes the sum exact, every fp32
// value being the sum of three bf16 values) and every term is multiplied
// against the exact bf16 weights with v_mfma_f32_16x16x32_bf16 into fp32
// accumulators.  With NT = 3 the products are exact and only the fp32
// accumulation rounds: the accuracy of an fp32 GEMM.
//
// Prologues (how A rows are formed) and epilogues (what is done with each
// output) are small functors; see kernels.hpp.
#include "kernels.hpp"

namespace clef {

namespace {

constexpr int SBM = kSgemmRows, SKC = 128;

// Tile: 64 rows x (32 * 4 / WR) columns.  The 4 waves form a WR x (4 / WR)
// grid; each wave owns 64 / WR rows and 32 columns.  Narrow tiles (WR = 2, 4)
// give more workgroups for narrow outputs, so that the whole chip streams
// the weights.
// order = 0: consecutive workgroups walk the row tiles of one column tile (the
// weights of that column tile stay in the XCD's L2); order = 1: they walk the
// column tiles of one row tile (that row tile's A rows stay in L2), for
// products with many row tiles and few weights.
template <int WR, int NT, class Ld, class Epi>
__global__ __launch_bounds__(256) void k_sgemm(Ld ld, Epi epi, const bf16_t* __restrict__ W, int M, int N,
                                               int K, int kchunk, int mtiles, int ntiles, int nsplit, int order,
                                               float* __restrict__ part) {
  constexpr int WC = 4 / WR, SBN = 32 * WC, RB = 4 / WR;
  // two buffers of each converted A term: [term][buffer][row * 16 + swizzled chunk], KC = 128 bf16 per row
  __shared__ uint4 sA[NT][2][SBM * 16];

  const int lt = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = order ? (lt / ntiles) % mtiles : lt % mtiles;
  const int tn = order ? lt % ntiles : (lt / mtiles) % ntiles;
  const int ks = lt / (mtiles * ntiles);
  const int m0 = tm * SBM, n0 = tn * SBN;
  const int kb = ks * kchunk, ke = min(K, kb + kchunk);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr0 = (w / WC) * (SBM / WR), wc0 = (w % WC) * 32;   // the wave's first row / column in the tile

  f32x4 acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // W is stored in fragment order (16 x 32 blocks of 1 KB, a 16-column strip's
  // blocks consecutive along K): the block of columns n16 and K step k32 starts
  // at element (n16 * K / 32 + k32) * 512, and lane l's fragment at 8 l in it.
  const bf16_t* wp[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) wp[cb] = W + (size_t)((n0 + wc0 + cb * 16) >> 4) * (K >> 5) * 512 + lane * 8;

  // Pipeline: while a chunk's MFMAs run, the next chunk's A rows (loaded one
  // chunk earlier) are converted into the other LDS buffer, the A rows of the
  // chunk after that and the next chunk's W fragments are in flight.  The
  // conversion (LayerNorm, hi/lo split) and the MFMAs are independent, so they
  // overlap; one barrier per chunk hands the converted buffer over.
  typename Ld::Raw ra[4];
  typename Ld::Row rw[4];                // the thread's 4 rows, resolved once
  typename Ld::Cst cq;                   // per-column constants of this thread's 8 columns
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid + 256 * i) >> 4;
    if (m0 + r < M) rw[i] = ld.row(m0 + r);
  }
  uint4 bq[2][4];
#define SG_FETCH_A(K0)                                                                   \
  {                                                                                      \
    cq = ld.cst((K0) + (tid & 15) * 8);                                                  \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
      const int v = tid + 256 * i, r = v >> 4, c = v & 15;                               \
      if (m0 + r < M) ra[i] = ld.fetch(rw[i], (K0) + c * 8);                             \
    }                                                                                    \
  }
#define SG_FETCH_W(K0)                                                                   \
  {                                                                                      \
    _Pragma("unroll") for (int cb = 0; cb < 2; ++cb)                                     \
      _Pragma("unroll") for (int kk = 0; kk < 4; ++kk)                                   \
        bq[cb][kk] = *reinterpret_cast<const uint4*>(wp[cb] + (size_t)(K0) * 16 + kk * 512); \
  }
#define SG_CONVERT(BUF, K0)                                                              \
  {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                      \
      const int v = tid + 256 * i;                                                       \
      const int r = v >> 4, c = v & 15;                                                  \
      float x[8];                                                                        \
      if (m0 + r < M) {                                                                  \
        ld.finish(ra[i], cq, m0 + r, (K0) + c * 8, x);                                   \
      } else {                                                                           \
        _Pragma("unroll") for (int e = 0; e < 8; ++e) x[e] = 0.f;                        \
      }                                                                                  \
      uint4 tt[NT];                                                                      \
      split_terms<NT>(x, tt);                                                            \
      const int idx = r * 16 + (c ^ (r & 15));                                           \
      _Pragma("unroll") for (int j = 0; j < NT; ++j) sA[j][BUF][idx] = tt[j];            \
    }                                                                                    \
  }
  SG_FETCH_A(kb)
  SG_FETCH_W(kb)
  SG_CONVERT(0, kb)
  if (kb + SKC < ke) SG_FETCH_A(kb + SKC)
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += SKC) {
    uint4 bc[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) bc[cb][kk] = bq[cb][kk];
    if (k0 + SKC < ke) {
      SG_FETCH_W(k0 + SKC)
      SG_CONVERT(buf ^ 1, k0 + SKC)
      if (k0 + 2 * SKC < ke) SG_FETCH_A(k0 + 2 * SKC)
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 4 + (lane >> 4);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int r = wr0 + rb * 16 + (lane & 15);
        bf16x8 a[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) a[j] = as_bf16x8(sA[j][buf][r * 16 + (c ^ (r & 15))]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const bf16x8 b = as_bf16x8(bc[cb][kk]);
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b, acc[rb][cb], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    buf ^= 1;
  }
#undef SG_CONVERT
#undef SG_FETCH_W
#undef SG_FETCH_A

  // 16x16 accumulator layout: lane holds column (lane & 15), rows 4 * (lane / 16) + e.
  if (nsplit == 1) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wr0 + rb * 16 + 4 * (lane >> 4) + e;
          const int n = n0 + wc0 + cb * 16 + (lane & 15);
          if (m < M) epi(m, n, acc[rb][cb][e]);
        }
    return;
  }

  // split-K: every workgroup writes its partial tile; k_splitk_reduce sums the
  // slices in order in a second launch (the kernel boundary orders the writes)
  const size_t Mp = (size_t)mtiles * SBM;
  float* P = part + (size_t)ks * Mp * N;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wr0 + rb * 16 + 4 * (lane >> 4) + e;
        const int n = n0 + wc0 + cb * 16 + (lane & 15);
        P[(size_t)m * N + n] = acc[rb][cb][e];
      }
}

// Sum the split-K slices in a fixed order and apply the epilogue; one thread
// per 4 consecutive outputs.  With stats (N = 1024, one block per row) the
// block also computes the two-pass LayerNorm statistics of the row it wrote.
template <class Epi>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int nsplit, size_t Mp, int M,
                                                       int N, Epi epi, float2* __restrict__ stats, float eps) {
  __shared__ float sm[4];
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (stats == nullptr && i >= (size_t)M * N) return;
  const int m = (int)(i / N), n = (int)(i - (size_t)m * N);
  // the epilogue's own loads and all slices in flight at once, summed in slice order
  const typename Epi::Pre pre = epi.pre4(m, n);
  float4 t[kMaxSplit];
#pragma unroll
  for (int q = 0; q < kMaxSplit; ++q)
    if (q < nsplit) t[q] = *reinterpret_cast<const float4*>(part + ((size_t)q * Mp + m) * N + n);
  float4 s = t[0];
#pragma unroll
  for (int q = 1; q < kMaxSplit; ++q)
    if (q < nsplit) { s.x += t[q].x; s.y += t[q].y; s.z += t[q].z; s.w += t[q].w; }
  const float4 o = epi.apply4(m, n, s, pre);
  const float a = o.x, b = o.y, c = o.z, d = o.w;
  if (stats != nullptr) {
    const float mu = block_sum<4>((a + b) + (c + d), sm) * (1.0f / 1024);
    const float va = block_sum<4>((a - mu) * (a - mu) + (b - mu) * (b - mu) + (c - mu) * (c - mu) + (d - mu) * (d - mu),
                                  sm) * (1.0f / 1024);
    if (threadIdx.x == 0) stats[m] = make_float2(mu, 1.0f / sqrtf(va + eps));
  }
}

}  // namespace

// The widest tile (128, 64 or 32 columns) whose grid, split along K towards
// 256 workgroups (at most kMaxSplit slices of 128-deep chunks), still has at
// least 128 workgroups.  Fewer, longer workgroups hold the CUs for less time
// in total, which matters most when another batch's kernels share the chip.
// When the consumer sums the slices itself (no reduction pass) the split goes
// towards 512 workgroups with at least 256.
SgemmShape sgemm_shape(int M, int N, int K, bool need_reduce, bool consumer_sums) {
  const int target = consumer_sums ? 512 : 256, least = consumer_sums ? 256 : 128;
  SgemmShape s{};
  s.mtiles = (M + SBM - 1) / SBM;
  const int kblocks = K / SKC;
  for (int wr = 1; wr <= 4; wr *= 2) {
    const int sbn = 128 / wr;
    s.wr = wr;
    s.ntiles = N / sbn;
    const int tiles = s.mtiles * s.ntiles;
    int split = (target + tiles - 1) / tiles;
    if (split > kMaxSplit) split = kMaxSplit;
    if (split > kblocks) split = kblocks;
    if (split < 1) split = 1;
    if (need_reduce && split < 2) split = 2;
    const int per = (kblocks + split - 1) / split;
    s.kchunk = per * SKC;
    s.nsplit = (kblocks + per - 1) / per;
    if (tiles * s.nsplit >= least || wr == 4 || (N / (sbn / 2)) * (sbn / 2) != N) break;
  }
  s.part_floats = s.nsplit > 1 ? (size_t)s.nsplit * s.mtiles * SBM * N : 0;
  return s;
}

template <int NT, class Ld, class Epi>
static void launch_tile_nt(const SgemmShape& s, hipStream_t st, const Ld& ld, const Epi& epi, const bf16_t* W,
                           int M, int N, int K, int order, float* part) {
  const dim3 grid(s.mtiles * s.ntiles * s.nsplit);
  if (s.wr == 1)
    hipLaunchKernelGGL((k_sgemm<1, NT, Ld, Epi>), grid, dim3(256), 0, st, ld, epi, W, M, N, K, s.kchunk, s.mtiles,
                       s.ntiles, s.nsplit, order, part);
  else if (s.wr == 2)
    hipLaunchKernelGGL((k_sgemm<2, NT, Ld, Epi>), grid, dim3(256), 0, st, ld, epi, W, M, N, K, s.kchunk, s.mtiles,
                       s.ntiles, s.nsplit, order, part);
  else
    hipLaunchKernelGGL((k_sgemm<4, NT, Ld, Epi>), grid, dim3(256), 0, st, ld, epi, W, M, N, K, s.kchunk, s.mtiles,
                       s.ntiles, s.nsplit, order, part);
}

template <class Ld, class Epi>
static void launch_tile(const SgemmShape& s, hipStream_t st, const Ld& ld, const Epi& epi, const bf16_t* W, int M,
                        int N, int K, float* part, int nt, int order) {
  if (nt == 3) launch_tile_nt<3>(s, st, ld, epi, W, M, N, K, order, part);
  else launch_tile_nt<2>(s, st, ld, epi, W, M, N, K, order, part);
}

template <class Ld, class Epi>
void launch_sgemm(hipStream_t st, const Ld& ld, const Epi& epi, const bf16_t* W, int M, int N, int K,
                  float* part, float2* stats, float eps, int nt, int order) {
  if (M == 0) return;
  const SgemmShape s = sgemm_shape(M, N, K, stats != nullptr);
  launch_tile(s, st, ld, epi, W, M, N, K, part, nt, order);
  if (s.nsplit > 1) {
    const size_t n4 = (size_t)M * N / 4;
    hipLaunchKernelGGL((k_splitk_reduce<Epi>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, s.nsplit,
                       (size_t)s.mtiles * SBM, M, N, epi, stats, eps);
  }
}

template <class Ld>
SgemmShape launch_sgemm_partial(hipStream_t st, const Ld& ld, const bf16_t* W, int M, int N, int K, float* part,
                                int nt) {
  const SgemmShape s = sgemm_shape(M, N, K, false, true);
  if (M == 0) return s;
  launch_tile(s, st, ld, EpPart{part, N}, W, M, N, K, part, nt, 0);
  return s;
}
template <class Epi>
void launch_splitk_reduce(hipStream_t st, const float* part, int nsplit, size_t Mp, int M, int N, const Epi& epi,
                          float2* stats, float eps) {
  if (M == 0) return;
  const size_t n4 = (size_t)M * N / 4;
  hipLaunchKernelGGL((k_splitk_reduce<Epi>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, nsplit, Mp,
                     M, N, epi, stats, eps);
}
template void launch_splitk_reduce<EpResid>(hipStream_t, const float*, int, size_t, int, int, const EpResid&, float2*,
                                            float);

template SgemmShape launch_sgemm_partial<LdLN>(hipStream_t, const LdLN&, const bf16_t*, int, int, int, float*, int);
template SgemmShape launch_sgemm_partial<LdZ>(hipStream_t, const LdZ&, const bf16_t*, int, int, int, float*, int);

#define INST(LD, EP)                                                                                   \
  template void launch_sgemm<LD, EP>(hipStream_t, const LD&, const EP&, const bf16_t*, int, int, int, \
                                     float*, float2*, float, int, int);
INST(LdRows, EpStore)
INST(LdRows, EpResid)
INST(LdLN, EpStore)
INST(LdLN, EpGelu)
INST(LdSeg2, EpAddRow)
INST(LdRows, EpSplit2)
INST(LdHid<false>, EpStore)
INST(LdHid<true>, EpStore)
INST(LdRows, EpHeads)
#undef INST

}  // namespace clef
