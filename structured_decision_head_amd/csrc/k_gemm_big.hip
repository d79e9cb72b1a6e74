// Dense bf16 MFMA GEMMs over the record rows: the memory projection (hidden
// width -> 1024) and the routing layers' K/V projections (1024 -> 2 x 1024 per
// layer).  These are the FLOP-dominant contractions of the head at long L.
//
// Operation (CoreML conversion metadata of clef-flash, "decision.head":
// LayerNorm(hidden) -> memory; clef-4bit page §三 step 2: every option attends
// over that memory).  LayerNorm is folded into the memory GEMM: with
// W' = W * diag(gamma), c_j = sum_k W'_jk and d_j = sum_k W_jk beta_k + b_j,
//     m_tj = rstd_t * ((W' x_t)_j - mu_t * c_j) + d_j,
// so the GEMM reads the raw bf16 hidden rows and the statistics enter only in
// the epilogue.
//
// Tile: 256 x 256 outputs per workgroup, K step 64, 8 waves in a 2 x 4 grid
// each owning 128 x 64 (4 x 2 v_mfma_f32_32x32x16_bf16 blocks).  A and B tiles
// are double-buffered in LDS (2 x 64 KB) with a 16-byte XOR swizzle; the next
// K step's global loads are in flight while the current one is multiplied.
#include "kernels.hpp"

namespace clef {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;

// One epilogue element: row in the packed row space, output column, fp32 sum.
struct EpiMem {
  const float2* stats;
  const float* c;
  const float* d;
  bf16_t* out;   // [rows][1024]
  DEV void operator()(int row, int col, float v) const {
    const float2 s = stats[row];
    out[(size_t)row * 1024 + col] = (bf16_t)f2bf(s.y * (v - s.x * c[col]) + d[col]);
  }
};

// Columns are [K_0 | V_0 | K_1 | V_1 | ...] (1024 each).  K is stored
// head-major [layer][head][row][64]; V is stored per 32-row block transposed,
// [layer][head][row / 32][64][32], the layout the attention kernel's MFMA
// operand wants.
struct EpiKV {
  const float* bias;
  bf16_t* kv;          // layer r: K at kv + (2r) * 16 * Tpad * 64, V at kv + (2r+1) * 16 * Tpad * 64
  long long Tpad;
  DEV void operator()(int row, int col, float v) const {
    const int r = col >> 11, isv = (col >> 10) & 1, h = (col >> 6) & 15, d = col & 63;
    const bf16_t val = (bf16_t)f2bf(v + bias[col]);
    bf16_t* base = kv + ((size_t)(2 * r + isv) * 16 + h) * (size_t)Tpad * 64;
    if (!isv)
      base[(size_t)row * 64 + d] = val;
    else
      base[((size_t)(row >> 5) * 64 + d) * 32 + (row & 31)] = val;
  }
};

template <class Epi>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm256(const bf16_t* __restrict__ A, int lda, const int4* __restrict__ tiles, int ntile_n,
               const bf16_t* __restrict__ W, int K, Epi epi) {
  __shared__ u32x4 smem[2][2][BM * 8];   // [buffer][A|B][row * 8 + swizzled 16-byte chunk]

  const int lt = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = lt / ntile_n, tn = lt - tm * ntile_n;
  const int4 T = tiles[tm];              // (first A row, first output row, valid rows, record)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;     // 2 x 4 waves, each 128 x 64

  // global -> register mapping: thread owns 16-byte chunk (tid & 7) of rows (tid >> 3) + 64 i.
  // A rows past the tile's valid count are clamped to its last valid row.
  const int lrow = tid >> 3, lch = tid & 7;
  const bf16_t* abase = A + (size_t)T.x * lda + lch * 8;
  const bf16_t* bbase = W + (size_t)(tn * BN + lrow) * K + lch * 8;
  const size_t bstep = (size_t)64 * K;
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = min(lrow + 64 * i, T.z - 1) * lda;
  u32x4 ra[4], rb[4];
#define GLOAD(k0)                                                              \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                              \
    ra[i] = *reinterpret_cast<const u32x4*>(abase + aoff[i] + (k0));           \
    rb[i] = *reinterpret_cast<const u32x4*>(bbase + i * bstep + (k0));         \
  }
#define SSTORE(buf)                                                            \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                              \
    const int r_ = lrow + 64 * i;                                              \
    const int idx_ = r_ * 8 + (lch ^ (r_ & 7));                                \
    smem[buf][0][idx_] = ra[i];                                                \
    smem[buf][1][idx_] = rb[i];                                                \
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = K / BK;
  GLOAD(0)
  SSTORE(0)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) { GLOAD((kt + 1) * BK) }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 128 + mi * 32 + (lane & 31);
        af[mi] = as_bf16x8(smem[cur][0][r * 8 + (ch ^ (r & 7))]);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int r = wn * 64 + ni * 32 + (lane & 31);
        bfr[ni] = as_bf16x8(smem[cur][1][r * 8 + (ch ^ (r & 7))]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) { SSTORE(cur ^ 1) }
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column (lane & 31) and rows
  // 8 * (e / 4) + 4 * (lane / 32) + (e % 4) of its block.  All 256 rows are
  // stored: rows past the valid count come from clamped (finite) inputs and
  // keep the padded part of the row space finite.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wm * 128 + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int col = tn * BN + wn * 64 + ni * 32 + (lane & 31);
        epi(T.y + r, col, acc[mi][ni][e]);
      }
#undef GLOAD
#undef SSTORE
}

}  // namespace

void launch_gemm_mem(hipStream_t st, const bf16_t* hidden, int H, const int4* tiles, int ntiles,
                     const bf16_t* Wm, const float2* stats, const float* c, const float* d, bf16_t* mem) {
  if (ntiles == 0) return;
  const int ntn = 1024 / BN;
  EpiMem epi{stats, c, d, mem};
  hipLaunchKernelGGL(k_gemm256<EpiMem>, dim3(ntiles * ntn), dim3(512), 0, st, hidden, H, tiles, ntn, Wm, H, epi);
}

void launch_gemm_kv(hipStream_t st, const bf16_t* mem, const int4* tiles, int ntiles, const bf16_t* Wkv,
                    const float* bkv, int n_layers, bf16_t* kv, long long Tpad) {
  if (ntiles == 0 || n_layers == 0) return;
  const int ntn = n_layers * 2048 / BN;
  EpiKV epi{bkv, kv, Tpad};
  hipLaunchKernelGGL(k_gemm256<EpiKV>, dim3(ntiles * ntn), dim3(512), 0, st, mem, 1024, tiles, ntn, Wkv, 1024, epi);
}

}  // namespace clef
