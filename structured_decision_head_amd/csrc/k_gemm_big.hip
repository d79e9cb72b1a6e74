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
// Tile: 256 x 256 outputs per workgroup, 4 waves in a 2 x 2 grid each owning
// 128 x 128 (4 x 4 v_mfma_f32_32x32x16_bf16 blocks, accumulators in AGPRs).
#include "kernels.hpp"

namespace clef {

namespace {

constexpr int BM = 256, BN = 256;

// Epilogues consume a wave's whole 128 x 128 accumulator block.  Accumulator
// (mi, ni, e) of lane l sits at block row 32 mi + 8 (e / 4) + 4 (l / 32) + e % 4
// and block column 32 ni + (l % 32).  row0 / col0 locate the block in the
// packed row space and the output columns; per-row and per-column values are
// hoisted out of the element loops.
struct EpiMem {
  const float2* stats;
  const float* c;
  const float* d;
  bf16_t* out;   // [rows][1024]
  static constexpr bool kHasTransposed = false;
  DEV bool transposed(int) const { return false; }
  DEV void tile(const f32x16 (&acc)[4][4], int row0, int col0, int lane) const {
    float cc[4], dd[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int col = col0 + ni * 32 + (lane & 31);
      cc[ni] = c[col];
      dd[ni] = d[col];
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const float2 st = stats[row];
        bf16_t* o = out + (size_t)row * 1024 + col0 + (lane & 31);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) o[ni * 32] = (bf16_t)f2bf(st.y * (acc[mi][ni][e] - st.x * cc[ni]) + dd[ni]);
      }
  }
};

// Columns are [K_0 | V_0 | K_1 | V_1 | ...] (1024 each).  K is stored
// head-major [layer][head][row][64]; V is stored per 32-row block transposed,
// [layer][head][row / 32][64][32] with the 32 keys of a block in
// vblock_pos() order, the layout the attention kernel's MFMA operand wants.
// V tiles are accumulated transposed (acc rows are output columns, acc
// columns are rows), so 32 lanes store 64 contiguous bytes.
struct EpiKV {
  const float* bias;
  bf16_t* kv;          // layer r: K at kv + (2r) * 16 * Tpad * 64, V at kv + (2r+1) * 16 * Tpad * 64
  long long Tpad;
  static constexpr bool kHasTransposed = true;
  DEV bool transposed(int tn) const { return ((tn * BN) >> 10) & 1; }
  DEV bf16_t* head_base(int col) const {
    const int r = col >> 11, isv = (col >> 10) & 1, h = (col >> 6) & 15;
    return kv + ((size_t)(2 * r + isv) * 16 + h) * (size_t)Tpad * 64;
  }
  // K: acc rows are rows, acc columns are output columns
  DEV void tile(const f32x16 (&acc)[4][4], int row0, int col0, int lane) const {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int col = col0 + ni * 32 + (lane & 31);
      const float b = bias[col];
      bf16_t* base = head_base(col) + (col & 63);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = row0 + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          base[(size_t)row * 64] = (bf16_t)f2bf(acc[mi][ni][e] + b);
        }
    }
  }
  // V: acc rows are output columns (col0 + ...), acc columns are rows (row0 + ...)
  DEV void tile_t(const f32x16 (&acc)[4][4], int row0, int col0, int lane) const {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int col = col0 + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const float b = bias[col];
        bf16_t* base = head_base(col) + (size_t)(col & 63) * 32 + vblock_pos(lane & 31);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int rb = (row0 + ni * 32) >> 5;   // 32-row block (row0 is a multiple of 32)
          base[(size_t)rb * 2048] = (bf16_t)f2bf(acc[mi][ni][e] + b);
        }
      }
  }
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with only the vector-memory counter constrained to <= n
#define WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
// s_waitcnt lgkmcnt(0) only
#define WAIT_LDS() __builtin_amdgcn_s_waitcnt((7 << 4) | 15 | (3 << 14))

// Operand tiles live in a 4-stage LDS ring of 32-wide K steps; rows are 64 B
// (four 16-byte chunks) and chunk c of row r sits at position c ^ ((r >> 2) & 3),
// which keeps the fragment reads free of bank conflicts.  Global -> LDS copies
// use global_load_lds_dwordx4: lane l of a wave writes the l-th 16-byte slot of
// a 1 KB block, so each lane fetches the chunk that belongs in its slot.
//
// Per K step a wave runs two 16-deep halves of 16 MFMAs; the fragments of the
// next half are read while the current half multiplies, and the stage consumed
// in this step is refilled (K step + 4) right after the mid-step barrier.
template <class Epi>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm256(const bf16_t* __restrict__ A, int lda, const int4* __restrict__ tiles, int ntile_n,
               const bf16_t* __restrict__ W, int K, Epi epi) {
  constexpr int KS = 32, NST = 4;
  __shared__ u32x4 smem[NST][2][BM * 4];   // [stage][A|B][row * 4 + swizzled chunk]

  const int lt = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = lt / ntile_n, tn = lt - tm * ntile_n;
  const int4 T = tiles[tm];              // (first A row, first output row, valid rows, record)
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;     // 2 x 2 waves, each 128 x 128
  // transposed tiles feed the W rows as the MFMA A operand: acc rows are then
  // output columns and acc columns are A rows
  const bool tr = epi.transposed(tn);
  const int ra_src = tr ? 1 : 0, rb_src = tr ? 0 : 1;
  const int wa = tr ? wn : wm, wb = tr ? wm : wn;

  // copy sources: instruction i of wave w fills rows 16 (4 w + i) .. +16 of a stage;
  // A rows past the tile's valid count are clamped to its last valid row
  const bf16_t* ga[4];
  const bf16_t* gb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * (w * 4 + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    ga[i] = A + (size_t)(T.x + min(row, T.z - 1)) * lda + c * 8;
    gb[i] = W + (size_t)(tn * BN + row) * K + c * 8;
  }
  // fragment positions: 32x32x16 operands, lane -> row (lane & 31), chunk 2 kk + (lane >> 5)
  int offA[2][4], offB[2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int ch = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wa * 128 + i * 32 + (lane & 31);
      const int rb = wb * 128 + i * 32 + (lane & 31);
      offA[kk][i] = ra_src * (BM * 4) + ra * 4 + (ch ^ ((ra >> 2) & 3));
      offB[kk][i] = rb_src * (BM * 4) + rb * 4 + (ch ^ ((rb >> 2) & 3));
    }
  }
#define COPY_STAGE(stage, k0)                                                                                  \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                              \
    __builtin_amdgcn_global_load_lds((const void*)(ga[i] + (k0)), (lds_ptr_t)&smem[stage][0][64 * (w * 4 + i)], \
                                     16, 0, 0);                                                                \
    __builtin_amdgcn_global_load_lds((const void*)(gb[i] + (k0)), (lds_ptr_t)&smem[stage][1][64 * (w * 4 + i)], \
                                     16, 0, 0);                                                                \
  }
#define LOAD_FRAGS(F, stage, kk)                                  \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                 \
    F##a[i] = as_bf16x8(smem[stage][0][offA[kk][i]]);             \
    F##b[i] = as_bf16x8(smem[stage][0][offB[kk][i]]);             \
  }
#define MULTIPLY(F)                                                                       \
  _Pragma("unroll") for (int mi = 0; mi < 4; ++mi)                                        \
  _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                                        \
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F##a[mi], F##b[ni], acc[mi][ni], 0, 0, 0);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  bf16x8 Xa[4], Xb[4], Ya[4], Yb[4];

  const int nk = K / KS;                 // >= 4 (K >= 128)
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) { COPY_STAGE(st, st * KS) }
  WAIT_VM(8 * (NST - 2));
  __builtin_amdgcn_s_barrier();
  COPY_STAGE(NST - 1, (NST - 1) * KS)
  LOAD_FRAGS(X, 0, 0)
  int kt = 0;
  for (; kt < nk - NST; ++kt) {          // steady state: refill the consumed stage with K step kt + 4
    const int cur = kt % NST;
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    LOAD_FRAGS(Y, cur, 1)
    MULTIPLY(X)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    WAIT_LDS();                          // this stage is in registers everywhere after the barrier
    WAIT_VM(8 * (NST - 2));              // the next stage has landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    COPY_STAGE(cur, (kt + NST) * KS)
    LOAD_FRAGS(X, (kt + 1) % NST, 0)
    MULTIPLY(Y)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);   // global -> LDS copy
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);   // LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  for (; kt < nk; ++kt) {                // drain the ring
    const int cur = kt % NST;
    WAIT_LDS();
    LOAD_FRAGS(Y, cur, 1)
    MULTIPLY(X)
    if (kt + 1 < nk) {
      const int ahead = (nk - 1) - (kt + 1);
      WAIT_LDS();
      if (ahead >= 2) WAIT_VM(16); else if (ahead == 1) WAIT_VM(8); else WAIT_VM(0);
      __builtin_amdgcn_s_barrier();
      LOAD_FRAGS(X, (kt + 1) % NST, 0)
    }
    MULTIPLY(Y)
  }
#undef COPY_STAGE
#undef LOAD_FRAGS
#undef MULTIPLY

  // All 256 rows are stored: rows past the valid count come from clamped
  // (finite) inputs and keep the padded part of the row space finite.
  if constexpr (Epi::kHasTransposed) {
    if (tr) {
      epi.tile_t(acc, T.y + wb * 128, tn * BN + wa * 128, lane);
      return;
    }
  }
  epi.tile(acc, T.y + wa * 128, tn * BN + wb * 128, lane);
}

}  // namespace

void launch_gemm_mem(hipStream_t st, const bf16_t* hidden, int H, const int4* tiles, int ntiles,
                     const bf16_t* Wm, const float2* stats, const float* c, const float* d, bf16_t* mem) {
  if (ntiles == 0) return;
  const int ntn = 1024 / BN;
  EpiMem epi{stats, c, d, mem};
  hipLaunchKernelGGL(k_gemm256<EpiMem>, dim3(ntiles * ntn), dim3(256), 0, st, hidden, H, tiles, ntn, Wm, H, epi);
}

void launch_gemm_kv(hipStream_t st, const bf16_t* mem, const int4* tiles, int ntiles, const bf16_t* Wkv,
                    const float* bkv, int n_layers, bf16_t* kv, long long Tpad) {
  if (ntiles == 0 || n_layers == 0) return;
  const int ntn = n_layers * 2048 / BN;
  EpiKV epi{bkv, kv, Tpad};
  hipLaunchKernelGGL(k_gemm256<EpiKV>, dim3(ntiles * ntn), dim3(256), 0, st, mem, 1024, tiles, ntn, Wkv, 1024, epi);
}

}  // namespace clef
