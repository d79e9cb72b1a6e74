// Dense bf16 MFMA GEMMs over the record rows: the memory projection (hidden
// width -> 1024) and the routing layers' K/V projections (1024 -> 2 x 1024 per
// layer).  These are the FLOP-dominant contractions of the head at long L.
//
// Operation (CoreML conversion metadata page of clef-flash, decision.head: the
// memory is a projection of the LayerNorm-ed hidden rows; clef-4bit page §三
// step 2: every option attends over that memory).  LayerNorm is folded into
// the memory GEMM: with
// W' = W * diag(gamma), c_j = sum_k W'_jk and d_j = sum_k W_jk beta_k + b_j,
//     m_tj = rstd_t * ((W' x_t)_j - mu_t * c_j) + d_j,
// so the GEMM reads the raw bf16 hidden rows and the statistics enter only in
// the epilogue.
//
// Tile: 256 x 256 outputs per workgroup, 4 waves in a 2 x 2 grid each owning
// 128 x 128 (4 x 4 v_mfma_f32_32x32x16_bf16 blocks, accumulators in AGPRs).
// With fp16 hidden rows the memory GEMM multiplies fp16 operands (an fp16 copy
// of W') with v_mfma_f32_32x32x16_f16 instead.  The fp32 head runs its
// memory and K/V products on the same tile as bf16 GEMMs of three times the
// depth with exact products (EpiMem32, EpiKV32 below).
#include "kernels.hpp"

namespace clef {

namespace {

constexpr int BM = 256, BN = 256;

// Epilogues.  Each tile is multiplied in the orientation that gives a lane
// runs of consecutive output elements: "transposed" tiles take the W rows as
// the MFMA A operand, so accumulator rows are output columns and a lane owns
// one output row with runs of 4 consecutive columns.  Accumulator (mi, ni, e)
// of lane l sits at block row 32 mi + 8 (e / 4) + 4 (l / 32) + e % 4 and block
// column 32 ni + (l % 32).
//
// A finished memory tile is converted to bf16 and written with 8-byte LDS
// stores into an image of its final memory layout (the operand ring is free
// by then); all 256 threads then copy the image out with 16-byte global
// stores, each wave instruction covering 1 KB of contiguous memory.  K/V
// tiles need no image: their fragment-order layouts let every lane store
// whole 16-byte chunks straight from the accumulators, again 1 KB per wave
// instruction.  Per-tile constants are loaded by thread tid when the kernel
// starts, so their latency hides under the main loop, held in registers, and
// parked in a small LDS area at the ring's end once the main loop is over.
constexpr int kConstFloats = 1024;

struct EpiMem {          // transposed tiles; rows of out are the packed row space
  const float2* stats;   // LayerNorm (mean, rstd) per output row
  const float* c;
  const float* d;
  bf16_t* out;           // [rows][1024]
  static constexpr bool kF16 = false;                  // operands bf16
  static constexpr bool kDirect = false;               // output staged through LDS
  static constexpr bool kRegs = false;
  static constexpr bool kBiasInit = false;
  static constexpr bool kPlain = false;                // every tile transposed
  static constexpr int kWrapW = 0;
  static constexpr int kLd = 264;                      // image row pitch (bf16): 512 B + 16 B
  static constexpr int kImageBytes = 256 * kLd * 2;
  DEV int a_wrap() const { return 0; }
  DEV bool transposed(int) const { return true; }
  // constants: [0, 256) c and [256, 512) d of the tile's columns, then (mean, rstd) of its rows
  DEV void load_consts(int orow0, int ocol0, int tid, float (&r)[4]) const {
    const float2 st = stats[orow0 + tid];
    r[0] = c[ocol0 + tid]; r[1] = d[ocol0 + tid]; r[2] = st.x; r[3] = st.y;
  }
  DEV void put_consts(float* cst, int tid, const float (&r)[4]) const {
    cst[tid] = r[0]; cst[256 + tid] = r[1]; cst[512 + 2 * tid] = r[2]; cst[513 + 2 * tid] = r[3];
  }
  // lr0 / lc0: tile-local first row / column of the wave's block
  DEV void stage_t(const f32x16 (&acc)[4][4], const float* cst, bf16_t* img, int lr0, int lc0, int lane) const {
    const int h4 = 4 * (lane >> 5);
    float2 st[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) st[ni] = *reinterpret_cast<const float2*>(cst + 512 + 2 * (lr0 + ni * 32 + (lane & 31)));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int lc = lc0 + mi * 32 + 8 * g + h4;
        const float4 cc = *reinterpret_cast<const float4*>(cst + lc);
        const float4 dd = *reinterpret_cast<const float4*>(cst + 256 + lc);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const float mu = st[ni].x, rs = st[ni].y;
          const f32x16& a = acc[mi][ni];
          uint2 v;
          v.x = pack_bf16x2(rs * (a[4 * g] - mu * cc.x) + dd.x, rs * (a[4 * g + 1] - mu * cc.y) + dd.y);
          v.y = pack_bf16x2(rs * (a[4 * g + 2] - mu * cc.z) + dd.z, rs * (a[4 * g + 3] - mu * cc.w) + dd.w);
          *reinterpret_cast<uint2*>(img + (lr0 + ni * 32 + (lane & 31)) * kLd + lc) = v;
        }
      }
  }
  DEV void store(const bf16_t* img, int orow0, int ocol0, int tid) const {
#pragma unroll 8
    for (int i = tid; i < 256 * 32; i += 256) {
      const int r = i >> 5, ch = i & 31;
      *reinterpret_cast<uint4*>(out + (size_t)(orow0 + r) * 1024 + ocol0 + ch * 8) =
          *reinterpret_cast<const uint4*>(img + r * kLd + ch * 8);
    }
  }
};

// Columns are [K_0 | V_0 | K_1 | V_1 | ...] (1024 each), so a 256-column tile
// is four heads of one K or one V, and the tile's 256 rows of one head are a
// contiguous 32 KB run in either layout.  Both are stored per head in blocks
// of 32 rows (4 KB), each block in the routing attention's MFMA fragment
// order, so that a wave reads 1 KB of contiguous memory per operand load:
//  * K block (key row r, dim d): 16-byte chunk (d / 8) of row r sits at
//    chunk index 64 (d / 16) + (r + 32 ((d / 8) & 1)) (kchunk());
//  * V block (dim f, key position p): the block is V^T [64][32] with the 32
//    keys in vblock_pos() order (plain tiles: a lane's accumulators
//    e = 8 q .. 8 q + 7 land on 8 consecutive key positions, one 16-byte run),
//    and 16-byte chunk (p / 8) of feature row f sits at chunk index
//    64 (2 (p / 16) + f / 32) + (f % 32 + 32 ((p / 8) & 1)) (vchunk()).
DEV int kchunk(int r, int c) { return 64 * (c >> 1) + (r & 31) + 32 * (c & 1); }
DEV int vchunk(int f, int c) { return 64 * (2 * (c >> 1) + (f >> 5)) + (f & 31) + 32 * (c & 1); }
// The same with fp16 hidden rows and an fp16 copy of W' (fp16 MFMA).
struct EpiMem16 : EpiMem {
  static constexpr bool kF16 = true;
};

struct EpiKV {
  const float* bias;
  bf16_t* kv;          // layer r: K at kv + (2r) * 16 * Tpad * 64, V at kv + (2r+1) * 16 * Tpad * 64
  long long Tpad;
  static constexpr bool kF16 = false;
  static constexpr bool kDirect = false;
  static constexpr bool kRegs = true;                  // stored from the accumulators
  static constexpr bool kBiasInit = true;              // accumulators start at the bias
  static constexpr bool kPlain = true;                 // V tiles are plain
  static constexpr int kWrapW = 0;
  static constexpr int kImageBytes = 0;
  DEV int a_wrap() const { return 0; }
  DEV bool transposed(int tn) const { return !(((tn * BN) >> 10) & 1); }
  DEV bf16_t* head_base(int col) const {
    const int r = col >> 11, isv = (col >> 10) & 1, h = (col >> 6) & 15;
    return kv + ((size_t)(2 * r + isv) * 16 + h) * (size_t)Tpad * 64;
  }
  DEV void load_consts(int, int, int, float (&)[4]) const {}
  DEV void put_consts(float*, int, const float (&)[4]) const {}
  // The accumulators start at the bias of their output column, so the
  // epilogue only converts and stores (accumulator layout as in store_regs):
  // bias_regs loads the values a lane needs when the tile starts (TR tiles
  // bq[mi][g] = columns ra0 + 32 mi + 8 g + 4 (l / 32) .. + 3; plain tiles
  // bq[ni][0].x = column rb0 + 32 ni + l % 32), fill_acc writes them once the
  // prologue's copies are in flight.
  template <bool TR>
  DEV void bias_regs(float4 (&bq)[4][4], int ocol0, int ra0, int rb0, int lane) const {
    if constexpr (TR) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          bq[mi][g] = *reinterpret_cast<const float4*>(bias + ocol0 + ra0 + mi * 32 + 8 * g + 4 * (lane >> 5));
    } else {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) bq[ni][0].x = bias[ocol0 + rb0 + ni * 32 + (lane & 31)];
    }
  }
  template <bool TR>
  DEV void fill_acc(f32x16 (&acc)[4][4], const float4 (&bq)[4][4]) const {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if constexpr (TR) {
            const float4 b = bq[mi][e >> 2];
            acc[mi][ni][e] = (e & 3) == 0 ? b.x : (e & 3) == 1 ? b.y : (e & 3) == 2 ? b.z : b.w;
          } else {
            acc[mi][ni][e] = bq[ni][0].x;
          }
        }
  }
  // Every store instruction of a wave writes one contiguous 1 KB run (64
  // consecutive 16-byte chunks of a 32-row block), with the non-temporal hint:
  // K and V are read once per routing layer, so they need not sit dirty in
  // the caches, where reads of the next batch's hidden rows would first have to
  // write them back.  orow0 / ocol0: the tile's
  // first output row / column; ra0 / rb0: tile-local first row of the wave's
  // MFMA A / B operand block (accumulator rows / columns).
  //  * K (transposed tile): accumulator (mi, ni, e) of lane l is dim
  //    ra0 + 32 mi + 8 (e / 4) + 4 (l / 32) + e % 4 of key rb0 + 32 ni + l % 32,
  //    so lanes l and l + 32 hold the two 8-byte halves of one chunk.  One
  //    v_permlane32_swap per 32-bit word gives lane l (< 32) the whole chunk of
  //    dim group 2p and lane l + 32 that of group 2p + 1: chunk indices
  //    64 (2 (mi & 1) + p) + l, i.e. kchunk() of the key and the 8-dim group.
  //  * V (plain tile): accumulator (mi, ni, e) of lane l is key
  //    ra0 + 32 mi + 8 (e / 4) + 4 (l / 32) + e % 4 of feature rb0 + 32 ni + l % 32;
  //    e = 8 q .. 8 q + 7 are key positions 8 (2 q + l / 32) .. + 7 of
  //    vblock_pos(), the 16-byte chunk vchunk(f, 2 q + l / 32) = 64 (2 q + f / 32) + l.
  template <bool TR>
  DEV void store_regs(const f32x16 (&acc)[4][4], const float* cst, int orow0, int ocol0, int ra0, int rb0,
                      int lane) const {
    if constexpr (TR) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int lcb = ra0 + mi * 32;
        bf16_t* hb = head_base(ocol0 + lcb) + (size_t)(64 * 2 * (mi & 1) + lane) * 8;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const f32x16& a = acc[mi][ni];
          bf16_t* blk = hb + (size_t)((orow0 + rb0 + ni * 32) >> 5) * 2048;
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int g0 = 2 * p, g1 = 2 * p + 1;
            const uint32_t p0 = pack_bf16x2(a[4 * g0], a[4 * g0 + 1]);
            const uint32_t p1 = pack_bf16x2(a[4 * g0 + 2], a[4 * g0 + 3]);
            const uint32_t q0 = pack_bf16x2(a[4 * g1], a[4 * g1 + 1]);
            const uint32_t q1 = pack_bf16x2(a[4 * g1 + 2], a[4 * g1 + 3]);
            const auto s0 = __builtin_amdgcn_permlane32_swap(p0, q0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(p1, q1, false, false);
            store_stream(blk + p * 512, u32x4{s0[0], s1[0], s0[1], s1[1]});
          }
        }
      }
    } else {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int lc = rb0 + ni * 32 + (lane & 31);
        bf16_t* hb = head_base(ocol0 + rb0 + ni * 32) + (size_t)(64 * ((lc >> 5) & 1) + lane) * 8;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const f32x16& a = acc[mi][ni];
          bf16_t* blk = hb + (size_t)((orow0 + ra0 + mi * 32) >> 5) * 2048;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int e = 8 * q;
            store_stream(blk + q * 1024, u32x4{pack_bf16x2(a[e], a[e + 1]), pack_bf16x2(a[e + 2], a[e + 3]),
                                               pack_bf16x2(a[e + 4], a[e + 5]), pack_bf16x2(a[e + 6], a[e + 7])});
          }
        }
      }
    }
  }
};

// fp32 head.  Its products run on this kernel as bf16 GEMMs of three times
// the depth in which every product is exact, so the MFMAs' fp32 accumulation
// is the only rounding: either the A rows hold the three exact bf16 terms of
// each fp32 value side by side ([t0 | t1 | t2], each K0 wide) and every term
// meets the same weight row (stored repeated, [W | W | W], for the memory
// product over fp16 hidden rows; read three times through the K-position
// wrap for the K/V product, whose 2 MB column group then stays in L2), or the
// A row is exact in bf16 already (bf16 hidden rows) and is read three times
// through its own K-position wrap against the weight's three terms.  All
// tiles are transposed: accumulator (mi, ni, e) of lane l is column ra0 +
// 32 mi + 8 (e / 4) + 4 (l / 32) + e % 4 of row rb0 + 32 ni + l % 32, four
// consecutive columns per (mi, ni, e / 4), stored straight from the
// accumulators.
//
// Memory rows, written as fp32 rows [rows][1024] and as the three bf16 terms
// of each value in [rows][3 x 1024] (the A operand of the K/V product):
//  * over LayerNorm-ed rows' terms against [W | W | W]: m = acc + b (c, stats
//    null; d = b);
//  * over the raw bf16 hidden rows, read three times (A's K position wraps at
//    awrap = H), against the three bf16 terms of fp32(W diag(gamma)): the
//    LayerNorm folded as in the bf16 mode, m = rstd (acc - mu c) + d, with
//    c_j the sum of the fp32 weights of row j and d = W beta + b.  The hidden
//    values are exact in bf16, so every product is exact here too.
// Both take the same arithmetic form: with c = 0 and (mu, rstd) = (0, 1)
// it gives acc + d exactly.
struct EpiMem32 {
  const float2* stats;   // (mean, rstd) per packed row, or null
  const float* c;        // or null
  const float* d;
  float* mem;            // [rows][1024] fp32, or null (only the terms are needed)
  bf16_t* planes;        // [rows][3 * 1024] bf16
  int awrap;             // A's K-position wrap (0: none)
  static constexpr bool kF16 = false;
  static constexpr bool kDirect = false;
  static constexpr bool kRegs = true;
  static constexpr bool kBiasInit = false;
  static constexpr bool kPlain = false;
  static constexpr int kWrapW = 0;
  static constexpr int kImageBytes = 0;
  DEV int a_wrap() const { return awrap; }
  DEV bool transposed(int) const { return true; }
  // constants: [0, 256) d and [256, 512) c of the tile's columns, then (mean, rstd) of its rows
  DEV void load_consts(int orow0, int ocol0, int tid, float (&r)[4]) const {
    const float2 st = stats ? stats[orow0 + tid] : make_float2(0.f, 1.f);
    r[0] = d[ocol0 + tid]; r[1] = c ? c[ocol0 + tid] : 0.f; r[2] = st.x; r[3] = st.y;
  }
  DEV void put_consts(float* cst, int tid, const float (&r)[4]) const {
    cst[tid] = r[0]; cst[256 + tid] = r[1]; cst[512 + 2 * tid] = r[2]; cst[513 + 2 * tid] = r[3];
  }
  template <bool TR>
  DEV void store_regs(const f32x16 (&acc)[4][4], const float* cst, int orow0, int ocol0, int ra0, int rb0,
                      int lane) const {
    const int h4 = 4 * (lane >> 5);
    float2 st[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) st[ni] = *reinterpret_cast<const float2*>(cst + 512 + 2 * (rb0 + ni * 32 + (lane & 31)));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int lc = ra0 + mi * 32 + 8 * g + h4;
        const float4 dd = *reinterpret_cast<const float4*>(cst + lc);
        const float4 cc = *reinterpret_cast<const float4*>(cst + 256 + lc);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const f32x16& a = acc[mi][ni];
          const float mu = st[ni].x, rs = st[ni].y;
          const size_t row = (size_t)(orow0 + rb0 + ni * 32 + (lane & 31));
          const float v[4] = {rs * (a[4 * g] - mu * cc.x) + dd.x, rs * (a[4 * g + 1] - mu * cc.y) + dd.y,
                              rs * (a[4 * g + 2] - mu * cc.z) + dd.z, rs * (a[4 * g + 3] - mu * cc.w) + dd.w};
          if (mem) *reinterpret_cast<float4*>(mem + row * 1024 + ocol0 + lc) = make_float4(v[0], v[1], v[2], v[3]);
          float r[4] = {v[0], v[1], v[2], v[3]}, h[4];
#pragma unroll
          for (int p = 0; p < 3; ++p) {
            const uint2 t = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
            *reinterpret_cast<uint2*>(planes + row * 3072 + p * 1024 + ocol0 + lc) = t;
            if (p < 2) {
              unpack4(t.x, t.y, h);
#pragma unroll
              for (int i = 0; i < 4; ++i) r[i] -= h[i];
            }
          }
        }
      }
  }
};

// K / V of the fp32 head: C = acc + b into head-major fp32 planes, columns
// [64 p, 64 p + 64) -> plane p of Tpad rows, in 32-row blocks of the fp32
// routing attention's fragment order (k32_off / v32_off).  K tiles are
// transposed, V tiles plain, so that each store instruction of a wave covers
// whole 16-byte runs of one block:
//  * K: accumulator (mi, ni, 4 g' + c) of lane l is dim d0 + c, d0 =
//    ra0 + 32 mi + 8 g' + 4 (l / 32), of key rb0 + 32 ni + l % 32; dims d0 and
//    d0 + 2 (d0 + 1 and d0 + 3) are consecutive floats of one parity run, the
//    two lanes l and l + 32 fill a 16-byte slot together (512 bytes a store);
//  * V: accumulator (mi, ni, 4 g' + c) of lane l is key ra0 + 32 mi + 8 g' +
//    4 (l / 32) + c of dim rb0 + 32 ni + l % 32: one 16-byte slot per lane,
//    64 (4 (d / 32) + g') + l in the block (1 KB a store).
// Stores carry the non-temporal hint, as in the bf16 K/V epilogue (K and V
// are read once per routing layer; left dirty in the caches they cost the
// next kernels' reads a write-back).
struct EpiKV32 {
  const float* bias;
  float* kv;
  long long Tpad;
  static constexpr bool kF16 = false;
  static constexpr bool kDirect = false;
  static constexpr bool kRegs = true;
  static constexpr bool kBiasInit = false;
  static constexpr bool kPlain = true;   // V tiles are plain
  static constexpr int kWrapW = 1024;    // one [N][1024] weight read three times: its 2 MB column group stays in L2
  static constexpr int kImageBytes = 0;
  DEV int a_wrap() const { return 0; }
  DEV bool transposed(int tn) const { return !(((tn * BN) >> 10) & 1); }
  DEV void load_consts(int, int ocol0, int tid, float (&r)[4]) const { r[0] = bias[ocol0 + tid]; }
  DEV void put_consts(float* cst, int tid, const float (&r)[4]) const { cst[tid] = r[0]; }
  template <bool TR>
  DEV void store_regs(const f32x16 (&acc)[4][4], const float* cst, int orow0, int ocol0, int ra0, int rb0,
                      int lane) const {
    const int hh = lane >> 5;
    if constexpr (TR) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int lc = ra0 + mi * 32 + 8 * g + 4 * hh, n = ocol0 + lc, d0 = n & 63;
          const float4 b = *reinterpret_cast<const float4*>(cst + lc);
          float* base = kv + (size_t)(n >> 6) * Tpad * 64 + (size_t)((d0 >> 3) * 64 + (lane & 31)) * 4 + ((d0 >> 1) & 3);
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const f32x16& a = acc[mi][ni];
            float* blk = base + (size_t)((orow0 + rb0 + ni * 32) >> 5) * 2048;
            store_stream(blk, u32x2{__float_as_uint(a[4 * g] + b.x), __float_as_uint(a[4 * g + 2] + b.z)});
            store_stream(blk + 128, u32x2{__float_as_uint(a[4 * g + 1] + b.y), __float_as_uint(a[4 * g + 3] + b.w)});
          }
        }
    } else {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int lc = rb0 + ni * 32 + (lane & 31), n = ocol0 + lc;
        const float b = cst[lc];
        float* base = kv + (size_t)(n >> 6) * Tpad * 64 + (size_t)(((n & 63) >> 5) * 256 + lane) * 4;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const f32x16& a = acc[mi][ni];
          float* blk = base + (size_t)((orow0 + ra0 + mi * 32) >> 5) * 2048;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store_stream(blk + g * 256, u32x4{__float_as_uint(a[4 * g] + b), __float_as_uint(a[4 * g + 1] + b),
                                              __float_as_uint(a[4 * g + 2] + b), __float_as_uint(a[4 * g + 3] + b)});
        }
      }
    }
  }
};

// Split-K partial sums: K slice s of a tile writes its raw fp32 accumulators to
// part[s][row][col] (row in the packed row space, N columns); a reduction
// kernel sums the slices in order and applies the memory or K/V epilogue.
// Transposed tiles: a lane owns one output row and runs of 4 columns.
template <bool F16>
struct EpiPart {
  float* part;
  long long Tpad;
  int N;
  static constexpr bool kF16 = F16;
  static constexpr bool kDirect = true;
  static constexpr bool kRegs = false;
  static constexpr bool kBiasInit = false;
  static constexpr bool kPlain = false;
  static constexpr int kWrapW = 0;
  static constexpr int kImageBytes = 0;
  DEV int a_wrap() const { return 0; }
  DEV bool transposed(int) const { return true; }
  DEV void load_consts(int, int, int, float (&)[4]) const {}
  DEV void put_consts(float*, int, const float (&)[4]) const {}
  // orow / ocol: first output row / column of the wave's 128 x 128 block
  DEV void store_acc(const f32x16 (&acc)[4][4], int orow, int ocol, int s, int lane) const {
    float* base = part + ((size_t)s * Tpad + orow + (lane & 31)) * N + ocol + 4 * (lane >> 5);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = acc[mi][ni];
          *reinterpret_cast<float4*>(base + (size_t)ni * 32 * N + mi * 32 + 8 * g) =
              make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
  }
};

// Output tile of workgroup b.  Workgroups are dealt to the 8 XCDs round-robin
// (b % 8), each XCD with its own L2.  Column tiles are grouped in fours
// (256 x 4 W rows: 2 MB at K = 1024, 8 MB at K = 4096); XCD x works on column
// group x % G and on part x / G of the row tiles, taken in order, so the W
// slice it multiplies stays in its L2 while the A rows stream past, and each
// A row tile is fetched by G XCDs instead of once per column tile pass.
DEV void tile_order(int b, int ntm, int ntn, int& tm, int& tn) {
  const int G = ntn >> 2;
  if ((ntn & 3) == 0 && G <= 8 && (8 % G) == 0 && ((ntm * ntn) & 7) == 0) {
    const int x = b & 7, j = b >> 3, R = 8 / G;
    const int cg = x % G, part = x / G;
    const int u = part * (4 * ntm / R) + j;   // index in the group's row-major list of 4 ntm tiles
    tm = u >> 2;
    tn = 4 * cg + (u & 3);
  } else {
    const int lt = xcd_remap(b, ntm * ntn);
    tm = lt / ntn;
    tn = lt - tm * ntn;
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One 32x32x16 MFMA step on 16-byte operand fragments of either 16-bit type.
template <bool F16>
DEV f32x16 mfma32(const u32x4 a, const u32x4 b, const f32x16 c) {
  if constexpr (F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained to <= n
#define WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
// s_waitcnt lgkmcnt(0) only
#define WAIT_LDS() __builtin_amdgcn_s_waitcnt((7 << 4) | 15 | (3 << 14))

// Operand tiles are 64-deep K steps of 256 rows; rows are 128 B (eight
// 16-byte chunks) and chunk c of row r sits at position c ^ ((r >> 1) & 7),
// which keeps the fragment reads of 16 lanes on distinct banks.  Global -> LDS
// copies use buffer_load_dwordx4 ... lds: lane l of a wave writes the l-th
// 16-byte slot of a 1 KB block (8 rows), so each lane fetches the chunk that
// belongs in its slot.  Whole 128-byte row segments per copy stream about
// twice as fast into a CU as 64-byte ones.
//
// Per stage a wave runs four 16-deep substeps of 16 MFMAs, reading the next
// substep's fragments while the current one multiplies.  Each substep is
// written out as 8 fenced groups of (2 MFMAs, 1 fragment read, 1 copy): with
// the copies spread between the MFMAs instead of issued 8 at a time, a copy
// that cannot issue (operands missing in L2) stalls one group, not the
// matrix core's whole queue.
//
// Ring of five operand tiles of 32 KB (one operand of one stage: 256 rows x
// 128 B), the whole 160 KB of LDS.  Tile q of the sequence A_0, W_0, A_1,
// W_1, ... sits in slot q mod 5, so the A tile of stage s + 2 and the W tile
// of stage s + 1 are in flight while stage s multiplies: 96 KB of copies
// outstanding per CU instead of the 64 KB a two-stage ring allows, and the A
// rows (the operand that misses in L2) get two stages to land.  The tile
// constants wait in registers until the main loop is over and are then
// parked at the ring's end (kCstOff), clear of the output image.
constexpr int kHalfSlot = BM * 8;                  // u32x4 per operand tile
constexpr int kLdsBytes = 5 * kHalfSlot * 16;      // 160 KB
constexpr int kCstOff = kLdsBytes - kConstFloats * 4;

// One output tile (or one K slice of it) in orientation TR (true: transposed,
// the W rows are the MFMA A operand).  lds: the workgroup's operand ring.
template <class Epi, bool TR>
DEV void gemm_tile(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ W, int K, int nsplit, int ks,
                   int tn, const int4 T, const Epi& epi, unsigned char* lds) {
  static_assert(Epi::kImageBytes <= kCstOff, "output image overlaps the parked constants");
  constexpr int KS = 64;
  u32x4* ring = reinterpret_cast<u32x4*>(lds);
  float* cst = reinterpret_cast<float*>(lds + kCstOff);
  const int kbase = ks * (K / nsplit);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;     // 2 x 2 waves, each 128 x 128
  // transposed tiles feed the W rows as the MFMA A operand: acc rows are then
  // output columns and acc columns are A rows
  const int wa = TR ? wn : wm, wb = TR ? wm : wn;

  // copy sources: instruction i of wave w fills rows 8 (8 w + i) .. +8 of a tile.
  // Buffer copies: a uniform resource per operand (its record count bounds every
  // copy to the tile's valid rows), a 32-bit byte offset per lane, the K position
  // as the scalar offset.
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)(A + (size_t)T.x * lda), 0, T.z * lda * 2, 0x00020000);   // valid rows only
  // W rows are K long, or Epi::kWrapW long when the product's depth repeats
  // the weight (K position k reads W column k mod kWrapW, a power of two)
  constexpr int kWrap = Epi::kWrapW;
  const int ldw = kWrap ? kWrap : K;
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)(W + (size_t)(tn * BN) * ldw), 0, BN * ldw * 2, 0x00020000);
  // rows of copy i are 8 i after those of copy 0, so their swizzle term
  // ((row >> 1) & 7) differs by 4 i mod 8: even and odd copies use two bases.
  // Rows past the tile's valid count read zeros (outside the A resource).
  const int crow = 64 * w + (lane >> 3);
  const int cch = (lane & 7) ^ ((crow >> 1) & 7);
  const uint32_t aoffE = (uint32_t)(crow * lda + cch * 8) * 2, aoffO = (uint32_t)(crow * lda + (cch ^ 4) * 8) * 2;
  const uint32_t woffE = (uint32_t)(crow * ldw + cch * 8) * 2, woffO = (uint32_t)(crow * ldw + (cch ^ 4) * 8) * 2;
  const uint32_t astep = (uint32_t)(8 * lda) * 2, wstep = (uint32_t)(8 * ldw) * 2;
#define WCOL(k) (kWrap ? ((k) & (kWrap - 1)) : (k))
  // A rows are K long, or awrap long when the product's depth repeats them
  // (K = 3 awrap; K position k reads A column k mod awrap)
  const int awrap = epi.a_wrap();
#define ACOL(k) (awrap ? ((k) >= 2 * awrap ? (k) - 2 * awrap : (k) >= awrap ? (k) - awrap : (k)) : (k))
  // fragment positions: 32x32x16 operands, lane -> row (lane & 31), chunk 2 kk + (lane >> 5).
  // Block bases are multiples of 32 rows, so the swizzle depends on the lane only
  // and block i of a substep sits 256 chunks after block 0.
  const int l31 = lane & 31, hl = lane >> 5, fsw = (l31 >> 1) & 7;
  const int fa0 = (wa * 128 + l31) * 8, fb0 = (wb * 128 + l31) * 8;
  // slot q holds the A tile of a stage, slot q + 1 (mod 5) its W tile; the
  // MFMA A operand is the W tile in transposed tiles
#define M5(x) ((x) >= 5 ? (x) - 5 : (x))
#define BASE_A(q) ((TR ? M5((q) + 1) : (q)) * kHalfSlot + fa0)
#define BASE_B(q) ((TR ? (q) : M5((q) + 1)) * kHalfSlot + fb0)
#define CPA1(slot, k0, i)                                                                                   \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)&ring[(slot) * kHalfSlot + 64 * (w * 8 + (i))], 16, \
                                           (((i) & 1) ? aoffO : aoffE) + (i) * astep, ACOL(kbase + (k0)) * 2, 0, 0);
#define CPB1(slot, k0, i)                                                                                   \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_ptr_t)&ring[(slot) * kHalfSlot + 64 * (w * 8 + (i))], 16, \
                                           (((i) & 1) ? woffO : woffE) + (i) * wstep, WCOL(kbase + (k0)) * 2, 0, 0);
#define COPY_A(slot, k0) _Pragma("unroll") for (int i = 0; i < 8; ++i) CPA1(slot, k0, i)
#define COPY_B(slot, k0) _Pragma("unroll") for (int i = 0; i < 8; ++i) CPB1(slot, k0, i)
#define LOAD_FRAGS(F, BA, BB, kk)                                                \
  {                                                                              \
    const int ph_ = (2 * (kk) + hl) ^ fsw;                                       \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                              \
      F##a[i] = ring[(BA) + ph_ + i * 256];                                      \
      F##b[i] = ring[(BB) + ph_ + i * 256];                                      \
    }                                                                            \
  }
#define MULTIPLY(F)                                                                       \
  _Pragma("unroll") for (int mi = 0; mi < 4; ++mi)                                        \
  _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                                        \
    acc[mi][ni] = mfma32<Epi::kF16>(F##a[mi], F##b[ni], acc[mi][ni]);

  float kc[4];
  epi.load_consts(T.y, tn * BN, tid, kc);   // parked in LDS after the main loop

  f32x16 acc[4][4];
  float4 bq[4][4];                       // bias of the lane's accumulators (bias-initialized epilogues)
  if constexpr (Epi::kBiasInit) {
    epi.template bias_regs<TR>(bq, tn * BN, wa * 128, wb * 128, lane);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  }
  u32x4 Xa[4], Xb[4], Ya[4], Yb[4];

  const int nk = K / nsplit / KS;        // >= 4 (K / nsplit a multiple of 128, at least 256)
  // The prologue copies tiles A_0, W_0, A_1, W_1, A_2 and waits for the first
  // two only.  Stage s runs four substeps; during the first it copies W_{s+1},
  // during the second A_{s+2}, into the slots stage s - 1 freed.  The barrier
  // before the fourth substep (whose fragments are already in registers) needs
  // A_{s+1} and W_{s+1} landed and lets A_{s+2} stay in flight; it also frees
  // stage s's slots.  Each substep is 8 fenced groups of (2 MFMAs of the
  // current fragments, 1 fragment read for the next substep, 1 global->LDS copy
  // in the first two substeps), so the compiler keeps the order.
  COPY_A(0, 0)
  COPY_B(1, 0)
  COPY_A(2, KS)
  COPY_B(3, KS)
  COPY_A(4, 2 * KS)
  WAIT_VM(24);                           // the tile constants, A_0 and W_0 have landed
  if constexpr (Epi::kBiasInit) epi.template fill_acc<TR>(acc, bq);
  __builtin_amdgcn_s_barrier();
  LOAD_FRAGS(X, BASE_A(0), BASE_B(0), 0)
#define MFMA2(F, t)                                                                         \
  acc[(t) >> 1][((t) & 1) * 2] =                                                            \
      mfma32<Epi::kF16>(F##a[(t) >> 1], F##b[((t) & 1) * 2], acc[(t) >> 1][((t) & 1) * 2]); \
  acc[(t) >> 1][((t) & 1) * 2 + 1] =                                                        \
      mfma32<Epi::kF16>(F##a[(t) >> 1], F##b[((t) & 1) * 2 + 1], acc[(t) >> 1][((t) & 1) * 2 + 1]);
#define FRAG1(G, BA, BB, kk, t)                                                                 \
  {                                                                                             \
    const int ph_ = (2 * (kk) + hl) ^ fsw;                                                      \
    if ((t) < 4) G##a[(t)] = ring[(BA) + ph_ + ((t) & 3) * 256];                                \
    else G##b[(t) - 4] = ring[(BB) + ph_ + ((t) & 3) * 256];                                    \
  }
#define HALF_CP(F, G, BA, BB, gkk, CP, cslot, ck0)                                              \
  _Pragma("unroll") for (int t = 0; t < 8; ++t) {                                               \
    MFMA2(F, t)                                                                                 \
    FRAG1(G, BA, BB, gkk, t)                                                                    \
    CP(cslot, ck0, t)                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }
#define HALF(F, G, BA, BB, gkk)                                                                 \
  _Pragma("unroll") for (int t = 0; t < 8; ++t) {                                               \
    MFMA2(F, t)                                                                                 \
    FRAG1(G, BA, BB, gkk, t)                                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }
  {
    // stage 0: its copies were all issued by the prologue
    const int ba = BASE_A(0), bb = BASE_B(0);
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(X, Y, ba, bb, 1)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(Y, X, ba, bb, 2)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(X, Y, ba, bb, 3)
    WAIT_LDS();
    WAIT_VM(8);                          // A_1, W_1 landed; A_2 may be in flight
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    HALF(Y, X, BASE_A(2), BASE_B(2), 0)
  }
  int q = 2;                             // slot of stage kt's A tile: 2 kt mod 5
  for (int kt = 1; kt + 2 < nk; ++kt) {
    const int ba = BASE_A(q), bb = BASE_B(q), qn = M5(q + 2);
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF_CP(X, Y, ba, bb, 1, CPB1, M5(q + 3), (kt + 1) * KS)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF_CP(Y, X, ba, bb, 2, CPA1, M5(q + 4), (kt + 2) * KS)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(X, Y, ba, bb, 3)
    WAIT_LDS();
    WAIT_VM(8);                          // A_{kt+1}, W_{kt+1} landed; A_{kt+2} may be in flight
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    HALF(Y, X, BASE_A(qn), BASE_B(qn), 0)
    q = qn;
  }
  {
    // stage nk - 2: copies the last W tile only
    const int ba = BASE_A(q), bb = BASE_B(q), qn = M5(q + 2);
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF_CP(X, Y, ba, bb, 1, CPB1, M5(q + 3), (nk - 1) * KS)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(Y, X, ba, bb, 2)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(X, Y, ba, bb, 3)
    WAIT_LDS();
    WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    HALF(Y, X, BASE_A(qn), BASE_B(qn), 0)
    q = qn;
  }
  {
    const int ba = BASE_A(q), bb = BASE_B(q);
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(X, Y, ba, bb, 1)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(Y, X, ba, bb, 2)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    HALF(X, Y, ba, bb, 3)
    WAIT_LDS();
    __builtin_amdgcn_sched_barrier(0);
    MULTIPLY(Y)
    __builtin_amdgcn_sched_barrier(0);
  }
#undef WCOL
#undef ACOL
#undef M5
#undef BASE_A
#undef BASE_B
#undef MFMA2
#undef FRAG1
#undef CPA1
#undef CPB1
#undef HALF_CP
#undef HALF
#undef COPY_A
#undef COPY_B
#undef LOAD_FRAGS
#undef MULTIPLY

  // All 256 rows are stored: rows past the valid count come from clamped
  // (finite) inputs and keep the padded part of the row space finite.
  if constexpr (Epi::kDirect) {
    epi.store_acc(acc, T.y + wb * 128, tn * BN + wa * 128, ks, lane);
  } else if constexpr (Epi::kBiasInit) {
    epi.template store_regs<TR>(acc, cst, T.y, tn * BN, wa * 128, wb * 128, lane);
  } else {
    __syncthreads();                     // every wave is done with the operand ring
    epi.put_consts(cst, tid, kc);
    __syncthreads();
    if constexpr (Epi::kRegs) {
      epi.template store_regs<TR>(acc, cst, T.y, tn * BN, wa * 128, wb * 128, lane);
    } else {
      bf16_t* img = reinterpret_cast<bf16_t*>(lds);
      epi.stage_t(acc, cst, img, wb * 128, wa * 128, lane);
      __syncthreads();
      epi.store(img, T.y, tn * BN, tid);
    }
  }
}

template <class Epi>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm256(const bf16_t* __restrict__ A, int lda, const int4* __restrict__ tiles, int ntile_n,
               const bf16_t* __restrict__ W, int K, int nsplit, Epi epi) {
  // operand ring: five tiles [row * 8 + swizzled chunk] (after the main loop
  // the same bytes hold the output image and the tile constants)
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  // nsplit > 1: workgroup b multiplies K slice b / (tiles) of length K / nsplit
  const int ntiles_mn = gridDim.x / nsplit;
  const int ks = blockIdx.x / ntiles_mn;
  int tm, tn;
  tile_order(blockIdx.x - ks * ntiles_mn, ntiles_mn / ntile_n, ntile_n, tm, tn);
  const int4 T = tiles[tm];              // (first A row, first output row, valid rows, record)
  // the orientation is uniform over the workgroup; each is compiled on its own
  if constexpr (Epi::kPlain) {
    if (!epi.transposed(tn)) {
      gemm_tile<Epi, false>(A, lda, W, K, nsplit, ks, tn, T, epi, lds);
      return;
    }
  }
  gemm_tile<Epi, true>(A, lda, W, K, nsplit, ks, tn, T, epi, lds);
}


// Sum of the split-K slices of the memory GEMM, then the folded-LayerNorm
// epilogue m = rstd (sum - mu c) + d (the same arithmetic as the unsplit
// epilogue); every row of the packed row space is written.  8 columns per thread.
__global__ __launch_bounds__(256) void k_mem_reduce(const float* __restrict__ part, int nsplit, long long Tpad,
                                                    long long row0, long long nrows,
                                                    const float2* __restrict__ stats, const float* __restrict__ c,
                                                    const float* __restrict__ d, bf16_t* __restrict__ out) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;   // 8-column group
  if ((i >> 7) >= nrows) return;
  const long long row = row0 + (i >> 7);
  const int col = (int)(i & 127) * 8;
  float a[8];
  const float* p = part + row * 1024 + col;
  {
    const float4 x = *reinterpret_cast<const float4*>(p), y = *reinterpret_cast<const float4*>(p + 4);
    a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w; a[4] = y.x; a[5] = y.y; a[6] = y.z; a[7] = y.w;
  }
  for (int s = 1; s < nsplit; ++s) {
    const float* q = p + (size_t)s * Tpad * 1024;
    const float4 x = *reinterpret_cast<const float4*>(q), y = *reinterpret_cast<const float4*>(q + 4);
    a[0] += x.x; a[1] += x.y; a[2] += x.z; a[3] += x.w; a[4] += y.x; a[5] += y.y; a[6] += y.z; a[7] += y.w;
  }
  const float2 st = stats[row];
  uint4 v;
  uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = pack_bf16x2(st.y * (a[2 * k] - st.x * c[col + 2 * k]) + d[col + 2 * k],
                       st.y * (a[2 * k + 1] - st.x * c[col + 2 * k + 1]) + d[col + 2 * k + 1]);
  *reinterpret_cast<uint4*>(out + row * 1024 + col) = v;
}

// Sum of the split-K slices of the K/V GEMM plus bias, written in the routing
// attention's layouts (32-row blocks of one head in fragment order, kchunk()
// and vchunk(); V keys at vblock_pos()).  One block per (32-row block, head of
// one K or V): the sums are staged in LDS, then written as one 4 KB block.
__global__ __launch_bounds__(256) void k_kv_reduce(const float* __restrict__ part, int nsplit, long long Tpad,
                                                   long long rbase, const float* __restrict__ bias,
                                                   bf16_t* __restrict__ kv) {
  __shared__ float tile[32][65];
  const long long row0 = rbase + (long long)blockIdx.x * 32;
  const int hc = blockIdx.y;                 // 64-column group: layer r = hc / 32, V if (hc / 16) & 1
  const int N = gridDim.y * 64;
  const int t = threadIdx.x, r = t >> 3, c8 = (t & 7) * 8;
  const float* p = part + (row0 + r) * N + hc * 64 + c8;
  float a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = p[k];
  for (int s = 1; s < nsplit; ++s) {
    const float* q = p + (size_t)s * Tpad * N;
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] += q[k];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) tile[r][c8 + k] = a[k] + bias[hc * 64 + c8 + k];
  __syncthreads();
  const bool isv = (hc >> 4) & 1;
  bf16_t* head = kv + (size_t)hc * (size_t)Tpad * 64;   // hc = (2 layer + isv) * 16 + head
  uint4 v;
  uint32_t* w = reinterpret_cast<uint32_t*>(&v);
  if (!isv) {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(tile[r][c8 + 2 * k], tile[r][c8 + 2 * k + 1]);
    *reinterpret_cast<uint4*>(head + (row0 >> 5) * 2048 + kchunk(r, c8 >> 3) * 8) = v;
  } else {
    const int f = t >> 2, p0 = (t & 3) * 8;  // feature row f, key positions p0 .. p0 + 7
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = pack_bf16x2(tile[vblock_pos(p0 + 2 * k)][f], tile[vblock_pos(p0 + 2 * k + 1)][f]);
    *reinterpret_cast<uint4*>(head + (row0 >> 5) * 2048 + vchunk(f, p0 >> 3) * 8) = v;
  }
}

}  // namespace

int big_gemm_split(int ntiles, int ntn, int K) {
  // Every slice adds 2 * Tpad * N * 4 bytes of partial-sum traffic, so the
  // split stops at 8 slices (16 were no faster on the single-record batch).
  // Grids of more than 64 tiles stay whole: the forward's side stream fills
  // the CUs they leave idle, and splitting them (B=1, L=2048 K/V GEMM; B=2,
  // L=4096 memory GEMM) made the whole forward slower.
  const int base = ntiles * ntn;
  if (base > 64) return 1;
  int s = 1;
  while (s < 8 && 2 * s * base <= 256 && K / (2 * s) >= 256 && (K / (2 * s)) % 128 == 0) s *= 2;
  return s;
}

void launch_gemm_mem(hipStream_t st, const bf16_t* hidden, int H, bool f16, const int4* tiles, int ntiles,
                     const bf16_t* Wm, const float2* stats, const float* c, const float* d, bf16_t* mem,
                     float* part, long long Tpad, int split, long long row0) {
  if (ntiles == 0) return;
  // the main loop needs at least 3 stages of 64: H is a multiple of 512 and every slice at least 256 deep
  const int ntn = 1024 / BN;
  const int S = !part ? 1 : split > 0 ? split : big_gemm_split(ntiles, ntn, H);
  const dim3 grid(ntiles * ntn * S);
  if (S > 1) {
    if (f16) {
      hipLaunchKernelGGL(k_gemm256<EpiPart<true>>, grid, dim3(256), 0, st, hidden, H, tiles, ntn, Wm, H, S,
                         EpiPart<true>{part, Tpad, 1024});
    } else {
      hipLaunchKernelGGL(k_gemm256<EpiPart<false>>, grid, dim3(256), 0, st, hidden, H, tiles, ntn, Wm, H, S,
                         EpiPart<false>{part, Tpad, 1024});
    }
    const long long nrows = (long long)ntiles * BM;
    hipLaunchKernelGGL(k_mem_reduce, dim3((unsigned)((nrows * 128 + 255) / 256)), dim3(256), 0, st, part, S, Tpad,
                       row0, nrows, stats, c, d, mem);
    return;
  }
  EpiMem epi{stats, c, d, mem};
  if (f16) {
    EpiMem16 e16;
    static_cast<EpiMem&>(e16) = epi;
    hipLaunchKernelGGL(k_gemm256<EpiMem16>, grid, dim3(256), 0, st, hidden, H, tiles, ntn, Wm, H, 1, e16);
  } else {
    hipLaunchKernelGGL(k_gemm256<EpiMem>, grid, dim3(256), 0, st, hidden, H, tiles, ntn, Wm, H, 1, epi);
  }
}

void launch_gemm_mem32(hipStream_t st, const bf16_t* xplanes, int H, const int4* tiles, int ntiles,
                       const bf16_t* Wm3, const float* bias, float* mem, bf16_t* mplanes) {
  if (ntiles == 0) return;
  hipLaunchKernelGGL(k_gemm256<EpiMem32>, dim3(ntiles * (1024 / BN)), dim3(256), 0, st, xplanes, 3 * H, tiles,
                     1024 / BN, Wm3, 3 * H, 1, EpiMem32{nullptr, nullptr, bias, mem, mplanes, 0});
}

void launch_gemm_mem32_folded(hipStream_t st, const bf16_t* hidden, int H, const int4* tiles, int ntiles,
                              const bf16_t* Wt3, const float2* stats, const float* c, const float* d, float* mem,
                              bf16_t* mplanes) {
  if (ntiles == 0) return;
  hipLaunchKernelGGL(k_gemm256<EpiMem32>, dim3(ntiles * (1024 / BN)), dim3(256), 0, st, hidden, H, tiles,
                     1024 / BN, Wt3, 3 * H, 1, EpiMem32{stats, c, d, mem, mplanes, H});
}

void launch_gemm_kv32(hipStream_t st, const bf16_t* mplanes, const int4* tiles, int ntiles, const bf16_t* Wkv,
                      const float* bias, int n_layers, float* kv, long long Tpad) {
  if (ntiles == 0 || n_layers == 0) return;
  const int ntn = n_layers * 2048 / BN;
  hipLaunchKernelGGL(k_gemm256<EpiKV32>, dim3(ntiles * ntn), dim3(256), 0, st, mplanes, 3 * 1024, tiles, ntn, Wkv,
                     3 * 1024, 1, EpiKV32{bias, kv, Tpad});
}

void launch_gemm_kv(hipStream_t st, const bf16_t* mem, const int4* tiles, int ntiles, const bf16_t* Wkv,
                    const float* bkv, int n_layers, bf16_t* kv, long long Tpad, float* part, int split,
                    long long row0) {
  if (ntiles == 0 || n_layers == 0) return;
  const int ntn = n_layers * 2048 / BN;
  const int S = !part ? 1 : split > 0 ? split : big_gemm_split(ntiles, ntn, 1024);
  if (S > 1) {
    hipLaunchKernelGGL(k_gemm256<EpiPart<false>>, dim3(ntiles * ntn * S), dim3(256), 0, st, mem, 1024, tiles, ntn,
                       Wkv, 1024, S, EpiPart<false>{part, Tpad, n_layers * 2048});
    hipLaunchKernelGGL(k_kv_reduce, dim3((unsigned)(ntiles * (BM / 32)), n_layers * 32), dim3(256), 0, st, part, S,
                       Tpad, row0, bkv, kv);
    return;
  }
  EpiKV epi{bkv, kv, Tpad};
  hipLaunchKernelGGL(k_gemm256<EpiKV>, dim3(ntiles * ntn), dim3(256), 0, st, mem, 1024, tiles, ntn, Wkv, 1024, 1,
                     epi);
}

}  // namespace clef
