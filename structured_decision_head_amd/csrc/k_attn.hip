// Attention kernels of the head.
//
// Evidence routing (clef-4bit page §三 step 2; Clef-Flash overview §三): all
// option queries of a record attend, per head, over every valid memory row of
// that record.  The keys are split into chunks (a multiple of 64 rows, chosen
// per batch); one wave owns (record, key chunk, block of 32 queries, head) and
// writes flash-decode partials (running max, running sum, unnormalised output)
// that k_route_combine merges.  Scores and the value mix run on the matrix
// cores in a transposed form (S^T = K Q^T, O^T = V^T P^T) so that each lane
// owns one query: the softmax statistics stay lane-local and the
// probabilities are already in the B-operand layout of the second product
// (v_mfma_f32_32x32x16_bf16 in the bf16 kernel, v_mfma_f32_32x32x2_f32 in
// the fp32 one).
//
// Field self-attention (clef-4bit page §三 step 3): every field of a record
// attends to every field of the same record; tiny (a few dozen fields), so
// fp32 vector arithmetic with an online softmax, followed on the matrix cores
// by the head's share of the output projection.
#include "kernels.hpp"

namespace clef {

namespace {

// K rows of one 32-key step (A operand of S^T = K Q^T) and the V^T fragments
// (A operand of O^T = V^T P^T) for both 16-key halves and both 32-dim halves.
struct KV32 {
  u32x4 k[4];
  u32x4 v[2][2];
};

// K and V are stored in 4 KB blocks of 32 keys already in fragment order:
// fragment q of the block holds lane l's 16 bytes at element 512 q + 8 l
// (K: q = 16-dim group kk; V: q = 2 t + dt), one contiguous 1 KB per load.
DEV void kv_load(KV32& r, const bf16_t* Kj, const bf16_t* Vj, int row0, int lane) {
  const bf16_t* kp = Kj + (size_t)(row0 >> 5) * 2048 + lane * 8;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) r.k[kk] = *reinterpret_cast<const u32x4*>(kp + kk * 512);
  const bf16_t* vp = Vj + (size_t)(row0 >> 5) * 2048 + lane * 8;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) r.v[t][dt] = *reinterpret_cast<const u32x4*>(vp + (2 * t + dt) * 512);
}

// One 32-key step of the online softmax for the wave's 32 queries.
// The queries carry the score scale (log2(e) / sqrt(64)), so scores come out
// in log2 units.
DEV void kv_step(const KV32& r, const bf16x8 (&qf)[4], int kb, int n, int g, float& m, float& l, f32x16 (&o)[2]) {
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(r.k[kk]), qf[kk], s, 0, 0, 0);
  // lane owns query (lane & 31) and keys kb + 8 (e / 4) + 4 g + (e % 4); only
  // the record's last step has keys past its end
  float mx = -INFINITY;
  if (kb + 32 <= n) {
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kb + 8 * (e >> 2) + 4 * g + (e & 3);
      s[e] = (key < n) ? s[e] : -INFINITY;
      mx = fmaxf(mx, s[e]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mn = fmaxf(m, mx);          // finite: key kb < n is always valid
  // v_exp_f32 directly, without the library's rescaling for results below
  // 2^-126 (those may come out as zero: no weight that small matters next to
  // the running maximum's weight of 1)
  const float alpha = __builtin_amdgcn_exp2f(m - mn);   // m = -inf gives 0
  float ls = 0.f, p[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    p[e] = __builtin_amdgcn_exp2f(s[e] - mn);
    ls += p[e];
  }
  ls += __shfl_xor(ls, 32, 64);
  l = l * alpha + ls;
  m = mn;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    o[0][e] *= alpha;
    o[1][e] *= alpha;
  }
  // the k-slot (g, e) of half t is key kb + 16 t + 8 (e / 4) + 4 g + (e % 4)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bf16x8 pf = as_bf16x8(pack8(p + 8 * t));
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(r.v[t][dt]), pf, o[dt], 0, 0, 0);
  }
}

}  // namespace

// rec: per record 8 ints: kv0 (first row in the packed padded row space),
// n (valid rows), o0 (first option), no (options), pbase, nc (chunks), q0, nq.
// One wave per (record, head, chunk of `chunk` keys, block of 32 queries);
// the next two 32-key steps' K and V are in flight while the current one is
// multiplied.  Query blocks of one chunk re-read the same K/V rows from cache.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_route_attn(const float* __restrict__ Q, const bf16_t* __restrict__ Kl,
                                                    const bf16_t* __restrict__ Vl, long long Tpad,
                                                    const int4* __restrict__ items, int nitems,
                                                    const int* __restrict__ rec, float* __restrict__ pm,
                                                    float* __restrict__ pl, float* __restrict__ po, long long Ptot,
                                                    int chunk, float scale_log2) {
  const int lane = threadIdx.x & 63;
  // consecutive item groups of one head (the query blocks of one key chunk)
  // go to the same XCD, so they share the chunk through its L2
  const int gx = gridDim.x;
  const int rl = xcd_remap(blockIdx.x + blockIdx.y * gx, gx * gridDim.y);
  const int it = (rl % gx) * 4 + (threadIdx.x >> 6);
  if (it >= nitems) return;
  const int j = rl / gx;
  const int4 bc = items[it];             // (record, chunk, first query of the block, -)
  const int* R = rec + 8 * bc.x;
  const int kv0 = R[0], n = R[1], o0 = R[2], no = R[3], pbase = R[4], nc = R[5];
  const int c = bc.y;
  const int k_lo = c * chunk, k_hi = min(n, k_lo + chunk);
  const bf16_t* Kj = Kl + (size_t)j * Tpad * 64;
  const bf16_t* Vj = Vl + (size_t)j * Tpad * 64;
  const int g = lane >> 5, l32 = lane & 31;

  {
    const int qi = bc.z + l32;
    const bool qvalid = qi < no;
    bf16x8 qf[4];
    {
      const float* qp = Q + (size_t)(o0 + (qvalid ? qi : 0)) * 1024 + j * 64 + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        float x[8];
        const float4 a = *reinterpret_cast<const float4*>(qp + kk * 16);
        const float4 b = *reinterpret_cast<const float4*>(qp + kk * 16 + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = qvalid ? x[e] * scale_log2 : 0.f;
        qf[kk] = as_bf16x8(pack8(x));
      }
    }
    float m = -INFINITY, l = 0.f;
    f32x16 o[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[0][e] = o[1][e] = 0.f;

    // three 32-key steps per iteration so that the triple buffer has static
    // registers: two steps' K and V are in flight while one is multiplied.
    // The loads are unconditional, their block clamped to the chunk's last
    // one (a step past the end re-reads it, from cache): a load under a
    // branch would make the compiler's wait before each step conservative,
    // waiting for the loads just issued instead of those two steps old.
    const int klast = kv0 + ((k_hi - 1) & ~31);
    KV32 a, b, c3;
    kv_load(a, Kj, Vj, kv0 + k_lo, lane);
    kv_load(b, Kj, Vj, min(kv0 + k_lo + 32, klast), lane);
    for (int kb = k_lo; kb < k_hi; kb += 96) {
      kv_load(c3, Kj, Vj, min(kv0 + kb + 64, klast), lane);
      kv_step(a, qf, kb, n, g, m, l, o);
      if (kb + 32 >= k_hi) break;
      kv_load(a, Kj, Vj, min(kv0 + kb + 96, klast), lane);
      kv_step(b, qf, kb + 32, n, g, m, l, o);
      if (kb + 64 >= k_hi) break;
      kv_load(b, Kj, Vj, min(kv0 + kb + 128, klast), lane);
      kv_step(c3, qf, kb + 64, n, g, m, l, o);
    }
    if (qvalid) {
      const size_t slot = (size_t)j * Ptot + pbase + (size_t)qi * nc + c;
      if (g == 0) {
        pm[slot] = m;
        pl[slot] = l;
      }
      float* op = po + slot * 64;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(op + dt * 32 + 8 * i + 4 * g) =
              make_float4(o[dt][4 * i], o[dt][4 * i + 1], o[dt][4 * i + 2], o[dt][4 * i + 3]);
    }
  }
}

void launch_route_attn(hipStream_t st, const float* Q, const bf16_t* Kl, const bf16_t* Vl, long long Tpad,
                       const int4* items, int nitems, const int* rec, float* pm, float* pl, float* po,
                       long long Ptot, int chunk) {
  if (nitems == 0) return;
  const float scale_log2 = 0.125f * 1.4426950408889634f;   // 1/sqrt(64) * log2(e)
  hipLaunchKernelGGL(k_route_attn, dim3((nitems + 3) / 4, 16), dim3(256), 0, st, Q, Kl, Vl, Tpad, items, nitems,
                     rec, pm, pl, po, Ptot, chunk, scale_log2);
}

namespace {

// fp32 K or V of one 32-key step: 8 fragments, fragment q at float4 index
// 64 q + lane of the 2048-float block (k32_off / v32_off order).
DEV void frag_load32(f32x4 (&r)[8], const float* P, int row0, int lane) {
  const float* p = P + (size_t)(row0 >> 5) * 2048 + lane * 4;
#pragma unroll
  for (int q = 0; q < 8; ++q) r[q] = *reinterpret_cast<const f32x4*>(p + q * 256);
}

// One 32-key step in fp32 on v_mfma_f32_32x32x2_f32 (A: lane l gives row
// l % 32 at depth l / 32; B: column l % 32 at depth l / 32).  S^T = K Q^T as
// 32 depth-2 products (product i: dims 2 i, 2 i + 1; lane l holds query l % 32
// at dims 2 i + l / 32); the lane then owns query l % 32 and keys
// kb + 8 (e / 4) + 4 g + (e % 4) as in the bf16 kernel, and product i of
// O^T = V^T P^T takes exactly those keys for e = i.
DEV void kv_step32(const f32x4 (&k)[8], const f32x4 (&v)[8], const float (&q)[32], int kb, int n, int g, float& m,
                   float& l, f32x16 (&o)[2]) {
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) s = __builtin_amdgcn_mfma_f32_32x32x2f32(k[i >> 2][i & 3], q[i], s, 0, 0, 0);
  float mx = -INFINITY;
  if (kb + 32 <= n) {
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kb + 8 * (e >> 2) + 4 * g + (e & 3);
      s[e] = (key < n) ? s[e] : -INFINITY;
      mx = fmaxf(mx, s[e]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mn = fmaxf(m, mx);          // finite: key kb < n is always valid
  // v_exp_f32 as in the bf16 kernel (its only difference from the library's
  // exp2f: results below 2^-126 may come out as zero)
  const float alpha = __builtin_amdgcn_exp2f(m - mn);   // m = -inf gives 0
  float ls = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    s[e] = __builtin_amdgcn_exp2f(s[e] - mn);
    ls += s[e];
  }
  ls += __shfl_xor(ls, 32, 64);
  l = l * alpha + ls;
  m = mn;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    o[0][e] *= alpha;
    o[1][e] *= alpha;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[4 * dt + (i >> 2)][i & 3], s[i], o[dt], 0, 0, 0);
}

}  // namespace

// fp32 routing attention (precision mode fp32): the bf16 kernel's work split
// (one wave per (record, chunk, 32-query block, head)) with fp32 operands on
// the matrix cores; the next 32-key step's keys and values are loaded while
// the current one is multiplied.  The queries carry log2(e) / sqrt(64) and the
// partials are written exactly as k_route_attn writes them, so
// k_route_combine merges either.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_route_attn32(
    const float* __restrict__ Q, const float* __restrict__ Kl, const float* __restrict__ Vl, long long Tpad,
    const int4* __restrict__ items, int nitems, const int* __restrict__ rec, float* __restrict__ pm,
    float* __restrict__ pl, float* __restrict__ po, long long Ptot, int chunk, float scale_log2) {
  const int lane = threadIdx.x & 63;
  const int gx = gridDim.x;
  const int rl = xcd_remap(blockIdx.x + blockIdx.y * gx, gx * gridDim.y);
  const int it = (rl % gx) * 4 + (threadIdx.x >> 6);
  if (it >= nitems) return;
  const int j = rl / gx;
  const int4 bc = items[it];             // (record, chunk, first query of the block, -)
  const int* R = rec + 8 * bc.x;
  const int kv0 = R[0], n = R[1], o0 = R[2], no = R[3], pbase = R[4], nc = R[5];
  const int c = bc.y;
  const int k_lo = c * chunk, k_hi = min(n, k_lo + chunk);   // every chunk holds at least one key
  const float* Kj = Kl + (size_t)j * Tpad * 64;
  const float* Vj = Vl + (size_t)j * Tpad * 64;
  const int g = lane >> 5, l32 = lane & 31;
  const int qi = bc.z + l32;
  const bool qvalid = qi < no;
  float q[32];
  {
    const float* qp = Q + (size_t)(o0 + (qvalid ? qi : 0)) * 1024 + j * 64;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(qp + 4 * t);   // dims 4 t .. 4 t + 3
      q[2 * t] = qvalid ? a[g] * scale_log2 : 0.f;
      q[2 * t + 1] = qvalid ? a[2 + g] * scale_log2 : 0.f;
    }
  }
  float m = -INFINITY, l = 0.f;
  f32x16 o[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[0][e] = o[1][e] = 0.f;

  // K is double-buffered (two 32-key steps per iteration, so that both
  // buffers have static registers); V has one buffer, refilled for the next
  // step as soon as the current step's value products have been issued, and
  // needed only after that step's scores and softmax
  // (loads unconditional, their block clamped to the chunk's last one, as in
  // the bf16 kernel, so that each wait covers only the loads it needs)
  const int klast = kv0 + ((k_hi - 1) & ~31);
  f32x4 ka[8], kb2[8], v[8];
  frag_load32(ka, Kj, kv0 + k_lo, lane);
  frag_load32(v, Vj, kv0 + k_lo, lane);
  for (int kb = k_lo; kb < k_hi; kb += 64) {
    frag_load32(kb2, Kj, min(kv0 + kb + 32, klast), lane);
    kv_step32(ka, v, q, kb, n, g, m, l, o);
    if (kb + 32 >= k_hi) break;
    frag_load32(v, Vj, kv0 + kb + 32, lane);
    frag_load32(ka, Kj, min(kv0 + kb + 64, klast), lane);
    kv_step32(kb2, v, q, kb + 32, n, g, m, l, o);
    frag_load32(v, Vj, min(kv0 + kb + 64, klast), lane);
  }
  if (qvalid) {
    const size_t slot = (size_t)j * Ptot + pbase + (size_t)qi * nc + c;
    if (g == 0) {
      pm[slot] = m;
      pl[slot] = l;
    }
    float* op = po + slot * 64;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(op + dt * 32 + 8 * i + 4 * g) =
            make_float4(o[dt][4 * i], o[dt][4 * i + 1], o[dt][4 * i + 2], o[dt][4 * i + 3]);
  }
}

void launch_route_attn32(hipStream_t st, const float* Q, const float* Kl, const float* Vl, long long Tpad,
                         const int4* items, int nitems, const int* rec, float* pm, float* pl, float* po,
                         long long Ptot, int chunk) {
  if (nitems == 0) return;
  const float scale_log2 = 0.125f * 1.4426950408889634f;   // 1/sqrt(64) * log2(e)
  hipLaunchKernelGGL(k_route_attn32, dim3((nitems + 3) / 4, 16), dim3(256), 0, st, Q, Kl, Vl, Tpad, items, nitems,
                     rec, pm, pl, po, Ptot, chunk, scale_log2);
}

// Merge the chunk partials of (option, head): one wave.  Lanes split the
// chunks to find the global max and the softmax denominator; then lane d sums
// the rescaled unnormalised outputs of every chunk for output dim d, with the
// chunk weights broadcast from the lane that computed them.
__global__ __launch_bounds__(256) void k_route_combine(const float* __restrict__ pm, const float* __restrict__ pl,
                                                       const float* __restrict__ po, long long Ptot,
                                                       const int* __restrict__ opt_rec, const int* __restrict__ rec,
                                                       int NO, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (k >= NO) return;
  const int j = blockIdx.y;
  const int* R = rec + 8 * opt_rec[k];
  const int o0 = R[2], pbase = R[4], nc = R[5];
  const size_t s0 = (size_t)j * Ptot + pbase + (size_t)(k - o0) * nc;
  float M = -INFINITY;
  for (int c = lane; c < nc; c += 64) M = fmaxf(M, pm[s0 + c]);
  M = wave_max(M);
  float Lsum = 0.f;
  for (int c = lane; c < nc; c += 64) Lsum += exp2f(pm[s0 + c] - M) * pl[s0 + c];
  Lsum = wave_sum(Lsum);
  float O = 0.f;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    const float a_mine = (c0 + lane < nc) ? exp2f(pm[s0 + c0 + lane] - M) : 0.f;
    const int cn = min(64, nc - c0);
    const float* pp = po + (s0 + c0) * 64 + lane;
    int c = 0;
    for (; c + 8 <= cn; c += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = pp[(size_t)(c + i) * 64];
#pragma unroll
      for (int i = 0; i < 8; ++i) O += __shfl(a_mine, c + i, 64) * v[i];
    }
    for (; c < cn; ++c) O += __shfl(a_mine, c, 64) * pp[(size_t)c * 64];
  }
  out[(size_t)k * 1024 + j * 64 + lane] = O / Lsum;
}

void launch_route_combine(hipStream_t st, const float* pm, const float* pl, const float* po, long long Ptot,
                          const int* opt_rec, const int* rec, int NO, float* out) {
  if (NO == 0) return;
  hipLaunchKernelGGL(k_route_combine, dim3((NO + 3) / 4, 16), dim3(256), 0, st, pm, pl, po, Ptot, opt_rec, rec, NO,
                     out);
}

// Field self-attention with its output projection: one 256-thread block per
// (record, head).  Thread t owns query row t / 4 of a 64-row block and 16 of
// its 64 dims (t % 4); a score is the sum of the four partial dot products
// (two lane exchanges).  Keys and values are staged in LDS 64 rows at a time
// with an online softmax, so any number of fields works.  QKV rows are
// [q | k | v] of width 3 x 1024.
//
// The head's 64 output dims then meet the matching 64 columns of W_o (the
// K range [64 j, 64 j + 64) of the [1024][1024] product): the block's rows
// go to LDS as NT exact-or-near bf16 terms (as in the small GEMMs) and the
// four waves multiply them with v_mfma_f32_16x16x32_bf16 against W_o's
// fragment-order blocks, 256 output columns each.  The result is split-K
// slice j of attn W_o^T, left at P + j * pstride + row * 1024 for the
// reduction that adds the 16 slices in order with the bias and the residual.
// With gridDim.z = cs > 1 (a small batch, fewer blocks than compute units)
// each block repeats the small attention and keeps only the output columns of
// part blockIdx.z, 1024 / cs of them, in 4 / cs passes instead of 4.
template <int NT>
__global__ __launch_bounds__(256) void k_field_attn(const float* __restrict__ QKV, int nsplit, size_t stride,
                                                    const float* __restrict__ bqkv, const int* __restrict__ rec,
                                                    const bf16_t* __restrict__ Wo, float* __restrict__ P,
                                                    size_t pstride) {
  __shared__ float4 sK[64][16], sV[64][16];
  __shared__ uint4 sO[NT][64][9];   // [term][row][8-dim chunk], one chunk of padding per row
  const int* R = rec + 8 * blockIdx.x;
  const int q0 = R[6], nq = R[7];
  const int j = blockIdx.y;
  const int t = threadIdx.x, qi_l = t >> 2, part = t & 3;
  const int w = t >> 6, lane = t & 63;
  // W_o block (16-column strip n16, K step k32) at (n16 * 32 + k32) * 512, lane
  // l's 8 values at 8 l.  The fragments of the wave's first pass are loaded
  // before the attention (they depend on the head only), each later pass's
  // while the previous pass multiplies.
  const int npass = 4 / gridDim.z;
  const int sw = (int)blockIdx.z * 16 * npass + 4 * npass * w;   // the wave's first 16-column strip
  const bf16_t* wo = Wo + ((size_t)sw * 32 + 2 * j) * 512 + lane * 8;
  uint4 b[4][2], bn[4][2];
#define FA_LOAD_WO(dst, GQ)                                                                           \
  _Pragma("unroll") for (int cb = 0; cb < 4; ++cb)                                                    \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk)                                                  \
      dst[cb][kk] = *reinterpret_cast<const uint4*>(wo + ((size_t)(4 * (GQ) + cb) * 32 + kk) * 512);
  FA_LOAD_WO(b, 0)
  for (int qb = 0; qb < nq; qb += 64) {
    const int qi = qb + qi_l;
    const bool valid = qi < nq;
    float4 q[4], o[4];
    const size_t qo = (size_t)(q0 + (valid ? qi : 0)) * 3072 + j * 64 + part * 16;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      q[c] = sum_slices4(QKV + qo + 4 * c, nsplit, stride, bqkv + j * 64 + part * 16 + 4 * c);
      q[c].x *= 0.125f; q[c].y *= 0.125f; q[c].z *= 0.125f; q[c].w *= 0.125f;
      o[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float m = -INFINITY, l = 0.f;
    for (int kb = 0; kb < nq; kb += 64) {
      const int nk = min(64, nq - kb);
      // the previous block's keys, or the previous query block's output terms, are still being read
      if (qb > 0 || kb > 0) __syncthreads();
      // 64 rows x 16 float4 each for K and V: 4 float4 per thread
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int idx = t + 256 * r, row = idx >> 4, c4 = idx & 15;
        if (row < nk) {
          const size_t ro = (size_t)(q0 + kb + row) * 3072 + j * 64 + 4 * c4;
          sK[row][c4] = sum_slices4(QKV + ro + 1024, nsplit, stride, bqkv + 1024 + j * 64 + 4 * c4);
          sV[row][c4] = sum_slices4(QKV + ro + 2048, nsplit, stride, bqkv + 2048 + j * 64 + 4 * c4);
        }
      }
      __syncthreads();
      for (int tk = 0; tk < nk; ++tk) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 k = sK[tk][part * 4 + c];
          s += q[c].x * k.x + q[c].y * k.y + q[c].z * k.z + q[c].w * k.w;
        }
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        const float mn = fmaxf(m, s);
        const float a = expf(m - mn), p = expf(s - mn);
        l = l * a + p;
        m = mn;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 v = sV[tk][part * 4 + c];
          o[c].x = o[c].x * a + p * v.x;
          o[c].y = o[c].y * a + p * v.y;
          o[c].z = o[c].z * a + p * v.z;
          o[c].w = o[c].w * a + p * v.w;
        }
      }
    }
    {
      // normalised output of this head (rows past the record: zeros) as NT bf16 terms
      const float inv = valid ? 1.0f / l : 0.f;
      float x[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[4 * c] = o[c].x * inv;
        x[4 * c + 1] = o[c].y * inv;
        x[4 * c + 2] = o[c].z * inv;
        x[4 * c + 3] = o[c].w * inv;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 tt[NT];
        split_terms<NT>(x + 8 * h, tt);
#pragma unroll
        for (int e = 0; e < NT; ++e) sO[e][qi_l][2 * part + h] = tt[e];
      }
    }
    __syncthreads();
    // 16x16x32 fragments: A lane l = row l % 16, dims 8 (l / 16) .. of a 32-dim step;
    // W_o block (16-column strip n16, K step k32) at (n16 * 32 + k32) * 512, lane l's 8 values at 8 l;
    // accumulator e of lane l = row 4 (l / 16) + e, column l % 16
    const int nrb = min(4, (nq - qb + 15) >> 4);
#pragma unroll 1
    for (int gq = 0; gq < npass; ++gq) {
      const int s0 = sw + 4 * gq;   // first 16-column strip of this pass
      // the next pass's fragments (after the last pass: the first pass's, for the next query block)
      if (npass > 1) {
        FA_LOAD_WO(bn, (gq + 1) & (npass - 1))
      }
#pragma unroll 1
      for (int rb = 0; rb < nrb; ++rb) {
        uint4 a[2][NT];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int e = 0; e < NT; ++e) a[kk][e] = sO[e][rb * 16 + (lane & 15)][4 * kk + (lane >> 4)];
        f32x4 acc[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < NT; ++e)
              acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[kk][e]), as_bf16x8(b[cb][kk]), acc[cb], 0,
                                                                0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = qb + rb * 16 + 4 * (lane >> 4) + e;
          if (row < nq) {
            float* pr = P + (size_t)j * pstride + (size_t)(q0 + row) * 1024 + (lane & 15);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) pr[(s0 + cb) * 16] = acc[cb][e];
          }
        }
      }
      if (npass > 1) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) b[cb][kk] = bn[cb][kk];
      }
    }
  }
#undef FA_LOAD_WO
}

void launch_field_attn(hipStream_t st, const float* qkv_part, int nsplit, size_t stride, const float* bqkv,
                       const int* rec, int nrec, const bf16_t* Wo, float* P, size_t pstride, int nt) {
  if (nrec == 0) return;
  // column parts: enough blocks to reach about one per compute unit
  const int cs = nrec <= 4 ? 4 : nrec <= 8 ? 2 : 1;
  if (nt == 3)
    hipLaunchKernelGGL(k_field_attn<3>, dim3(nrec, 16, cs), dim3(256), 0, st, qkv_part, nsplit, stride, bqkv, rec, Wo,
                       P, pstride);
  else
    hipLaunchKernelGGL(k_field_attn<2>, dim3(nrec, 16, cs), dim3(256), 0, st, qkv_part, nsplit, stride, bqkv, rec, Wo,
                       P, pstride);
}

}  // namespace clef
