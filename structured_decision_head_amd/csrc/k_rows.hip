// Row-streaming kernels of the head: LayerNorm row statistics over the hidden
// width, span mean-pooling of LayerNorm-ed rows, lexical gather-mean with the
// cosine prior, and row statistics of fp32 width-1024 activations.
//
// Operation (CoreML conversion metadata of clef-flash, "decision.head"; clef-4bit
// page §三 steps 1 and 4): x_hat = LayerNorm(hidden row); question / option
// context vectors are means of x_hat over half-open spans; the global vector is
// x_hat at the record's last position; the option lexical vector is the mean of
// lm_head rows over the option's token ids; the prior is the cosine of the
// lexical vector with (question vector + global vector).
#include "kernels.hpp"

namespace clef {

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}

void launch_fill_u32(hipStream_t st, void* p, size_t bytes, uint32_t v) {
  const size_t n = bytes / 4;
  if (n == 0) return;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<uint32_t*>(p), n, v);
}

// ---------------------------------------------------------------------------
// mu / rstd of every row of a 256-row tile (one wave per row, 4 rows per
// block; grid = (64, tiles), so consecutive workgroups read consecutive rows).  Rows past the tile's valid count get (0, 0) so
// that padded rows of the packed row space stay finite downstream.  Hidden
// elements are bf16, or fp16 when F16 (the CoreML packaging feeds fp16 hidden
// states to the head, CoreML conversion metadata page "decision.head").
// ---------------------------------------------------------------------------
template <int NCH, bool F16>
__global__ __launch_bounds__(256) void k_rowstats(const bf16_t* __restrict__ X,
                                                       const int4* __restrict__ tiles,
                                                       float2* __restrict__ stats, float eps) {
  constexpr int H = NCH * 512;
  const int4 t = tiles[blockIdx.y];
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= t.z) {
    if (lane == 0) stats[t.y + r] = make_float2(0.f, 0.f);
    return;
  }
  const uint4* row = reinterpret_cast<const uint4*>(X + (size_t)(t.x + r) * H);
  uint4 q[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) q[c] = row[c * 64 + lane];
  float v[NCH * 8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) unpack8_hidden<F16>(q[c], v + 8 * c);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NCH * 8; ++i) s += v[i];
  const float mu = wave_sum(s) * (1.0f / H);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NCH * 8; ++i) {
    const float d = v[i] - mu;
    ss += d * d;
  }
  const float var = wave_sum(ss) * (1.0f / H);
  if (lane == 0) stats[t.y + r] = make_float2(mu, 1.0f / sqrtf(var + eps));
}

void launch_rowstats(hipStream_t st, const bf16_t* X, int H, bool f16, const int4* tiles, int ntiles,
                     float2* stats, float eps) {
  const dim3 grid(64, ntiles), block(256);
  switch (H / 512) {
#define CASE(n)                                                                              \
  case n:                                                                                    \
    if (f16) hipLaunchKernelGGL((k_rowstats<n, true>), grid, block, 0, st, X, tiles, stats, eps); \
    else hipLaunchKernelGGL((k_rowstats<n, false>), grid, block, 0, st, X, tiles, stats, eps);    \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
  }
}

// ---------------------------------------------------------------------------
// fp32 head: the LayerNorm-ed rows x_hat = (x - mu) rstd gamma + beta of every
// valid row of a 256-row tile (one wave per row, grid as k_rowstats), each fp32
// element written as its three bf16 terms (t0 + t1 + t2 = x_hat exactly) into
// planes[row][p * H + k], p = 0, 1, 2: the A operand of the memory product run
// as a bf16 GEMM of depth 3 H against the weight repeated three times.  The
// arithmetic is the fp32 row loader's (LdHid).  Rows past the valid count are
// written as zeros (the GEMM multiplies whole tiles, and those rows must stay
// finite).
// ---------------------------------------------------------------------------
template <int NCH, bool F16>
__global__ __launch_bounds__(256) void k_ln_split3(const bf16_t* __restrict__ X, const int4* __restrict__ tiles,
                                                   const float2* __restrict__ stats, const float* __restrict__ gamma,
                                                   const float* __restrict__ beta, bf16_t* __restrict__ planes) {
  constexpr int H = NCH * 512;
  const int4 t = tiles[blockIdx.y];
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  bf16_t* out = planes + (size_t)(t.y + r) * 3 * H;
  if (r >= t.z) {
    for (int i = lane; i < 3 * H / 8; i += 64) reinterpret_cast<uint4*>(out)[i] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const float2 st = stats[t.y + r];
  const uint4* row = reinterpret_cast<const uint4*>(X + (size_t)(t.x + r) * H);
#pragma unroll 2
  for (int c = 0; c < NCH; ++c) {
    const int k = (c * 64 + lane) * 8;
    float v[8], x[8];
    unpack8_hidden<F16>(row[c * 64 + lane], v);
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + k), g1 = *reinterpret_cast<const float4*>(gamma + k + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(beta + k), b1 = *reinterpret_cast<const float4*>(beta + k + 4);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (v[i] - st.x) * st.y * gg[i] + bb[i];
    uint4 tt[3];
    split_terms<3>(x, tt);
#pragma unroll
    for (int p = 0; p < 3; ++p) *reinterpret_cast<uint4*>(out + (size_t)p * H + k) = tt[p];
  }
}

void launch_ln_split3(hipStream_t st, const bf16_t* X, int H, bool f16, const int4* tiles, int ntiles,
                      const float2* stats, const float* gamma, const float* beta, bf16_t* planes) {
  if (ntiles == 0) return;
  const dim3 grid(64, ntiles), block(256);
  switch (H / 512) {
#define CASE(n)                                                                                                  \
  case n:                                                                                                        \
    if (f16) hipLaunchKernelGGL((k_ln_split3<n, true>), grid, block, 0, st, X, tiles, stats, gamma, beta, planes); \
    else hipLaunchKernelGGL((k_ln_split3<n, false>), grid, block, 0, st, X, tiles, stats, gamma, beta, planes);    \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
  }
}

// ---------------------------------------------------------------------------
// Span gathers (pooling and the lexical mean).  One block of 4 waves per
// entry; wave w takes the entry's rows w, w + 4, w + 8, ..., R at a time with
// all R rows' loads in flight (R = 4, or 2 for rows wider than 4096 elements,
// whose loads would not fit the registers), and every lane covers the whole row width in
// 512-element chunks (lane l holds elements 8 l .. 8 l + 7 of each chunk, so a
// wave's load of a chunk reads 1 KB of contiguous memory).  The four waves'
// sums are then added in wave order through LDS, one chunk at a time, so the
// result does not depend on timing.
// ---------------------------------------------------------------------------
namespace {

// Sum over waves in fixed order: every thread gets the block total of chunk c
// for its two elements 2 t, 2 t + 1 (t = threadIdx.x) of the 512.  red holds
// 4 x 512 floats; the call ends with a barrier.
DEV float2 wave_order_sum(const float (&acc)[8], float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float4* dst = reinterpret_cast<float4*>(red + w * 512 + lane * 8);
  dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  const int e = threadIdx.x * 2;
  float2 r = *reinterpret_cast<const float2*>(red + e);
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    const float2 v = *reinterpret_cast<const float2*>(red + i * 512 + e);
    r.x += v.x;
    r.y += v.y;
  }
  __syncthreads();
  return r;
}

}  // namespace

// Span pooling.  Entry e = (first hidden row, length, first stats row, output
// slot): out[slot] = gamma * mean_t((x_t - mu_t) * rstd_t) + beta, the mean of
// the LayerNorm-ed rows.
template <int NCH, bool F16>
__global__ __launch_bounds__(256) void k_pool(const bf16_t* __restrict__ X, const int4* __restrict__ ent,
                                              const float2* __restrict__ stats, const float* __restrict__ gamma,
                                              const float* __restrict__ beta, float* __restrict__ out) {
  constexpr int H = NCH * 512;
  __shared__ __attribute__((aligned(16))) float red[4 * 512];
  const int4 e = ent[blockIdx.x];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float acc[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
  constexpr int R = NCH <= 8 ? 4 : 2;
  for (int t = w; t < e.y; t += 4 * R) {
    uint4 q[R][NCH];
    float2 sr[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (t + 4 * j < e.y) {
        const uint4* row = reinterpret_cast<const uint4*>(X + (size_t)(e.x + t + 4 * j) * H) + lane;
#pragma unroll
        for (int c = 0; c < NCH; ++c) q[j][c] = row[c * 64];
        sr[j] = stats[e.z + t + 4 * j];
      }
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (t + 4 * j < e.y) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          float x[8];
          unpack8_hidden<F16>(q[j][c], x);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[c][i] += (x[i] - sr[j].x) * sr[j].y;
        }
      }
  }
  const float inv = 1.0f / (float)e.y;
  float* o = out + (size_t)e.w * H;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const float2 v = wave_order_sum(acc[c], red);
    const int k = c * 512 + threadIdx.x * 2;
    const float2 g = *reinterpret_cast<const float2*>(gamma + k), b = *reinterpret_cast<const float2*>(beta + k);
    *reinterpret_cast<float2*>(o + k) = make_float2(g.x * (v.x * inv) + b.x, g.y * (v.y * inv) + b.y);
  }
}

void launch_pool(hipStream_t st, const bf16_t* X, int H, bool f16, const int4* ent, int nent, const float2* stats,
                 const float* gamma, const float* beta, float* out) {
  if (nent == 0) return;
  switch (H / 512) {
#define CASE(n)                                                                                              \
  case n:                                                                                                    \
    if (f16) hipLaunchKernelGGL((k_pool<n, true>), dim3(nent), dim3(256), 0, st, X, ent, stats, gamma, beta, out); \
    else hipLaunchKernelGGL((k_pool<n, false>), dim3(nent), dim3(256), 0, st, X, ent, stats, gamma, beta, out);    \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
  }
}

// Lexical gather-mean and prior.  Entry k = (first id, count, question slot,
// global slot) in the pooled buffer: e_k = mean of table rows; prior_k =
// cos(e_k, pooled[q] + pooled[g]) with norms clamped at 1e-8.
template <int NCH>
__global__ __launch_bounds__(256) void k_lex_prior(const bf16_t* __restrict__ E, const int4* __restrict__ ent,
                                                   const int* __restrict__ ids, const float* __restrict__ pooled,
                                                   float* __restrict__ ebar, float* __restrict__ prior) {
  constexpr int H = NCH * 512;
  __shared__ __attribute__((aligned(16))) float red[4 * 512];
  __shared__ float sm[4];
  const int4 e = ent[blockIdx.x];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float acc[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
  constexpr int R = NCH <= 8 ? 4 : 2;
  for (int t = w; t < e.y; t += 4 * R) {
    uint4 q[R][NCH];
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (t + 4 * j < e.y) {
        const uint4* row = reinterpret_cast<const uint4*>(E + (size_t)ids[e.x + t + 4 * j] * H) + lane;
#pragma unroll
        for (int c = 0; c < NCH; ++c) q[j][c] = row[c * 64];
      }
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (t + 4 * j < e.y) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          float x[8];
          unpack8(q[j][c], x);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[c][i] += x[i];
        }
      }
  }
  const float inv = 1.0f / (float)e.y;
  const float* qv = pooled + (size_t)e.z * H;
  const float* gv = pooled + (size_t)e.w * H;
  float* eo = ebar + (size_t)blockIdx.x * H;
  float ea = 0.f, ee = 0.f, aa = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const float2 v = wave_order_sum(acc[c], red);
    const int k = c * 512 + threadIdx.x * 2;
    const float2 r = make_float2(v.x * inv, v.y * inv);
    const float2 q = *reinterpret_cast<const float2*>(qv + k), g = *reinterpret_cast<const float2*>(gv + k);
    const float a0 = q.x + g.x, a1 = q.y + g.y;
    ea += r.x * a0 + r.y * a1;
    ee += r.x * r.x + r.y * r.y;
    aa += a0 * a0 + a1 * a1;
    *reinterpret_cast<float2*>(eo + k) = r;
  }
  ea = block_sum<4>(ea, sm);
  ee = block_sum<4>(ee, sm);
  aa = block_sum<4>(aa, sm);
  if (threadIdx.x == 0)
    prior[blockIdx.x] = ea / (fmaxf(sqrtf(ee), 1e-8f) * fmaxf(sqrtf(aa), 1e-8f));
}

void launch_lex_prior(hipStream_t st, const bf16_t* E, int H, const int4* ent, int nent, const int* ids,
                      const float* pooled, float* ebar, float* prior) {
  if (nent == 0) return;
  switch (H / 512) {
#define CASE(n) case n: hipLaunchKernelGGL(k_lex_prior<n>, dim3(nent), dim3(256), 0, st, E, ent, ids, pooled, ebar, prior); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
  }
}

}  // namespace clef
