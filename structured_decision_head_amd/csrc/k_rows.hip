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

// ---------------------------------------------------------------------------
// mu / rstd of every row of a 256-row tile (one wave per row, 4 rows per
// block; grid = (tiles, 64)).  Rows past the tile's valid count get (0, 0) so
// that padded rows of the packed row space stay finite downstream.  Hidden
// elements are bf16, or fp16 when F16 (the CoreML packaging feeds fp16 hidden
// states to the head, CoreML conversion metadata page "decision.head").
// ---------------------------------------------------------------------------
template <int NCH, bool F16>
__global__ __launch_bounds__(256) void k_rowstats(const bf16_t* __restrict__ X,
                                                       const int4* __restrict__ tiles,
                                                       float2* __restrict__ stats, float eps) {
  constexpr int H = NCH * 512;
  const int4 t = tiles[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
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
  const dim3 grid(ntiles, 64), block(256);
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
// Span pooling.  Entry e = (first hidden row, length, first stats row, output
// slot): out[slot] = gamma * mean_t((x_t - mu_t) * rstd_t) + beta, which is
// the mean of the LayerNorm-ed rows.  One block per entry.
// ---------------------------------------------------------------------------
template <int NV, bool F16>
__global__ __launch_bounds__(256) void k_pool(const bf16_t* __restrict__ X, int H,
                                              const int4* __restrict__ ent,
                                              const float2* __restrict__ stats,
                                              const float* __restrict__ gamma,
                                              const float* __restrict__ beta, float* __restrict__ out) {
  const int4 e = ent[blockIdx.x];
  const int nvec = H >> 3;
  float acc[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
  for (int t = 0; t < e.y; ++t) {
    const float2 s = stats[e.z + t];
    const uint4* row = reinterpret_cast<const uint4*>(X + (size_t)(e.x + t) * H);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = threadIdx.x + 256 * j;
      if (v < nvec) {
        float x[8];
        unpack8_hidden<F16>(row[v], x);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] += (x[i] - s.x) * s.y;
      }
    }
  }
  const float inv = 1.0f / (float)e.y;
  float* o = out + (size_t)e.w * H;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = threadIdx.x + 256 * j;
    if (v < nvec) {
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = gamma[8 * v + i] * (acc[j][i] * inv) + beta[8 * v + i];
      reinterpret_cast<float4*>(o)[2 * v] = make_float4(r[0], r[1], r[2], r[3]);
      reinterpret_cast<float4*>(o)[2 * v + 1] = make_float4(r[4], r[5], r[6], r[7]);
    }
  }
}

void launch_pool(hipStream_t st, const bf16_t* X, int H, bool f16, const int4* ent, int nent, const float2* stats,
                 const float* gamma, const float* beta, float* out) {
  if (nent == 0) return;
  const int nv = (H / 8 + 255) / 256;
  switch (nv) {
#define CASE(n)                                                                                            \
  case n:                                                                                                  \
    if (f16) hipLaunchKernelGGL((k_pool<n, true>), dim3(nent), dim3(256), 0, st, X, H, ent, stats, gamma, beta, out); \
    else hipLaunchKernelGGL((k_pool<n, false>), dim3(nent), dim3(256), 0, st, X, H, ent, stats, gamma, beta, out);    \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4)
#undef CASE
  }
}

// ---------------------------------------------------------------------------
// Lexical gather-mean and prior.  Entry k = (first id, count, question slot,
// global slot) in the pooled buffer: e_k = mean of table rows; prior_k =
// cos(e_k, pooled[q] + pooled[g]) with norms clamped at 1e-8.
// ---------------------------------------------------------------------------
template <int NV>
__global__ __launch_bounds__(256) void k_lex_prior(const bf16_t* __restrict__ E, int H,
                                                   const int4* __restrict__ ent,
                                                   const int* __restrict__ ids,
                                                   const float* __restrict__ pooled,
                                                   float* __restrict__ ebar, float* __restrict__ prior) {
  __shared__ float sm[4];
  const int4 e = ent[blockIdx.x];
  const int nvec = H >> 3;
  float acc[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
  for (int t = 0; t < e.y; ++t) {
    const uint4* row = reinterpret_cast<const uint4*>(E + (size_t)ids[e.x + t] * H);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = threadIdx.x + 256 * j;
      if (v < nvec) {
        float x[8];
        unpack8(row[v], x);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] += x[i];
      }
    }
  }
  const float inv = 1.0f / (float)e.y;
  const float* qv = pooled + (size_t)e.z * H;
  const float* gv = pooled + (size_t)e.w * H;
  float* eo = ebar + (size_t)blockIdx.x * H;
  float ea = 0.f, ee = 0.f, aa = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = threadIdx.x + 256 * j;
    if (v < nvec) {
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        r[i] = acc[j][i] * inv;
        const float a = qv[8 * v + i] + gv[8 * v + i];
        ea += r[i] * a;
        ee += r[i] * r[i];
        aa += a * a;
      }
      reinterpret_cast<float4*>(eo)[2 * v] = make_float4(r[0], r[1], r[2], r[3]);
      reinterpret_cast<float4*>(eo)[2 * v + 1] = make_float4(r[4], r[5], r[6], r[7]);
    }
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
  const int nv = (H / 8 + 255) / 256;
  switch (nv) {
#define CASE(n) case n: hipLaunchKernelGGL(k_lex_prior<n>, dim3(nent), dim3(256), 0, st, E, H, ent, ids, pooled, ebar, prior); break;
    CASE(1) CASE(2) CASE(3) CASE(4)
#undef CASE
  }
}

}  // namespace clef
