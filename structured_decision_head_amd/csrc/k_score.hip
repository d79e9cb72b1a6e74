// Field aggregation and the fused final scoring kernel.
//
// Field vector (clef-4bit page §三 step 3): base projection of the question
// vector + option-weighted summary of the routed option vectors + projection
// of the global vector + type embedding.  The summary weights are a softmax
// over the question's options of a learned score w_s . u_k + b_s.
//
// Logit (clef-4bit page §三 step 4; architecture page §3.2): prior +
// sigmoid(gate) * (joint_scale * cos(u_k, f_q) + MLP(k)); then a softmax over
// each question's options (CoreML metadata page, "softmax": fp32, T = 1) and
// the index of the first maximal logit.  Optionally the kernel also maps each
// question's softmax to its answer (metadata page "decision.response"): the
// value and confidence per question and 4-decimal copies of them and of every
// probability.
#include "kernels.hpp"

namespace clef {

namespace {
DEV float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
DEV float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

// Round half to even at the fourth decimal (the response rounds to four places).  For an
// fp32 x the product x * 10^4 is exact in double (24 + 10 significant bits), rint
// breaks ties to even, and k / 10^4 is the double nearest the decimal k * 10^-4,
// narrowed to fp32.
DEV float round_4dp(float x) {
  const double k = rint((double)x * 10000.0);
  return (float)(k / 10000.0);
}
}  // namespace

constexpr int kQW = 8;                 // waves per question block
constexpr int kQT = kQW * 64;

// Lane l of a wave owns elements 4 l + 256 c .. + 3 (c = 0..3) of a 1024-wide
// row, so each float4 load of a wave reads 1 KB of contiguous memory.
DEV int el(int lane, int c) { return lane * 4 + 256 * c; }

// One block (8 waves) per question.  The option scores w_s . u_k + b_s are
// computed one option per wave (wave-level sums, no block barrier between
// options); the softmax-weighted option sum is formed with two elements per
// thread; the new field row's LayerNorm statistics close the kernel.
__global__ __launch_bounds__(kQT) void k_field_agg(const float* __restrict__ U, const int* __restrict__ o_off,
                                                   const float* __restrict__ sw, float sb,
                                                   const float* __restrict__ qv, const float* __restrict__ gp,
                                                   const int* __restrict__ q_rec, const int* __restrict__ q_type,
                                                   const float* __restrict__ temb, float* __restrict__ F,
                                                   float2* __restrict__ fstats, float eps) {
  __shared__ float sm[kQW];
  __shared__ float sc[kMaxOptions];
  const int q = blockIdx.x;
  const int o0 = o_off[q], no = o_off[q + 1] - o0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float4 wv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) wv[c] = ld4(sw + el(lane, c));
  for (int k = w; k < no; k += kQW) {
    const float* u = U + (size_t)(o0 + k) * 1024;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) s += dot4(wv[c], ld4(u + el(lane, c)));
    s = wave_sum(s);
    if (lane == 0) sc[k] = s + sb;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int k = threadIdx.x; k < no; k += kQT) m = fmaxf(m, sc[k]);
  m = block_max<kQW>(m, sm);
  float z = 0.f;
  for (int k = threadIdx.x; k < no; k += kQT) z += expf(sc[k] - m);
  z = block_sum<kQW>(z, sm);
  const float iz = 1.0f / z;
  // two consecutive elements per thread
  const int e = threadIdx.x * 2;
  float a0 = 0.f, a1 = 0.f;
  for (int k = 0; k < no; ++k) {
    const float b = expf(sc[k] - m) * iz;
    const float2 u = *reinterpret_cast<const float2*>(U + (size_t)(o0 + k) * 1024 + e);
    a0 += b * u.x;
    a1 += b * u.y;
  }
  const float2 a = *reinterpret_cast<const float2*>(qv + (size_t)q * 1024 + e);
  const float2 g = *reinterpret_cast<const float2*>(gp + (size_t)q_rec[q] * 1024 + e);
  const float2 t = *reinterpret_cast<const float2*>(temb + (size_t)q_type[q] * 1024 + e);
  const float r0 = a.x + a0 + g.x + t.x, r1 = a.y + a1 + g.y + t.y;
  *reinterpret_cast<float2*>(F + (size_t)q * 1024 + e) = make_float2(r0, r1);
  // LayerNorm statistics of the new field row (input of the first field layer)
  const float mu = block_sum<kQW>(r0 + r1, sm) * (1.0f / 1024);
  const float va = block_sum<kQW>((r0 - mu) * (r0 - mu) + (r1 - mu) * (r1 - mu), sm) * (1.0f / 1024);
  if (threadIdx.x == 0) fstats[q] = make_float2(mu, 1.0f / sqrtf(va + eps));
}

void launch_field_agg(hipStream_t st, const float* U, const int* o_off, const float* sw, float sb, const float* qv,
                      const float* gp, const int* q_rec, const int* q_type, const float* temb, int NQ, float* F,
                      float2* fstats, float eps) {
  if (NQ == 0) return;
  hipLaunchKernelGGL(k_field_agg, dim3(NQ), dim3(kQT), 0, st, U, o_off, sw, sb, qv, gp, q_rec, q_type, temb, F,
                     fstats, eps);
}

// One block (16 waves) per question.  Each option's 1024 dims are split in
// four quarters (a lane's float4 c = quarter c), and the waves take the
// (option, quarter) pairs in turn, so that a question's few options still
// spread over all its waves.  The hidden layer GELU(W1 z + b1) is formed here
// from the split-K slices of W1 z (hpart, nsplit slices hstride floats apart,
// rows of 1024; unused when joint == 0); each wave leaves its quarter's three
// partial dot products (u.f, u.u, w2.h) in LDS and one thread per option adds
// the four quarters in order.  Softmax and first-index argmax run over the
// whole block.  jcos / mlp may be null.
constexpr int kSW = 16, kST = kSW * 64;
__global__ __launch_bounds__(kST) void k_score(const float* __restrict__ U, const float* __restrict__ F,
                                               const float* __restrict__ hpart, int nsplit, size_t hstride,
                                               const float* __restrict__ b1, const float* __restrict__ w2, float b2,
                                               const float* __restrict__ prior, float gate, float lam, int joint,
                                               const int* __restrict__ o_off, float* __restrict__ logits,
                                               float* __restrict__ probs, int* __restrict__ amax,
                                               float* __restrict__ jcos, float* __restrict__ mlp,
                                               const int* __restrict__ q_type, AnswerOut ans) {
  __shared__ float sm[kSW];
  __shared__ int si[kSW];
  __shared__ float sl[kMaxOptions];
  __shared__ float sp[kMaxOptions][4][3];   // per option and quarter: u.f, u.u, w2.h
  const int q = blockIdx.x;
  const int o0 = o_off[q], no = o_off[q + 1] - o0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (joint) {
    float ff = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 f = ld4(F + (size_t)q * 1024 + el(lane, c));
      ff += dot4(f, f);
    }
    ff = wave_sum(ff);
    for (int i = w; i < 4 * no; i += kSW) {
      const int k = i >> 2, c = i & 3;
      const size_t row = (size_t)(o0 + k) * 1024;
      const float4 f = ld4(F + (size_t)q * 1024 + el(lane, c));
      const float4 wv = ld4(w2 + el(lane, c));
      const float4 u = ld4(U + row + el(lane, c));
      float4 h = sum_slices4(hpart + row + el(lane, c), nsplit, hstride, b1 + el(lane, c));
      h.x = gelu_erf(h.x); h.y = gelu_erf(h.y); h.z = gelu_erf(h.z); h.w = gelu_erf(h.w);
      const float uf = wave_sum(dot4(u, f)), uu = wave_sum(dot4(u, u)), r = wave_sum(dot4(wv, h));
      if (lane == 0) {
        sp[k][c][0] = uf;
        sp[k][c][1] = uu;
        sp[k][c][2] = r;
      }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < no; k += kST) {
      const float uf = ((sp[k][0][0] + sp[k][1][0]) + sp[k][2][0]) + sp[k][3][0];
      const float uu = ((sp[k][0][1] + sp[k][1][1]) + sp[k][2][1]) + sp[k][3][1];
      const float r = (((sp[k][0][2] + sp[k][1][2]) + sp[k][2][2]) + sp[k][3][2]) + b2;
      const float cs = uf / (fmaxf(sqrtf(uu), 1e-8f) * fmaxf(sqrtf(ff), 1e-8f));
      sl[k] = prior[o0 + k] + gate * (lam * cs + r);
      if (jcos) jcos[o0 + k] = cs;
      if (mlp) mlp[o0 + k] = r;
    }
  } else {
    for (int k = threadIdx.x; k < no; k += kST) sl[k] = prior[o0 + k];
  }
  __syncthreads();
  // first maximal index: larger value wins, ties go to the smaller index
  float m = -INFINITY;
  int best = 0x7fffffff;
  for (int k = threadIdx.x; k < no; k += kST)
    if (sl[k] > m) { m = sl[k]; best = k; }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float mo = __shfl_xor(m, o, 64);
    const int bo = __shfl_xor(best, o, 64);
    if (mo > m || (mo == m && bo < best)) { m = mo; best = bo; }
  }
  if (lane == 0) { sm[w] = m; si[w] = best; }
  __syncthreads();
  m = sm[0];
  best = si[0];
#pragma unroll
  for (int i = 1; i < kSW; ++i)
    if (sm[i] > m || (sm[i] == m && si[i] < best)) { m = sm[i]; best = si[i]; }
  __syncthreads();
  float z = 0.f;
  for (int k = threadIdx.x; k < no; k += kST) z += expf(sl[k] - m);
  z = block_sum<kSW>(z, sm);
  if (best == 0x7fffffff) best = 0;   // no comparable value: index 0
  for (int k = threadIdx.x; k < no; k += kST) {
    const float p = expf(sl[k] - m) / z;
    logits[o0 + k] = sl[k];
    probs[o0 + k] = p;
    if (ans.probs_4dp) ans.probs_4dp[o0 + k] = round_4dp(p);
    sl[k] = p;                        // each thread rewrites only the entries it read
  }
  if (threadIdx.x == 0) amax[q] = best;
  if (!ans.value && !ans.confidence && !ans.value_4dp && !ans.confidence_4dp) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    // answer of the question (metadata page "decision.response"): noul -> p(true), option 0 by the
    // noul option order [true, false]; choice -> p of the answer; score -> mean level, levels 0..n-1
    const int t = q_type[q];
    const float conf = sl[best];
    float v = conf;
    if (t == 0) {
      v = sl[0];
    } else if (t == 2) {
      v = 0.f;
      for (int k = 1; k < no; ++k) v += (float)k * sl[k];
    }
    if (ans.value) ans.value[q] = v;
    if (ans.confidence) ans.confidence[q] = conf;
    if (ans.value_4dp) ans.value_4dp[q] = round_4dp(v);
    if (ans.confidence_4dp) ans.confidence_4dp[q] = round_4dp(conf);
  }
}

void launch_score(hipStream_t st, const float* U, const float* F, const float* hpart, int nsplit, size_t hstride,
                  const float* b1, const float* w2, float b2, const float* prior, float gate, float lam, int joint,
                  const int* o_off, int NQ, float* logits, float* probs, int* amax, float* jcos, float* mlp,
                  const int* q_type, const AnswerOut& ans) {
  if (NQ == 0) return;
  hipLaunchKernelGGL(k_score, dim3(NQ), dim3(kST), 0, st, U, F, hpart, nsplit, hstride, b1, w2, b2, prior, gate, lam,
                     joint, o_off, logits, probs, amax, jcos, mlp, q_type, ans);
}

}  // namespace clef
