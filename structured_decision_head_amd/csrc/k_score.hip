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
// the index of the first maximal logit.
#include "kernels.hpp"

namespace clef {

namespace {
DEV float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
DEV float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }
}  // namespace

// One block (256 threads, 4 elements each) per question.
__global__ __launch_bounds__(256) void k_field_agg(const float* __restrict__ U, const int* __restrict__ o_off,
                                                   const float* __restrict__ sw, float sb,
                                                   const float* __restrict__ qv, const float* __restrict__ gp,
                                                   const int* __restrict__ q_rec, const int* __restrict__ q_type,
                                                   const float* __restrict__ temb, float* __restrict__ F,
                                                   float2* __restrict__ fstats, float eps) {
  __shared__ float sm[4];
  __shared__ float sc[kMaxOptions];
  const int q = blockIdx.x;
  const int o0 = o_off[q], o1 = o_off[q + 1];
  const int e = threadIdx.x * 4;
  const float4 w = ld4(sw + e);
  for (int k = o0; k < o1; ++k) {
    const float s = block_sum<4>(dot4(w, ld4(U + (size_t)k * 1024 + e)), sm);
    if (threadIdx.x == 0) sc[k - o0] = s + sb;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int k = 0; k < o1 - o0; ++k) mx = fmaxf(mx, sc[k]);
  float z = 0.f;
  for (int k = 0; k < o1 - o0; ++k) z += expf(sc[k] - mx);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = o0; k < o1; ++k) {
    const float b = expf(sc[k - o0] - mx) / z;
    const float4 u = ld4(U + (size_t)k * 1024 + e);
    acc.x += b * u.x; acc.y += b * u.y; acc.z += b * u.z; acc.w += b * u.w;
  }
  const float4 a = ld4(qv + (size_t)q * 1024 + e);
  const float4 g = ld4(gp + (size_t)q_rec[q] * 1024 + e);
  const float4 t = ld4(temb + (size_t)q_type[q] * 1024 + e);
  float4 r;
  r.x = a.x + acc.x + g.x + t.x;
  r.y = a.y + acc.y + g.y + t.y;
  r.z = a.z + acc.z + g.z + t.z;
  r.w = a.w + acc.w + g.w + t.w;
  *reinterpret_cast<float4*>(F + (size_t)q * 1024 + e) = r;
  // LayerNorm statistics of the new field row (input of the first field layer)
  const float mu = block_sum<4>((r.x + r.y) + (r.z + r.w), sm) * (1.0f / 1024);
  const float va = block_sum<4>((r.x - mu) * (r.x - mu) + (r.y - mu) * (r.y - mu) + (r.z - mu) * (r.z - mu) +
                                    (r.w - mu) * (r.w - mu), sm) * (1.0f / 1024);
  if (threadIdx.x == 0) fstats[q] = make_float2(mu, 1.0f / sqrtf(va + eps));
}

void launch_field_agg(hipStream_t st, const float* U, const int* o_off, const float* sw, float sb, const float* qv,
                      const float* gp, const int* q_rec, const int* q_type, const float* temb, int NQ, float* F,
                      float2* fstats, float eps) {
  if (NQ == 0) return;
  hipLaunchKernelGGL(k_field_agg, dim3(NQ), dim3(256), 0, st, U, o_off, sw, sb, qv, gp, q_rec, q_type, temb, F,
                     fstats, eps);
}

// One block per question.  The hidden layer GELU(W1 z + b1) of option k is
// formed here from the split-K slices of W1 z (hpart, nsplit slices
// hstride floats apart, rows of 1024; unused when joint == 0).  jcos / mlp may
// be null.
__global__ __launch_bounds__(256) void k_score(const float* __restrict__ U, const float* __restrict__ F,
                                               const float* __restrict__ hpart, int nsplit, size_t hstride,
                                               const float* __restrict__ b1, const float* __restrict__ w2, float b2,
                                               const float* __restrict__ prior, float gate, float lam, int joint,
                                               const int* __restrict__ o_off, float* __restrict__ logits,
                                               float* __restrict__ probs, int* __restrict__ amax,
                                               float* __restrict__ jcos, float* __restrict__ mlp) {
  __shared__ float sm[4];
  __shared__ float sl[kMaxOptions];
  const int q = blockIdx.x;
  const int o0 = o_off[q], o1 = o_off[q + 1];
  const int e = threadIdx.x * 4;
  if (joint) {
    const float4 f = ld4(F + (size_t)q * 1024 + e);
    const float4 w = ld4(w2 + e);
    const float ff = block_sum<4>(dot4(f, f), sm);
    for (int k = o0; k < o1; ++k) {
      const float4 u = ld4(U + (size_t)k * 1024 + e);
      float4 h = sum_slices4(hpart + (size_t)k * 1024 + e, nsplit, hstride, b1 + e);
      h.x = gelu_erf(h.x); h.y = gelu_erf(h.y); h.z = gelu_erf(h.z); h.w = gelu_erf(h.w);
      const float uf = block_sum<4>(dot4(u, f), sm);
      const float uu = block_sum<4>(dot4(u, u), sm);
      const float r = block_sum<4>(dot4(w, h), sm) + b2;
      if (threadIdx.x == 0) {
        const float c = uf / (fmaxf(sqrtf(uu), 1e-8f) * fmaxf(sqrtf(ff), 1e-8f));
        sl[k - o0] = prior[k] + gate * (lam * c + r);
        if (jcos) jcos[k] = c;
        if (mlp) mlp[k] = r;
      }
    }
  } else if (threadIdx.x == 0) {
    for (int k = o0; k < o1; ++k) sl[k - o0] = prior[k];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mx = sl[0];
    int best = 0;
    for (int k = 1; k < o1 - o0; ++k)
      if (sl[k] > mx) { mx = sl[k]; best = k; }
    float z = 0.f;
    for (int k = 0; k < o1 - o0; ++k) z += expf(sl[k] - mx);
    for (int k = 0; k < o1 - o0; ++k) {
      logits[o0 + k] = sl[k];
      probs[o0 + k] = expf(sl[k] - mx) / z;
    }
    amax[q] = best;
  }
}

void launch_score(hipStream_t st, const float* U, const float* F, const float* hpart, int nsplit, size_t hstride,
                  const float* b1, const float* w2, float b2, const float* prior, float gate, float lam, int joint,
                  const int* o_off, int NQ, float* logits, float* probs, int* amax, float* jcos, float* mlp) {
  if (NQ == 0) return;
  hipLaunchKernelGGL(k_score, dim3(NQ), dim3(256), 0, st, U, F, hpart, nsplit, hstride, b1, w2, b2, prior, gate, lam,
                     joint, o_off, logits, probs, amax, jcos, mlp);
}

}  // namespace clef
