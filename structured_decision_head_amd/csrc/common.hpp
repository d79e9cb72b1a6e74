// Device helpers shared by the gfx950 kernels: bf16 conversion, wave64
// reductions, MFMA operand vector types and the XCD-aware block remap.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;                                                  // bf16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));                // MFMA operand
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));           // 16-byte register vector
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define DEV __device__ __forceinline__

// Two floats to two bf16 (round to nearest even, hardware conversion), a in the low half.
DEV uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte store with the non-temporal hint (16-byte aligned): the line is
// written through rather than kept dirty in L2 and the memory-side cache.
DEV void store_stream(void* p, const u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }
DEV void store_stream(void* p, const u32x2 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p)); }

// Unpack 8 bf16 held in a uint4 into floats.
DEV void unpack8(const uint4 v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

// Eight floats to eight bf16 (round to nearest even, hardware conversion, one
// instruction per pair).
DEV uint4 pack8(const float* f) {
  uint4 v;
  v.x = pack_bf16x2(f[0], f[1]);
  v.y = pack_bf16x2(f[2], f[3]);
  v.z = pack_bf16x2(f[4], f[5]);
  v.w = pack_bf16x2(f[6], f[7]);
  return v;
}

// Split 8 floats into NT bf16 terms whose sum approximates (NT = 2) or equals
// (NT = 3) each float: t0 = bf16(x), t1 = bf16(x - t0), t2 = bf16(x - t0 - t1).
// Every difference is exact in fp32 (x - bf16(x) needs at most 16 significant
// bits, and the next remainder at most 8).
template <int NT>
DEV void split_terms(const float* f, uint4 (&t)[NT]) {
  float r[8], h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = f[i];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    t[j] = pack8(r);
    if (j + 1 < NT) {
      unpack8(t[j], h);
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] -= h[i];
    }
  }
}

DEV bf16x8 as_bf16x8(const uint4 v) { return __builtin_bit_cast(bf16x8, v); }
DEV bf16x8 as_bf16x8(const u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// IEEE half precision: hidden states may arrive as fp16 instead of bf16.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));               // MFMA operand
DEV f16x8 as_f16x8(const u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Unpack 8 fp16 held in a uint4 into floats (exact).
DEV void unpack8_f16(const uint4 v, float* f) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 a = __builtin_bit_cast(h2, v.x), b = __builtin_bit_cast(h2, v.y);
  const h2 c = __builtin_bit_cast(h2, v.z), d = __builtin_bit_cast(h2, v.w);
  f[0] = (float)a.x; f[1] = (float)a.y; f[2] = (float)b.x; f[3] = (float)b.y;
  f[4] = (float)c.x; f[5] = (float)c.y; f[6] = (float)d.x; f[7] = (float)d.y;
}

// Unpack 4 bf16 held in two 32-bit words into floats.
DEV void unpack4(uint32_t a, uint32_t b, float* f) {
  f[0] = __uint_as_float(a << 16); f[1] = __uint_as_float(a & 0xffff0000u);
  f[2] = __uint_as_float(b << 16); f[3] = __uint_as_float(b & 0xffff0000u);
}

// Unpack 8 16-bit values of the hidden element type (fp16 if F16, else bf16).
template <bool F16>
DEV void unpack8_hidden(const uint4 v, float* f) {
  if constexpr (F16) unpack8_f16(v, f);
  else unpack8(v, f);
}

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Maximum over a whole block of NW waves; every thread gets the result.
template <int NW>
DEV float block_max(float v, float* sm) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm[w] = v;
  __syncthreads();
  float t = sm[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) t = fmaxf(t, sm[i]);
  __syncthreads();
  return t;
}

// Sum over a whole block of NW waves; every thread gets the result.  `sm`
// needs NW floats; the call ends with a barrier so `sm` can be reused.
template <int NW>
DEV float block_sum(float v, float* sm) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += sm[i];
  __syncthreads();
  return t;
}

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on
// XCD b % 8).  Return a logical tile index such that consecutive logical
// tiles land on the same XCD, so tiles that share operand rows share that
// XCD's L2.  Bijective for any grid size.
DEV int xcd_remap(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

DEV float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
