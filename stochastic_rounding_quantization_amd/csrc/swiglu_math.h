// Element arithmetic of the SwiGLU backward glue, shared by the glue kernels and
// the quantizer that computes the glue's results on the fly.
//
// The S3R page times a whole SwiGLU FFN block ("Setup", single-block FFN
// benchmarks; Table III).  Between the down projection's backward (which gives
// dH) and the gate / up projections' backward sit the gradients of
// H = silu(A_gate) * A_up with respect to the two pre-activations:
//   G_up   = dH * silu(A_gate)
//   G_gate = dH * A_up * silu'(A_gate),  silu'(a) = s (1 + a (1 - s)),  s = 1 / (1 + exp(-a)).
// The arithmetic is fixed here (the pages leave it open): fp32, one rounding
// per operation in the order below (no contraction), an exponential built from
// a Cody-Waite reduction by ln 2 and the degree-7 Taylor polynomial, results
// rounded to bf16 (nearest, ties to even).  Every element is independent, so
// the results do not depend on the launch shape.
#pragma once

#include "s3r_internal.h"

namespace s3r {

constexpr float kGlueLog2e = 1.4426950408889634f;
constexpr float kGlueLn2Hi = 0.693145751953125f;        // 15 significant bits: n * kGlueLn2Hi is exact for |n| < 512
constexpr float kGlueLn2Lo = 1.4286068203094173e-06f;   // ln 2 - kGlueLn2Hi
constexpr float kGlueXMin = -104.f, kGlueXMax = 89.f;   // exp under- / overflows fp32 beyond these

__device__ __forceinline__ float glue_exp32(float x) {
  const float xc = x < kGlueXMin ? kGlueXMin : (x > kGlueXMax ? kGlueXMax : x);   // NaN passes through
  const float n = __builtin_rintf(xc * kGlueLog2e);
  const float r = (xc - n * kGlueLn2Hi) - n * kGlueLn2Lo;
  float p = (float)(1.0 / 5040.0);
  p = p * r + (float)(1.0 / 720.0);
  p = p * r + (float)(1.0 / 120.0);
  p = p * r + (float)(1.0 / 24.0);
  p = p * r + (float)(1.0 / 6.0);
  p = p * r + 0.5f;
  p = p * r + 1.f;
  p = p * r + 1.f;
  const int ni = n != n ? 0 : (int)n;
  return __builtin_ldexpf(p, ni);
}

__device__ __forceinline__ uint32_t glue_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if (v != v) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// (G_gate, G_up) of one element, as bf16 bit patterns.
__device__ __forceinline__ void glue1(float dh, float a, float u, uint32_t& gg, uint32_t& gu) {
  const float e = glue_exp32(-a);
  const float s = __fdiv_rn(1.f, 1.f + e);
  const float silu = a * s;
  const float ds = s * (1.f + a * (1.f - s));
  gu = glue_bf16_rne(dh * silu);
  gg = glue_bf16_rne((dh * u) * ds);
}

// 8 consecutive elements from their loaded values (dH as two float4, A_gate and A_up as eight packed bf16
// each): G_gate and G_up as packed bf16 pairs (og, ou: elements 2i, 2i+1 in word i, the memory order).
__device__ __forceinline__ void glue8_vals(const float4& h0, const float4& h1, const uint4& va, const uint4& vu,
                                           uint32_t (&og)[4], uint32_t (&ou)[4]) {
  const float h[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
  const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wu[4] = {vu.x, vu.y, vu.z, vu.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t g0, u0, g1, u1;
    glue1(h[2 * i], __uint_as_float(wa[i] << 16), __uint_as_float(wu[i] << 16), g0, u0);
    glue1(h[2 * i + 1], __uint_as_float(wa[i] & 0xFFFF0000u), __uint_as_float(wu[i] & 0xFFFF0000u), g1, u1);
    og[i] = g0 | (g1 << 16);
    ou[i] = u0 | (u1 << 16);
  }
}

// The same from memory: dh, ag, au point at 8 elements, 16-byte aligned.
__device__ __forceinline__ void glue8(const float* __restrict__ dh, const uint16_t* __restrict__ ag,
                                      const uint16_t* __restrict__ au, uint32_t (&og)[4], uint32_t (&ou)[4]) {
  const float4 h0 = ld_stream_f4(dh);
  const float4 h1 = ld_stream_f4(dh + 4);
  const uint4 va = ld_stream_u4(ag);
  const uint4 vu = ld_stream_u4(au);
  __builtin_amdgcn_sched_barrier(0);   // all four loads in flight before any is waited for
  glue8_vals(h0, h1, va, vu, og, ou);
}

}  // namespace s3r
