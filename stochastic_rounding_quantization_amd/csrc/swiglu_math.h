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

// The exponential.  The clamp is one median instruction: it equals the two comparisons for every number,
// and an argument that is NaN comes only from a NaN pre-activation, whose two results are NaN whatever
// the exponential returns.  n converts with the hardware's float-to-int (NaN gives 0).
__device__ __forceinline__ float glue_exp32(float x) {
  const float xc = __builtin_amdgcn_fmed3f(x, kGlueXMin, kGlueXMax);
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
  int ni;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(ni) : "v"(n));
  return __builtin_ldexpf(p, ni);
}

// 1/d, correctly rounded, for d = 1 + e >= 1 (NaN only for a NaN pre-activation): the hardware
// reciprocal and one fused correction step equal the correctly rounded quotient for every float in
// [1, 2^126]; above that the quotient is subnormal or zero and glue_slow_recip says so.
__device__ __forceinline__ float glue_recip(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  const float e = fmaf(-d, y, 1.f);
  return fmaf(e, y, y);
}
__device__ __forceinline__ bool glue_slow_recip(float d) { return d > 0x1p126f; }

typedef __bf16 glue_bf16x2 __attribute__((ext_vector_type(2)));
typedef float glue_f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as packed bf16 (lo in the low half): round to nearest, ties to even, by the conversion
// instruction, which gives the same bits as rounding the fp32 bit pattern for every value but NaN; a NaN
// is made the canonical 0x7FC00000 first, so it becomes 0x7FC0.
__device__ __forceinline__ uint32_t glue_pack_bf16(float lo, float hi) {
  lo = lo != lo ? __uint_as_float(0x7FC00000u) : lo;
  hi = hi != hi ? __uint_as_float(0x7FC00000u) : hi;
  const glue_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, glue_bf16x2));
}

// (G_gate, G_up) of one element before rounding to bf16, given s = 1 / (1 + exp(-a)).
__device__ __forceinline__ void glue_tail(float dh, float a, float u, float s, float& gg, float& gu) {
  const float silu = a * s;
  const float ds = s * (1.f + a * (1.f - s));
  gu = dh * silu;
  gg = (dh * u) * ds;
}

// (G_gate, G_up) of one element, as bf16 bit patterns.
__device__ __forceinline__ void glue1(float dh, float a, float u, uint32_t& gg, uint32_t& gu) {
  const float d = 1.f + glue_exp32(-a);
  const float s = glue_slow_recip(d) ? __fdiv_rn(1.f, d) : glue_recip(d);
  float fg, fu;
  glue_tail(dh, a, u, s, fg, fu);
  gg = glue_pack_bf16(fg, 0.f) & 0xFFFFu;
  gu = glue_pack_bf16(fu, 0.f) & 0xFFFFu;
}

// 8 consecutive elements from their loaded values (dH as two float4, A_gate and A_up as eight packed bf16
// each): G_gate and G_up as packed bf16 pairs (og, ou: elements 2i, 2i+1 in word i, the memory order).
// The rare reciprocal below 2^-126 is one branch for the wave.
__device__ __forceinline__ void glue8_vals(const float4& h0, const float4& h1, const uint4& va, const uint4& vu,
                                           uint32_t (&og)[4], uint32_t (&ou)[4]) {
  const float h[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
  const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wu[4] = {vu.x, vu.y, vu.z, vu.w};
  float a[8], u[8], d[8], s[8];
  bool slow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[2 * i] = __uint_as_float(wa[i] << 16);
    a[2 * i + 1] = __uint_as_float(wa[i] & 0xFFFF0000u);
    u[2 * i] = __uint_as_float(wu[i] << 16);
    u[2 * i + 1] = __uint_as_float(wu[i] & 0xFFFF0000u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    d[i] = 1.f + glue_exp32(-a[i]);
    s[i] = glue_recip(d[i]);
    slow |= glue_slow_recip(d[i]);
  }
  if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (glue_slow_recip(d[i])) s[i] = __fdiv_rn(1.f, d[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float g0, u0, g1, u1;
    glue_tail(h[2 * i], a[2 * i], u[2 * i], s[2 * i], g0, u0);
    glue_tail(h[2 * i + 1], a[2 * i + 1], u[2 * i + 1], s[2 * i + 1], g1, u1);
    og[i] = glue_pack_bf16(g0, g1);
    ou[i] = glue_pack_bf16(u0, u1);
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
