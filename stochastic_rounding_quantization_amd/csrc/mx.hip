// MXFP4 variant of the quantized backward for gfx950: G rounded (RTNE, SR or
// S3R) to E2M1 with one E8M0 scale per 32 elements along each GEMM's
// contraction, and the block-scaled FP4 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The S3R page names MXFP4 as the 4-bit setting where deterministic rounding
// fails the backward pass (Introduction; Related Work) but fixes none of its
// arithmetic; the readings here:
//   scale   2^k, k the smallest integer with max|block| <= 6 * 2^k (nothing
//           saturates), clamped to [-127, 127]; all-zero block: k = -127;
//           a non-finite max: the NaN scale (byte 255), zero codes, a flag;
//   round   y = g / 2^k (exact); spacing s = 0.5 below |y| 2, 1 below 4, 2 up
//           to 6; RTNE s * rint(y / s); SR / S3R the exact floor
//           s * floor(y / s + r) with the INT8 path's thresholds;
//   layout  two E2M1 codes per byte, the first in the low nibble; scales one
//           byte per block, grouped by K step of 128 (4 blocks): for a
//           matrix of R rows the scales of step j are R 4-byte words (row r's
//           blocks 4j .. 4j+3), so byte (r, b) sits at (b / 4) ld + 4 r + b % 4.
//           A GEMM step then reads its rows' scale words contiguously.
// Every GEMM operand is K-major (the contraction contiguous): G is quantized
// twice, Q_h [T x D] blocked along D for dX and Q_t [D x T] (G transposed,
// blocked along T) for dW, with the same thresholds; the forward operands W
// [D x d_in] and X [T x d_in] are stored transposed, blocked along D and T.
// The correction (S3R-EC) is taken per quantization on E = dequant(Q) - G.
#include "s3r_internal.h"

namespace s3r {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit dword format

// ------------------------------------------------------ E2M1 rounding ----
// Block exponent of amax bits (ordered fp32 bits): the smallest k with
// a <= 6 * 2^k, clamped; returns 255 (NaN) for a non-finite max.
__device__ __forceinline__ int block_scale_byte(uint32_t abits) {
  if (!(abits < 0x7F800000u)) return 255;
  if (abits == 0) return 0;                                       // k = -127
  int E;
  const float m = __builtin_frexpf(__uint_as_float(abits), &E);  // a = m 2^E, m in [0.5, 1)
  int k = m <= 0.75f ? E - 3 : E - 2;
  k = k < -127 ? -127 : (k > 127 ? 127 : k);
  return k + 127;
}

// 2^-k as fp32 for a scale byte (k = byte - 127), exact for every k in [-127, 127].
__device__ __forceinline__ float inv_scale(int byte) { return __builtin_ldexpf(1.f, 127 - byte); }

// E2M1 code (sign << 3 | index) of y, |y| <= 6: RTNE (R < 0) or floor(y / s + r) with
// R = r * 2^24.  The floor is exact: t = y / s * 2^24 is an exact power-of-two scaling
// (|t| < 2^28), X = floor(t) by one conversion, and floor(y / s + r) = (X + R) >> 24.
__device__ __forceinline__ uint32_t e2m1_code(float y, int32_t R, float& qv) {
  const float a = fabsf(y);
  const float s = a < 2.f ? 0.5f : (a < 4.f ? 1.f : 2.f);
  const float ys = y * (a < 2.f ? 2.f : (a < 4.f ? 1.f : 0.5f));  // y / s, exact: s is a power of two
  int32_t n;                                                      // the multiple of s
  if (R < 0) {
    n = (int32_t)__builtin_rintf(ys);
  } else {
    const float t = ys * 16777216.f;
    int32_t X;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(X) : "v"(t));
    n = (X + R) >> 24;
  }
  qv = (float)n * s;                                              // a grid value in [-6, 6]
  const float m = fabsf(qv);
  // index into 0, 0.5, 1, 1.5, 2, 3, 4, 6
  const uint32_t idx = m < 2.f ? (uint32_t)(m * 2.f) : (m < 4.f ? (uint32_t)m + 2u : (m < 5.f ? 6u : 7u));
  return (qv < 0.f ? 8u : 0u) | idx;
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t i = c & 7u;
  const float m = i < 4u ? 0.5f * (float)i : (i == 4u ? 2.f : (i == 5u ? 3.f : (i == 6u ? 4.f : 6.f)));
  return (c & 8u) ? -m : m;
}

template <typename TIn>
__device__ __forceinline__ float load_elem(const TIn* p) {
  if constexpr (sizeof(TIn) == 2) return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
  else return *reinterpret_cast<const float*>(p);
}

struct MxQuant {
  int64_t R, C, S;          // rows, columns of the source, rows per example
  int64_t ld;               // source leading dim (elements)
  int mode;                 // 0 RTNE, 1 SR, 2 S3R
  uint32_t layer; uint64_t seed; uint32_t stream_word;
  int64_t D_index;          // SR element index e = t * D_index + j (G's row-major index)
};

// ------------------------------------------ blocks along the columns ----
// Source M [R x C] row-major, blocks of 32 along C.  A block of 256 threads
// covers 64 rows x 512 columns; a lane handles 8 consecutive elements, four
// lanes a block.  Out: codes [R x C/2] (row-major, ld_out bytes), scales in
// the step-grouped layout [C/128][R][4] (ld_s bytes per step).  With EC: the error row sums of each row over the
// tile's 512 columns (row_part[t * n_ct + ctile]) and the error column sums of
// the tile's 64 rows (col_part[rtile * C + j]).
template <typename TIn, bool EC>
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(MxQuant p, const TIn* __restrict__ M,
                                                            uint8_t* __restrict__ out, int64_t ld_out,
                                                            uint8_t* __restrict__ sc, int64_t ld_s,
                                                            float* __restrict__ row_part, float* __restrict__ col_part,
                                                            uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int64_t j0 = (int64_t)blockIdx.y * 512 + lane * 8;
  const int n_ct = (int)((p.C + 511) / 512);
  __shared__ float s_col[4][512];
  float col[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) col[i] = 0.f;
  const bool active = j0 < p.C;                     // C % 32 == 0: a lane is all in or all out
  float rs[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t t = r0 + wave + 4 * k;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = active ? load_elem<TIn>(M + t * p.ld + j0 + i) : 0.f;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
    const int sb = block_scale_byte(m);
    const bool bad = sb == 255;
    const float inv = bad ? 0.f : inv_scale(sb);
    int32_t Rt[8];
    if (p.mode == 2) {
      const int32_t r = s3r_threshold_units24(t, p.layer, p.seed, kTagS3R + p.stream_word);
#pragma unroll
      for (int i = 0; i < 8; ++i) Rt[i] = r;
    } else if (p.mode == 1) {
#pragma unroll
      for (int i = 0; i < 8; i += 4) {
        const uint64_t e = (uint64_t)t * (uint64_t)p.D_index + (uint64_t)(j0 + i);   // e % 4 == 0
        const U4 w = philox4x32_10((uint32_t)(e >> 2), (uint32_t)(e >> 34), p.layer, kTagSR + p.stream_word,
                                   (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
        Rt[i] = sr_units24(w.x); Rt[i + 1] = sr_units24(w.y); Rt[i + 2] = sr_units24(w.z); Rt[i + 3] = sr_units24(w.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) Rt[i] = -1;
    }
    uint32_t packed = 0;
    float es = 0.f;
    const float scale = bad ? 0.f : __builtin_ldexpf(1.f, sb - 127);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float qv;
      const uint32_t c = bad ? 0u : e2m1_code(v[i] * inv, Rt[i], qv);
      packed |= c << (4 * i);
      if constexpr (EC) {
        const float e = bad ? 0.f : qv * scale - v[i];
        es += e;
        col[i] += e;
      }
    }
    if (active) {
      *reinterpret_cast<uint32_t*>(out + t * ld_out + j0 / 2) = packed;
      if ((lane & 3) == 0) sc[(j0 / 128) * ld_s + t * 4 + ((j0 / 32) & 3)] = (uint8_t)sb;
      if (bad && flags && (lane & 3) == 0) atomicOr(flags, S3R_FLAG_NONFINITE);
    }
    rs[k] = es;
  }
  if constexpr (EC) {
    // reduce-scatter of the 16 row sums across the wave: lane l then holds row k = l >> 2
    float r8[8], r4[4], r2[2], r1;
    const bool hi32 = lane & 32, hi16 = lane & 16, hi8 = lane & 8, hi4 = lane & 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float send = hi32 ? rs[i] : rs[i + 8];
      r8[i] = (hi32 ? rs[i + 8] : rs[i]) + __shfl_xor(send, 32, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float send = hi16 ? r8[i] : r8[i + 4];
      r4[i] = (hi16 ? r8[i + 4] : r8[i]) + __shfl_xor(send, 16, 64);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float send = hi8 ? r4[i] : r4[i + 2];
      r2[i] = (hi8 ? r4[i + 2] : r4[i]) + __shfl_xor(send, 8, 64);
    }
    {
      const float send = hi4 ? r2[0] : r2[1];
      r1 = (hi4 ? r2[1] : r2[0]) + __shfl_xor(send, 4, 64);
    }
    r1 += __shfl_xor(r1, 2, 64);
    r1 += __shfl_xor(r1, 1, 64);
    if ((lane & 3) == 0) row_part[(r0 + wave + 4 * (lane >> 2)) * n_ct + blockIdx.y] = r1;
#pragma unroll
    for (int i = 0; i < 8; ++i) s_col[wave][lane * 8 + i] = col[i];
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += 256) {
      const int64_t j = (int64_t)blockIdx.y * 512 + c;
      if (j < p.C) col_part[(int64_t)blockIdx.x * p.C + j] = ((s_col[0][c] + s_col[1][c]) + s_col[2][c]) + s_col[3][c];
    }
  }
}

// ------------------------------------------------ blocks along the rows ----
// Source M [R x C] row-major, blocks of 32 along R, output transposed:
// codes [C x R/2] (row c holds column c of M), scales [R/128][C][4].  A block of
// 256 threads covers 128 rows x 64 columns: lane = column, wave = one 32-row
// block.  Per thread: the amax of its 32 values, the scale, 32 codes = 16
// bytes written contiguously (the four waves write 64 contiguous bytes of an
// output row).  VSUM: the column sums of the dequantized values of the block
// (vsum_part[rblk * C + c]).  EC: the error column sums (col_part[rblk * C + c])
// and the error row sums over the tile's 64 columns (row_part[t * n_ct + ctile]).
template <typename TIn, bool EC, bool VSUM>
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(MxQuant p, const TIn* __restrict__ M,
                                                            uint8_t* __restrict__ out, int64_t ld_out,
                                                            uint8_t* __restrict__ sc, int64_t ld_s,
                                                            float* __restrict__ row_part, float* __restrict__ col_part,
                                                            float* __restrict__ vsum_part, uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.y * 64 + lane;
  const int64_t t0 = (int64_t)blockIdx.x * 128 + wave * 32;        // this wave's block of 32 rows
  const bool active = c < p.C;
  const int n_ct = (int)((p.C + 63) / 64);
  __shared__ int32_t s_thr[128];
  if (p.mode == 2 && threadIdx.x < 128)
    s_thr[threadIdx.x] = s3r_threshold_units24((int64_t)blockIdx.x * 128 + threadIdx.x, p.layer, p.seed,
                                               kTagS3R + p.stream_word);
  __syncthreads();
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = active ? load_elem<TIn>(M + (t0 + i) * p.ld + c) : 0.f;
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  const int sb = block_scale_byte(m);
  const bool bad = sb == 255;
  const float inv = bad ? 0.f : inv_scale(sb);
  const float scale = bad ? 0.f : __builtin_ldexpf(1.f, sb - 127);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  float es[32];
  float csum = 0.f, vsum = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t t = t0 + i;
    int32_t R = -1;
    if (p.mode == 2) {
      R = s_thr[wave * 32 + i];
    } else if (p.mode == 1) {
      const uint64_t e = (uint64_t)t * (uint64_t)p.D_index + (uint64_t)c;
      const U4 u = philox4x32_10((uint32_t)(e >> 2), (uint32_t)(e >> 34), p.layer, kTagSR + p.stream_word,
                                 (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
      R = sr_units24(u4_word(u, (uint32_t)e & 3u));
    }
    float qv;
    const uint32_t code = bad ? 0u : e2m1_code(v[i] * inv, R, qv);
    w[i >> 3] |= code << (4 * (i & 7));
    const float dq = bad ? 0.f : qv * scale;
    const float e = bad ? 0.f : dq - v[i];
    es[i] = active ? e : 0.f;
    csum += e;
    vsum += dq;
  }
  if (active) {
    *reinterpret_cast<uint4*>(out + c * ld_out + t0 / 2) = make_uint4(w[0], w[1], w[2], w[3]);
    sc[(t0 / 128) * ld_s + c * 4 + ((t0 / 32) & 3)] = (uint8_t)sb;
    if (bad && flags) atomicOr(flags, S3R_FLAG_NONFINITE);
    const int64_t rblk = t0 / 32;
    if constexpr (EC) col_part[rblk * p.C + c] = csum;
    if constexpr (VSUM) vsum_part[rblk * p.C + c] = vsum;
  }
  if constexpr (EC) {
    // row sums of the 32 rows over the wave's 64 columns: reduce-scatter, lane l then holds row l >> 1
    float h16[16], h8[8], h4[4], h2[2], h1;
    const bool b32 = lane & 32, b16 = lane & 16, b8 = lane & 8, b4 = lane & 4, b2 = lane & 2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float send = b32 ? es[i] : es[i + 16];
      h16[i] = (b32 ? es[i + 16] : es[i]) + __shfl_xor(send, 32, 64);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float send = b16 ? h16[i] : h16[i + 8];
      h8[i] = (b16 ? h16[i + 8] : h16[i]) + __shfl_xor(send, 16, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float send = b8 ? h8[i] : h8[i + 4];
      h4[i] = (b8 ? h8[i + 4] : h8[i]) + __shfl_xor(send, 8, 64);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float send = b4 ? h4[i] : h4[i + 2];
      h2[i] = (b4 ? h4[i + 2] : h4[i]) + __shfl_xor(send, 4, 64);
    }
    {
      const float send = b2 ? h2[0] : h2[1];
      h1 = (b2 ? h2[1] : h2[0]) + __shfl_xor(send, 2, 64);
    }
    h1 += __shfl_xor(h1, 1, 64);
    if ((lane & 1) == 0) row_part[(t0 + (lane >> 1)) * n_ct + blockIdx.y] = h1;
  }
}

// Statistics from the partials, fixed order, fp64 sums.  Blocks [0, ncb): one
// item per (example b, column j): the error column mean over the example's
// row blocks (ec_col) and / or the sum of the dequantized values (vsum_out).
// Blocks past ncb: the token means eps_t from the row partials.
__global__ __launch_bounds__(256) void mx_finalize_kernel(int64_t B, int64_t C, int64_t S, int rows_per_part,
                                                          int n_ct, int ncb, const float* __restrict__ col_part,
                                                          const float* __restrict__ vsum_part,
                                                          const float* __restrict__ row_part, float* __restrict__ ec_col,
                                                          float* __restrict__ vsum_out, float* __restrict__ ec_row,
                                                          int64_t R) {
  if ((int)blockIdx.x < ncb) {
    constexpr int kLanes = 8;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t idx = g / kLanes;
    const int sub = (int)(g % kLanes);
    const bool ok = idx < B * C;
    const int64_t b = ok ? idx / C : 0, j = ok ? idx % C : 0;
    const int64_t pe = S / rows_per_part;                 // partial blocks per example
    double a = 0.0, v = 0.0;
    for (int64_t k = sub; k < pe; k += kLanes) {
      const int64_t at = (b * pe + k) * C + j;
      if (ec_col) a += (double)col_part[at];
      if (vsum_out) v += (double)vsum_part[at];
    }
    for (int o = 1; o < kLanes; o <<= 1) {
      a += __shfl_xor(a, o, 64);
      v += __shfl_xor(v, o, 64);
    }
    if (!ok || sub != 0) return;
    if (ec_col) ec_col[idx] = (float)(a / (double)S);
    if (vsum_out) vsum_out[idx] = (float)v;
    return;
  }
  const int64_t t = (int64_t)(blockIdx.x - ncb) * 256 + threadIdx.x;
  if (t >= R) return;
  double a = 0.0;
  for (int k = 0; k < n_ct; ++k) a += (double)row_part[t * n_ct + k];
  ec_row[t] = (float)(a / (double)C);
}

// ec_mean[b] = mean of the example's token means, one block per example, fixed order.
__global__ __launch_bounds__(256) void mx_mean_kernel(int64_t S, const float* __restrict__ ec_row,
                                                      float* __restrict__ ec_mean) {
  const int64_t a = (int64_t)blockIdx.x * S;
  double s = 0.0;
  for (int64_t t = threadIdx.x; t < S; t += 256) s += (double)ec_row[a + t];
  __shared__ double red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) ec_mean[blockIdx.x] = (float)(red[0] / (double)S);
}

// ------------------------------------------------------------- FP4 GEMM ----
// out [M x N] (f32) = A [M x K] . B [N x K]^T with both operands MXFP4 and
// K-major: codes 2 per byte (ld in bytes), E8M0 scales [K/128][rows][4].  256 x
// 256 tile per 256-thread workgroup, four waves of 128 x 128 (4 x 4 blocks of
// v_mfma_scale_f32_32x32x64_f8f6f4), K step 128 (64 bytes per row).  A stage
// holds the A and B tiles (256 rows x 64 B each, 16-byte chunks swizzled as
// c ^ f(row)) and their scale words (one 4-byte word per row = the 4 blocks of
// the K step), all moved global -> LDS by buffer-load DMA; a ring of 4 stages.
// Operand lane layout of the FP4 MFMA (checked on the device): lane l holds row
// (or column) l % 32 and K elements 32 (l / 32) .. + 31, 16 bytes, the first in
// the low nibble; byte 0 of its scale register is that (row, K block)'s E8M0.
// Output: lane l, register r -> row (r / 4) 8 + (l / 32) 4 + r % 4, column l % 32.
constexpr int kMxStages = 4;
constexpr int kMxStageBytes = 32768 + 2048;
// Four separate LDS objects rather than one indexed array: the compiler then
// sees that a step's LDS reads and the DMA refilling another stage touch
// different memory, and does not drain every outstanding load before the reads.
__shared__ __attribute__((aligned(1024))) uint8_t g_mx0[kMxStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_mx1[kMxStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_mx2[kMxStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_mx3[kMxStageBytes];
template <int S>
__device__ __forceinline__ uint8_t* mx_stage() {
  if constexpr (S == 0) return g_mx0;
  else if constexpr (S == 1) return g_mx1;
  else if constexpr (S == 2) return g_mx2;
  else return g_mx3;
}

struct MxGemm {
  const uint8_t* A; int64_t lda; const uint8_t* As; int64_t ldas;
  const uint8_t* B; int64_t ldb; const uint8_t* Bs; int64_t ldbs;
  int64_t M, N, K;
  int tiles_m, tiles_n;
};

// Epilogue: out = acc - correction.  DX: rows are tokens; corr = v[b][n] +
// (eps_t - mu_b) rW[n].  DW: rows are channels; corr = sum_b ebar[b][m] xs[b][n] + u[n].
struct MxEpi {
  const float* ec_row; const float* ec_mean; const float* vec; const float* rW;
  const float* ebar; const float* xs; const float* u;
  int64_t S, B;
  float* out; int64_t ld_out;
};
constexpr int kMxMaxB = 8;

__device__ __forceinline__ int mx_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

struct MxRsrc { __amdgpu_buffer_rsrc_t a, b, sa, sb, z; int nk; };

// Stage kt of the K loop; past the last step (kt >= nk) every load goes through
// an empty descriptor and lands zeros, which add nothing to the accumulators.
__device__ __forceinline__ void mx_load_stage(const MxGemm& g, uint8_t* st, int64_t m0, int64_t n0, int kt,
                                              const MxRsrc& r) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool live = kt < r.nk;
  const MxRsrc rs{live ? r.a : r.z, live ? r.b : r.z, live ? r.sa : r.z, live ? r.sb : r.z, r.z, r.nk};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int blk = wave * 4 + q;
    const int row = blk * 16 + (lane >> 2);
    const int c = (lane & 3) ^ mx_swz(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.a, (lds_void*)(st + blk * 1024), 16,
                                             (uint32_t)((m0 + row) * g.lda + c * 16), (uint32_t)kt * 64u, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.b, (lds_void*)(st + 16384 + blk * 1024), 16,
                                             (uint32_t)((n0 + row) * g.ldb + c * 16), (uint32_t)kt * 64u, 0, 0);
  }
  // scale words: this wave's 64 rows of A and of B, one dword per lane
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.sa, (lds_void*)(st + 32768 + wave * 256), 4,
                                           (uint32_t)((m0 + wave * 64 + lane) * 4), (uint32_t)(kt * g.ldas), 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.sb, (lds_void*)(st + 33792 + wave * 256), 4,
                                           (uint32_t)((n0 + wave * 64 + lane) * 4), (uint32_t)(kt * g.ldbs), 0, 0);
}

// s_waitcnt: at most n vector-memory ops outstanding, no LDS ops.
#define S3R_MX_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x70 | 0xF00)
#define S3R_MX_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

constexpr int kMxSgMfma = 0x008, kMxSgDsRead = 0x100, kMxSgVmem = 0x010;

// One K step (128 elements) on stage S = kt % 4: wait for this wave's loads of
// the stage, barrier (all waves' loads visible; the stage read in the previous
// step is retired), refill that retired stage with step kt + 3, then 2 x 16
// MFMAs with the second half-step's fragments read during the first half's.
template <int S>
__device__ __forceinline__ void mx_step(const MxGemm& g, int64_t m0, int64_t n0, int kt, const MxRsrc& rs,
                                        v16f (&acc)[4][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r31 = lane & 31, hk = lane >> 5;
  S3R_MX_WAIT_VM(20);
  S3R_MX_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  mx_load_stage(g, mx_stage<(S + 3) % 4>(), m0, n0, kt + 3, rs);
  const uint8_t* st = mx_stage<S>();
  uint32_t sa[4], sb[4];
  v8i fa[2][4], fb[2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c = kk * 2 + hk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra_ = wm * 128 + i * 32 + r31, rb_ = wn * 128 + i * 32 + r31;
      const uint4 x = *reinterpret_cast<const uint4*>(st + ra_ * 64 + ((c ^ mx_swz(ra_)) << 4));
      const uint4 y = *reinterpret_cast<const uint4*>(st + 16384 + rb_ * 64 + ((c ^ mx_swz(rb_)) << 4));
      fa[kk][i] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
      fb[kk][i] = v8i{(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
    }
    if (kk == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa[i] = *reinterpret_cast<const uint32_t*>(st + 32768 + (wm * 128 + i * 32 + r31) * 4);
        sb[i] = *reinterpret_cast<const uint32_t*>(st + 33792 + (wn * 128 + i * 32 + r31) * 4);
      }
    }
  }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int sh = 8 * (kk * 2 + hk);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[kk][i], fb[kk][j], acc[i][j], 4, 4, 0,
                                                                    (int)((sa[i] >> sh) & 0xFFu), 0,
                                                                    (int)((sb[j] >> sh) & 0xFFu));
  }
  // schedule: the first half-step's fragment and scale reads, then its MFMAs with
  // the second half-step's reads between them, and the refill's 10 buffer loads
  // spread one per MFMA pair, so that no burst of loads stalls the MFMA issue
  __builtin_amdgcn_sched_group_barrier(kMxSgDsRead, 16, 0);
#pragma unroll
  for (int x = 0; x < 32; ++x) {
    __builtin_amdgcn_sched_group_barrier(kMxSgMfma, 1, 0);
    if (x < 8) __builtin_amdgcn_sched_group_barrier(kMxSgDsRead, 1, 0);
    if ((x & 1) && x < 20) __builtin_amdgcn_sched_group_barrier(kMxSgVmem, 1, 0);
  }
}

template <bool DW, bool EC, int NB>
__global__ __launch_bounds__(256, 1) void mx_gemm_kernel(MxGemm g, MxEpi ep) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int bid = blockIdx.x;
  const int nblocks = g.tiles_m * g.tiles_n;
  if (nblocks % 8 == 0) bid = (bid % 8) * (nblocks / 8) + bid / 8;   // a contiguous range of tiles per XCD
  const int group = 8 * g.tiles_n;
  const int first_m = (bid / group) * 8;
  const int gsz = min(g.tiles_m - first_m, 8);
  const int tm = first_m + (bid % group) % gsz, tn = (bid % group) / gsz;
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int nk = (int)(g.K / 128);
  // descriptors over whole operands: rows past M (N) read zeros
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, (int)(uint32_t)(g.M * g.lda), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)g.B, (short)0, (int)(uint32_t)(g.N * g.ldb), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)g.As, (short)0, (int)(uint32_t)(nk * g.ldas), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)g.Bs, (short)0, (int)(uint32_t)(nk * g.ldbs), kRsrcWord3);

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Stages 0..2 up front; every step refills one stage, so a step always finds
  // exactly the loads of the two following stages in flight.
  // The step count is rounded up to a multiple of 4 (the stage ring's period);
  // the extra steps multiply zeros.
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, 0, kRsrcWord3);
  const MxRsrc rs{ra, rb, rsa, rsb, rz, nk};
  mx_load_stage(g, mx_stage<0>(), m0, n0, 0, rs);
  mx_load_stage(g, mx_stage<1>(), m0, n0, 1, rs);
  mx_load_stage(g, mx_stage<2>(), m0, n0, 2, rs);
  for (int kt = 0; kt < nk; kt += 4) {
    mx_step<0>(g, m0, n0, kt, rs, acc);
    mx_step<1>(g, m0, n0, kt + 1, rs, acc);
    mx_step<2>(g, m0, n0, kt + 2, rs, acc);
    mx_step<3>(g, m0, n0, kt + 3, rs, acc);
  }
  S3R_MX_WAIT_VM(0);
  S3R_MX_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  const int r31 = lane & 31, hk = lane >> 5;

  // epilogue: per-row values of the tile staged in LDS (the stages are free now),
  // per-column values in registers
  float* s_rowc = reinterpret_cast<float*>(mx_stage<0>());             // dX: eps_t - mu_b; dW: ebar[b][row] (b-major)
  int* s_rowb = reinterpret_cast<int*>(mx_stage<1>());                // dX: the row's example, relative to the tile's first
  float* s_v = reinterpret_cast<float*>(mx_stage<2>());               // dX: v[b0 + b][tile column], b < NB
  const int64_t b_first = DW ? 0 : m0 / ep.S;
  if constexpr (EC) {
    for (int r = threadIdx.x; r < 256; r += 256) {
      const int64_t m = m0 + r;
      if constexpr (!DW) {
        const int64_t b = m < g.M ? m / ep.S : b_first;
        s_rowc[r] = m < g.M ? ep.ec_row[m] - ep.ec_mean[b] : 0.f;
        s_rowb[r] = (int)(b - b_first);
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) s_rowc[b * 256 + r] = (b < ep.B && m < g.M) ? ep.ebar[b * g.M + m] : 0.f;
      }
    }
    if constexpr (!DW) {
      const int64_t nbt = min((int64_t)NB, ep.B - b_first);
      for (int x = threadIdx.x; x < NB * 256; x += 256) {
        const int b = x / 256, cc = x % 256;
        const int64_t n = n0 + cc;
        s_v[x] = (b < nbt && n < g.N) ? ep.vec[(b_first + b) * g.N + n] : 0.f;
      }
    }
  }
  __syncthreads();
  const int rows_here = (int)min((int64_t)256, g.M - m0);
  const uint32_t ld4 = (uint32_t)ep.ld_out * 4u;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ep.out + m0 * ep.ld_out), (short)0, (int)((uint32_t)rows_here * ld4), kRsrcWord3);
  float cA[4], cU[4], xsb[4][NB];
  bool n_ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 128 + j * 32 + r31;
    n_ok[j] = n < g.N;
    cA[j] = 0.f; cU[j] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) xsb[j][b] = 0.f;
    if (EC && n_ok[j]) {
      if constexpr (!DW) cA[j] = ep.rW[n];
      else {
        cU[j] = ep.u[n];
#pragma unroll
        for (int b = 0; b < NB; ++b) xsb[j][b] = b < ep.B ? ep.xs[b * g.N + n] : 0.f;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      // four consecutive rows of this lane: lr = wm * 128 + i * 32 + rq * 8 + hk * 4 + rr
      float rc[4], eb[4][NB];
      int rb[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int lr = wm * 128 + i * 32 + rq * 8 + hk * 4 + rr;
        rc[rr] = 0.f; rb[rr] = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) eb[rr][b] = 0.f;
        if constexpr (EC) {
          if constexpr (!DW) { rc[rr] = s_rowc[lr]; rb[rr] = s_rowb[lr]; }
          else {
#pragma unroll
            for (int b = 0; b < NB; ++b) eb[rr][b] = s_rowc[b * 256 + lr];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!n_ok[j]) continue;
        const int cc = wn * 128 + j * 32 + r31;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float o = acc[i][j][rq * 4 + rr];
          if constexpr (EC) {
            if constexpr (!DW) {
              o -= s_v[rb[rr] * 256 + cc] + rc[rr] * cA[j];
            } else {
              float t = cU[j];
#pragma unroll
              for (int b = 0; b < NB; ++b) t = fmaf(eb[rr][b], xsb[j][b], t);
              o -= t;
            }
          }
          const uint32_t urow = (uint32_t)(wm * 128 + i * 32 + rq * 8 + rr);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(o), ro,
                                                (uint32_t)(hk * 4) * ld4 + (uint32_t)(cc * 4 + n0 * 4), urow * ld4, 0);
        }
      }
    }
}

// ------------------------------------------------ correction products ----
// out[b][n] = sum over k of coef[b][k] * dequant(P[n][k]) for b < nb, P an MXFP4
// matrix [N x K] (K-major codes, scales [K/128][N][4]).  A block of 4 waves owns
// 4 * RPW rows (RPW per wave); K runs in chunks of 2048 in which lane l takes
// the 32-element block l: its 16 code bytes, its scale, and the chunk's
// coefficients from LDS, stored [b][i4][lane] (float4 units) so that a wave's
// reads are conflict-free.  Fixed order: per-lane sums, then an xor butterfly.
constexpr int kRdChunk = 2048;

__device__ __forceinline__ float e2m1_times(uint32_t c, float sc) { return e2m1_value(c) * sc; }

template <int NB, int RPW>
__global__ __launch_bounds__(256) void mx_rowdot_kernel(const uint8_t* __restrict__ P, int64_t ldp,
                                                        const uint8_t* __restrict__ Ps, int64_t ldps, int64_t N,
                                                        int64_t K, int nb, const float* __restrict__ coef,
                                                        float* __restrict__ out) {
  __shared__ float4 s_c[NB][8][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
  float acc[RPW][NB];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
  for (int64_t kc = 0; kc < K; kc += kRdChunk) {
    __syncthreads();                                    // the previous chunk's coefficients are consumed
    for (int x = threadIdx.x; x < NB * kRdChunk; x += 256) {
      const int b = x / kRdChunk, e = x % kRdChunk;    // element e of the chunk -> lane e / 32, i4 (e % 32) / 4
      const float v = (b < nb && kc + e < K) ? coef[(int64_t)b * K + kc + e] : 0.f;
      reinterpret_cast<float*>(&s_c[b][(e & 31) >> 2][e >> 5])[e & 3] = v;
    }
    __syncthreads();
    const int64_t k = kc + lane * 32;
    if (k >= K) continue;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int64_t n = n0 + r;
      if (n >= N) break;
      const uint4 w = *reinterpret_cast<const uint4*>(P + n * ldp + k / 2);
      const float sc = __builtin_ldexpf(1.f, (int)Ps[(k / 128) * ldps + n * 4 + ((k / 32) & 3)] - 127);
      const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i4 = 0; i4 < 8; ++i4) {
        const uint32_t word = wv[i4 >> 1] >> (16 * (i4 & 1));
        const float x0 = e2m1_times(word & 15u, sc), x1 = e2m1_times((word >> 4) & 15u, sc);
        const float x2 = e2m1_times((word >> 8) & 15u, sc), x3 = e2m1_times((word >> 12) & 15u, sc);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b >= nb) break;
          const float4 c = s_c[b][i4][lane];
          float a = acc[r][b];
          a = fmaf(c.x, x0, a);
          a = fmaf(c.y, x1, a);
          a = fmaf(c.z, x2, a);
          a = fmaf(c.w, x3, a);
          acc[r][b] = a;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float a = acc[r][b];
      for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
      if (lane == 0 && b < nb && n0 + r < N) out[(int64_t)b * N + n0 + r] = a;
    }
}

// c[t] = ec_row[t] - ec_mean[t / S]
__global__ void mx_token_coef_kernel(int64_t T, int64_t S, const float* __restrict__ ec_row,
                                     const float* __restrict__ ec_mean, float* __restrict__ c) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < T) c[t] = ec_row[t] - ec_mean[t / S];
}

}  // namespace

// ------------------------------------------------------------- launchers ----
namespace {

bool al(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct MxQuantWs { size_t rph, cph, rpt, cpt, total; };
MxQuantWs mx_quant_ws(int64_t T, int64_t D, bool ec) {
  MxQuantWs w{};
  size_t off = kWsHeaderBytes;
  if (ec) {
    w.rph = off; off = align_up(off + (size_t)T * ((D + 511) / 512) * 4, 256);
    w.cph = off; off = align_up(off + (size_t)(T / 64) * D * 4, 256);
    w.rpt = off; off = align_up(off + (size_t)T * ((D + 63) / 64) * 4, 256);
    w.cpt = off; off = align_up(off + (size_t)(T / 32) * D * 4, 256);
  }
  w.total = off;
  return w;
}

template <typename TIn>
hipError_t mx_quant_both(const MxQuantArgs& a, const MxQuantWs& L, hipStream_t st) {
  MxQuant p{};
  p.R = a.T; p.C = a.D; p.S = a.S; p.ld = a.ld_g; p.mode = a.mode; p.layer = a.layer; p.seed = a.seed;
  p.stream_word = a.stream << 16; p.D_index = a.D;
  const TIn* G = (const TIn*)a.G;
  float* rph = (float*)(a.ws + L.rph); float* cph = (float*)(a.ws + L.cph);
  float* rpt = (float*)(a.ws + L.rpt); float* cpt = (float*)(a.ws + L.cpt);
  const dim3 gh((unsigned)(a.T / 64), (unsigned)((a.D + 511) / 512));
  const dim3 gt((unsigned)(a.T / 128), (unsigned)((a.D + 63) / 64));
  if (a.ec) {
    hipLaunchKernelGGL((mx_quant_rows_kernel<TIn, true>), gh, dim3(256), 0, st, p, G, a.Qh, a.ld_qh, a.Qhs, a.ld_qhs,
                       rph, cph, a.flags);
    hipLaunchKernelGGL((mx_quant_cols_kernel<TIn, true, false>), gt, dim3(256), 0, st, p, G, a.Qt, a.ld_qt, a.Qts,
                       a.ld_qts, rpt, cpt, (float*)nullptr, a.flags);
    const int64_t B = a.T / a.S;
    const int64_t ncb = (B * a.D * 8 + 255) / 256, nrb = (a.T + 255) / 256;
    hipLaunchKernelGGL(mx_finalize_kernel, dim3((unsigned)(ncb + nrb)), dim3(256), 0, st, B, a.D, a.S, 64,
                       (int)((a.D + 511) / 512), (int)ncb, (const float*)cph, (const float*)nullptr,
                       (const float*)rph, a.ec_col_h, (float*)nullptr, a.ec_row_h, a.T);
    hipLaunchKernelGGL(mx_finalize_kernel, dim3((unsigned)(ncb + nrb)), dim3(256), 0, st, B, a.D, a.S, 32,
                       (int)((a.D + 63) / 64), (int)ncb, (const float*)cpt, (const float*)nullptr,
                       (const float*)rpt, a.ec_col_t, (float*)nullptr, a.ec_row_t, a.T);
    hipLaunchKernelGGL(mx_mean_kernel, dim3((unsigned)B), dim3(256), 0, st, a.S, (const float*)a.ec_row_h,
                       a.ec_mean_h);
    hipLaunchKernelGGL(mx_mean_kernel, dim3((unsigned)B), dim3(256), 0, st, a.S, (const float*)a.ec_row_t,
                       a.ec_mean_t);
  } else {
    hipLaunchKernelGGL((mx_quant_rows_kernel<TIn, false>), gh, dim3(256), 0, st, p, G, a.Qh, a.ld_qh, a.Qhs, a.ld_qhs,
                       (float*)nullptr, (float*)nullptr, a.flags);
    hipLaunchKernelGGL((mx_quant_cols_kernel<TIn, false, false>), gt, dim3(256), 0, st, p, G, a.Qt, a.ld_qt, a.Qts,
                       a.ld_qts, (float*)nullptr, (float*)nullptr, (float*)nullptr, a.flags);
  }
  return hipGetLastError();
}

template <typename TIn>
hipError_t mx_operand_t(const MxOperandArgs& a, hipStream_t st) {
  MxQuant p{};
  p.R = a.R; p.C = a.C; p.S = a.S; p.ld = a.ld; p.mode = 0; p.D_index = a.C;
  float* vsp = (float*)(a.ws + kWsHeaderBytes);
  const dim3 gt((unsigned)(a.R / 128), (unsigned)((a.C + 63) / 64));
  if (a.colsum) {
    hipLaunchKernelGGL((mx_quant_cols_kernel<TIn, false, true>), gt, dim3(256), 0, st, p, (const TIn*)a.M, a.Mt,
                       a.ld_t, a.Mts, a.ld_ts, (float*)nullptr, (float*)nullptr, vsp, a.flags);
    const int64_t B = a.R / a.S;
    const int64_t ncb = (B * a.C * 8 + 255) / 256;
    hipLaunchKernelGGL(mx_finalize_kernel, dim3((unsigned)ncb), dim3(256), 0, st, B, a.C, a.S, 32, 1, (int)ncb,
                       (const float*)nullptr, (const float*)vsp, (const float*)nullptr, (float*)nullptr, a.colsum,
                       (float*)nullptr, (int64_t)0);
  } else {
    hipLaunchKernelGGL((mx_quant_cols_kernel<TIn, false, false>), gt, dim3(256), 0, st, p, (const TIn*)a.M, a.Mt,
                       a.ld_t, a.Mts, a.ld_ts, (float*)nullptr, (float*)nullptr, (float*)nullptr, a.flags);
  }
  return hipGetLastError();
}

template <bool DW, bool EC, int NB>
void run_mx_gemm(const MxGemm& g, const MxEpi& ep, hipStream_t st) {
  GemmTiming& tm = gemm_timing();
  const GemmTiming ev = tm;
  tm = GemmTiming{};
  if (ev.start) (void)hipEventRecord(ev.start, st);
  hipLaunchKernelGGL((mx_gemm_kernel<DW, EC, NB>), dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(256), 0, st, g, ep);
  if (ev.stop) (void)hipEventRecord(ev.stop, st);
}

MxGemm make_mx_gemm(const uint8_t* A, int64_t lda, const uint8_t* As, int64_t ldas, const uint8_t* B, int64_t ldb,
                    const uint8_t* Bs, int64_t ldbs, int64_t M, int64_t N, int64_t K) {
  MxGemm g{A, lda, As, ldas, B, ldb, Bs, ldbs, M, N, K, (int)((M + 255) / 256), (int)((N + 255) / 256)};
  return g;
}

}  // namespace

size_t mx_quant_workspace(int64_t T, int64_t D, int ec) { return mx_quant_ws(T, D, ec != 0).total; }
size_t mx_operand_workspace(int64_t R, int64_t C) { return kWsHeaderBytes + align_up((size_t)(R / 32) * C * 4, 256); }
size_t mx_backward_workspace(int64_t T, int64_t d_in, int64_t B) {
  return kWsHeaderBytes + align_up((size_t)B * d_in * 4, 256) + align_up((size_t)T * 4, 256) +
         align_up((size_t)d_in * 4, 256);
}

hipError_t launch_mx_quantize(const MxQuantArgs& a, hipStream_t st) {
  const MxQuantWs L = mx_quant_ws(a.T, a.D, a.ec != 0);
  return a.g_dtype == S3R_BF16 ? mx_quant_both<uint16_t>(a, L, st) : mx_quant_both<float>(a, L, st);
}

hipError_t launch_mx_operand(const MxOperandArgs& a, hipStream_t st) {
  return a.dtype == S3R_BF16 ? mx_operand_t<uint16_t>(a, st) : mx_operand_t<float>(a, st);
}

hipError_t launch_mx_backward_dx(const MxBwArgs& a, hipStream_t st) {
  const int64_t B = a.T / a.S;
  MxEpi ep{};
  ep.S = a.S; ep.B = B; ep.out = a.out; ep.ld_out = a.ld_out;
  if (a.ec) {
    float* v = (float*)(a.ws + kWsHeaderBytes);
    // v_b[i] = sum_j ebar_b[j] dq(W)[j][i]: rows of the K-major Wt [d_in x D], eight examples per pass
    for (int64_t b0 = 0; b0 < B; b0 += 4)
      hipLaunchKernelGGL((mx_rowdot_kernel<4, 8>), dim3((unsigned)((a.d_in + 31) / 32)), dim3(256), 0, st, a.B, a.ldb,
                         a.Bs, a.ldbs, a.d_in, a.K, (int)min((int64_t)4, B - b0), a.ec_col + b0 * a.K,
                         v + b0 * a.d_in);
    ep.ec_row = a.ec_row; ep.ec_mean = a.ec_mean; ep.vec = v; ep.rW = a.vcol;
  }
  const MxGemm g = make_mx_gemm(a.A, a.lda, a.As, a.ldas, a.B, a.ldb, a.Bs, a.ldbs, a.T, a.d_in, a.K);
  if (a.ec) run_mx_gemm<false, true, 4>(g, ep, st);
  else run_mx_gemm<false, false, 1>(g, ep, st);
  return hipGetLastError();
}

hipError_t launch_mx_backward_dw(const MxBwArgs& a, hipStream_t st) {
  const int64_t B = a.T / a.S;
  MxEpi ep{};
  ep.S = a.S; ep.B = B; ep.out = a.out; ep.ld_out = a.ld_out;
  if (a.ec) {
    float* coef = (float*)(a.ws + kWsHeaderBytes + align_up((size_t)B * a.d_in * 4, 256));
    float* u = (float*)(a.ws + kWsHeaderBytes + align_up((size_t)B * a.d_in * 4, 256) + align_up((size_t)a.T * 4, 256));
    hipLaunchKernelGGL(mx_token_coef_kernel, dim3((unsigned)((a.T + 255) / 256)), dim3(256), 0, st, a.T, a.S,
                       a.ec_row, a.ec_mean, coef);
    // u[i] = sum_t (eps_t - mu_b) dq(X)[t][i]: rows of the K-major Xt [d_in x T]
    hipLaunchKernelGGL((mx_rowdot_kernel<1, 8>), dim3((unsigned)((a.d_in + 31) / 32)), dim3(256), 0, st, a.B, a.ldb,
                       a.Bs, a.ldbs, a.d_in, a.T, 1, (const float*)coef, u);
    ep.ebar = a.ec_col; ep.xs = a.vcol; ep.u = u;
  }
  // dW [D x d_in] = Qt [D x T] . Xt [d_in x T]^T
  const MxGemm g = make_mx_gemm(a.A, a.lda, a.As, a.ldas, a.B, a.ldb, a.Bs, a.ldbs, a.D, a.d_in, a.T);
  if (!a.ec) run_mx_gemm<true, false, 1>(g, ep, st);
  else if (B <= 1) run_mx_gemm<true, true, 1>(g, ep, st);
  else if (B <= 2) run_mx_gemm<true, true, 2>(g, ep, st);
  else if (B <= 4) run_mx_gemm<true, true, 4>(g, ep, st);
  else run_mx_gemm<true, true, 8>(g, ep, st);
  return hipGetLastError();
}

}  // namespace s3r
