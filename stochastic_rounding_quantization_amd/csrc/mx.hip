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

// Code layout of every MXFP4 matrix (R rows, K contraction elements, two codes a byte): blocks of
// 256 rows x 128 elements, 64 bytes a row and 16 KiB a block, row-major inside; block (rb, kb)
// starts at rb * ld + kb * 16384 (ld >= 128 K, the stride between 256-row blocks). A GEMM step of
// a 256-row tile is then one contiguous 16 KiB run, which its DMA reads in whole cache lines.
constexpr int kMxBlkBytes = 16384;
__device__ __forceinline__ int64_t mx_code_off(int64_t row, int64_t byte, int64_t ld) {
  return (row >> 8) * ld + (byte >> 6) * kMxBlkBytes + (row & 255) * 64 + (byte & 63);
}

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

// E2M1 code of v in a block with scale exponent k (kp1 = k + 1), on the
// block's grid in units of the spacing s = 2^(M - k - 2), M = max(e(v), k + 1)
// with e(v) the frexp exponent (|v| = m 2^e, m in [0.5, 1)), taken from the
// exponent field (zero and subnormals give -126 <= k + 1): s is 0.5, 1 or 2
// as |v / 2^k| lies below 2, in [2, 4) or in [4, 6].  t = v / s * 2^24 is an
// exact power-of-two scaling; n = floor(t / 2^24 + R / 2^24) = (floor(t) + R)
// >> 24 (SR / S3R, R the threshold in units of 2^-24) or rint(v / s) (RTNE).
// |n| + 2 (M - k - 1) is the index into 0, 0.5, 1, 1.5, 2, 3, 4, 6, and the
// dequantized value n s 2^k = n 2^(M - 2).
template <bool RT>
__device__ __forceinline__ uint32_t e2m1_round(float v, int kp1, int32_t R, int& n, int& M) {
  M = max((int)((__float_as_uint(v) >> 23) & 0xFFu) - 126, kp1);
  if constexpr (RT) {
    n = (int)__builtin_rintf(__builtin_ldexpf(v, 2 - M));
  } else {
    const float t = __builtin_ldexpf(v, 26 - M);
    int32_t X;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(X) : "v"(t));
    n = (X + R) >> 24;
  }
  const uint32_t idx = (uint32_t)(abs(n) + 2 * (M - kp1));
  return (n < 0 ? 8u : 0u) | idx;
}

// Scale byte of a block of 32 values (255: a non-finite value in the block).
__device__ __forceinline__ int mx_scale(const float (&v)[32]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  return block_scale_byte(m);
}

// Element i of a block with scale byte sb: its code ORed into w[i / 8], and
// (EC) its error dequant - v.  A non-finite block (sb 255) gets zero codes and
// zero errors.
template <bool RT>
__device__ __forceinline__ float mx_elem(float v, int sb, int32_t R, int i, uint32_t (&w)[4]) {
  int n, M;
  const uint32_t c = e2m1_round<RT>(v, sb - 126, R, n, M);
  const bool bad = sb == 255;
  w[i >> 3] |= (bad ? 0u : c) << (4 * (i & 7));
  return bad ? 0.f : __builtin_ldexpf((float)n, M - 2) - v;
}

// Quantize 32 values with one block scale: codes packed 8 per word into w[4],
// (EC) the errors into e[32]; returns the scale byte.
template <bool EC, bool RT>
__device__ __forceinline__ int mx_block(const float (&v)[32], const int32_t (&R)[32], uint32_t (&w)[4],
                                        float (&e)[32]) {
  const int sb = mx_scale(v);
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float x = mx_elem<RT>(v[i], sb, R[i], i, w);
    if constexpr (EC) e[i] = x;
  }
  return sb;
}

// ------------------------------------------- both blockings of G, fused ----
// One read of G gives Q_h (blocks of 32 along D) and Q_t (blocks of 32 along
// T, stored transposed).  A block of 256 threads owns a tile of 64 tokens x
// 256 channels, staged in LDS as read:
//   phase A  thread (row tid / 8 + 32 h, block tid % 8), h = 0, 1: 32
//            consecutive elements of a row (coalesced 16-byte loads) and its
//            Q_h block: scale byte and 16 code bytes;
//   phase B  thread (channels 2 p, 2 p + 1 with p = tid % 128, token block
//            tid / 128): 2 x 32 elements from LDS, two Q_t blocks: scale
//            bytes and 16 code bytes into rows 2 p, 2 p + 1 of Q_t.
// Thresholds: S3R per token from LDS; SR per element from the same counters as
// the INT8 path (element e = t D + j, word e % 4 of counter e / 4).  In phase
// B a counter's four channels belong to two adjacent lanes: each draws the
// counters of every other token and the two swap the word pairs.
// EC partials (fixed order, fp32): E_h row sums over the tile's channels
// (rph[t * n_ct + ctile]) and column sums over its 64 tokens (cph[ttile * D +
// j]), both from phase A by lane reductions; E_t column sums per 32-token
// block (cpt[tblk * D + j]) and row sums over the tile's channels (rpt[t *
// n_ct + ctile]) from phase B.
constexpr int kFusedRows = 64, kFusedCols = 256;

template <typename TIn>
struct FusedLds {
  static constexpr int kPad = 16 / (int)sizeof(TIn);        // one 16-byte chunk per row
  TIn g[kFusedRows][kFusedCols + kPad];
  int32_t thr[kFusedRows];
  float colh[4][kFusedCols];
  float red[4][32];
};

template <typename TIn>
__device__ __forceinline__ void load32(const TIn* src, float (&v)[32], bool active) {
  if constexpr (sizeof(TIn) == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = active ? reinterpret_cast<const uint4*>(src)[q] : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[q * 8 + 2 * i] = __uint_as_float(ww[i] << 16);
        v[q * 8 + 2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 w = active ? reinterpret_cast<const float4*>(src)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[q * 4] = w.x; v[q * 4 + 1] = w.y; v[q * 4 + 2] = w.z; v[q * 4 + 3] = w.w;
    }
  }
}

// two adjacent channels of one staged row
__device__ __forceinline__ void lds_pair(const uint16_t* p, float& a, float& b) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  a = __uint_as_float(w << 16);
  b = __uint_as_float(w & 0xFFFF0000u);
}
__device__ __forceinline__ void lds_pair(const float* p, float& a, float& b) {
  const float2 w = *reinterpret_cast<const float2*>(p);
  a = w.x;
  b = w.y;
}

template <typename TIn, bool EC, int MODE>
__global__ __launch_bounds__(256, sizeof(TIn) == 2 ? 3 : 2) void mx_quant_fused_kernel(MxQuant p, const TIn* __restrict__ G,
                                                             uint8_t* __restrict__ Qh, int64_t ld_qh,
                                                             uint8_t* __restrict__ Qhs, int64_t ld_qhs,
                                                             uint8_t* __restrict__ Qt, int64_t ld_qt,
                                                             uint8_t* __restrict__ Qts, int64_t ld_qts,
                                                             float* __restrict__ rph, float* __restrict__ cph,
                                                             float* __restrict__ rpt, float* __restrict__ cpt,
                                                             uint32_t* __restrict__ flags) {
  constexpr bool RT = MODE == 0;
  __shared__ __attribute__((aligned(16))) FusedLds<TIn> L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kFusedRows, c0 = (int64_t)blockIdx.y * kFusedCols;
  const int n_ct = (int)((p.C + kFusedCols - 1) / kFusedCols);
  const uint32_t key0 = (uint32_t)p.seed, key1 = (uint32_t)(p.seed >> 32);
  if (MODE == 2 && tid < kFusedRows)
    L.thr[tid] = s3r_threshold_units24(t0 + tid, p.layer, p.seed, kTagS3R + p.stream_word);
  __syncthreads();
  bool any_bad = false;

  // ---- phase A: Q_h
  const int cb = tid & 7;
  const int64_t ca = c0 + cb * 32;
  const bool act_a = ca < p.C;                       // C % 32 == 0
  float ecol[EC ? 32 : 1];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (tid >> 3) + 32 * h;
    const int64_t t = t0 + r;
    float v[32];
    load32<TIn>(G + t * p.ld + ca, v, act_a);
    {
      // stage the raw tile
      constexpr int kChunks = 32 * (int)sizeof(TIn) / 16;
#pragma unroll
      for (int q = 0; q < kChunks; ++q) {
        uint4 x;
        if constexpr (sizeof(TIn) == 2) {
          x = make_uint4((__float_as_uint(v[q * 8]) >> 16) | (__float_as_uint(v[q * 8 + 1]) & 0xFFFF0000u),
                         (__float_as_uint(v[q * 8 + 2]) >> 16) | (__float_as_uint(v[q * 8 + 3]) & 0xFFFF0000u),
                         (__float_as_uint(v[q * 8 + 4]) >> 16) | (__float_as_uint(v[q * 8 + 5]) & 0xFFFF0000u),
                         (__float_as_uint(v[q * 8 + 6]) >> 16) | (__float_as_uint(v[q * 8 + 7]) & 0xFFFF0000u));
        } else {
          x = make_uint4(__float_as_uint(v[q * 4]), __float_as_uint(v[q * 4 + 1]), __float_as_uint(v[q * 4 + 2]),
                         __float_as_uint(v[q * 4 + 3]));
        }
        reinterpret_cast<uint4*>(&L.g[r][cb * 32])[q] = x;
      }
    }
    const int sb = mx_scale(v);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    float es = 0.f;
    const int32_t rs3 = MODE == 2 ? L.thr[r] : -1;
#pragma unroll
    for (int i4 = 0; i4 < 8; ++i4) {
      int32_t R4[4] = {rs3, rs3, rs3, rs3};
      if constexpr (MODE == 1) {
        const uint64_t e = (uint64_t)t * (uint64_t)p.D_index + (uint64_t)(ca + 4 * i4);   // e % 4 == 0
        const U4 u = philox4x32_10((uint32_t)(e >> 2), (uint32_t)(e >> 34), p.layer, kTagSR + p.stream_word,
                                   key0, key1);
        R4[0] = sr_units24(u.x); R4[1] = sr_units24(u.y); R4[2] = sr_units24(u.z); R4[3] = sr_units24(u.w);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * i4 + j;
        const float x = mx_elem<RT>(v[i], sb, R4[j], i, w);
        if constexpr (EC) {
          es += x;
          ecol[i] = h == 0 ? x : ecol[i] + x;
        }
      }
    }
    if (act_a) {
      *reinterpret_cast<uint4*>(Qh + mx_code_off(t, ca / 2, ld_qh)) = make_uint4(w[0], w[1], w[2], w[3]);
      const int64_t blk = ca / 32;
      Qhs[(blk / 4) * ld_qhs + t * 4 + (blk & 3)] = (uint8_t)sb;
      any_bad |= sb == 255;
    }
    if constexpr (EC) {
      es += __shfl_xor(es, 1, 64);
      es += __shfl_xor(es, 2, 64);
      es += __shfl_xor(es, 4, 64);
      if (cb == 0) rph[t * n_ct + blockIdx.y] = es;
    }
    asm volatile("" ::: "memory");                   // the second item's loads after the first's work
  }
  if constexpr (EC) {
    // E_h column sums over the tile's 64 rows: the lanes with this block (lane bits 5..3 vary)
    // reduce-scatter the 32 columns, 4 per lane, then the 4 waves add through LDS
#pragma unroll
    for (int o = 16; o >= 4; o >>= 1) {
      const bool hi = lane & (2 * o);      // lane bits 5, 4, 3 for o = 16, 8, 4
#pragma unroll
      for (int i = 0; i < o; ++i) {
        const float send = hi ? ecol[i] : ecol[i + o];
        ecol[i] = (hi ? ecol[i + o] : ecol[i]) + __shfl_xor(send, 2 * o, 64);
      }
    }
    const int j0 = cb * 32 + ((lane >> 5) & 1) * 16 + ((lane >> 4) & 1) * 8 + ((lane >> 3) & 1) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) L.colh[wave][j0 + j] = ecol[j];
  }
  __syncthreads();
  if constexpr (EC) {
    const int64_t c = c0 + tid;
    if (c < p.C) cph[(t0 / 64) * p.C + c] = ((L.colh[0][tid] + L.colh[1][tid]) + L.colh[2][tid]) + L.colh[3][tid];
  }

  // ---- phase B: Q_t, channels c0 + 2 pp, + 1, tokens t0 + 32 tb ..
  const int pp = tid & 127, tb = tid >> 7;
  const int64_t cpair = c0 + 2 * pp;
  const bool act_b = cpair < p.C;                    // C even: both channels or neither
  // first pass over the staged column pair: the two block scales; the values are read again below
  uint32_t ma = 0, mb = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float xa, xb;
    lds_pair(&L.g[32 * tb + i][2 * pp], xa, xb);
    ma = max(ma, __float_as_uint(xa) & 0x7FFFFFFFu);
    mb = max(mb, __float_as_uint(xb) & 0x7FFFFFFFu);
  }
  const int sba = block_scale_byte(ma), sbb = block_scale_byte(mb);
  uint32_t wa[4] = {0u, 0u, 0u, 0u}, wb[4] = {0u, 0u, 0u, 0u};
  float csa = 0.f, csb = 0.f;
  const int q = pp & 1;                              // SR: lane parity within a 4-channel counter
  // four groups of 8 rows, not unrolled (few live registers); after each group the code
  // words shift down one place, so wa[g] ends holding group g's eight codes
#pragma unroll 1
  for (int g = 0; g < 4; ++g) {
    float xs[8];                                     // EC: this thread's two channels' errors, rows 8g ..
    uint32_t ga[4] = {0u, 0u, 0u, 0u}, gb[4] = {0u, 0u, 0u, 0u};   // codes land in word 0
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const int r2 = 32 * tb + 8 * g + 2 * mm;       // staged rows r2, r2 + 1
      int32_t ra[2], rb[2];
      if constexpr (MODE == 2) {
        ra[0] = rb[0] = L.thr[r2];
        ra[1] = rb[1] = L.thr[r2 + 1];
      } else if constexpr (MODE == 1) {
        // this lane draws the counter of token r2 + q (channels cpair - 2q .. + 3) and swaps the
        // other channel pair's words with its neighbour, which drew token r2 + 1 - q
        const int64_t tq = t0 + r2 + q;
        const uint64_t e = (uint64_t)tq * (uint64_t)p.D_index + (uint64_t)(cpair - 2 * q);
        const U4 u = philox4x32_10((uint32_t)(e >> 2), (uint32_t)(e >> 34), p.layer, kTagSR + p.stream_word,
                                   key0, key1);
        const uint32_t own0 = q ? u.z : u.x, own1 = q ? u.w : u.y;
        const uint32_t give0 = q ? u.x : u.z, give1 = q ? u.y : u.w;
        const uint32_t got0 = (uint32_t)__shfl_xor((int)give0, 1, 64);
        const uint32_t got1 = (uint32_t)__shfl_xor((int)give1, 1, 64);
        ra[q] = sr_units24(own0); rb[q] = sr_units24(own1);
        ra[1 - q] = sr_units24(got0); rb[1 - q] = sr_units24(got1);
      } else {
        ra[0] = ra[1] = rb[0] = rb[1] = -1;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = 2 * mm + j;                    // position within the group's code word
        float va, vb;
        lds_pair(&L.g[r2 + j][2 * pp], va, vb);
        const float xa = mx_elem<RT>(va, sba, ra[j], i, ga);
        const float xb = mx_elem<RT>(vb, sbb, rb[j], i, gb);
        if constexpr (EC) {
          csa += xa;
          csb += xb;
          xs[i] = xa + xb;
        }
      }
    }
    wa[0] = wa[1]; wa[1] = wa[2]; wa[2] = wa[3]; wa[3] = ga[0];
    wb[0] = wb[1]; wb[1] = wb[2]; wb[2] = wb[3]; wb[3] = gb[0];
    if constexpr (EC) {
      // the 8 rows over the lanes that differ in bits 5..3 (reduce-scatter: lane keeps row
      // 8g + lane / 8), then over bits 2..0; the two waves of this token block add through LDS
#pragma unroll
      for (int o = 4; o >= 1; o >>= 1) {
        const bool hi = lane & (8 * o);
#pragma unroll
        for (int i = 0; i < o; ++i) {
          const float send = hi ? xs[i] : xs[i + o];
          xs[i] = (hi ? xs[i + o] : xs[i]) + __shfl_xor(send, 8 * o, 64);
        }
      }
      float x = xs[0];
      x += __shfl_xor(x, 1, 64);
      x += __shfl_xor(x, 2, 64);
      x += __shfl_xor(x, 4, 64);
      if ((lane & 7) == 0) L.red[wave][8 * g + (lane >> 3)] = x;
    }
  }
  const int64_t tblk = t0 / 32 + tb;
  if (act_b) {
    *reinterpret_cast<uint4*>(Qt + mx_code_off(cpair, tblk * 16, ld_qt)) = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    *reinterpret_cast<uint4*>(Qt + mx_code_off(cpair + 1, tblk * 16, ld_qt)) = make_uint4(wb[0], wb[1], wb[2], wb[3]);
    uint8_t* sp = Qts + (tblk / 4) * ld_qts + cpair * 4 + (tblk & 3);
    sp[0] = (uint8_t)sba;
    sp[4] = (uint8_t)sbb;
    any_bad |= sba == 255 || sbb == 255;
  }
  if (any_bad && flags) atomicOr(flags, S3R_FLAG_NONFINITE);
  if constexpr (EC) {
    if (act_b) {
      cpt[tblk * p.C + cpair] = csa;
      cpt[tblk * p.C + cpair + 1] = csb;
    }
    __syncthreads();
    if (tid < kFusedRows) {
      const int b2 = tid >> 5, i = tid & 31;
      rpt[(t0 + tid) * n_ct + blockIdx.y] = L.red[2 * b2][i] + L.red[2 * b2 + 1][i];
    }
  }
}

// --------------------------------------------- forward-operand prep ----
// RTNE MXFP4 of a forward operand M [R x C] row-major, blocks of 32 along R,
// output transposed: codes [C x R/2] (row c holds column c of M), scales
// [R/128][C][4].  A block of 256 threads covers 128 rows x 64 columns: lane =
// column, wave = one 32-row block; per thread the block's scale and 16 code
// bytes (the four waves write 64 contiguous bytes of an output row).  VSUM:
// the column sums of the dequantized values of each block (vsum_part[rblk * C
// + c]).
template <typename TIn, bool VSUM>
__global__ __launch_bounds__(256) void mx_operand_kernel(MxQuant p, const TIn* __restrict__ M,
                                                         uint8_t* __restrict__ out, int64_t ld_out,
                                                         uint8_t* __restrict__ sc, int64_t ld_s,
                                                         float* __restrict__ vsum_part, uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.y * 64 + lane;
  const int64_t t0 = (int64_t)blockIdx.x * 128 + wave * 32;        // this wave's block of 32 rows
  const bool active = c < p.C;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = active ? load_elem<TIn>(M + (t0 + i) * p.ld + c) : 0.f;
  int32_t R[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) R[i] = -1;
  uint32_t w[4];
  float e[32];
  const int sb = mx_block<VSUM, true>(v, R, w, e);
  if (active) {
    *reinterpret_cast<uint4*>(out + mx_code_off(c, t0 / 2, ld_out)) = make_uint4(w[0], w[1], w[2], w[3]);
    sc[(t0 / 128) * ld_s + c * 4 + ((t0 / 32) & 3)] = (uint8_t)sb;
    if (sb == 255 && flags) atomicOr(flags, S3R_FLAG_NONFINITE);
    if constexpr (VSUM) {
      float vsum = 0.f;                                  // dequantized = error + value
#pragma unroll
      for (int i = 0; i < 32; ++i) vsum += sb == 255 ? 0.f : e[i] + v[i];
      vsum_part[(t0 / 32) * p.C + c] = vsum;
    }
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
// out [M x N] (f32) = A [M x K] . B [N x K]^T with both operands MXFP4: codes in
// the 256-row block layout (ld: the bytes between 256-row blocks), E8M0 scales
// [K/128][rows][4].  256 x 128 tile per 256-thread workgroup, four waves of 128
// x 64 (4 x 2 blocks of v_mfma_scale_f32_32x32x64_f8f6f4, 128 accumulator
// registers a lane), so two workgroups share a CU and one's epilogue (128 KiB of
// f32 results) runs beside the other's K loop.  A 256 x 256 tile with one
// workgroup per CU left the matrix cores idle while its results were stored,
// which at the dX's short K loop (K = d_out) was much of the time: the down
// projection's dX took 357 against 308 us in 256 x 128 tiles, its dW 290 against
// 264 us.  A stage holds one 128-element step: the A tile's 256 rows and the B
// tile's 128 rows of 64 bytes as they lie in their code blocks (16 + 8 KiB), and
// both operands' scale words; three stages (78 KiB a workgroup) form a ring in
// which a step waits for its own stage and loads the step two ahead into the
// slot of the step before, all moved global -> LDS by buffer-load DMA.
// Operand lane layout of the FP4 MFMA (checked on the device): lane l holds row
// (or column) l % 32 and K elements 32 (l / 32) .. + 31, 16 bytes, the first in
// the low nibble; byte 0 of its scale register is that (row, K block)'s E8M0.
// Output: lane l, register r -> row (r / 4) 8 + (l / 32) 4 + r % 4, column l % 32.
constexpr int kMxB = 16384, kMxSA = 24576, kMxSB = 25600, kMxSBSpare = 26112, kMxStageBytes = 26624;
// Separate LDS objects rather than one indexed array: the compiler then sees that
// a stage's LDS reads and the DMA filling another stage touch different memory,
// and does not drain every outstanding load before the reads.
__shared__ __attribute__((aligned(1024))) uint8_t g_mx0[kMxStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_mx1[kMxStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_mx2[kMxStageBytes];
template <int S>
__device__ __forceinline__ uint8_t* mx_stage() {
  if constexpr (S == 0) return g_mx0;
  else if constexpr (S == 1) return g_mx1;
  else return g_mx2;
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

// LDS layout of a stage's A tile (and, 16 KiB on, B's): [rows][64 bytes] as in the step's code block,
// with the four 16-byte chunks of a row at permuted positions: chunk q of row r at position
// q ^ ((r >> 2) & 3), so the 16 rows of a quarter-wave's 16-byte read hit 16 different bank groups.
__device__ __forceinline__ int mx_pos(int r, int q) { return q ^ ((r >> 2) & 3); }

struct MxRsrc { __amdgpu_buffer_rsrc_t a, b, sa, sb, z; int nk; };

// Step kt (K elements 128 kt .., code block kt of the tiles' 256-row blocks) into stage st.  Every
// wave issues 8 loads: four 1 KiB pieces of A and two of B (16 rows x 64 bytes each; lane l lands at
// LDS offset 16 l of its piece and loads the chunk that belongs there), 64 of A's 256 scale words,
// and 64 of B's 128 (waves 2 and 3 load the same words as waves 0 and 1, into a spare copy, so the
// wait counts are the same in every wave).  Past the last step every load reads zeros.
__device__ __forceinline__ void mx_load(const MxGemm& g, uint8_t* st, int64_t m0, int64_t n0, int kt,
                                        const MxRsrc& r) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool live = kt < r.nk;
  const __amdgpu_buffer_rsrc_t ra = live ? r.a : r.z, rb = live ? r.b : r.z;
  const __amdgpu_buffer_rsrc_t rsa = live ? r.sa : r.z, rsb = live ? r.sb : r.z;
  // A: the tile's 256-row block; B: the 128 rows from n0 of its 256-row block (n0 % 256 is 0 or 128,
  // so a row's chunk permutation is the same counted from either)
  const uint32_t a_blk = (uint32_t)((m0 >> 8) * g.lda), b_blk = (uint32_t)((n0 >> 8) * g.ldb + (n0 & 255) * 64);
  const uint32_t koff = (uint32_t)kt * (uint32_t)kMxBlkBytes;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int piece = wave * 4 + q;
    const int row = piece * 16 + (lane >> 2);
    const uint32_t off = (uint32_t)(row * 64 + mx_pos(row, lane & 3) * 16);   // an involution
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + piece * 1024), 16, a_blk + off, koff, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int piece = wave * 2 + q;
    const int row = piece * 16 + (lane >> 2);
    const uint32_t off = (uint32_t)(row * 64 + mx_pos(row, lane & 3) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + kMxB + piece * 1024), 16, b_blk + off, koff, 0, 0);
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + kMxSA + wave * 256), 4,
                                           (uint32_t)((m0 + wave * 64 + lane) * 4), (uint32_t)(kt * g.ldas), 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + (wave < 2 ? kMxSB : kMxSBSpare) + (wave & 1) * 256),
                                           4, (uint32_t)((n0 + (wave & 1) * 64 + lane) * 4), (uint32_t)(kt * g.ldbs),
                                           0, 0);
}

// s_waitcnt: at most n vector-memory ops outstanding, no LDS ops.
#define S3R_MX_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x70 | 0xF00)
#define S3R_MX_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

constexpr int kMxSgMfma = 0x008, kMxSgDsRead = 0x100, kMxSgVmem = 0x010;

// Fragments of half-step h (K elements 64 h .. 64 h + 63 of the step): lane l holds rows (columns)
// i * 32 + l % 32 of its wave's, the 16 bytes of chunk 2 h + l / 32 of the row.
struct MxFrag { v8i a[4], b[2]; };

__device__ __forceinline__ void mx_read_frag(const uint8_t* st, int h, MxFrag& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r31 = lane & 31, c = h * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra_ = wm * 128 + i * 32 + r31;
    const uint4 x = *reinterpret_cast<const uint4*>(st + ra_ * 64 + (mx_pos(ra_, c) << 4));
    f.a[i] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rb_ = wn * 64 + j * 32 + r31;
    const uint4 y = *reinterpret_cast<const uint4*>(st + kMxB + rb_ * 64 + (mx_pos(rb_, c) << 4));
    f.b[j] = v8i{(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
  }
}

__device__ __forceinline__ void mx_read_scales(const uint8_t* st, uint32_t (&sa)[4], uint32_t (&sb)[2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r31 = lane & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sa[i] = *reinterpret_cast<const uint32_t*>(st + kMxSA + (wm * 128 + i * 32 + r31) * 4);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    sb[j] = *reinterpret_cast<const uint32_t*>(st + kMxSB + (wn * 64 + j * 32 + r31) * 4);
}

__device__ __forceinline__ void mx_mfma8(const MxFrag& f, const uint32_t (&sa)[4], const uint32_t (&sb)[2], int kk,
                                         v16f (&acc)[4][2]) {
  const int sh = 8 * (kk * 2 + ((threadIdx.x & 63) >> 5));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 4, 4, 0,
                                                                  (int)((sa[i] >> sh) & 0xFFu), 0,
                                                                  (int)((sb[j] >> sh) & 0xFFu));
}

// Step kt on stage S = kt % 3.  Its loads were issued two steps ago and step kt + 1's since; the wait
// leaves those 8 in flight.  The barrier makes every wave's loads of step kt visible and retires step
// kt - 1's stage, which takes step kt + 2.
template <int S>
__device__ __forceinline__ void mx_step(const MxGemm& g, int64_t m0, int64_t n0, int kt, const MxRsrc& rs,
                                        v16f (&acc)[4][2]) {
  S3R_MX_WAIT_VM(8);
  S3R_MX_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  const uint8_t* st = mx_stage<S>();
  uint32_t sa[4], sb[2];
  MxFrag f0, f1;
  mx_read_frag(st, 0, f0);
  mx_read_scales(st, sa, sb);
  mx_load(g, mx_stage<(S + 2) % 3>(), m0, n0, kt + 2, rs);
  mx_read_frag(st, 1, f1);
  mx_mfma8(f0, sa, sb, 0, acc);
  mx_mfma8(f1, sa, sb, 1, acc);
  // order: the loads of step kt + 2, the first half-step's 12 reads, then its 8 MFMAs each followed (the
  // first six) by one fragment read of the second half-step, then the second half-step's MFMAs
  __builtin_amdgcn_sched_group_barrier(kMxSgVmem, 8, 0);
  __builtin_amdgcn_sched_group_barrier(kMxSgDsRead, 12, 0);
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    __builtin_amdgcn_sched_group_barrier(kMxSgMfma, 1, 0);
    if (x < 6) __builtin_amdgcn_sched_group_barrier(kMxSgDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMxSgMfma, 8, 0);
}

// Epilogue of a tile: out = acc - correction, per-row values of the tile staged in LDS (two stages of
// the ring, free now), per-column values in registers.
template <bool DW, bool EC, int NB>
__device__ __forceinline__ void mx_epilogue(const MxGemm& g, const MxEpi& ep, int64_t m0, int64_t n0,
                                            v16f (&acc)[4][2]) {
  constexpr int TN = 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r31 = lane & 31, hk = lane >> 5;
  float* s_rowc = reinterpret_cast<float*>(mx_stage<0>());            // dX: eps_t - mu_b; dW: ebar[b][row] (b-major)
  int* s_rowb = reinterpret_cast<int*>(mx_stage<1>());                // dX: the row's example, relative to the tile's first
  float* s_v = reinterpret_cast<float*>(mx_stage<1>() + 4096);        // dX: v[b0 + b][tile column], b < NB
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
      for (int x = threadIdx.x; x < NB * TN; x += 256) {
        const int b = x / TN, cc = x % TN;
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
  // per-column values, loaded from a clamped column without a branch and waited for once here: a
  // load still pending inside the store loop would make each group of stores wait for every store
  // before it (vmcnt counts stores too)
  float cA[2], cU[2], xsb[2][NB];
  bool n_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + j * 32 + r31;
    n_ok[j] = n < g.N;
    const int64_t nc = n_ok[j] ? n : 0;
    cA[j] = 0.f; cU[j] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) xsb[j][b] = 0.f;
    if constexpr (EC) {
      if constexpr (!DW) cA[j] = ep.rW[nc];
      else {
        cU[j] = ep.u[nc];
#pragma unroll
        for (int b = 0; b < NB; ++b) xsb[j][b] = ep.xs[(b < ep.B ? b : 0) * g.N + nc] * (b < ep.B ? 1.f : 0.f);
      }
    }
  }
  S3R_MX_WAIT_VM(0);
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
      for (int j = 0; j < 2; ++j) {
        if (!n_ok[j]) continue;
        const int cc = wn * 64 + j * 32 + r31;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float o = acc[i][j][rq * 4 + rr];
          if constexpr (EC) {
            if constexpr (!DW) {
              o -= s_v[rb[rr] * TN + cc] + rc[rr] * cA[j];
            } else {
              float t = cU[j];
#pragma unroll
              for (int b = 0; b < NB; ++b) t = fmaf(eb[rr][b], xsb[j][b], t);
              o -= t;
            }
          }
          const uint32_t urow = (uint32_t)(wm * 128 + i * 32 + rq * 8 + rr);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(o), ro,
                                                (uint32_t)(hk * 4) * ld4 + (uint32_t)(cc * 4 + n0 * 4), urow * ld4,
                                                2 /* nontemporal: written once, kept out of the last-level cache */);
        }
      }
    }
}

template <bool DW, bool EC, int NB>
__global__ __launch_bounds__(256, 2) void mx_gemm_kernel(MxGemm g, MxEpi ep) {
  int bid = blockIdx.x;
  const int nblocks = g.tiles_m * g.tiles_n;
  if (nblocks % 8 == 0) bid = (bid % 8) * (nblocks / 8) + bid / 8;   // a contiguous range of tiles per XCD
  const int group = 8 * g.tiles_n;
  const int first_m = (bid / group) * 8;
  const int gsz = min(g.tiles_m - first_m, 8);
  const int tm = first_m + (bid % group) % gsz, tn = (bid % group) / gsz;
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 128;
  const int nk = (int)(g.K / 128);
  // descriptors over whole operands, every 256-row block of codes (rows past M or N inside the last
  // block reach only outputs that are not stored)
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.A, (short)0, (int)(uint32_t)(((g.M + 255) >> 8) * g.lda), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.B, (short)0, (int)(uint32_t)(((g.N + 255) >> 8) * g.ldb), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)g.As, (short)0, (int)(uint32_t)(nk * g.ldas), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)g.Bs, (short)0, (int)(uint32_t)(nk * g.ldbs), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, 0, kRsrcWord3);
  const MxRsrc rs{ra, rb, rsa, rsb, rz, nk};

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  mx_load(g, mx_stage<0>(), m0, n0, 0, rs);
  mx_load(g, mx_stage<1>(), m0, n0, 1, rs);
  for (int kt = 0; kt < nk; kt += 3) {
    mx_step<0>(g, m0, n0, kt, rs, acc);
    if (kt + 1 < nk) mx_step<1>(g, m0, n0, kt + 1, rs, acc);
    if (kt + 2 < nk) mx_step<2>(g, m0, n0, kt + 2, rs, acc);
  }
  S3R_MX_WAIT_VM(0);
  S3R_MX_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  mx_epilogue<DW, EC, NB>(g, ep, m0, n0, acc);
}

// ------------------------------------------------ correction products ----
// part[kc][b][n] = sum over k in chunk kc of coef[b][k] * dequant(P[n][k]) for
// b < nb, P an MXFP4 matrix [N x K] (K-major codes, scales [K/128][N][4]).
// Block (x, y): RG groups of 4 RPW rows (RPW per wave, every group's loads
// issued first, the coefficients staged once for all of them), K chunk y of 2048, in
// which lane l takes the 32-element block l: its 16 code bytes, its scale and
// the chunk's coefficients from LDS, stored [b][i4][lane] (float4 units) so a
// wave's reads are conflict-free.  Codes decode to signed multiples of 0.5,
// counted in halves (exact integers), by the hardware conversion; the block
// scale / 2 multiplies the lane's sum.  Fixed order: per-lane sums, a
// reduce-scatter of the RPW x NB sums across the wave, and mx_sum_parts over
// the chunks.
typedef float v2f __attribute__((ext_vector_type(2)));
constexpr int kRdChunk = 2048;   // 64 lanes x one 32-element block each

template <int NB, int RPW, int RG>
__global__ __launch_bounds__(256) void mx_rowdot_kernel(const uint8_t* __restrict__ P, int64_t ldp,
                                                        const uint8_t* __restrict__ Ps, int64_t ldps, int64_t N,
                                                        int64_t K, int nb, const float* __restrict__ coef,
                                                        const float* __restrict__ mean, int64_t S,
                                                        float* __restrict__ part) {
  constexpr int V = RPW * NB;                           // sums per wave
  static_assert(V == 4 || V == 8 || V == 16 || V == 32, "reduce-scatter shape");
  __shared__ float4 s_c[NB][8][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t kc = (int64_t)blockIdx.y * kRdChunk;
  const int64_t k = kc + lane * 32;
  const bool kv = k < K;
  // every row of the block's RG groups loaded first, their latency overlapping the staging (rows past N
  // re-read row N - 1; their sums are not stored)
  uint4 wr[RG][RPW];
  int sbr[RG][RPW];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int64_t n = min((((int64_t)blockIdx.x * RG + g) * 4 + wave) * RPW + r, N - 1);
      wr[g][r] = kv ? *reinterpret_cast<const uint4*>(P + mx_code_off(n, k / 2, ldp)) : make_uint4(0u, 0u, 0u, 0u);
      sbr[g][r] = kv ? (int)Ps[(k / 128) * ldps + n * 4 + ((k / 32) & 3)] : 127;
    }
  // the chunk's coefficients, staged once for the block's RG row groups: elements e .. e+3 of
  // example b go to s_c[b][(e % 32) / 4][e / 32], one float4
  for (int x = threadIdx.x; x < NB * (kRdChunk / 4); x += 256) {
    const int b = x / (kRdChunk / 4), e = (x % (kRdChunk / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < nb) {
      const float* src = coef + (int64_t)b * K + kc + e;
      if (kc + e + 4 <= K && ((uintptr_t)src & 15u) == 0) {
        v = *reinterpret_cast<const float4*>(src);
      } else {
        v.x = kc + e < K ? src[0] : 0.f;
        v.y = kc + e + 1 < K ? src[1] : 0.f;
        v.z = kc + e + 2 < K ? src[2] : 0.f;
        v.w = kc + e + 3 < K ? src[3] : 0.f;
      }
      if (mean) {                                       // per-token coefficients c_t = eps_t - mu_(t / S)
        const int64_t t = kc + e, q = t / S, r = t - q * S;  // one division; t + i crosses into q + 1 at most
        const float m0 = t < K ? mean[q] : 0.f;
        const float m1 = r + 3 >= S && t + (S - r) < K ? mean[q + 1] : m0;   // t + S - r: example q + 1's first
        if (t < K) v.x -= m0;
        if (t + 1 < K) v.y -= r + 1 < S ? m0 : m1;
        if (t + 2 < K) v.z -= r + 2 < S ? m0 : m1;
        if (t + 3 < K) v.w -= r + 3 < S ? m0 : m1;
      }
    }
    s_c[b][(e & 31) >> 2][e >> 5] = v;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int64_t n0 = (((int64_t)blockIdx.x * RG + g) * 4 + wave) * RPW;
    float acc[V];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint32_t wv[4] = {wr[g][r].x, wr[g][r].y, wr[g][r].z, wr[g][r].w};
      float a[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) a[b] = 0.f;
      // the hardware FP4 -> f32 conversion decodes one byte (two codes, the low nibble first) per
      // instruction, times 2: signed multiples of 0.5 become exact integers of halves
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        const v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv[wi], 2.f, 0);
        const v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv[wi], 2.f, 1);
        const v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv[wi], 2.f, 2);
        const v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv[wi], 2.f, 3);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float4 c0 = s_c[b][2 * wi][lane], c1 = s_c[b][2 * wi + 1][lane];
          a[b] = fmaf(c0.x, p0.x, a[b]);
          a[b] = fmaf(c0.y, p0.y, a[b]);
          a[b] = fmaf(c0.z, p1.x, a[b]);
          a[b] = fmaf(c0.w, p1.y, a[b]);
          a[b] = fmaf(c1.x, p2.x, a[b]);
          a[b] = fmaf(c1.y, p2.y, a[b]);
          a[b] = fmaf(c1.z, p3.x, a[b]);
          a[b] = fmaf(c1.w, p3.y, a[b]);
        }
      }
      const float half_scale = __builtin_ldexpf(1.f, sbr[g][r] - 128);
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r * NB + b] = a[b] * half_scale;
    }
    // reduce-scatter of the V sums over the lane bits 5 .. log2(64 / V), then the remaining low bits
    constexpr int kLow = 64 / V;                        // lanes that end up sharing one sum
#pragma unroll
    for (int o = V / 2; o >= 1; o >>= 1) {
      const int bit = o * kLow;
      const bool hi = lane & bit;
#pragma unroll
      for (int i = 0; i < o; ++i) {
        const float send = hi ? acc[i] : acc[i + o];
        acc[i] = (hi ? acc[i + o] : acc[i]) + __shfl_xor(send, bit, 64);
      }
    }
    float tot = acc[0];
#pragma unroll
    for (int o = 1; o < kLow; o <<= 1) tot += __shfl_xor(tot, o, 64);
    const int vi = lane / kLow, r = vi / NB, b = vi % NB;
    if (lane % kLow == 0 && b < nb && n0 + r < N) part[((int64_t)blockIdx.y * NB + b) * N + n0 + r] = tot;
  }
}

// The four-example product (nb <= 4) on the matrix cores.  Block (x, y) takes rows 4 G x .. 4 G x + 4 G - 1
// (G groups of four) and K chunk y, wave w the chunk's quarter w (512 elements), in which lane l = 4 j + i
// takes the 32-element block j.  The lane carries, as the A operand of v_mfma_f32_4x4x1f32, coefficient
// row i over its block (registers, read once for all groups) and, as the B operand, the decoded codes of
// row i of the current group over the same block.  The instruction forms, in each group of four lanes, the
// outer product D[4 j + c][r] = A(4 j + r) B(4 j + c), so after the block's 32 elements the lane's four
// accumulators hold the products of its row with the four coefficient rows, counted in halves; the
// block scale / 2 multiplies them.  Fixed order: the two interleaved accumulator chains (even and odd
// elements), a reduce-scatter over the 16 blocks of the wave, the four quarters of the chunk in wave
// order, and mx_sum_parts over the chunks.
typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kRdQuarter = kRdChunk / 4;

template <int G>
__global__ __launch_bounds__(256) void mx_rowdot4_mfma_kernel(const uint8_t* __restrict__ P, int64_t ldp,
                                                              const uint8_t* __restrict__ Ps, int64_t ldps,
                                                              int64_t N, int64_t K, int nb,
                                                              const float* __restrict__ coef,
                                                              float* __restrict__ part) {
  __shared__ float red[4][G * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 3;
  const int64_t k = (int64_t)blockIdx.y * kRdChunk + wave * kRdQuarter + (lane >> 2) * 32;
  const bool kv = k < K;
  float cf[32];
  {
    const float* src = coef + (int64_t)i * K + k;
    if (i < nb && k + 32 <= K && ((uintptr_t)src & 15u) == 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = reinterpret_cast<const float4*>(src)[q];
        cf[4 * q] = v.x; cf[4 * q + 1] = v.y; cf[4 * q + 2] = v.z; cf[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) cf[e] = i < nb && k + e < K ? src[e] : 0.f;
    }
  }
  // every group's codes loaded before any is used (rows past N re-read row N - 1; their sums are not stored)
  uint4 wr[G];
  int sbr[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t n = min(((int64_t)blockIdx.x * G + g) * 4 + i, N - 1);
    wr[g] = kv ? *reinterpret_cast<const uint4*>(P + mx_code_off(n, k / 2, ldp)) : make_uint4(0u, 0u, 0u, 0u);
    sbr[g] = kv ? (int)Ps[(k / 128) * ldps + n * 4 + ((k / 32) & 3)] : 127;
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t wv[4] = {wr[g].x, wr[g].y, wr[g].z, wr[g].w};
    v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      // byte s of word wi: elements 8 wi + 2 s (low nibble) and 8 wi + 2 s + 1, as exact halves
      const v2f p[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv[wi], 2.f, 0),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv[wi], 2.f, 1),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv[wi], 2.f, 2),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv[wi], 2.f, 3)};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[8 * wi + 2 * s], p[s].x, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(cf[8 * wi + 2 * s + 1], p[s].y, a1, 0, 0, 0);
      }
    }
    const float half_scale = __builtin_ldexpf(1.f, sbr[g] - 128);
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (a0[r] + a1[r]) * half_scale;
    // lane bit 5 splits the four sums in pairs, bit 4 within the pair (the lane keeps example lane >> 4),
    // then bits 3 and 2 finish the sum over the wave's 16 blocks
    {
      const bool hi = lane & 32;
      const float s0 = hi ? v[0] : v[2], s1 = hi ? v[1] : v[3];
      v[0] = (hi ? v[2] : v[0]) + __shfl_xor(s0, 32, 64);
      v[1] = (hi ? v[3] : v[1]) + __shfl_xor(s1, 32, 64);
    }
    {
      const bool hi = lane & 16;
      const float s0 = hi ? v[0] : v[1];
      v[0] = (hi ? v[1] : v[0]) + __shfl_xor(s0, 16, 64);
    }
    float t = v[0];
    t += __shfl_xor(t, 8, 64);
    t += __shfl_xor(t, 4, 64);
    if ((lane & 12) == 0) red[wave][g * 16 + (lane >> 4) * 4 + i] = t;
  }
  __syncthreads();
  if (threadIdx.x < G * 16) {
    const int x = threadIdx.x, g = x >> 4, r = (x >> 2) & 3, c = x & 3;
    const float s = red[0][x] + red[1][x] + red[2][x] + red[3][x];
    const int64_t n = ((int64_t)blockIdx.x * G + g) * 4 + c;
    if (r < nb && n < N) part[((int64_t)blockIdx.y * 4 + r) * N + n] = s;
  }
}

// dW correction terms of examples 8 .. B-1 (the GEMM epilogue applies examples 0 .. 7):
// dW[j][n] -= sum_b ebar_b[j] * xs_b[n].
__global__ __launch_bounds__(256) void mx_dw_rank_update_kernel(float* __restrict__ dW, int64_t ld, int64_t D,
                                                                int64_t N, int64_t B, const float* __restrict__ ebar,
                                                                const float* __restrict__ xs) {
  const int64_t j = blockIdx.y;
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int64_t b = 8; b < B; ++b) s = fmaf(ebar[b * D + j], xs[b * N + n], s);
  dW[j * ld + n] -= s;
}

// out[b][n] = sum over the chunks kc (in order) of part[kc][b][n], b < nb, NB slots per chunk.
__global__ void mx_sum_parts_kernel(int64_t N, int nb, int NB, int nkc, const float* __restrict__ part,
                                    float* __restrict__ out) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= (int64_t)nb * N) return;
  const int64_t b = x / N, n = x % N;
  float s = 0.f;
  for (int kc = 0; kc < nkc; ++kc) s += part[((int64_t)kc * NB + b) * N + n];
  out[x] = s;
}

}  // namespace

// ------------------------------------------------------------- launchers ----
namespace {

bool al(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct MxQuantWs { size_t rph, cph, rpt, cpt, total; };
MxQuantWs mx_quant_ws(int64_t T, int64_t D, bool ec) {
  MxQuantWs w{};
  size_t off = 0;
  if (ec) {
    const size_t n_ct = (size_t)((D + kFusedCols - 1) / kFusedCols);
    w.rph = off; off = align_up(off + (size_t)T * n_ct * 4, 256);
    w.cph = off; off = align_up(off + (size_t)(T / 64) * D * 4, 256);
    w.rpt = off; off = align_up(off + (size_t)T * n_ct * 4, 256);
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
  const int n_ct = (int)((a.D + kFusedCols - 1) / kFusedCols);
  const dim3 grid((unsigned)(a.T / kFusedRows), (unsigned)n_ct);
  float* np_ = nullptr;
  if (a.ec) {
    // EC requires S3R
    hipLaunchKernelGGL((mx_quant_fused_kernel<TIn, true, 2>), grid, dim3(256), 0, st, p, G, a.Qh, a.ld_qh, a.Qhs,
                       a.ld_qhs, a.Qt, a.ld_qt, a.Qts, a.ld_qts, rph, cph, rpt, cpt, a.flags);
    const int64_t B = a.T / a.S;
    const int64_t ncb = (B * a.D * 8 + 255) / 256, nrb = (a.T + 255) / 256;
    hipLaunchKernelGGL(mx_finalize_kernel, dim3((unsigned)(ncb + nrb)), dim3(256), 0, st, B, a.D, a.S, 64, n_ct,
                       (int)ncb, (const float*)cph, (const float*)nullptr, (const float*)rph, a.ec_col_h,
                       (float*)nullptr, a.ec_row_h, a.T);
    hipLaunchKernelGGL(mx_finalize_kernel, dim3((unsigned)(ncb + nrb)), dim3(256), 0, st, B, a.D, a.S, 32, n_ct,
                       (int)ncb, (const float*)cpt, (const float*)nullptr, (const float*)rpt, a.ec_col_t,
                       (float*)nullptr, a.ec_row_t, a.T);
    hipLaunchKernelGGL(mx_mean_kernel, dim3((unsigned)B), dim3(256), 0, st, a.S, (const float*)a.ec_row_h,
                       a.ec_mean_h);
    hipLaunchKernelGGL(mx_mean_kernel, dim3((unsigned)B), dim3(256), 0, st, a.S, (const float*)a.ec_row_t,
                       a.ec_mean_t);
  } else if (a.mode == 0) {
    hipLaunchKernelGGL((mx_quant_fused_kernel<TIn, false, 0>), grid, dim3(256), 0, st, p, G, a.Qh, a.ld_qh, a.Qhs,
                       a.ld_qhs, a.Qt, a.ld_qt, a.Qts, a.ld_qts, np_, np_, np_, np_, a.flags);
  } else if (a.mode == 1) {
    hipLaunchKernelGGL((mx_quant_fused_kernel<TIn, false, 1>), grid, dim3(256), 0, st, p, G, a.Qh, a.ld_qh, a.Qhs,
                       a.ld_qhs, a.Qt, a.ld_qt, a.Qts, a.ld_qts, np_, np_, np_, np_, a.flags);
  } else {
    hipLaunchKernelGGL((mx_quant_fused_kernel<TIn, false, 2>), grid, dim3(256), 0, st, p, G, a.Qh, a.ld_qh, a.Qhs,
                       a.ld_qhs, a.Qt, a.ld_qt, a.Qts, a.ld_qts, np_, np_, np_, np_, a.flags);
  }
  return hipGetLastError();
}

template <typename TIn>
hipError_t mx_operand_t(const MxOperandArgs& a, hipStream_t st) {
  MxQuant p{};
  p.R = a.R; p.C = a.C; p.S = a.S; p.ld = a.ld; p.mode = 0; p.D_index = a.C;
  float* vsp = (float*)(a.ws);
  const dim3 gt((unsigned)(a.R / 128), (unsigned)((a.C + 63) / 64));
  if (a.colsum) {
    hipLaunchKernelGGL((mx_operand_kernel<TIn, true>), gt, dim3(256), 0, st, p, (const TIn*)a.M, a.Mt, a.ld_t, a.Mts,
                       a.ld_ts, vsp, a.flags);
    const int64_t B = a.R / a.S;
    const int64_t ncb = (B * a.C * 8 + 255) / 256;
    hipLaunchKernelGGL(mx_finalize_kernel, dim3((unsigned)ncb), dim3(256), 0, st, B, a.C, a.S, 32, 1, (int)ncb,
                       (const float*)nullptr, (const float*)vsp, (const float*)nullptr, (float*)nullptr, a.colsum,
                       (float*)nullptr, (int64_t)0);
  } else {
    hipLaunchKernelGGL((mx_operand_kernel<TIn, false>), gt, dim3(256), 0, st, p, (const TIn*)a.M, a.Mt, a.ld_t,
                       a.Mts, a.ld_ts, (float*)nullptr, a.flags);
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
  MxGemm g{A, lda, As, ldas, B, ldb, Bs, ldbs, M, N, K, (int)((M + 255) / 256), (int)((N + 127) / 128)};
  return g;
}

}  // namespace

size_t mx_quant_workspace(int64_t T, int64_t D, int ec) { return mx_quant_ws(T, D, ec != 0).total; }
size_t mx_operand_workspace(int64_t R, int64_t C) { return align_up((size_t)(R / 32) * C * 4, 256); }
// Backward workspace: v [B x d_in] (dX) | u [d_in] (dW) | the correction products' chunk partials.
size_t mx_backward_workspace(int64_t T, int64_t D, int64_t d_in, int64_t B) {
  const int64_t parts = max(((D + kRdChunk - 1) / kRdChunk) * 4, (T + kRdChunk - 1) / kRdChunk);
  return align_up((size_t)B * d_in * 4, 256) + align_up((size_t)d_in * 4, 256) +
         align_up((size_t)parts * d_in * 4, 256);
}

namespace {
// coef [nb x K] (row stride K) against the rows of P [N x K] into out [nb x N], NB <= 4 or 1.
template <int NB>
void run_rowdot(const MxBwArgs& a, int64_t N, int64_t K, int nb, const float* coef, float* out, float* part,
                hipStream_t st, const float* mean = nullptr, int64_t S = 1) {
  const int nkc = (int)((K + kRdChunk - 1) / kRdChunk);
  float* dst = nkc == 1 ? out : part;
  if constexpr (NB == 4) {
    constexpr int G = 8;                               // 32 rows per block (16: same time)
    hipLaunchKernelGGL((mx_rowdot4_mfma_kernel<G>), dim3((unsigned)((N + 4 * G - 1) / (4 * G)), (unsigned)nkc),
                       dim3(256), 0, st, a.B, a.ldb, a.Bs, a.ldbs, N, K, nb, coef, dst);
  } else {
    constexpr int RPW = 4;                             // 16 rows per group, each wave's loads in flight together
    constexpr int RG = 1;                              // one group per block: 16 rows (4 or 2 groups: 16-20 % slower)
    hipLaunchKernelGGL((mx_rowdot_kernel<NB, RPW, RG>),
                       dim3((unsigned)((N + 4 * RPW * RG - 1) / (4 * RPW * RG)), (unsigned)nkc), dim3(256), 0, st,
                       a.B, a.ldb, a.Bs, a.ldbs, N, K, nb, coef, mean, S, dst);
  }
  if (nkc > 1)
    hipLaunchKernelGGL(mx_sum_parts_kernel, dim3((unsigned)((nb * N + 255) / 256)), dim3(256), 0, st, N, nb, NB, nkc,
                       (const float*)part, out);
}

float* mx_parts(const MxBwArgs& a) {
  const int64_t B = a.T / a.S;
  return (float*)(a.ws + align_up((size_t)B * a.d_in * 4, 256) + align_up((size_t)a.d_in * 4, 256));
}
}  // namespace

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
    float* v = (float*)(a.ws);
    // v_b[i] = sum_j ebar_b[j] dq(W)[j][i]: rows of the K-major Wt [d_in x D], four examples per pass
    for (int64_t b0 = 0; b0 < B; b0 += 4)
      run_rowdot<4>(a, a.d_in, a.K, (int)min((int64_t)4, B - b0), a.ec_col + b0 * a.K, v + b0 * a.d_in, mx_parts(a),
                    st);
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
    float* u = (float*)(a.ws + align_up((size_t)B * a.d_in * 4, 256));
    // u[i] = sum_t (eps_t - mu_b) dq(X)[t][i]: rows of the K-major Xt [d_in x T], the coefficients formed
    // as they are staged
    run_rowdot<1>(a, a.d_in, a.T, 1, a.ec_row, u, mx_parts(a), st, a.ec_mean, a.S);
    ep.ebar = a.ec_col; ep.xs = a.vcol; ep.u = u;
  }
  // dW [D x d_in] = Qt [D x T] . Xt [d_in x T]^T
  const MxGemm g = make_mx_gemm(a.A, a.lda, a.As, a.ldas, a.B, a.ldb, a.Bs, a.ldbs, a.D, a.d_in, a.T);
  if (!a.ec) run_mx_gemm<true, false, 1>(g, ep, st);
  else if (B <= 1) run_mx_gemm<true, true, 1>(g, ep, st);
  else if (B <= 2) run_mx_gemm<true, true, 2>(g, ep, st);
  else if (B <= 4) run_mx_gemm<true, true, 4>(g, ep, st);
  else run_mx_gemm<true, true, 8>(g, ep, st);
  if (a.ec && B > 8)
    hipLaunchKernelGGL(mx_dw_rank_update_kernel, dim3((unsigned)((a.d_in + 255) / 256), (unsigned)a.D), dim3(256), 0,
                       st, a.out, a.ld_out, a.D, a.d_in, B, a.ec_col, a.vcol);
  return hipGetLastError();
}

}  // namespace s3r
