// Fused INT8 quantizer of the upstream gradient for gfx950.
//
// S3R page, "Quantized Backpropagation with Stochastic Rounding": fold the
// forward scales into G (G' = diag(s_x) G diag(s_w)), take one step
// Delta = max|G'|/127 and write the S8 codes Q = SR(G'; R)/Delta once, for
// both GEMMs.  "Structured Subspace Randomness": S3R shares one threshold per
// token across the hidden dimension and never materialises R.  "Two-Way
// Correction": the quantizer knows the rounding error exactly and reduces it
// to the per-token and per-example per-channel means.
//
// Kernels (all HBM-bound for RTNE / S3R / S3R-EC):
//   amax_tensor  per-tensor max|G'| -> one partial per block       (pass 1)
//   amax_rows    per-token max|G'| -> step per row                  (pass 1)
//   quantize     codes + error sums, tile of 64 rows x 512 columns  (pass 2)
//   finalize_*   fixed-order sums of the per-tile partials          (tiny)
//
// Exactness: G' = fl(fl(G*s_x)*s_w), inv = fl(127/amax); the code of
// floor(x + r) with x = fl(G'*inv) is computed in integers on the 2^-24 grid:
// X = floor(fl(G'*inv*2^24)), q = (clamp(X) + r*2^24) >> 24.  Scaling by 2^24
// is exact except where G'*inv is subnormal, and there both forms give the
// same code.  The build disables FP contraction.
#include "s3r_internal.h"
#include "swiglu_math.h"

#include <algorithm>
#include <type_traits>

namespace s3r {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerTile = 64;             // rows of one quantize tile
constexpr int kColsPerTile = kWave * 8;      // 512 columns: 8 per lane
constexpr int kAmaxBlocks = 1024;

// Load 8 consecutive elements G[row][j0 .. j0+7] as fp32, zero past D.
template <typename TIn, bool VEC>
__device__ __forceinline__ void load8(const TIn* __restrict__ row, int64_t j0, int64_t D, float v[8]) {
  if (VEC && j0 + 8 <= D) {
    if constexpr (sizeof(TIn) == 2) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + j0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(row + j0);
      const float4 b = *reinterpret_cast<const float4*>(row + j0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = 0.f;
      if (j0 + i < D) {
        if constexpr (sizeof(TIn) == 2) x = bf16_to_f32(row[j0 + i]);
        else x = row[j0 + i];
      }
      v[i] = x;
    }
  }
}

__device__ __forceinline__ void load8_scale(const float* __restrict__ sw, int64_t j0, int64_t D,
                                            bool vec, float v[8]) {
  if (sw == nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 1.f;
  } else if (vec && j0 + 8 <= D) {
    const float4 a = *reinterpret_cast<const float4*>(sw + j0);
    const float4 b = *reinterpret_cast<const float4*>(sw + j0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (j0 + i < D) ? sw[j0 + i] : 1.f;
  }
}

template <bool VEC>
__device__ __forceinline__ void store8(int8_t* __restrict__ row, int64_t j0, int64_t D, const int q[8]) {
  if (VEC && j0 + 8 <= D) {
    uint2 p;
    p.x = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) | ((uint32_t)(q[2] & 0xFF) << 16) |
          ((uint32_t)q[3] << 24);
    p.y = (uint32_t)(q[4] & 0xFF) | ((uint32_t)(q[5] & 0xFF) << 8) | ((uint32_t)(q[6] & 0xFF) << 16) |
          ((uint32_t)q[7] << 24);
    *reinterpret_cast<uint2*>(row + j0) = p;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (j0 + i < D) row[j0 + i] = (int8_t)q[i];
  }
}

// |v| as ordered bits: for non-negative floats uint order == float order, and
// NaN (> 0x7F800000) wins every max, so a NaN anywhere reaches the step.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Step from amax bits: Delta = fl(a/127), inv = fl(127/a) (a == 0: 1 and 0).
struct Step { float delta, inv, inv24; uint32_t flag; };
__device__ __forceinline__ Step make_step(uint32_t abits) {
  const float a = __uint_as_float(abits);
  Step s;
  s.flag = 0;
  if (abits == 0) { s.delta = 1.f; s.inv = 0.f; s.inv24 = 0.f; return s; }
  s.delta = __fdiv_rn(a, 127.f);
  s.inv = __fdiv_rn(127.f, a);
  s.inv24 = s.inv * 16777216.f;
  if (!(abits < 0x7F800000u)) s.flag |= S3R_FLAG_NONFINITE;
  else if (!(__float_as_uint(s.inv24) < 0x7F800000u)) s.flag |= S3R_FLAG_TINY_STEP;
  return s;
}

// ---------------------------------------------------------------- pass 1 ----
// Up to kAmaxBlocks blocks (amax_blocks: at least kAmaxRows rows each), each a contiguous band of rows; a thread loads one
// 16-byte column chunk of kAmaxRows rows at a time, straight-line when the band
// and the chunk are full.
constexpr int kAmaxRows = 8;
// Blocks of the per-tensor amax pass: one per kAmaxRows rows, at most kAmaxBlocks (a small
// tensor gets few blocks, and each code-pass block then reduces few partials).
int amax_blocks(int64_t T) { return (int)std::max<int64_t>(1, std::min<int64_t>(kAmaxBlocks, (T + kAmaxRows - 1) / kAmaxRows)); }

template <typename TIn, bool VEC>
__global__ __launch_bounds__(kThreads) void amax_tensor_kernel(
    const TIn* __restrict__ G, int64_t ld, int64_t T, int64_t D,
    const float* __restrict__ sx, const float* __restrict__ sw, uint32_t* __restrict__ part) {
  const int64_t cpr = (D + 7) / 8;  // 8-element chunks per row
  const int64_t rpb = (T + gridDim.x - 1) / gridDim.x;   // rows per block
  const int64_t rb0 = (int64_t)blockIdx.x * rpb, rb1 = min(rb0 + rpb, T);
  // |fl(fl(g * s_x) * s_w)|, its bits compared as unsigned (NaN above every number)
  auto fold_bits = [](float g, float fx, float s) { return __float_as_uint((g * fx) * s) & 0x7FFFFFFFu; };
  uint32_t m = 0;
  for (int64_t t0 = rb0; t0 < rb1; t0 += kAmaxRows) {
    const bool rows_full = t0 + kAmaxRows <= rb1;
    float fx[kAmaxRows];
#pragma unroll
    for (int u = 0; u < kAmaxRows; ++u) fx[u] = (t0 + u < rb1 && sx) ? sx[t0 + u] : 1.f;
    int64_t c = threadIdx.x;
    if constexpr (sizeof(TIn) == 2 && VEC) {
      // full bands of bf16: two chunk columns per pass, their 16 rows' raw words all loaded
      // before any is decoded (4 registers per 8 elements keeps every block resident)
      if (rows_full) {
        for (; c + kThreads < cpr && (c + kThreads) * 8 + 8 <= D; c += 2 * kThreads) {
          uint4 raw[2][kAmaxRows];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int u = 0; u < kAmaxRows; ++u)
              raw[h][u] = ld_stream_u4(G + (t0 + u) * ld + (c + h * kThreads) * 8);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float s[8];
            load8_scale(sw, (c + h * kThreads) * 8, D, true, s);
#pragma unroll
            for (int u = 0; u < kAmaxRows; ++u) {
              const uint32_t w[4] = {raw[h][u].x, raw[h][u].y, raw[h][u].z, raw[h][u].w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t b0 = fold_bits(__uint_as_float(w[i] << 16), fx[u], s[2 * i]);
                const uint32_t b1 = fold_bits(__uint_as_float(w[i] & 0xFFFF0000u), fx[u], s[2 * i + 1]);
                m = max(m, max(b0, b1));
              }
            }
          }
        }
      }
    }
    // the rest (other dtypes, partial bands, ragged chunks): one chunk column at a time
    for (; c < cpr; c += kThreads) {
      float v[kAmaxRows][8];
      float s[8];
      load8_scale(sw, c * 8, D, VEC, s);
#pragma unroll
      for (int u = 0; u < kAmaxRows; ++u) {
        if (t0 + u < rb1) load8<TIn, VEC>(G + (t0 + u) * ld, c * 8, D, v[u]);
        else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[u][i] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kAmaxRows; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = max(m, fold_bits(v[u][i], fx[u], s[i]));
    }
  }
  __shared__ uint32_t red[kThreads / kWave];
  m = wave_max_u32(m);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int w = 1; w < kThreads / kWave; ++w) r = r > red[w] ? r : red[w];
    part[blockIdx.x] = r;
  }
}

// Per-token step: one wavefront per row.  Writes amax bits to `abits`, the step
// to delta[t] and OR-s flags.
template <typename TIn, bool VEC>
__global__ __launch_bounds__(kThreads) void amax_rows_kernel(
    const TIn* __restrict__ G, int64_t ld, int64_t T, int64_t D,
    const float* __restrict__ sx, const float* __restrict__ sw,
    uint32_t* __restrict__ abits, float* __restrict__ delta, uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const int64_t cpr = (D + 7) / 8;
  const TIn* row = G + t * ld;
  const float fx = sx ? sx[t] : 1.f;
  uint32_t m = 0;
  for (int64_t c = lane; c < cpr; c += kWave) {
    float v[8], s[8];
    load8<TIn, VEC>(row, c * 8, D, v);
    load8_scale(sw, c * 8, D, VEC, s);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = abs_bits((v[i] * fx) * s[i]);
      m = m > b ? m : b;
    }
  }
  m = wave_max_u32(m);
  if (lane == 0) {
    const Step s = make_step(m);
    abits[t] = m;
    delta[t] = (m > 0x7F800000u) ? __uint_as_float(m) : s.delta;
    if (s.flag && flags) atomicOr(flags, s.flag);
  }
}

// ---------------------------------------------------------------- pass 2 ----
struct QuantTile {
  int64_t T, D, S, ld_g, ld_q;
  int tiles_per_example, n_ctiles;
  uint32_t layer; uint64_t seed;
  uint32_t stream_word;   // 65536 * threshold stream, added to counter word 3
  int bcast;              // shared-threshold mode: one threshold per example (Phi_bcast), not per token
};

// MODE: 0 RTNE, 1 SR, 2 S3R.  EC: accumulate rounding errors.  PT: per-token step.
// Grouped problems: rows sorted by group, per-group steps and statistics (the
// group is the example), per-group column scales sw + e * D.
struct GroupArgs {
  const int64_t* offsets; const int32_t* tiles64; const uint32_t* amax; int64_t G;
};

// The SR thresholds of elements (t, j0 .. j0+7), r * 2^24, when D % 4 == 0: two Philox blocks.
__device__ __forceinline__ void sr_thresholds8(const QuantTile& p, int64_t t, int64_t j0, int32_t (&R)[8]) {
  const uint64_t blk = ((uint64_t)t * (uint64_t)p.D + (uint64_t)j0) >> 2;
  const U4 w0 = philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), p.layer, kTagSR + p.stream_word,
                              (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
  const U4 w1 = philox4x32_10((uint32_t)(blk + 1), (uint32_t)((blk + 1) >> 32), p.layer, kTagSR + p.stream_word,
                              (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
  R[0] = sr_units24(w0.x); R[1] = sr_units24(w0.y); R[2] = sr_units24(w0.z); R[3] = sr_units24(w0.w);
  R[4] = sr_units24(w1.x); R[5] = sr_units24(w1.y); R[6] = sr_units24(w1.z); R[7] = sr_units24(w1.w);
}

// Fast-path codes of 8 elements v of row t (columns j0 .. j0+7, all in range; SR needs D % 4 == 0), packed
// four to a word in pw.  rt: the row's S3R threshold (MODE 2; read only for a finite step).  With EC the rounding errors on the 2^24 grid
// are added to es (the row) and col (each column).
//   RTNE: clamp, then add 1.5 * 2^23, whose round-to-nearest-even sum holds rint(x) in its low byte.
//   SR / S3R: t = clamp(floor(x * 2^24)) + r * 2^24 holds floor(x + r) in its top byte, and t & 0xFF000000
//   is that code times 2^24; the error 2^24 (q - x) = fl(that - x * 2^24) is the rounding error on the
//   2^24 grid, one rounding (its sums are scaled back by 2^-24 exactly).
template <int MODE, bool EC>
__device__ __forceinline__ void code8_packed(const QuantTile& p, const Step& st, const int32_t* rt, int64_t t, int64_t j0,
                                             float fx, const float (&v)[8], const float (&sw8)[8],
                                             uint32_t (&pw)[2], float& es, float (&col)[8]) {
  if (st.flag) {
    pw[0] = pw[1] = 0u;
  } else if constexpr (MODE == 0) {
    uint32_t y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = ((v[i] * fx) * sw8[i]) * st.inv;
      y[i] = __float_as_uint(fminf(fmaxf(x, -127.f), 127.f) + 12582912.f);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)   // low bytes of y[4h..4h+3]
      pw[h] = __builtin_amdgcn_perm(y[4 * h + 1], y[4 * h], 0x0C0C0400u) |
              __builtin_amdgcn_perm(y[4 * h + 3], y[4 * h + 2], 0x04000C0Cu);
  } else {
    int32_t R[8];
    if constexpr (MODE == 2) {
      const int32_t r = *rt;
#pragma unroll
      for (int i = 0; i < 8; ++i) R[i] = r;
    } else {
      sr_thresholds8(p, t, j0, R);
    }
    uint32_t tv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x24 = ((v[i] * fx) * sw8[i]) * st.inv24;
      int32_t X;
      asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(X) : "v"(x24));   // floor; x24 is finite here
      X = min(max(X, -(127 << 24)), 127 << 24);
      tv[i] = (uint32_t)(X + R[i]);
      if constexpr (EC) {
        const float e24 = (float)(int32_t)(tv[i] & 0xFF000000u) - x24;
        es += e24;
        col[i] += e24;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)   // top bytes of tv[4h..4h+3]
      pw[h] = __builtin_amdgcn_perm(tv[4 * h + 1], tv[4 * h], 0x0C0C0703u) |
              __builtin_amdgcn_perm(tv[4 * h + 3], tv[4 * h + 2], 0x07030C0Cu);
  }
}

// Reduce-scatter of a wave's 16 row sums (rows k = 0..15 in rsum[k] of every lane): the result's lane l
// holds the sum over the wave of row k = l >> 2.  Every lane of the wave must call it.
__device__ __forceinline__ float row_sums16(const float (&rsum)[16], int lane) {
  float r8[8], r4[4], r2[2], r1s;
  const bool hi32 = lane & 32, hi16 = lane & 16, hi8 = lane & 8, hi4 = lane & 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float send = hi32 ? rsum[i] : rsum[i + 8];
    r8[i] = (hi32 ? rsum[i + 8] : rsum[i]) + __shfl_xor(send, 32, kWave);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float send = hi16 ? r8[i] : r8[i + 4];
    r4[i] = (hi16 ? r8[i + 4] : r8[i]) + __shfl_xor(send, 16, kWave);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = hi8 ? r4[i] : r4[i + 2];
    r2[i] = (hi8 ? r4[i + 2] : r4[i]) + __shfl_xor(send, 8, kWave);
  }
  {
    const float send = hi4 ? r2[0] : r2[1];
    r1s = (hi4 ? r2[1] : r2[0]) + __shfl_xor(send, 4, kWave);
  }
  r1s += __shfl_xor(r1s, 2, kWave);
  r1s += __shfl_xor(r1s, 1, kWave);
  return r1s;
}

// General-path codes q and errors e (q - x, in steps) of 8 elements v of row t, columns j0 .. j0+7 (values
// past D are zeros, coded but not stored).  rt: the row's S3R threshold (MODE 2; read only for a finite step).
template <int MODE>
__device__ __forceinline__ void code8(const QuantTile& p, const Step& s, const int32_t* rt, int64_t t, int64_t j0, float fx,
                                      const float* v, const float (&sw8)[8], int (&q)[8], float (&e)[8]) {
  if (s.flag) {
#pragma unroll
    for (int i = 0; i < 8; ++i) { q[i] = 0; e[i] = 0.f; }
  } else if constexpr (MODE == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = ((v[i] * fx) * sw8[i]) * s.inv;
      const float r = fminf(fmaxf(__builtin_rintf(x), -127.f), 127.f);
      q[i] = (int)r;
      e[i] = (float)q[i] - x;
    }
  } else {
    int32_t R[8];
    if constexpr (MODE == 2) {
      const int32_t r = *rt;
#pragma unroll
      for (int i = 0; i < 8; ++i) R[i] = r;
    } else {
      if ((p.D & 3) == 0) {
        sr_thresholds8(p, t, j0, R);   // elements e0 .. e0+7 with e0 % 4 == 0: exactly two Philox blocks
      } else {
        const uint64_t e0 = (uint64_t)t * (uint64_t)p.D + (uint64_t)j0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint64_t ei = e0 + i;
          const uint64_t blk = ei >> 2;
          const U4 w = philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), p.layer, kTagSR + p.stream_word,
                                     (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
          R[i] = sr_units24(u4_word(w, (uint32_t)ei & 3u));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x24 = ((v[i] * fx) * sw8[i]) * s.inv24;
      int32_t X = (int32_t)floorf(x24);
      X = min(max(X, -(127 << 24)), 127 << 24);
      q[i] = (X + R[i]) >> 24;
      e[i] = fmaf(x24, -0x1p-24f, (float)q[i]);
    }
  }
}

template <typename TIn, bool VEC, int MODE, bool EC, bool PT, bool COLSUM, bool GR = false>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    QuantTile p, const TIn* __restrict__ G, const float* __restrict__ sx, const float* __restrict__ sw,
    int8_t* __restrict__ Q, float* __restrict__ delta_out, uint32_t* __restrict__ flags,
    const uint32_t* __restrict__ amax_part, int n_amax_part, const uint32_t* __restrict__ amax_rows,
    float* __restrict__ row_part, float* __restrict__ col_part, int32_t* __restrict__ colq_part,
    uint32_t* __restrict__ fin_counter, GroupArgs gr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rtile = blockIdx.x;
  const int ctile = blockIdx.y;
  int64_t b, r0, r1;
  bool first_tile;               // this row tile writes its group's (or the tensor's) step
  if constexpr (GR) {
    const GroupHit h = find_group_wave(gr.tiles64, gr.offsets, gr.G, rtile);
    if (h.e < 0) return;         // past the last tile of the last group
    const int e = h.e;
    b = e;
    r0 = h.r0 + (int64_t)(rtile - h.t0) * kRowsPerTile;
    r1 = min(r0 + kRowsPerTile, h.r1);
    first_tile = rtile == h.t0;
    if (sw) sw += e * p.D;
    amax_part = gr.amax + e;
    n_amax_part = 1;
    delta_out += e;
  } else {
    b = rtile / p.tiles_per_example;
    r0 = b * p.S + (int64_t)(rtile % p.tiles_per_example) * kRowsPerTile;
    r1 = min(r0 + kRowsPerTile, (b + 1) * p.S);
    first_tile = rtile == 0;
  }
  const int64_t j0 = (int64_t)ctile * kColsPerTile + lane * 8;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *fin_counter = 0u;   // for the finalize kernel

  __shared__ int32_t s_thr[kRowsPerTile];
  __shared__ uint32_t s_red[kThreads / kWave];
  __shared__ float s_col[kThreads / kWave][kColsPerTile];
  __shared__ int32_t s_colq[COLSUM ? kThreads / kWave : 1][COLSUM ? kColsPerTile : 1];

  // per-tensor step from the pass-1 partials (every block reduces them itself)
  Step st{};
  if constexpr (!PT) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < n_amax_part; i += kThreads) m = m > amax_part[i] ? m : amax_part[i];
    m = wave_max_u32(m);
    if (lane == 0) s_red[wave] = m;
  }
  if constexpr (MODE == 2) {
    if (threadIdx.x < r1 - r0)
      s_thr[threadIdx.x] = row_threshold_units24(r0 + threadIdx.x, p.layer, p.seed, p.bcast, p.S, p.stream_word);
  }
  __syncthreads();
  if constexpr (!PT) {
    uint32_t m = s_red[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) m = m > s_red[w] ? m : s_red[w];
    st = make_step(m);
    if (first_tile && blockIdx.y == 0 && threadIdx.x == 0) {
      delta_out[0] = (m > 0x7F800000u) ? __uint_as_float(m) : st.delta;
      if (st.flag && flags) atomicOr(flags, st.flag);
    }
  }

  float sw8[8];
  load8_scale(sw, j0, p.D, VEC, sw8);
  float col[8];
  int colq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { col[i] = 0.f; colq[i] = 0; }

  // Fast path (contiguous bf16 G, a full 64-row tile, 8 columns in range, per-tensor step):
  // the 16 rows of this wave (t = r0 + wave + 4k) are loaded as raw bf16 in groups of 4, each
  // group's loads issued when the previous group's coding starts (one group ahead); the 16 row
  // sums of the errors are one reduce-scatter across the wave at the end.
  // The choice is per wave: both paths end in cross-lane sums of the row errors, which must see every
  // lane of the wave on the same path.
  bool done = false;
  if constexpr (sizeof(TIn) == 2 && VEC && !PT && !COLSUM) {
    constexpr int kWR = kRowsPerTile / (kThreads / kWave);   // 16 rows per wave
    const bool fast_lane = r1 - r0 == kRowsPerTile && j0 + 8 <= p.D && (MODE != 1 || (p.D & 3) == 0);
    if (__builtin_amdgcn_ballot_w64(!fast_lane) == 0) {
      done = true;
      constexpr int kGroup = 4;
      uint4 raw[kWR];
      float rsum[kWR];
      // the 16 rows' s_x, lane k holding row k's, read out per row with readlane: a per-row
      // load would wait on every load in flight, the rows' G included
      const float sx_rows = (sx && lane < kWR) ? sx[r0 + wave + 4 * lane] : 1.f;
#pragma unroll
      for (int kk = 0; kk < kGroup; ++kk)
        raw[kk] = ld_stream_u4(G + (r0 + wave + 4 * kk) * p.ld_g + j0);
#pragma unroll
      for (int k = 0; k < kWR; ++k) {
        if (k % kGroup == 0 && k + kGroup < kWR) {
          __builtin_amdgcn_sched_barrier(0);        // the next group's loads, in row order
#pragma unroll
          for (int kk = k + kGroup; kk < k + 2 * kGroup; ++kk)
            raw[kk] = ld_stream_u4(G + (r0 + wave + 4 * kk) * p.ld_g + j0);
          __builtin_amdgcn_sched_barrier(0);
        }
        const int64_t t = r0 + wave + 4 * k;
        const float fx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sx_rows), k));
        float v[8];
        const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(w[i] << 16);
          v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
        uint32_t pw[2];
        float es = 0.f;
        code8_packed<MODE, EC>(p, st, &s_thr[t - r0], t, j0, fx, v, sw8, pw, es, col);
        rsum[k] = es;
        *reinterpret_cast<uint2*>(Q + t * p.ld_q + j0) = make_uint2(pw[0], pw[1]);
      }
      if constexpr (EC) {
        const float r1s = row_sums16(rsum, lane);   // lane l: row l >> 2
        if ((lane & 3) == 0) row_part[(r0 + wave + 4 * (lane >> 2)) * p.n_ctiles + ctile] = r1s * 0x1p-24f;
#pragma unroll
        for (int i = 0; i < 8; ++i) col[i] *= 0x1p-24f;   // to the units the slow path sums in
      }
    }
  }

  // rows t = r0 + wave + 4u: kUnroll rows' loads are issued before any is used
  constexpr int kUnroll = 4;
  for (int64_t tb = r0 + wave; tb < r1 && !done; tb += (kThreads / kWave) * kUnroll) {
  float vb[kUnroll][8];
  if (VEC && tb + (kThreads / kWave) * (kUnroll - 1) < r1 && j0 + 8 <= p.D) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load8<TIn, true>(G + (tb + (int64_t)u * (kThreads / kWave)) * p.ld_g, j0, p.D, vb[u]);
  } else {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = tb + (int64_t)u * (kThreads / kWave);
      if (t < r1 && j0 < p.D) load8<TIn, VEC>(G + t * p.ld_g, j0, p.D, vb[u]);
      else {
#pragma unroll
        for (int i = 0; i < 8; ++i) vb[u][i] = 0.f;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t t = tb + (int64_t)u * (kThreads / kWave);
    if (t >= r1) break;
    Step s = st;
    if constexpr (PT) s = make_step(amax_rows[t]);
    const float fx = sx ? sx[t] : 1.f;
    const float* v = vb[u];
    int q[8];
    float e[8];
    code8<MODE>(p, s, &s_thr[t - r0], t, j0, fx, v, sw8, q, e);
    if (j0 < p.D) store8<VEC>(Q + t * p.ld_q, j0, p.D, q);
    if constexpr (EC) {
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ei = (j0 + i < p.D) ? e[i] : 0.f;
        rs += ei;
        col[i] += PT ? ei * s.delta : ei;
      }
      rs = wave_sum(rs);
      if (lane == 0) row_part[t * p.n_ctiles + ctile] = rs;
    }
    if constexpr (COLSUM) {
#pragma unroll
      for (int i = 0; i < 8; ++i) colq[i] += q[i];
    }
  }
  }

  if constexpr (EC || COLSUM) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (EC) s_col[wave][lane * 8 + i] = col[i];
      if constexpr (COLSUM) s_colq[wave][lane * 8 + i] = colq[i];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < kColsPerTile; c += kThreads) {
      const int64_t j = (int64_t)ctile * kColsPerTile + c;
      if (j >= p.D) continue;
      if constexpr (EC) {
        float a = s_col[0][c];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) a += s_col[w][c];
        col_part[(int64_t)rtile * p.D + j] = a;
      }
      if constexpr (COLSUM) {
        int32_t a = s_colq[0][c];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) a += s_colq[w][c];
        colq_part[(int64_t)rtile * p.D + j] = a;
      }
    }
  }
}

// ------------------------------------------- quantizer with the glue in it ----
// The gate and up projections' code pass with the SwiGLU glue computed in it: per element the glue's two
// bf16 results, from dH, A_gate and A_up, are coded at once for both projections, so G_gate and G_up are
// never written.  The steps come from a glue pass that found the two per-tensor maxima only (amax[0] gate,
// amax[1] up).  Same tiles, lane mapping, fast and general paths, code arithmetic and order of the error
// sums as quantize_kernel, so codes, steps and statistics are exactly those of the glue followed by the two
// quantizers.
struct GlueIn {
  const float* dH; int64_t ld_dh; const uint16_t* Ag; const uint16_t* Au; int64_t ld_a;
};
struct QuantOut {
  const float* sw; int8_t* Q; float* delta; float* row_part; float* col_part; uint32_t* fin_counter;
};

template <bool VEC, int MODE, bool EC>
__global__ __launch_bounds__(kThreads) void swiglu_quantize_kernel(QuantTile pg, QuantTile pu, GlueIn in,
                                                                   const float* __restrict__ sx, QuantOut og,
                                                                   QuantOut ou, const uint32_t* __restrict__ amax,
                                                                   uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rtile = blockIdx.x;
  const int ctile = blockIdx.y;
  const int64_t D = pg.D;
  const int64_t b = rtile / pg.tiles_per_example;
  const int64_t r0 = b * pg.S + (int64_t)(rtile % pg.tiles_per_example) * kRowsPerTile;
  const int64_t r1 = min(r0 + kRowsPerTile, (b + 1) * pg.S);
  const int64_t j0 = (int64_t)ctile * kColsPerTile + lane * 8;
  if (EC && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    *og.fin_counter = 0u;   // for the finalize kernels
    *ou.fin_counter = 0u;
  }
  __shared__ int32_t s_thr[2][kRowsPerTile];
  __shared__ float s_col[EC ? 2 : 1][kThreads / kWave][EC ? kColsPerTile : 1];

  const uint32_t mg = amax[0], mu = amax[1];
  const Step stg = make_step(mg), stu = make_step(mu);
  if (rtile == 0 && ctile == 0 && threadIdx.x == 0) {
    og.delta[0] = (mg > 0x7F800000u) ? __uint_as_float(mg) : stg.delta;
    ou.delta[0] = (mu > 0x7F800000u) ? __uint_as_float(mu) : stu.delta;
    if ((stg.flag | stu.flag) && flags) atomicOr(flags, stg.flag | stu.flag);
  }
  if constexpr (MODE == 2) {
    if (threadIdx.x < r1 - r0) {
      s_thr[0][threadIdx.x] = row_threshold_units24(r0 + threadIdx.x, pg.layer, pg.seed, pg.bcast, pg.S, pg.stream_word);
      s_thr[1][threadIdx.x] = row_threshold_units24(r0 + threadIdx.x, pu.layer, pu.seed, pu.bcast, pu.S, pu.stream_word);
    }
    __syncthreads();
  }

  float swg[8], swu[8];
  load8_scale(og.sw, j0, D, VEC, swg);
  load8_scale(ou.sw, j0, D, VEC, swu);
  float colg[8], colu[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { colg[i] = 0.f; colu[i] = 0.f; }

  // Fast path (a full 64-row tile, 8 columns in range, aligned rows), chosen per wave: the wave's 16 rows
  // t = r0 + wave + 4k in four groups of 4, each group's dH, A_gate and A_up loaded while the group before
  // it is coded.  The group loop is not unrolled (16 rows of glue would not fit); the 16 per-row error sums
  // shift down by a group per iteration, so they end in row order without indexing registers.
  bool done = false;
  if constexpr (VEC) {
    constexpr int kWR = kRowsPerTile / (kThreads / kWave);   // 16 rows per wave
    constexpr int kGroup = 4;
    const bool fast_lane = r1 - r0 == kRowsPerTile && j0 + 8 <= D && (MODE != 1 || (D & 3) == 0);
    if (__builtin_amdgcn_ballot_w64(!fast_lane) == 0) {
      done = true;
      struct Raw { float4 h0, h1; uint4 a, u; };
      Raw cur[kGroup], nxt[kGroup];
      float rsg[kWR], rsu[kWR];
#pragma unroll
      for (int k = 0; k < kWR; ++k) { rsg[k] = 0.f; rsu[k] = 0.f; }
      const float sx_rows = (sx && lane < kWR) ? sx[r0 + wave + 4 * lane] : 1.f;
      auto load_group = [&](Raw (&dst)[kGroup], int g) {
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          const int64_t t = r0 + wave + 4 * (g * kGroup + u);
          const float* dh = in.dH + t * in.ld_dh + j0;
          dst[u].h0 = ld_stream_f4(dh);
          dst[u].h1 = ld_stream_f4(dh + 4);
          dst[u].a = ld_stream_u4(in.Ag + t * in.ld_a + j0);
          dst[u].u = ld_stream_u4(in.Au + t * in.ld_a + j0);
        }
      };
      load_group(cur, 0);
#pragma unroll 1
      for (int g = 0; g < kWR / kGroup; ++g) {
        if (g + 1 < kWR / kGroup) {
          __builtin_amdgcn_sched_barrier(0);        // the next group's loads, in row order
          load_group(nxt, g + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        float ng[kGroup], nu[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          const int k = g * kGroup + u;
          const int64_t t = r0 + wave + 4 * k;
          const float fx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sx_rows), k));
          uint32_t gg[4], gu[4];
          glue8_vals(cur[u].h0, cur[u].h1, cur[u].a, cur[u].u, gg, gu);
          float vg[8], vu[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vg[2 * i] = __uint_as_float(gg[i] << 16);
            vg[2 * i + 1] = __uint_as_float(gg[i] & 0xFFFF0000u);
            vu[2 * i] = __uint_as_float(gu[i] << 16);
            vu[2 * i + 1] = __uint_as_float(gu[i] & 0xFFFF0000u);
          }
          uint32_t pwg[2], pwu[2];
          float esg = 0.f, esu = 0.f;
          code8_packed<MODE, EC>(pg, stg, &s_thr[0][t - r0], t, j0, fx, vg, swg, pwg, esg, colg);
          code8_packed<MODE, EC>(pu, stu, &s_thr[1][t - r0], t, j0, fx, vu, swu, pwu, esu, colu);
          ng[u] = esg;
          nu[u] = esu;
          *reinterpret_cast<uint2*>(og.Q + t * pg.ld_q + j0) = make_uint2(pwg[0], pwg[1]);
          *reinterpret_cast<uint2*>(ou.Q + t * pu.ld_q + j0) = make_uint2(pwu[0], pwu[1]);
        }
#pragma unroll
        for (int k = 0; k < kWR - kGroup; ++k) { rsg[k] = rsg[k + kGroup]; rsu[k] = rsu[k + kGroup]; }
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          rsg[kWR - kGroup + u] = ng[u];
          rsu[kWR - kGroup + u] = nu[u];
          cur[u] = nxt[u];
        }
      }
      if constexpr (EC) {
        const float sg = row_sums16(rsg, lane), su = row_sums16(rsu, lane);   // lane l: row l >> 2
        if ((lane & 3) == 0) {
          const int64_t t = r0 + wave + 4 * (lane >> 2);
          og.row_part[t * pg.n_ctiles + ctile] = sg * 0x1p-24f;
          ou.row_part[t * pu.n_ctiles + ctile] = su * 0x1p-24f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) { colg[i] *= 0x1p-24f; colu[i] *= 0x1p-24f; }
      }
    }
  }

  // General path: rows t = r0 + wave + 4u one at a time, elements past D coded as zeros and not stored.
  for (int64_t t = r0 + wave; t < r1 && !done; t += kThreads / kWave) {
    float vg[8], vu[8];
    if (VEC && j0 + 8 <= D) {
      uint32_t gg[4], gu[4];
      glue8(in.dH + t * in.ld_dh + j0, in.Ag + t * in.ld_a + j0, in.Au + t * in.ld_a + j0, gg, gu);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vg[2 * i] = __uint_as_float(gg[i] << 16);
        vg[2 * i + 1] = __uint_as_float(gg[i] & 0xFFFF0000u);
        vu[2 * i] = __uint_as_float(gu[i] << 16);
        vu[2 * i + 1] = __uint_as_float(gu[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vg[i] = 0.f;
        vu[i] = 0.f;
        if (j0 + i < D) {
          uint32_t g, u;
          glue1(in.dH[t * in.ld_dh + j0 + i], bf16_to_f32(in.Ag[t * in.ld_a + j0 + i]),
                bf16_to_f32(in.Au[t * in.ld_a + j0 + i]), g, u);
          vg[i] = __uint_as_float(g << 16);
          vu[i] = __uint_as_float(u << 16);
        }
      }
    }
    const float fx = sx ? sx[t] : 1.f;
    int qg[8], qu[8];
    float eg[8], eu[8];
    code8<MODE>(pg, stg, &s_thr[0][t - r0], t, j0, fx, vg, swg, qg, eg);
    code8<MODE>(pu, stu, &s_thr[1][t - r0], t, j0, fx, vu, swu, qu, eu);
    if (j0 < D) {
      store8<VEC>(og.Q + t * pg.ld_q, j0, D, qg);
      store8<VEC>(ou.Q + t * pu.ld_q, j0, D, qu);
    }
    if constexpr (EC) {
      float rg = 0.f, ru = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = (j0 + i < D) ? eg[i] : 0.f, c = (j0 + i < D) ? eu[i] : 0.f;
        rg += a;
        ru += c;
        colg[i] += a;
        colu[i] += c;
      }
      rg = wave_sum(rg);
      ru = wave_sum(ru);
      if (lane == 0) {
        og.row_part[t * pg.n_ctiles + ctile] = rg;
        ou.row_part[t * pu.n_ctiles + ctile] = ru;
      }
    }
  }

  if constexpr (EC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s_col[0][wave][lane * 8 + i] = colg[i];
      s_col[1][wave][lane * 8 + i] = colu[i];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < 2 * kColsPerTile; c += kThreads) {
      const int k = c / kColsPerTile, cc = c % kColsPerTile;
      const int64_t j = (int64_t)ctile * kColsPerTile + cc;
      if (j >= D) continue;
      float a = s_col[k][0][cc];
#pragma unroll
      for (int w = 1; w < kThreads / kWave; ++w) a += s_col[k][w][cc];
      (k ? ou.col_part : og.col_part)[(int64_t)rtile * D + j] = a;
    }
  }
}

// ------------------------------------------------------------- finalize ----
// One launch.  Blocks [0, ncb): per-example channel means and code column sums,
// fixed-order sums over the row tiles of each example.  Blocks [ncb, ncb+nrb):
// token means eps_t of up to 256 rows of one example, and that block's sum of
// eps; the last row block to finish (counter reset to 0 by the quantize kernel)
// adds the block sums of each example in order to get its grand mean mu_b.
constexpr int kFinRows = 256;
static_assert(kThreads / kWave == 4, "the finalize kernel's column blocks add four waves' sums");

// Sums of partials in a fixed order: the n values p[0], p[stride], ... added one after another (fp64 for the
// float partials), their loads issued eight at a time so that they are in flight together.
__device__ __forceinline__ double sum_in_order(const float* __restrict__ p, int64_t stride, int n) {
  double a = 0.0;
  int k = 0;
  for (; k + 8 <= n; k += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(k + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) a += (double)v[u];
  }
  for (; k < n; ++k) a += (double)p[(int64_t)k * stride];
  return a;
}
__device__ __forceinline__ int32_t sum_in_order(const int32_t* __restrict__ p, int64_t stride, int n) {
  int32_t a = 0;
  int k = 0;
  for (; k + 8 <= n; k += 8) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(k + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) a += v[u];
  }
  for (; k < n; ++k) a += p[(int64_t)k * stride];
  return a;
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(
    int64_t B, int64_t D, int64_t S, int tiles_per_example, int n_ctiles, int per_token, int ncb,
    int blocks_per_example, const float* __restrict__ delta, const float* __restrict__ col_part,
    const int32_t* __restrict__ colq_part, const float* __restrict__ row_part, float* __restrict__ ec_col,
    int32_t* __restrict__ code_colsum, float* __restrict__ ec_row, float* __restrict__ ec_mean,
    double* __restrict__ blk_sum, uint32_t* __restrict__ counter) {
  if ((int)blockIdx.x < ncb) {
    // A block takes 64 consecutive (example, column) items, one per lane, so a
    // wave's loads are contiguous; wave w adds the example's row tiles k = w mod 4
    // in order, and the four waves' sums are added in wave order.
    __shared__ double csum[kThreads / kWave][kWave];
    __shared__ int32_t qsum[kThreads / kWave][kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t idx = (int64_t)blockIdx.x * kWave + lane;
    const bool ok = idx < B * D;
    const int64_t b = ok ? idx / D : 0, j = ok ? idx % D : 0;
    double a = 0.0;
    int32_t aq = 0;
    if (ok) {
      constexpr int kStep = kThreads / kWave;
      const int n = wave < tiles_per_example ? (tiles_per_example - wave + kStep - 1) / kStep : 0;
      const int64_t at = (b * tiles_per_example + wave) * D + j;
      if (ec_col) a = sum_in_order(col_part + at, (int64_t)kStep * D, n);
      if (code_colsum) aq = sum_in_order(colq_part + at, (int64_t)kStep * D, n);
    }
    csum[wave][lane] = a;
    qsum[wave][lane] = aq;
    __syncthreads();
    if (!ok || wave != 0) return;
    a = ((csum[0][lane] + csum[1][lane]) + csum[2][lane]) + csum[3][lane];
    aq = qsum[0][lane] + qsum[1][lane] + qsum[2][lane] + qsum[3][lane];
    if (ec_col) {
      const double d = per_token ? 1.0 : (double)delta[0];
      ec_col[idx] = (float)(a * d / (double)S);
    }
    if (code_colsum) code_colsum[idx] = aq;
    return;
  }
  // row block rb covers rows [b*S + k*256, min(b*S + (k+1)*256, (b+1)*S)) of example b
  const int rb = (int)blockIdx.x - ncb;
  const int64_t b = rb / blocks_per_example;
  const int64_t r0 = b * S + (int64_t)(rb % blocks_per_example) * kFinRows;
  const int64_t r1 = min(r0 + kFinRows, (b + 1) * S);
  const int64_t t = r0 + threadIdx.x;
  double eps = 0.0;
  if (t < r1) {
    const double a = sum_in_order(row_part + t * n_ctiles, 1, n_ctiles);
    const double d = per_token ? (double)delta[t] : (double)delta[0];
    eps = D > 0 ? a * d / (double)D : 0.0;
    ec_row[t] = (float)eps;
  }
  __shared__ double red[kThreads];
  red[threadIdx.x] = eps;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  __shared__ bool last;
  if (threadIdx.x == 0) {
    blk_sum[rb] = red[0];
    __threadfence();
    const uint32_t done = atomicAdd(counter, 1u);
    last = done == (uint32_t)(B * blocks_per_example) - 1u;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int64_t bb = threadIdx.x; bb < B; bb += kThreads) {
    double a = 0.0;
    for (int k = 0; k < blocks_per_example; ++k) a += blk_sum[bb * blocks_per_example + k];
    ec_mean[bb] = (float)(a / (double)S);
  }
}

// --------------------------------------------------------- grouped path ----
// Pass 1 of a grouped per-tensor quantizer: one block per (64-row tile of a
// group, 512 columns), the tiling of the code pass; the block's max of |G'|
// (column scales of its group) goes to amax[e] with an integer atomic max
// (order-free, so the result is deterministic).
template <typename TIn, bool VEC>
__global__ __launch_bounds__(kThreads) void grouped_amax_kernel(
    const TIn* __restrict__ G, int64_t ld, int64_t D, const float* __restrict__ sx, const float* __restrict__ sw,
    GroupArgs gr, uint32_t* __restrict__ amax) {
  const GroupHit h = find_group_wave(gr.tiles64, gr.offsets, gr.G, blockIdx.x);
  if (h.e < 0) return;
  const int e = h.e;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t r0 = h.r0 + (int64_t)(blockIdx.x - h.t0) * kRowsPerTile;
  const int64_t r1 = min(r0 + kRowsPerTile, h.r1);
  const int64_t j0 = (int64_t)blockIdx.y * kColsPerTile + lane * 8;
  float s[8];
  load8_scale(sw ? sw + e * D : nullptr, j0, D, VEC, s);
  uint32_t m = 0;
  constexpr int kW = kThreads / kWave;
  // Lanes with eight whole columns: every row of the wave's share loaded at
  // once with no branch around a load, so the loads overlap instead of waiting
  // in turn.  Rows past the group re-read its last row, and the other lanes
  // read their row's first eight columns (D >= 8); both are masked.
  const bool full = VEC && j0 + 8 <= D;
  if (VEC && D >= 8) {
    constexpr int kRB = sizeof(TIn) == 2 ? kRowsPerTile / kW : kRowsPerTile / kW / 2;
    const TIn* __restrict__ col = G + (full ? j0 : 0);
#pragma unroll 1
    for (int64_t tb = r0 + wave; tb < r1; tb += kW * kRB) {
      uint4 w[kRB][sizeof(TIn) / 2];     // the raw rows: eight bf16 or eight f32 values each
      float fx[kRB];
#pragma unroll
      for (int u = 0; u < kRB; ++u) {
        const int64_t t = min(tb + (int64_t)u * kW, r1 - 1);
        const uint4* row = reinterpret_cast<const uint4*>(col + t * ld);
#pragma unroll
        for (int h = 0; h < (int)(sizeof(TIn) / 2); ++h) w[u][h] = row[h];
        fx[u] = sx ? sx[t] : 1.f;
      }
#pragma unroll
      for (int u = 0; u < kRB; ++u) {
        const bool ok = full && tb + (int64_t)u * kW < r1;
        float v[8];
        if constexpr (sizeof(TIn) == 2) {
          const uint32_t x[4] = {w[u][0].x, w[u][0].y, w[u][0].z, w[u][0].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(x[i] << 16);
            v[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
          }
        } else {
          const uint32_t x[8] = {w[u][0].x, w[u][0].y, w[u][0].z, w[u][0].w,
                                 w[u][1].x, w[u][1].y, w[u][1].z, w[u][1].w};
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(x[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t b = abs_bits((v[i] * fx[u]) * s[i]);
          m = (ok && b > m) ? b : m;
        }
      }
    }
  }
  if (!full && j0 < D) {                  // a ragged last column group, or unaligned rows
    constexpr int kU = 4;
    for (int64_t tb = r0 + wave; tb < r1; tb += kW * kU) {
      float v[kU][8];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t t = tb + (int64_t)u * kW;
        if (t < r1) load8<TIn, false>(G + t * ld, j0, D, v[u]);
        else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[u][i] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t t = tb + (int64_t)u * kW;
        const float fx = (t < r1 && sx) ? sx[t] : 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t b = abs_bits((v[u][i] * fx) * s[i]);
          m = m > b ? m : b;
        }
      }
    }
  }
  __shared__ uint32_t red[kThreads / kWave];
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int w = 1; w < kThreads / kWave; ++w) r = r > red[w] ? r : red[w];
    if (r) atomicMax(&amax[e], r);
  }
}

// The group of row t: offsets[e] <= t < offsets[e+1] (binary search; t < offsets[G]).
__device__ __forceinline__ int row_group(const int64_t* __restrict__ offsets, int64_t G, int64_t t) {
  int lo = 0, hi = (int)G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Blocks [0, ncb): per-group channel means and code column sums; kFinLanes
// lanes share an item, each adding every kFinLanes-th row tile of the group in
// order, then a fixed xor butterfly adds the lanes (a long group's sum is not
// one serial chain).  Blocks past ncb: token means eps_t (EC).
constexpr int kFinLanes = 16;

__global__ __launch_bounds__(kThreads) void grouped_finalize_kernel(
    int64_t D, int64_t R, int n_ctiles, int per_token, int ncb, GroupArgs gr, const float* __restrict__ delta,
    const float* __restrict__ col_part, const int32_t* __restrict__ colq_part, const float* __restrict__ row_part,
    float* __restrict__ ec_col, int32_t* __restrict__ code_colsum, float* __restrict__ ec_row) {
  if ((int)blockIdx.x < ncb) {
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t idx = g / kFinLanes;
    const int sub = (int)(g % kFinLanes);
    const bool ok = idx < gr.G * D;            // the item count is uniform over a lane group
    const int64_t e = ok ? idx / D : 0, j = ok ? idx - e * D : 0;
    const int k0 = ok ? gr.tiles64[e] : 0, k1 = ok ? gr.tiles64[e + 1] : 0;
    double a = 0.0;
    int32_t aq = 0;
    const int cnt = k0 + sub < k1 ? (k1 - k0 - sub + kFinLanes - 1) / kFinLanes : 0;
    if (ec_col) a = sum_in_order(col_part + (int64_t)(k0 + sub) * D + j, (int64_t)kFinLanes * D, cnt);
    if (code_colsum) aq = sum_in_order(colq_part + (int64_t)(k0 + sub) * D + j, (int64_t)kFinLanes * D, cnt);
    for (int o = 1; o < kFinLanes; o <<= 1) {
      a += __shfl_xor(a, o, kWave);
      aq += __shfl_xor(aq, o, kWave);
    }
    if (!ok || sub != 0) return;
    const int64_t n = gr.offsets[e + 1] - gr.offsets[e];
    if (ec_col) {
      const double d = per_token ? 1.0 : (double)delta[e];
      ec_col[idx] = n > 0 ? (float)(a * d / (double)n) : 0.f;
    }
    if (code_colsum) code_colsum[idx] = aq;
    return;
  }
  const int64_t t = (int64_t)(blockIdx.x - ncb) * kThreads + threadIdx.x;
  if (t >= R) return;
  const int e = row_group(gr.offsets, gr.G, t);
  const double a = sum_in_order(row_part + t * n_ctiles, 1, n_ctiles);
  const double d = per_token ? (double)delta[t] : (double)delta[e];
  ec_row[t] = D > 0 ? (float)(a * d / (double)D) : 0.f;
}

// ec_mean[e]: mean of the group's token means, one block per group, in fp64, in a fixed order (each thread's
// rows in four interleaved partial sums, so a thread's loads are in flight together, then a tree over the
// block); 1024 threads, since the largest groups' rows are the kernel's time.  Nothing is read when the
// offsets were found invalid.
constexpr int kMeanThreads = 1024;
__global__ __launch_bounds__(kMeanThreads) void grouped_mean_kernel(const int64_t* __restrict__ offsets,
                                                                    const uint32_t* __restrict__ status,
                                                                    const float* __restrict__ ec_row,
                                                                    float* __restrict__ ec_mean) {
  const int64_t e = blockIdx.x;
  const bool ok = status[0] == 0;
  const int64_t a = ok ? offsets[e] : 0, b = ok ? offsets[e + 1] : 0;
  double p[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t t = a + threadIdx.x;
  for (; t + 3 * kMeanThreads < b; t += 4 * kMeanThreads) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ec_row[t + u * kMeanThreads];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] += (double)v[u];
  }
  for (int u = 0; t < b; t += kMeanThreads, ++u) p[u & 3] += (double)ec_row[t];
  __shared__ double red[kMeanThreads];
  red[threadIdx.x] = (p[0] + p[1]) + (p[2] + p[3]);
  __syncthreads();
  for (int o = kMeanThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) ec_mean[e] = b > a ? (float)(red[0] / (double)(b - a)) : 0.f;
}

// Degenerate shapes (T == 0 or D == 0): steps of 1, zero statistics.
__global__ void empty_kernel(int64_t T, int64_t D, int64_t B, int per_token, float* delta,
                             float* ec_row, float* ec_col, float* ec_mean, int32_t* code_colsum) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nd = per_token ? T : 1;
  if (i < nd) delta[i] = 1.f;
  if (ec_row && i < T) ec_row[i] = 0.f;
  if (ec_mean && i < B) ec_mean[i] = 0.f;
  if (ec_col && i < B * D) ec_col[i] = 0.f;
  if (code_colsum && i < B * D) code_colsum[i] = 0;
}

struct WsLayout {
  size_t amax_part, amax_rows, row_part, col_part, colq_part, blk_sum, counter, total;
};

WsLayout ws_layout(int64_t T, int64_t D, int64_t S, int ec, int scale, bool colsum) {
  WsLayout w{};
  const int64_t B = S > 0 ? T / S : 0;
  const int64_t tpe = (S + kRowsPerTile - 1) / kRowsPerTile;
  const int64_t n_rt = B * tpe;
  const int64_t n_ct = (D + kColsPerTile - 1) / kColsPerTile;
  size_t off = 0;
  w.amax_part = off; off = align_up(off + (scale == S3R_PER_TENSOR ? kAmaxBlocks * 4 : 0), 256);
  w.amax_rows = off; off = align_up(off + (scale == S3R_PER_TOKEN ? (size_t)T * 4 : 0), 256);
  w.row_part = off;  off = align_up(off + (ec ? (size_t)T * n_ct * 4 : 0), 256);
  w.col_part = off;  off = align_up(off + (ec ? (size_t)n_rt * D * 4 : 0), 256);
  w.colq_part = off; off = align_up(off + (colsum ? (size_t)n_rt * D * 4 : 0), 256);
  const int64_t bpe = (S + kFinRows - 1) / kFinRows;
  w.blk_sum = off;   off = align_up(off + (ec ? (size_t)B * bpe * 8 : 0), 256);
  w.counter = off;   off = align_up(off + 4, 256);
  w.total = off;
  return w;
}

template <typename TIn, bool VEC, int MODE, bool EC, bool PT, bool COLSUM>
void launch_q(const QuantArgs& a, const WsLayout& L, const QuantTile& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((quantize_kernel<TIn, VEC, MODE, EC, PT, COLSUM>), grid, dim3(kThreads), 0, st, p,
                     (const TIn*)a.G, a.sx, a.sw, a.Q, a.delta, a.flags,
                     a.amax_in ? a.amax_in : (const uint32_t*)(a.ws + L.amax_part), a.amax_in ? 1 : amax_blocks(a.T),
                     (const uint32_t*)(a.ws + L.amax_rows),
                     (float*)(a.ws + L.row_part), (float*)(a.ws + L.col_part), (int32_t*)(a.ws + L.colq_part),
                     (uint32_t*)(a.ws + L.counter), GroupArgs{});
}

template <typename TIn, bool VEC, int MODE, bool EC>
void dispatch_pt(const QuantArgs& a, const WsLayout& L, const QuantTile& p, dim3 grid, hipStream_t st) {
  const bool cs = a.code_colsum != nullptr;
  if (a.scale == S3R_PER_TOKEN) {
    if (cs) launch_q<TIn, VEC, MODE, EC, true, true>(a, L, p, grid, st);
    else launch_q<TIn, VEC, MODE, EC, true, false>(a, L, p, grid, st);
  } else {
    if (cs) launch_q<TIn, VEC, MODE, EC, false, true>(a, L, p, grid, st);
    else launch_q<TIn, VEC, MODE, EC, false, false>(a, L, p, grid, st);
  }
}

template <typename TIn, bool VEC>
void dispatch_mode(const QuantArgs& a, const WsLayout& L, const QuantTile& p, dim3 grid, hipStream_t st) {
  switch (a.mode) {
    case S3R_RTNE: dispatch_pt<TIn, VEC, 0, false>(a, L, p, grid, st); break;
    case S3R_SR: dispatch_pt<TIn, VEC, 1, false>(a, L, p, grid, st); break;
    default:
      if (a.ec) dispatch_pt<TIn, VEC, 2, true>(a, L, p, grid, st);
      else dispatch_pt<TIn, VEC, 2, false>(a, L, p, grid, st);
  }
}

template <typename TIn, bool VEC>
void run_quantize(const QuantArgs& a, const WsLayout& L, hipStream_t st) {
  const TIn* G = (const TIn*)a.G;
  if (a.scale == S3R_PER_TENSOR) {
    if (!a.amax_in)   // otherwise the step comes from the caller's amax: G is read once
      hipLaunchKernelGGL((amax_tensor_kernel<TIn, VEC>), dim3(amax_blocks(a.T)), dim3(kThreads), 0, st, G, a.ld_g,
                         a.T, a.D, a.sx, a.sw, (uint32_t*)(a.ws + L.amax_part));
  } else {
    const unsigned nb = (unsigned)((a.T + kThreads / kWave - 1) / (kThreads / kWave));
    hipLaunchKernelGGL((amax_rows_kernel<TIn, VEC>), dim3(nb), dim3(kThreads), 0, st, G, a.ld_g, a.T, a.D,
                       a.sx, a.sw, (uint32_t*)(a.ws + L.amax_rows), a.delta, a.flags);
  }
  QuantTile p;
  p.T = a.T; p.D = a.D; p.S = a.S; p.ld_g = a.ld_g; p.ld_q = a.ld_q;
  p.tiles_per_example = (int)((a.S + kRowsPerTile - 1) / kRowsPerTile);
  p.n_ctiles = (int)((a.D + kColsPerTile - 1) / kColsPerTile);
  p.layer = a.layer; p.seed = a.seed;
  p.stream_word = a.stream << 16;
  p.bcast = a.mode == S3R_S3R_BCAST;
  const int64_t B = a.T / a.S;
  dim3 grid((unsigned)(B * p.tiles_per_example), (unsigned)p.n_ctiles);
  dispatch_mode<TIn, VEC>(a, L, p, grid, st);
  if (a.ec || a.code_colsum) {
    const int64_t ncb = (B * a.D + kWave - 1) / kWave;
    const int bpe = (int)((a.S + kFinRows - 1) / kFinRows);
    const int64_t nrb = a.ec ? B * bpe : 0;
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)(ncb + nrb)), dim3(kThreads), 0, st, B, a.D, a.S,
                       p.tiles_per_example, p.n_ctiles, a.scale == S3R_PER_TOKEN ? 1 : 0, (int)ncb, bpe, a.delta,
                       (const float*)(a.ws + L.col_part), (const int32_t*)(a.ws + L.colq_part),
                       (const float*)(a.ws + L.row_part), a.ec ? a.ec_col : nullptr, a.code_colsum, a.ec_row,
                       a.ec_mean, (double*)(a.ws + L.blk_sum), (uint32_t*)(a.ws + L.counter));
  }
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct GroupedWs { size_t tables, counter, amax_rows, row_part, col_part, colq_part, total; };

GroupedWs grouped_ws(int64_t R, int64_t D, int64_t Gn, int ec, int scale, bool colsum) {
  GroupedWs w{};
  const int64_t n_rt = R / kRowsPerTile + Gn;                 // bound on the groups' 64-row tiles
  const int64_t n_ct = (D + kColsPerTile - 1) / kColsPerTile;
  size_t off = 0;
  w.tables = off;    off = align_up(off + group_tables_bytes(Gn), 256);
  w.counter = off;   off = align_up(off + 4, 256);
  w.amax_rows = off; off = align_up(off + (scale == S3R_PER_TOKEN ? (size_t)R * 4 : 0), 256);
  w.row_part = off;  off = align_up(off + (ec ? (size_t)R * n_ct * 4 : 0), 256);
  w.col_part = off;  off = align_up(off + (ec ? (size_t)n_rt * D * 4 : 0), 256);
  w.colq_part = off; off = align_up(off + (colsum ? (size_t)n_rt * D * 4 : 0), 256);
  w.total = off;
  return w;
}

template <typename TIn, bool VEC, int MODE, bool EC, bool PT, bool COLSUM>
void launch_gq(const QuantArgs& a, const GroupedWs& L, const QuantTile& p, const GroupArgs& gr, dim3 grid,
               hipStream_t st) {
  hipLaunchKernelGGL((quantize_kernel<TIn, VEC, MODE, EC, PT, COLSUM, true>), grid, dim3(kThreads), 0, st, p,
                     (const TIn*)a.G, a.sx, a.sw, a.Q, a.delta, a.flags, gr.amax, 1,
                     (const uint32_t*)(a.ws + L.amax_rows), (float*)(a.ws + L.row_part), (float*)(a.ws + L.col_part),
                     (int32_t*)(a.ws + L.colq_part), (uint32_t*)(a.ws + L.counter), gr);
}

template <typename TIn, bool VEC>
void run_grouped(const QuantArgs& a, const GroupedWs& L, const GroupArgs& gr, const uint32_t* status,
                 hipStream_t st) {
  const TIn* G = (const TIn*)a.G;
  const int64_t n_rt = a.T / kRowsPerTile + gr.G;
  if (a.scale == S3R_PER_TENSOR) {
    hipLaunchKernelGGL((grouped_amax_kernel<TIn, VEC>),
                       dim3((unsigned)n_rt, (unsigned)((a.D + kColsPerTile - 1) / kColsPerTile)), dim3(kThreads), 0,
                       st, G, a.ld_g, a.D, a.sx, a.sw, gr, (uint32_t*)gr.amax);
  } else {
    const unsigned nb = (unsigned)((a.T + kThreads / kWave - 1) / (kThreads / kWave));
    hipLaunchKernelGGL((amax_rows_kernel<TIn, VEC>), dim3(nb), dim3(kThreads), 0, st, G, a.ld_g, a.T, a.D,
                       a.sx, a.sw, (uint32_t*)(a.ws + L.amax_rows), a.delta, a.flags);
  }
  QuantTile p{};
  p.T = a.T; p.D = a.D; p.S = 1; p.ld_g = a.ld_g; p.ld_q = a.ld_q;
  p.tiles_per_example = 1;
  p.n_ctiles = (int)((a.D + kColsPerTile - 1) / kColsPerTile);
  p.layer = a.layer; p.seed = a.seed;
  p.stream_word = a.stream << 16;
  p.bcast = 0;
  dim3 grid((unsigned)n_rt, (unsigned)p.n_ctiles);
  const bool cs = a.code_colsum != nullptr;
  const bool pt = a.scale == S3R_PER_TOKEN;
  switch (a.mode) {
    case S3R_RTNE:
      if (pt) { if (cs) launch_gq<TIn, VEC, 0, false, true, true>(a, L, p, gr, grid, st);
                else launch_gq<TIn, VEC, 0, false, true, false>(a, L, p, gr, grid, st); }
      else launch_gq<TIn, VEC, 0, false, false, false>(a, L, p, gr, grid, st);
      break;
    case S3R_SR: launch_gq<TIn, VEC, 1, false, false, false>(a, L, p, gr, grid, st); break;
    default:
      if (a.ec) launch_gq<TIn, VEC, 2, true, false, false>(a, L, p, gr, grid, st);
      else launch_gq<TIn, VEC, 2, false, false, false>(a, L, p, gr, grid, st);
  }
  if (a.ec || cs) {
    const int64_t ncb = (gr.G * a.D * kFinLanes + kThreads - 1) / kThreads;
    const int64_t nrb = a.ec ? (a.T + kThreads - 1) / kThreads : 0;
    hipLaunchKernelGGL(grouped_finalize_kernel, dim3((unsigned)(ncb + nrb)), dim3(kThreads), 0, st, a.D, a.T,
                       p.n_ctiles, pt ? 1 : 0, (int)ncb, gr, a.delta, (const float*)(a.ws + L.col_part),
                       (const int32_t*)(a.ws + L.colq_part), (const float*)(a.ws + L.row_part),
                       a.ec ? a.ec_col : nullptr, a.code_colsum, a.ec_row);
    if (a.ec)
      hipLaunchKernelGGL(grouped_mean_kernel, dim3((unsigned)gr.G), dim3(kMeanThreads), 0, st, gr.offsets, status,
                         a.ec_row, a.ec_mean);
  }
}

}  // namespace

size_t grouped_quant_workspace(int64_t R, int64_t D, int64_t Gn, int ec, int scale, bool colsum) {
  return grouped_ws(R, D, Gn, ec, scale, colsum).total;
}

// Grouped quantizer: per-group per-tensor steps (or per-token steps), the
// group as the correction's example, per-group column scales.  Supported:
// RTNE / SR / S3R per tensor, S3R-EC, and RTNE per token with code column sums
// (the forward operands' prep).
hipError_t launch_grouped_quantize(const QuantArgs& a, int64_t Gn, const int64_t* offsets, hipStream_t st) {
  const GroupedWs L = grouped_ws(a.T, a.D, Gn, a.ec, a.scale, a.code_colsum != nullptr);
  const GroupTables tab = group_tables(a.ws + L.tables, Gn, offsets);
  hipError_t e = launch_group_tables(tab, a.T, a.flags, st, a.scale == S3R_PER_TENSOR ? a.delta : nullptr);
  if (e != hipSuccess) return e;
  GroupArgs gr{offsets, tab.tiles64, tab.amax, Gn};
  if (a.D == 0) return hipSuccess;
  const size_t es = a.g_dtype == S3R_BF16 ? 2 : 4;
  const bool vec = aligned(a.G, 16) && (a.ld_g * (int64_t)es) % 16 == 0 && aligned(a.Q, 8) && a.ld_q % 8 == 0 &&
                   (a.sw == nullptr || (aligned(a.sw, 16) && a.D % 4 == 0));
  if (a.g_dtype == S3R_BF16) {
    if (vec) run_grouped<uint16_t, true>(a, L, gr, tab.status, st);
    else run_grouped<uint16_t, false>(a, L, gr, tab.status, st);
  } else {
    if (vec) run_grouped<float, true>(a, L, gr, tab.status, st);
    else run_grouped<float, false>(a, L, gr, tab.status, st);
  }
  return hipGetLastError();
}

size_t quant_workspace(int64_t T, int64_t D, int64_t S, int ec, int scale, bool colsum) {
  return ws_layout(T, D, S, ec, scale, colsum).total;
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st) {
  const WsLayout L = ws_layout(a.T, a.D, a.S, a.ec, a.scale, a.code_colsum != nullptr);
  if (a.T == 0 || a.D == 0) {
    const int64_t B = a.S > 0 ? a.T / a.S : 0;
    int64_t n = a.T > 1 ? a.T : 1;
    if (B * a.D > n) n = B * a.D;
    hipLaunchKernelGGL(empty_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, a.T,
                       a.D, B, a.scale == S3R_PER_TOKEN ? 1 : 0, a.delta, a.ec_row, a.ec_col, a.ec_mean,
                       a.code_colsum);
    return hipGetLastError();
  }
  const size_t es = a.g_dtype == S3R_BF16 ? 2 : 4;
  const bool vec = aligned(a.G, 16) && (a.ld_g * (int64_t)es) % 16 == 0 && aligned(a.Q, 8) && a.ld_q % 8 == 0 &&
                   (a.sw == nullptr || aligned(a.sw, 16));
  if (a.g_dtype == S3R_BF16) {
    if (vec) run_quantize<uint16_t, true>(a, L, st);
    else run_quantize<uint16_t, false>(a, L, st);
  } else {
    if (vec) run_quantize<float, true>(a, L, st);
    else run_quantize<float, false>(a, L, st);
  }
  return hipGetLastError();
}

size_t swiglu_quant_workspace(int64_t T, int64_t D, int64_t S, int ec) {
  const size_t per = ws_layout(T, D, S, ec, S3R_PER_TENSOR, false).total;
  return align_up(swiglu_amax_workspace(T, D), 256) + 256 + 2 * per;
}

namespace {
template <bool VEC, int MODE, bool EC>
void launch_sq(const SwigluQuantArgs& a, const QuantTile (&p)[2], const QuantOut (&o)[2], const uint32_t* amax,
               dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((swiglu_quantize_kernel<VEC, MODE, EC>), grid, dim3(kThreads), 0, st, p[0], p[1],
                     GlueIn{a.dH, a.ld_dh, a.Ag, a.Au, a.ld_a}, a.sx, o[0], o[1], amax, a.flags);
}

template <bool VEC>
void dispatch_sq(const SwigluQuantArgs& a, const QuantTile (&p)[2], const QuantOut (&o)[2], const uint32_t* amax,
                 dim3 grid, hipStream_t st) {
  switch (a.mode) {
    case S3R_RTNE: launch_sq<VEC, 0, false>(a, p, o, amax, grid, st); break;
    case S3R_SR: launch_sq<VEC, 1, false>(a, p, o, amax, grid, st); break;
    default:
      if (a.ec) launch_sq<VEC, 2, true>(a, p, o, amax, grid, st);
      else launch_sq<VEC, 2, false>(a, p, o, amax, grid, st);
  }
}
}  // namespace

// Workspace: the glue pass's per-block maxima, the two amax words, then one quantizer layout per projection.
hipError_t launch_swiglu_quantize(const SwigluQuantArgs& a, hipStream_t st) {
  const WsLayout L = ws_layout(a.T, a.D, a.S, a.ec, S3R_PER_TENSOR, false);
  const int64_t B = a.S > 0 ? a.T / a.S : 0;
  if (a.T == 0 || a.D == 0) {
    const int64_t n = std::max<int64_t>({1, a.T, B * a.D});
    for (int k = 0; k < 2; ++k)
      hipLaunchKernelGGL(empty_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, a.T,
                         a.D, B, 0, a.delta[k], a.ec_row[k], a.ec_col[k], a.ec_mean[k], (int32_t*)nullptr);
    return hipGetLastError();
  }
  uint32_t* amax = (uint32_t*)(a.ws + align_up(swiglu_amax_workspace(a.T, a.D), 256));
  char* wk[2] = {(char*)amax + 256, (char*)amax + 256 + L.total};
  hipError_t e = launch_swiglu_backward_amax(a.T, a.D, a.dH, a.ld_dh, a.Ag, a.Au, a.ld_a, nullptr, nullptr, 0, a.sx,
                                             a.sw[0], a.sw[1], amax, a.ws, st);
  if (e != hipSuccess) return e;
  QuantTile p[2];
  QuantOut o[2];
  bool vec = aligned(a.dH, 16) && aligned(a.Ag, 16) && aligned(a.Au, 16) && a.ld_dh % 4 == 0 && a.ld_a % 8 == 0 &&
             a.ld_q % 8 == 0;
  for (int k = 0; k < 2; ++k) {
    p[k] = QuantTile{};
    p[k].T = a.T; p[k].D = a.D; p[k].S = a.S; p[k].ld_g = 0; p[k].ld_q = a.ld_q;
    p[k].tiles_per_example = (int)((a.S + kRowsPerTile - 1) / kRowsPerTile);
    p[k].n_ctiles = (int)((a.D + kColsPerTile - 1) / kColsPerTile);
    p[k].layer = a.layer[k]; p[k].seed = a.seed[k];
    p[k].stream_word = a.stream[k] << 16;
    p[k].bcast = a.mode == S3R_S3R_BCAST;
    o[k] = QuantOut{a.sw[k], a.Q[k], a.delta[k], (float*)(wk[k] + L.row_part), (float*)(wk[k] + L.col_part),
                    (uint32_t*)(wk[k] + L.counter)};
    vec = vec && aligned(a.Q[k], 8) && (a.sw[k] == nullptr || aligned(a.sw[k], 16));
  }
  const dim3 grid((unsigned)(B * p[0].tiles_per_example), (unsigned)p[0].n_ctiles);
  if (vec) dispatch_sq<true>(a, p, o, amax, grid, st);
  else dispatch_sq<false>(a, p, o, amax, grid, st);
  if (a.ec) {
    const int64_t ncb = (B * a.D + kWave - 1) / kWave;
    const int bpe = (int)((a.S + kFinRows - 1) / kFinRows);
    const int64_t nrb = B * bpe;
    for (int k = 0; k < 2; ++k)
      hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)(ncb + nrb)), dim3(kThreads), 0, st, B, a.D, a.S,
                         p[k].tiles_per_example, p[k].n_ctiles, 0, (int)ncb, bpe, a.delta[k],
                         (const float*)(wk[k] + L.col_part), (const int32_t*)(wk[k] + L.colq_part),
                         (const float*)(wk[k] + L.row_part), a.ec_col[k], (int32_t*)nullptr, a.ec_row[k],
                         a.ec_mean[k], (double*)(wk[k] + L.blk_sum), (uint32_t*)(wk[k] + L.counter));
  }
  return hipGetLastError();
}

}  // namespace s3r
