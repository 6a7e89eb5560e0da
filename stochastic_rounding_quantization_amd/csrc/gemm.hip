// INT8 backward GEMMs on the gfx950 matrix cores, with the dequantisation and
// S3R-EC epilogues, and the two small products the correction needs.
//
// S3R page, "Quantized Backpropagation with Stochastic Rounding": each
// backward product is an S8 x S8 GEMM with S32 accumulation and a rescale;
// one S8 tensor Q feeds both, contracting its channels (dX) and its tokens
// (dW).  "Two-Way Correction": after the unchanged GEMMs subtract the averages
// times W from dX (the token means times the row sums r_W) and the inputs
// times the same averages from dW.
//
//   dX [T x d_in] = Q [T x D] . Wq [D x d_in]    A: K-contiguous, B: N-contiguous
//   dW [D x d_in] = Q^T        . Xq [T x d_in]   A: M-contiguous, B: N-contiguous
//
// Tiling: 256 x 256 output tile per 256-thread workgroup (four 64-lane waves,
// 2 x 2, each 128 x 128 = 4 x 4 blocks of v_mfma_i32_32x32x32_i8), K step 64,
// LDS double buffer (2 x (16 + 16) KB).  LDS holds every operand K-contiguous:
// row r of a tile is 64 bytes in four 16-byte chunks, chunk c stored at
// position c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3, so the 16-byte
// fragment reads of 8 or 16 consecutive rows hit distinct banks.  Operands
// that are contiguous along M or N are transposed on the way in: each thread
// loads an 8 (k) x 8 (mn) byte block with eight 8-byte loads and transposes
// it with byte permutes before one 8-byte LDS write per mn row.
// Workgroups are numbered so that the 32 consecutive tiles of one XCD share
// rows of A and columns of B (grouped order), for L2 reuse.
#include "s3r_internal.h"

namespace s3r {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmThreads = 256;
constexpr int kTileBytes = BM * BK;   // 16 KB per operand tile
constexpr int kGroupM = 8;            // grouped tile order: 8 tile-rows per group
constexpr int kNumXcd = 8;

enum { EPI_RAW = 0, EPI_DX = 1, EPI_DW = 2 };

struct EpiParams {
  const float* delta; int per_token;
  const float* row_scale;            // s_x (dX) or s_w (dW); null = 1
  int ec;                            // apply the correction
  // dX: rW [N] int32, ec_row [M], ec_mean [B], v [B x N] f32
  // dW: ebar [B x M] f32 (row index j), xs [B x N] int32, u [N] f32
  const int32_t* colsum; const float* ec_row; const float* ec_mean; const float* vec;
  const float* ebar; const float* u;
  int64_t S, B;
  void* out; int64_t ld_out; int out_i32;
};

struct GemmParams {
  const int8_t* A; int64_t lda;
  const int8_t* B; int64_t ldb;
  int64_t M, N, K;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// 4 x 4 byte transpose: out[j] byte i = in[i] byte j.
__device__ __forceinline__ void transpose4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t o[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // a0.0 a1.0 a0.1 a1.1
  const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // a0.2 a1.2 a0.3 a1.3
  const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);  // a2.0 a3.0 a2.1 a3.1
  const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);  // a2.2 a3.2 a2.3 a3.3
  o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);               // a0.0 a1.0 a2.0 a3.0
  o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);               // a0.1 a1.1 a2.1 a3.1
  o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// ---------------------------------------------------- global -> registers ----
// K-contiguous operand: rows (m or n) of 64 bytes; thread owns 4 chunks.
struct KStage { uint4 v[4]; };
// MN-contiguous operand: 64 k-rows of 256 bytes; thread owns an 8 x 8 block.
struct MStage { uint2 v[8]; };

template <bool MASKED>
__device__ __forceinline__ void load_k(KStage& s, const int8_t* __restrict__ P, int64_t ld, int64_t rows,
                                       int64_t K, int64_t r0, int64_t k0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = it * 64 + (tid >> 2);
    const int c = tid & 3;
    const int64_t gr = r0 + row, gk = k0 + c * 16;
    if (!MASKED) {
      s.v[it] = *reinterpret_cast<const uint4*>(P + gr * ld + gk);
    } else {
      uint32_t w[4] = {0, 0, 0, 0};
      if (gr < rows) {
        const int8_t* p = P + gr * ld + gk;
        if (gk + 16 <= K) {
          const uint4 u = *reinterpret_cast<const uint4*>(p);
          w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
        } else {
          for (int b = 0; b < 16; ++b)
            if (gk + b < K) w[b >> 2] |= (uint32_t)(uint8_t)p[b] << (8 * (b & 3));
        }
      }
      s.v[it] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

__device__ __forceinline__ void store_k(const KStage& s, uint8_t* __restrict__ lds) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = it * 64 + (tid >> 2);
    const int c = tid & 3;
    *reinterpret_cast<uint4*>(lds + row * 64 + ((c ^ swz(row)) << 4)) = s.v[it];
  }
}

template <bool MASKED>
__device__ __forceinline__ void load_m(MStage& s, const int8_t* __restrict__ P, int64_t ld, int64_t cols,
                                       int64_t K, int64_t c0, int64_t k0) {
  const int tid = threadIdx.x;
  const int kg = tid >> 5, mg = tid & 31;
  const int64_t gc = c0 + mg * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t gk = k0 + kg * 8 + i;
    if (!MASKED) {
      s.v[i] = *reinterpret_cast<const uint2*>(P + gk * ld + gc);
    } else {
      uint32_t w[2] = {0, 0};
      if (gk < K) {
        const int8_t* p = P + gk * ld + gc;
        if (gc + 8 <= cols) {
          const uint2 u = *reinterpret_cast<const uint2*>(p);
          w[0] = u.x; w[1] = u.y;
        } else {
          for (int b = 0; b < 8; ++b)
            if (gc + b < cols) w[b >> 2] |= (uint32_t)(uint8_t)p[b] << (8 * (b & 3));
        }
      }
      s.v[i] = make_uint2(w[0], w[1]);
    }
  }
}

__device__ __forceinline__ void store_m(const MStage& s, uint8_t* __restrict__ lds) {
  const int tid = threadIdx.x;
  const int kg = tid >> 5, mg = tid & 31;
  uint32_t lo0[4], lo1[4], hi0[4], hi1[4];
  // rows k 0..3 / 4..7 of the block, columns mn 0..3 (.x) and 4..7 (.y)
  transpose4(s.v[0].x, s.v[1].x, s.v[2].x, s.v[3].x, lo0);
  transpose4(s.v[4].x, s.v[5].x, s.v[6].x, s.v[7].x, lo1);
  transpose4(s.v[0].y, s.v[1].y, s.v[2].y, s.v[3].y, hi0);
  transpose4(s.v[4].y, s.v[5].y, s.v[6].y, s.v[7].y, hi1);
  const int c = kg >> 1, half = (kg & 1) << 3;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = mg * 8 + j;
    const uint2 v = j < 4 ? make_uint2(lo0[j], lo1[j]) : make_uint2(hi0[j - 4], hi1[j - 4]);
    *reinterpret_cast<uint2*>(lds + row * 64 + ((c ^ swz(row)) << 4) + half) = v;
  }
}

// ----------------------------------------------------------------- kernel ----
template <bool A_KMAJOR, int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_i8_kernel(GemmParams g, EpiParams ep) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];
  // buffer b: A tile at smem + 2b * 16 KB, B tile right after it
#define S3R_SA(b) (smem + (b) * 2 * kTileBytes)
#define S3R_SB(b) (smem + (b) * 2 * kTileBytes + kTileBytes)

  // XCD-aware numbering: hardware block ids go round-robin over the 8 XCDs;
  // give each XCD a contiguous range of logical tiles.
  const int nblocks = g.tiles_m * g.tiles_n;
  int bid = blockIdx.x;
  if (nblocks % kNumXcd == 0) bid = (bid % kNumXcd) * (nblocks / kNumXcd) + bid / kNumXcd;
  const int group = kGroupM * g.tiles_n;
  const int first_m = (bid / group) * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int tm = first_m + (bid % group) % gsz;
  const int tn = (bid % group) / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  const bool mn_inside = (m0 + BM <= g.M) && (n0 + BN <= g.N);
  const int nk = (int)((g.K + BK - 1) / BK);

  KStage ka; MStage ma; MStage mb;
  auto load_stage = [&](int64_t k0) {
    if (mn_inside && k0 + BK <= g.K) {
      if constexpr (A_KMAJOR) load_k<false>(ka, g.A, g.lda, g.M, g.K, m0, k0);
      else load_m<false>(ma, g.A, g.lda, g.M, g.K, m0, k0);
      load_m<false>(mb, g.B, g.ldb, g.N, g.K, n0, k0);
    } else {
      if constexpr (A_KMAJOR) load_k<true>(ka, g.A, g.lda, g.M, g.K, m0, k0);
      else load_m<true>(ma, g.A, g.lda, g.M, g.K, m0, k0);
      load_m<true>(mb, g.B, g.ldb, g.N, g.K, n0, k0);
    }
  };
  auto store_stage = [&](int buf) {
    if constexpr (A_KMAJOR) store_k(ka, S3R_SA(buf));
    else store_m(ma, S3R_SA(buf));
    store_m(mb, S3R_SB(buf));
  };

  if (nk > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage((int64_t)(kt + 1) * BK);
    const uint8_t* a_s = S3R_SA(buf);
    const uint8_t* b_s = S3R_SB(buf);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      v4i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const v4i*>(a_s + r * 64 + ((c ^ swz(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + j * 32 + (lane & 31);
        bf[j] = *reinterpret_cast<const v4i*>(b_s + r * 64 + ((c ^ swz(r)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

#undef S3R_SA
#undef S3R_SB
  // ------------------------------------------------------------ epilogue ----
  // Output layout of a 32x32 block: lane l, register r -> row (r/4)*8 + (l/32)*4 + r%4, column l%32.
  float* rowf = reinterpret_cast<float*>(smem);   // per-row factors, 4 floats per tile row
  if constexpr (EPI == EPI_DX) {
    // alpha = Delta_t / s_x[t], beta = 1 / s_x[t], gamma = (eps_t - mu_b) / s_x[t]
    for (int r = threadIdx.x; r < BM; r += kGemmThreads) {
      const int64_t t = m0 + r;
      float a = 0.f, be = 0.f, ga = 0.f;
      if (t < g.M) {
        const float d = ep.per_token ? ep.delta[t] : ep.delta[0];
        const float inv = ep.row_scale ? __fdiv_rn(1.f, ep.row_scale[t]) : 1.f;
        a = d * inv;
        be = inv;
        if (ep.ec) ga = (ep.ec_row[t] - ep.ec_mean[t / ep.S]) * inv;
      }
      rowf[r * 4 + 0] = a; rowf[r * 4 + 1] = be; rowf[r * 4 + 2] = ga;
    }
    __syncthreads();
  } else if constexpr (EPI == EPI_DW) {
    // alpha = Delta / s_w[j], beta = 1 / s_w[j]
    for (int r = threadIdx.x; r < BM; r += kGemmThreads) {
      const int64_t j = m0 + r;
      float a = 0.f, be = 0.f;
      if (j < g.M) {
        const float inv = ep.row_scale ? __fdiv_rn(1.f, ep.row_scale[j]) : 1.f;
        a = ep.delta[0] * inv;
        be = inv;
      }
      rowf[r * 4 + 0] = a; rowf[r * 4 + 1] = be;
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
    const bool n_ok = n < g.N;
    float cu = 0.f, crw = 0.f;
    if constexpr (EPI == EPI_DX) {
      if (ep.ec && n_ok) crw = (float)ep.colsum[n];
    } else if constexpr (EPI == EPI_DW) {
      if (ep.ec && n_ok) cu = ep.u[n];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int64_t m = m0 + lr;
        if (!(n_ok && m < g.M)) continue;
        const int32_t v = acc[i][j][r];
        if constexpr (EPI == EPI_RAW) {
          reinterpret_cast<int32_t*>(ep.out)[m * ep.ld_out + n] = v;
        } else if constexpr (EPI == EPI_DX) {
          const float4 f = *reinterpret_cast<const float4*>(rowf + lr * 4);
          float corr = 0.f;
          if (ep.ec) corr = fmaf(f.z, crw, f.y * ep.vec[(m / ep.S) * g.N + n]);
          reinterpret_cast<float*>(ep.out)[m * ep.ld_out + n] = fmaf(f.x, (float)v, -corr);
        } else {
          const float4 f = *reinterpret_cast<const float4*>(rowf + lr * 4);
          float corr = 0.f;
          if (ep.ec) {
            float s = cu;
            for (int64_t b = 0; b < ep.B; ++b) s = fmaf(ep.ebar[b * g.M + m], (float)ep.colsum[b * g.N + n], s);
            corr = f.y * s;
          }
          reinterpret_cast<float*>(ep.out)[m * ep.ld_out + n] = fmaf(f.x, (float)v, -corr);
        }
      }
    }
  }
}

// -------------------------------------------------------------- GEMVs ----
// out_part[jc][b][n] = sum over k in chunk jc of coef(b, k) * P[k][n]  (P int8 [K x N])
// Coefficients: VEC mode coef(b, k) = C[b * K + k] (the channel means ebar);
// TOKEN mode (b = 0 only) coef(k) = ec_row[k] - ec_mean[k / S].
constexpr int kGvThreads = 256;
constexpr int kGvCols = 8;         // columns per thread
constexpr int kGvRows = 128;       // k rows per chunk
constexpr int kGvB = 4;            // coefficient rows per pass

__global__ __launch_bounds__(kGvThreads) void gemv_partial_kernel(
    const int8_t* __restrict__ P, int64_t ld, int64_t K, int64_t N, int64_t nb, int token_mode,
    const float* __restrict__ C, const float* __restrict__ ec_row, const float* __restrict__ ec_mean, int64_t S,
    float* __restrict__ part) {
  const int64_t n0 = ((int64_t)blockIdx.x * kGvThreads + threadIdx.x) * kGvCols;
  const int64_t k0 = (int64_t)blockIdx.y * kGvRows;
  const int64_t k1 = min(k0 + kGvRows, K);
  const int jc = blockIdx.y;
  for (int64_t b0 = 0; b0 < nb; b0 += kGvB) {
    float acc[kGvB][kGvCols];
#pragma unroll
    for (int b = 0; b < kGvB; ++b)
#pragma unroll
      for (int c = 0; c < kGvCols; ++c) acc[b][c] = 0.f;
    for (int64_t k = k0; k < k1; ++k) {
      int8_t w[kGvCols];
      const int8_t* p = P + k * ld + n0;
      if (n0 + kGvCols <= N) {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
#pragma unroll
        for (int c = 0; c < 4; ++c) { w[c] = (int8_t)(u.x >> (8 * c)); w[c + 4] = (int8_t)(u.y >> (8 * c)); }
      } else {
#pragma unroll
        for (int c = 0; c < kGvCols; ++c) w[c] = (n0 + c < N) ? p[c] : (int8_t)0;
      }
      float cf[kGvB];
#pragma unroll
      for (int b = 0; b < kGvB; ++b) {
        float x = 0.f;
        if (b0 + b < nb) x = token_mode ? ec_row[k] - ec_mean[k / S] : C[(b0 + b) * K + k];
        cf[b] = x;
      }
#pragma unroll
      for (int c = 0; c < kGvCols; ++c) {
        const float wf = (float)w[c];
#pragma unroll
        for (int b = 0; b < kGvB; ++b) acc[b][c] = fmaf(cf[b], wf, acc[b][c]);
      }
    }
#pragma unroll
    for (int b = 0; b < kGvB; ++b) {
      if (b0 + b >= nb) break;
#pragma unroll
      for (int c = 0; c < kGvCols; ++c)
        if (n0 + c < N) part[((int64_t)jc * nb + b0 + b) * N + n0 + c] = acc[b][c];
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ part, int64_t nchunks,
                                                          int64_t count, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  double a = 0.0;
  for (int64_t c = 0; c < nchunks; ++c) a += (double)part[c * count + i];
  out[i] = (float)a;
}

hipError_t run_gemv(const int8_t* P, int64_t ld, int64_t K, int64_t N, int64_t nb, int token_mode, const float* C,
                    const float* ec_row, const float* ec_mean, int64_t S, float* part, float* out, hipStream_t st) {
  const int64_t nchunks = (K + kGvRows - 1) / kGvRows;
  const int64_t cols_per_block = (int64_t)kGvThreads * kGvCols;
  dim3 grid((unsigned)((N + cols_per_block - 1) / cols_per_block), (unsigned)nchunks);
  hipLaunchKernelGGL(gemv_partial_kernel, grid, dim3(kGvThreads), 0, st, P, ld, K, N, nb, token_mode, C, ec_row,
                     ec_mean, S, part);
  const int64_t count = nb * N;
  hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, part, nchunks,
                     count, out);
  return hipGetLastError();
}

size_t gemv_part_bytes(int64_t K, int64_t N, int64_t nb) {
  const int64_t nchunks = (K + kGvRows - 1) / kGvRows;
  return align_up((size_t)nchunks * nb * N * 4, 256);
}

template <bool A_KMAJOR, int EPI>
hipError_t run_gemm(const GemmParams& g, const EpiParams& ep, hipStream_t st) {
  GemmTiming& tm = gemm_timing();
  const GemmTiming ev = tm;
  tm = GemmTiming{};
  const int nblocks = g.tiles_m * g.tiles_n;
  if (ev.start) hipEventRecord(ev.start, st);
  if (nblocks > 0)
    hipLaunchKernelGGL((gemm_i8_kernel<A_KMAJOR, EPI>), dim3((unsigned)nblocks), dim3(kGemmThreads), 0, st, g, ep);
  if (ev.stop) hipEventRecord(ev.stop, st);
  return hipGetLastError();
}

GemmParams make_gemm(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, int64_t M, int64_t N, int64_t K) {
  GemmParams g;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.M = M; g.N = N; g.K = K;
  g.tiles_m = (int)((M + BM - 1) / BM);
  g.tiles_n = (int)((N + BN - 1) / BN);
  return g;
}

}  // namespace

GemmTiming& gemm_timing() {
  static thread_local GemmTiming t;
  return t;
}

size_t dx_workspace(int64_t T, int64_t D, int64_t d_in, int64_t S, int ec) {
  if (!ec || S <= 0) return 0;
  const int64_t B = T / S;
  return gemv_part_bytes(D, d_in, B) + align_up((size_t)B * d_in * 4, 256);
}

size_t dw_workspace(int64_t T, int64_t D, int64_t d_in, int64_t S, int ec) {
  (void)D; (void)S;
  if (ec != S3R_EC_TWO_WAY) return 0;
  return gemv_part_bytes(T, d_in, 1) + align_up((size_t)d_in * 4, 256);
}

hipError_t launch_backward_dx(const DxArgs& a, hipStream_t st) {
  const int64_t B = a.S > 0 ? a.T / a.S : 0;
  EpiParams ep{};
  ep.delta = a.delta; ep.per_token = a.per_token; ep.row_scale = a.sx;
  ep.ec = (a.ec != S3R_EC_NONE) && a.out_dt == S3R_F32;
  ep.colsum = a.rW; ep.ec_row = a.ec_row; ep.ec_mean = a.ec_mean;
  ep.S = a.S; ep.B = B;
  ep.out = a.out; ep.ld_out = a.ld_out; ep.out_i32 = a.out_dt == S3R_I32_RAW;
  if (ep.ec && a.T > 0 && a.d_in > 0) {
    float* part = (float*)a.ws;
    float* v = (float*)(a.ws + gemv_part_bytes(a.D, a.d_in, B));
    if (a.D > 0) {
      hipError_t e = run_gemv(a.W, a.ld_w, a.D, a.d_in, B, 0, a.ec_col, nullptr, nullptr, a.S, part, v, st);
      if (e != hipSuccess) return e;
    } else {
      hipError_t e = fill_zero(v, B * a.d_in, st);
      if (e != hipSuccess) return e;
    }
    ep.vec = v;
  }
  const GemmParams g = make_gemm(a.Q, a.ld_q, a.W, a.ld_w, a.T, a.d_in, a.D);
  if (a.out_dt == S3R_I32_RAW) return run_gemm<true, EPI_RAW>(g, ep, st);
  return run_gemm<true, EPI_DX>(g, ep, st);
}

hipError_t launch_backward_dw(const DwArgs& a, hipStream_t st) {
  const int64_t B = a.S > 0 ? a.T / a.S : 0;
  EpiParams ep{};
  ep.delta = a.delta; ep.per_token = 0; ep.row_scale = a.sw;
  ep.ec = (a.ec == S3R_EC_TWO_WAY) && a.out_dt == S3R_F32;
  ep.colsum = a.xs; ep.ebar = a.ec_col; ep.ec_row = a.ec_row; ep.ec_mean = a.ec_mean;
  ep.S = a.S; ep.B = B;
  ep.out = a.out; ep.ld_out = a.ld_out; ep.out_i32 = a.out_dt == S3R_I32_RAW;
  if (ep.ec && a.D > 0 && a.d_in > 0) {
    float* part = (float*)a.ws;
    float* u = (float*)(a.ws + gemv_part_bytes(a.T, a.d_in, 1));
    if (a.T > 0) {
      hipError_t e = run_gemv(a.X, a.ld_x, a.T, a.d_in, 1, 1, nullptr, a.ec_row, a.ec_mean, a.S, part, u, st);
      if (e != hipSuccess) return e;
    } else {
      hipError_t e = fill_zero(u, a.d_in, st);
      if (e != hipSuccess) return e;
    }
    ep.u = u;
  }
  // dW = Q^T Xq: A[m=j][k=t] = Q[t][j] (M-contiguous), B = Xq [T x d_in] (N-contiguous)
  const GemmParams g = make_gemm(a.Q, a.ld_q, a.X, a.ld_x, a.D, a.d_in, a.T);
  if (a.out_dt == S3R_I32_RAW) return run_gemm<false, EPI_RAW>(g, ep, st);
  return run_gemm<false, EPI_DW>(g, ep, st);
}

}  // namespace s3r
