// SwiGLU backward glue of an FFN block, for gfx950 (an HBM-bound elementwise pass).
// The element arithmetic (swiglu_math.h) is fixed to one rounding per fp32
// operation, so the results do not depend on the launch shape.
#include "swiglu_math.h"

namespace s3r {
namespace {

// Thread mapping of both glue kernels: blockIdx.x * 256 + threadIdx.x is an 8-element chunk column
// of the rows (16-byte loads and stores), fixed for the thread; blockIdx.y strides over the rows. A row
// of a block is one contiguous span of 2048 columns, and the per-chunk index arithmetic is one add.

template <bool VEC>
__global__ __launch_bounds__(256) void swiglu_backward_kernel(
    int64_t T, int64_t F, const float* __restrict__ dH, int64_t ld_dh, const uint16_t* __restrict__ Ag,
    const uint16_t* __restrict__ Au, int64_t ld_a, uint16_t* __restrict__ Gg, uint16_t* __restrict__ Gu,
    int64_t ld_g) {
  const int64_t j0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (j0 >= F) return;
  const bool full = VEC && j0 + 8 <= F;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    const float* dh = dH + t * ld_dh + j0;
    const uint16_t* ag = Ag + t * ld_a + j0;
    const uint16_t* au = Au + t * ld_a + j0;
    uint16_t* gg = Gg + t * ld_g + j0;
    uint16_t* gu = Gu + t * ld_g + j0;
    if (full) {
      uint32_t og[4], ou[4];
      glue8(dh, ag, au, og, ou);
      *reinterpret_cast<uint4*>(gg) = make_uint4(og[0], og[1], og[2], og[3]);
      *reinterpret_cast<uint4*>(gu) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
    } else {
      for (int i = 0; i < 8 && j0 + i < F; ++i) {
        uint32_t g, u;
        glue1(dh[i], bf16_to_f32(ag[i]), bf16_to_f32(au[i]), g, u);
        gg[i] = (uint16_t)g;
        gu[i] = (uint16_t)u;
      }
    }
  }
}

// ------------------------------------------------ glue + per-tensor amax ----
// The same glue, and in the same pass the per-tensor amax that the gate and up
// projections' quantizers need: max |fl(fl(G * s_x[t]) * s_w[j])| over the
// bf16-rounded results (the quantizer's fold of its own input), as ordered fp32
// bits (NaN above every number).  Same thread mapping as the plain glue; block
// b = blockIdx.y * gridDim.x + blockIdx.x writes its two maxima to part[0][b]
// and part[1][b], and swiglu_amax_finalize_kernel reduces them.  STORE false
// finds the maxima only (G_gate and G_up are never written: the quantizer that
// follows computes them again).
constexpr int kAmaxGlueBlocks = 4096;

__device__ __forceinline__ uint32_t fold_abs_bits(uint32_t bf16, float fx, float sw) {
  return __float_as_uint((__uint_as_float(bf16 << 16) * fx) * sw) & 0x7FFFFFFFu;
}

template <bool VEC, bool STORE>
__global__ __launch_bounds__(256) void swiglu_amax_kernel(
    int64_t T, int64_t F, const float* __restrict__ dH, int64_t ld_dh, const uint16_t* __restrict__ Ag,
    const uint16_t* __restrict__ Au, int64_t ld_a, uint16_t* __restrict__ Gg, uint16_t* __restrict__ Gu,
    int64_t ld_g, const float* __restrict__ sx, const float* __restrict__ swg, const float* __restrict__ swu,
    uint32_t* __restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  uint32_t mg = 0, mu = 0;
  if (j0 < F) {
    const bool full = VEC && j0 + 8 <= F;
    for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
      const float fx = sx ? sx[t] : 1.f;
      const float* dh = dH + t * ld_dh + j0;
      const uint16_t* ag = Ag + t * ld_a + j0;
      const uint16_t* au = Au + t * ld_a + j0;
      uint16_t* gg = STORE ? Gg + t * ld_g + j0 : nullptr;
      uint16_t* gu = STORE ? Gu + t * ld_g + j0 : nullptr;
      if (full) {
        // the column scales are re-read per row (cache hits) rather than held in 16 registers across
        // the loop, which made the compiler wait for the row's first loads before issuing the last
        float cg[8], cu[8];
        if (swg) {
          const float4 a = *reinterpret_cast<const float4*>(swg + j0), b = *reinterpret_cast<const float4*>(swg + j0 + 4);
          cg[0] = a.x; cg[1] = a.y; cg[2] = a.z; cg[3] = a.w; cg[4] = b.x; cg[5] = b.y; cg[6] = b.z; cg[7] = b.w;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) cg[i] = 1.f;
        }
        if (swu) {
          const float4 a = *reinterpret_cast<const float4*>(swu + j0), b = *reinterpret_cast<const float4*>(swu + j0 + 4);
          cu[0] = a.x; cu[1] = a.y; cu[2] = a.z; cu[3] = a.w; cu[4] = b.x; cu[5] = b.y; cu[6] = b.z; cu[7] = b.w;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) cu[i] = 1.f;
        }
        uint32_t og[4], ou[4];
        glue8(dh, ag, au, og, ou);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mg = max(mg, max(fold_abs_bits(og[i] & 0xFFFFu, fx, cg[2 * i]), fold_abs_bits(og[i] >> 16, fx, cg[2 * i + 1])));
          mu = max(mu, max(fold_abs_bits(ou[i] & 0xFFFFu, fx, cu[2 * i]), fold_abs_bits(ou[i] >> 16, fx, cu[2 * i + 1])));
        }
        if constexpr (STORE) {
          *reinterpret_cast<uint4*>(gg) = make_uint4(og[0], og[1], og[2], og[3]);
          *reinterpret_cast<uint4*>(gu) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
        }
      } else {
        for (int i = 0; i < 8 && j0 + i < F; ++i) {
          uint32_t g, u;
          glue1(dh[i], bf16_to_f32(ag[i]), bf16_to_f32(au[i]), g, u);
          if constexpr (STORE) {
            gg[i] = (uint16_t)g;
            gu[i] = (uint16_t)u;
          }
          mg = max(mg, fold_abs_bits(g, fx, swg ? swg[j0 + i] : 1.f));
          mu = max(mu, fold_abs_bits(u, fx, swu ? swu[j0 + i] : 1.f));
        }
      }
    }
  }
  __shared__ uint32_t red[2][4];
  mg = wave_max_u32(mg);
  mu = wave_max_u32(mu);
  if (lane == 0) { red[0][wave] = mg; red[1][wave] = mu; }
  __syncthreads();
  if (threadIdx.x < 2) {
    const int k = threadIdx.x;
    const int64_t nblk = (int64_t)gridDim.x * gridDim.y, b = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    part[k * nblk + b] = max(max(red[k][0], red[k][1]), max(red[k][2], red[k][3]));
  }
}

// amax_bits[k] = max over the blocks' partials part[k][*], k = 0 (gate), 1 (up).
__global__ __launch_bounds__(256) void swiglu_amax_finalize_kernel(const uint32_t* __restrict__ part, int nblk,
                                                                   uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t red[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t m[2] = {0u, 0u};
  int i = threadIdx.x;
  for (; i + 7 * 256 < nblk; i += 8 * 256) {       // eight loads of each array in flight together
    uint32_t a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = part[i + u * 256];
      b[u] = part[nblk + i + u * 256];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      m[0] = max(m[0], a[u]);
      m[1] = max(m[1], b[u]);
    }
  }
  for (; i < nblk; i += 256) {
    m[0] = max(m[0], part[i]);
    m[1] = max(m[1], part[nblk + i]);
  }
  for (int k = 0; k < 2; ++k) {
    const uint32_t w = wave_max_u32(m[k]);
    if (lane == 0) red[k][wave] = w;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const int k = threadIdx.x;
    amax_bits[k] = max(max(red[k][0], red[k][1]), max(red[k][2], red[k][3]));
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Grid of the glue kernels: x over the 256-chunk column blocks, y over rows (at most max_blocks in all,
// unless the columns alone need more).
dim3 glue_grid(int64_t T, int64_t F, int64_t max_blocks) {
  if (T <= 0 || F <= 0) return dim3(0, 0, 1);
  const int64_t gx = ((F + 7) / 8 + 255) / 256;
  const int64_t gy = std::max<int64_t>(1, std::min<int64_t>({T, max_blocks / gx, 65535}));
  return dim3((unsigned)gx, (unsigned)gy, 1);
}

int64_t amax_blocks(int64_t T, int64_t F) {
  const dim3 g = glue_grid(T, F, kAmaxGlueBlocks);
  return (int64_t)g.x * g.y;
}

}  // namespace

size_t swiglu_amax_workspace(int64_t T, int64_t F) {
  return align_up((size_t)std::max<int64_t>(amax_blocks(T, F), 1) * 2 * 4, 256);
}

hipError_t launch_swiglu_backward_amax(int64_t T, int64_t F, const float* dH, int64_t ld_dh, const uint16_t* Ag,
                                       const uint16_t* Au, int64_t ld_a, uint16_t* Gg, uint16_t* Gu, int64_t ld_g,
                                       const float* sx, const float* swg, const float* swu, uint32_t* amax_bits,
                                       char* ws, hipStream_t st) {
  uint32_t* part = (uint32_t*)(ws);
  const int64_t nblk = amax_blocks(T, F);
  const bool store = Gg != nullptr;   // the C ABI passes both outputs or (for the fused quantizer) neither
  if (nblk > 0) {
    const bool vec = aligned16(dH) && aligned16(Ag) && aligned16(Au) && ld_dh % 4 == 0 && ld_a % 8 == 0 &&
                     (!store || (aligned16(Gg) && aligned16(Gu) && ld_g % 8 == 0)) && (!swg || aligned16(swg)) &&
                     (!swu || aligned16(swu));
    const dim3 grid = glue_grid(T, F, kAmaxGlueBlocks);
    auto kern = vec ? (store ? swiglu_amax_kernel<true, true> : swiglu_amax_kernel<true, false>)
                    : (store ? swiglu_amax_kernel<false, true> : swiglu_amax_kernel<false, false>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, T, F, dH, ld_dh, Ag, Au, ld_a, Gg, Gu, ld_g, sx, swg, swu, part);
  }
  hipLaunchKernelGGL(swiglu_amax_finalize_kernel, dim3(1), dim3(256), 0, st, part, (int)nblk, amax_bits);
  return hipGetLastError();
}

hipError_t launch_swiglu_backward(int64_t T, int64_t F, const float* dH, int64_t ld_dh, const uint16_t* Ag,
                                  const uint16_t* Au, int64_t ld_a, uint16_t* Gg, uint16_t* Gu, int64_t ld_g,
                                  hipStream_t st) {
  if (T == 0 || F == 0) return hipSuccess;
  const bool vec = aligned16(dH) && aligned16(Ag) && aligned16(Au) && aligned16(Gg) && aligned16(Gu) &&
                   ld_dh % 4 == 0 && ld_a % 8 == 0 && ld_g % 8 == 0;
  const dim3 grid = glue_grid(T, F, 8192);
  if (vec)
    hipLaunchKernelGGL(swiglu_backward_kernel<true>, grid, dim3(256), 0, st, T, F, dH, ld_dh, Ag, Au, ld_a, Gg, Gu,
                       ld_g);
  else
    hipLaunchKernelGGL(swiglu_backward_kernel<false>, grid, dim3(256), 0, st, T, F, dH, ld_dh, Ag, Au, ld_a, Gg, Gu,
                       ld_g);
  return hipGetLastError();
}

}  // namespace s3r
