// Grouped (mixture-of-experts) problems: rows sorted by group, group e owning
// rows [offsets[e], offsets[e+1]) of every row-indexed tensor.  The offsets
// live on the device (a router produces them there), so every grouped kernel
// is launched with a grid sized by an upper bound on its tile count, and each
// workgroup finds its group in tables that one small kernel derives from the
// offsets at the start of every grouped call:
//   tiles64[e]  = sum over e' < e of ceil(n_e' / 64)   (quantizer and GEMV bands)
//   tiles256[e] = sum over e' < e of ceil(n_e' / 256)  (GEMM row tiles)
//   order[k]    = the k-th largest group (ties by index), the dW GEMMs' schedule
// S3R page, Table IV and the MoE paragraph after it: the correction runs over
// the expert-sorted rows.
#include "s3r_internal.h"

namespace s3r {
namespace {

constexpr int kTabThreads = 1024;

// One workgroup.  Offsets that are not a non-decreasing sequence from 0 to R
// set status[0] = 1, raise S3R_FLAG_BAD_GROUPS in the caller's flags (if given)
// and give empty tables (every grouped kernel then finds no work).  amax[0 .. G)
// is cleared for the grouped quantizer's atomic maxima; with empty_delta and
// valid offsets, an empty group gets the step 1 there (no code tile writes it).
// The offsets are read once, into LDS; thread i owns groups i*per .. i*per+per-1,
// and the tile counts are one exclusive scan (wave scans, then the waves' totals).
__global__ __launch_bounds__(kTabThreads) void group_tables_kernel(const int64_t* __restrict__ offsets, int64_t G,
                                                                   int64_t R, int32_t* __restrict__ tiles64,
                                                                   int32_t* __restrict__ tiles256,
                                                                   int32_t* __restrict__ order,
                                                                   uint32_t* __restrict__ status,
                                                                   uint32_t* __restrict__ amax,
                                                                   uint32_t* __restrict__ flags,
                                                                   float* __restrict__ empty_delta) {
  constexpr int kWaves = kTabThreads / 64;
  __shared__ int64_t off[kMaxGroups + 1];
  __shared__ int32_t rows[kMaxGroups];
  __shared__ int32_t wtot[2][kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int64_t e = tid; e <= G; e += kTabThreads) off[e] = offsets[e];
  __syncthreads();
  int bad = (tid == 0 && (off[0] != 0 || off[G] != R)) ? 1 : 0;
  for (int64_t e = tid; e < G; e += kTabThreads) bad |= off[e + 1] < off[e] ? 1 : 0;
  const bool ok = __syncthreads_or(bad) == 0;
  const int per = (int)((G + kTabThreads - 1) / kTabThreads);
  int32_t c64 = 0, c256 = 0;                 // this thread's tile counts
  for (int i = 0; i < per; ++i) {
    const int64_t e = (int64_t)tid * per + i;
    if (e < G) {
      const int32_t n = ok ? (int32_t)(off[e + 1] - off[e]) : 0;
      rows[e] = n;
      c64 += (n + 63) / 64;
      c256 += (n + 255) / 256;
    }
  }
  int32_t s64 = c64, s256 = c256;            // inclusive scan within the wave
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t a64 = __shfl_up(s64, o, 64), a256 = __shfl_up(s256, o, 64);
    if (lane >= o) { s64 += a64; s256 += a256; }
  }
  if (lane == 63) { wtot[0][wave] = s64; wtot[1][wave] = s256; }
  __syncthreads();
  int32_t p64 = 0, p256 = 0;                 // the waves before this one
  for (int w = 0; w < wave; ++w) { p64 += wtot[0][w]; p256 += wtot[1][w]; }
  int32_t x64 = p64 + s64 - c64, x256 = p256 + s256 - c256;
  for (int i = 0; i < per; ++i) {
    const int64_t e = (int64_t)tid * per + i;
    if (e < G) {
      const int32_t n = rows[e];
      tiles64[e] = x64;
      tiles256[e] = x256;
      x64 += (n + 63) / 64;
      x256 += (n + 255) / 256;
    }
  }
  if (tid == kTabThreads - 1) {
    tiles64[G] = p64 + s64;
    tiles256[G] = p256 + s256;
    status[0] = ok ? 0u : 1u;
    if (!ok && flags) atomicOr(flags, S3R_FLAG_BAD_GROUPS);
  }
  __syncthreads();
  // order: rank of e among the groups by descending rows, ties by index (G <= kMaxGroups)
  for (int64_t e = tid; e < G; e += kTabThreads) {
    const int32_t n = rows[e];
    int32_t rank = 0;
    for (int64_t f = 0; f < G; ++f) rank += (rows[f] > n) || (rows[f] == n && f < e);
    order[rank] = (int32_t)e;
    amax[e] = 0u;
    if (empty_delta && ok && n == 0) empty_delta[e] = 1.f;
  }
}

}  // namespace

size_t group_tables_bytes(int64_t G) {
  return 3 * align_up((size_t)(G + 1) * 4, 256) + 256 + align_up((size_t)G * 4, 256);
}

GroupTables group_tables(char* base, int64_t G, const int64_t* offsets) {
  GroupTables t;
  t.offsets = offsets;
  t.G = G;
  char* p = base;
  t.tiles64 = (int32_t*)p;  p += align_up((size_t)(G + 1) * 4, 256);
  t.tiles256 = (int32_t*)p; p += align_up((size_t)(G + 1) * 4, 256);
  t.order = (int32_t*)p;    p += align_up((size_t)(G + 1) * 4, 256);
  t.status = (uint32_t*)p;  p += 256;
  t.amax = (uint32_t*)p;
  return t;
}

hipError_t launch_group_tables(const GroupTables& t, int64_t R, uint32_t* flags, hipStream_t st, float* empty_delta) {
  hipLaunchKernelGGL(group_tables_kernel, dim3(1), dim3(kTabThreads), 0, st, t.offsets, t.G, R, t.tiles64, t.tiles256,
                     t.order, t.status, t.amax, flags, empty_delta);
  return hipGetLastError();
}

}  // namespace s3r
