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
// and give empty tables (every grouped kernel then finds no work).  amax[0 .. G) is cleared for the grouped quantizer's atomic maxima.
__global__ __launch_bounds__(kTabThreads) void group_tables_kernel(const int64_t* __restrict__ offsets, int64_t G,
                                                                   int64_t R, int32_t* __restrict__ tiles64,
                                                                   int32_t* __restrict__ tiles256,
                                                                   int32_t* __restrict__ order,
                                                                   uint32_t* __restrict__ status,
                                                                   uint32_t* __restrict__ amax,
                                                                   uint32_t* __restrict__ flags) {
  __shared__ int bad;
  __shared__ int32_t carry[2];
  __shared__ int32_t scan[2][kTabThreads];
  const int tid = threadIdx.x;
  if (tid == 0) {
    bad = (offsets[0] != 0 || offsets[G] != R) ? 1 : 0;
    carry[0] = carry[1] = 0;
  }
  __syncthreads();
  for (int64_t e = tid; e < G; e += kTabThreads)
    if (offsets[e + 1] < offsets[e]) atomicOr(&bad, 1);
  __syncthreads();
  const bool ok = bad == 0;
  for (int64_t base = 0; base < G; base += kTabThreads) {
    const int64_t e = base + tid;
    const int64_t n = (ok && e < G) ? offsets[e + 1] - offsets[e] : 0;
    scan[0][tid] = (int32_t)((n + 63) / 64);
    scan[1][tid] = (int32_t)((n + 255) / 256);
    __syncthreads();
    for (int o = 1; o < kTabThreads; o <<= 1) {          // inclusive Hillis-Steele scan
      int32_t a0 = 0, a1 = 0;
      if (tid >= o) { a0 = scan[0][tid - o]; a1 = scan[1][tid - o]; }
      __syncthreads();
      scan[0][tid] += a0;
      scan[1][tid] += a1;
      __syncthreads();
    }
    if (e < G) {                                         // exclusive prefix at e
      tiles64[e] = carry[0] + scan[0][tid] - (int32_t)((n + 63) / 64);
      tiles256[e] = carry[1] + scan[1][tid] - (int32_t)((n + 255) / 256);
    }
    __syncthreads();
    if (tid == kTabThreads - 1) { carry[0] += scan[0][tid]; carry[1] += scan[1][tid]; }
    __syncthreads();
  }
  if (tid == 0) {
    tiles64[G] = carry[0];
    tiles256[G] = carry[1];
    status[0] = ok ? 0u : 1u;
    if (!ok && flags) atomicOr(flags, S3R_FLAG_BAD_GROUPS);
  }
  // order: rank of e among the groups by descending rows, ties by index (G <= kMaxGroups)
  __shared__ int32_t rows[kMaxGroups];
  for (int64_t e = tid; e < G; e += kTabThreads) rows[e] = ok ? (int32_t)(offsets[e + 1] - offsets[e]) : 0;
  __syncthreads();
  for (int64_t e = tid; e < G; e += kTabThreads) {
    const int32_t n = rows[e];
    int32_t rank = 0;
    for (int64_t f = 0; f < G; ++f) rank += (rows[f] > n) || (rows[f] == n && f < e);
    order[rank] = (int32_t)e;
    amax[e] = 0u;
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

hipError_t launch_group_tables(const GroupTables& t, int64_t R, uint32_t* flags, hipStream_t st) {
  hipLaunchKernelGGL(group_tables_kernel, dim3(1), dim3(kTabThreads), 0, st, t.offsets, t.G, R, t.tiles64, t.tiles256,
                     t.order, t.status, t.amax, flags);
  return hipGetLastError();
}

}  // namespace s3r
