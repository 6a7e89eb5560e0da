// Internal declarations of libs3r.so: device helpers and kernel launchers.
// Written for gfx950 (CDNA4): 64-lane wavefronts, MFMA int8, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/s3r.h"

namespace s3r {

constexpr int kWave = 64;

// ---------------------------------------------------------------- Philox ----
// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64 products
// and xors, with the key bumped by the Weyl constants between rounds.
struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
  }
  return U4{c0, c1, c2, c3};
}

__device__ __forceinline__ uint32_t u4_word(const U4& v, uint32_t i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Counter tags (word 3 of the counter) separating the threshold streams; a
// second, independent stream s adds 65536 * s (the conventional configuration
// that quantizes the gradient separately for the weight-gradient product).
constexpr uint32_t kTagSR = 0;
constexpr uint32_t kTagS3R = 1;
constexpr uint32_t kTagBcast = 2;

// Per-token (S3R, tag kTagS3R) or per-example (Phi_bcast, tag kTagBcast, i the
// example index) threshold of index i in units of 2^-24: r*2^24 = (2b+1)*2^16,
// b the top 7 bits of byte i&3 of word (i>>2)&3 of block i>>4.
__device__ __forceinline__ int32_t s3r_threshold_units24(uint64_t i, uint32_t layer, uint64_t seed, uint32_t word3) {
  const uint64_t blk = i >> 4;
  const U4 v = philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), layer, word3,
                             (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t w = u4_word(v, (uint32_t)(i >> 2) & 3u);
  const uint32_t byte = (w >> (8u * ((uint32_t)i & 3u))) & 0xFFu;
  return (int32_t)(((byte >> 1) * 2u + 1u) << 16);
}

// Threshold of row t for the shared-threshold modes: per token, or (bcast) per
// example of S rows.
__device__ __forceinline__ int32_t row_threshold_units24(uint64_t t, uint32_t layer, uint64_t seed, bool bcast,
                                                         int64_t S, uint32_t stream_word) {
  return bcast ? s3r_threshold_units24(t / (uint64_t)S, layer, seed, kTagBcast + stream_word)
               : s3r_threshold_units24(t, layer, seed, kTagS3R + stream_word);
}

// Independent-SR threshold of one 32-bit word, in units of 2^-24: 2*(w>>9)+1.
__device__ __forceinline__ int32_t sr_units24(uint32_t w) { return (int32_t)(((w >> 9) << 1) | 1u); }

// ------------------------------------------------------------ reductions ----
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { uint32_t w = __shfl_xor(v, o, kWave); v = v > w ? v : w; }
  return v;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// 16-byte loads with the nontemporal hint, for streams read once. Regular loads of data that is
// not cached allocate in the last-level cache (MALL) and first evict, and write back, the dirty
// lines an earlier kernel's writes left there; marked loads do not, and read a cold stream about
// 1.5x faster.
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream_u4(const void* p) {
  const v4u32 t = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 ld_stream_f4(const void* p) {
  const v4f32 t = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}


// ------------------------------------------------------------- launchers ----
// Quantizer (quantize.hip).
struct QuantArgs {
  const void* G; int g_dtype; int64_t ld_g;
  const float* sx; const float* sw;
  int8_t* Q; int64_t ld_q;
  float* delta;
  int32_t* code_colsum;
  float* ec_row; float* ec_col; float* ec_mean;
  uint32_t* flags;
  int64_t T, D, S;
  int mode, ec, scale;
  uint32_t layer; uint64_t seed;
  uint32_t stream;           // threshold stream (0: the shared draw)
  char* ws;
  const uint32_t* amax_in;   // per-tensor amax bits already known on the device, or null
};
size_t quant_workspace(int64_t T, int64_t D, int64_t S, int ec, int scale, bool colsum);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t st);
size_t grouped_quant_workspace(int64_t R, int64_t D, int64_t Gn, int ec, int scale, bool colsum);
hipError_t launch_grouped_quantize(const QuantArgs& a, int64_t Gn, const int64_t* offsets, hipStream_t st);

// Backward GEMMs (gemm.hip).
struct DxArgs {
  const int8_t* Q; int64_t ld_q; const float* delta; int per_token;
  const int8_t* W; int64_t ld_w;
  int64_t T, D, d_in, S;
  const float* sx; const int32_t* rW;
  const float* ec_row; const float* ec_col; const float* ec_mean; int ec;
  void* out; int out_dt; int64_t ld_out;
  char* ws;
};
struct DwArgs {
  const int8_t* Q; int64_t ld_q; const float* delta; int per_token;
  const int8_t* X; int64_t ld_x;
  int64_t T, D, d_in, S;
  const float* sw; const int32_t* xs;
  const float* ec_row; const float* ec_col; const float* ec_mean; int ec;
  void* out; int out_dt; int64_t ld_out;
  char* ws;
};
// Events to record around the next GEMM launch on this thread (measurement aid).
struct GemmTiming { hipEvent_t start = nullptr, stop = nullptr; };
GemmTiming& gemm_timing();

size_t dx_workspace(int64_t T, int64_t D, int64_t d_in, int64_t S, int ec);
size_t dw_workspace(int64_t T, int64_t D, int64_t d_in, int64_t S, int ec, int per_token);
hipError_t launch_backward_dx(const DxArgs& a, hipStream_t st);
hipError_t launch_backward_dw(const DwArgs& a, hipStream_t st);
// Two per-tensor dW products of one shape sharing X (a0.X == a1.X, a0.ld_q == a1.ld_q), one GEMM launch;
// each DwArgs brings its own workspace.
hipError_t launch_backward_dw_pair(const DwArgs& a0, const DwArgs& a1, hipStream_t st);
size_t grouped_dx_workspace(int64_t R, int64_t D, int64_t d_in, int64_t G, int ec);
size_t grouped_dw_workspace(int64_t R, int64_t D, int64_t d_in, int64_t G, int ec);
hipError_t launch_grouped_backward_dx(const DxArgs& a, int64_t G, const int64_t* offsets, int64_t w_stride,
                                      uint32_t* flags, hipStream_t st);
hipError_t launch_grouped_backward_dw(const DwArgs& a, int64_t G, const int64_t* offsets, int64_t out_stride,
                                     uint32_t* flags, hipStream_t st);

// MXFP4 variant (mx.hip).
struct MxQuantArgs {
  const void* G; int g_dtype; int64_t ld_g;
  int64_t T, D, S;
  int mode, ec; uint32_t layer; uint64_t seed; uint32_t stream;
  uint8_t* Qh; int64_t ld_qh; uint8_t* Qhs; int64_t ld_qhs;
  uint8_t* Qt; int64_t ld_qt; uint8_t* Qts; int64_t ld_qts;
  float* ec_row_h; float* ec_col_h; float* ec_mean_h;
  float* ec_row_t; float* ec_col_t; float* ec_mean_t;
  uint32_t* flags; char* ws;
};
struct MxOperandArgs {
  const void* M; int dtype; int64_t ld; int64_t R, C, S;
  uint8_t* Mt; int64_t ld_t; uint8_t* Mts; int64_t ld_ts;
  float* colsum; uint32_t* flags; char* ws;
};
struct MxBwArgs {        // out [rows x d_in] = A [rows x K] . B [d_in x K]^T - correction
  const uint8_t* A; int64_t lda; const uint8_t* As; int64_t ldas;
  const uint8_t* B; int64_t ldb; const uint8_t* Bs; int64_t ldbs;
  int64_t T, D, d_in, S, K;
  int ec;
  const float* vcol;     // dX: r_W [d_in]; dW: xs [B x d_in]
  const float* ec_row; const float* ec_col; const float* ec_mean;
  float* out; int64_t ld_out; char* ws;
};
size_t mx_quant_workspace(int64_t T, int64_t D, int ec);
size_t mx_operand_workspace(int64_t R, int64_t C);
size_t mx_backward_workspace(int64_t T, int64_t D, int64_t d_in, int64_t B);
hipError_t launch_mx_quantize(const MxQuantArgs& a, hipStream_t st);
hipError_t launch_mx_operand(const MxOperandArgs& a, hipStream_t st);
hipError_t launch_mx_backward_dx(const MxBwArgs& a, hipStream_t st);
hipError_t launch_mx_backward_dw(const MxBwArgs& a, hipStream_t st);

// SwiGLU backward glue (swiglu.hip).
hipError_t launch_swiglu_backward(int64_t T, int64_t F, const float* dH, int64_t ld_dh, const uint16_t* Ag,
                                  const uint16_t* Au, int64_t ld_a, uint16_t* Gg, uint16_t* Gu, int64_t ld_g,
                                  hipStream_t st);

size_t swiglu_amax_workspace(int64_t T, int64_t F);
// Gg == Gu == nullptr: the per-tensor maxima only, nothing else written.
hipError_t launch_swiglu_backward_amax(int64_t T, int64_t F, const float* dH, int64_t ld_dh, const uint16_t* Ag,
                                       const uint16_t* Au, int64_t ld_a, uint16_t* Gg, uint16_t* Gu, int64_t ld_g,
                                       const float* sx, const float* swg, const float* swu, uint32_t* amax_bits,
                                       char* ws, hipStream_t st);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The gate and up projections' quantizers with the SwiGLU glue computed in them (quantize.hip): G_gate
// and G_up are never written.  Per-tensor steps; the two quantizers share the shape, mode and correction
// and may differ in layer, seed and threshold stream.
struct SwigluQuantArgs {
  const float* dH; int64_t ld_dh; const uint16_t* Ag; const uint16_t* Au; int64_t ld_a;
  const float* sx; const float* sw[2];              // [0] gate, [1] up
  int8_t* Q[2]; int64_t ld_q; float* delta[2];
  float* ec_row[2]; float* ec_col[2]; float* ec_mean[2];
  uint32_t* flags;
  int64_t T, D, S;
  int mode, ec;
  uint32_t layer[2]; uint64_t seed[2]; uint32_t stream[2];
  char* ws;
};
size_t swiglu_quant_workspace(int64_t T, int64_t D, int64_t S, int ec);
hipError_t launch_swiglu_quantize(const SwigluQuantArgs& a, hipStream_t st);

// Grouped problems (groups.hip): tables derived on the device from the group
// offsets, in a workspace region of group_tables_bytes(G).  At most kMaxGroups groups.
constexpr int64_t kMaxGroups = 4096;
struct GroupTables {
  const int64_t* offsets;   // [G+1] (caller's, device)
  int64_t G;
  int32_t* tiles64;         // [G+1] prefix sums of ceil(n_e / 64)
  int32_t* tiles256;        // [G+1] prefix sums of ceil(n_e / 256)
  int32_t* order;           // [G] groups by descending rows
  uint32_t* status;         // [1] 0: offsets valid; 1: invalid (tables empty)
  uint32_t* amax;           // [G] cleared; the grouped quantizer's per-group amax bits
};
size_t group_tables_bytes(int64_t G);
GroupTables group_tables(char* base, int64_t G, const int64_t* offsets);
// empty_delta (a grouped per-tensor quantizer's steps, or null): 1 for every empty group.
hipError_t launch_group_tables(const GroupTables& t, int64_t R, uint32_t* flags, hipStream_t st,
                               float* empty_delta = nullptr);

// The group e with tiles[e] <= i < tiles[e+1], its first tile tiles[e] and its
// rows [offsets[e], offsets[e+1]), found by the whole wave in a 64-ary search:
// one round of loads per level and a ballot across the lanes, one level for up
// to 64 groups.  The last level also loads the candidates' offsets, so group
// and rows arrive in one round of loads instead of a chain of dependent ones.
// Every lane of the wave must be active; the result is wave-uniform.
// e = -1 past the last tile of the last group.
struct GroupHit { int e; int32_t t0; int64_t r0, r1; };
__device__ __forceinline__ GroupHit find_group_wave(const int32_t* __restrict__ tiles,
                                                    const int64_t* __restrict__ offsets, int64_t G, int64_t i) {
  const int lane = (int)(threadIdx.x & 63);
  const int32_t total = tiles[G];
  int lo = 0, hi = (int)G;                 // tiles[lo] <= i < tiles[hi] when i < total
  while (hi - lo > 64) {
    const int step = (hi - lo + 63) / 64;
    const int c = lo + lane * step;
    const uint64_t m = __builtin_amdgcn_ballot_w64(c < hi && tiles[c] <= i);   // a prefix of the lanes
    const int last = m ? 63 - __builtin_clzll(m) : 0;
    lo += last * step;
    hi = min(lo + step, hi);
  }
  const int c = lo + lane;
  int32_t tc = 0;
  int64_t o0 = 0, o1 = 0;
  bool hit = false;
  if (c < hi) {
    tc = tiles[c];
    o0 = offsets[c];
    o1 = offsets[c + 1];
    hit = tc <= i;
  }
  const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
  const int last = m ? 63 - __builtin_clzll(m) : 0;
  GroupHit h;
  h.e = (m != 0 && i < total) ? lo + last : -1;
  h.t0 = __builtin_amdgcn_readlane(tc, last);
  h.r0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(o0 >> 32), last) << 32) |
                   (uint32_t)__builtin_amdgcn_readlane((int)o0, last));
  h.r1 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(o1 >> 32), last) << 32) |
                   (uint32_t)__builtin_amdgcn_readlane((int)o1, last));
  return h;
}

}  // namespace s3r
