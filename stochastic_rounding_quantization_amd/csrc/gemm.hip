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
// 2 x 2, each 128 x 128 = 4 x 4 blocks of v_mfma_i32_32x32x32_i8), K step 64.
// Operands go from global memory straight into LDS (buffer_load_dwordx4 with
// the LDS bit, 16 bytes per lane, lane l landing at 16*l of a 1 KB block);
// nothing is transposed on the way in.  Two rings fill the CU's 160 KB:
//   M-contiguous A (dW): five stages of 32 KB, each one K step of A and B,
//     loads issued four steps ahead.
//   K-contiguous A (dX): A in units of two K steps (whole 128-byte lines per
//     row), three units of 32 KB beside four B stages of 16 KB.
//   M/N-contiguous tiles: 64 k-rows x 256 B; chunk c of k-row r sits at
//     c ^ swz_m(r), swz_m(r) = (r & 7) << 1: a half-wave of a transpose read
//     takes an aligned pair of chunks from each of 8 consecutive k-rows, and
//     the swizzle puts those 8 pairs in the 8 different 32-byte bank groups
//     (rocprofv3 counts no LDS bank conflicts); fragments are read with two
//     ds_read_b64_tr_b8: within each
//     16-lane group, lane L fetches 8 bytes of k-row kb + L/2 at column
//     nb + 8(L%2), and the hardware hands lane i the bytes of column nb + i
//     from the 8 k-rows, so a lane ends up with 16 consecutive k of one
//     column, the same k order a K-contiguous ds_read_b128 gives.
// The chunk position is chosen on the global side (which lane loads which
// chunk), so the swizzles cost nothing at load time, and the 16-byte reads of
// 16 consecutive rows / the 8 k-rows of a transpose read hit distinct banks.
// The descriptors' range checks return zeros past the operands' ends.
// Workgroups are numbered so that the consecutive tiles of one XCD share rows
// of A and columns of B (grouped order), for L2 reuse.
#include "s3r_internal.h"

namespace s3r {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmThreads = 256;
constexpr int kStageBytes = 32768;    // A tile (16 KB) + B tile (16 KB)
constexpr int kHalf = 16384;
constexpr int kGroupM = 8;            // grouped tile order: 8 tile-rows per group
constexpr int kNumXcd = 8;
// Cache-policy bits of the epilogue's output stores: nontemporal (bit 1 on gfx950). The outputs are
// written once and not read back by this kernel; unmarked, they would fill the last-level cache with
// dirty lines that the next kernels' reads must first evict.
constexpr int kStoreNT = 2;

// The pipeline stages are separate LDS objects so that the compiler can tell a
// stage being read from the stages being filled by in-flight DMA.
constexpr int kStages = 5;            // 5 x 32 KB = the CU's 160 KB of LDS
__shared__ __attribute__((aligned(1024))) uint8_t g_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage1[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage2[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage3[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage4[kStageBytes];

template <int S>
__device__ __forceinline__ uint8_t* stage() {
  if constexpr (S == 0) return g_stage0;
  else if constexpr (S == 1) return g_stage1;
  else if constexpr (S == 2) return g_stage2;
  else if constexpr (S == 3) return g_stage3;
  else return g_stage4;
}

// With a K-contiguous A the rows of A bring 64 bytes per K step, half a cache
// line: in one-step stages every line of A is fetched twice, in two halves,
// which costs the dX GEMM 50 % more L2 requests than the dW GEMM and ~10 %
// of its time.  That kernel keeps A in units of two K steps instead (256 rows
// x 128 bytes, whole lines), loaded half a unit (128 rows) per K step, beside
// B stages of one K step: three A units and four B stages fill the 160 KB.
constexpr int kUnitBytes = 32768, kBStageBytes = 16384;
__shared__ __attribute__((aligned(1024))) uint8_t g_unit0[kUnitBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_unit1[kUnitBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_unit2[kUnitBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_bst0[kBStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_bst1[kBStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_bst2[kBStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_bst3[kBStageBytes];

template <int U>
__device__ __forceinline__ uint8_t* a_unit() {
  if constexpr (U == 0) return g_unit0;
  else if constexpr (U == 1) return g_unit1;
  else return g_unit2;
}
template <int S>
__device__ __forceinline__ uint8_t* b_stage() {
  if constexpr (S == 0) return g_bst0;
  else if constexpr (S == 1) return g_bst1;
  else if constexpr (S == 2) return g_bst2;
  else return g_bst3;
}

struct EpiParams {
  const float* delta; int per_token;
  const float* row_scale;            // s_x (dX) or s_w (dW); null = 1
  int ec;                            // apply the correction
  // dX: rW [N] int32, ec_row [M], ec_mean [B], v [B x N] f32
  // dW: ebar [B x M] f32 (row index j), xs [B x N] int32, u [N] f32
  const int32_t* colsum; const float* ec_row; const float* ec_mean; const float* vec;
  const float* ebar; const float* u;
  const float* colstep;              // dW with per-token steps: the per-column step c [N] of Zq
  int64_t S, B;
  void* out; int64_t ld_out; int out_i32;
};

struct GemmParams {
  const int8_t* A; int64_t lda;
  const int8_t* B; int64_t ldb;
  int64_t M, N, K;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ int swz_m(int r) { return (r & 7) << 1; }

// s_waitcnt immediates (gfx9 encoding): wait for at most n vector-memory ops / no LDS ops.
#define S3R_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x70 | 0xF00)
#define S3R_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// ------------------------------------------------ tile loads into a stage ----
// Loads are buffer loads with the LDS bit (16 bytes per lane, lane l landing at
// 16*l of a 1 KB block of the stage) through a buffer descriptor that spans the
// whole operand matrix, rows * ld bytes.  The hardware's range check returns
// zeros past the end of the matrix.  Every operand's K dimension is either its
// row index (M/N-contiguous operands) or is paired with one that is, so k >= K
// always multiplies a zero; reads past the M or N edge inside the matrix only
// reach output rows or columns that are never stored.
// Each wave fills 4 of the 16 1-KB blocks of the A tile and 4 of the B tile.
// Block blk, lane l (M/N-contiguous): k-row = 4 blk + l/16, position p = l%16
// holds chunk c = p ^ swz_m(k-row).  (The K-contiguous A has its own ring below.)
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit dword format (gfx9 family)

// The DMAs are issued as inline assembly, which the compiler does not see as
// LDS writes; otherwise its tracking of the DMA targets drains every load in
// flight (vmcnt(0)) before many of the fragment reads.  Every ordering the
// rings need is explicit: the waits, the barrier, and a fixed instruction
// order inside a K step (sched_barrier after each MFMA group).
__device__ __forceinline__ v4i rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return v4i{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), (int)bytes, kRsrcWord3};
}

// One 1 KB DMA: 16 bytes per lane from rsrc + voff + soff to LDS address lds + 16 * lane.
// M0 holds the LDS address; no compiler-generated instruction of this file
// reads or writes M0 (a reserved register, which a clobber list cannot name;
// the CPU tests check the compiled assembly for it).
__device__ __forceinline__ void dma_1k(v4i rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff));
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

struct LoadMap {           // per-thread byte offsets (tile origin + position), for 4 blocks of A and of B
  uint32_t a_off[4], b_off[4];
  uint32_t a_step, b_step; // advance per K step (uniform)
  v4i ra, rb;              // buffer descriptors (raw words)
};

__device__ __forceinline__ LoadMap make_loadmap(const GemmParams& g, int64_t m0, int64_t n0) {
  LoadMap m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int blk = wave * 4 + q;
    const int kr = blk * 4 + (lane >> 4);
    const int c = (lane & 15) ^ swz_m(kr);
    m.a_off[q] = (uint32_t)(kr * g.lda + m0 + c * 16);
    m.b_off[q] = (uint32_t)(kr * g.ldb + n0 + c * 16);
  }
  m.a_step = (uint32_t)(BK * g.lda);
  m.b_step = (uint32_t)(BK * g.ldb);
  m.ra = rsrc_words(g.A, (uint32_t)(g.K * g.lda));
  m.rb = rsrc_words(g.B, (uint32_t)(g.K * g.ldb));
  return m;
}

template <int S>
__device__ __forceinline__ void stage_dma(const LoadMap& m, int q, int wave, int kt) {
  if (q < 4)
    dma_1k(m.ra, lds_addr(stage<S>()) + (uint32_t)(wave * 4 + q) * 1024u, m.a_off[q], (uint32_t)kt * m.a_step);
  else
    dma_1k(m.rb, lds_addr(stage<S>()) + (uint32_t)(kHalf + (wave * 4 + q - 4) * 1024), m.b_off[q - 4],
           (uint32_t)kt * m.b_step);
}
template <int S>
__device__ __forceinline__ void load_stage(const LoadMap& m, int kt) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // LDS DMA base must be wave-uniform
#pragma unroll
  for (int q = 0; q < 8; ++q) stage_dma<S>(m, q, wave, kt);
}

// ------------------------------------------------------------ fragments ----
struct FragMap {
  int a_t[4];      // M-contiguous A: byte offset of block i (kk adds 8192, second read 2048)
  int b_t[4];      // N-contiguous B (within the B half)
};

__device__ __forceinline__ FragMap make_fragmap() {
  FragMap f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int grp = lane >> 4, L = lane & 15;
  const int krow = 16 * (grp >> 1) + (L >> 1);        // k-row for kk = 0, first read
  const int x = swz_m(krow);                           // also the swizzle of krow + 8 and krow + 32
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ca = (wm * 128 + i * 32 + 16 * (grp & 1)) >> 4;
    f.a_t[i] = krow * 256 + ((ca ^ x) << 4) + 8 * (L & 1);
    const int cb = (wn * 128 + i * 32 + 16 * (grp & 1)) >> 4;
    f.b_t[i] = krow * 256 + ((cb ^ x) << 4) + 8 * (L & 1);
  }
  return f;
}

__device__ __forceinline__ v4i tr_pair(const uint8_t* p) {
  const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
  const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p + 2048));   // k-rows + 8
  return v4i{lo.x, lo.y, hi.x, hi.y};
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100, kSgVmem = 0x010;

struct Frags { v4i a[4], b[4]; };

// Fragments of half-step kk (k 32kk .. 32kk+31) of stage S.
template <int S>
__device__ __forceinline__ void read_frags(const FragMap& f, int kk, Frags& fr) {
  const uint8_t* st = stage<S>();
#pragma unroll
  for (int i = 0; i < 4; ++i) fr.a[i] = tr_pair(st + f.a_t[i] + kk * 8192);
#pragma unroll
  for (int j = 0; j < 4; ++j) fr.b[j] = tr_pair(st + kHalf + f.b_t[j] + kk * 8192);
}

__device__ __forceinline__ void mfma16(const Frags& fr, v16i (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fr.a[i], fr.b[j], acc[i][j], 0, 0, 0);
}

// 16 MFMAs with the NR LDS reads issued in between, one after each MFMA, and
// (NV > 0) the stage refill's NV buffer loads spread over the MFMAs, so the
// memory pipeline is never handed a burst that stalls instruction issue.
template <int NR, int NV>
__device__ __forceinline__ void interleave_schedule() {
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if (x < NR) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    if (NV > 0 && (x % (16 / (NV > 0 ? NV : 1))) == 0) __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
  }
}

// One K step on stage S = kt % kStages.  On entry `cur` holds the stage's
// first half-step fragments.  The barrier publishes stage kt+1 (this wave has
// waited for its own loads of it) and retires stage kt-1, which is refilled
// with step kt+4.  First half-step: MFMA x on `cur`, then fragment read x of
// the second half-step, and after every other MFMA one of the refill's 8
// DMAs.  Second half-step: MFMA x on `nxt`, then fragment read x of the next
// stage's first half-step.  Read x < 8 is a transposed half of A block x/2,
// the rest of B block (x-8)/2.
template <int S>
__device__ __forceinline__ void stage_read(const FragMap& f, int kk, int x, Frags& fr) {
  const int blk = (x & 7) >> 1, hi = x & 1;
  const uint8_t* p = x < 8 ? stage<S>() + f.a_t[blk] : stage<S>() + kHalf + f.b_t[blk];
  const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p + kk * 8192 + hi * 2048));
  v4i& d = x < 8 ? fr.a[blk] : fr.b[blk];
  if (hi) { d.z = v.x; d.w = v.y; }
  else { d.x = v.x; d.y = v.y; }
}
template <int S>
__device__ __forceinline__ void k_step(const LoadMap& lm, const FragMap& fm, int kt, Frags& cur,
                                       v16i (&acc)[4][4]) {
  // Every step refills one stage, also past the last step (those loads read past
  // the end of the data or land in retired stages), so exactly the loads of
  // stages kt+2 and kt+3 may still be in flight here.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  S3R_WAIT_VM(16);
  S3R_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frags nxt;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    acc[x >> 2][x & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[x >> 2], cur.b[x & 3], acc[x >> 2][x & 3], 0, 0, 0);
    stage_read<S>(fm, 1, x, nxt);
    if ((x & 1) == 0) stage_dma<(S + 4) % kStages>(lm, x >> 1, wave, kt + 4);
    __builtin_amdgcn_sched_barrier(0);
  }
  // next stage's first fragments (after the last step this reads a stale stage; unused)
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    acc[x >> 2][x & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(nxt.a[x >> 2], nxt.b[x & 3], acc[x >> 2][x & 3], 0, 0, 0);
    stage_read<(S + 1) % kStages>(fm, 0, x, cur);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------- the unit ring (K-contiguous A) ----
// A unit holds K steps 2u and 2u+1 of the tile's 256 rows: half h (16 KB) is
// rows 128h .. 128h+127, each row 128 bytes (k 128u .. 128u+127), and 16-byte
// chunk c of local row r sits at position c ^ swz_u(r), swz_u(r) = (r >> 1) & 7,
// so the sixteen rows a ds_read_b128 quarter-wave touches hit sixteen different
// bank groups.  Each 1 KB DMA block is eight whole rows: eight lanes fetch one
// 128-byte line.  Wave wm only reads half wm.
// Schedule: K step kt computes from unit kt/2 (slot (kt/2) % 3) and B stage kt
// (slot kt % 4), and refills B stage kt+3 and half kt%2 of unit kt/2+2; the
// slots refilled are those of B stage kt-1 and unit kt/2-1, retired by the
// barrier.  Data for step kt+1 was issued at steps kt-2 or earlier, so the
// loads of one step (8 per wave) may be in flight at the wait.
__device__ __forceinline__ int swz_u(int r) { return (r >> 1) & 7; }

// Its DMAs are the inline assembly above (with seven DMA targets the compiler's
// own tracking drained the loads in flight before most fragment reads).
struct UnitMap {
  uint32_t a_off[2][4], b_off[4];
  uint32_t b_step;
  v4i ra, rb;            // buffer descriptors (raw words)
};

__device__ __forceinline__ UnitMap make_unitmap(const GemmParams& g, int64_t m0, int64_t n0) {
  UnitMap m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int blk = wave * 4 + q;                  // 1 KB block of a 16 KB half or B stage
    const int row = blk * 8 + (lane >> 3);         // local row of the half
    const int c = (lane & 7) ^ swz_u(row);
#pragma unroll
    for (int h = 0; h < 2; ++h) m.a_off[h][q] = (uint32_t)((m0 + h * 128 + row) * g.lda + c * 16);
    const int kr = blk * 4 + (lane >> 4);
    const int cb = (lane & 15) ^ swz_m(kr);
    m.b_off[q] = (uint32_t)(kr * g.ldb + n0 + cb * 16);
  }
  m.b_step = (uint32_t)(BK * g.ldb);
  m.ra = rsrc_words(g.A, (uint32_t)(g.M * g.lda));
  m.rb = rsrc_words(g.B, (uint32_t)(g.K * g.ldb));
  return m;
}

// DMA q (0..7) of a K step: q < 4 fill B stage SB with K step kt_b, q >= 4 fill
// half H of unit slot SU with unit u.
template <int SB, int SU, int H>
__device__ __forceinline__ void unit_dma(const UnitMap& m, int q, int wave, int kt_b, int u) {
  if (q < 4)
    dma_1k(m.rb, lds_addr(b_stage<SB>()) + (uint32_t)(wave * 4 + q) * 1024u, m.b_off[q], (uint32_t)kt_b * m.b_step);
  else
    dma_1k(m.ra, lds_addr(a_unit<SU>()) + (uint32_t)(H * 16384 + (wave * 4 + q - 4) * 1024), m.a_off[H][q - 4],
           (uint32_t)u * 128u);
}
template <int SB>
__device__ __forceinline__ void load_b_stage(const UnitMap& m, int kt) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < 4; ++q) unit_dma<SB, 0, 0>(m, q, wave, kt, 0);
}
template <int SU, int H>
__device__ __forceinline__ void load_a_half(const UnitMap& m, int u) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 4; q < 8; ++q) unit_dma<0, SU, H>(m, q, wave, 0, u);
}

struct UnitFragMap {
  int a[2][2];     // A: byte offset in the unit for (step parity, half-step kk); block i adds i * 4096
  int b_t[4];      // B: as FragMap::b_t, within a B stage
};

__device__ __forceinline__ UnitFragMap make_unit_fragmap() {
  UnitFragMap f;
  const FragMap t = make_fragmap();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1;
  const int r = lane & 31;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = sub * 4 + kk * 2 + (lane >> 5);
      f.a[sub][kk] = wm * 16384 + r * 128 + ((c ^ swz_u(r)) << 4);
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b_t[j] = t.b_t[j];
  return f;
}

// Fragment read x (0..11) of half-step kk: x < 4 the A block x, then the two
// transposed halves of B block (x - 4) / 2.
template <int SU, int SUB, int SB>
__device__ __forceinline__ void unit_read(const UnitFragMap& f, int kk, int x, Frags& fr) {
  if (x < 4) {
    fr.a[x] = *reinterpret_cast<const v4i*>(a_unit<SU>() + f.a[SUB][kk] + x * 4096);
  } else {
    const int j = (x - 4) >> 1, hi = (x - 4) & 1;
    const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_v2i*)(b_stage<SB>() + f.b_t[j] + kk * 8192 + hi * 2048));
    if (hi) { fr.b[j].z = v.x; fr.b[j].w = v.y; }
    else { fr.b[j].x = v.x; fr.b[j].y = v.y; }
  }
}
template <int SU, int SUB, int SB>
__device__ __forceinline__ void read_unit_frags(const UnitFragMap& f, int kk, Frags& fr) {
#pragma unroll
  for (int x = 0; x < 12; ++x) unit_read<SU, SUB, SB>(f, kk, x, fr);
}

// K step kt with P = kt % 12 (the schedule repeats every 12 steps).  First
// half-step: MFMA x on `cur`, then fragment read x of the second half-step, and
// after every other MFMA one of the step's 8 DMAs.  Second half-step: MFMA x on
// `nxt`, then fragment read x of the next step's first half-step.
template <int P>
__device__ __forceinline__ void unit_step(const UnitMap& lm, const UnitFragMap& fm, int kt, Frags& cur,
                                          v16i (&acc)[4][4]) {
  constexpr int SU = (P / 2) % 3, SUB = P % 2, SB = P % 4;
  constexpr int P1 = (P + 1) % 12;
  constexpr int SU1 = (P1 / 2) % 3, SUB1 = P1 % 2, SB1 = P1 % 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kt_b = kt + 3, u = (kt >> 1) + 2;
  S3R_WAIT_VM(8);
  S3R_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frags nxt;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    acc[x >> 2][x & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[x >> 2], cur.b[x & 3], acc[x >> 2][x & 3], 0, 0, 0);
    if (x < 12) unit_read<SU, SUB, SB>(fm, 1, x, nxt);
    if ((x & 1) == 0) unit_dma<(P + 3) % 4, (P / 2 + 2) % 3, SUB>(lm, x >> 1, wave, kt_b, u);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the next step's first fragments (after the last step this reads a stale slot; unused)
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    acc[x >> 2][x & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(nxt.a[x >> 2], nxt.b[x & 3], acc[x >> 2][x & 3], 0, 0, 0);
    if (x < 12) unit_read<SU1, SUB1, SB1>(fm, 0, x, cur);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------- epilogue ----
// 32x32 block output layout: lane l, register r -> row (r/4)*8 + (l/32)*4 + r%4, column l%32.
// Stores go through a buffer descriptor over the tile's rows of the output
// (rows past M fall outside it and are dropped by the range check); columns
// past N are masked per column block.  Per-row byte offsets are uniform.
// EPI_DXA: dX added into the output.  EPI_DWC: dW whose B operand is the per-column
// requantized Zq of per-token steps, dequantized by its column step c[n].
enum { EPI_RAW = 0, EPI_DX = 1, EPI_DW = 2, EPI_DXA = 3, EPI_DWC = 4 };
__host__ __device__ constexpr bool is_dx(int epi) { return epi == EPI_DX || epi == EPI_DXA; }
__host__ __device__ constexpr bool is_dw(int epi) { return epi == EPI_DW || epi == EPI_DWC; }
constexpr int kMaxB = 8;   // examples whose dW correction terms the epilogue applies

__device__ __forceinline__ int row_in_block(int r) { return (r >> 2) * 8 + (r & 3); }

// NB: number of examples whose dW terms are applied here (a compile-time bound,
// so the per-element sum has no runtime trip count; slots b >= B hold zeros).
// DROP: columns past N are not skipped by a branch around their stores but given an offset past the
// output descriptor's range, where the hardware drops the store.  Measured faster for the grouped dW,
// whose narrow outputs leave many tiles partial in N, and slower for the dense GEMMs, whose tiles are
// whole.  Needs (rows + 127) * ld_out * 4 < 2^32 (the C ABI bounds ld_out for the grouped dW).
// NJ: 32-column blocks per wave (4 in the 256 x 256 tiles, 2 in the 256 x 128 tiles of the grouped dW).
// Per-column factors of a lane's NJ column blocks: A (dX: r_W[n]; dW: u[n]), V (dX: v_b[n] of the tile's
// example), B (dW: xs_b[n], slots past B hold 0), S (per-token dW: the column's step).  Every lane loads from
// a valid column (its own, or column 0 past N, whose value is then discarded).
template <int NB, int NJ> struct ColF { float A[NJ], V[NJ], B[NB][NJ], S[NJ]; };

template <int EPI, bool EC, int NB, int NJ>
__device__ __forceinline__ void load_cols(const GemmParams& g, const EpiParams& ep, int64_t m0, int64_t n0,
                                          ColF<NB, NJ>& c) {
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t n = n0 + wn * (NJ * 32) + j * 32 + (lane & 31);
    const int64_t nc = n < g.N ? n : 0;
    c.A[j] = 0.f; c.V[j] = 0.f; c.S[j] = 1.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) c.B[b][j] = 0.f;
    if constexpr (EPI == EPI_DWC) c.S[j] = ep.colstep[nc];
    if constexpr (EC && is_dx(EPI)) {
      c.A[j] = (float)ep.colsum[nc];
      c.V[j] = ep.vec[(m0 / ep.S) * g.N + nc];       // the example of the tile's first row (unused when gathered)
    } else if constexpr (EC && is_dw(EPI)) {
      c.A[j] = ep.u[nc];
#pragma unroll
      for (int b = 0; b < NB; ++b) c.B[b][j] = (float)ep.colsum[(b < ep.B ? b : 0) * g.N + nc] * (b < ep.B ? 1.f : 0.f);
    }
  }
}

// pre (optional): the column factors, loaded by the caller ahead of time; otherwise they are loaded here.
template <int EPI, bool EC, bool GATHER, int NB, bool DROP = false, int NJ = 4>
__device__ __forceinline__ void epilogue(const GemmParams& g, const EpiParams& ep, int64_t m0, int64_t n0,
                                         const float4* rowf, const float* roweb, v16i (&acc)[4][NJ],
                                         const ColF<NB, NJ>* pre = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int rows_here = (int)min((int64_t)BM, g.M - m0);
  const uint32_t esz = 4;
  const uint32_t ld4 = (uint32_t)ep.ld_out * esz;
  __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((char*)ep.out + (m0 * ep.ld_out) * esz), (short)0, (int)((uint32_t)rows_here * ld4), kRsrcWord3);
  // rowf: per-row factors; roweb (dW): ebar[b][row] / s_w[row]
  const int lane_row = wm * 128 + (lane >> 5) * 4;                  // + i*32 + row_in_block(r)

  // per-column values of this lane, one per column block j, loaded outside any branch (or ahead of time by
  // the caller) and waited for once here: a load still pending inside the store loop would make each group
  // of stores wait for every store before it (vmcnt counts stores too).
  // DROP: a column past N gets an offset past the descriptor's range, where the hardware drops the store.
  ColF<NB, NJ> cf;
  if (pre) cf = *pre;
  else load_cols<EPI, EC, NB, NJ>(g, ep, m0, n0, cf);
  const float (&colA)[NJ] = cf.A;
  const float (&colV)[NJ] = cf.V;
  const float (&colS)[NJ] = cf.S;
  const float (&colB)[NB][NJ] = cf.B;
  bool n_ok[NJ];
  uint32_t voff[NJ];
  const uint32_t off_none = (uint32_t)rows_here * ld4;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t n = n0 + wn * (NJ * 32) + j * 32 + (lane & 31);
    n_ok[j] = n < g.N;
    voff[j] = (DROP && !n_ok[j]) ? off_none : (uint32_t)(lane_row * ld4 + n * esz);
  }
  S3R_WAIT_VM(0);

  // EPI_DXA: the current output values of a block-row, loaded one block-row ahead: the loads of
  // block-row i+1 are issued before the stores of block-row i, so waiting for them does not wait
  // for those stores (vmcnt counts loads and stores in issue order)
  float old[2][4][NJ][4];
  auto load_old = [&](int i, float (&dst)[4][NJ][4]) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          dst[rq][j][rr] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              ro, voff[j], (uint32_t)(i * 32 + rq * 8 + rr) * ld4, 0));
  };
  if constexpr (EPI == EPI_DXA) load_old(0, old[0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (EPI == EPI_DXA)
      if (i + 1 < 4) load_old(i + 1, old[(i + 1) & 1]);
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      // four consecutive rows of this lane: lr = lane_row + i*32 + rq*8 + rr
      float4 f[4];
      float eb[4][NB];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int lr = lane_row + i * 32 + rq * 8 + rr;
        if constexpr (EPI != EPI_RAW) f[rr] = rowf[lr];
        if constexpr (is_dw(EPI) && EC) {
#pragma unroll
          for (int b = 0; b < NB; ++b) eb[rr][b] = roweb[b * BM + lr];
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (!DROP && !n_ok[j]) continue;
        float gv[4];
        if constexpr (is_dx(EPI) && EC && GATHER) {
          const int64_t n = n0 + wn * (NJ * 32) + j * 32 + (lane & 31);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) gv[rr] = ep.vec[(int64_t)__float_as_int(f[rr].w) * g.N + n];
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = rq * 4 + rr;
          const int32_t v = acc[i][j][r];
          const uint32_t soff = (uint32_t)(i * 32 + rq * 8 + rr) * ld4;
          if constexpr (EPI == EPI_RAW) {
            __builtin_amdgcn_raw_buffer_store_b32(v, ro, voff[j], soff, 0);
          } else {
            float corr = 0.f;
            if constexpr (EC && is_dx(EPI)) corr = fmaf(f[rr].z, colA[j], f[rr].y * (GATHER ? gv[rr] : colV[j]));
            if constexpr (EC && is_dw(EPI)) {
              float t = f[rr].y * colA[j];
#pragma unroll
              for (int b = 0; b < NB; ++b) t = fmaf(eb[rr][b], colB[b][j], t);
              corr = t;
            }
            const float scale = EPI == EPI_DWC ? f[rr].x * colS[j] : f[rr].x;
            float o = fmaf(scale, (float)v, -corr);
            if constexpr (EPI == EPI_DXA) o = old[i & 1][rq][j][rr] + o;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(o), ro, voff[j], soff, kStoreNT);
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------- kernel ----
// Grouped launches (GRP != 0): rows sorted by group, group e owning rows
// [offsets[e], offsets[e+1]).  GRP_DX: a row tile of one group's Q against
// its own weight codes (B + e * b_stride); the grid is an upper bound on the
// groups' row tiles times the column tiles.  GRP_DW (gemm_dw128_kernel): one
// output matrix per group (out + e * out_stride), K = the group's rows; groups
// are taken largest first (order[]), so the longest K loops start first.  Each
// workgroup rebases the operand, output and epilogue pointers to its group,
// after which the dense kernel body runs unchanged.  Nothing runs if the
// offsets were invalid.  GRP_PAIR: two problems of one shape that share the B
// operand (the dW products of two projections of one input), tiles [0, per) of
// the first and [per, 2 per) of the second; the second's A operand and
// epilogue come from gg.
enum { GRP_NONE = 0, GRP_DX = 1, GRP_DW = 2, GRP_PAIR = 3 };
template <typename T>
__device__ __forceinline__ const T* advance(const T* p, int64_t k) { return p ? p + k : p; }
struct GroupGemm {
  const int64_t* offsets; const int32_t* tiles256; const int32_t* order; const uint32_t* status;
  int64_t G;
  int64_t b_stride;      // GRP_DX: bytes between the groups' B operands
  int64_t out_stride;    // GRP_DW: elements between the groups' outputs
  int tiles_m_all;       // GRP_DX: the grid's row-tile bound
  const int8_t* A2;      // GRP_PAIR: the second problem's A operand and epilogue
  EpiParams ep2;
};

static_assert(BM == kGemmThreads, "the GEMM kernels load one output row's epilogue factors per thread");

template <bool A_KMAJOR, int EPI, bool EC, int NB, int GRP = GRP_NONE>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_i8_kernel(GemmParams g, EpiParams ep, GroupGemm gg) {
  int tm, tn;
  if constexpr (GRP == GRP_NONE) {
    // XCD-aware numbering: hardware block ids go round-robin over the 8 XCDs;
    // give each XCD a contiguous range of logical tiles.
    const int nblocks = g.tiles_m * g.tiles_n;
    int bid = blockIdx.x;
    if (nblocks % kNumXcd == 0) bid = (bid % kNumXcd) * (nblocks / kNumXcd) + bid / kNumXcd;
    const int group = kGroupM * g.tiles_n;
    const int first_m = (bid / group) * kGroupM;
    const int gsz = min(g.tiles_m - first_m, kGroupM);
    tm = first_m + (bid % group) % gsz;
    tn = (bid % group) / gsz;
  } else if constexpr (GRP == GRP_DX) {
    if (gg.status[0] != 0) return;
    const int nblocks = gg.tiles_m_all * g.tiles_n;
    int bid = blockIdx.x;
    if (nblocks % kNumXcd == 0) bid = (bid % kNumXcd) * (nblocks / kNumXcd) + bid / kNumXcd;
    const int mt = bid / g.tiles_n;
    const GroupHit h = find_group_wave(gg.tiles256, gg.offsets, gg.G, mt);
    if (h.e < 0) return;
    const int e = h.e;
    const int64_t r0 = h.r0, n = h.r1 - r0;
    g.A += r0 * g.lda;
    g.M = n;
    g.B += e * gg.b_stride;
    ep.delta += e;
    ep.row_scale = advance(ep.row_scale, r0);
    ep.ec_row = advance(ep.ec_row, r0);
    ep.ec_mean = advance(ep.ec_mean, e);
    ep.colsum = advance(ep.colsum, e * g.N);
    ep.vec = advance(ep.vec, e * g.N);
    ep.out = (char*)ep.out + r0 * ep.ld_out * 4;
    ep.S = n > 0 ? n : 1;
    ep.B = 1;
    tm = mt - h.t0;
    tn = bid % g.tiles_n;
  } else {
    static_assert(GRP == GRP_PAIR, "the grouped dW runs in gemm_dw128_kernel");
    // XCD-aware numbering over both problems' tiles, then the grouped order within a problem
    const int per = g.tiles_m * g.tiles_n;
    const int nblocks = 2 * per;
    int bid = blockIdx.x;
    if (nblocks % kNumXcd == 0) bid = (bid % kNumXcd) * (nblocks / kNumXcd) + bid / kNumXcd;
    int local = bid;
    if (bid >= per) {
      local = bid - per;
      g.A = gg.A2;
      ep = gg.ep2;
    }
    const int group = kGroupM * g.tiles_n;
    const int first_m = (local / group) * kGroupM;
    const int gsz = min(g.tiles_m - first_m, kGroupM);
    tm = first_m + (local % group) % gsz;
    tn = (local % group) / gsz;
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int nk = (int)((g.K + BK - 1) / BK);

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  // The dense dX kernels load the epilogue's factors now, ahead of the ring's first loads, so their latency
  // hides behind the K loop: this thread's output row (BM == kGemmThreads) and the lane's columns.  (The
  // paired dW and the grouped dX keep their registers for the loop: there the values would spill.)
  constexpr bool PRE = A_KMAJOR && GRP == GRP_NONE && EPI != EPI_RAW;
  ColF<NB, 4> cf;
  const int64_t prow = m0 + threadIdx.x;
  const int64_t prc = prow < g.M ? prow : 0;
  float p_d = 1.f, p_s = 1.f, p_er = 0.f, p_em = 0.f, p_eb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) p_eb[b] = 0.f;
  if constexpr (PRE) {
    load_cols<EPI, EC, NB, 4>(g, ep, m0, n0, cf);
    if (ep.row_scale) p_s = ep.row_scale[prc];
    if constexpr (is_dx(EPI)) {
      p_d = ep.per_token ? ep.delta[prc] : ep.delta[0];
      if (EC) {
        p_er = ep.ec_row[prc];
        p_em = ep.ec_mean[prc / ep.S];
      }
    } else {
      p_d = ep.delta[0];
      if (EC)
#pragma unroll
        for (int b = 0; b < NB; ++b) p_eb[b] = b < ep.B ? ep.ebar[b * g.M + prc] : 0.f;
    }
  }

  if constexpr (A_KMAJOR) {
    const UnitMap lm = make_unitmap(g, m0, n0);
    const UnitFragMap fm = make_unit_fragmap();
    load_a_half<0, 0>(lm, 0);
    load_a_half<0, 1>(lm, 0);
    load_b_stage<0>(lm, 0);
    load_b_stage<1>(lm, 1);
    load_a_half<1, 0>(lm, 1);
    load_b_stage<2>(lm, 2);
    load_a_half<1, 1>(lm, 1);
    Frags cur;
    S3R_WAIT_VM(16);
    __builtin_amdgcn_s_barrier();
    read_unit_frags<0, 0, 0>(fm, 0, cur);
    for (int kt = 0; kt < nk; kt += 12) {
      unit_step<0>(lm, fm, kt, cur, acc);
      if (kt + 1 < nk) unit_step<1>(lm, fm, kt + 1, cur, acc);
      if (kt + 2 < nk) unit_step<2>(lm, fm, kt + 2, cur, acc);
      if (kt + 3 < nk) unit_step<3>(lm, fm, kt + 3, cur, acc);
      if (kt + 4 < nk) unit_step<4>(lm, fm, kt + 4, cur, acc);
      if (kt + 5 < nk) unit_step<5>(lm, fm, kt + 5, cur, acc);
      if (kt + 6 < nk) unit_step<6>(lm, fm, kt + 6, cur, acc);
      if (kt + 7 < nk) unit_step<7>(lm, fm, kt + 7, cur, acc);
      if (kt + 8 < nk) unit_step<8>(lm, fm, kt + 8, cur, acc);
      if (kt + 9 < nk) unit_step<9>(lm, fm, kt + 9, cur, acc);
      if (kt + 10 < nk) unit_step<10>(lm, fm, kt + 10, cur, acc);
      if (kt + 11 < nk) unit_step<11>(lm, fm, kt + 11, cur, acc);
    }
  } else {
    const LoadMap lm = make_loadmap(g, m0, n0);
    const FragMap fm = make_fragmap();
    load_stage<0>(lm, 0);
    load_stage<1>(lm, 1);
    load_stage<2>(lm, 2);
    load_stage<3>(lm, 3);
    Frags cur;
    S3R_WAIT_VM(24);
    __builtin_amdgcn_s_barrier();
    read_frags<0>(fm, 0, cur);
    for (int kt = 0; kt < nk; kt += kStages) {
      k_step<0>(lm, fm, kt, cur, acc);
      if (kt + 1 < nk) k_step<1>(lm, fm, kt + 1, cur, acc);
      if (kt + 2 < nk) k_step<2>(lm, fm, kt + 2, cur, acc);
      if (kt + 3 < nk) k_step<3>(lm, fm, kt + 3, cur, acc);
      if (kt + 4 < nk) k_step<4>(lm, fm, kt + 4, cur, acc);
    }
  }
  S3R_WAIT_VM(0);
  S3R_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();

  // per-row factors of the tile into LDS (the ring is free now)
  float4* rowf = reinterpret_cast<float4*>(A_KMAJOR ? g_unit0 : g_stage0);
  float* roweb = reinterpret_cast<float*>(A_KMAJOR ? g_unit1 : g_stage1);
  const int r = threadIdx.x;
  if constexpr (!PRE && EPI != EPI_RAW) {         // the row factors, loaded now
    if (ep.row_scale) p_s = ep.row_scale[prc];
    if constexpr (is_dx(EPI)) {
      p_d = ep.per_token ? ep.delta[prc] : ep.delta[0];
      if (EC) {
        p_er = ep.ec_row[prc];
        p_em = ep.ec_mean[prc / ep.S];
      }
    } else {
      p_d = ep.delta[0];
      if (EC)
#pragma unroll
        for (int b = 0; b < NB; ++b) p_eb[b] = b < ep.B ? ep.ebar[b * g.M + prc] : 0.f;
    }
  }
  if constexpr (is_dx(EPI)) {
    // x: Delta_t / s_x[t], y: 1 / s_x[t], z: (eps_t - mu_b) / s_x[t], w: example index
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (prow < g.M) {
      const float inv = ep.row_scale ? __fdiv_rn(1.f, p_s) : 1.f;
      f.x = p_d * inv;
      f.y = inv;
      if (EC) {
        f.z = (p_er - p_em) * inv;
        f.w = __int_as_float((int)(prow / ep.S));
      }
    }
    rowf[r] = f;
  } else if constexpr (is_dw(EPI)) {
    // x: Delta / s_w[j] (EPI_DWC: 1 / s_w[j], the step is per column), y: 1 / s_w[j];
    // roweb[b * BM + r] = ebar[b][j] / s_w[j]
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (prow < g.M) {
      const float inv = ep.row_scale ? __fdiv_rn(1.f, p_s) : 1.f;
      f.x = EPI == EPI_DWC ? inv : p_d * inv;
      f.y = inv;
    }
    if (EC)
#pragma unroll
      for (int b = 0; b < NB; ++b) roweb[b * BM + r] = (b < ep.B && prow < g.M) ? p_eb[b] * f.y : 0.f;
    rowf[r] = f;
  }
  __syncthreads();
  const ColF<NB, 4>* pre = PRE ? &cf : nullptr;
  if constexpr (is_dx(EPI) && EC) {
    const int64_t last = min(m0 + BM, g.M) - 1;
    if (m0 / ep.S == last / ep.S) epilogue<EPI, EC, false, NB>(g, ep, m0, n0, rowf, roweb, acc, pre);
    else epilogue<EPI, EC, true, NB>(g, ep, m0, n0, rowf, roweb, acc, pre);
  } else {
    epilogue<EPI, EC, false, NB>(g, ep, m0, n0, rowf, roweb, acc, pre);
  }
}

// ------------------------------------------------ dW in 256 x 128 tiles ----
// With one workgroup per CU (256 accumulator registers per lane) a CU's matrix
// cores idle while its tile's 256 KiB of f32 results are stored.  Tiles of
// 256 x 128 (four waves of 128 x 64, 128 accumulator registers) and a ring of
// three 24 KiB stages let two workgroups share a CU, so one's epilogue runs
// beside the other's K loop.  The grouped (MoE) dW, whose K loops are an
// expert's rows, and every single dW run here (measured faster at the FFN
// block's down projection, whose 896 tiles of 256 x 256 leave the last round of
// the CUs half empty: here a lone workgroup of that round has its CU to
// itself).  It costs LDS bandwidth (a K step reads 1.5x the operand bytes per
// multiply of the 256 x 256 tile), so the paired gate / up dW, whose 1792 tiles
// of 256 x 256 fill whole rounds, stays there.
// A is laid out as in the 256 x 256 ring; B's k-rows are 128 bytes (8 chunks
// of 16), chunk c of k-row r at position c ^ swz_n(r), swz_n(r) =
// ((r >> 1) & 3) << 1: the 8 k-rows of a transpose read hold two k-rows per
// 256-byte bank row, and the swizzle puts their aligned chunk pairs in the 8
// different 32-byte bank groups.  A K step loads the step two ahead into the
// slot of the step before (waiting for it at its own start), and reads each
// half-step's fragments inside the step.
constexpr int BN2 = 128;
constexpr int kStage2Bytes = 24576;      // A tile (16 KB) + B tile (8 KB)
__shared__ __attribute__((aligned(1024))) uint8_t g_nst0[kStage2Bytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_nst1[kStage2Bytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_nst2[kStage2Bytes];

template <int S>
__device__ __forceinline__ uint8_t* nstage() {
  if constexpr (S == 0) return g_nst0;
  else if constexpr (S == 1) return g_nst1;
  else return g_nst2;
}

__device__ __forceinline__ int swz_n(int r) { return ((r >> 1) & 3) << 1; }

struct LoadMap2 {          // per-thread byte offsets: 4 blocks of A, 2 of B
  uint32_t a_off[4], b_off[2];
  uint32_t a_step, b_step;
  v4i ra, rb;
};

__device__ __forceinline__ LoadMap2 make_loadmap2(const GemmParams& g, int64_t m0, int64_t n0) {
  LoadMap2 m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 4; ++q) {             // A block: 4 k-rows of 256 bytes
    const int blk = wave * 4 + q;
    const int kr = blk * 4 + (lane >> 4);
    const int c = (lane & 15) ^ swz_m(kr);
    m.a_off[q] = (uint32_t)(kr * g.lda + m0 + c * 16);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {             // B block: 8 k-rows of 128 bytes
    const int blk = wave * 2 + q;
    const int kr = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_n(kr);
    m.b_off[q] = (uint32_t)(kr * g.ldb + n0 + c * 16);
  }
  m.a_step = (uint32_t)(BK * g.lda);
  m.b_step = (uint32_t)(BK * g.ldb);
  m.ra = rsrc_words(g.A, (uint32_t)(g.K * g.lda));
  m.rb = rsrc_words(g.B, (uint32_t)(g.K * g.ldb));
  return m;
}

template <int S>
__device__ __forceinline__ void stage_dma2(const LoadMap2& m, int q, int wave, int kt) {
  if (q < 4)
    dma_1k(m.ra, lds_addr(nstage<S>()) + (uint32_t)(wave * 4 + q) * 1024u, m.a_off[q], (uint32_t)kt * m.a_step);
  else
    dma_1k(m.rb, lds_addr(nstage<S>()) + (uint32_t)(kHalf + (wave * 2 + q - 4) * 1024), m.b_off[q - 4],
           (uint32_t)kt * m.b_step);
}
template <int S>
__device__ __forceinline__ void load_stage2(const LoadMap2& m, int kt) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < 6; ++q) stage_dma2<S>(m, q, wave, kt);
}

struct FragMap2 { int a_t[4]; int b_t[2]; };

__device__ __forceinline__ FragMap2 make_fragmap2() {
  FragMap2 f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int grp = lane >> 4, L = lane & 15;
  const int krow = 16 * (grp >> 1) + (L >> 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ca = (wm * 128 + i * 32 + 16 * (grp & 1)) >> 4;
    f.a_t[i] = krow * 256 + ((ca ^ swz_m(krow)) << 4) + 8 * (L & 1);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int cb = (wn * 64 + j * 32 + 16 * (grp & 1)) >> 4;
    f.b_t[j] = krow * 128 + ((cb ^ swz_n(krow)) << 4) + 8 * (L & 1);
  }
  return f;
}

struct Frags2 { v4i a[4], b[2]; };

// Fragment x of half-step kk of stage S: x < 4 the A block x, else the B block x - 4.
template <int S>
__device__ __forceinline__ void read_frag2(const FragMap2& f, int kk, int x, Frags2& fr) {
  if (x < 4) {
    const uint8_t* p = nstage<S>() + f.a_t[x] + kk * 8192;
    const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
    const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p + 2048));   // k-rows + 8
    fr.a[x] = v4i{lo.x, lo.y, hi.x, hi.y};
  } else {
    const uint8_t* p = nstage<S>() + kHalf + f.b_t[x - 4] + kk * 4096;
    const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
    const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p + 1024));   // k-rows + 8
    fr.b[x - 4] = v4i{lo.x, lo.y, hi.x, hi.y};
  }
}

// One K step on stage S = kt % 3.  The loads of step kt+1 may still be in flight at its start; the
// barrier then publishes stage kt and retires stage kt-1, whose slot takes step kt+2.
template <int S>
__device__ __forceinline__ void k_step2(const LoadMap2& lm, const FragMap2& fm, int kt, v16i (&acc)[4][2]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  S3R_WAIT_VM(6);
  S3R_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frags2 cur, nxt;
#pragma unroll
  for (int x = 0; x < 6; ++x) read_frag2<S>(fm, 0, x, cur);
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    acc[x >> 1][x & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[x >> 1], cur.b[x & 1], acc[x >> 1][x & 1], 0, 0, 0);
    if (x < 6) {
      read_frag2<S>(fm, 1, x, nxt);
      stage_dma2<(S + 2) % 3>(lm, x, wave, kt + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int x = 0; x < 8; ++x)
    acc[x >> 1][x & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(nxt.a[x >> 1], nxt.b[x & 1], acc[x >> 1][x & 1], 0, 0, 0);
}

// The dW GEMMs in 256 x 128 tiles, two workgroups per CU.  g.tiles_n counts 128-column tiles.  GRP:
// GRP_NONE (one product) or GRP_DW (one product per group).  EPI: EPI_DW, EPI_DWC or EPI_RAW; NB: the
// examples whose correction terms the epilogue applies.
template <int EPI, bool EC, int NB, int GRP>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_dw128_kernel(GemmParams g, EpiParams ep, GroupGemm gg) {
  static_assert(GRP == GRP_NONE || GRP == GRP_DW, "one product, or one per group");
  int local;
  if constexpr (GRP == GRP_DW) {
    if (gg.status[0] != 0) return;
    const int per = g.tiles_m * g.tiles_n;
    const int slot = blockIdx.x / per;
    local = blockIdx.x % per;
    if (slot >= gg.G) return;
    const int e = gg.order[slot];
    const int64_t r0 = gg.offsets[e], n = gg.offsets[e + 1] - r0;
    g.A += r0 * g.lda;
    g.B += r0 * g.ldb;
    g.K = n;
    ep.delta += e;
    ep.row_scale = advance(ep.row_scale, e * g.M);
    ep.ebar = advance(ep.ebar, e * g.M);
    ep.colsum = advance(ep.colsum, e * g.N);
    ep.u = advance(ep.u, e * g.N);
    ep.out = (char*)ep.out + e * gg.out_stride * 4;
    ep.S = n > 0 ? n : 1;
    ep.B = 1;
  } else {
    // XCD-aware numbering, then the grouped order
    const int nblocks = g.tiles_m * g.tiles_n;
    local = blockIdx.x;
    if (nblocks % kNumXcd == 0) local = (local % kNumXcd) * (nblocks / kNumXcd) + local / kNumXcd;
  }
  const int group = kGroupM * g.tiles_n;
  const int first_m = (local / group) * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int tm = first_m + (local % group) % gsz;
  const int tn = (local % group) / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN2;
  const int nk = (int)((g.K + BK - 1) / BK);

  v16i acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  // The epilogue's factors are loaded now, ahead of the ring's first loads, so their latency hides behind
  // the K loop: this thread's row (Delta, s_w[j] and ebar[b][j]) and the lane's columns (u[n], xs[b][n] and
  // the per-column steps of its two column blocks).
  const int64_t jrow = m0 + threadIdx.x;                    // BM == kGemmThreads
  float pre_sw = 1.f, pre_d = 1.f, pre_eb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) pre_eb[b] = 0.f;
  ColF<NB, 2> pre;
  if constexpr (EPI != EPI_RAW) {
    const int64_t jc = jrow < g.M ? jrow : 0;
    pre_d = ep.delta[0];
    if (ep.row_scale) pre_sw = ep.row_scale[jc];
    if (EC)
#pragma unroll
      for (int b = 0; b < NB; ++b) pre_eb[b] = b < ep.B ? ep.ebar[b * g.M + jc] : 0.f;
    load_cols<EPI, EC, NB, 2>(g, ep, m0, n0, pre);
  }
  const LoadMap2 lm = make_loadmap2(g, m0, n0);
  const FragMap2 fm = make_fragmap2();
  load_stage2<0>(lm, 0);
  load_stage2<1>(lm, 1);
  for (int kt = 0; kt < nk; kt += 3) {
    k_step2<0>(lm, fm, kt, acc);
    if (kt + 1 < nk) k_step2<1>(lm, fm, kt + 1, acc);
    if (kt + 2 < nk) k_step2<2>(lm, fm, kt + 2, acc);
  }
  S3R_WAIT_VM(0);
  S3R_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();

  // per-row factors of the tile into LDS (the ring is free now): x = Delta / s_w[j] (EPI_DWC: 1 / s_w[j], the
  // step is per column), y = 1 / s_w[j]; roweb[b * BM + r] = ebar[b][j] / s_w[j]
  float4* rowf = reinterpret_cast<float4*>(g_nst0);
  float* roweb = reinterpret_cast<float*>(g_nst1);
  if constexpr (EPI != EPI_RAW) {
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (jrow < g.M) {
      const float inv = ep.row_scale ? __fdiv_rn(1.f, pre_sw) : 1.f;
      f.x = EPI == EPI_DWC ? inv : pre_d * inv;
      f.y = inv;
    }
    if (EC)
#pragma unroll
      for (int b = 0; b < NB; ++b) roweb[b * BM + threadIdx.x] = (b < ep.B && jrow < g.M) ? pre_eb[b] * f.y : 0.f;
    rowf[threadIdx.x] = f;
  }
  __syncthreads();
  // The grouped dW drops the stores of columns past N by an offset past the output descriptor (its callers bound
  // ld so that offset cannot wrap); the others branch around them.
  epilogue<EPI, EC, false, NB, GRP == GRP_DW, 2>(g, ep, m0, n0, rowf, roweb, acc, EPI != EPI_RAW ? &pre : nullptr);
}

// dW correction terms of examples 8 .. B-1 (the GEMM epilogue applies examples 0 .. 7):
// dW[j][i] -= sum_b ebar[b][j] * xs[b][i] / s_w[j].
__global__ __launch_bounds__(256) void dw_rank_update_kernel(float* __restrict__ dW, int64_t ld, int64_t D,
                                                             int64_t N, int64_t B, const float* __restrict__ ebar,
                                                             const int32_t* __restrict__ xs,
                                                             const float* __restrict__ sw) {
  const int64_t j = blockIdx.y;
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int64_t b = 8; b < B; ++b) s = fmaf(ebar[b * D + j], (float)xs[b * N + n], s);
  const float inv = sw ? __fdiv_rn(1.f, sw[j]) : 1.f;
  dW[j * ld + n] -= inv * s;
}

// -------------------------------------------------------------- GEMVs ----
// out[b][n] = sum over rows k of coef(b, k) * P[k][n]   (P int8 [K x N])
// Coefficients: VEC mode coef(b, k) = C[b * K + k] (the channel means ebar);
// TOKEN mode (one row, b = 0) coef(k) = ec_row[k] - ec_mean[k / S].
// HBM-bound.  A block covers 512 columns (8 per lane, 8-byte loads) and a band
// of kGvRows rows, a quarter per wave, with all of a wave's row loads in flight
// at once; few registers, so many waves per SIMD.  Each band writes its sums
// part[band][b][n]; gemv_reduce_kernel adds the bands in order in fp64.
constexpr int kGvThreads = 256;
constexpr int kGvColsPerLane = 8;
constexpr int kGvCols = 64 * kGvColsPerLane;   // 512 columns per block
constexpr int kGvRows = 64;                    // rows per band
constexpr int kGvRowsPerWave = kGvRows / 4;

// Grouped launches: gridDim.z groups of VEC mode, group z using P + z * pstride
// and coefficients C + z * nb * K (its outputs are vectors z*nb .. z*nb+nb-1);
// or (goff != null) grouped TOKEN mode, band blockIdx.y being a 64-row tile of
// one group (tables from the group offsets), coef(k) = ec_row[k] - ec_mean[e].
template <int NB>
__global__ __launch_bounds__(kGvThreads) void gemv_partial_kernel(
    const int8_t* __restrict__ P, int64_t ld, int64_t K, int64_t N, int64_t nb, int token_mode,
    const float* __restrict__ C, const float* __restrict__ ec_row, const float* __restrict__ ec_mean, int64_t S,
    float* __restrict__ part, int64_t pstride, const int64_t* __restrict__ goff, const int32_t* __restrict__ gtiles,
    int64_t G) {
  __shared__ float red[4][NB][kGvCols];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * kGvCols + lane * kGvColsPerLane;
  int64_t k0 = (int64_t)blockIdx.y * kGvRows;
  int rows = (int)min((int64_t)kGvRows, K - k0);
  int grp = -1;
  if (goff) {
    const GroupHit h = find_group_wave(gtiles, goff, G, blockIdx.y);
    if (h.e < 0) return;
    grp = h.e;
    k0 = h.r0 + (int64_t)(blockIdx.y - h.t0) * kGvRows;
    rows = (int)min((int64_t)kGvRows, h.r1 - k0);
  }
  P += blockIdx.z * pstride;
  if (C) C += blockIdx.z * nb * K;
  const int64_t nb_all = nb * gridDim.z, zb = blockIdx.z * nb;
  // The band through one buffer descriptor (no load addresses a row past it);
  // columns past N (the last lanes of a ragged row) are cleared by the mask at use.
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(P + k0 * ld), (short)0, (int)((uint32_t)rows * (uint32_t)ld), kRsrcWord3);
  const uint32_t voff = (uint32_t)n0;
  uint2 mask = make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
  if (n0 + kGvColsPerLane > N) {
    const int64_t keep = max((int64_t)0, N - n0);
    mask.x = keep >= 4 ? 0xFFFFFFFFu : (uint32_t)((1ull << (8 * keep)) - 1);
    mask.y = keep >= 8 ? 0xFFFFFFFFu : keep <= 4 ? 0u : (uint32_t)((1ull << (8 * (keep - 4))) - 1);
  }
  for (int64_t b0 = 0; b0 < nb; b0 += NB) {
    uint2 u[kGvRowsPerWave];
#pragma unroll
    for (int i = 0; i < kGvRowsPerWave; ++i) {
      // rows past the band repeat its last row; their coefficients are 0
      const uint32_t soff = (uint32_t)min(wave + 4 * i, rows - 1) * (uint32_t)ld;
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, 0);
      u[i] = make_uint2(w[0], w[1]);
    }
    // lane l holds the coefficients of this wave's row wave + 4l; the row loop
    // takes them as uniform values with readlane
    float cf[NB];
    {
      const int r = wave + 4 * lane;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float x = 0.f;
        if (lane < kGvRowsPerWave && r < rows && b0 + b < nb) {
          const int64_t k = k0 + r;
          x = token_mode ? ec_row[k] - ec_mean[grp >= 0 ? (int64_t)grp : (int64_t)((uint64_t)k / (uint64_t)S)]
                         : C[(b0 + b) * K + k];
        }
        cf[b] = x;
      }
    }
    float acc[NB][kGvColsPerLane];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int c = 0; c < kGvColsPerLane; ++c) acc[b][c] = 0.f;
#pragma unroll
    for (int i = 0; i < kGvRowsPerWave; ++i) {
      float c8[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        c8[b] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cf[b]), i));
      const uint32_t w[2] = {u[i].x & mask.x, u[i].y & mask.y};
#pragma unroll
      for (int c = 0; c < kGvColsPerLane; ++c) {
        const float x = (float)(int8_t)(w[c >> 2] >> (8 * (c & 3)));
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][c] = fmaf(c8[b], x, acc[b][c]);
      }
    }
    __syncthreads();                              // the previous pass is done with red
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int c = 0; c < kGvColsPerLane; ++c) red[wave][b][lane * kGvColsPerLane + c] = acc[b][c];
    __syncthreads();
    for (int i = threadIdx.x; i < NB * kGvCols; i += kGvThreads) {
      const int b = i / kGvCols, c = i % kGvCols;
      const int64_t n = (int64_t)blockIdx.x * kGvCols + c;
      if (b0 + b < nb && n < N) {
        const float v = ((red[0][b][c] + red[1][b][c]) + red[2][b][c]) + red[3][b][c];
        part[((int64_t)blockIdx.y * nb_all + zb + b0 + b) * N + n] = v;
      }
    }
  }
}

// The dense VEC-mode GEMV of up to four vectors (the examples' channel means ebar_b against the weight codes,
// the dX correction's v_b) on the matrix cores: its multiply-adds (four per weight byte) otherwise issue as
// many VALU instructions as the whole band takes to load.  v_mfma_f32_4x4x1f32 runs 16 blocks of a 4 x 4
// outer product: D[i][j] of block k / 4 is lane 4 (k / 4) + j, register i, its A[i] from lane 4 (k / 4) + i
// and its B[j] from lane k.  With A = the four coefficients of one row (lane m holds vector m % 4) and B =
// lane l's weight of that row in one of its 8 columns, register b of accumulator c holds vector b at the
// lane's column c.  Same blocks, bands, partial sums and reduction as gemv_partial_kernel.
typedef float v4f_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kGvThreads) void gemv_mfma_kernel(const int8_t* __restrict__ P, int64_t ld, int64_t K,
                                                              int64_t N, int64_t nb, const float* __restrict__ C,
                                                              float* __restrict__ part) {
  __shared__ float red[4][4][kGvCols];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * kGvCols + lane * kGvColsPerLane;
  const int64_t k0 = (int64_t)blockIdx.y * kGvRows;
  const int rows = (int)min((int64_t)kGvRows, K - k0);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(P + k0 * ld), (short)0, (int)((uint32_t)rows * (uint32_t)ld), kRsrcWord3);
  const uint32_t voff = (uint32_t)n0;
  uint2 mask = make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
  if (n0 + kGvColsPerLane > N) {
    const int64_t keep = max((int64_t)0, N - n0);
    mask.x = keep >= 4 ? 0xFFFFFFFFu : (uint32_t)((1ull << (8 * keep)) - 1);
    mask.y = keep >= 8 ? 0xFFFFFFFFu : keep <= 4 ? 0u : (uint32_t)((1ull << (8 * (keep - 4))) - 1);
  }
  for (int64_t b0 = 0; b0 < nb; b0 += 4) {
    uint2 u[kGvRowsPerWave];
#pragma unroll
    for (int i = 0; i < kGvRowsPerWave; ++i) {
      // rows past the band repeat its last row; their coefficients are 0
      const uint32_t soff = (uint32_t)min(wave + 4 * i, rows - 1) * (uint32_t)ld;
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, 0);
      u[i] = make_uint2(w[0], w[1]);
    }
    // lane m: vector b0 + m % 4 at this wave's row i = m / 4 (row wave + 4 i of the band)
    float cf = 0.f;
    {
      const int b = lane & 3, r = wave + 4 * (lane >> 2);
      if (r < rows && b0 + b < nb) cf = C[(b0 + b) * K + k0 + r];
    }
    v4f_t acc[kGvColsPerLane];
#pragma unroll
    for (int c = 0; c < kGvColsPerLane; ++c) acc[c] = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kGvRowsPerWave; ++i) {
      // A: lane m takes the coefficient of vector m % 4 at row i (from lane 4 i + m % 4)
      const float a = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute((4 * i + (lane & 3)) * 4, __builtin_bit_cast(int, cf)));
      const uint32_t w[2] = {u[i].x & mask.x, u[i].y & mask.y};
#pragma unroll
      for (int c = 0; c < kGvColsPerLane; ++c) {
        const float x = (float)(int8_t)(w[c >> 2] >> (8 * (c & 3)));
        acc[c] = __builtin_amdgcn_mfma_f32_4x4x1f32(a, x, acc[c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < kGvColsPerLane; ++c) red[wave][b][lane * kGvColsPerLane + c] = acc[c][b];
    __syncthreads();
    for (int i = threadIdx.x; i < 4 * kGvCols; i += kGvThreads) {
      const int b = i / kGvCols, c = i % kGvCols;
      const int64_t n = (int64_t)blockIdx.x * kGvCols + c;
      if (b0 + b < nb && n < N) {
        const float v = ((red[0][b][c] + red[1][b][c]) + red[2][b][c]) + red[3][b][c];
        part[((int64_t)blockIdx.y * nb + b0 + b) * N + n] = v;
      }
    }
    __syncthreads();                              // red is reused by the next pass
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


// out[i] = sum over bands c of part[c][i], in fp64.  A block takes 64
// consecutive outputs, one per lane, so each load of a wave is 256 contiguous
// bytes; wave w adds the bands c = w mod 4 in order (eight loads in flight),
// and the four waves' sums are added in wave order.
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ part, int64_t nbands,
                                                          int64_t count, float* __restrict__ out) {
  __shared__ double wsum[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  double a = 0.0;
  if (i < count) {
    for (int64_t c = wave; c < nbands; c += 32) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t cc = c + (int64_t)u * 4;
        const float v = part[min(cc, nbands - 1) * count + i];
        t[u] = cc < nbands ? v : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) a += (double)t[u];
    }
  }
  wsum[wave][lane] = a;
  __syncthreads();
  if (wave == 0 && i < count) out[i] = (float)(((wsum[0][lane] + wsum[1][lane]) + wsum[2][lane]) + wsum[3][lane]);
}

hipError_t run_gemv(const int8_t* P, int64_t ld, int64_t K, int64_t N, int64_t nb, int token_mode, const float* C,
                    const float* ec_row, const float* ec_mean, int64_t S, float* part, float* out, hipStream_t st) {
  const int64_t nbands = (K + kGvRows - 1) / kGvRows;
  dim3 grid((unsigned)((N + kGvCols - 1) / kGvCols), (unsigned)nbands);
  if (token_mode || nb == 1)
    hipLaunchKernelGGL(gemv_partial_kernel<1>, grid, dim3(kGvThreads), 0, st, P, ld, K, N, nb, token_mode, C, ec_row,
                       ec_mean, S, part, (int64_t)0, (const int64_t*)nullptr, (const int32_t*)nullptr, (int64_t)0);
  else
    hipLaunchKernelGGL(gemv_mfma_kernel, grid, dim3(kGvThreads), 0, st, P, ld, K, N, nb, C, part);
  const int64_t count = nb * N;
  hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((count + 63) / 64)), dim3(256), 0, st, part, nbands, count,
                     out);
  return hipGetLastError();
}

// out[e][n] = sum over the 64-row bands k of group e (tiles[e] .. tiles[e+1]) of
// part[k][n], fp64, zero for an empty group.  16 lanes share an output: each
// adds every 16th band in order, then a fixed xor butterfly adds the lanes.
__global__ __launch_bounds__(256) void grouped_band_reduce_kernel(const float* __restrict__ part,
                                                                  const int32_t* __restrict__ tiles, int64_t G,
                                                                  int64_t N, float* __restrict__ out) {
  constexpr int kLanes = 16;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t idx = g / kLanes;
  const int sub = (int)(g % kLanes);
  const bool ok = idx < G * N;
  const int64_t e = ok ? idx / N : 0, n = ok ? idx - e * N : 0;
  const int k1 = ok ? tiles[e + 1] : 0;
  double a = 0.0;
  for (int k = (ok ? tiles[e] : 0) + sub; k < k1; k += kLanes) a += (double)part[(int64_t)k * N + n];
  for (int o = 1; o < kLanes; o <<= 1) a += __shfl_xor(a, o, 64);
  if (ok && sub == 0) out[idx] = (float)a;
}

size_t gemv_part_bytes(int64_t K, int64_t N, int64_t nb) {
  const int64_t nbands = (K + kGvRows - 1) / kGvRows;
  return align_up((size_t)nbands * nb * N * 4, 256);
}

// ---------------------------------------- per-token steps: dW operand ----
// With one step Delta_t per token the weight gradient's exact product is
// Q^T diag(Delta) Xq, which no S8 GEMM applies after its accumulation over the
// tokens.  The steps are folded into the input codes instead,
// Z[t][n] = fl(Delta_t * Xq[t][n]), and Z is requantized per column with the
// forward operands' absmax RTNE rule: c_n = fl(a_n / 127), inv_n = fl(127 / a_n),
// Zq = clamp(rint(fl(Z * inv_n)), +-127), a_n = max_t |Z[t][n]| (a_n == 0: c = 1,
// codes 0; a non-finite a_n or inv_n: codes 0).  dW's GEMM then runs on Zq and
// its epilogue scales column n by c_n.
// Both kernels: a block covers 512 columns (8 per lane) and a band of kZRows
// rows, a quarter per wave, through buffer descriptors over the band; no load
// or store addresses a row past the band.
constexpr int kZRows = 256;
constexpr int kZUnroll = 8;

__device__ __forceinline__ void decode_i8x8(uint32_t lo, uint32_t hi, float v[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[c] = (float)(int8_t)(lo >> (8 * c));
    v[c + 4] = (float)(int8_t)(hi >> (8 * c));
  }
}

// cbits[n] = max over the band of |fl(Delta_t * Xq[t][n])| as ordered fp32 bits
// (NaN above every number), combined over the bands with an integer atomic max.
__global__ __launch_bounds__(256) void zcol_amax_kernel(const int8_t* __restrict__ X, int64_t ld, int64_t T,
                                                        int64_t N, const float* __restrict__ delta,
                                                        uint32_t* __restrict__ cbits) {
  __shared__ uint32_t red[4][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 512 + lane * 8;
  const int64_t t0 = (int64_t)blockIdx.y * kZRows;
  const int rows = (int)min((int64_t)kZRows, T - t0);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + t0 * ld), (short)0, (int)((uint32_t)rows * (uint32_t)ld), kRsrcWord3);
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r0 = wave; r0 < rows && n0 < N; r0 += 4 * kZUnroll) {
    uint2 u[kZUnroll];
    float d[kZUnroll];
#pragma unroll
    for (int k = 0; k < kZUnroll; ++k) {
      const int r = min(r0 + 4 * k, rows - 1);      // rows past the band repeat its last row, weighted 0
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(rsrc, (uint32_t)n0, (uint32_t)r * (uint32_t)ld, 0);
      u[k] = make_uint2(w[0], w[1]);
      d[k] = r0 + 4 * k < rows ? delta[t0 + r] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kZUnroll; ++k) {
      float v[8];
      decode_i8x8(u[k].x, u[k].y, v);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t b = __float_as_uint(d[k] * v[c]) & 0x7FFFFFFFu;
        m[c] = m[c] > b ? m[c] : b;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) red[wave][lane * 8 + c] = m[c];
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int64_t n = (int64_t)blockIdx.x * 512 + i;
    uint32_t a = red[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) a = a > red[w][i] ? a : red[w][i];
    if (n < N && a) atomicMax(&cbits[n], a);
  }
}

// Zq [T x ldz] from Xq and the column maxima; block row 0 also writes c[n].
// Columns past N (up to the 8-column boundary) get code 0.
__global__ __launch_bounds__(256) void zcol_quant_kernel(const int8_t* __restrict__ X, int64_t ld, int64_t T,
                                                         int64_t N, const float* __restrict__ delta,
                                                         const uint32_t* __restrict__ cbits, int8_t* __restrict__ Zq,
                                                         int64_t ldz, float* __restrict__ cval) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 512 + lane * 8;
  if (n0 >= N) return;
  const int64_t t0 = (int64_t)blockIdx.y * kZRows;
  const int rows = (int)min((int64_t)kZRows, T - t0);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + t0 * ld), (short)0, (int)((uint32_t)rows * (uint32_t)ld), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t zsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Zq + t0 * ldz), (short)0, (int)((uint32_t)rows * (uint32_t)ldz), kRsrcWord3);
  float inv[8];
  bool zero[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int64_t n = n0 + c;
    const uint32_t ab = n < N ? cbits[n] : 0u;
    const float a = __uint_as_float(ab);
    const float cs = ab == 0 ? 1.f : __fdiv_rn(a, 127.f);
    inv[c] = ab == 0 ? 0.f : __fdiv_rn(127.f, a);
    zero[c] = !(ab < 0x7F800000u) || !(__float_as_uint(inv[c]) < 0x7F800000u) || n >= N;
    if (blockIdx.y == 0 && wave == 0 && n < N) cval[n] = (ab > 0x7F800000u) ? a : cs;
  }
  for (int r0 = wave; r0 < rows; r0 += 4 * kZUnroll) {
    uint2 u[kZUnroll];
    float d[kZUnroll];
#pragma unroll
    for (int k = 0; k < kZUnroll; ++k) {
      const int r = min(r0 + 4 * k, rows - 1);      // rows past the band repeat its last row, weighted 0
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(rsrc, (uint32_t)n0, (uint32_t)r * (uint32_t)ld, 0);
      u[k] = make_uint2(w[0], w[1]);
      d[k] = r0 + 4 * k < rows ? delta[t0 + r] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kZUnroll; ++k) {
      float v[8];
      decode_i8x8(u[k].x, u[k].y, v);
      uint32_t q[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float z = d[k] * v[c];
        const float x = fminf(fmaxf(__builtin_rintf(z * inv[c]), -127.f), 127.f);
        q[c] = zero[c] ? 0u : (uint32_t)(int32_t)x & 0xFFu;
      }
      const uint32_t lo = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
      const uint32_t hi = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
      const int r = r0 + 4 * k;
      typedef uint32_t v2u __attribute__((ext_vector_type(2)));
      if (r < rows)
        __builtin_amdgcn_raw_buffer_store_b64(v2u{lo, hi}, zsrc, (uint32_t)n0, (uint32_t)r * (uint32_t)ldz, 0);
    }
  }
}

size_t zq_ld(int64_t N) { return (size_t)((N + 15) / 16 * 16); }

template <bool A_KMAJOR, int EPI, bool EC, int NB = 1, int GRP = GRP_NONE>
hipError_t run_gemm(const GemmParams& g, const EpiParams& ep, hipStream_t st, const GroupGemm& gg = GroupGemm{}) {
  GemmTiming& tm = gemm_timing();
  const GemmTiming ev = tm;
  tm = GemmTiming{};
  const int nblocks = GRP == GRP_NONE ? g.tiles_m * g.tiles_n
                      : GRP == GRP_DX   ? gg.tiles_m_all * g.tiles_n
                                        : 2 * g.tiles_m * g.tiles_n;
  if (ev.start && hipEventRecord(ev.start, st) != hipSuccess) return hipErrorInvalidValue;
  if (nblocks > 0)
    hipLaunchKernelGGL((gemm_i8_kernel<A_KMAJOR, EPI, EC, NB, GRP>), dim3((unsigned)nblocks), dim3(kGemmThreads), 0,
                       st, g, ep, gg);
  hipError_t e = hipGetLastError();
  if (ev.stop && hipEventRecord(ev.stop, st) != hipSuccess && e == hipSuccess) e = hipErrorInvalidValue;
  return e;
}

// The dW GEMMs in 256 x 128 tiles (gemm_dw128_kernel), with the same timing hook as run_gemm.
template <int EPI, bool EC, int NB, int GRP>
hipError_t run_dw128(GemmParams g, const EpiParams& ep, hipStream_t st, const GroupGemm& gg = GroupGemm{}) {
  GemmTiming& tm = gemm_timing();
  const GemmTiming ev = tm;
  tm = GemmTiming{};
  g.tiles_n = (int)((g.N + BN2 - 1) / BN2);
  const int64_t per = (int64_t)g.tiles_m * g.tiles_n;
  const int64_t nblocks = GRP == GRP_DW ? gg.G * per : per;
  if (ev.start && hipEventRecord(ev.start, st) != hipSuccess) return hipErrorInvalidValue;
  if (nblocks > 0)
    hipLaunchKernelGGL((gemm_dw128_kernel<EPI, EC, NB, GRP>), dim3((unsigned)nblocks), dim3(kGemmThreads), 0, st, g,
                       ep, gg);
  hipError_t e = hipGetLastError();
  if (ev.stop && hipEventRecord(ev.stop, st) != hipSuccess && e == hipSuccess) e = hipErrorInvalidValue;
  return e;
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

// dW workspace: two-way EC: GEMV band partials, u [d_in] | per-token
// steps: Zq [T x ldz], column maxima (bits) [d_in], column steps [d_in].
struct DwLayout { size_t part, u, zq, cbits, cval, total; };

DwLayout dw_layout(int64_t T, int64_t d_in, int ec, int per_token) {
  DwLayout L{};
  size_t off = 0;
  if (ec == S3R_EC_TWO_WAY || ec == S3R_EC_DW_ONLY) {
    L.part = off; off += gemv_part_bytes(T, d_in, 1);
    L.u = off;    off += align_up((size_t)d_in * 4, 256);
  }
  if (per_token) {
    L.zq = off;    off += align_up((size_t)T * zq_ld(d_in), 256);
    L.cbits = off; off += align_up((size_t)d_in * 4, 256);
    L.cval = off;  off += align_up((size_t)d_in * 4, 256);
  }
  L.total = off;
  return L;
}

size_t dw_workspace(int64_t T, int64_t D, int64_t d_in, int64_t S, int ec, int per_token) {
  (void)D; (void)S;
  return dw_layout(T, d_in, ec, per_token).total;
}

hipError_t launch_backward_dx(const DxArgs& a, hipStream_t st) {
  const int64_t B = a.S > 0 ? a.T / a.S : 0;
  EpiParams ep{};
  ep.delta = a.delta; ep.per_token = a.per_token; ep.row_scale = a.sx;
  ep.ec = (a.ec != S3R_EC_NONE) && (a.out_dt == S3R_F32 || a.out_dt == S3R_F32_ACC);
  ep.colsum = a.rW; ep.ec_row = a.ec_row; ep.ec_mean = a.ec_mean;
  ep.S = a.S; ep.B = B;
  ep.out = a.out; ep.ld_out = a.ld_out; ep.out_i32 = a.out_dt == S3R_I32_RAW;
  if (ep.ec && a.T > 0 && a.d_in > 0) {
    float* part = (float*)(a.ws);
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
  if (a.out_dt == S3R_I32_RAW) return run_gemm<true, EPI_RAW, false>(g, ep, st);
  if (a.out_dt == S3R_F32_ACC)
    return ep.ec ? run_gemm<true, EPI_DXA, true>(g, ep, st) : run_gemm<true, EPI_DXA, false>(g, ep, st);
  if (ep.ec) return run_gemm<true, EPI_DX, true>(g, ep, st);
  return run_gemm<true, EPI_DX, false>(g, ep, st);
}

namespace {
// The dW epilogue's parameters, and (two-way correction) u = sum_t (eps_t - mu_b) Xq[t, :] by the
// correction GEMV into the workspace.
hipError_t dw_epilogue(const DwArgs& a, EpiParams& ep, hipStream_t st) {
  const int64_t B = a.S > 0 ? a.T / a.S : 0;
  const DwLayout L = dw_layout(a.T, a.d_in, a.ec, a.per_token);
  ep = EpiParams{};
  ep.delta = a.delta; ep.per_token = 0; ep.row_scale = a.sw;
  ep.ec = (a.ec == S3R_EC_TWO_WAY || a.ec == S3R_EC_DW_ONLY) && a.out_dt == S3R_F32;
  ep.colsum = a.xs; ep.ebar = a.ec_col; ep.ec_row = a.ec_row; ep.ec_mean = a.ec_mean;
  ep.S = a.S; ep.B = B;
  ep.out = a.out; ep.ld_out = a.ld_out; ep.out_i32 = a.out_dt == S3R_I32_RAW;
  if (ep.ec && a.D > 0 && a.d_in > 0) {
    float* part = (float*)(a.ws + L.part);
    float* u = (float*)(a.ws + L.u);
    if (a.T > 0) {
      hipError_t e = run_gemv(a.X, a.ld_x, a.T, a.d_in, 1, 1, nullptr, a.ec_row, a.ec_mean, a.S, part, u, st);
      if (e != hipSuccess) return e;
    } else {
      hipError_t e = fill_zero(u, a.d_in, st);
      if (e != hipSuccess) return e;
    }
    ep.u = u;
  }
  return hipSuccess;
}

// Examples past the epilogue's NB slots: the rest of the correction's rank-B term, sum_b ebar_b[j] xs_b[i]
// for b >= NB, subtracted by a pass over the output.
hipError_t dw_rank_update(const DwArgs& a, const EpiParams& ep, hipStream_t st) {
  if (!ep.ec || ep.B <= 8 || a.D == 0 || a.d_in == 0) return hipSuccess;
  hipLaunchKernelGGL(dw_rank_update_kernel, dim3((unsigned)((a.d_in + 255) / 256), (unsigned)a.D), dim3(256), 0, st,
                     (float*)a.out, a.ld_out, a.D, a.d_in, ep.B, a.ec_col, a.xs, a.sw);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_backward_dw(const DwArgs& a, hipStream_t st) {
  const int64_t B = a.S > 0 ? a.T / a.S : 0;
  const DwLayout L = dw_layout(a.T, a.d_in, a.ec, a.per_token);
  EpiParams ep;
  {
    hipError_t e = dw_epilogue(a, ep, st);
    if (e != hipSuccess) return e;
  }
  // B operand: the input codes, or (per-token steps) their per-column requantization Zq
  const int8_t* Bop = a.X;
  int64_t ldb = a.ld_x;
  if (a.per_token && a.d_in > 0) {
    uint32_t* cbits = (uint32_t*)(a.ws + L.cbits);
    float* cval = (float*)(a.ws + L.cval);
    int8_t* zq = (int8_t*)(a.ws + L.zq);
    hipError_t e = fill_zero((float*)cbits, a.d_in, st);
    if (e != hipSuccess) return e;
    if (a.T > 0) {
      dim3 grid((unsigned)((a.d_in + 511) / 512), (unsigned)((a.T + kZRows - 1) / kZRows));
      hipLaunchKernelGGL(zcol_amax_kernel, grid, dim3(256), 0, st, a.X, a.ld_x, a.T, a.d_in, a.delta, cbits);
      hipLaunchKernelGGL(zcol_quant_kernel, grid, dim3(256), 0, st, a.X, a.ld_x, a.T, a.d_in, a.delta, cbits, zq,
                         (int64_t)zq_ld(a.d_in), cval);
    } else {
      hipLaunchKernelGGL(zcol_quant_kernel, dim3((unsigned)((a.d_in + 511) / 512), 1), dim3(256), 0, st, a.X,
                         a.ld_x, a.T, a.d_in, a.delta, cbits, zq, (int64_t)zq_ld(a.d_in), cval);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    Bop = zq;
    ldb = (int64_t)zq_ld(a.d_in);
    ep.colstep = cval;
  }
  // dW = Q^T B: A[m=j][k=t] = Q[t][j] (M-contiguous), B [T x d_in] (N-contiguous)
  const GemmParams g = make_gemm(a.Q, a.ld_q, Bop, ldb, a.D, a.d_in, a.T);
  if (a.out_dt == S3R_I32_RAW) return run_dw128<EPI_RAW, false, 1, GRP_NONE>(g, ep, st);
  hipError_t e;
  if (a.per_token) {
    if (!ep.ec) e = run_dw128<EPI_DWC, false, 1, GRP_NONE>(g, ep, st);
    else if (B <= 1) e = run_dw128<EPI_DWC, true, 1, GRP_NONE>(g, ep, st);
    else if (B <= 2) e = run_dw128<EPI_DWC, true, 2, GRP_NONE>(g, ep, st);
    else if (B <= 4) e = run_dw128<EPI_DWC, true, 4, GRP_NONE>(g, ep, st);
    else e = run_dw128<EPI_DWC, true, kMaxB, GRP_NONE>(g, ep, st);
  } else {
    if (!ep.ec) e = run_dw128<EPI_DW, false, 1, GRP_NONE>(g, ep, st);
    else if (B <= 1) e = run_dw128<EPI_DW, true, 1, GRP_NONE>(g, ep, st);
    else if (B <= 2) e = run_dw128<EPI_DW, true, 2, GRP_NONE>(g, ep, st);
    else if (B <= 4) e = run_dw128<EPI_DW, true, 4, GRP_NONE>(g, ep, st);
    else e = run_dw128<EPI_DW, true, kMaxB, GRP_NONE>(g, ep, st);
  }
  if (e != hipSuccess) return e;
  return dw_rank_update(a, ep, st);
}

hipError_t launch_backward_dw_pair(const DwArgs& a0, const DwArgs& a1, hipStream_t st) {
  const int64_t B = a0.S > 0 ? a0.T / a0.S : 0;
  EpiParams ep0, ep1;
  hipError_t e = dw_epilogue(a0, ep0, st);
  if (e == hipSuccess) e = dw_epilogue(a1, ep1, st);
  if (e != hipSuccess) return e;
  const GemmParams g = make_gemm(a0.Q, a0.ld_q, a0.X, a0.ld_x, a0.D, a0.d_in, a0.T);
  GroupGemm gg{};
  gg.A2 = a1.Q;
  gg.ep2 = ep1;
  if (a0.out_dt == S3R_I32_RAW) e = run_gemm<false, EPI_RAW, false, 1, GRP_PAIR>(g, ep0, st, gg);
  else if (!ep0.ec) e = run_gemm<false, EPI_DW, false, 1, GRP_PAIR>(g, ep0, st, gg);
  else if (B <= 1) e = run_gemm<false, EPI_DW, true, 1, GRP_PAIR>(g, ep0, st, gg);
  else if (B <= 2) e = run_gemm<false, EPI_DW, true, 2, GRP_PAIR>(g, ep0, st, gg);
  else if (B <= 4) e = run_gemm<false, EPI_DW, true, 4, GRP_PAIR>(g, ep0, st, gg);
  else e = run_gemm<false, EPI_DW, true, kMaxB, GRP_PAIR>(g, ep0, st, gg);
  if (e == hipSuccess) e = dw_rank_update(a0, ep0, st);
  if (e == hipSuccess) e = dw_rank_update(a1, ep1, st);
  return e;
}

// ---------------------------------------------------------- grouped calls ----
// Workspace: group tables | dX: v band partials [bands(D) x G x N], v [G x N]
//                                  | dW: u band partials [R/64 + G bands x N], u [G x N]
struct GroupedBwLayout { size_t tables, part, vec, total; };

GroupedBwLayout grouped_bw_layout(int64_t R, int64_t D, int64_t d_in, int64_t G, bool dx, bool ec) {
  GroupedBwLayout L{};
  size_t off = 0;
  L.tables = off; off = align_up(off + group_tables_bytes(G), 256);
  if (ec) {
    const int64_t bands = dx ? (D + kGvRows - 1) / kGvRows : R / kGvRows + G;
    L.part = off; off = align_up(off + (size_t)bands * (dx ? G : 1) * d_in * 4, 256);
    L.vec = off;  off = align_up(off + (size_t)G * d_in * 4, 256);
  }
  L.total = off;
  return L;
}

size_t grouped_dx_workspace(int64_t R, int64_t D, int64_t d_in, int64_t G, int ec) {
  return grouped_bw_layout(R, D, d_in, G, true, ec != 0).total;
}
size_t grouped_dw_workspace(int64_t R, int64_t D, int64_t d_in, int64_t G, int ec) {
  return grouped_bw_layout(R, D, d_in, G, false, ec != 0).total;
}

// dX rows of every group: Q rows of group e times its weight codes W + e * w_stride.
hipError_t launch_grouped_backward_dx(const DxArgs& a, int64_t G, const int64_t* offsets, int64_t w_stride,
                                      uint32_t* flags, hipStream_t st) {
  const GroupedBwLayout L = grouped_bw_layout(a.T, a.D, a.d_in, G, true, a.ec != 0);
  const GroupTables tab = group_tables(a.ws + L.tables, G, offsets);
  hipError_t e = launch_group_tables(tab, a.T, flags, st);
  if (e != hipSuccess || a.d_in == 0 || a.T == 0) return e;
  EpiParams ep{};
  ep.delta = a.delta; ep.per_token = 0; ep.row_scale = a.sx;
  ep.ec = (a.ec != S3R_EC_NONE) && (a.out_dt == S3R_F32 || a.out_dt == S3R_F32_ACC);
  ep.colsum = a.rW; ep.ec_row = a.ec_row; ep.ec_mean = a.ec_mean;
  ep.S = 1; ep.B = 1;
  ep.out = a.out; ep.ld_out = a.ld_out; ep.out_i32 = a.out_dt == S3R_I32_RAW;
  if (ep.ec) {
    float* part = (float*)(a.ws + L.part);
    float* v = (float*)(a.ws + L.vec);
    if (a.D > 0) {
      // v_e = ebar_e . W_e for every group: gridDim.z = G
      const int64_t nbands = (a.D + kGvRows - 1) / kGvRows;
      dim3 grid((unsigned)((a.d_in + kGvCols - 1) / kGvCols), (unsigned)nbands, (unsigned)G);
      hipLaunchKernelGGL(gemv_partial_kernel<1>, grid, dim3(kGvThreads), 0, st, a.W, a.ld_w, a.D, a.d_in, (int64_t)1,
                         0, a.ec_col, (const float*)nullptr, (const float*)nullptr, (int64_t)1, part, w_stride,
                         (const int64_t*)nullptr, (const int32_t*)nullptr, (int64_t)0);
      const int64_t count = G * a.d_in;
      hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((count + 63) / 64)), dim3(256), 0, st, part, nbands,
                         count, v);
    } else {
      e = fill_zero(v, G * a.d_in, st);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ep.vec = v;
  }
  GemmParams g = make_gemm(a.Q, a.ld_q, a.W, a.ld_w, a.T, a.d_in, a.D);
  GroupGemm gg{offsets, tab.tiles256, tab.order, tab.status, G, w_stride, 0, (int)(a.T / BM + G)};
  if (a.out_dt == S3R_I32_RAW) return run_gemm<true, EPI_RAW, false, 1, GRP_DX>(g, ep, st, gg);
  if (a.out_dt == S3R_F32_ACC)
    return ep.ec ? run_gemm<true, EPI_DXA, true, 1, GRP_DX>(g, ep, st, gg)
                 : run_gemm<true, EPI_DXA, false, 1, GRP_DX>(g, ep, st, gg);
  return ep.ec ? run_gemm<true, EPI_DX, true, 1, GRP_DX>(g, ep, st, gg)
               : run_gemm<true, EPI_DX, false, 1, GRP_DX>(g, ep, st, gg);
}

// dW_e = Q_e^T X_e of every group into out + e * out_stride (per-tensor steps).
hipError_t launch_grouped_backward_dw(const DwArgs& a, int64_t G, const int64_t* offsets, int64_t out_stride,
                                      uint32_t* flags, hipStream_t st) {
  const GroupedBwLayout L = grouped_bw_layout(a.T, a.D, a.d_in, G, false, a.ec != 0);
  const GroupTables tab = group_tables(a.ws + L.tables, G, offsets);
  hipError_t e = launch_group_tables(tab, a.T, flags, st);
  if (e != hipSuccess || a.d_in == 0 || a.D == 0) return e;
  EpiParams ep{};
  ep.delta = a.delta; ep.per_token = 0; ep.row_scale = a.sw;
  ep.ec = (a.ec == S3R_EC_TWO_WAY || a.ec == S3R_EC_DW_ONLY) && a.out_dt == S3R_F32;
  ep.colsum = a.xs; ep.ebar = a.ec_col; ep.ec_row = a.ec_row; ep.ec_mean = a.ec_mean;
  ep.S = 1; ep.B = 1;
  ep.out = a.out; ep.ld_out = a.ld_out; ep.out_i32 = a.out_dt == S3R_I32_RAW;
  if (ep.ec) {
    float* part = (float*)(a.ws + L.part);
    float* u = (float*)(a.ws + L.vec);
    const int64_t bands = a.T / kGvRows + G;
    dim3 grid((unsigned)((a.d_in + kGvCols - 1) / kGvCols), (unsigned)bands, 1);
    hipLaunchKernelGGL(gemv_partial_kernel<1>, grid, dim3(kGvThreads), 0, st, a.X, a.ld_x, a.T, a.d_in, (int64_t)1, 1,
                       (const float*)nullptr, a.ec_row, a.ec_mean, (int64_t)1, part, (int64_t)0, offsets,
                       (const int32_t*)tab.tiles64, G);
    hipLaunchKernelGGL(grouped_band_reduce_kernel, dim3((unsigned)((G * a.d_in * 16 + 255) / 256)), dim3(256), 0, st,
                       part,
                       (const int32_t*)tab.tiles64, G, a.d_in, u);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ep.u = u;
  }
  GemmParams g = make_gemm(a.Q, a.ld_q, a.X, a.ld_x, a.D, a.d_in, a.T);
  GroupGemm gg{offsets, tab.tiles256, tab.order, tab.status, G, 0, out_stride, 0};
  if (a.out_dt == S3R_I32_RAW) return run_dw128<EPI_RAW, false, 1, GRP_DW>(g, ep, st, gg);
  return ep.ec ? run_dw128<EPI_DW, true, 1, GRP_DW>(g, ep, st, gg) : run_dw128<EPI_DW, false, 1, GRP_DW>(g, ep, st, gg);
}

}  // namespace s3r
