/*
 * s3r.h -- C ABI of libs3r.so: the stochastically rounded INT8 backward pass
 * of a linear layer on AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "Efficient Quantization Training with Stochastic
 * Rounding via Structured Subspace Randomness" (the S3R page below):
 *   - section "Quantized Backpropagation with Stochastic Rounding": the
 *     upstream gradient G [tokens x hidden] is scaled, rounded to S8 and fed
 *     to two S8 x S8 -> S32 GEMMs, dX = G W^T and dW = X^T G, then rescaled;
 *     the forward scales s_x (per token) and s_w (per output channel) are
 *     folded into G, G' = diag(s_x) G diag(s_w), with one step
 *     Delta = max|G'|/127 and codes Q = SR(G'; R)/Delta (eq. (2)), written
 *     once for both GEMMs;
 *   - section "Structured Subspace Randomness": S3R draws one threshold per
 *     token and shares it across the hidden dimension (Phi_2D);
 *   - section "Structured Error Correction (S3R-EC)": the per-token and
 *     per-example per-channel mean rounding errors are subtracted after the
 *     unchanged GEMMs, from dX and dW (two-way) or from dX only.
 *
 * Conventions (all calls):
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device.
 *     Matrices are row-major with an explicit leading dimension in ELEMENTS.
 *   - The caller owns every buffer, including the workspace.  The library
 *     allocates nothing, never synchronises, and enqueues all work on the
 *     given stream; results are ready when that stream reaches them.
 *   - Argument checks happen on the host before anything is enqueued; a
 *     nonzero return means nothing was enqueued (except S3R_ERR_HIP, which
 *     reports a launch failure).
 *   - Results are bitwise deterministic: no floating-point atomics, all
 *     reductions in a fixed order.
 *   - Workspaces hold scratch partial results only: their contents need no
 *     initialisation and are not kept between calls.  One workspace may serve
 *     quantize and backward calls; calls that overlap in time (different
 *     streams) must not share a workspace.
 *   - Weight layout: W is stored [D x d_in] (PyTorch Linear layout, the
 *     page's W^T), Wq likewise; X is [T x d_in].
 */
#ifndef S3R_H
#define S3R_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define S3R_OK                0
#define S3R_ERR_INVALID_ARG  -1  /* null pointer, bad size/leading dim/alignment, T % S != 0 */
#define S3R_ERR_UNSUPPORTED  -2  /* unsupported dtype / mode / ec / scale combination */
#define S3R_ERR_WORKSPACE    -3  /* workspace too small */
#define S3R_ERR_ARCH         -4  /* current device is not gfx950 */
#define S3R_ERR_HIP          -5  /* a HIP call or kernel launch failed */

/* ---- enums ------------------------------------------------------------- */
/* S3R_F32_ACC (s3r_backward_dx only): add the f32 result into the f32 output
 * (dX of two projections of the same input, e.g. the gate and up projections
 * of a SwiGLU block). */
typedef enum { S3R_F32 = 0, S3R_BF16 = 1, S3R_I32_RAW = 2, S3R_F32_ACC = 3 } s3r_dtype;
/* Rounding of G' (S3R page, "Compared Configurations"):
 *   RTNE  deterministic round to nearest even;
 *   SR    independent SR, one Philox4x32-10 32-bit word per element;
 *   S3R   one threshold per token shared across the hidden dimension (Phi_2D);
 *   S3R_BCAST  one threshold per example of rows_per_example tokens, shared by
 *         all its tokens and channels (Phi_bcast, the page's ablation). */
typedef enum { S3R_RTNE = 0, S3R_SR = 1, S3R_S3R = 2, S3R_S3R_BCAST = 3 } s3r_mode;
/* S3R-EC (section "Structured Error Correction"): NONE, the dX-only variant,
 * the two-way correction of both products, or (the ablation of Table II,
 * "dW-only corr.") the weight-gradient term alone.  Requires mode S3R or
 * S3R_BCAST. */
typedef enum { S3R_EC_NONE = 0, S3R_EC_DX_ONLY = 1, S3R_EC_TWO_WAY = 2, S3R_EC_DW_ONLY = 3 } s3r_ec;
/* Step granularity.  PER_TENSOR is the page's single step Delta (the only one
 * the dW GEMM can apply after S32 accumulation).  PER_TOKEN gives one step
 * per row; it is the forward operands' rule (per-token s_x, per-output-channel
 * s_w) and is also accepted for G by s3r_quantize, s3r_backward_dx and (through
 * a per-column requantization of the inputs, see there) s3r_backward_dw. */
typedef enum { S3R_PER_TENSOR = 0, S3R_PER_TOKEN = 1 } s3r_scale;

/* Bits OR-ed into the optional device flags word by s3r_quantize. */
#define S3R_FLAG_NONFINITE  1u  /* an amax was Inf/NaN: affected codes are 0 */
#define S3R_FLAG_TINY_STEP  2u  /* an amax so small that 127*2^24/amax overflows fp32: codes 0 */
/* bit 4u is unused (reserved) */
#define S3R_FLAG_BAD_GROUPS 8u  /* grouped calls: the group offsets are not a non-decreasing
                                   sequence from 0 to the row count; nothing was computed */

/* Problem descriptor of one quantized tensor G [rows x cols]. */
typedef struct s3r_qdesc {
  int64_t  rows;              /* T, tokens (>= 0) */
  int64_t  cols;              /* D, hidden size of G (>= 0) */
  int64_t  rows_per_example;  /* S, tokens per example; T % S == 0, S >= 1 */
  int32_t  mode;              /* s3r_mode */
  int32_t  ec;                /* s3r_ec */
  int32_t  scale;             /* s3r_scale */
  uint32_t layer_id;          /* Philox counter word 2: separates layers */
  uint64_t seed;              /* Philox key */
  uint32_t stream;            /* threshold stream, 0..65535: 0 is the one draw shared by both
                                 backward products; quantizing G a second time for the weight
                                 gradient with stream 1 gives the independent draw R^RHS of the
                                 conventional configuration ("Quantized Backpropagation...") */
  uint32_t reserved;          /* must be 0 */
} s3r_qdesc;

/* ---- quantizer ---------------------------------------------------------
 * s3r_quantize: fold, step, round and (optionally) error statistics.
 * S3R page, "Quantized Backpropagation with Stochastic Rounding" (eqs. (1),
 * (2)), "Structured Subspace Randomness" (Phi_2D, 7-bit thresholds on a
 * half-step grid), "Two-Way Correction" (the two averages of E).
 *
 *   G        [T x D] F32 or BF16 (g_dtype), leading dim ld_g >= D.
 *   row_scale [T] f32 (s_x) or NULL (= 1);  col_scale [D] f32 (s_w) or NULL.
 *            G'[t,j] = fl(fl(G[t,j] * s_x[t]) * s_w[j]).
 *   Q        [T x D] int8 codes in [-127, 127], leading dim ld_q >= D.
 *   delta    [1] (PER_TENSOR) or [T] (PER_TOKEN) f32: Delta = fl(amax/127),
 *            1 for an all-zero tensor (row).
 *   code_colsum [B x D] int32 or NULL: per-example column sums of Q
 *            (B = T/S).  Used by the forward-operand prep to form the
 *            weight's row sums r_W = Wq^T 1 (S = D rows of W) and the
 *            per-example input sums xs_b (S tokens of X).
 *   ec_row [T], ec_col [B x D], ec_mean [B] f32: required iff ec != NONE,
 *            NULL otherwise.  With E' = Delta_t (q - x), x = G'/Delta:
 *            ec_row[t] = mean_j E'[t,j]   (eps_t, the token mean),
 *            ec_col[b,j] = mean_{t in b} E'[t,j]   (the channel means),
 *            ec_mean[b] = mean over example b of E' (its grand mean).
 *   flags    device uint32 or NULL: S3R_FLAG_* bits are OR-ed in (the caller
 *            clears it).
 *   ws       device workspace of at least s3r_quantize_workspace(desc) bytes,
 *            256-byte aligned.
 * A per-tensor step reads G twice (the amax pass, then the code pass); no
 * kernel waits on another workgroup, so the results do not depend on what
 * else runs on the device.
 * Thresholds: SR element (t,j) uses Philox4x32-10 block e>>2 of e = t*D + j
 * (counter {lo,hi}(e>>2), layer_id, 0; key = seed), word e&3, r =
 * (2*(w>>9)+1)/2^24; S3R token t uses block t>>4 (counter ..., layer_id, 1),
 * word (t>>2)&3, byte t&3, r = (2*(byte>>1)+1)/256; S3R_BCAST uses the same map
 * on the example index b = t / rows_per_example with tag 2.  Counter word 3 is
 * tag + 65536 * stream.  Code = clamp(floor(x+r)).
 */
size_t s3r_quantize_workspace(const s3r_qdesc* desc);
int s3r_quantize(const s3r_qdesc* desc,
                 const void* G, int32_t g_dtype, int64_t ld_g,
                 const float* row_scale, const float* col_scale,
                 int8_t* Q, int64_t ld_q, float* delta,
                 int32_t* code_colsum,
                 float* ec_row, float* ec_col, float* ec_mean,
                 uint32_t* flags,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_quantize_with_amax: s3r_quantize for a per-tensor step whose amax is
 * already on the device, so G is read once.  amax_bits [1] (device, read
 * only) holds max_{t,j} |G'[t,j]| as the bit pattern of a non-negative fp32
 * (a NaN anywhere gives a NaN pattern, which orders above every number), for
 * example as written by s3r_swiglu_backward_amax.  With that value the codes,
 * step, flags and statistics are exactly those s3r_quantize computes.  Same
 * arguments, layouts and workspace as s3r_quantize except: desc->scale must be
 * PER_TENSOR (else S3R_ERR_UNSUPPORTED) and there is no code_colsum output.
 * An amax that does not match G's actual maximum is the caller's error: codes
 * are still clamped to [-127, 127].
 */
int s3r_quantize_with_amax(const s3r_qdesc* desc,
                           const void* G, int32_t g_dtype, int64_t ld_g,
                           const float* row_scale, const float* col_scale,
                           const uint32_t* amax_bits,
                           int8_t* Q, int64_t ld_q, float* delta,
                           float* ec_row, float* ec_col, float* ec_mean,
                           uint32_t* flags,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_quantize_noalloc: s3r_quantize without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, checks,
 * kernels and results as s3r_quantize; the partial results live in one
 * library-owned device array of S3R_NOALLOC_SCRATCH_BYTES on each device the
 * library runs on, held until the process ends.  The call allocates nothing:
 * no hipMalloc, no hipFree, no allocating library routine.  The first call on
 * a device looks up that device's array address (hipGetSymbolAddress).
 *   Size limit: a call whose partials exceed S3R_NOALLOC_SCRATCH_BYTES (the
 *   workspace s3r_quantize would need, counting the code column sums only
 *   when code_colsum is not NULL) returns S3R_ERR_WORKSPACE and enqueues
 *   nothing.  32 MiB covers, with EC, T = 8192 tokens up to D = 14336 with
 *   code column sums, and larger T at smaller D.
 *   Concurrency: every call on one device shares its array, so calls that
 *   overlap in time on one device (different streams, or other threads'
 *   streams) race and give undefined results.  Calls in one stream's order
 *   are safe: nothing in the array has to start at zero, and no call depends
 *   on what an earlier call left there.
 */
#define S3R_NOALLOC_SCRATCH_BYTES (32u << 20)
int s3r_quantize_noalloc(const s3r_qdesc* desc,
                         const void* G, int32_t g_dtype, int64_t ld_g,
                         const float* row_scale, const float* col_scale,
                         int8_t* Q, int64_t ld_q, float* delta,
                         int32_t* code_colsum,
                         float* ec_row, float* ec_col, float* ec_mean,
                         uint32_t* flags, hipStream_t stream);

/* ---- backward GEMMs ----------------------------------------------------
 * Common: Q [T x D] int8 codes with ld_q, delta as written by s3r_quantize
 * (desc->scale selects [1] or [T]).  INT8 GEMMs on the MFMA units with int32
 * accumulation.  GEMM operands (Q, Wq, Xq) need 16-byte-aligned base
 * pointers, leading dims that are multiples of 16 and below 2^24, and
 * (rows + 320) * ld < 2^32 bytes; K <= 131072.
 * out_dt: S3R_F32 (dequantised, corrected per desc->ec), S3R_F32_ACC (the same,
 * added into the existing output; dX only) or S3R_I32_RAW (raw int32
 * accumulators, no dequantisation, no correction); the output's leading
 * dim must be below 2^22 and its base 4-byte aligned.
 *
 * s3r_backward_dx: dX [T x d_in] = diag(1/s_x) (Delta Q - P(E')) Wq.
 * S3R page, "Quantized Backpropagation" (activation-gradient product) and
 * "Two-Way Correction" (subtract the averages times W: v_b = ebar_b Wq, and
 * the token means times the row sums r_W).  The correction applies for
 * ec == DX_ONLY or TWO_WAY.
 *   Wq [D x d_in] int8 (ld_w), s_x [T] f32 (NULL = 1),
 *   r_W [d_in] int32 (required iff the correction applies), ec_* as from
 *   s3r_quantize.
 *   ws: s3r_backward_workspace(desc, d_in) bytes (dX needs none without EC).
 */
int s3r_backward_dx(const s3r_qdesc* desc,
                    const int8_t* Q, int64_t ld_q, const float* delta,
                    const int8_t* Wq, int64_t ld_w, int64_t d_in,
                    const float* s_x, const int32_t* r_W,
                    const float* ec_row, const float* ec_col, const float* ec_mean,
                    void* dX, int32_t out_dt, int64_t ld_dx,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_backward_dw: dW [D x d_in] = diag(1/s_w) (Delta Q - P(E'))^T Xq.
 * S3R page, "Quantized Backpropagation" (weight-gradient product) and
 * "Two-Way Correction" (subtract the inputs times the same averages:
 * sum_b ebar_b[j] xs_b[i] + sum_t (eps_t - mu_b) Xq[t,i]).  The correction
 * applies for ec == TWO_WAY or DW_ONLY.
 *   Xq [T x d_in] int8 (ld_x), s_w [D] f32 (NULL = 1),
 *   xs_b [B x d_in] int32 (required iff the correction applies).
 * Per-token steps (desc->scale == PER_TOKEN, delta [T]) are a reading beyond
 * the page, which explains that only a per-tensor step survives the S32
 * accumulation over the tokens: the steps are folded into the inputs,
 * Z = diag(Delta) Xq (fp32 products), Z is requantized per input column i with
 * the absmax RTNE rule (c_i = fl(max_t |Z[t,i]| / 127), codes
 * clamp(rint(fl(Z * fl(127 / max))), +-127); columns with a non-finite or
 * subnormal-range max get zero codes), and dW = diag(1/s_w) (Q^T Zq diag(c) -
 * correction).  Zq lives in the workspace; S3R_I32_RAW then returns Q^T Zq.
 * ws: s3r_backward_workspace(desc, d_in) bytes, 256-byte aligned (none is
 * needed for per-tensor steps without the two-way correction).
 */
int s3r_backward_dw(const s3r_qdesc* desc,
                    const int8_t* Q, int64_t ld_q, const float* delta,
                    const int8_t* Xq, int64_t ld_x, int64_t d_in,
                    const float* s_w, const int32_t* xs_b,
                    const float* ec_row, const float* ec_col, const float* ec_mean,
                    void* dW, int32_t out_dt, int64_t ld_dw,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_backward_dw_pair: the dW products of two projections of the same input
 * (the gate and up projections of a SwiGLU block), dW0 from (Q0, delta0, s_w0,
 * ec_*0) and dW1 from (Q1, delta1, s_w1, ec_*1), both against the shared input
 * codes Xq and column sums xs_b.  Each product is the one s3r_backward_dw
 * defines (same page passages), bit for bit; the two run as one GEMM launch, so
 * the GPU's compute units are filled by both products' tiles (a single product
 * whose tile count is not a multiple of the CU count leaves CUs idle in its last
 * round).  Both codes share desc (shape, ec, rows_per_example) and ld_q;
 * desc->scale must be PER_TENSOR (else S3R_ERR_UNSUPPORTED).  out_dt: S3R_F32
 * or S3R_I32_RAW; both outputs use ld_dw.
 *   ws: s3r_backward_dw_pair_workspace(desc, d_in) bytes, 256-byte aligned
 *   (the two correction GEMVs' halves; none without the dW correction).
 */
size_t s3r_backward_dw_pair_workspace(const s3r_qdesc* desc, int64_t d_in);
int s3r_backward_dw_pair(const s3r_qdesc* desc,
                         const int8_t* Q0, const int8_t* Q1, int64_t ld_q,
                         const float* delta0, const float* delta1,
                         const int8_t* Xq, int64_t ld_x, int64_t d_in,
                         const float* s_w0, const float* s_w1, const int32_t* xs_b,
                         const float* ec_row0, const float* ec_col0, const float* ec_mean0,
                         const float* ec_row1, const float* ec_col1, const float* ec_mean1,
                         void* dW0, void* dW1, int32_t out_dt, int64_t ld_dw,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace for either backward call (the larger of the two). */
size_t s3r_backward_workspace(const s3r_qdesc* desc, int64_t d_in);

/* ---- grouped (mixture-of-experts) calls ---------------------------------
 * The expert path of an MoE layer: every row-indexed tensor (G, Q, X, Xq, dX,
 * s_x, ec_row) holds its rows sorted by group (expert), group e owning rows
 * [offsets[e], offsets[e+1]).  Each group is one linear layer with its own
 * weight; its backward is the dense path above applied to its rows, with the
 * group as the one example of the correction.  S3R page, Table IV and the MoE
 * paragraph after it (the correction over the expert-sorted rows).
 *   groups   G, 1 .. 4096;
 *   offsets  DEVICE int64 [G+1], non-decreasing from 0 to desc->rows (the
 *            router's output stays on the device: grids are sized by bounds
 *            and each workgroup looks its group up).  If the offsets are not
 *            valid, S3R_FLAG_BAD_GROUPS is raised in *flags (when given) and
 *            nothing is computed: the outputs keep their contents.
 *   desc     rows = R (< 2^31) sorted rows, cols = D; rows_per_example is not
 *            used (pass 1); mode RTNE, SR or S3R (not S3R_BCAST); thresholds
 *            are keyed on the global row index exactly as in s3r_quantize.
 *   ws       s3r_grouped_workspace(desc, G, d_in) bytes serve all three calls
 *            (256-byte aligned).
 * Empty groups are allowed: their step is 1, their statistics 0, their dW 0.
 */
size_t s3r_grouped_workspace(const s3r_qdesc* desc, int64_t groups, int64_t d_in);

/* s3r_grouped_quantize: per-group per-tensor steps delta [G] (PER_TENSOR;
 * Delta_e = fl(max over the group's rows of |G'| / 127)), or per-row steps
 * delta [R] (PER_TOKEN).  col_scale [G x D] (each group's s_w) or NULL;
 * row_scale [R] or NULL.  ec_row [R], ec_col [G x D], ec_mean [G] as in
 * s3r_quantize with the group as the example (ec requires mode S3R).
 * code_colsum [G x D] (per-group column sums of the codes) only with
 * RTNE + PER_TOKEN + EC_NONE: the forward-operand prep of the experts' inputs
 * (the correction's xs_e). */
int s3r_grouped_quantize(const s3r_qdesc* desc, int64_t groups, const int64_t* offsets,
                         const void* G, int32_t g_dtype, int64_t ld_g,
                         const float* row_scale, const float* col_scale,
                         int8_t* Q, int64_t ld_q, float* delta, int32_t* code_colsum,
                         float* ec_row, float* ec_col, float* ec_mean,
                         uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_grouped_backward_dx: dX rows of group e = diag(1/s_x)(Delta_e Q_e - P(E'_e)) Wq_e.
 * Wq_e = Wq + e * w_group_stride bytes, each [D x d_in] with ld_w (16-byte
 * aligned stride >= D * ld_w); r_W [G x d_in] (each expert's code column sums);
 * delta [G] per-tensor steps (PER_TENSOR only).  Same operand rules, output
 * dtypes and correction variants as s3r_backward_dx. */
int s3r_grouped_backward_dx(const s3r_qdesc* desc, int64_t groups, const int64_t* offsets,
                            const int8_t* Q, int64_t ld_q, const float* delta,
                            const int8_t* Wq, int64_t ld_w, int64_t w_group_stride, int64_t d_in,
                            const float* s_x, const int32_t* r_W,
                            const float* ec_row, const float* ec_col, const float* ec_mean,
                            void* dX, int32_t out_dt, int64_t ld_dx, uint32_t* flags,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_grouped_backward_dw: dW_e = diag(1/s_w,e)(Delta_e Q_e - P(E'_e))^T Xq_e for
 * every group, into dW + e * dw_group_stride elements (each [D x d_in] with
 * ld_dw below 2^21, stride >= D * ld_dw).  s_w [G x D], xs [G x d_in]
 * (per-group column sums of Xq).  The groups run largest first.  PER_TENSOR
 * only. */
int s3r_grouped_backward_dw(const s3r_qdesc* desc, int64_t groups, const int64_t* offsets,
                            const int8_t* Q, int64_t ld_q, const float* delta,
                            const int8_t* Xq, int64_t ld_x, int64_t d_in,
                            const float* s_w, const int32_t* xs,
                            const float* ec_row, const float* ec_col, const float* ec_mean,
                            void* dW, int32_t out_dt, int64_t ld_dw, int64_t dw_group_stride, uint32_t* flags,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- SwiGLU FFN block glue --------------------------------------------
 * s3r_swiglu_backward: the gradients of H = silu(A_gate) * A_up with respect to
 * the two pre-activations, between the down projection's backward (dH) and the
 * gate / up projections' backward.  Not part of the method: the S3R page times
 * a whole SwiGLU FFN block ("Setup", single-block FFN benchmarks; Table III).
 *   G_up   = dH * silu(A_gate)
 *   G_gate = dH * A_up * silu'(A_gate),  silu'(a) = s (1 + a (1 - s)),  s = 1/(1 + exp(-a))
 * Arithmetic: fp32, one rounding per operation in exactly the order written
 * above, in which s = 1 / (1 + e) with e = exp(-a), silu = a * s, and
 * exp(x) = Taylor7(r) * 2^n with x clamped to [-104, 89], n = rint(x log2 e),
 * r = (x - n ln2_hi) - n ln2_lo (ln2_hi = 0.693145751953125,
 * ln2_lo = 1.4286068203094173e-6, Horner from 1/5040 down to 1); the results
 * are rounded to bf16 (nearest, ties to even; NaN -> 0x7FC0).
 *   dH [T x F] f32 (ld_dh), A_gate / A_up [T x F] bf16 bit patterns (ld_a),
 *   G_gate / G_up [T x F] bf16 bit patterns (ld_g), all device pointers,
 *   row-major.  16-byte-aligned pointers with ld_dh % 4 == 0 and
 *   ld_a, ld_g % 8 == 0 take the vector path; any layout is accepted.
 */
int s3r_swiglu_backward(int64_t T, int64_t F, const float* dH, int64_t ld_dh,
                        const uint16_t* A_gate, const uint16_t* A_up, int64_t ld_a,
                        uint16_t* G_gate, uint16_t* G_up, int64_t ld_g, hipStream_t stream);

/* s3r_swiglu_backward_amax: s3r_swiglu_backward (same arguments, arithmetic
 * and results) and, from the same pass, the per-tensor amax that the gate and
 * up projections' quantizers need, so that s3r_quantize_with_amax reads each
 * result once.  S3R page, "Quantized Backpropagation with Stochastic Rounding"
 * (the step of the folded gradient, Delta = max|G'|/127).
 *   row_scale [T] f32 (s_x of the block input) or NULL (= 1);
 *   col_scale_gate, col_scale_up [F] f32 (s_w of W_gate, W_up) or NULL.
 *   amax_bits [2] device uint32, written:
 *     [0] = max |fl(fl(G_gate[t,j] * s_x[t]) * s_w_gate[j])|,
 *     [1] = the same for G_up with s_w_up,
 *   over the bf16 results, as ordered fp32 bit patterns (NaN above every
 *   number; 0 for an empty tensor) -- the values s3r_quantize would find for
 *   G_gate and G_up with those scales.
 *   ws: s3r_swiglu_amax_workspace(T, F) bytes, 256-byte aligned (per-block
 *   partial maxima after the common 64 KiB header).
 */
size_t s3r_swiglu_amax_workspace(int64_t T, int64_t F);
int s3r_swiglu_backward_amax(int64_t T, int64_t F, const float* dH, int64_t ld_dh,
                             const uint16_t* A_gate, const uint16_t* A_up, int64_t ld_a,
                             uint16_t* G_gate, uint16_t* G_up, int64_t ld_g,
                             const float* row_scale, const float* col_scale_gate, const float* col_scale_up,
                             uint32_t* amax_bits, void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_swiglu_quantize: the gate and up projections' quantizers with the glue
 * computed inside them, so that G_gate and G_up are never written to memory.
 * S3R page, "Structured Subspace Randomness" (inter-operand sharing: the
 * quantized gradient is produced once, by one fused pass) and "Quantized
 * Backpropagation with Stochastic Rounding" (the per-tensor step of the folded
 * gradient).  One glue pass finds the two per-tensor maxima without storing
 * anything; a second pass computes the glue again and writes both projections'
 * codes and error statistics.  The results are exactly those of
 * s3r_swiglu_backward_amax followed by s3r_quantize_with_amax on G_gate (with
 * desc_gate, col_scale_gate) and on G_up (desc_up, col_scale_up): codes,
 * steps, flags and statistics, bit for bit.
 *   desc_gate, desc_up: rows = T, cols = F; both PER_TENSOR (else
 *     S3R_ERR_UNSUPPORTED); rows, cols, rows_per_example, mode and ec must be
 *     equal (else S3R_ERR_INVALID_ARG); layer_id, seed and stream may differ.
 *   dH, A_gate, A_up, ld_dh, ld_a: as s3r_swiglu_backward (device pointers).
 *   row_scale [T] (s_x of the block input, shared by both projections) or NULL;
 *   col_scale_gate, col_scale_up [F] (s_w of W_gate, W_up) or NULL.
 *   Q_gate, Q_up [T x F] int8, one leading dim ld_q >= F; delta_gate,
 *   delta_up [1]; ec_* as s3r_quantize for each projection (required iff
 *   ec != NONE, NULL otherwise); flags: S3R_FLAG_* of both are OR-ed in.
 *   ws: s3r_swiglu_quantize_workspace(desc_gate) bytes, 256-byte aligned.
 * 16-byte-aligned dH, A_gate, A_up and column scales with ld_dh % 4 == 0,
 * ld_a % 8 == 0, 8-byte-aligned codes with ld_q % 8 == 0 take the vector path;
 * any layout is accepted.
 */
size_t s3r_swiglu_quantize_workspace(const s3r_qdesc* desc_gate);
int s3r_swiglu_quantize(const s3r_qdesc* desc_gate, const s3r_qdesc* desc_up,
                        const float* dH, int64_t ld_dh,
                        const uint16_t* A_gate, const uint16_t* A_up, int64_t ld_a,
                        const float* row_scale, const float* col_scale_gate, const float* col_scale_up,
                        int8_t* Q_gate, int8_t* Q_up, int64_t ld_q, float* delta_gate, float* delta_up,
                        float* ec_row_gate, float* ec_col_gate, float* ec_mean_gate,
                        float* ec_row_up, float* ec_col_up, float* ec_mean_up,
                        uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- MXFP4 variant ------------------------------------------------------
 * The 4-bit setting the S3R page names as the one where deterministic
 * rounding of the backward fails (Introduction; Related Work, on NVFP4 /
 * MXFP4 training recipes).  The page fixes none of the 4-bit arithmetic; the
 * readings (OCP microscaling MXFP4 with the page's rounding carried over):
 *   codes    E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; code = sign << 3 |
 *            index), two per byte, the first element in the low nibble;
 *            a matrix of R rows and K (contraction) elements is stored in
 *            blocks of 256 rows x 128 elements (64 bytes a row, 16384 bytes a
 *            block, row-major inside): block (rb, kb) starts at rb * ld +
 *            kb * 16384, so element (r, k) is the nibble k % 2 of byte
 *            (r / 256) * ld + (k / 128) * 16384 + (r % 256) * 64 + (k % 128) / 2.
 *            ld, the bytes between 256-row blocks, is a multiple of 16384 and
 *            at least 128 K; the buffer holds ceil(R / 256) * ld bytes (rows
 *            past R in the last block are never written and their contents
 *            reach no result).  A GEMM step of a 256-row tile is then one
 *            contiguous 16 KiB run;
 *   scales   one E8M0 byte per 32 consecutive elements along a GEMM's
 *            contraction, grouped by steps of 128: the K/128 steps are rows of
 *            ld_s bytes, step j holding R 4-byte words (row r's blocks 4j ..
 *            4j+3), so the scale of (row r, block b) is at
 *            (b / 4) * ld_s + 4 r + b % 4  (ld_s >= 4 R, a multiple of 4);
 *            the value is 2^k with k the smallest integer such that
 *            max|block| <= 6 * 2^k (nothing saturates), clamped to
 *            [-127, 127]; an all-zero block has k = -127; a block with a
 *            non-finite element gets byte 255 (NaN), zero codes and
 *            S3R_FLAG_NONFINITE;
 *   rounding y = g / 2^k onto the grid with spacing s (0.5 below |y| 2, 1
 *            below 4, 2 up to 6): RTNE s * rint(y / s); SR and S3R the exact
 *            floor s * floor(y / s + r) with the thresholds of s3r_quantize
 *            (same Philox counters, same element and token indices);
 *   layout   every GEMM operand is K-major: G is quantized twice, Q_h [T x D]
 *            blocked along D (the dX operand) and Q_t [D x T] = G^T blocked
 *            along T (the dW operand), both with the same thresholds; the
 *            forward operands are stored transposed (Wt [d_in x D] from W
 *            [D x d_in], Xt [d_in x T] from X [T x d_in]), RTNE;
 *   EC       S3R-EC per quantization on E = dequant(Q) - G, with the INT8
 *            path's statistics (eps_t, ebar_b, mu_b) and projection, all in
 *            dequantized units (no per-token / per-channel scale folding: the
 *            block scales take its place).
 * Shapes: T, D and rows_per_example multiples of 128 (a 128-element step of
 * the FP4 matrix cores), T, D < 2^24; scale must be S3R_PER_TENSOR (it names
 * no scale here); mode RTNE, SR or S3R; ec requires S3R.  Codes: 16-byte
 * aligned bases, ld_* as above, ceil(R / 256) * ld_* < 2^32.  Scales: byte
 * leading dimensions that are multiples of 4 with 4-byte aligned bases (a GEMM
 * step reads its rows' scale words as one contiguous run).
 * Device pointers throughout, row-major.
 */

/* s3r_mx_workspace: bytes of ws for s3r_mx_quantize and both backward calls
 * (256-byte aligned; no initial contents required). */
size_t s3r_mx_workspace(const s3r_qdesc* desc, int64_t d_in);
size_t s3r_mx_operand_workspace(int64_t rows, int64_t cols);

/* s3r_mx_operand: the forward operand M [rows x cols] (f32 or bf16, ld
 * elements) to RTNE MXFP4 blocked along the rows, stored transposed: Mt, the
 * codes of cols rows x rows elements (block layout, ld_t), Mt_scales
 * [rows/128][cols][4] (ld_ts bytes per step).
 * W [D x d_in] gives Wt for dX, X [T x d_in] gives Xt for dW.  colsum
 * (optional, f32 [rows/rows_per_example x cols]): per-group column sums of the
 * dequantized operand in groups of rows_per_example rows (a multiple of 128
 * dividing rows) -- r_W with rows_per_example = D, xs_b with the examples'
 * length.  rows a multiple of 128. */
int s3r_mx_operand(int64_t rows, int64_t cols, int64_t rows_per_example,
                   const void* M, int32_t dtype, int64_t ld,
                   uint8_t* Mt, int64_t ld_t, uint8_t* Mt_scales, int64_t ld_ts,
                   float* colsum, uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_mx_quantize: G [T x D] (f32 or bf16) to Q_h (codes of T rows x D
 * elements, scales [D/128][T][4]) and Q_t (codes of D rows x T elements,
 * scales [T/128][D][4]), codes in the block layout.  G is read
 * in 16-byte pieces: its base is 16-byte aligned and ld_g a multiple of 8
 * (bf16) or 4 (f32) elements.  With EC: the
 * statistics of each quantization's error, ec_row_* [T] (eps_t), ec_col_*
 * [B x D] (ebar_b), ec_mean_* [B] (mu_b); all six pointers given exactly when
 * desc->ec != S3R_EC_NONE.  Both quantizations are written whatever the
 * variant. */
int s3r_mx_quantize(const s3r_qdesc* desc, const void* G, int32_t g_dtype, int64_t ld_g,
                    uint8_t* Qh, int64_t ld_qh, uint8_t* Qh_scales, int64_t ld_qhs,
                    uint8_t* Qt, int64_t ld_qt, uint8_t* Qt_scales, int64_t ld_qts,
                    float* ec_row_h, float* ec_col_h, float* ec_mean_h,
                    float* ec_row_t, float* ec_col_t, float* ec_mean_t,
                    uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_mx_backward_dx: dX [T x d_in] f32 = dq(Q_h) dq(W) - v_b - (eps_t - mu_b) r_W
 * with v_b = ebar_b dq(W) (S3R page, "Structured Error Correction": the
 * projection's two terms); the correction only with ec DX_ONLY or TWO_WAY,
 * which need r_W [d_in] (s3r_mx_operand's colsum of W with rows_per_example
 * = D) and the _h statistics.  fp32 accumulation in the matrix cores. */
int s3r_mx_backward_dx(const s3r_qdesc* desc, const uint8_t* Qh, int64_t ld_qh,
                       const uint8_t* Qh_scales, int64_t ld_qhs,
                       const uint8_t* Wt, int64_t ld_wt, const uint8_t* Wt_scales, int64_t ld_wts,
                       int64_t d_in, const float* r_W,
                       const float* ec_row_h, const float* ec_col_h, const float* ec_mean_h,
                       float* dX, int64_t ld_dx, void* ws, size_t ws_bytes, hipStream_t stream);

/* s3r_mx_backward_dw: dW [D x d_in] f32 = dq(G)^T dq(X), from Q_t and Xt,
 * minus sum_b ebar'_b xs_b^T and 1 u'^T with u' = sum_t (eps'_t - mu'_b)
 * dq(X)[t,:] (the _t statistics); the correction only with ec TWO_WAY or
 * DW_ONLY, which need xs [B x d_in] (s3r_mx_operand's colsum of X with the
 * examples' length), B = T / rows_per_example.  The GEMM epilogue applies the
 * first eight examples' terms and a rank-update pass the rest. */
int s3r_mx_backward_dw(const s3r_qdesc* desc, const uint8_t* Qt, int64_t ld_qt,
                       const uint8_t* Qt_scales, int64_t ld_qts,
                       const uint8_t* Xt, int64_t ld_xt, const uint8_t* Xt_scales, int64_t ld_xts,
                       int64_t d_in, const float* xs,
                       const float* ec_row_t, const float* ec_col_t, const float* ec_mean_t,
                       float* dW, int64_t ld_dw, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- measurement aid --------------------------------------------------
 * s3r_time_next_gemm: record `start` immediately before and `stop` immediately
 * after the GEMM kernel launched by the next s3r_backward_dx / s3r_backward_dw
 * (INT8) or s3r_mx_backward_dx / s3r_mx_backward_dw (FP4) call made on this
 * host thread (on that call's stream), so
 * hipEventElapsedTime gives that one kernel's duration.  Thread-local; the
 * request is consumed by that call.  Pass NULLs to cancel.  Returns S3R_OK. */
int s3r_time_next_gemm(hipEvent_t start, hipEvent_t stop);

/* ---- misc -------------------------------------------------------------- */
const char* s3r_status_string(int status);
int s3r_version(void);   /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* S3R_H */
