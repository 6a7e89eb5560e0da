// C ABI of libs3r.so (declared in include/s3r.h): argument checks on the host,
// then asynchronous launches on the caller's stream.  Nothing here allocates
// or synchronises.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "s3r_internal.h"

namespace {

using namespace s3r;

constexpr int64_t kMaxK = 131072;   // int32 accumulators: K * 127^2 < 2^31
constexpr int64_t kMaxLdOut = (int64_t)1 << 22;   // one 256-row output tile stays below 2^32 bytes

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Current device must be gfx950.  The answer is cached per device id.
int check_arch() {
  static std::mutex mu;
  static int cache[64];  // 0 unknown, 1 ok, 2 not gfx950
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S3R_ERR_HIP;
  if (dev < 0 || dev >= 64) return S3R_ERR_ARCH;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return S3R_ERR_HIP;
    cache[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  return cache[dev] == 1 ? S3R_OK : S3R_ERR_ARCH;
}

int check_desc(const s3r_qdesc* d) {
  if (!d) return S3R_ERR_INVALID_ARG;
  if (d->rows < 0 || d->cols < 0 || d->rows_per_example < 1) return S3R_ERR_INVALID_ARG;
  if (d->rows % d->rows_per_example != 0) return S3R_ERR_INVALID_ARG;
  if (d->rows > (int64_t)1 << 31 || d->cols > (int64_t)1 << 31) return S3R_ERR_INVALID_ARG;
  if (d->mode < S3R_RTNE || d->mode > S3R_S3R_BCAST) return S3R_ERR_UNSUPPORTED;
  if (d->ec < S3R_EC_NONE || d->ec > S3R_EC_DW_ONLY) return S3R_ERR_UNSUPPORTED;
  if (d->scale != S3R_PER_TENSOR && d->scale != S3R_PER_TOKEN) return S3R_ERR_UNSUPPORTED;
  if (d->stream > 65535 || d->reserved != 0) return S3R_ERR_INVALID_ARG;
  return S3R_OK;
}

bool shared_threshold(int mode) { return mode == S3R_S3R || mode == S3R_S3R_BCAST; }
bool dx_corrected(int ec) { return ec == S3R_EC_DX_ONLY || ec == S3R_EC_TWO_WAY; }
bool dw_corrected(int ec) { return ec == S3R_EC_TWO_WAY || ec == S3R_EC_DW_ONLY;
}

int finish(hipError_t e) { return e == hipSuccess ? S3R_OK : S3R_ERR_HIP; }

// s3r_quantize's checks and launch, for a workspace of ws_bytes of which the call needs `need`.
int quantize_checked(const s3r_qdesc* d, const void* G, int32_t g_dtype, int64_t ld_g, const float* row_scale,
                     const float* col_scale, int8_t* Q, int64_t ld_q, float* delta, int32_t* code_colsum,
                     float* ec_row, float* ec_col, float* ec_mean, uint32_t* flags, void* ws, size_t ws_bytes,
                     size_t need, hipStream_t stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (g_dtype != S3R_F32 && g_dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  if (d->ec != S3R_EC_NONE && !shared_threshold(d->mode)) return S3R_ERR_UNSUPPORTED;
  const int64_t T = d->rows, D = d->cols;
  const bool nonempty = T > 0 && D > 0;
  const int64_t B = T / d->rows_per_example;
  // a pointer is required exactly when its output is nonempty (empty tensors may be NULL)
  if (!delta && (d->scale == S3R_PER_TENSOR || T > 0)) return S3R_ERR_INVALID_ARG;
  if (nonempty && (!G || !Q)) return S3R_ERR_INVALID_ARG;
  if (ld_g < D || ld_q < D || ld_g < 0 || ld_q < 0) return S3R_ERR_INVALID_ARG;
  if (d->ec != S3R_EC_NONE) {
    if ((T > 0 && !ec_row) || (B * D > 0 && !ec_col) || (B > 0 && !ec_mean)) return S3R_ERR_INVALID_ARG;
  } else if (ec_row || ec_col || ec_mean) {
    return S3R_ERR_INVALID_ARG;
  }
  if (ws_bytes < need) return S3R_ERR_WORKSPACE;
  if (need > 0 && (!ws || ((uintptr_t)ws & 255u))) return S3R_ERR_INVALID_ARG;
  if ((rc = check_arch())) return rc;
  QuantArgs a{};
  a.G = G; a.g_dtype = g_dtype; a.ld_g = ld_g; a.sx = row_scale; a.sw = col_scale;
  a.Q = Q; a.ld_q = ld_q; a.delta = delta; a.code_colsum = code_colsum;
  a.ec_row = ec_row; a.ec_col = ec_col; a.ec_mean = ec_mean; a.flags = flags;
  a.T = T; a.D = D; a.S = d->rows_per_example;
  a.mode = d->mode; a.ec = d->ec; a.scale = d->scale; a.layer = d->layer_id; a.seed = d->seed;
  a.stream = d->stream;
  a.ws = (char*)ws;
  return finish(launch_quantize(a, stream));
}

// Scratch of s3r_quantize_noalloc, for callers that cannot allocate: one array on every device the library
// runs on, kept until the process ends.  Its host-side name is not a device address: host code uses only
// the address hipGetSymbolAddress returns for the current device, taken once per device.  Every call on a
// device shares that device's array; the quantize kernels write every partial they read (the finalize
// counter is reset by the code pass), so nothing in it has to start at zero.
__device__ __align__(256) uint8_t scratch[S3R_NOALLOC_SCRATCH_BYTES];

int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S3R_ERR_HIP;
  if (dev < 0 || dev >= 64) return S3R_ERR_ARCH;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return S3R_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return S3R_OK;
}

}  // namespace

extern "C" {

size_t s3r_quantize_workspace(const s3r_qdesc* d) {
  if (check_desc(d) != S3R_OK) return 0;
  return quant_workspace(d->rows, d->cols, d->rows_per_example, d->ec != S3R_EC_NONE, d->scale, true);
}

int s3r_quantize(const s3r_qdesc* d, const void* G, int32_t g_dtype, int64_t ld_g, const float* row_scale,
                 const float* col_scale, int8_t* Q, int64_t ld_q, float* delta, int32_t* code_colsum,
                 float* ec_row, float* ec_col, float* ec_mean, uint32_t* flags, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  return quantize_checked(d, G, g_dtype, ld_g, row_scale, col_scale, Q, ld_q, delta, code_colsum, ec_row, ec_col,
                          ec_mean, flags, ws, ws_bytes, s3r_quantize_workspace(d), stream);
}

int s3r_quantize_noalloc(const s3r_qdesc* d, const void* G, int32_t g_dtype, int64_t ld_g, const float* row_scale,
                         const float* col_scale, int8_t* Q, int64_t ld_q, float* delta, int32_t* code_colsum,
                         float* ec_row, float* ec_col, float* ec_mean, uint32_t* flags, hipStream_t stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  // the scratch this call needs (its code column sums only if asked for), against the array's size
  const size_t need = quant_workspace(d->rows, d->cols, d->rows_per_example, d->ec != S3R_EC_NONE, d->scale,
                                      code_colsum != nullptr);
  if (need > (size_t)S3R_NOALLOC_SCRATCH_BYTES) return S3R_ERR_WORKSPACE;
  if ((rc = check_arch())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return quantize_checked(d, G, g_dtype, ld_g, row_scale, col_scale, Q, ld_q, delta, code_colsum, ec_row, ec_col,
                          ec_mean, flags, ws, S3R_NOALLOC_SCRATCH_BYTES, need, stream);
}

int s3r_quantize_with_amax(const s3r_qdesc* d, const void* G, int32_t g_dtype, int64_t ld_g, const float* row_scale,
                           const float* col_scale, const uint32_t* amax_bits, int8_t* Q, int64_t ld_q, float* delta,
                           float* ec_row, float* ec_col, float* ec_mean, uint32_t* flags, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->scale != S3R_PER_TENSOR) return S3R_ERR_UNSUPPORTED;
  if (!amax_bits) return S3R_ERR_INVALID_ARG;
  if (d->rows == 0 || d->cols == 0)   // nothing to quantize: the step of an empty tensor is 1
    return s3r_quantize(d, G, g_dtype, ld_g, row_scale, col_scale, Q, ld_q, delta, nullptr, ec_row, ec_col, ec_mean,
                        flags, ws, ws_bytes, stream);
  if (g_dtype != S3R_F32 && g_dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  if (d->ec != S3R_EC_NONE && !shared_threshold(d->mode)) return S3R_ERR_UNSUPPORTED;
  const int64_t T = d->rows, D = d->cols;
  const int64_t B = T / d->rows_per_example;
  if (!delta || !G || !Q) return S3R_ERR_INVALID_ARG;
  if (ld_g < D || ld_q < D) return S3R_ERR_INVALID_ARG;
  if (d->ec != S3R_EC_NONE) {
    if (!ec_row || (B * D > 0 && !ec_col) || (B > 0 && !ec_mean)) return S3R_ERR_INVALID_ARG;
  } else if (ec_row || ec_col || ec_mean) {
    return S3R_ERR_INVALID_ARG;
  }
  const size_t need = s3r_quantize_workspace(d);
  if (ws_bytes < need) return S3R_ERR_WORKSPACE;
  if (need > 0 && (!ws || ((uintptr_t)ws & 255u))) return S3R_ERR_INVALID_ARG;
  if ((rc = check_arch())) return rc;
  QuantArgs a{};
  a.G = G; a.g_dtype = g_dtype; a.ld_g = ld_g; a.sx = row_scale; a.sw = col_scale;
  a.Q = Q; a.ld_q = ld_q; a.delta = delta; a.code_colsum = nullptr;
  a.ec_row = ec_row; a.ec_col = ec_col; a.ec_mean = ec_mean; a.flags = flags;
  a.T = T; a.D = D; a.S = d->rows_per_example;
  a.mode = d->mode; a.ec = d->ec; a.scale = d->scale; a.layer = d->layer_id; a.seed = d->seed;
  a.stream = d->stream;
  a.ws = (char*)ws;
  a.amax_in = amax_bits;
  return finish(launch_quantize(a, stream));
}

size_t s3r_backward_workspace(const s3r_qdesc* d, int64_t d_in) {
  if (check_desc(d) != S3R_OK || d_in < 0) return 0;
  const size_t a = dx_workspace(d->rows, d->cols, d_in, d->rows_per_example, dx_corrected(d->ec) ? d->ec : 0);
  const size_t b = dw_workspace(d->rows, d->cols, d_in, d->rows_per_example, dw_corrected(d->ec) ? d->ec : 0,
                                d->scale == S3R_PER_TOKEN);
  return a > b ? a : b;
}

size_t s3r_backward_dw_pair_workspace(const s3r_qdesc* d, int64_t d_in) {
  if (check_desc(d) != S3R_OK || d_in < 0 || d->scale != S3R_PER_TENSOR) return 0;
  return 2 * align_up(dw_workspace(d->rows, d->cols, d_in, d->rows_per_example, dw_corrected(d->ec) ? d->ec : 0, 0),
                      256);
}

static int check_gemm_operand(const int8_t* p, int64_t ld, int64_t rows, int64_t cols, bool nonempty) {
  // the GEMM addresses each operand through a buffer descriptor with 32-bit byte
  // offsets, including up to one tile (256 rows, 64 k-rows) past the last row
  if (ld < cols || ld < 0 || ld >= ((int64_t)1 << 24)) return S3R_ERR_INVALID_ARG;
  if ((rows + 320) * ld >= ((int64_t)1 << 32)) return S3R_ERR_INVALID_ARG;
  if (nonempty && (!p || !al16(p) || (ld & 15))) return S3R_ERR_INVALID_ARG;
  return S3R_OK;
}

int s3r_backward_dx(const s3r_qdesc* d, const int8_t* Q, int64_t ld_q, const float* delta, const int8_t* Wq,
                    int64_t ld_w, int64_t d_in, const float* s_x, const int32_t* r_W, const float* ec_row,
                    const float* ec_col, const float* ec_mean, void* dX, int32_t out_dt, int64_t ld_dx, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (out_dt != S3R_F32 && out_dt != S3R_I32_RAW && out_dt != S3R_F32_ACC) return S3R_ERR_UNSUPPORTED;
  const int64_t T = d->rows, D = d->cols;
  if (d_in < 0 || D > kMaxK) return S3R_ERR_INVALID_ARG;
  const bool out_nonempty = T > 0 && d_in > 0;
  if (!delta || (out_nonempty && !dX) || ld_dx < d_in || ld_dx >= kMaxLdOut) return S3R_ERR_INVALID_ARG;
  if (out_nonempty && ((uintptr_t)dX & 3u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_gemm_operand(Q, ld_q, T, D, T > 0 && D > 0))) return rc;
  if ((rc = check_gemm_operand(Wq, ld_w, D, d_in, D > 0 && d_in > 0))) return rc;
  const bool ec = dx_corrected(d->ec) && out_dt != S3R_I32_RAW;
  if (ec && (!r_W || !ec_row || !ec_col || !ec_mean)) return S3R_ERR_INVALID_ARG;
  const size_t need = ec ? dx_workspace(T, D, d_in, d->rows_per_example, d->ec) : 0;
  if (ws_bytes < need || (need && (!ws || ((uintptr_t)ws & 255u)))) return S3R_ERR_WORKSPACE;
  if ((rc = check_arch())) return rc;
  DxArgs a{};
  a.Q = Q; a.ld_q = ld_q; a.delta = delta; a.per_token = d->scale == S3R_PER_TOKEN;
  a.W = Wq; a.ld_w = ld_w; a.T = T; a.D = D; a.d_in = d_in; a.S = d->rows_per_example;
  a.sx = s_x; a.rW = r_W; a.ec_row = ec_row; a.ec_col = ec_col; a.ec_mean = ec_mean; a.ec = ec ? d->ec : 0;
  a.out = dX; a.out_dt = out_dt; a.ld_out = ld_dx; a.ws = (char*)ws;
  return finish(launch_backward_dx(a, stream));
}

int s3r_backward_dw(const s3r_qdesc* d, const int8_t* Q, int64_t ld_q, const float* delta, const int8_t* Xq,
                    int64_t ld_x, int64_t d_in, const float* s_w, const int32_t* xs_b, const float* ec_row,
                    const float* ec_col, const float* ec_mean, void* dW, int32_t out_dt, int64_t ld_dw, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (out_dt != S3R_F32 && out_dt != S3R_I32_RAW) return S3R_ERR_UNSUPPORTED;
  const int64_t T = d->rows, D = d->cols;
  if (d_in < 0 || T > kMaxK) return S3R_ERR_INVALID_ARG;
  const bool out_nonempty = D > 0 && d_in > 0;
  if (!delta || (out_nonempty && !dW) || ld_dw < d_in || ld_dw >= kMaxLdOut) return S3R_ERR_INVALID_ARG;
  if (out_nonempty && ((uintptr_t)dW & 3u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_gemm_operand(Q, ld_q, T, D, T > 0 && D > 0))) return rc;
  if ((rc = check_gemm_operand(Xq, ld_x, T, d_in, T > 0 && d_in > 0))) return rc;
  const bool ec = dw_corrected(d->ec) && out_dt == S3R_F32;
  if (ec && (!xs_b || !ec_row || !ec_col || !ec_mean)) return S3R_ERR_INVALID_ARG;
  const int per_token = d->scale == S3R_PER_TOKEN;
  const size_t need = dw_workspace(T, D, d_in, d->rows_per_example, ec ? d->ec : 0, per_token);
  if (ws_bytes < need || (need && (!ws || ((uintptr_t)ws & 255u)))) return S3R_ERR_WORKSPACE;
  if ((rc = check_arch())) return rc;
  DwArgs a{};
  a.Q = Q; a.ld_q = ld_q; a.delta = delta; a.per_token = per_token; a.X = Xq; a.ld_x = ld_x;
  a.T = T; a.D = D; a.d_in = d_in; a.S = d->rows_per_example;
  a.sw = s_w; a.xs = xs_b; a.ec_row = ec_row; a.ec_col = ec_col; a.ec_mean = ec_mean; a.ec = ec ? d->ec : 0;
  a.out = dW; a.out_dt = out_dt; a.ld_out = ld_dw; a.ws = (char*)ws;
  return finish(launch_backward_dw(a, stream));
}

int s3r_backward_dw_pair(const s3r_qdesc* d, const int8_t* Q0, const int8_t* Q1, int64_t ld_q, const float* delta0,
                         const float* delta1, const int8_t* Xq, int64_t ld_x, int64_t d_in, const float* s_w0,
                         const float* s_w1, const int32_t* xs_b, const float* ec_row0, const float* ec_col0,
                         const float* ec_mean0, const float* ec_row1, const float* ec_col1, const float* ec_mean1,
                         void* dW0, void* dW1, int32_t out_dt, int64_t ld_dw, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (out_dt != S3R_F32 && out_dt != S3R_I32_RAW) return S3R_ERR_UNSUPPORTED;
  if (d->scale != S3R_PER_TENSOR) return S3R_ERR_UNSUPPORTED;
  const int64_t T = d->rows, D = d->cols;
  if (d_in < 0 || T > kMaxK) return S3R_ERR_INVALID_ARG;
  const bool out_nonempty = D > 0 && d_in > 0;
  if (!delta0 || !delta1 || (out_nonempty && (!dW0 || !dW1)) || ld_dw < d_in || ld_dw >= kMaxLdOut)
    return S3R_ERR_INVALID_ARG;
  if (out_nonempty && (((uintptr_t)dW0 | (uintptr_t)dW1) & 3u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_gemm_operand(Q0, ld_q, T, D, T > 0 && D > 0))) return rc;
  if ((rc = check_gemm_operand(Q1, ld_q, T, D, T > 0 && D > 0))) return rc;
  if ((rc = check_gemm_operand(Xq, ld_x, T, d_in, T > 0 && d_in > 0))) return rc;
  const bool ec = dw_corrected(d->ec) && out_dt == S3R_F32;
  if (ec && (!xs_b || !ec_row0 || !ec_col0 || !ec_mean0 || !ec_row1 || !ec_col1 || !ec_mean1))
    return S3R_ERR_INVALID_ARG;
  const size_t one = align_up(dw_workspace(T, D, d_in, d->rows_per_example, ec ? d->ec : 0, 0), 256);
  if (ws_bytes < 2 * one || (one && (!ws || ((uintptr_t)ws & 255u)))) return S3R_ERR_WORKSPACE;
  if ((rc = check_arch())) return rc;
  DwArgs a[2]{};
  const int8_t* Q[2] = {Q0, Q1};
  const float* delta[2] = {delta0, delta1};
  const float* s_w[2] = {s_w0, s_w1};
  const float* er[2] = {ec_row0, ec_row1};
  const float* ecol[2] = {ec_col0, ec_col1};
  const float* em[2] = {ec_mean0, ec_mean1};
  void* out[2] = {dW0, dW1};
  for (int i = 0; i < 2; ++i) {
    a[i].Q = Q[i]; a[i].ld_q = ld_q; a[i].delta = delta[i]; a[i].per_token = 0; a[i].X = Xq; a[i].ld_x = ld_x;
    a[i].T = T; a[i].D = D; a[i].d_in = d_in; a[i].S = d->rows_per_example;
    a[i].sw = s_w[i]; a[i].xs = xs_b; a[i].ec_row = er[i]; a[i].ec_col = ecol[i]; a[i].ec_mean = em[i];
    a[i].ec = ec ? d->ec : 0;
    a[i].out = out[i]; a[i].out_dt = out_dt; a[i].ld_out = ld_dw; a[i].ws = (char*)ws + i * one;
  }
  return finish(launch_backward_dw_pair(a[0], a[1], stream));
}

int s3r_swiglu_backward(int64_t T, int64_t F, const float* dH, int64_t ld_dh, const uint16_t* A_gate,
                        const uint16_t* A_up, int64_t ld_a, uint16_t* G_gate, uint16_t* G_up, int64_t ld_g,
                        hipStream_t stream) {
  if (T < 0 || F < 0 || ld_dh < F || ld_a < F || ld_g < F) return S3R_ERR_INVALID_ARG;
  if (T > 0 && F > 0 && (!dH || !A_gate || !A_up || !G_gate || !G_up)) return S3R_ERR_INVALID_ARG;
  int rc;
  if ((rc = check_arch())) return rc;
  return finish(launch_swiglu_backward(T, F, dH, ld_dh, A_gate, A_up, ld_a, G_gate, G_up, ld_g, stream));
}

size_t s3r_swiglu_amax_workspace(int64_t T, int64_t F) {
  if (T < 0 || F < 0) return 0;
  return swiglu_amax_workspace(T, F);
}

int s3r_swiglu_backward_amax(int64_t T, int64_t F, const float* dH, int64_t ld_dh, const uint16_t* A_gate,
                             const uint16_t* A_up, int64_t ld_a, uint16_t* G_gate, uint16_t* G_up, int64_t ld_g,
                             const float* row_scale, const float* col_scale_gate, const float* col_scale_up,
                             uint32_t* amax_bits, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || F < 0 || ld_dh < F || ld_a < F || ld_g < F) return S3R_ERR_INVALID_ARG;
  if (T > 0 && F > 0 && (!dH || !A_gate || !A_up || !G_gate || !G_up)) return S3R_ERR_INVALID_ARG;
  if (!amax_bits) return S3R_ERR_INVALID_ARG;
  if (ws_bytes < swiglu_amax_workspace(T, F)) return S3R_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return S3R_ERR_INVALID_ARG;
  int rc;
  if ((rc = check_arch())) return rc;
  return finish(launch_swiglu_backward_amax(T, F, dH, ld_dh, A_gate, A_up, ld_a, G_gate, G_up, ld_g, row_scale,
                                            col_scale_gate, col_scale_up, amax_bits, (char*)ws, stream));
}

size_t s3r_swiglu_quantize_workspace(const s3r_qdesc* d) {
  if (check_desc(d) != S3R_OK || d->scale != S3R_PER_TENSOR) return 0;
  return swiglu_quant_workspace(d->rows, d->cols, d->rows_per_example, d->ec != S3R_EC_NONE);
}

int s3r_swiglu_quantize(const s3r_qdesc* dg, const s3r_qdesc* du, const float* dH, int64_t ld_dh,
                        const uint16_t* A_gate, const uint16_t* A_up, int64_t ld_a, const float* row_scale,
                        const float* col_scale_gate, const float* col_scale_up, int8_t* Q_gate, int8_t* Q_up,
                        int64_t ld_q, float* delta_gate, float* delta_up, float* ec_row_gate, float* ec_col_gate,
                        float* ec_mean_gate, float* ec_row_up, float* ec_col_up, float* ec_mean_up, uint32_t* flags,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc;
  if (!dg || !du) return S3R_ERR_INVALID_ARG;
  if ((rc = check_desc(dg)) || (rc = check_desc(du))) return rc;
  if (dg->scale != S3R_PER_TENSOR || du->scale != S3R_PER_TENSOR) return S3R_ERR_UNSUPPORTED;
  if (dg->rows != du->rows || dg->cols != du->cols || dg->rows_per_example != du->rows_per_example ||
      dg->mode != du->mode || dg->ec != du->ec)
    return S3R_ERR_INVALID_ARG;
  if (dg->ec != S3R_EC_NONE && !shared_threshold(dg->mode)) return S3R_ERR_UNSUPPORTED;
  const int64_t T = dg->rows, F = dg->cols;
  const int64_t B = T / dg->rows_per_example;
  if (ld_dh < F || ld_a < F || ld_q < F) return S3R_ERR_INVALID_ARG;
  if (T > 0 && F > 0 && (!dH || !A_gate || !A_up || !Q_gate || !Q_up)) return S3R_ERR_INVALID_ARG;
  if (!delta_gate || !delta_up) return S3R_ERR_INVALID_ARG;
  float* ec_row[2] = {ec_row_gate, ec_row_up};
  float* ec_col[2] = {ec_col_gate, ec_col_up};
  float* ec_mean[2] = {ec_mean_gate, ec_mean_up};
  for (int k = 0; k < 2; ++k) {
    if (dg->ec != S3R_EC_NONE) {
      if ((T > 0 && !ec_row[k]) || (B * F > 0 && !ec_col[k]) || (B > 0 && !ec_mean[k])) return S3R_ERR_INVALID_ARG;
    } else if (ec_row[k] || ec_col[k] || ec_mean[k]) {
      return S3R_ERR_INVALID_ARG;
    }
  }
  const size_t need = s3r_swiglu_quantize_workspace(dg);
  if (ws_bytes < need) return S3R_ERR_WORKSPACE;
  if (need > 0 && (!ws || ((uintptr_t)ws & 255u))) return S3R_ERR_INVALID_ARG;
  if ((rc = check_arch())) return rc;
  SwigluQuantArgs a{};
  a.dH = dH; a.ld_dh = ld_dh; a.Ag = A_gate; a.Au = A_up; a.ld_a = ld_a;
  a.sx = row_scale; a.sw[0] = col_scale_gate; a.sw[1] = col_scale_up;
  a.Q[0] = Q_gate; a.Q[1] = Q_up; a.ld_q = ld_q; a.delta[0] = delta_gate; a.delta[1] = delta_up;
  for (int k = 0; k < 2; ++k) { a.ec_row[k] = ec_row[k]; a.ec_col[k] = ec_col[k]; a.ec_mean[k] = ec_mean[k]; }
  a.flags = flags;
  a.T = T; a.D = F; a.S = dg->rows_per_example; a.mode = dg->mode; a.ec = dg->ec != S3R_EC_NONE;
  a.layer[0] = dg->layer_id; a.layer[1] = du->layer_id;
  a.seed[0] = dg->seed; a.seed[1] = du->seed;
  a.stream[0] = dg->stream; a.stream[1] = du->stream;
  a.ws = (char*)ws;
  return finish(launch_swiglu_quantize(a, stream));
}

// ---- grouped (MoE expert) calls
static int check_groups(const s3r_qdesc* d, int64_t groups, const int64_t* offsets) {
  if (groups < 1 || groups > kMaxGroups || !offsets) return S3R_ERR_INVALID_ARG;
  if (d->rows >= ((int64_t)1 << 31)) return S3R_ERR_INVALID_ARG;
  if (d->mode == S3R_S3R_BCAST) return S3R_ERR_UNSUPPORTED;
  return S3R_OK;
}

size_t s3r_grouped_workspace(const s3r_qdesc* d, int64_t groups, int64_t d_in) {
  if (check_desc(d) != S3R_OK || groups < 1 || groups > kMaxGroups || d_in < 0) return 0;
  const int ec = d->ec != S3R_EC_NONE;
  size_t w = grouped_quant_workspace(d->rows, d->cols, groups, ec, d->scale, d->scale == S3R_PER_TOKEN);
  w = std::max(w, grouped_dx_workspace(d->rows, d->cols, d_in, groups, dx_corrected(d->ec)));
  w = std::max(w, grouped_dw_workspace(d->rows, d->cols, d_in, groups, dw_corrected(d->ec)));
  return w;
}

int s3r_grouped_quantize(const s3r_qdesc* d, int64_t groups, const int64_t* offsets, const void* G, int32_t g_dtype,
                         int64_t ld_g, const float* row_scale, const float* col_scale, int8_t* Q, int64_t ld_q,
                         float* delta, int32_t* code_colsum, float* ec_row, float* ec_col, float* ec_mean,
                         uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_desc(d);
  if (rc || (rc = check_groups(d, groups, offsets))) return rc;
  if (g_dtype != S3R_F32 && g_dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  if (d->ec != S3R_EC_NONE && d->mode != S3R_S3R) return S3R_ERR_UNSUPPORTED;
  if (code_colsum && !(d->scale == S3R_PER_TOKEN && d->mode == S3R_RTNE && d->ec == S3R_EC_NONE))
    return S3R_ERR_UNSUPPORTED;
  const int64_t R = d->rows, D = d->cols;
  if (!delta || (R > 0 && D > 0 && (!G || !Q)) || ld_g < D || ld_q < D) return S3R_ERR_INVALID_ARG;
  if (d->ec != S3R_EC_NONE) {
    if (!ec_row || !ec_col || !ec_mean) return S3R_ERR_INVALID_ARG;
  } else if (ec_row || ec_col || ec_mean) {
    return S3R_ERR_INVALID_ARG;
  }
  const size_t need = grouped_quant_workspace(R, D, groups, d->ec != S3R_EC_NONE, d->scale, code_colsum != nullptr);
  if (ws_bytes < need) return S3R_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_arch())) return rc;
  QuantArgs a{};
  a.G = G; a.g_dtype = g_dtype; a.ld_g = ld_g; a.sx = row_scale; a.sw = col_scale;
  a.Q = Q; a.ld_q = ld_q; a.delta = delta; a.code_colsum = code_colsum;
  a.ec_row = ec_row; a.ec_col = ec_col; a.ec_mean = ec_mean; a.flags = flags;
  a.T = R; a.D = D; a.S = 1;
  a.mode = d->mode; a.ec = d->ec; a.scale = d->scale; a.layer = d->layer_id; a.seed = d->seed;
  a.stream = d->stream;
  a.ws = (char*)ws;
  return finish(launch_grouped_quantize(a, groups, offsets, stream));
}

int s3r_grouped_backward_dx(const s3r_qdesc* d, int64_t groups, const int64_t* offsets, const int8_t* Q, int64_t ld_q,
                            const float* delta, const int8_t* Wq, int64_t ld_w, int64_t w_group_stride, int64_t d_in,
                            const float* s_x, const int32_t* r_W, const float* ec_row, const float* ec_col,
                            const float* ec_mean, void* dX, int32_t out_dt, int64_t ld_dx, uint32_t* flags, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  int rc = check_desc(d);
  if (rc || (rc = check_groups(d, groups, offsets))) return rc;
  if (d->scale != S3R_PER_TENSOR) return S3R_ERR_UNSUPPORTED;
  if (out_dt != S3R_F32 && out_dt != S3R_I32_RAW && out_dt != S3R_F32_ACC) return S3R_ERR_UNSUPPORTED;
  const int64_t R = d->rows, D = d->cols;
  if (d_in < 0 || D > kMaxK) return S3R_ERR_INVALID_ARG;
  if (!delta || (R > 0 && d_in > 0 && !dX) || ld_dx < d_in || ld_dx >= kMaxLdOut) return S3R_ERR_INVALID_ARG;
  if (R > 0 && d_in > 0 && ((uintptr_t)dX & 3u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_gemm_operand(Q, ld_q, R, D, R > 0 && D > 0))) return rc;
  if ((rc = check_gemm_operand(Wq, ld_w, D, d_in, D > 0 && d_in > 0))) return rc;
  if (D > 0 && d_in > 0 && (w_group_stride < D * ld_w || (w_group_stride & 15))) return S3R_ERR_INVALID_ARG;
  const bool ec = dx_corrected(d->ec) && out_dt != S3R_I32_RAW;
  if (ec && (!r_W || !ec_row || !ec_col || !ec_mean)) return S3R_ERR_INVALID_ARG;
  const size_t need = grouped_dx_workspace(R, D, d_in, groups, ec);
  if (ws_bytes < need || !ws || ((uintptr_t)ws & 255u)) return S3R_ERR_WORKSPACE;
  if ((rc = check_arch())) return rc;
  DxArgs a{};
  a.Q = Q; a.ld_q = ld_q; a.delta = delta; a.per_token = 0;
  a.W = Wq; a.ld_w = ld_w; a.T = R; a.D = D; a.d_in = d_in; a.S = 1;
  a.sx = s_x; a.rW = r_W; a.ec_row = ec_row; a.ec_col = ec_col; a.ec_mean = ec_mean; a.ec = ec ? d->ec : 0;
  a.out = dX; a.out_dt = out_dt; a.ld_out = ld_dx; a.ws = (char*)ws;
  return finish(launch_grouped_backward_dx(a, groups, offsets, w_group_stride, flags, stream));
}

int s3r_grouped_backward_dw(const s3r_qdesc* d, int64_t groups, const int64_t* offsets, const int8_t* Q, int64_t ld_q,
                            const float* delta, const int8_t* Xq, int64_t ld_x, int64_t d_in, const float* s_w,
                            const int32_t* xs, const float* ec_row, const float* ec_col, const float* ec_mean,
                            void* dW, int32_t out_dt, int64_t ld_dw, int64_t dw_group_stride, uint32_t* flags,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_desc(d);
  if (rc || (rc = check_groups(d, groups, offsets))) return rc;
  if (d->scale != S3R_PER_TENSOR) return S3R_ERR_UNSUPPORTED;
  if (out_dt != S3R_F32 && out_dt != S3R_I32_RAW) return S3R_ERR_UNSUPPORTED;
  const int64_t R = d->rows, D = d->cols;
  if (d_in < 0 || R > kMaxK) return S3R_ERR_INVALID_ARG;
  // the grouped dW drops the stores of columns past d_in by an offset past its output descriptor, which
  // must not wrap 32 bits: (256 + 127) rows of ld_dw floats
  if (!delta || (D > 0 && d_in > 0 && !dW) || ld_dw < d_in || ld_dw >= kMaxLdOut / 2) return S3R_ERR_INVALID_ARG;
  if (D > 0 && d_in > 0 && (((uintptr_t)dW & 3u) || dw_group_stride < D * ld_dw)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_gemm_operand(Q, ld_q, R, D, R > 0 && D > 0))) return rc;
  if ((rc = check_gemm_operand(Xq, ld_x, R, d_in, R > 0 && d_in > 0))) return rc;
  const bool ec = dw_corrected(d->ec) && out_dt == S3R_F32;
  if (ec && (!xs || !ec_row || !ec_col || !ec_mean)) return S3R_ERR_INVALID_ARG;
  const size_t need = grouped_dw_workspace(R, D, d_in, groups, ec);
  if (ws_bytes < need || !ws || ((uintptr_t)ws & 255u)) return S3R_ERR_WORKSPACE;
  if ((rc = check_arch())) return rc;
  DwArgs a{};
  a.Q = Q; a.ld_q = ld_q; a.delta = delta; a.per_token = 0; a.X = Xq; a.ld_x = ld_x;
  a.T = R; a.D = D; a.d_in = d_in; a.S = 1;
  a.sw = s_w; a.xs = xs; a.ec_row = ec_row; a.ec_col = ec_col; a.ec_mean = ec_mean; a.ec = ec ? d->ec : 0;
  a.out = dW; a.out_dt = out_dt; a.ld_out = ld_dw; a.ws = (char*)ws;
  return finish(launch_grouped_backward_dw(a, groups, offsets, dw_group_stride, flags, stream));
}

// ---- MXFP4 variant
static bool mul_of(int64_t x, int64_t m) { return x >= 0 && x % m == 0; }
static int check_mx_desc(const s3r_qdesc* d) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->scale != S3R_PER_TENSOR || d->mode == S3R_S3R_BCAST) return S3R_ERR_UNSUPPORTED;
  if (d->ec != S3R_EC_NONE && d->mode != S3R_S3R) return S3R_ERR_UNSUPPORTED;
  if (!mul_of(d->rows, 128) || !mul_of(d->cols, 128) || !mul_of(d->rows_per_example, 128)) return S3R_ERR_INVALID_ARG;
  if (d->rows == 0 || d->cols == 0 || d->rows >= ((int64_t)1 << 24) || d->cols >= ((int64_t)1 << 24))
    return S3R_ERR_INVALID_ARG;
  return S3R_OK;
}

size_t s3r_mx_operand_workspace(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return mx_operand_workspace(rows, cols);
}

size_t s3r_mx_workspace(const s3r_qdesc* d, int64_t d_in) {
  if (check_mx_desc(d) != S3R_OK || d_in < 0) return 0;
  // at least one 256-byte block: every MX call takes a non-null, aligned ws, also where it uses none
  return std::max({mx_quant_workspace(d->rows, d->cols, d->ec != S3R_EC_NONE),
                   mx_backward_workspace(d->rows, d->cols, d_in, d->rows / d->rows_per_example), (size_t)256});
}

// Codes of an MXFP4 matrix in the 256-row block layout: ld (bytes between 256-row blocks) a multiple
// of 16384 covering the K / 128 blocks of a row block, every block addressable with 32-bit offsets.
static bool mx_codes_ok(const uint8_t* p, int64_t ld, int64_t rows, int64_t K) {
  return p && al16(p) && ld % 16384 == 0 && ld >= 128 * K && ((rows + 255) / 256) * ld < ((int64_t)1 << 32);
}

int s3r_mx_operand(int64_t rows, int64_t cols, int64_t rows_per_example, const void* M, int32_t dtype, int64_t ld,
                   uint8_t* Mt, int64_t ld_t, uint8_t* Mt_scales, int64_t ld_ts, float* colsum, uint32_t* flags,
                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dtype != S3R_F32 && dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || !mul_of(rows, 128) || rows >= ((int64_t)1 << 24) || cols >= ((int64_t)1 << 24))
    return S3R_ERR_INVALID_ARG;
  if (rows_per_example < 128 || rows % rows_per_example || rows_per_example % 128) return S3R_ERR_INVALID_ARG;
  if (!M || !Mt || !Mt_scales || ld < cols || ld_ts < 4 * cols) return S3R_ERR_INVALID_ARG;
  if (!mx_codes_ok(Mt, ld_t, cols, rows)) return S3R_ERR_INVALID_ARG;
  if (ws_bytes < s3r_mx_operand_workspace(rows, cols)) return S3R_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return S3R_ERR_INVALID_ARG;
  int rc;
  if ((rc = check_arch())) return rc;
  MxOperandArgs a{};
  a.M = M; a.dtype = dtype; a.ld = ld; a.R = rows; a.C = cols; a.S = rows_per_example;
  a.Mt = Mt; a.ld_t = ld_t; a.Mts = Mt_scales; a.ld_ts = ld_ts; a.colsum = colsum; a.flags = flags; a.ws = (char*)ws;
  return finish(launch_mx_operand(a, stream));
}

int s3r_mx_quantize(const s3r_qdesc* d, const void* G, int32_t g_dtype, int64_t ld_g, uint8_t* Qh, int64_t ld_qh,
                    uint8_t* Qh_scales, int64_t ld_qhs, uint8_t* Qt, int64_t ld_qt, uint8_t* Qt_scales, int64_t ld_qts,
                    float* ec_row_h, float* ec_col_h, float* ec_mean_h, float* ec_row_t, float* ec_col_t,
                    float* ec_mean_t, uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_mx_desc(d);
  if (rc) return rc;
  if (g_dtype != S3R_F32 && g_dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  const int64_t T = d->rows, D = d->cols;
  if (!G || !Qh || !Qh_scales || !Qt || !Qt_scales || ld_g < D) return S3R_ERR_INVALID_ARG;
  if (!al16(G) || (ld_g * (g_dtype == S3R_BF16 ? 2 : 4)) % 16) return S3R_ERR_INVALID_ARG;   // 16-byte row chunks
  if (!mx_codes_ok(Qh, ld_qh, T, D) || ld_qhs < 4 * T || !mx_codes_ok(Qt, ld_qt, D, T) || ld_qts < 4 * D)
    return S3R_ERR_INVALID_ARG;
  const bool ec = d->ec != S3R_EC_NONE;
  if (ec != (ec_row_h && ec_col_h && ec_mean_h && ec_row_t && ec_col_t && ec_mean_t)) return S3R_ERR_INVALID_ARG;
  if (ws_bytes < mx_quant_workspace(T, D, ec)) return S3R_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_arch())) return rc;
  MxQuantArgs a{};
  a.G = G; a.g_dtype = g_dtype; a.ld_g = ld_g; a.T = T; a.D = D; a.S = d->rows_per_example;
  a.mode = d->mode; a.ec = ec; a.layer = d->layer_id; a.seed = d->seed; a.stream = d->stream;
  a.Qh = Qh; a.ld_qh = ld_qh; a.Qhs = Qh_scales; a.ld_qhs = ld_qhs;
  a.Qt = Qt; a.ld_qt = ld_qt; a.Qts = Qt_scales; a.ld_qts = ld_qts;
  a.ec_row_h = ec_row_h; a.ec_col_h = ec_col_h; a.ec_mean_h = ec_mean_h;
  a.ec_row_t = ec_row_t; a.ec_col_t = ec_col_t; a.ec_mean_t = ec_mean_t;
  a.flags = flags; a.ws = (char*)ws;
  return finish(launch_mx_quantize(a, stream));
}

static int check_mx_operand(const uint8_t* p, int64_t ld, const uint8_t* s, int64_t lds, int64_t rows, int64_t K) {
  if (!mx_codes_ok(p, ld, rows, K) || !s || ((uintptr_t)s & 3u) || (lds & 3) || lds < 4 * rows)
    return S3R_ERR_INVALID_ARG;
  if ((K / 128 + 1) * lds >= ((int64_t)1 << 32)) return S3R_ERR_INVALID_ARG;
  return S3R_OK;
}

int s3r_mx_backward_dx(const s3r_qdesc* d, const uint8_t* Qh, int64_t ld_qh, const uint8_t* Qh_scales, int64_t ld_qhs,
                       const uint8_t* Wt, int64_t ld_wt, const uint8_t* Wt_scales, int64_t ld_wts, int64_t d_in,
                       const float* r_W, const float* ec_row_h, const float* ec_col_h, const float* ec_mean_h,
                       float* dX, int64_t ld_dx, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_mx_desc(d);
  if (rc) return rc;
  const int64_t T = d->rows, D = d->cols, B = T / d->rows_per_example;
  if (d_in < 1 || !dX || ld_dx < d_in || ld_dx >= ((int64_t)1 << 22) || ((uintptr_t)dX & 3u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_mx_operand(Qh, ld_qh, Qh_scales, ld_qhs, T, D))) return rc;
  if ((rc = check_mx_operand(Wt, ld_wt, Wt_scales, ld_wts, d_in, D))) return rc;
  const bool ec = d->ec == S3R_EC_DX_ONLY || d->ec == S3R_EC_TWO_WAY;
  if (ec && (!r_W || !ec_row_h || !ec_col_h || !ec_mean_h)) return S3R_ERR_INVALID_ARG;
  if (ws_bytes < mx_backward_workspace(T, D, d_in, B)) return S3R_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_arch())) return rc;
  MxBwArgs a{};
  a.A = Qh; a.lda = ld_qh; a.As = Qh_scales; a.ldas = ld_qhs; a.B = Wt; a.ldb = ld_wt; a.Bs = Wt_scales; a.ldbs = ld_wts;
  a.T = T; a.D = D; a.d_in = d_in; a.S = d->rows_per_example; a.K = D; a.ec = ec;
  a.vcol = r_W; a.ec_row = ec_row_h; a.ec_col = ec_col_h; a.ec_mean = ec_mean_h;
  a.out = dX; a.ld_out = ld_dx; a.ws = (char*)ws;
  return finish(launch_mx_backward_dx(a, stream));
}

int s3r_mx_backward_dw(const s3r_qdesc* d, const uint8_t* Qt, int64_t ld_qt, const uint8_t* Qt_scales, int64_t ld_qts,
                       const uint8_t* Xt, int64_t ld_xt, const uint8_t* Xt_scales, int64_t ld_xts, int64_t d_in,
                       const float* xs, const float* ec_row_t, const float* ec_col_t, const float* ec_mean_t,
                       float* dW, int64_t ld_dw, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_mx_desc(d);
  if (rc) return rc;
  const int64_t T = d->rows, D = d->cols, B = T / d->rows_per_example;
  if (d_in < 1 || !dW || ld_dw < d_in || ld_dw >= ((int64_t)1 << 22) || ((uintptr_t)dW & 3u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_mx_operand(Qt, ld_qt, Qt_scales, ld_qts, D, T))) return rc;
  if ((rc = check_mx_operand(Xt, ld_xt, Xt_scales, ld_xts, d_in, T))) return rc;
  const bool ec = d->ec == S3R_EC_TWO_WAY || d->ec == S3R_EC_DW_ONLY;
  if (ec && (!xs || !ec_row_t || !ec_col_t || !ec_mean_t)) return S3R_ERR_INVALID_ARG;
  if (ws_bytes < mx_backward_workspace(T, D, d_in, B)) return S3R_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return S3R_ERR_INVALID_ARG;
  if ((rc = check_arch())) return rc;
  MxBwArgs a{};
  a.A = Qt; a.lda = ld_qt; a.As = Qt_scales; a.ldas = ld_qts; a.B = Xt; a.ldb = ld_xt; a.Bs = Xt_scales; a.ldbs = ld_xts;
  a.T = T; a.D = D; a.d_in = d_in; a.S = d->rows_per_example; a.K = T; a.ec = ec;
  a.vcol = xs; a.ec_row = ec_row_t; a.ec_col = ec_col_t; a.ec_mean = ec_mean_t;
  a.out = dW; a.ld_out = ld_dw; a.ws = (char*)ws;
  return finish(launch_mx_backward_dw(a, stream));
}

int s3r_time_next_gemm(hipEvent_t start, hipEvent_t stop) {
  GemmTiming& t = gemm_timing();
  t.start = start;
  t.stop = stop;
  return S3R_OK;
}

const char* s3r_status_string(int s) {
  switch (s) {
    case S3R_OK: return "ok";
    case S3R_ERR_INVALID_ARG: return "invalid argument";
    case S3R_ERR_UNSUPPORTED: return "unsupported combination";
    case S3R_ERR_WORKSPACE: return "workspace too small";
    case S3R_ERR_ARCH: return "device is not gfx950";
    case S3R_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int s3r_version(void) { return 200; }

}  // extern "C"
