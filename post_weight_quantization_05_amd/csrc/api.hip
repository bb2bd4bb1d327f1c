// C ABI of libgptq_mi355x: argument validation, workspace sizing and launch sequencing. Every check runs
// on the host before anything is launched, so an argument error writes nothing.
#include <cmath>
#include <cstring>

#include "common.h"

using namespace gptq;

namespace {

bool valid_dtype(int t) { return t == GPTQ_F32 || t == GPTQ_BF16; }

int hip_status(hipError_t e) { return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP; }

// Sizes are bounded so that every index the kernels form fits their int arithmetic.
constexpr int64_t MAX_IN = 65536;
constexpr int64_t MAX_OUT = 1 << 20;

}  // namespace

extern "C" {

const char* gptq_status_string(int status) {
  switch (status) {
    case GPTQ_OK: return "GPTQ_OK";
    case GPTQ_ERR_INVALID_ARG: return "GPTQ_ERR_INVALID_ARG";
    case GPTQ_ERR_UNSUPPORTED: return "GPTQ_ERR_UNSUPPORTED";
    case GPTQ_ERR_NOT_SPD: return "GPTQ_ERR_NOT_SPD";
    case GPTQ_ERR_NONFINITE: return "GPTQ_ERR_NONFINITE";
    case GPTQ_ERR_WORKSPACE: return "GPTQ_ERR_WORKSPACE";
    case GPTQ_ERR_HIP: return "GPTQ_ERR_HIP";
    default: return "GPTQ_ERR_UNKNOWN";
  }
}

const char* gptq_version(void) { return "gptq_mi355x 0.1 (gfx950)"; }

size_t gptq_hessian_workspace_bytes(int64_t n_rows, int64_t in, int x_dtype) {
  if (n_rows < 1 || in < 1 || in > MAX_IN || !valid_dtype(x_dtype)) return 0;
  return hessian_plan(n_rows, in, x_dtype).total_bytes;
}

int gptq_hessian_accumulate(const void* X, int x_dtype, int64_t n_rows, int64_t in, int64_t ld_x, double* S,
                            double* colsq, int64_t* n_total, void* ws, size_t ws_bytes, void* stream) {
  if (!X || !S || !colsq || !n_total) return GPTQ_ERR_INVALID_ARG;
  if (n_rows < 1 || in < 1 || in > MAX_IN || ld_x < in || !valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (*n_total < 0) return GPTQ_ERR_INVALID_ARG;
  HessianPlan p = hessian_plan(n_rows, in, x_dtype);
  p.ld = ld_x;
  if (!ws || ws_bytes < p.total_bytes) return GPTQ_ERR_WORKSPACE;
  const int st =
      hip_status(hessian_launch(p, X, S, colsq, ws, reinterpret_cast<hipStream_t>(stream), *n_total == 0));
  if (st == GPTQ_OK) *n_total += n_rows;
  return st;
}

size_t gptq_prepare_workspace_bytes(int64_t in) {
  if (in < 1 || in > MAX_IN) return 0;
  return prepare_ws_bytes(in);
}

int gptq_prepare_chol(const double* S, const double* colsq, int64_t n_total, int64_t in, double damp, int act_order,
                      unsigned flags, double* U, int32_t* perm, uint8_t* dead, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!S || !colsq || !U || !perm || !dead) return GPTQ_ERR_INVALID_ARG;
  if (in < 1 || in > MAX_IN || n_total < 1) return GPTQ_ERR_INVALID_ARG;
  if (!(damp >= 0.0) || !std::isfinite(damp)) return GPTQ_ERR_INVALID_ARG;
  if (flags != GPTQ_FACTOR_REVERSED && flags != GPTQ_FACTOR_INVERSE_RECHOL && flags != GPTQ_FACTOR_R_FORM)
    return GPTQ_ERR_INVALID_ARG;
  if (flags == GPTQ_FACTOR_R_FORM && in % 64 != 0) return GPTQ_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < prepare_ws_bytes(in)) return GPTQ_ERR_WORKSPACE;
  unsigned dev_status = 0;
  hipError_t e = prepare_launch(S, colsq, n_total, in, damp, act_order ? 1 : 0, flags, U, perm, dead, ws,
                                reinterpret_cast<hipStream_t>(stream), &dev_status);
  if (e != hipSuccess) return GPTQ_ERR_HIP;
  if (dev_status & DEV_STATUS_NONFINITE) return GPTQ_ERR_NONFINITE;
  if (dev_status & DEV_STATUS_NOT_SPD) return GPTQ_ERR_NOT_SPD;
  return GPTQ_OK;
}

size_t gptq_quantize_workspace_bytes(int64_t out, int64_t in) {
  if (out < 1 || in < 1 || in > MAX_IN || out > MAX_OUT) return 0;
  return quantize_ws_bytes(out, in, false);
}

size_t gptq_quantize_r_workspace_bytes(int64_t out, int64_t in) {
  if (out < 1 || in < 1 || in > MAX_IN || out > MAX_OUT) return 0;
  return quantize_ws_bytes(out, in, true);
}

int gptq_quantize_layer_ex(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ld_w, const double* U,
                           const int32_t* perm, const uint8_t* dead, int bits, int group, int grid, int8_t* codes,
                           float* scales, int32_t* zeros, int32_t* g_idx, double* row_loss, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!W || !U || !perm || !dead || !codes || !scales) return GPTQ_ERR_INVALID_ARG;
  if (grid != GPTQ_GRID_SYMMETRIC && grid != GPTQ_GRID_ASYMMETRIC) return GPTQ_ERR_INVALID_ARG;
  if (grid == GPTQ_GRID_ASYMMETRIC && !zeros) return GPTQ_ERR_INVALID_ARG;
  if (out < 1 || in < 1 || in > MAX_IN || out > MAX_OUT || ld_w < in || !valid_dtype(w_dtype))
    return GPTQ_ERR_INVALID_ARG;
  if (bits < 2 || bits > 8 || group < 0) return GPTQ_ERR_INVALID_ARG;
  if (group != 0 && !(128 % group == 0 || group % 128 == 0)) return GPTQ_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < quantize_ws_bytes(out, in, false)) return GPTQ_ERR_WORKSPACE;
  unsigned dev_status = 0;
  const hipError_t e = quantize_launch(W, w_dtype, out, in, ld_w, U, perm, dead, bits, group, grid, codes, scales,
                                       zeros, g_idx, row_loss, ws, reinterpret_cast<hipStream_t>(stream), &dev_status);
  if (e != hipSuccess) return GPTQ_ERR_HIP;
  return (dev_status & DEV_STATUS_NONFINITE) ? GPTQ_ERR_NONFINITE : GPTQ_OK;
}

int gptq_quantize_layer_r(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ld_w, const double* R,
                          const int32_t* perm, const uint8_t* dead, int bits, int group, int grid, int8_t* codes,
                          float* scales, int32_t* zeros, int32_t* g_idx, double* row_loss, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!W || !R || !perm || !dead || !codes || !scales) return GPTQ_ERR_INVALID_ARG;
  if (grid != GPTQ_GRID_SYMMETRIC && grid != GPTQ_GRID_ASYMMETRIC) return GPTQ_ERR_INVALID_ARG;
  if (grid == GPTQ_GRID_ASYMMETRIC && !zeros) return GPTQ_ERR_INVALID_ARG;
  if (out < 1 || in < 1 || in > MAX_IN || out > MAX_OUT || ld_w < in || !valid_dtype(w_dtype))
    return GPTQ_ERR_INVALID_ARG;
  if (bits < 2 || bits > 8 || group < 0) return GPTQ_ERR_INVALID_ARG;
  if (in % 64 != 0 || (group != 0 && 128 % group != 0)) return GPTQ_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < quantize_ws_bytes(out, in, true)) return GPTQ_ERR_WORKSPACE;
  unsigned dev_status = 0;
  const hipError_t e = quantize_launch(W, w_dtype, out, in, ld_w, R, perm, dead, bits, group, grid, codes, scales,
                                       zeros, g_idx, row_loss, ws, reinterpret_cast<hipStream_t>(stream), &dev_status,
                                       true);
  if (e != hipSuccess) return GPTQ_ERR_HIP;
  return (dev_status & DEV_STATUS_NONFINITE) ? GPTQ_ERR_NONFINITE : GPTQ_OK;
}

int gptq_quantize_layer(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ld_w, const double* U,
                        const int32_t* perm, const uint8_t* dead, int bits, int group, int8_t* codes, float* scales,
                        int32_t* g_idx, double* row_loss, void* ws, size_t ws_bytes, void* stream) {
  return gptq_quantize_layer_ex(W, w_dtype, out, in, ld_w, U, perm, dead, bits, group, GPTQ_GRID_SYMMETRIC, codes,
                                scales, nullptr, g_idx, row_loss, ws, ws_bytes, stream);
}

int64_t gptq_packed_words_per_row(int64_t in, int bits) {
  if (in < 1 || bits < 2 || bits > 8) return 0;
  return packed_words_per_row(in, bits);
}

int gptq_pack_codes(const int8_t* codes, int64_t out, int64_t in, int bits, int grid, uint32_t* packed,
                    void* stream) {
  if (!codes || !packed) return GPTQ_ERR_INVALID_ARG;
  if (out < 1 || in < 1 || in > MAX_IN || out > MAX_OUT || bits < 2 || bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (grid != GPTQ_GRID_SYMMETRIC && grid != GPTQ_GRID_ASYMMETRIC) return GPTQ_ERR_INVALID_ARG;
  return hip_status(pack_launch(codes, out, in, bits, grid, packed, reinterpret_cast<hipStream_t>(stream)));
}

int gptq_dequant_matmul(const void* X, int x_dtype, int64_t n, int64_t in, int64_t ld_x, const uint32_t* packed,
                        const float* scales, const int32_t* zeros, const int32_t* g_idx, int64_t out, int bits,
                        int grid, int group, const float* bias, int relu, float* Y, int64_t ld_y, void* stream) {
  if (!X || !packed || !scales || !g_idx || !Y) return GPTQ_ERR_INVALID_ARG;
  if (grid != GPTQ_GRID_SYMMETRIC && grid != GPTQ_GRID_ASYMMETRIC) return GPTQ_ERR_INVALID_ARG;
  if (grid == GPTQ_GRID_ASYMMETRIC && !zeros) return GPTQ_ERR_INVALID_ARG;
  if (n < 1 || in < 1 || out < 1 || in > MAX_IN || out > MAX_OUT || n > ((int64_t)1 << 31) - 1)
    return GPTQ_ERR_INVALID_ARG;
  if (ld_x < in || ld_y < out || !valid_dtype(x_dtype) || bits < 2 || bits > 8 || group < 0 || (relu != 0 && relu != 1))
    return GPTQ_ERR_INVALID_ARG;
  // one workgroup of 256 work-items per 64 x 64 tile of Y, in a 1-D grid of at most 2^32 - 1 work-items
  if (((n + 63) / 64) * ((out + 63) / 64) > (int64_t)(UINT32_MAX / 256)) return GPTQ_ERR_INVALID_ARG;
  const int n_groups = group ? (int)((in + group - 1) / group) : 1;
  return hip_status(dequant_matmul_launch(X, x_dtype, n, in, ld_x, packed, scales, zeros, g_idx, out, bits, grid,
                                          n_groups, bias, relu, Y, ld_y, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
