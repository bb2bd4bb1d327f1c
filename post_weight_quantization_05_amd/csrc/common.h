// Shared device/host definitions of libgptq_mi355x (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gptq_mi355x.h"

namespace gptq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) double f64x4;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Device status word bits (written with atomicOr, read once by the host at the end of prepare and of quantize).
enum : unsigned {
  DEV_STATUS_NOT_SPD = 1u,
  DEV_STATUS_NONFINITE = 2u,
};

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// ---- kernel launchers (defined in the .hip files) --------------------------------------------------

// Hessian (hessian.hip)
struct HessianPlan {
  int64_t n_rows, in, ld;
  int dtype;
  int tile;        // square output tile (256)
  int n_tb;        // tile blocks per side = ceil(in / tile)
  int n_tiles;     // lower-triangle tiles = n_tb (n_tb + 1) / 2
  int splits;      // row slices (split-K) of one launch
  int64_t rows_per_split;
  int64_t chunk_rows;  // rows per launch (splits * rows_per_split at most); longer inputs take several
  size_t part_bytes, colsq_part_bytes, total_bytes;
};
// max_bytes != 0: use no more row slices than keep total_bytes within max_bytes (one slice at least;
// the caller checks total_bytes)
HessianPlan hessian_plan(int64_t n_rows, int64_t in, int dtype, size_t max_bytes = 0);
// first: S's lower triangle and colsq are written (not added to): the first chunk of a stream
hipError_t hessian_launch(const HessianPlan& p, const void* X, double* S, double* colsq, void* ws,
                          hipStream_t stream, bool first);

// Prepare + factorization (factor.hip)
size_t prepare_ws_bytes(int64_t in);
hipError_t prepare_launch(const double* S, const double* colsq, int64_t n_total, int64_t in, double damp,
                          int act_order, unsigned flags, double* U, int32_t* perm, uint8_t* dead, void* ws,
                          hipStream_t stream, unsigned* host_status);

// Quantize (quant.hip)
size_t quantize_ws_bytes(int64_t out, int64_t in, bool rform);
hipError_t quantize_launch(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ld_w, const double* U,
                           const int32_t* perm, const uint8_t* dead, int bits, int group, int grid, int8_t* codes,
                           float* scales, int32_t* zeros, int32_t* g_idx, double* row_loss, void* ws,
                           hipStream_t stream, unsigned* host_status, bool rform = false);

// Packed codes and the dequantizing matmul (pack.hip)
int64_t packed_words_per_row(int64_t in, int bits);
hipError_t pack_launch(const int8_t* codes, int64_t out, int64_t in, int bits, int grid, uint32_t* packed,
                       hipStream_t stream);
hipError_t dequant_matmul_launch(const void* X, int x_dtype, int64_t n, int64_t in, int64_t ld_x,
                                 const uint32_t* packed, const float* scales, const int32_t* zeros,
                                 const int32_t* g_idx, int64_t out, int bits, int grid, int n_groups,
                                 const float* bias, int relu, float* Y, int64_t ld_y, hipStream_t stream);

}  // namespace gptq
