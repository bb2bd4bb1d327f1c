// Packed codes and their consumer on gfx950.
//
// GPTQ guide ("GPTQ", herodthegreater.github.io/pigeon/guide/gptq/), "When it breaks": a quantized layer
// is stored as integer codes plus per-group scales, and with act_order the groups follow the
// quantization order, so a consumer needs g_idx to find a column's group. Handbook page "GPTQ >
// Implementation with AutoGPTQ": int4 storage packs the codes at 4 bits each.
//
//  k_pack            codes (int8, out x in) -> one little-endian bit stream per row, code j at bits
//                    [b j, b (j + 1)). Symmetric codes are stored offset by 2^(b-1); asymmetric codes
//                    (0..2^b - 1, read as uint8) as they are. One thread per 32-bit word.
//  k_dequant_matmul  Y = X Q^T with Q dequantized while it is staged: Q[r][c] = scale[r][g] * (code -
//                    zero[r][g]), g = g_idx[c] (zero = 0 on the symmetric grid), then optionally + bias
//                    and ReLU: the forward of one quantized layer of an MLP, which the guide's layer-wise
//                    driver feeds to the next layer ("How it works", apply_layerwise). 64 x 64 tiles of
//                    Y, 4 waves of 32 x 32 on v_mfma_f32_16x16x4f32; X (bf16 widened exactly, or fp32)
//                    and the dequantized weights go through LDS as [k][i] in chunks of 16 inputs.
#include <algorithm>

#include "common.h"

namespace gptq {

namespace {

// word idx = r * wpr + w of the packed output: the (at most 32 / bits + 1) codes that touch it
__device__ __forceinline__ void pack_word(const int8_t* __restrict__ codes, int in, int bits, int offset, int wpr,
                                          int64_t idx, uint32_t* __restrict__ packed) {
  const int64_t r = idx / wpr;
  const int w = (int)(idx - r * wpr);
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t bit0 = (int64_t)w * 32;
  const int j0 = (int)(bit0 / bits);
  const int j1 = (int)min<int64_t>(in - 1, (bit0 + 31) / bits);
  const int8_t* crow = codes + r * in;
  uint32_t word = 0u;
  for (int j = j0; j <= j1; ++j) {
    const uint32_t v = ((uint32_t)(uint8_t)crow[j] + (uint32_t)offset) & mask;
    const int64_t pos = (int64_t)j * bits - bit0;  // bit position of the code inside this word
    word |= (pos >= 0) ? (v << pos) : (v >> (-pos));
  }
  packed[idx] = word;
}

// one thread per output word, in a grid-stride loop over the out * wpr words (up to 2^34 of them)
__global__ __launch_bounds__(256) void k_pack(const int8_t* __restrict__ codes, int out, int in, int bits,
                                              int offset, int wpr, uint32_t* __restrict__ packed) {
  const int64_t total = (int64_t)out * wpr;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256)
    pack_word(codes, in, bits, offset, wpr, idx, packed);
}

// code (r, c) from the packed stream: the word holding its first bit and, when it straddles, the next one
__device__ __forceinline__ uint32_t unpack_code(const uint32_t* __restrict__ prow, int c, int bits, int wpr) {
  const int64_t bit = (int64_t)c * bits;
  const int w = (int)(bit >> 5), sh = (int)(bit & 31);
  uint32_t v = prow[w] >> sh;
  if (sh + bits > 32 && w + 1 < wpr) v |= prow[w + 1] << (32 - sh);
  return v & ((1u << bits) - 1u);
}

constexpr int DT = 64;   // Y tile edge
constexpr int DK = 16;   // inputs per chunk
constexpr int DPAD = 4;

template <bool XBF16>
__global__ __launch_bounds__(256) void k_dequant_matmul(const void* __restrict__ Xv, int64_t ld_x, int n, int in,
                                                        const uint32_t* __restrict__ packed, int wpr,
                                                        const float* __restrict__ scales,
                                                        const int32_t* __restrict__ zeros,
                                                        const int32_t* __restrict__ g_idx, int n_groups, int out,
                                                        int bits, int offset, const float* __restrict__ bias,
                                                        int relu, float* __restrict__ Y, int64_t ld_y) {
  __shared__ float As[DK][DT + DPAD];  // As[k][i] = X[i0 + i][k0 + k]
  __shared__ float Bs[DK][DT + DPAD];  // Bs[k][j] = Q[j0 + j][k0 + k]
  const int ntn = (out + DT - 1) / DT;
  const int i0 = (blockIdx.x / ntn) * DT, j0 = (blockIdx.x % ntn) * DT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // staging: 64 rows x 16 inputs per operand = 4 elements per thread: row tid / 4, inputs (tid % 4) * 4 + q
  const int sr = tid >> 2, sk = (tid & 3) * 4;
  for (int k0 = 0; k0 < in; k0 += DK) {
    {
      const int gi = i0 + sr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gk = k0 + sk + q;
        float v = 0.f;
        if (gi < n && gk < in) {
          if (XBF16) {
            const uint16_t h = reinterpret_cast<const uint16_t*>(Xv)[(int64_t)gi * ld_x + gk];
            v = __uint_as_float(((uint32_t)h) << 16);
          } else {
            v = reinterpret_cast<const float*>(Xv)[(int64_t)gi * ld_x + gk];
          }
        }
        As[sk + q][sr] = v;
      }
      const int gj = j0 + sr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gk = k0 + sk + q;
        float v = 0.f;
        if (gj < out && gk < in) {
          const int g = min(max(g_idx[gk], 0), n_groups - 1);
          const int code = (int)unpack_code(packed + (int64_t)gj * wpr, gk, bits, wpr) - offset;
          const float zr = zeros ? (float)zeros[(int64_t)gj * n_groups + g] : 0.f;
          v = scales[(int64_t)gj * n_groups + g] * ((float)code - zr);
        }
        Bs[sk + q][sr] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k4 = 0; k4 < DK; k4 += 4) {
      const int kr = k4 + (lane >> 4);
      float fa[2], fb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) fa[a] = As[kr][wm * 32 + a * 16 + (lane & 15)];
#pragma unroll
      for (int b = 0; b < 2; ++b) fb[b] = Bs[kr][wn * 32 + b * 16 + (lane & 15)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
  // D layout of 16x16x4 f32: register r of lane l holds row 4 (l / 16) + r, column l % 16
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = i0 + wm * 32 + a * 16 + 4 * (lane >> 4) + r;
        const int gj = j0 + wn * 32 + b * 16 + (lane & 15);
        if (gi < n && gj < out) {
          float y = acc[a][b][r];
          if (bias) y += bias[gj];
          if (relu) y = fmaxf(y, 0.f);
          Y[(int64_t)gi * ld_y + gj] = y;
        }
      }
}

}  // namespace

int64_t packed_words_per_row(int64_t in, int bits) { return (in * bits + 31) / 32; }

hipError_t pack_launch(const int8_t* codes, int64_t out, int64_t in, int bits, int grid, uint32_t* packed,
                       hipStream_t stream) {
  const int wpr = (int)packed_words_per_row(in, bits);
  const int offset = (grid == GPTQ_GRID_ASYMMETRIC) ? 0 : (1 << (bits - 1));
  const int64_t total = out * (int64_t)wpr;
  const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(total, 256), 1 << 20);
  hipLaunchKernelGGL(k_pack, dim3(blocks), dim3(256), 0, stream, codes, (int)out, (int)in, bits, offset, wpr,
                     packed);
  return hipGetLastError();
}

hipError_t dequant_matmul_launch(const void* X, int x_dtype, int64_t n, int64_t in, int64_t ld_x,
                                 const uint32_t* packed, const float* scales, const int32_t* zeros,
                                 const int32_t* g_idx, int64_t out, int bits, int grid, int n_groups,
                                 const float* bias, int relu, float* Y, int64_t ld_y, hipStream_t stream) {
  const int wpr = (int)packed_words_per_row(in, bits);
  const int offset = (grid == GPTQ_GRID_ASYMMETRIC) ? 0 : (1 << (bits - 1));
  const int64_t tiles = ceil_div(n, DT) * ceil_div(out, DT);
  const int32_t* z = (grid == GPTQ_GRID_ASYMMETRIC) ? zeros : nullptr;
  if (x_dtype == GPTQ_BF16)
    hipLaunchKernelGGL(k_dequant_matmul<true>, dim3((unsigned)tiles), dim3(256), 0, stream, X, ld_x, (int)n, (int)in,
                       packed, wpr, scales, z, g_idx, n_groups, (int)out, bits, offset, bias, relu, Y, ld_y);
  else
    hipLaunchKernelGGL(k_dequant_matmul<false>, dim3((unsigned)tiles), dim3(256), 0, stream, X, ld_x, (int)n,
                       (int)in, packed, wpr, scales, z, g_idx, n_groups, (int)out, bits, offset, bias, relu, Y,
                       ld_y);
  return hipGetLastError();
}

}  // namespace gptq
