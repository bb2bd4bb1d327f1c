// Hessian accumulation S += X^T X (lower triangle) and colsq += sum x^2, on gfx950 matrix cores.
//
// GPTQ guide ("GPTQ", herodthegreater.github.io/pigeon/guide/gptq/), "The idea": H = 2 X^T X / n over
// the calibration inputs; the 2/n scaling is applied in the prepare step, this file only sums.
//
// Design (bf16 X, the transformer workloads):
//  * Output tiles of 256 x 256 over the lower triangle only (i-block >= j-block); the n calibration rows
//    are cut into `splits` row slices so that tiles x splits fills the chip (split-K).
//  * X is row-major (rows = tokens). The MFMA operands (v_mfma_f32_32x32x16_bf16; bf16 x bf16 products are
//    exact in fp32) need 8 consecutive k per lane: they are read from LDS with ds_read_b64_tr_b16, which
//    transposes a 4 x 16 block of 16-bit elements across 16 lanes.
//  * Rows 16-byte aligned (k_xtx_bf16_dma): 8 waves of 128 x 64 per tile; 32-row stages of both operand
//    blocks go HBM -> LDS with buffer_load_dwordx4 ... lds, four stages ahead, no staging registers.
//    Otherwise (k_xtx_bf16): 4 waves of 128 x 128, register-staged double-buffered loads.
//  * Diagonal tiles read one column block (A = B); the waves whose block lies above the diagonal form the
//    fp64 column sums of squares instead (x^2 of a bf16/fp32 value is exact in fp64).
//  * Each (slice, tile) writes an fp32 partial; a second kernel (k_xtx_reduce) adds the slices in a fixed
//    order in fp64 to S, so the result is bitwise reproducible.
//  * Workgroup index -> (slice, tile) is remapped so that the workgroups resident on one XCD (dispatch is
//    round-robin over the 8 XCDs) work on a narrow set of column blocks of the same row slice and share
//    those rows in that XCD's L2.
// fp32 X (small layers) uses the same structure with v_mfma_f32_16x16x4f32 on 128 x 128 tiles; fp32
// operands need no transpose (one k per lane).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace gptq {

namespace {

constexpr int BT = 256;       // bf16 tile edge
constexpr int BK = 32;        // rows per stage
constexpr int BROW = BT + 32; // LDS row stride in bf16 elements (576 B; the pad spreads rows over banks)

constexpr int FT = 128;       // fp32 tile edge
constexpr int FK = 16;        // rows per stage
constexpr int FROW = FT + 4;  // LDS row stride in floats

__device__ __forceinline__ void tile_coords(int t, int& I, int& J) {
  // t = I (I + 1) / 2 + J with 0 <= J <= I
  int I0 = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((I0 + 1) * (I0 + 2) / 2 <= t) ++I0;
  while (I0 * (I0 + 1) / 2 > t) --I0;
  I = I0;
  J = t - I0 * (I0 + 1) / 2;
}

// Position p of the lower tiles listed in super-tile order: blocks are grouped 4 at a time, super-tiles
// (A >= B) are visited in order and the tiles inside each one row by row. Consecutive positions then
// share few column blocks, so a contiguous run of positions (one XCD's share) reads a narrow set of
// X's columns.
__device__ __forceinline__ void supertile_coords(int p, int n_tb, int& I, int& J) {
  constexpr int SB = 4;
  const int ns = (n_tb + SB - 1) / SB;
  for (int A = 0; A < ns; ++A) {
    const int i0 = A * SB, i1 = min(n_tb, i0 + SB);
    for (int B = 0; B <= A; ++B) {
      const int j0 = B * SB, j1 = min(n_tb, j0 + SB);
      int cnt;
      if (A != B) cnt = (i1 - i0) * (j1 - j0);
      else cnt = (i1 - i0) * (i1 - i0 + 1) / 2;
      if (p < cnt) {
        if (A != B) {
          I = i0 + p / (j1 - j0);
          J = j0 + p % (j1 - j0);
        } else {
          int r = 0;
          while ((r + 1) * (r + 2) / 2 <= p) ++r;
          I = i0 + r;
          J = i0 + (p - r * (r + 1) / 2);
        }
        return;
      }
      p -= cnt;
    }
  }
  I = J = 0;  // not reached for p < n_tiles
}

// Load 8 consecutive bf16 of one row (cols c..c+7), zero outside [0, d) or beyond the valid rows.
template <bool VEC>
__device__ __forceinline__ uint4 load8_bf16(const uint16_t* __restrict__ X, int64_t ld, int64_t row, bool row_ok,
                                            int c, int d) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (!row_ok) return v;
  const uint16_t* p = X + row * ld + c;
  if (VEC && c + 8 <= d) {
    v = *reinterpret_cast<const uint4*>(p);
  } else {
    uint16_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = (c + q < d) ? p[q] : (uint16_t)0;
    v.x = e[0] | ((uint32_t)e[1] << 16);
    v.y = e[2] | ((uint32_t)e[3] << 16);
    v.z = e[4] | ((uint32_t)e[5] << 16);
    v.w = e[6] | ((uint32_t)e[7] << 16);
  }
  return v;
}

__device__ __forceinline__ void sq_accum8(double* acc, uint4 v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    double lo = (double)__uint_as_float(w[q] << 16);
    double hi = (double)__uint_as_float(w[q] & 0xFFFF0000u);
    acc[2 * q] = fma(lo, lo, acc[2 * q]);
    acc[2 * q + 1] = fma(hi, hi, acc[2 * q + 1]);
  }
}

// Split-K combine, a kernel of its own after the accumulation: workgroup (tile, 16-row chunk) sums the
// slices' fp32 partials of its rows in slice order in fp64 and adds them to S's lower triangle; the first
// chunk of a diagonal tile also combines that tile's column sums into colsq. The order of every sum is
// fixed, so results are bitwise reproducible. Each thread keeps FIN_G x FIN_SB 16-byte loads in flight
// (its 4-column groups, eight slices at a time), and the n_tiles x TILE/16 workgroups spread the
// combine over every CU.
constexpr int FIN_RC = 16;  // rows per workgroup
constexpr int FIN_SB = 8;   // slices in flight

template <int TILE>
__global__ __launch_bounds__(256) void k_xtx_reduce(const float* __restrict__ part,
                                                    const double* __restrict__ colsq_part, int colsq_stride,
                                                    int n_tiles, int splits, int d, double* __restrict__ S,
                                                    double* __restrict__ colsq, int first) {
  constexpr int Q = TILE / 4;                 // 4-column groups per tile row
  constexpr int NCH = TILE / FIN_RC;          // row chunks per tile
  constexpr int FIN_G = FIN_RC * Q / 256;     // groups per thread
  static_assert(FIN_G * 256 == FIN_RC * Q, "groups per thread");
  const int t = blockIdx.x / NCH, rc = blockIdx.x - (blockIdx.x / NCH) * NCH;
  int I, J;
  tile_coords(t, I, J);
  const int tid = threadIdx.x;
  const int64_t tsz = (int64_t)TILE * TILE;
  const int64_t sstride4 = (int64_t)n_tiles * tsz / 4;  // one slice's partials, in float4
  const float4* p0 = reinterpret_cast<const float4*>(part + (int64_t)t * tsz);
  int e4[FIN_G], gi[FIN_G], gj[FIN_G];
  bool live[FIN_G];
  double acc[FIN_G][4];
#pragma unroll
  for (int k = 0; k < FIN_G; ++k) {
    const int e = tid + 256 * k;               // group within the chunk
    const int r = rc * FIN_RC + e / Q, c4 = (e % Q) * 4;
    e4[k] = r * Q + e % Q;                     // float4 index within the tile
    gi[k] = I * TILE + r;
    gj[k] = J * TILE + c4;
    live[k] = gi[k] < d && gj[k] <= gi[k] && gj[k] < d;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[k][c] = 0.0;
  }
  for (int s0 = 0; s0 < splits; s0 += FIN_SB) {
    // unconditional loads from clamped (valid) addresses, then a select: no branch between the loads
    float4 v[FIN_G][FIN_SB];
#pragma unroll
    for (int k = 0; k < FIN_G; ++k)
#pragma unroll
      for (int u = 0; u < FIN_SB; ++u) {
        const int sl = min(s0 + u, splits - 1);
        const float4 x = p0[e4[k] + (int64_t)sl * sstride4];
        const bool use = live[k] && s0 + u < splits;
        v[k][u] = make_float4(use ? x.x : 0.f, use ? x.y : 0.f, use ? x.z : 0.f, use ? x.w : 0.f);
      }
    // slice order; a slice past the end adds an exact zero
#pragma unroll
    for (int k = 0; k < FIN_G; ++k)
#pragma unroll
      for (int u = 0; u < FIN_SB; ++u) {
        acc[k][0] += (double)v[k][u].x;
        acc[k][1] += (double)v[k][u].y;
        acc[k][2] += (double)v[k][u].z;
        acc[k][3] += (double)v[k][u].w;
      }
  }
  // read the S entries first (clamped to valid addresses), then store only the lower-triangle ones
  double old[FIN_G][4];
#pragma unroll
  for (int k = 0; k < FIN_G; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) old[k][c] = first ? 0.0 : S[(int64_t)min(gi[k], d - 1) * d + min(gj[k] + c, d - 1)];
#pragma unroll
  for (int k = 0; k < FIN_G; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (live[k] && gj[k] + c <= gi[k] && gj[k] + c < d) S[(int64_t)gi[k] * d + gj[k] + c] = old[k][c] + acc[k][c];
  if (I == J && rc == 0) {
    for (int c = tid; c < TILE; c += 256) {
      const int gc = I * TILE + c;
      if (gc >= d) break;
      double sum = 0.0;
      for (int s0 = 0; s0 < splits; s0 += FIN_SB) {
        double w[FIN_SB];
#pragma unroll
        for (int u = 0; u < FIN_SB; ++u) {
          const double x = colsq_part[(int64_t)min(s0 + u, splits - 1) * colsq_stride + gc];
          w[u] = (s0 + u < splits) ? x : 0.0;
        }
#pragma unroll
        for (int u = 0; u < FIN_SB; ++u) sum += w[u];
      }
      colsq[gc] = first ? sum : colsq[gc] + sum;
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(256, 1) void k_xtx_bf16(const uint16_t* __restrict__ X, int64_t ld, int64_t n_rows,
                                                     int d, int n_tiles, int64_t rps, int remap, int splits,
                                                     float* __restrict__ part, double* __restrict__ colsq_part,
                                                     int colsq_stride) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][BK][BROW];

  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int L = remap ? (b % 8) * (G / 8) + b / 8 : b;
  const int split = L / n_tiles;
  const int t = L - split * n_tiles;
  int I, J;
  tile_coords(t, I, J);
  const bool diag = (I == J);
  const int colA = I * BT, colB = J * BT;
  const int64_t r0 = (int64_t)split * rps;
  const int64_t r1 = min(n_rows, r0 + rps);
  const int nk = (int)((r1 - r0 + BK - 1) / BK);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool active = !(diag && wm == 0 && wn == 1);  // upper-right quadrant of a diagonal tile

  // global -> register staging: pass p covers rows (tid/32) + 8p, 8 columns at (tid%32)*8
  const int ld_row = tid >> 5;
  const int ld_col = (tid & 31) * 8;
  uint4 ra[4], rb[4];
  double csq[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) csq[q] = 0.0;

  auto gload = [&](int kt) {
    const int64_t base = r0 + (int64_t)kt * BK;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t row = base + ld_row + 8 * p;
      const bool ok = row < r1;
      ra[p] = load8_bf16<VEC>(X, ld, row, ok, colA + ld_col, d);
      if (!diag) rb[p] = load8_bf16<VEC>(X, ld, row, ok, colB + ld_col, d);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      *reinterpret_cast<uint4*>(&lds[st][0][ld_row + 8 * p][ld_col]) = ra[p];
      if (!diag) *reinterpret_cast<uint4*>(&lds[st][1][ld_row + 8 * p][ld_col]) = rb[p];
    }
    if (diag) {
#pragma unroll
      for (int p = 0; p < 4; ++p) sq_accum8(csq, ra[p]);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  const int g = lane >> 4, s = lane & 15;
  const int opB = diag ? 0 : 1;

  if (nk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    if (active) {
#pragma unroll 1
      for (int k16 = 0; k16 < BK; k16 += 16) {
        const int kb = k16 + 8 * (g >> 1) + (s >> 2);
        const int ioff = 16 * (g & 1) + (s & 3) * 4;
        bf16x8 fa[4], fb[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int ic = wm * 128 + mb * 32 + ioff;
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&lds[st][0][kb][ic]);
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&lds[st][0][kb + 4][ic]);
          fa[mb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int jc = wn * 128 + nb * 32 + ioff;
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&lds[st][opB][kb][jc]);
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&lds[st][opB][kb + 4][jc]);
          fb[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // fp32 partial of this (slice, tile): element (i, j) at i * 256 + j
  if (active) {
    float* dst = part + ((int64_t)split * n_tiles + t) * (BT * BT);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int j = wn * 128 + nb * 32 + (lane & 31);
          dst[i * BT + j] = acc[mb][nb][r];
        }
  }
  if (diag) {
    // reduce the 8 row-groups of column sums in a fixed order
    double* red = reinterpret_cast<double*>(&lds[0][0][0][0]);  // 8 x 256 doubles = 16 KB
#pragma unroll
    for (int q = 0; q < 8; ++q) red[ld_row * BT + ld_col + q] = csq[q];
    __syncthreads();
    double sum = 0.0;
#pragma unroll
    for (int rg = 0; rg < 8; ++rg) sum += red[rg * BT + tid];
    colsq_part[(int64_t)split * colsq_stride + colA + tid] = sum;
  }
}

// ---------------------------------------------------------------------------------------------------
// bf16 X, 16-byte aligned rows: direct-to-LDS pipeline
//
// Each 32-row stage of a 256-column operand block is fetched with buffer_load_dwordx4 ... lds (no staging
// registers) into one of NSTG LDS stage buffers, NSTG - 1 stages ahead of the MFMAs. One DMA instruction
// moves 1 KB = two 512-byte rows. Rows are stored unpadded; the 16-byte chunks of row k are XOR-swizzled
// by 4 * (k mod 4), so the four rows that one transposing read touches (64 B each) fall on four disjoint
// quarters of the 64 banks. Rows past the slice end and columns past `in` are outside the buffer range
// and arrive as zeros. Stage buffers are separate LDS arrays addressed with compile-time indices, so the
// compiler can tell a DMA into one stage from reads of another and only the explicit vmcnt waits order
// them. With five stages the ring fills the 160 KB of LDS; four stages (128 KB) are in flight per CU,
// which is what covers the fabric latency at this request rate.
// ---------------------------------------------------------------------------------------------------
#ifndef GPTQ_XTX_STAGES
#define GPTQ_XTX_STAGES 5
#endif
constexpr int NSTG = GPTQ_XTX_STAGES;
constexpr int ROW_B = 512;               // one row of a 256-column bf16 operand block
constexpr int OP_B = BK * ROW_B;         // 16384 B per operand per stage
constexpr int STG_B = 2 * OP_B;          // 32768 B per stage
#ifndef GPTQ_XTX_WAVES
#define GPTQ_XTX_WAVES 8
#endif
constexpr int XWAVES = GPTQ_XTX_WAVES;   // waves per workgroup: 2 (M) x XWAVES/2 (N)
constexpr int XWN = XWAVES / 2;          // waves along N
constexpr int XNB = (BT / XWN) / 32;     // 32-column MFMA blocks per wave along N
constexpr int DMA_PAIRS = (BK / 2) / XWAVES;  // row pairs per wave per operand per stage
static_assert(NSTG >= 3 && NSTG <= 5, "stage count");

__shared__ __attribute__((aligned(1024))) uint8_t g_stage0[STG_B];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage1[STG_B];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage2[STG_B];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage3[STG_B];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage4[STG_B];

template <int S>
__device__ __forceinline__ uint8_t* stage_buf() {
  if constexpr (S == 0) return g_stage0;
  else if constexpr (S == 1) return g_stage1;
  else if constexpr (S == 2) return g_stage2;
  else if constexpr (S == 3) return g_stage3;
  else return g_stage4;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// byte offset of (row k, 8-element chunk q) inside one operand's stage buffer
__device__ __forceinline__ int stage_off(int k, int q) {
  return k * ROW_B + ((q ^ ((k & 3) << 2)) << 4);
}

// s_waitcnt with vmcnt = N (expcnt and lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef __attribute__((ext_vector_type(4))) int i32x4;

struct DmaCtx {
  i32x4 rsrc;         // buffer resource of this workgroup's row slice (out-of-range reads return 0)
  int64_t row_bytes;  // ld * 2
  int colA, colB, d;
  int wave, lane;
};

// buffer_load_dwordx4 ... lds: 64 lanes x 16 B to LDS[m0 + lane * 16]. Written as inline asm so that the
// compiler does not add its own (conservative, vmcnt(0)) waits before every LDS read that follows; the
// stage pipeline orders the DMA with explicit vmcnt waits and barriers, and the main loop issues no other
// vector-memory instruction.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// One DMA instruction of stage kt: row pair wave * DMA_PAIRS + pp of operand slot `op` (block `col0`).
template <int S>
__device__ __forceinline__ void dma_one(const DmaCtx& c, int kt, int op, int col0, int pp) {
  const uint32_t base = (uint32_t)(uintptr_t)(stage_buf<S>() + op * OP_B);
  const int half = c.lane >> 5;
  const int p = c.wave * DMA_PAIRS + pp;
  const int k = 2 * p + half;
  const int q = (c.lane & 31) ^ ((k & 3) << 2);
  const int col = col0 + 8 * q;
  const int row = kt * BK + k;
  const uint32_t voff = (col < c.d) ? (uint32_t)(row * c.row_bytes + col * 2) : 0x80000000u;
  dma16(c.rsrc, __builtin_amdgcn_readfirstlane(base + p * 2 * ROW_B), voff);
}

// Issue the DMA of stage kt (32 rows) of operand block `col0` into operand slot `op` of stage buffer S.
template <int S>
__device__ __forceinline__ void dma_stage(const DmaCtx& c, int kt, int op, int col0) {
  const uint32_t base = (uint32_t)(uintptr_t)(stage_buf<S>() + op * OP_B);
  const int half = c.lane >> 5;
#pragma unroll
  for (int pp = 0; pp < DMA_PAIRS; ++pp) {
    const int p = c.wave * DMA_PAIRS + pp;    // row pair within the stage
    const int k = 2 * p + half;               // row within the stage; LDS chunk (lane & 31) of it holds
    const int q = (c.lane & 31) ^ ((k & 3) << 2);  // logical chunk q (the swizzle of stage_off)
    const int col = col0 + 8 * q;
    const int row = kt * BK + k;              // row within the slice
    const uint32_t voff = (col < c.d) ? (uint32_t)(row * c.row_bytes + col * 2) : 0x80000000u;
    dma16(c.rsrc, __builtin_amdgcn_readfirstlane(base + p * 2 * ROW_B), voff);
  }
}

// load the 2 x 4 bf16 of an MFMA operand fragment (32 x 16 block starting at column c0, k-rows k16..k16+15)
__device__ __forceinline__ bf16x8 frag_tr(const uint8_t* opbase, int k16, int c0, int g, int s) {
  const int k = k16 + 8 * (g >> 1) + (s >> 2);
  const int c = c0 + 16 * (g & 1) + (s & 3) * 4;
  const int off = stage_off(k, c >> 3) + (c & 7) * 2;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(opbase + off));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(opbase + off + 4 * ROW_B));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int I, int N, typename F>
__device__ __forceinline__ void xstatic_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    xstatic_for<I + 1, N>(f);
  }
}

// One 32-row stage: wait for this stage's DMA, barrier, read all 2 x (4 + XNB) operand fragments of the
// stage, then issue the DMA of the stage NSTG - 1 ahead one instruction at a time between the first
// half's MFMAs (a burst of DMA instructions would stall the issuing waves while the address unit drains
// it, leaving the matrix units idle), then the second half's MFMAs. The DMA is issued unconditionally:
// past the slice end its offsets are out of range and it fetches zeros into a stage buffer that is never
// read, which keeps the vmcnt bookkeeping uniform. Two waves share each SIMD, so one wave's MFMAs cover
// the other's barrier and LDS waits. In diagonal tiles the waves whose block lies above the diagonal
// add the fp64 squares of the stage instead (4 columns per lane).
template <bool DIAG, int S>
__device__ __forceinline__ void xtx_stage(const DmaCtx& c, int kt, f32x16 (&acc)[4][XNB], double (&csq)[4], int wm,
                                          int wn, bool active) {
  constexpr int PER = (DIAG ? 1 : 2) * DMA_PAIRS;  // DMA instructions per wave per stage
  constexpr int SN = (S + NSTG - 1) % NSTG;        // buffer of stage kt + NSTG - 1
  wait_vmcnt<(NSTG - 2) * PER>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const uint8_t* A = stage_buf<S>();
  const uint8_t* B = DIAG ? A : A + OP_B;
  const int g = c.lane >> 4, s = c.lane & 15;
  auto dma_i = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
    dma_one<SN>(c, kt + NSTG - 1, i / DMA_PAIRS, (i / DMA_PAIRS) ? c.colB : c.colA, i % DMA_PAIRS);
  };
  if (active) {
    bf16x8 fa0[4], fb0[XNB], fa1[4], fb1[XNB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) fa0[mb] = frag_tr(A, 0, wm * 128 + mb * 32, g, s);
#pragma unroll
    for (int nb = 0; nb < XNB; ++nb) fb0[nb] = frag_tr(B, 0, wn * (BT / XWN) + nb * 32, g, s);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) fa1[mb] = frag_tr(A, 16, wm * 128 + mb * 32, g, s);
#pragma unroll
    for (int nb = 0; nb < XNB; ++nb) fb1[nb] = frag_tr(B, 16, wn * (BT / XWN) + nb * 32, g, s);
    constexpr int NM = 4 * XNB;     // MFMAs per half
    constexpr int GM = NM / PER;    // first-half MFMAs after each DMA instruction
    static_assert(NM % PER == 0, "MFMA groups");
    xstatic_for<0, PER>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_sched_barrier(0);
      dma_i(ic);
      __builtin_amdgcn_sched_barrier(0);
      xstatic_for<0, GM>([&](auto jc) {
        constexpr int f = i * GM + decltype(jc)::value;
        acc[f / XNB][f % XNB] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[f / XNB], fb0[f % XNB], acc[f / XNB][f % XNB], 0, 0, 0);
      });
    });
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < XNB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[mb], fb1[nb], acc[mb][nb], 0, 0, 0);
  } else {
    xstatic_for<0, PER>(dma_i);
    if (DIAG) {
      // the waves above the diagonal of a diagonal tile share the stage's rows between them
      constexpr int NIDLE = XWN / 2;          // waves (0, wn) with wn >= XWN/2
      constexpr int RPW = BK / NIDLE;         // rows per idle wave
      const int cc = c.lane * 4;              // columns cc..cc+3
      const int kr = (wn - XWN / 2) * RPW;
#pragma unroll 4
      for (int k = 0; k < RPW; ++k) {
        const uint2 v = *reinterpret_cast<const uint2*>(A + stage_off(kr + k, cc >> 3) + (cc & 7) * 2);
        const double x0 = (double)__uint_as_float(v.x << 16), x1 = (double)__uint_as_float(v.x & 0xFFFF0000u);
        const double x2 = (double)__uint_as_float(v.y << 16), x3 = (double)__uint_as_float(v.y & 0xFFFF0000u);
        csq[0] = fma(x0, x0, csq[0]);
        csq[1] = fma(x1, x1, csq[1]);
        csq[2] = fma(x2, x2, csq[2]);
        csq[3] = fma(x3, x3, csq[3]);
      }
    }
  }
}

// stages kt + S .. kt + NSTG - 1 of one turn of the ring; false once the slice is done
template <bool DIAG, int S>
__device__ __forceinline__ bool xtx_ring(const DmaCtx& c, int kt, int nk, f32x16 (&acc)[4][XNB], double (&csq)[4],
                                         int wm, int wn, bool active) {
  if constexpr (S == NSTG) {
    return true;
  } else {
    if (kt + S >= nk) return false;
    xtx_stage<DIAG, S>(c, kt + S, acc, csq, wm, wn, active);
    return xtx_ring<DIAG, S + 1>(c, kt, nk, acc, csq, wm, wn, active);
  }
}

template <bool DIAG, int S>
__device__ __forceinline__ void xtx_prologue(const DmaCtx& c) {
  if constexpr (S < NSTG - 1) {
    dma_stage<S>(c, S, 0, c.colA);
    if (!DIAG) dma_stage<S>(c, S, 1, c.colB);
    xtx_prologue<DIAG, S + 1>(c);
  }
}

template <bool DIAG>
__device__ __forceinline__ void xtx_dma_body(const DmaCtx& c, int nk, f32x16 (&acc)[4][XNB], double (&csq)[4], int wm,
                                             int wn, bool active) {
  xtx_prologue<DIAG, 0>(c);  // stages 0 .. NSTG-2 in flight (stages past the slice fetch zeros)
  for (int kt = 0; kt < nk; kt += NSTG)
    if (!xtx_ring<DIAG, 0>(c, kt, nk, acc, csq, wm, wn, active)) break;
  wait_vmcnt<0>();  // no DMA may still be writing LDS when the workgroup moves on
  __builtin_amdgcn_s_barrier();
}

__global__ __launch_bounds__(XWAVES * 64, 1) void k_xtx_bf16_dma(const uint16_t* __restrict__ X, int64_t ld, int64_t n_rows,
                                                         int d, int n_tiles, int64_t rps, int remap, int splits,
                                                         float* __restrict__ part, double* __restrict__ colsq_part,
                                                         int colsq_stride) {
  // Workgroup b runs on XCD b % 8 (round-robin dispatch). Each XCD owns a contiguous run of `cs` tiles in
  // super-tile order and walks the row slices in order; all XCDs are on the same slices at the same time,
  // so each slice comes from HBM about once and the XCDs share it through the last-level cache.
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int m = b >> 3;
  const int cs = remap;  // tiles per XCD
  const int split = m / cs;
  const int p = xcd * cs + (m - split * cs);
  if (p >= n_tiles) return;  // padding slot (tile count not a multiple of 8)
  int I, J;
  supertile_coords(p, (int)((d + BT - 1) / BT), I, J);
  int t = I * (I + 1) / 2 + J;
  const bool diag = (I == J);
  const int64_t r0 = (int64_t)split * rps;
  const int64_t r1 = min(n_rows, r0 + rps);
  const int nk = (int)((r1 - r0 + BK - 1) / BK);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / XWN, wn = wave % XWN;  // 2 x XWN waves of 128 x (256 / XWN)
  const bool active = !(diag && wm == 0 && wn >= XWN / 2);  // blocks above the diagonal of a diagonal tile

  DmaCtx c;
  {
    const uint64_t addr = (uint64_t)(uintptr_t)(X + r0 * ld);
    c.rsrc = (i32x4){__builtin_amdgcn_readfirstlane((int)(uint32_t)addr),
                     __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32) & 0xFFFF),
                     __builtin_amdgcn_readfirstlane((int)((r1 - r0) * ld * 2)), 0x00020000};
  }
  c.row_bytes = ld * 2;
  c.colA = I * BT;
  c.colB = J * BT;
  c.d = d;
  c.wave = wave;
  c.lane = lane;

  f32x16 acc[4][XNB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < XNB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;
  double csq[4] = {0.0, 0.0, 0.0, 0.0};

  if (diag) xtx_dma_body<true>(c, nk, acc, csq, wm, wn, active);
  else xtx_dma_body<false>(c, nk, acc, csq, wm, wn, active);

  if (active) {
    float* dst = part + ((int64_t)split * n_tiles + t) * (BT * BT);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < XNB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int j = wn * (BT / XWN) + nb * 32 + (lane & 31);
          dst[i * BT + j] = acc[mb][nb][r];
        }
  }
  if (diag) {
    // the column-sum waves hold disjoint row ranges of every stage; add them in a fixed order
    constexpr int NIDLE = XWN / 2;
    double* red = reinterpret_cast<double*>(g_stage0);  // NIDLE x 256 doubles; the DMA ring is drained
    if (!active) {
#pragma unroll
      for (int q = 0; q < 4; ++q) red[(wn - XWN / 2) * 256 + lane * 4 + q] = csq[q];
    }
    __syncthreads();
    if (tid < BT) {
      double sum = red[tid];
#pragma unroll
      for (int w = 1; w < NIDLE; ++w) sum += red[w * 256 + tid];
      colsq_part[(int64_t)split * colsq_stride + c.colA + tid] = sum;
    }
  }
}

// ---------------------------------------------------------------------------------------------------
// fp32 X
// ---------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void k_xtx_f32(const float* __restrict__ X, int64_t ld, int64_t n_rows, int d,
                                                    int n_tiles, int64_t rps, int remap, int splits,
                                                    float* __restrict__ part, double* __restrict__ colsq_part,
                                                    int colsq_stride) {
  __shared__ __attribute__((aligned(16))) float lds[2][2][FK][FROW];
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int L = remap ? (b % 8) * (G / 8) + b / 8 : b;
  const int split = L / n_tiles;
  const int t = L - split * n_tiles;
  int I, J;
  tile_coords(t, I, J);
  const bool diag = (I == J);
  const int colA = I * FT, colB = J * FT;
  const int64_t r0 = (int64_t)split * rps;
  const int64_t r1 = min(n_rows, r0 + rps);
  const int nk = (int)((r1 - r0 + FK - 1) / FK);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool active = !(diag && wm == 0 && wn == 1);

  // staging: 16 rows x 128 floats per operand = 2048 floats = 8 per thread: row tid/16 (0..15), cols (tid%16)*8
  const int ld_row = tid >> 4;
  const int ld_col = (tid & 15) * 8;
  float ra[8], rb[8];
  double csq[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) csq[q] = 0.0;

  auto gload = [&](int kt) {
    const int64_t row = r0 + (int64_t)kt * FK + ld_row;
    const bool ok = row < r1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int ca = colA + ld_col + q, cb = colB + ld_col + q;
      ra[q] = (ok && ca < d) ? X[row * ld + ca] : 0.0f;
      rb[q] = (!diag && ok && cb < d) ? X[row * ld + cb] : 0.0f;
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      lds[st][0][ld_row][ld_col + q] = ra[q];
      if (!diag) lds[st][1][ld_row][ld_col + q] = rb[q];
    }
    if (diag) {
#pragma unroll
      for (int q = 0; q < 8; ++q) csq[q] = fma((double)ra[q], (double)ra[q], csq[q]);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int opB = diag ? 0 : 1;

  if (nk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    if (active) {
#pragma unroll
      for (int k4 = 0; k4 < FK; k4 += 4) {
        const int k = k4 + (lane >> 4);
        float fa[4], fb[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) fa[mb] = lds[st][0][k][wm * 64 + mb * 16 + (lane & 15)];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) fb[nb] = lds[st][opB][k][wn * 64 + nb * 16 + (lane & 15)];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }
  if (active) {
    float* dst = part + ((int64_t)split * n_tiles + t) * (FT * FT);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = wm * 64 + mb * 16 + 4 * (lane >> 4) + r;
          const int j = wn * 64 + nb * 16 + (lane & 15);
          dst[i * FT + j] = acc[mb][nb][r];
        }
  }
  if (diag) {
    double* red = reinterpret_cast<double*>(&lds[0][0][0][0]);  // 16 x 128 doubles = 16 KB
#pragma unroll
    for (int q = 0; q < 8; ++q) red[ld_row * FT + ld_col + q] = csq[q];
    __syncthreads();
    if (tid < FT) {
      double sum = 0.0;
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) sum += red[rg * FT + tid];
      colsq_part[(int64_t)split * colsq_stride + colA + tid] = sum;
    }
  }
}

}  // namespace

// Rows of X that one fp32 partial sum may cover: every (slice, tile) item sums at most this many rows on
// the matrix cores before its partial goes to the fp64 combine. The fp32 rounding error of S grows with
// the square root of the chain length, and it decides how many near-tie codes of a sensitive layer flip
// (3-bit, groups, act_order at in = 11008: 193 / 1135 / 556 of 2.8 M sampled codes with 4096 / 8192 /
// ~12k-row slices, the spread being the cascades that follow a flip). Shorter slices cost partial-sum
// traffic: q_proj's Hessian took 5.04 / 4.62 / 4.69 ms with a cap of 4096 / 8192 / 16384 rows.
#ifndef GPTQ_XTX_SLICE_ROWS
#define GPTQ_XTX_SLICE_ROWS 8192
#endif
constexpr int64_t SLICE_ROWS = GPTQ_XTX_SLICE_ROWS;
static_assert(SLICE_ROWS % BK == 0 && SLICE_ROWS % FK == 0 && SLICE_ROWS >= 1024, "slice length");
constexpr int MAX_SPLITS = 64;  // slices per launch; longer inputs are processed in chunks

HessianPlan hessian_plan(int64_t n_rows, int64_t in, int dtype, size_t max_bytes) {
  HessianPlan p{};
  p.n_rows = n_rows;
  p.in = in;
  p.dtype = dtype;
  p.tile = (dtype == GPTQ_BF16) ? BT : FT;
  const int kstep = (dtype == GPTQ_BF16) ? BK : FK;
  p.n_tb = (int)ceil_div(in, p.tile);
  p.n_tiles = p.n_tb * (p.n_tb + 1) / 2;
  const size_t per_split = (size_t)p.n_tiles * p.tile * p.tile * sizeof(float) + (size_t)p.n_tb * p.tile * sizeof(double);
  // Rows per launch: at most MAX_SPLITS slices of SLICE_ROWS (fewer when the partials must fit max_bytes)
  int64_t cap = MAX_SPLITS;
  if (max_bytes) cap = std::max<int64_t>(1, std::min<int64_t>(cap, (int64_t)(max_bytes / (per_split + 512))));
  p.chunk_rows = std::min<int64_t>(n_rows, cap * SLICE_ROWS);
  // Slices of one chunk: enough that none covers more than SLICE_ROWS rows; beyond that, balance
  // tiles x slices over the CUs (one resident workgroup per CU), keep slices at least 1024 rows long,
  // and charge a little for every extra slice (its fp32 partial is written and read once).
  const int cus = 256;  // planning constant (MI355X); the launch itself works for any CU count
  const int64_t s_min = ceil_div(p.chunk_rows, SLICE_ROWS);
  const int64_t s_max = std::max<int64_t>(s_min, std::min<int64_t>(cap, p.chunk_rows / 1024));
  double best = 1e30;
  int best_s = (int)s_min;
  for (int64_t s = s_min; s <= s_max; ++s) {
    const double rounds = (double)ceil_div((int64_t)p.n_tiles * s, cus);
    const double cost = rounds / s + 0.004 * s;
    if (cost < best - 1e-12) {
      best = cost;
      best_s = (int)s;
    }
  }
  p.splits = best_s;
  p.rows_per_split = ceil_div(ceil_div(p.chunk_rows, p.splits), kstep) * kstep;
  p.splits = (int)ceil_div(p.chunk_rows, p.rows_per_split);
  p.part_bytes = align_up((size_t)p.splits * p.n_tiles * p.tile * p.tile * sizeof(float), 256);
  p.colsq_part_bytes = align_up((size_t)p.splits * p.n_tb * p.tile * sizeof(double), 256);
  p.total_bytes = p.part_bytes + p.colsq_part_bytes;
  p.ld = 0;
  return p;
}

// One chunk of at most p.chunk_rows rows: the accumulation kernel (p.splits slices or fewer) and the
// fp64 combine into S / colsq.
static hipError_t hessian_chunk(const HessianPlan& p, const void* X, int64_t n_rows, double* S, double* colsq,
                                void* ws, hipStream_t stream, bool first) {
  float* part = reinterpret_cast<float*>(ws);
  double* cpart = reinterpret_cast<double*>(reinterpret_cast<char*>(ws) + p.part_bytes);
  const int splits = (int)ceil_div(n_rows, p.rows_per_split);
  const int grid = splits * p.n_tiles;
  const int remap = (grid % 8 == 0) ? 1 : 0;
  const int cs = (p.n_tiles + 7) / 8;         // tiles per XCD for the direct-to-LDS kernel
  const int grid_dma = 8 * cs * splits;
  const int cstride = p.n_tb * p.tile;
  if (p.dtype == GPTQ_BF16) {
    const bool vec = (p.ld % 8 == 0) && (p.in % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    const bool dma = vec && (p.rows_per_split * p.ld * 2 < ((int64_t)1 << 31));
    if (dma)
      hipLaunchKernelGGL(k_xtx_bf16_dma, dim3(grid_dma), dim3(XWAVES * 64), 0, stream, (const uint16_t*)X, p.ld,
                         n_rows, (int)p.in, p.n_tiles, p.rows_per_split, cs, splits, part, cpart, cstride);
    else if (vec)
      hipLaunchKernelGGL(k_xtx_bf16<true>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)X, p.ld, n_rows,
                         (int)p.in, p.n_tiles, p.rows_per_split, remap, splits, part, cpart, cstride);
    else
      hipLaunchKernelGGL(k_xtx_bf16<false>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)X, p.ld, n_rows,
                         (int)p.in, p.n_tiles, p.rows_per_split, remap, splits, part, cpart, cstride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_xtx_reduce<BT>, dim3((unsigned)(p.n_tiles * (BT / FIN_RC))), dim3(256), 0, stream, part,
                       cpart, cstride, p.n_tiles, splits, (int)p.in, S, colsq, first ? 1 : 0);
  } else {
    hipLaunchKernelGGL(k_xtx_f32, dim3(grid), dim3(256), 0, stream, (const float*)X, p.ld, n_rows, (int)p.in,
                       p.n_tiles, p.rows_per_split, remap, splits, part, cpart, cstride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_xtx_reduce<FT>, dim3((unsigned)(p.n_tiles * (FT / FIN_RC))), dim3(256), 0, stream, part,
                       cpart, cstride, p.n_tiles, splits, (int)p.in, S, colsq, first ? 1 : 0);
  }
  return hipGetLastError();
}

hipError_t hessian_launch(const HessianPlan& p, const void* X, double* S, double* colsq, void* ws,
                          hipStream_t stream, bool first) {
  const size_t esz = (p.dtype == GPTQ_BF16) ? 2 : 4;
  for (int64_t r0 = 0; r0 < p.n_rows; r0 += p.chunk_rows) {
    const void* Xc = reinterpret_cast<const char*>(X) + (size_t)r0 * (size_t)p.ld * esz;
    const hipError_t e =
        hessian_chunk(p, Xc, std::min(p.chunk_rows, p.n_rows - r0), S, colsq, ws, stream, first && r0 == 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gptq
