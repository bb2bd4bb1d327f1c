// The error-compensation loop on gfx950 (fp64 working copy).
//
// Lesson "GPTQ's error-compensation loop" (herodthegreater.github.io/pigeon/school/gptq_loop/): the columns
// are taken in order; each weight of column j is snapped to the grid, its residual divided by the pivot
// U[j][j] is that row's error, and the row's later columns k take off error * U[j][k]. GPTQ guide ("GPTQ", herodthegreater.github.io/pigeon/guide/gptq/),
// "The code, line by line": one scale per row from the starting weights, or, with groups, a scale from
// the already-updated weights of columns [j, j + group) at each group boundary; codes are
// clip(round(w / scale), -qmax, qmax). "Simplifications" mentions lazy 128-column batch updates.
//
// Schedule (right-looking, 128-column panels):
//  k_rowprep   W (bf16/fp32) -> fp64 working copy in quantization order, dead columns zeroed, per-row
//              start scale (block max reduction), or start scale and zero point (min and max).
//  k_panel     per panel: 16 lanes per row (lane c holds columns c, c+16, ..., c+112 in registers), the
//              upper part of the 128 x 128 block of U in LDS. Each step j broadcasts w_j from its owner
//              lane with DPP (row_newbcast), every lane of the row rounds it (IEEE division, round-half-even), and
//              updates its own columns with U[j][col] from LDS. Group maxima are 16-lane DPP max
//              reductions. Codes and errors stay in registers and are stored once per panel.
//  trailing    two levels of lazy updates on the fp64 MFMA GEMM core. Panels are grouped into outer
//              blocks of OB columns. After a panel, only the rest of its outer block is updated,
//              W[:, b1:ob1] -= Err[:, panel] U[panel, b1:ob1] (K = 128); after the last panel of an outer
//              block, every later column gets the whole block at once, W[:, ob1:] -= Err[:, block]
//              U[block, ob1:] (K = OB). The products are the ones of the column-by-column loop; only
//              their grouping (and so the floating-point summation order) changes, and the fp64 W is
//              read and written a few times instead of once per panel.
// The R route (gptq_quantize_layer_r) runs the same schedule from R = U^-1 and U's 128 x 128 diagonal
// blocks: the loop gives W0 - Q = Err U, so Err = D R with D = W0 - Q, and a panel P starts from
// W0_P + T_P U_PP with T = sum over earlier panels B of D_B R_BP. The lazy updates accumulate T += D R
// (the same products, into T instead of W), the working copy keeps W0, and k_panel<.., RF = true> writes
// D in place of Err and starts from W0 + T U_PP: with one grid per row T enters the loop's steps (step j
// propagates e_j - T_j), with groups inside the panel T_P U_PP is formed first on the matrix cores.
// Grids. Symmetric ([guide] "The code, line by line"): codes -qmax..qmax, qmax = 2^(b-1) - 1, scale =
// max(max|w|, 1e-12) / qmax, code = clip(round(w / scale)), value = code * scale. Asymmetric ([handbook]
// quantize_weight, dequantize_weight, gptq_quantize_row; the paper's default per the guide's
// "Simplifications"): codes 0..L, L = 2^b - 1, scale = (max - min) / L (1 when max = min), zero =
// clip(round(-min / scale), 0, L), code = clip(round(w / scale + zero), 0, L), value = scale (code - zero).
// Every division is correctly rounded and every rounding is to nearest even, as in the definition.
#include <atomic>
#include <type_traits>
#include <utility>

#include "common.h"
#include "dgemm.h"
#include "divide.h"

namespace gptq {

namespace {

constexpr int PW = 128;  // panel width
// the panel's U block in LDS, row a stored from column 16 (a / 16) on: urow(a) is where row a starts
__host__ __device__ constexpr int urow(int a) {
  return 2048 * (a >> 4) - 128 * (a >> 4) * ((a >> 4) - 1) + (a & 15) * (128 - 16 * (a >> 4));
}
constexpr int UPACK = urow(PW);
static_assert(PW == 128 && UPACK == 9216, "panel layout");
#ifndef GPTQ_QUANT_OB
#define GPTQ_QUANT_OB 1024
#endif
constexpr int OB = GPTQ_QUANT_OB;  // outer block of the lazy updates (a multiple of PW)
static_assert(OB % PW == 0, "outer block");
constexpr double SCALE_FLOOR = 1e-12;

template <int J, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (J < N) {
    f(std::integral_constant<int, J>{});
    static_for<J + 1, N>(f);
  }
}

// value of lane K of this lane's 16-lane row (one v_mov_b64_dpp, row_newbcast)
template <int K>
__device__ __forceinline__ double bcast16(double v) {
  return __builtin_amdgcn_mov_dpp(v, 0x150 + K, 0xF, 0xF, false);
}

// the value of v in lane addr / 4 (ds_bpermute on both halves)
__device__ __forceinline__ double bpermute_f64(int addr, double v) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_ds_bpermute(addr, (int)x);
  const int hi = __builtin_amdgcn_ds_bpermute(addr, (int)(x >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// value of lane (i - R) mod 16 of this lane's 16-lane row (DPP row_ror; 64-bit DPP takes only row_newbcast,
// so the two halves move separately)
template <int R>
__device__ __forceinline__ double ror16(double v) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(x & 0xFFFFFFFFll), 0x120 + R, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(x >> 32), 0x120 + R, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ double max16(double v) {
  v = fmax(v, ror16<8>(v));
  v = fmax(v, ror16<4>(v));
  v = fmax(v, ror16<2>(v));
  v = fmax(v, ror16<1>(v));
  return v;
}

__device__ __forceinline__ double min16(double v) {
  v = fmin(v, ror16<8>(v));
  v = fmin(v, ror16<4>(v));
  v = fmin(v, ror16<2>(v));
  v = fmin(v, ror16<1>(v));
  return v;
}

__device__ __forceinline__ double sum16(double v) {
  v += ror16<8>(v);
  v += ror16<4>(v);
  v += ror16<2>(v);
  v += ror16<1>(v);
  return v;
}

template <typename T>
__device__ __forceinline__ double to_f64(T v);
template <>
__device__ __forceinline__ double to_f64<float>(float v) { return (double)v; }
template <>
__device__ __forceinline__ double to_f64<uint16_t>(uint16_t v) {
  return (double)__uint_as_float(((uint32_t)v) << 16);
}

// One workgroup per row: Wq[r][j] = W[r][perm[j]] (0 for dead inputs). Symmetric: scale_row[r] =
// max(max|w|, 1e-12) / qmax. Asymmetric: scale_row[r] and zero_row[r] from the row's min and max. With
// group == 0 these are also the outputs.
template <typename T, bool ASYM>
__global__ __launch_bounds__(256) void k_rowprep(const T* __restrict__ W, int64_t ld_w, int in,
                                                 const int32_t* __restrict__ perm, const uint8_t* __restrict__ dead,
                                                 double qmax, int group, double* __restrict__ Wq,
                                                 double* __restrict__ scale_row, double* __restrict__ zero_row,
                                                 float* __restrict__ scales, int32_t* __restrict__ zeros,
                                                 double* __restrict__ row_loss, unsigned* __restrict__ status) {
  __shared__ double red[256];
  __shared__ double red2[256];
  const int r = blockIdx.x;
  const T* wr = W + (int64_t)r * ld_w;
  double* q = Wq + (int64_t)r * in;
  double mx = ASYM ? -INFINITY : 0.0, mn = INFINITY;
  bool bad = false;  // a NaN or Inf among the row's live weights
  // sixteen columns per thread per pass (one pass at in = 4096): the index loads, then the gathered loads,
  // all in flight together
  constexpr int CPT = 16;
  for (int j0 = threadIdx.x; j0 < in; j0 += 256 * CPT) {
    int p[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = j0 + 256 * u;
      p[u] = (j < in) ? min(max(perm[j], 0), in - 1) : 0;
    }
    double v[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const bool dd = dead[p[u]] != 0;
      const double x = to_f64<T>(wr[p[u]]);
      v[u] = dd ? 0.0 : x;
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = j0 + 256 * u;
      if (j < in) {
        q[j] = v[u];
        bad = bad || !isfinite(v[u]);
        if (ASYM) {
          mx = fmax(mx, v[u]);
          mn = fmin(mn, v[u]);
        } else {
          mx = fmax(mx, fabs(v[u]));
        }
      }
    }
  }
  if (bad) atomicOr(status, DEV_STATUS_NONFINITE);
  red[threadIdx.x] = mx;
  red2[threadIdx.x] = mn;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + s]);
      red2[threadIdx.x] = fmin(red2[threadIdx.x], red2[threadIdx.x + s]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double s, z = 0.0;
    if (ASYM) {
      const double hi = red[0], lo = red2[0];
      s = (hi > lo) ? (hi - lo) / qmax : 1.0;
      z = fmin(fmax(rint(-lo / s), 0.0), qmax);
    } else {
      s = fmax(red[0], SCALE_FLOOR) / qmax;
    }
    scale_row[r] = s;
    if (ASYM) zero_row[r] = z;
    if (group == 0) {
      scales[r] = (float)s;
      if (ASYM) zeros[r] = (int32_t)z;
    }
    if (row_loss) row_loss[r] = 0.0;
  }
}

// INPANEL = false: one scale per row, or groups that are multiples of 128 (the scale is recomputed at
// panels where b0 % group == 0 and carried across panels in scale_row); INPANEL = true: groups dividing
// 128 (boundaries inside the panel at j % group == 0).
// RF: the factor comes in the R form (GPTQ_FACTOR_R_FORM): the block's U is read from the reversed lower part of
// R's diagonal block, 1 / U[j][j] is R[j][j], Wq holds the starting weights W0 and T the accumulated D R of
// the earlier panels; the rows start from W0_P + T_P U_PP (with INPANEL formed first on the matrix cores,
// otherwise folded into the steps), and D = W0 - Q is stored instead of the errors for the products that
// follow.
// GC: the group size when it is known at compile time (INPANEL with group 32, 64 or 128); the column steps
// are then expanded at compile time and only the steps that open a group carry the group's grid code
// (groups of 64 and 128 keep the 74 registers of the one-grid-per-row form, against 151; groups of 32 take
// 256 without spilling, which two workgroups per CU still hold). GC = 0: the group size comes from `group`
// (one grid per row, or in-panel groups of 1 .. 16, whose steps stay a loop over the 16-column blocks:
// expanded, groups of 16 spill, faster at 4096 rows and slower at 11008).
template <bool INPANEL, bool ASYM, bool RF, int GC>
__global__ __launch_bounds__(256) void k_panel(double* __restrict__ Wq, int out, int in, int b0,
                                               const double* __restrict__ U, const int32_t* __restrict__ perm,
                                               double* __restrict__ scale_row, double* __restrict__ zero_row,
                                               double qmax, int group, int n_groups, int8_t* __restrict__ codes,
                                               float* __restrict__ scales, int32_t* __restrict__ zeros,
                                               double* __restrict__ Err, int ld_err, double* __restrict__ row_loss,
                                               const double* __restrict__ T, int t_valid) {
  // U panel block, upper part only: row a holds columns 16 (a / 16) .. 127 (the 16-column blocks that reach
  // the diagonal, zeros left of it), 72 KB instead of 128, so two panel workgroups fit in a CU (see
  // launch_panel)
  __shared__ double Us[UPACK];
  __shared__ double rdiag[PW];
  __shared__ int pidx[PW];
  const int tid = threadIdx.x;
  const int pw = min(PW, in - b0);
  const int c = tid & 15;
  const int r = blockIdx.x * 16 + (tid >> 4);
  const bool rok = r < out;
  // Every global load of the prologue is issued before the first wait: addresses are clamped into their
  // operands and the values selected afterwards, so that no load sits behind a branch (with the loads
  // guarded, the compiler kept each 16-row block's loads behind the previous block's LDS stores: eight
  // round trips to memory instead of one). The row's weights (16 lanes per row, lane c holding columns
  // c + 16 m), RF: the row's T_P, the pivot and permutation entry of column tid, then the U block.
  const int64_t rbase = (int64_t)(rok ? r : 0) * in + b0;
  double w[8], t[8];  // the raw loads first; the out-of-range ones are zeroed after the U block's loads
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int col = c + 16 * m;
    w[m] = Wq[rbase + (rok && col < pw ? col : 0)];
    if constexpr (RF) t[m] = T[rbase + (t_valid && rok && col < pw ? col : 0)];
  }
  // the row's grid from the row prep or the previous panel (one grid per row, or a group carried over)
  const double s_row = scale_row[rok ? r : 0];
  const double z_row = ASYM ? zero_row[rok ? r : 0] : 0.0;
  static_assert(PW <= 256, "one thread per panel column");
  const bool dcol = tid < pw;
  const int dc = dcol ? tid : 0;
  const double udiag_x = U[(int64_t)(b0 + dc) * in + b0 + dc];  // RF: R[j][j] = 1 / U[j][j]
  const int pcol_x = perm[b0 + dc];
  const double udiag = dcol ? udiag_x : 0.0;
  const int pcol = dcol ? pcol_x : 0;
  // the U block, 16-row block k holding 16 rows of 128 - 16k stored columns (8 - k elements per thread):
  // element (a, b) of the panel's U_PP, b >= a (RF: b > a, the diagonal comes below), read from
  // U[b0 + a][b0 + b], or (RF) from the R form's reversed lower part at (b0 + pw - 1 - a, b0 + pw - 1 - b)
  auto u_elem = [&](int k, int q, bool& valid) -> int64_t {
    const int RL = PW - 16 * k;
    const int i = tid + 256 * q;
    const int a = 16 * k + i / RL, b = 16 * k + i % RL;
    valid = a < pw && b < pw && (RF ? b > a : b >= a);
    const int aa = valid ? a : 0, bb = valid ? b : 0;
    return RF ? (int64_t)(b0 + pw - 1 - aa) * in + b0 + pw - 1 - bb : (int64_t)(b0 + aa) * in + b0 + bb;
  };
  double uv[36];  // 8 + 7 + ... + 1
  static_for<0, 8>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int OFF = 8 * k - k * (k - 1) / 2;
#pragma unroll
    for (int q = 0; q < 8 - k; ++q) {
      bool valid;
      uv[OFF + q] = U[u_elem(k, q, valid)];
    }
  });
  // empty uses here keep the compiler from sinking the loads above to their first real uses (past the
  // barrier, or into the branch that stores the pivots), which cost a round trip each
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::"v"(udiag_x), "v"(pcol_x), "v"(s_row), "v"(z_row));
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int col = c + 16 * m;
    w[m] = (rok && col < pw) ? w[m] : 0.0;
    if constexpr (RF) t[m] = (t_valid && rok && col < pw) ? t[m] : 0.0;
    asm volatile("" ::"v"(w[m]));
    if constexpr (RF) asm volatile("" ::"v"(t[m]));
  }
  static_for<0, 8>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int OFF = 8 * k - k * (k - 1) / 2;
#pragma unroll
    for (int q = 0; q < 8 - k; ++q) {
      bool valid;
      (void)u_elem(k, q, valid);
      Us[urow(16 * k) + tid + 256 * q] = valid ? uv[OFF + q] : 0.0;
    }
  });
  if (RF) __syncthreads();  // the block's stores above are done before the diagonal is written
  if (tid < PW) {
    if (RF) {
      rdiag[tid] = udiag;
      if (dcol) Us[urow(tid) + tid - 16 * (tid >> 4)] = 1.0 / udiag;  // U[j][j], for the first product below
    } else {
      rdiag[tid] = dcol ? 1.0 / udiag : 0.0;
    }
    pidx[tid] = dcol ? min(max(pcol, 0), in - 1) : 0;
  }
  __syncthreads();

  double w0[8];  // RF: the starting weights of the lane's columns, for D = W0 - Q
  if constexpr (RF) {
#pragma unroll
    for (int m = 0; m < 8; ++m) w0[m] = w[m];
    if constexpr (!INPANEL) {
      if (t_valid) {
        // one grid per row (group 0, the only case without in-panel groups that the R form takes): only
        // the column being decided needs its current value, so the panel starts from W0_k + T_k U_kk and
        // the rest of T_P U_PP enters the loop, where step j takes off (e_j - T_j) U_jk, not e_j U_jk
#pragma unroll
        for (int m = 0; m < 8; ++m) w[m] = fma(t[m], Us[urow(c + 16 * m) + c], w[m]);
      }
    } else if (t_valid) {
      // groups inside the panel: a group's grid is set from the current values of all its columns, so the
      // whole T_P U_PP is added first, on the matrix cores with w as the accumulator.
      // v_mfma_f64_4x4x4f64 forms four 4 x 4 x 4 block products at once: lane l supplies A[l % 16][l / 16]
      // and B[l / 16][l % 16], block g takes A's rows 4g .. 4g + 3 and B's columns 4g .. 4g + 3, and its
      // entry (i, j) lands in lane 16 i + 4 g + j. With the wave's four rows of T_P as the A rows of every
      // block and 16 columns of U_PP as B, lane 16 r + c receives row r, column c of the product, which is
      // the layout in which the lanes hold w. U_PP's rows come from LDS; the A values come from the lanes
      // that hold them (T_P[r][k] is in lane 16 r + k % 16, register k / 16), through ds_bpermute.
      const int lane = tid & 63, lr = lane & 15, lk = lane >> 4;
      static_for<0, PW / 4>([&](auto kc) {
        constexpr int k0 = 4 * decltype(kc)::value, mb = k0 / 16;
        const double a = bpermute_f64(4 * (16 * (lane & 3) + (k0 & 15) + lk), t[mb]);
        const int rb = urow(k0 + lk) + lr - 16 * mb;  // row k0 + lk of U_PP, stored from column 16 mb on
#pragma unroll
        for (int m = mb; m < 8; ++m) w[m] = __builtin_amdgcn_mfma_f64_4x4x4f64(a, Us[rb + 16 * m], w[m], 0, 0, 0);
      });
    }
  }

  double s = 1.0;
  double sy = 1.0;  // RN(1 / s)
  double z = 0.0;   // zero point (asymmetric grid)
  // grid parameters of a group from the current weights: lo/hi are the group's min and max (asymmetric)
  // or 0 and max|w| (symmetric)
  auto set_params = [&](double lo, double hi) {
    if (ASYM) {
      s = (hi > lo) ? (hi - lo) / qmax : 1.0;
      sy = 1.0 / s;
      z = fmin(fmax(rint(div_rn(-lo, s, sy)), 0.0), qmax);
    } else {
      s = fmax(hi, SCALE_FLOOR) / qmax;
      sy = 1.0 / s;
    }
  };
  if (!INPANEL) {
    if (group != 0 && b0 % group == 0) {
      const int glen = min(group, in - b0);
      double hi = ASYM ? -INFINITY : 0.0, lo = INFINITY;
      if (rok)
        for (int col = c; col < glen; col += 16) {
          const double v = Wq[rbase + col];
          hi = ASYM ? fmax(hi, v) : fmax(hi, fabs(v));
          lo = fmin(lo, v);
        }
      hi = max16(hi);
      if (ASYM) lo = min16(lo);
      set_params(lo, hi);
      if (rok && c == 0) {
        scale_row[r] = s;
        scales[(int64_t)r * n_groups + b0 / group] = (float)s;
        if (ASYM) {
          zero_row[r] = z;
          zeros[(int64_t)r * n_groups + b0 / group] = (int32_t)z;
        }
      }
    } else {
      s = rok ? s_row : 1.0;
      sy = 1.0 / s;
      if (ASYM) z = rok ? z_row : 0.0;
    }
  }

  int code_m[8];
  double err_m[8], d_m[8];  // d_m: RF, W0 - Q of the lane's columns
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    code_m[m] = 0;
    err_m[m] = 0.0;
    d_m[m] = 0.0;
  }

  // row j of the U block and 1/U[j][j] are read from LDS one step ahead, so the LDS latency stays off
  // the chain of dependent steps
  double ucur[8], unext[8];
  double dcur = rdiag[0], dnext = 0.0;
#pragma unroll
  for (int m = 0; m < 8; ++m) ucur[m] = Us[c + 16 * m];
  // the 16 steps of column block jm
  auto block_steps = [&](const int jm) __attribute__((always_inline)) {
    // steps past the panel edge (j >= pw) need no guard: there w = 0, U = 0 and 1/U = 0, so they
    // change nothing and their codes are never stored
    static_for<0, 16>([&](auto jlc) {
      constexpr int jl = decltype(jlc)::value;
      const int j = jm * 16 + jl;
      if (j + 1 < PW) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
          if (m >= (j + 1) / 16) unext[m] = Us[urow(j + 1) + c + 16 * (m - (j + 1) / 16)];
        dnext = rdiag[j + 1];
      }
      {
        // a group opens at this step (with GC a constant once the steps are expanded)
        const bool gstart = INPANEL && (GC > 0 ? (j % (GC > 0 ? GC : 1)) == 0 : (j % group) == 0);
        if (gstart) {
          double hi = ASYM ? -INFINITY : 0.0, lo = INFINITY;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int col = c + 16 * m;
            const bool in_g = col >= j && col < j + (GC > 0 ? GC : group) && col < pw;
            hi = in_g ? (ASYM ? fmax(hi, w[m]) : fmax(hi, fabs(w[m]))) : hi;
            lo = in_g ? fmin(lo, w[m]) : lo;
          }
          hi = max16(hi);
          if (ASYM) lo = min16(lo);
          set_params(lo, hi);
          if (rok && c == 0 && j < pw) {
            scales[(int64_t)r * n_groups + (b0 + j) / group] = (float)s;
            if (ASYM) zeros[(int64_t)r * n_groups + (b0 + j) / group] = (int32_t)z;
          }
        }
        const double wj = bcast16<jl>(w[jm]);
        // the code and err = (w - q) / U[j][j] with the rounding steps of the definition (no fused
        // multiply-add): a weight that sits exactly on the grid leaves err = 0
        double cq, qv;
        if (ASYM) {
          cq = fmin(fmax(rint(__dadd_rn(div_rn(wj, s, sy), z)), 0.0), qmax);
          qv = s * (cq - z);
        } else {
          cq = fmin(fmax(rint(div_rn(wj, s, sy)), -qmax), qmax);
          qv = cq * s;
        }
        asm volatile("" : "+v"(qv));  // q is rounded before the subtraction (no contraction into an FMA)
        const double dq = wj - qv;
        const double e = dq * dcur;
        double f = e;  // what the later columns k take off, times U[j][k]
        if constexpr (RF && !INPANEL) f = fma(dq, dcur, -bcast16<jl>(t[jm]));  // e_j - T_j, rounded once
        code_m[jm] = (c == jl) ? (int)cq : code_m[jm];
        err_m[jm] = (c == jl) ? e : err_m[jm];
        if constexpr (RF && INPANEL) {
          // the scale changes at group boundaries inside the panel, so D is formed here (and here, so that q
          // is not kept for all 128 steps); with one scale per row it is formed after the loop
          d_m[jm] = (c == jl) ? w0[jm] - qv : d_m[jm];
          asm volatile("" : "+v"(code_m[jm]), "+v"(err_m[jm]), "+v"(d_m[jm]));
        } else {
          asm volatile("" : "+v"(code_m[jm]), "+v"(err_m[jm]));
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (m >= jm) w[m] = fma(-f, ucur[m], w[m]);
        }
        if (j + 1 < PW) {
#pragma unroll
          for (int m = 0; m < 8; ++m)
            if (m >= (j + 1) / 16) ucur[m] = unext[m];
          dcur = dnext;
        }
      }
    });
  };
  if constexpr (INPANEL && GC == 0) {
#pragma unroll
    for (int jm = 0; jm < 8; ++jm) block_steps(jm);
  } else {
    static_for<0, 8>([&](auto jmc) { block_steps(decltype(jmc)::value); });
  }

  double lsum = 0.0;
  if (rok) {
    int8_t* crow = codes + (int64_t)r * in;
    double* erow = Err + (int64_t)r * ld_err;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int col = c + 16 * m;
      if (col < pw) {
        crow[pidx[col]] = (int8_t)code_m[m];
        if constexpr (RF && !INPANEL) {
          // group 0 (the only one without in-panel groups that the R form takes): the row's one grid gives
          // back the loop's q from the code, rounded as there before the subtraction
          const double cq = (double)code_m[m];
          double qv = ASYM ? s * (cq - z) : cq * s;
          asm volatile("" : "+v"(qv));
          d_m[m] = w0[m] - qv;
        }
        erow[col] = RF ? d_m[m] : err_m[m];
        lsum = fma(err_m[m], err_m[m], lsum);
      }
    }
  }
  if (row_loss) {
    lsum = sum16(lsum);
    if (rok && c == 0) row_loss[r] += lsum;
  }
}

__global__ void k_clear_status(unsigned* p) { *p = 0u; }

__global__ void k_gidx(const int32_t* __restrict__ perm, int in, int group, int32_t* __restrict__ g_idx) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= in) return;
  const int p = min(max(perm[j], 0), in - 1);
  g_idx[p] = group ? j / group : 0;
}

}  // namespace

size_t quantize_ws_bytes(int64_t out, int64_t in, bool rform) {
  size_t b = 0;
  b += align_up((size_t)out * in * sizeof(double), 256);  // working copy
  b += align_up((size_t)out * OB * sizeof(double), 256);  // errors (or, R form, D = W0 - Q) of one outer block
  b += align_up((size_t)out * sizeof(double), 256);       // current fp64 scale per row
  b += align_up((size_t)out * sizeof(double), 256);       // current zero point per row (asymmetric grid)
  b += 256;                                                // status word
  if (rform) b += align_up((size_t)out * in * sizeof(double), 256);  // T, the accumulated D R
  return b;
}

template <bool ASYM>
static hipError_t launch_rowprep(const void* W, int w_dtype, int out, int in, int64_t ld_w, const int32_t* perm,
                                 const uint8_t* dead, double qmax, int group, double* Wq, double* scale_row,
                                 double* zero_row, float* scales, int32_t* zeros, double* row_loss,
                                 unsigned* status, hipStream_t stream) {
  if (w_dtype == GPTQ_BF16)
    hipLaunchKernelGGL((k_rowprep<uint16_t, ASYM>), dim3(out), dim3(256), 0, stream, (const uint16_t*)W, ld_w, in,
                       perm, dead, qmax, group, Wq, scale_row, zero_row, scales, zeros, row_loss, status);
  else
    hipLaunchKernelGGL((k_rowprep<float, ASYM>), dim3(out), dim3(256), 0, stream, (const float*)W, ld_w, in, perm,
                       dead, qmax, group, Wq, scale_row, zero_row, scales, zeros, row_loss, status);
  return hipGetLastError();
}

// A panel workgroup takes 73.5 KB of LDS, so two fit in a CU. Below one workgroup per CU, a launch reserves
// this much more (dynamic LDS, unused) so that the dispatcher gives each workgroup a CU of its own: packed
// two to a CU, 256 workgroups (4096 rows) measured 4 % slower over the whole loop; with more workgroups than
// CUs, two per CU save a round (11008 rows: 7.29 ms against 7.99 at one per CU).
constexpr size_t PANEL_SPREAD_LDS = 8192;
static int cu_count() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n > 0) return n;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  cached.store(n, std::memory_order_relaxed);
  return n;
}

template <bool ASYM, bool RF>
static hipError_t launch_panel(bool inpanel, dim3 grid, double* Wq, int out, int in, int b0, const double* U,
                               const int32_t* perm, double* scale_row, double* zero_row, double qmax, int group,
                               int n_groups, int8_t* codes, float* scales, int32_t* zeros, double* errp,
                               int ld_err, double* row_loss, const double* T, int t_valid, hipStream_t stream) {
  const size_t lds = ((int)grid.x <= cu_count()) ? PANEL_SPREAD_LDS : 0;
  auto go = [&](auto inp, auto gc) {
    k_panel<decltype(inp)::value, ASYM, RF, decltype(gc)::value><<<grid, dim3(256), lds, stream>>>(
        Wq, out, in, b0, U, perm, scale_row, zero_row, qmax, group, n_groups, codes, scales, zeros, errp, ld_err,
        row_loss, T, t_valid);
  };
  using std::integral_constant;
  if (!inpanel) go(integral_constant<bool, false>{}, integral_constant<int, 0>{});
  else if (group == 128) go(integral_constant<bool, true>{}, integral_constant<int, 128>{});
  else if (group == 64) go(integral_constant<bool, true>{}, integral_constant<int, 64>{});
  else if (group == 32) go(integral_constant<bool, true>{}, integral_constant<int, 32>{});
  else go(integral_constant<bool, true>{}, integral_constant<int, 0>{});
  return hipGetLastError();
}

hipError_t quantize_launch(const void* W, int w_dtype, int64_t out64, int64_t in64, int64_t ld_w, const double* U,
                           const int32_t* perm, const uint8_t* dead, int bits, int group, int grid, int8_t* codes,
                           float* scales, int32_t* zeros, int32_t* g_idx, double* row_loss, void* ws,
                           hipStream_t stream, unsigned* host_status, bool rform) {
  const int out = (int)out64, in = (int)in64;
  const bool asym = (grid == GPTQ_GRID_ASYMMETRIC);
  char* w = reinterpret_cast<char*>(ws);
  double* Wq = reinterpret_cast<double*>(w);
  w += align_up((size_t)out * in * sizeof(double), 256);
  double* Err = reinterpret_cast<double*>(w);
  w += align_up((size_t)out * OB * sizeof(double), 256);
  double* scale_row = reinterpret_cast<double*>(w);
  w += align_up((size_t)out * sizeof(double), 256);
  double* zero_row = reinterpret_cast<double*>(w);
  w += align_up((size_t)out * sizeof(double), 256);
  unsigned* status = reinterpret_cast<unsigned*>(w);
  w += 256;
  double* Tacc = rform ? reinterpret_cast<double*>(w) : nullptr;  // R form only (see quantize_ws_bytes)
  // largest code: qmax of the symmetric grid, or the top level 2^b - 1 of the asymmetric one
  const double qmax = asym ? (double)((1 << bits) - 1) : (double)((1 << (bits - 1)) - 1);
  const int n_groups = group ? (int)ceil_div(in, group) : 1;
  // outer blocks must not split a group whose parameters come from columns beyond the current panel:
  // groups that are multiples of the panel width but neither divide nor are multiples of OB fall back
  // to one panel per outer block (every later column updated after every panel)
  const int ob = (group > PW && OB % group != 0 && group % OB != 0) ? PW : OB;

  hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(1), 0, stream, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = asym ? launch_rowprep<true>(W, w_dtype, out, in, ld_w, perm, dead, qmax, group, Wq, scale_row, zero_row,
                                  scales, zeros, row_loss, status, stream)
           : launch_rowprep<false>(W, w_dtype, out, in, ld_w, perm, dead, qmax, group, Wq, scale_row, zero_row,
                                   scales, zeros, row_loss, status, stream);
  if (e != hipSuccess) return e;

  // R form: the products accumulate T += D R (alpha +1) instead of W -= E U; T is written before it is read
  // (beta 0 for the first panel's update inside the first outer block and for the first block update, the
  // first products to reach each column; the first panel has no T)
  const double alpha = rform ? 1.0 : -1.0;
  double* Cw = rform ? Tacc : Wq;
  const dim3 pgrid((unsigned)ceil_div(out, 16));
  for (int ob0 = 0; ob0 < in; ob0 += ob) {
    const int ob1 = min(in, ob0 + ob);
    for (int b0 = ob0; b0 < ob1; b0 += PW) {
      double* errp = Err + (b0 - ob0);  // this panel's columns of the outer block's error matrix
      const bool inpanel = group != 0 && PW % group == 0;
      const int t_valid = b0 > 0 ? 1 : 0;
      if (rform)
        e = asym ? launch_panel<true, true>(inpanel, pgrid, Wq, out, in, b0, U, perm, scale_row, zero_row, qmax,
                                            group, n_groups, codes, scales, zeros, errp, OB, row_loss, Tacc,
                                            t_valid, stream)
                 : launch_panel<false, true>(inpanel, pgrid, Wq, out, in, b0, U, perm, scale_row, zero_row, qmax,
                                             group, n_groups, codes, scales, zeros, errp, OB, row_loss, Tacc,
                                             t_valid, stream);
      else
        e = asym ? launch_panel<true, false>(inpanel, pgrid, Wq, out, in, b0, U, perm, scale_row, zero_row, qmax,
                                             group, n_groups, codes, scales, zeros, errp, OB, row_loss, nullptr, 0,
                                             stream)
                 : launch_panel<false, false>(inpanel, pgrid, Wq, out, in, b0, U, perm, scale_row, zero_row, qmax,
                                              group, n_groups, codes, scales, zeros, errp, OB, row_loss, nullptr,
                                              0, stream);
      if (e != hipSuccess) return e;
      const int b1 = b0 + PW;
      if (b1 < ob1) {  // the rest of the outer block: W[:, b1:ob1] -= Err[:, panel] U[b0:b1, b1:ob1]
        DgemmArgs t{};
        t.A = errp; t.lda = OB;
        t.B = U + (int64_t)b0 * in + b1; t.ldb = in;
        t.C = Cw + b1; t.ldc = in;
        t.M = out; t.N = ob1 - b1; t.K = PW;
        t.alpha = alpha; t.beta = (rform && b0 == 0) ? 0.0 : 1.0;
        t.kmode = KMODE_FULL;
        e = dgemm_launch(t, false, false, 1, stream);
        if (e != hipSuccess) return e;
      }
    }
    if (ob1 < in) {  // every later column: W[:, ob1:] -= Err[:, block] U[ob0:ob1, ob1:]
      DgemmArgs t{};
      t.A = Err; t.lda = OB;
      t.B = U + (int64_t)ob0 * in + ob1; t.ldb = in;
      t.C = Cw + ob1; t.ldc = in;
      t.M = out; t.N = in - ob1; t.K = ob1 - ob0;
      t.alpha = alpha; t.beta = (rform && ob0 == 0) ? 0.0 : 1.0;
      t.kmode = KMODE_FULL;
      e = dgemm_launch(t, false, false, 1, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (g_idx) {
    hipLaunchKernelGGL(k_gidx, dim3((unsigned)ceil_div(in, 256)), dim3(256), 0, stream, perm, in, group, g_idx);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the row-prep pass flagged non-finite live weights: one read of the status word at the end
  e = hipMemcpyAsync(host_status, status, sizeof(unsigned), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(stream);
}

}  // namespace gptq
