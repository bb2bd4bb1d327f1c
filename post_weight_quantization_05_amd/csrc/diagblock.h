// Factorization of one 64 x 64 diagonal block (fp64, gfx950): its Cholesky factor and the inverse of
// the factor. Used by the block-column step of the blocked factorization (k_colstep), where the
// workgroups of the panel each factor the block from the same inputs.
//
// GPTQ guide ("GPTQ", herodthegreater.github.io/pigeon/guide/gptq/), "GPTQ's two tricks", trick 2: U is
// a Cholesky factor; these blocks are the diagonal steps of the blocked factorization that yields it.
#pragma once
#include <type_traits>

#include "common.h"

namespace gptq {
namespace diagblock {

constexpr int NB = 64;

// compile-time loop (a runtime index into a register-resident row would move it to scratch memory)
template <int K, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for<K + 1, N>(f);
  }
}

// 1/sqrt(a) for finite a >= 2^-1000, to about 1 ulp without an IEEE square root or division: the
// hardware estimate (about 2^-24 relative) refined by one third-order Newton step, y (1 + e/2 + 3e^2/8)
// with e = 1 - a y^2 (truncation error about e^3, below 2^-70). Smaller pivots are flagged by the caller.
__device__ __forceinline__ double rsqrt_refined(double a) {
  const double y = __builtin_amdgcn_rsq(a);
  const double e = fma(-(a * y), y, 1.0);
  const double p = fma(e, 0.375, 0.5);
  return fma(y * e, p, y);
}

// ------------------------------------------------------------------------------------------------------
// Blocked factorization of one 64 x 64 diagonal block, L and L^-1 both (256 threads, 4 waves).
//
// The block goes through four 16-column sub-blocks b. Each wave factors the 16 x 16 diagonal sub-block
// in registers (all four DPP rows of every wave redundantly, so no barrier sits between the waves): lane
// i of a row of 16 lanes holds row i; pivot k is broadcast from lane k (DPP row_newbcast), its 1/sqrt
// comes from rsqrt_refined, and L's column k reaches the lanes that update with it by further row
// broadcasts (one v_mov_b64_dpp each; fp64 matrix cores run no faster than the vector unit on this
// part, so the 16 x 16 steps gain nothing from them). The inverse of the sub-block's factor follows by
// forward substitution on its unit-diagonal form, each DPP row g solving columns g, g + 4, g + 8,
// g + 12: lane (i, g) then holds exactly the v_mfma_f64_16x16x4f64 operand fragments of that inverse
// (A[i][4t + g] or B[4t + g][i] in k-step t). With it the panel below is solved on the matrix cores
// (P = A_panel L_bb^-T, one 16-row tile per wave) and the trailing lower tiles are updated (A -= P P^T).
// Last, the blocks of L^-1 below the diagonal, M_ij = -M_ii sum_k L_ik M_kj, in three dependent levels
// of 16 x 16 products. Rows/columns past the matrix edge are staged as the identity and stay the
// identity in L and L^-1. About 28k cycles per block (the one-wave elimination it replaces: 49k).
// ------------------------------------------------------------------------------------------------------
constexpr int BS = 65;  // LDS row stride (doubles)

struct BlockSmem {
  double A[NB][BS];  // the block (lower part, zeros above), then L
  double M[NB][BS];  // L^-1 (lower part, zeros above)
};

template <int K>
__device__ __forceinline__ double row_bcast(double v) {  // value of lane K of this lane's row of 16
  return __builtin_amdgcn_mov_dpp(v, 0x150 + K, 0xF, 0xF, false);  // one v_mov_b64_dpp (row_newbcast)
}

__device__ __forceinline__ f64x4 mfma16(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// Factor sm.A (staged by the caller, followed by a barrier) into L (in sm.A) and L^-1 (in sm.M). Returns
// the bad-pivot flags (the same in every lane). Ends with a barrier.
__device__ __forceinline__ unsigned factor_invert_blocked(BlockSmem& sm) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  // L^-1 starts as zeros (its diagonal and lower blocks are written below)
  for (int e = tid; e < NB * BS; e += 256) (&sm.M[0][0])[e] = 0.0;
  double xb[4][4];  // xb[b][t] = (L_bb^-1)[i][4t + g]
  static_for<0, 4>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    constexpr int o = 16 * b;
    // ---- the 16 x 16 diagonal sub-block: factor and inverse, in registers ----
    // Pivot k comes from lane k; a pivot that is not finite or below 2^-1000 takes 1/sqrt = 1, so the
    // values stay finite, and it shows on L's diagonal (checked at the end).
    double r[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) r[k] = sm.A[o + i][o + k];
    double yown = 1.0;  // 1 / L[i][i]
    double lh[16];      // lh[k] = L[i][k] / L[k][k] below the diagonal, 0 on and above it
    static_for<0, 16>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const double piv = row_bcast<k>(r[k]);
      const bool ok = (piv >= 0x1p-1000) && (piv < INFINITY);
      const double y = ok ? rsqrt_refined(piv) : 1.0;  // a select (nothing to skip in a branch)
      const double l = r[k] * y;  // lane k: L[k][k]; lanes below: L[i][k]; lanes above: unused
      r[k] = l;
      yown = (i == k) ? y : yown;
      lh[k] = (i > k) ? l * y : 0.0;
      static_for<k + 1, 16>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        r[j] = fma(-l, row_bcast<j>(l), r[j]);
      });
    });
    // L^-1 = D^-1 Lh^-1 with Lh = L D^-1 unit lower (D = diag L): forward substitution on the unit factor
    // (no division, no select), then row i scaled by 1 / L[i][i]. Lane (i, g) holds columns g + 4t.
    double x[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) x[t] = (i == g + 4 * t) ? 1.0 : 0.0;
    static_for<0, 15>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = fma(-lh[k], row_bcast<k>(x[t]), x[t]);
    });
#pragma unroll
    for (int t = 0; t < 4; ++t) x[t] *= yown;
#pragma unroll
    for (int t = 0; t < 4; ++t) xb[b][t] = x[t];
    if constexpr (b < 3) {
      // ---- panel below: P = A[p0:p0+16][o:o+16] L_bb^-T, one tile per wave, in place ----
      if (w < 3 - b) {
        const int p0 = 16 * (b + 1 + w);
        double a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = sm.A[p0 + i][o + 4 * t + g];
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = mfma16(a[t], x[t], acc);
#pragma unroll
        for (int q = 0; q < 4; ++q) sm.A[p0 + 4 * q + g][o + i] = acc[q];
      }
    }
    // every wave has read the diagonal sub-block (and its panel tile) before L_bb replaces it
    __syncthreads();
    if (w == 0) {
      if (g == 0) {
#pragma unroll
        for (int k = 0; k < 16; ++k) sm.A[o + i][o + k] = (k <= i) ? r[k] : 0.0;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) sm.M[o + i][o + 4 * t + g] = x[t];
    }
    if constexpr (b < 3) {
      // ---- trailing lower tiles: A[I][J] -= P_I P_J^T for b < J <= I < 4 (rows and columns past o + 16,
      // apart from the sub-block L_bb and L^-1 that wave 0 writes meanwhile) ----
      constexpr int NT = (3 - b) * (4 - b) / 2;
      for (int tt = w; tt < NT; tt += 4) {
        int I = b + 1, J = b + 1, c = tt;
        while (c >= I - b) {  // tiles in order (b+1,b+1), (b+2,b+1), (b+2,b+2), ...
          c -= I - b;
          ++I;
        }
        J = b + 1 + c;
        double a[4], bb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          a[t] = sm.A[16 * I + i][o + 4 * t + g];
          bb[t] = sm.A[16 * J + i][o + 4 * t + g];
        }
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = mfma16(a[t], bb[t], acc);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 4 * q + g;
          if (I != J || row >= i) sm.A[16 * I + row][16 * J + i] -= acc[q];
        }
      }
    }
    __syncthreads();
  });
  // ---- blocks of L^-1 below the diagonal, level by level: M_ij = -M_ii sum_{k=j}^{i-1} L_ik M_kj ----
  static_for<1, 4>([&](auto ic) {
    constexpr int bi = decltype(ic)::value;
    if (w < bi) {
      const int bj = w;
      f64x4 T = {0.0, 0.0, 0.0, 0.0};
      for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          T = mfma16(sm.A[16 * bi + i][16 * bk + 4 * t + g], sm.M[16 * bk + 4 * t + g][16 * bj + i], T);
      }
      f64x4 R = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int t = 0; t < 4; ++t) R = mfma16(xb[bi][t], T[t], R);  // T's acc layout is the B operand of k-step t
#pragma unroll
      for (int q = 0; q < 4; ++q) sm.M[16 * bi + 4 * q + g][16 * bj + i] = -R[q];
    }
    __syncthreads();
  });
  // bad pivots, read off L's diagonal: a good pivot p >= 2^-1000 leaves L[k][k] = sqrt(p) > 2^-501 (and
  // finite); a bad one leaves p itself (1/sqrt taken as 1): below 2^-1000, infinite or NaN
  const double dg = sm.A[lane][lane];
  const bool good = (dg > 0x1p-501) && (dg < INFINITY);
  const unsigned long long nonfinite = __ballot(!good && !isfinite(dg));
  const unsigned long long small = __ballot(!good && isfinite(dg));
  return (nonfinite ? DEV_STATUS_NONFINITE : 0u) | (small ? DEV_STATUS_NOT_SPD : 0u);
}

}  // namespace diagblock
}  // namespace gptq
