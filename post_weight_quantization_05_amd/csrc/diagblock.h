// Factorization of one 64 x 64 diagonal block (fp64, gfx950): its Cholesky factor and the inverse of
// the factor. Used by the block-column step of the blocked factorization (k_colstep), where the
// workgroups of the next panel each factor the block from the same inputs.
//
// GPTQ guide ("GPTQ", herodthegreater.github.io/pigeon/guide/gptq/), "GPTQ's two tricks", trick 2: U is
// a Cholesky factor; these blocks are the diagonal steps of the blocked factorization that yields it.
#pragma once
#include <type_traits>

#include "common.h"

namespace gptq {
namespace diagblock {

constexpr int NB = 64;

// compile-time loop (the 64-step elimination loops are too large for the unroller, and a runtime index
// into the register-resident row would move it to scratch memory)
template <int K, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for<K + 1, N>(f);
  }
}

__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(x & 0xFFFFFFFFll), l);
  const int hi = __builtin_amdgcn_readlane((int)(x >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
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

// v from lane 4q + R of each quad of lanes (DPP quad_perm [R, R, R, R]), both halves of the double
template <int R>
__device__ __forceinline__ double quad_bcast(double v) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(x & 0xFFFFFFFFll), R * 0x55, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(x >> 32), R * 0x55, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Factorization of one diagonal block staged in LDS (lower part; rows/columns past the matrix edge as
// the identity): its Cholesky factor L and L^-1. 256 threads. Outputs are optional: L to global memory,
// L^-1 to global memory, the status bits; or, instead of L^-1, the solution X of X L^T = T for a 64-row
// tile T staged in LDS.
//  Cholesky (wave 0): lane i holds row i in registers and eliminates right-looking. Pivot k is
//  r_k[k]; 1/L[k][k] comes from rsqrt_refined, so no square root or division sits on the chain. After
//  scaling column k, every lane updates its entries j > k with column k, which goes through LDS. The
//  next pivot r_{k+1}[k+1] - L[k+1][k]^2 uses lane k+1's own registers only, so its square-root
//  estimate overlaps the LDS round trip of the column.
//  Inverse (all 4 waves): a quad of lanes owns column j of L^-1 (lane 4j + r holds rows i = r mod 4) and
//  eliminates right-looking; the finished entry (L^-1)[k][j] reaches the other lanes of its quad by
//  DPP. Column k of L is kept in LDS as Lc[k][r][m] = L[4m + r][k], with the four r-rows 144 bytes apart
//  so a quad's four reads hit distinct banks.
// Rows/columns past the matrix edge act as the identity. Pivots below 2^-1000 or not finite set the
// status bits (and are treated as 1 from there on).
constexpr int LC_STRIDE = 18;  // doubles per (k, r) row of Lc

struct DiagSmem {
  double Ls[NB][NB + 1];                                // the block, later L (row-major)
  __attribute__((aligned(16))) double Lc[NB][4][LC_STRIDE];  // Lc[k][r][m] = L[4m + r][k]
  double col[NB];                                       // column k during the elimination
  double rdg[NB];                                       // 1 / L[k][k]
};

// Factor the block in sm.Ls (staged by the caller, followed by a barrier). m is the block's size.
//   Lout (nullable): L written to Lout[i * ldo + j] for i, j < m, zeros above the diagonal;
//   Dout (nullable): L^-1 as a row-major 64 x 64 block, the identity past the edge;
//   status (nullable): flags of bad pivots;
//   rhs (nullable, LDS, 64 rows of stride NB + 1): instead of L^-1, the substitution solves
//   X L^T = rhs (each row x of X from L x^T = row^T), and row i < xrows, column j < m of X goes to
//   Xout[i * ldx + j]. Dout must then be null.
__device__ __forceinline__ void diag_factor(DiagSmem& sm, int m, double* __restrict__ Lout, int64_t ldo,
                                            double* __restrict__ Dout, unsigned* status,
                                            const double* rhs = nullptr, double* Xout = nullptr, int64_t ldx = 0,
                                            int xrows = 0) {
  auto& Ls = sm.Ls;
  auto& Lc = sm.Lc;
  auto& col = sm.col;
  auto& rdg = sm.rdg;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int i = tid;
    unsigned flags = 0;
    double r[NB];
    int ir = i;
    asm volatile("" : "+v"(ir));
#pragma unroll
    for (int j = 0; j < NB; ++j) r[j] = Ls[ir][j];
    // A pivot that is not finite, or below 2^-1000 (not > 0 in particular), is flagged and its 1/sqrt
    // replaced by 1, so a matrix that is not positive definite leaves finite values behind; the caller
    // reports the status. The test runs beside the pivot chain and only the final select joins it.
    auto inv_sqrt = [&](double p) {
      const bool ok = (p >= 0x1p-1000) && (p < INFINITY);
      flags |= ok ? 0u : (isfinite(p) ? DEV_STATUS_NOT_SPD : DEV_STATUS_NONFINITE);
      const double yr = rsqrt_refined(p);
      return ok ? yr : 1.0;
    };
    double piv = readlane_d(r[0], 0);
    double y = inv_sqrt(piv);
    double ydiag = 0.0;
    static_for<0, NB>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      r[k] = r[k] * y;  // lane k: piv y = L[k][k]; lanes below: L[i][k]
      ydiag = (i == k) ? y : ydiag;
      if constexpr (k + 1 < NB) {
        // next pivot from lane k+1's own entries: r[k+1] - L[k+1][k]^2 (no LDS on this path)
        const double pn = readlane_d(fma(-r[k], r[k], r[k + 1]), k + 1);
        col[i] = r[k];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int F = ((k + 1) & ~7), NC = (NB - F) / 8;  // chunks of 8 holding the entries > k
        double buf[4][8];
        auto rd = [&](auto cc) {
          constexpr int c = decltype(cc)::value;
#pragma unroll
          for (int q = 0; q < 8; ++q) buf[c & 3][q] = col[F + 8 * c + q];
        };
        static_for<0, (NC < 3 ? NC : 3)>(rd);
        __builtin_amdgcn_sched_barrier(0);
        // the next pivot's 1/sqrt runs while the column reads are in flight
        const double yn = inv_sqrt(pn);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, NC>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if constexpr (c + 3 < NC) rd(std::integral_constant<int, c + 3>{});
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (F + 8 * c + q > k) r[F + 8 * c + q] = fma(-r[k], buf[c & 3][q], r[F + 8 * c + q]);
          }
        });
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = k + 1; j < NB; ++j) asm volatile("" : "+v"(r[j]));
        piv = pn;
        y = yn;
      }
    });
    rdg[i] = ydiag;
    // a fresh copy of the row index, so the compiler forms these addresses here instead of keeping the
    // load addresses of the same rows alive through the elimination
    int iw = i;
    asm volatile("" : "+v"(iw));
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      Ls[iw][j] = (j <= iw) ? r[j] : 0.0;
      Lc[j][iw & 3][iw >> 2] = (j < iw) ? r[j] : 0.0;
    }
    if (status && flags && i == 0) atomicOr(status, flags);
  }
  __syncthreads();
  // a fresh copy of the thread index for the later phases (keeps the first phase's addresses from
  // staying alive, and spilling, across the elimination)
  int tw = tid;
  asm volatile("" : "+v"(tw));
  if (Lout) {
    double v[NB * NB / 256];
#pragma unroll
    for (int t = 0; t < NB * NB / 256; ++t) {
      const int e = tw + 256 * t;
      v[t] = Ls[e / NB][e % NB];
    }
#pragma unroll
    for (int t = 0; t < NB * NB / 256; ++t) {
      const int e = tw + 256 * t, i = e / NB, j = e % NB;
      if (i < m && j < m) Lout[(int64_t)i * ldo + j] = v[t];
    }
  }
  // inverse: lane 4j + r holds c[q] = (L^-1)[4q + r][j], starting from e_j (or, with rhs, the solution
  // of L x = (row j of rhs)^T, starting from that row)
  const int jc = tw >> 2, rr = tw & 3;
  double c[16];
  if (rhs) {
#pragma unroll
    for (int q = 0; q < 16; ++q) c[q] = rhs[jc * (NB + 1) + 4 * q + rr];
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) c[q] = (4 * q + rr == jc) ? 1.0 : 0.0;
  }
  // column k of L and 1/L[k][k] are read one step ahead, so their LDS latency is off the chain. Every
  // read goes through one per-lane base (Lc[0][rr]) with a constant offset.
  const double* lb = &Lc[0][rr][0];
  double lcur[16], lnext[16];
  double dcur = rdg[0], dnext = 0.0;
#pragma unroll
  for (int q = 0; q < 16; ++q) lcur[q] = lb[q];
  static_for<0, NB>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int mk = k >> 2, rk = k & 3;
    if constexpr (k + 1 < NB) {
#pragma unroll
      for (int q = (k + 1) >> 2; q < 16; ++q) lnext[q] = lb[(k + 1) * 4 * LC_STRIDE + q];
      dnext = rdg[k + 1];
    }
    const double own = c[mk] * dcur;
    c[mk] = (rr == rk) ? own : c[mk];
    if constexpr (k + 1 < NB) {
      const double b = quad_bcast<rk>(c[mk]);  // (L^-1)[k][j]
#pragma unroll
      for (int q = mk; q < 16; ++q) {
        const double t = fma(-lcur[q], b, c[q]);
        c[q] = (q > mk || rr > rk) ? t : c[q];
      }
#pragma unroll
      for (int q = (k + 1) >> 2; q < 16; ++q) lcur[q] = lnext[q];
      dcur = dnext;
    }
  });
  if (Dout) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 4 * q + rr;
      Dout[row * NB + jc] = (row < m && jc < m) ? c[q] : ((row == jc) ? 1.0 : 0.0);
    }
  }
  if (rhs && jc < xrows) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int col = 4 * q + rr;
      if (col < m) Xout[(int64_t)jc * ldx + col] = c[q];
    }
  }
}

}  // namespace diagblock
}  // namespace gptq
