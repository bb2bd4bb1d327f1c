// fp64 tiled GEMM on gfx950 matrix cores (v_mfma_f64_4x4x4_f64, four 4x4x4 blocks per instruction), the
// shared core of the blocked factorization (trailing SYRK updates, triangular-inverse levels) and of the
// quantize loop's trailing update W[:, b1:] -= Err U[b0:b1, b1:].
//
//   C[i][j] = alpha * sum_{k in K-range(tile)} opA(A)[i][k] opB(B)[k][j] + beta * C[i][j]
//   opA(A)[i][k] = TA ? A[k][i] : A[i][k],  opB(B)[k][j] = TB ? B[j][k] : B[k][j]  (row-major storage)
//
// Tiles are T x T (T = 64: 256 threads, 4 waves of 32 x 32); K runs in chunks of 16 through
// double-buffered LDS. Options: only lower-triangle tiles (I >= J) of a square C; per-tile K-range
// restrictions for triangular operands (their zero triangle is then never multiplied); and a batch index
// (blockIdx.y) with per-operand strides and a per-batch row limit.
#include "common.h"
#include "dgemm.h"

namespace gptq {

namespace {

#ifndef GPTQ_DGEMM_TK
#define GPTQ_DGEMM_TK 16
#endif
constexpr int TK = GPTQ_DGEMM_TK;  // K per LDS chunk

// LDS layouts. An operand whose rows run along the tile's M (or N) dimension in memory (A^T, B) is kept
// as [k][i] with rows padded to T + 16 doubles: the 16 consecutive i that a 16-lane group reads sit on
// one half of the banks, the next k row on the other half. An operand whose rows run along k (A, B^T)
// is kept as [i][k] with rows of 18 doubles: 16 lanes reading 16 rows at one k hit 16 distinct bank
// pairs (9 i mod 16 is a permutation), and the next k shifts them by one pair. Both are filled with
// 16-byte stores of two consecutive doubles.
template <int T>
struct Lds {
  static constexpr int KI = T + 16;  // [k][i] row stride
  static constexpr int IK = TK + 2;  // [i][k] row stride (= 2 mod 32)
  static constexpr int SZ = (TK * KI > T * IK) ? TK * KI : T * IK;
};

// T x T tile, 4 waves in 2 x 2, each (T/2) x (T/2). Operand chunks of
// T x 16 are fetched as 16-byte vectors into registers while the MFMAs of the previous chunk run, then
// stored to the other LDS buffer.
template <bool TA, bool TB, int T>
__global__ __launch_bounds__(256) void k_dgemm(DgemmArgs a) {
  constexpr int NV = T * TK / 2 / 256;   // 16-byte loads per thread per operand and chunk
  using L = Lds<T>;
  __shared__ __attribute__((aligned(16))) double As[2][L::SZ];
  __shared__ __attribute__((aligned(16))) double Bs[2][L::SZ];

  const int batch = blockIdx.y;
  int I, J;
  if (a.tri_tiles) {
    const int t = blockIdx.x;
    int I0 = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while ((I0 + 1) * (I0 + 2) / 2 <= t) ++I0;
    while (I0 * (I0 + 1) / 2 > t) --I0;
    I = I0;
    J = t - I0 * (I0 + 1) / 2;
  } else {
    const int ntn = (a.N + T - 1) / T;
    I = blockIdx.x / ntn;
    J = blockIdx.x - I * ntn;
    // Triangular K-ranges make a tile's work depend on J (KMODE_GE_J) or on I (the other modes). The
    // workgroups that share a CU are about 256 apart in dispatch order (8 XCDs x 32 CUs), so in every
    // other run of 256 workgroups the K-determining coordinate is mirrored: long and short tiles then
    // share CUs instead of piling up on the same ones. Both maps are permutations of the tile set.
    if (a.kmode == KMODE_GE_J) {
      const int64_t first = (int64_t)blockIdx.y * gridDim.x + (int64_t)I * ntn;  // this row's first tile
      if ((first / 256) & 1) J = ntn - 1 - J;
    } else if (a.kmode != KMODE_FULL) {
      const int nti = (int)(gridDim.x / ntn);
      const int R = max(1, 256 / ntn);  // tile rows per run of 256 workgroups
      const int G = (nti + R - 1) / R;
      const int g = I / R;
      if ((((int)blockIdx.y * G + g) & 1) && (g + 1) * R <= nti) I = g * R + (R - 1 - (I - g * R));
    }
  }
  const int M = (a.m_step != 0) ? min(a.M, a.m_lim - batch * a.m_step) : a.M;
  const int N = a.N;
  const int K = a.k_by_m ? M : a.K;
  const int i0 = I * T, j0 = J * T;
  if (i0 >= M || j0 >= N) return;

  // no __restrict__: the factorization's panel solve reads and writes the same block (each workgroup
  // reads all of its rows before it writes them)
  const double* A = a.A + (int64_t)batch * a.strideA;
  const double* B = a.B + (int64_t)batch * a.strideB;
  double* C = a.C + (int64_t)batch * a.strideC;

  int klo = 0, khi = K;
  if (a.kmode == KMODE_GE_J) klo = j0;                        // B lower triangular: B[k][j] = 0 for k < j
  else if (a.kmode == KMODE_LT_I_END) khi = min(K, i0 + T);   // A lower triangular: A[i][k] = 0 for k > i
  else if (a.kmode == KMODE_GE_I) klo = i0;                   // A^T with A lower: A[k][i] = 0 for k < i
  klo = (klo / TK) * TK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // vector loads need 16-byte aligned pairs; otherwise two scalar loads
  const bool a_vec = ((a.lda & 1) == 0) && ((reinterpret_cast<uintptr_t>(A) & 15) == 0);
  const bool b_vec = ((a.ldb & 1) == 0) && ((reinterpret_cast<uintptr_t>(B) & 15) == 0);

  // element pair (r, c2..c2+1) of a row-major source, zero outside [0, rlim) x [clo, clim)
  auto ld2 = [](const double* P, int64_t ld, int r, int c2, int rlim, int clo, int clim, bool vec) {
    double2 v = make_double2(0.0, 0.0);
    if (r < rlim) {
      const double* q = P + (int64_t)r * ld + c2;
      if (vec && c2 >= clo && c2 + 1 < clim) {
        v = *reinterpret_cast<const double2*>(q);
      } else {
        if (c2 >= clo && c2 < clim) v.x = q[0];
        if (c2 + 1 >= clo && c2 + 1 < clim) v.y = q[1];
      }
    }
    return v;
  };
  // thread element e of a chunk: along-k operands (A, B^T) as rows x 8 pairs, along-tile operands as
  // 16 k-rows x T/2 pairs; both map 8 (resp. T/2) consecutive threads onto one contiguous row segment
  double2 ra[NV], rb[NV];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int e = tid + 256 * q;
      if (!TA) {
        const int ii = e / (TK / 2), kk = (e % (TK / 2)) * 2;
        ra[q] = ld2(A, a.lda, i0 + ii, k0 + kk, M, klo, khi, a_vec);
      } else {
        const int kk = e / (T / 2), ii = (e % (T / 2)) * 2;
        ra[q] = (k0 + kk < khi) ? ld2(A, a.lda, k0 + kk, i0 + ii, K, 0, M, a_vec) : make_double2(0.0, 0.0);
      }
      if (!TB) {
        const int kk = e / (T / 2), jj = (e % (T / 2)) * 2;
        rb[q] = (k0 + kk < khi) ? ld2(B, a.ldb, k0 + kk, j0 + jj, K, 0, N, b_vec) : make_double2(0.0, 0.0);
      } else {
        const int jj = e / (TK / 2), kk = (e % (TK / 2)) * 2;
        rb[q] = ld2(B, a.ldb, j0 + jj, k0 + kk, N, klo, khi, b_vec);
      }
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int e = tid + 256 * q;
      if (!TA) *reinterpret_cast<double2*>(&As[st][(e / (TK / 2)) * L::IK + (e % (TK / 2)) * 2]) = ra[q];
      else *reinterpret_cast<double2*>(&As[st][(e / (T / 2)) * L::KI + (e % (T / 2)) * 2]) = ra[q];
      if (!TB) *reinterpret_cast<double2*>(&Bs[st][(e / (T / 2)) * L::KI + (e % (T / 2)) * 2]) = rb[q];
      else *reinterpret_cast<double2*>(&Bs[st][(e / (TK / 2)) * L::IK + (e % (TK / 2)) * 2]) = rb[q];
    }
  };

  // v_mfma_f64_4x4x4f64 runs four independent 4 x 4 x 4 products per instruction at the fp64 rate.
  // Block b of an instruction takes A[i][k] from lane
  // 16 k + 4 b + i, B[k][j] from lane 16 k + 4 b + j and leaves D[i][j] in lane 16 i + 4 b + j. Giving
  // all four blocks the same 4 rows of A and consecutive 4-column groups of B makes one instruction a
  // 4 x 16 tile of C: lane l supplies A[r0 + l % 4][k0 + l / 16] and B[k0 + l / 16][c0 + l % 16] and
  // holds C[r0 + l / 16][c0 + l % 16]. A wave's (T/2) x (T/2) block is PR x PC such tiles.
  constexpr int PR = T / 8;   // 4-row groups per wave
  constexpr int PC = T / 32;  // 16-column groups per wave
  double acc[PR][PC];
#pragma unroll
  for (int p = 0; p < PR; ++p)
#pragma unroll
    for (int q = 0; q < PC; ++q) acc[p][q] = 0.0;

  const int nk = (khi > klo) ? (khi - klo + TK - 1) / TK : 0;
  if (nk > 0) {
    gload(klo);
    lstore(0);
  }
  __syncthreads();
  const int lr = lane & 3, lk = lane >> 4, lc = lane & 15;
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(klo + (kt + 1) * TK);
#pragma unroll
    for (int k4 = 0; k4 < TK; k4 += 4) {
      const int kr = k4 + lk;
      double fa[PR], fb[PC];
#pragma unroll
      for (int p = 0; p < PR; ++p) {
        const int i = wm * (T / 2) + p * 4 + lr;
        fa[p] = TA ? As[st][kr * L::KI + i] : As[st][i * L::IK + kr];
      }
#pragma unroll
      for (int q = 0; q < PC; ++q) {
        const int j = wn * (T / 2) + q * 16 + lc;
        fb[q] = TB ? Bs[st][j * L::IK + kr] : Bs[st][kr * L::KI + j];
      }
#pragma unroll
      for (int p = 0; p < PR; ++p)
#pragma unroll
        for (int q = 0; q < PC; ++q) acc[p][q] = __builtin_amdgcn_mfma_f64_4x4x4f64(fa[p], fb[q], acc[p][q], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int p = 0; p < PR; ++p)
#pragma unroll
    for (int q = 0; q < PC; ++q) {
      const int gi = i0 + wm * (T / 2) + p * 4 + lk;
      const int gj = j0 + wn * (T / 2) + q * 16 + lc;
      if (gi < M && gj < N) {
        double* ptr = C + (int64_t)gi * a.ldc + gj;
        const double v = a.alpha * acc[p][q];
        *ptr = (a.beta == 0.0) ? v : fma(a.beta, *ptr, v);
      }
    }
}

}  // namespace

template <int T>
static hipError_t dgemm_launch_t(const DgemmArgs& a, bool ta, bool tb, int batches, hipStream_t stream) {
  int tiles;
  if (a.tri_tiles) {
    const int nt = (a.M + T - 1) / T;
    tiles = nt * (nt + 1) / 2;
  } else {
    tiles = ((a.M + T - 1) / T) * ((a.N + T - 1) / T);
  }
  dim3 grid(tiles, batches);
  if (!ta && !tb) k_dgemm<false, false, T><<<grid, dim3(256), 0, stream>>>(a);
  else if (!ta && tb) k_dgemm<false, true, T><<<grid, dim3(256), 0, stream>>>(a);
  else if (ta && !tb) k_dgemm<true, false, T><<<grid, dim3(256), 0, stream>>>(a);
  else k_dgemm<true, true, T><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t dgemm_launch(const DgemmArgs& a, bool ta, bool tb, int batches, hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0 || batches <= 0) return hipSuccess;
  // 64 x 64 tiles only: the triangular K-ranges rely on zeros above the diagonal inside the
  // factorization's 64 x 64 diagonal blocks, which is exactly one tile
  return dgemm_launch_t<64>(a, ta, tb, batches, stream);
}

}  // namespace gptq
