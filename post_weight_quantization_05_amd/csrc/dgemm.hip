// fp64 tiled GEMM on gfx950 matrix cores (v_mfma_f64_16x16x4_f64), the shared core of the blocked
// factorization (trailing SYRK updates, triangular-inverse levels, H^-1 = L^-T L^-1) and of the
// quantize loop's trailing update W[:, b1:] -= Err U[b0:b1, b1:].
//
//   C[i][j] = alpha * sum_{k in K-range(tile)} opA(A)[i][k] opB(B)[k][j] + beta * C[i][j]
//   opA(A)[i][k] = TA ? A[k][i] : A[i][k],  opB(B)[k][j] = TB ? B[j][k] : B[k][j]  (row-major storage)
//
// Tiles are 64 x 64 (256 threads, 4 waves of 32 x 32, 2 x 2 MFMA blocks each); K runs in chunks of 16
// through double-buffered LDS. Options: only lower-triangle tiles (I >= J) of a square C; per-tile
// K-range restrictions for triangular operands (their zero triangle is then never multiplied); and a
// batch index (blockIdx.y) with per-operand strides and a per-batch row limit.
// fp64 MFMA on MI355X runs at the fp64 vector rate; using it keeps operand traffic low (one operand per
// lane per 16x16x4 step instead of a register micro-tile).
#include "common.h"
#include "dgemm.h"

namespace gptq {

namespace {

constexpr int TM = 64, TN = 64, TK = 16;
constexpr int LPAD = 4;

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void k_dgemm(DgemmArgs a) {
  __shared__ double As[2][TK][TM + LPAD];
  __shared__ double Bs[2][TK][TN + LPAD];

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
    const int ntn = (a.N + TN - 1) / TN;
    I = blockIdx.x / ntn;
    J = blockIdx.x - I * ntn;
  }
  const int M = (a.m_step != 0) ? min(a.M, a.m_lim - batch * a.m_step) : a.M;
  const int N = a.N;
  const int K = a.k_by_m ? M : a.K;
  const int i0 = I * TM, j0 = J * TN;
  if (i0 >= M || j0 >= N) return;

  // no __restrict__: the factorization's panel solve reads and writes the same block (each workgroup
  // reads all of its rows before it writes them)
  const double* A = a.A + (int64_t)batch * a.strideA;
  const double* B = a.B + (int64_t)batch * a.strideB;
  double* C = a.C + (int64_t)batch * a.strideC;

  int klo = 0, khi = K;
  if (a.kmode == KMODE_GE_J) klo = j0;                 // B lower triangular: B[k][j] = 0 for k < j
  else if (a.kmode == KMODE_LT_I_END) khi = min(K, i0 + TM);  // A lower triangular: A[i][k] = 0 for k > i
  else if (a.kmode == KMODE_GE_I) klo = i0;            // A^T with A lower: A[k][i] = 0 for k < i
  klo = (klo / TK) * TK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  double ra[4], rb[4];
  auto gload = [&](int k0) {
    // A tile: TM x TK of opA
    if (!TA) {
      const int ii = tid >> 2, kk = (tid & 3) * 4;
      const int gi = i0 + ii;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gk = k0 + kk + q;
        ra[q] = (gi < M && gk < khi) ? A[(int64_t)gi * a.lda + gk] : 0.0;
      }
    } else {
      const int kk = tid >> 4, ii = (tid & 15) * 4;
      const int gk = k0 + kk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gi = i0 + ii + q;
        ra[q] = (gi < M && gk < khi) ? A[(int64_t)gk * a.lda + gi] : 0.0;
      }
    }
    if (!TB) {
      const int kk = tid >> 4, jj = (tid & 15) * 4;
      const int gk = k0 + kk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gj = j0 + jj + q;
        rb[q] = (gj < N && gk < khi) ? B[(int64_t)gk * a.ldb + gj] : 0.0;
      }
    } else {
      const int jj = tid >> 2, kk = (tid & 3) * 4;
      const int gj = j0 + jj;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gk = k0 + kk + q;
        rb[q] = (gj < N && gk < khi) ? B[(int64_t)gj * a.ldb + gk] : 0.0;
      }
    }
  };
  auto lstore = [&](int st) {
    if (!TA) {
      const int ii = tid >> 2, kk = (tid & 3) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) As[st][kk + q][ii] = ra[q];
    } else {
      const int kk = tid >> 4, ii = (tid & 15) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) As[st][kk][ii + q] = ra[q];
    }
    if (!TB) {
      const int kk = tid >> 4, jj = (tid & 15) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) Bs[st][kk][jj + q] = rb[q];
    } else {
      const int jj = tid >> 2, kk = (tid & 3) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) Bs[st][kk + q][jj] = rb[q];
    }
  };

  f64x4 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = (f64x4){0.0, 0.0, 0.0, 0.0};

  const int nk = (khi > klo) ? (khi - klo + TK - 1) / TK : 0;
  if (nk > 0) {
    gload(klo);
    lstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(klo + (kt + 1) * TK);
#pragma unroll
    for (int k4 = 0; k4 < TK; k4 += 4) {
      const int kr = k4 + (lane >> 4);
      double fa[2], fb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) fa[mb] = As[st][kr][wm * 32 + mb * 16 + (lane & 15)];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) fb[nb] = Bs[st][kr][wn * 32 + nb * 16 + (lane & 15)];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // D layout of 16x16x4 f64: register r of lane l holds row (l / 16) + 4 r, column l % 16
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = i0 + wm * 32 + mb * 16 + (lane >> 4) + 4 * r;
        const int gj = j0 + wn * 32 + nb * 16 + (lane & 15);
        if (gi < M && gj < N) {
          double* p = C + (int64_t)gi * a.ldc + gj;
          const double v = a.alpha * acc[mb][nb][r];
          *p = (a.beta == 0.0) ? v : fma(a.beta, *p, v);
        }
      }
}

}  // namespace

hipError_t dgemm_launch(const DgemmArgs& a, bool ta, bool tb, int batches, hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0 || batches <= 0) return hipSuccess;
  int tiles;
  if (a.tri_tiles) {
    const int nt = (a.M + TM - 1) / TM;
    tiles = nt * (nt + 1) / 2;
  } else {
    tiles = ((a.M + TM - 1) / TM) * ((a.N + TN - 1) / TN);
  }
  dim3 grid(tiles, batches);
  if (!ta && !tb) k_dgemm<false, false><<<grid, dim3(256), 0, stream>>>(a);
  else if (!ta && tb) k_dgemm<false, true><<<grid, dim3(256), 0, stream>>>(a);
  else if (ta && !tb) k_dgemm<true, false><<<grid, dim3(256), 0, stream>>>(a);
  else k_dgemm<true, true><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace gptq
