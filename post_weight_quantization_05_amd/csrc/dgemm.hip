// fp64 tiled GEMM on gfx950 matrix cores (v_mfma_f64_16x16x4_f64), the
// shared core of the blocked factorization (trailing SYRK updates, triangular-inverse levels) and of the
// quantize loop's trailing update W[:, b1:] -= Err U[b0:b1, b1:].
//
//   C[i][j] = alpha * sum_{k in K-range(tile)} opA(A)[i][k] opB(B)[k][j] + beta * C[i][j]
//   opA(A)[i][k] = TA ? A[k][i] : A[i][k],  opB(B)[k][j] = TB ? B[j][k] : B[k][j]  (row-major storage)
//
// Tiles are T x T (T = 64: 256 threads, 4 waves of 32 x 32); K runs in chunks of 16 through
// double-buffered LDS, fed from a register ring that keeps PD chunks of global loads in flight.
// Options: only lower-triangle tiles (I >= J) of a square C; per-tile K-range
// restrictions for triangular operands (their zero triangle is then never multiplied); and a batch index
// (blockIdx.y) with per-operand strides and a per-batch row limit.
#include <type_traits>

#include "common.h"
#include "dgemm.h"
#include "diagblock.h"

namespace gptq {

namespace {

#ifndef GPTQ_DGEMM_TK
#define GPTQ_DGEMM_TK 16
#endif
constexpr int TK = GPTQ_DGEMM_TK;  // K per LDS chunk
constexpr int PD = 3;  // operand chunks in flight (register ring)

template <int K, int N, typename F>
__device__ __forceinline__ void static_for_d(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for_d<K + 1, N>(f);
  }
}

// LDS layouts. An operand whose rows run along the tile's M (or N) dimension in memory (A^T, B) is kept
// as [k][i] with rows padded to T + 16 doubles; an operand whose rows run along k (A, B^T) is kept as
// [i][k] with rows of TK + 4 doubles. A 16 x 4 fragment read (16 consecutive i, 4 consecutive k) then
// touches every bank pair exactly twice in both layouts. Both are filled with 16-byte stores of two
// consecutive doubles.
template <int T>
struct Lds {
  static constexpr int KI = T + 16;  // [k][i] row stride
  static constexpr int IK = TK + 4;  // [i][k] row stride
  static constexpr int SZ = (TK * KI > T * IK) ? TK * KI : T * IK;
};

// acc = sum over k in [klo, khi) of opA(A)[i0 + i][k] opB(B)[k][j0 + j] for the T x T tile at (i0, j0)
// (zero outside M x N x K). 4 waves in 2 x 2, each (T/2) x (T/2). Operand chunks of T x 16 are fetched
// as 16-byte vectors into registers while the MFMAs of earlier chunks run, then stored to the other LDS
// buffer. Ends with a barrier, so the LDS buffers may be reused at once.
template <bool TA, bool TB, int T>
__device__ __forceinline__ void tile_product(const DgemmArgs& a, const double* A, const double* B, int M, int N,
                                             int K, int i0, int j0, int klo, int khi,
                                             double (*As)[Lds<T>::SZ], double (*Bs)[Lds<T>::SZ],
                                             f64x4 (&acc)[T / 32][T / 32]) {
  constexpr int NV = T * TK / 2 / 256;   // 16-byte loads per thread per operand and chunk
  using L = Lds<T>;
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
  // register ring: PD chunks of both operands in flight, so short-K and few-tile products (the panel
  // solves and small updates of the factorization) wait for one global-memory latency, not one per chunk
  double2 ra[PD][NV], rb[PD][NV];
  auto gload = [&](auto slot_c, int k0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int e = tid + 256 * q;
      if (!TA) {
        const int ii = e / (TK / 2), kk = (e % (TK / 2)) * 2;
        ra[slot][q] = ld2(A, a.lda, i0 + ii, k0 + kk, M, klo, khi, a_vec);
      } else {
        const int kk = e / (T / 2), ii = (e % (T / 2)) * 2;
        ra[slot][q] = (k0 + kk < khi) ? ld2(A, a.lda, k0 + kk, i0 + ii, K, 0, M, a_vec) : make_double2(0.0, 0.0);
      }
      if (!TB) {
        const int kk = e / (T / 2), jj = (e % (T / 2)) * 2;
        rb[slot][q] = (k0 + kk < khi) ? ld2(B, a.ldb, k0 + kk, j0 + jj, K, 0, N, b_vec) : make_double2(0.0, 0.0);
      } else {
        const int jj = e / (TK / 2), kk = (e % (TK / 2)) * 2;
        rb[slot][q] = ld2(B, a.ldb, j0 + jj, k0 + kk, N, klo, khi, b_vec);
      }
    }
  };
  auto lstore = [&](auto slot_c, int st) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int e = tid + 256 * q;
      if (!TA) *reinterpret_cast<double2*>(&As[st][(e / (TK / 2)) * L::IK + (e % (TK / 2)) * 2]) = ra[slot][q];
      else *reinterpret_cast<double2*>(&As[st][(e / (T / 2)) * L::KI + (e % (T / 2)) * 2]) = ra[slot][q];
      if (!TB) *reinterpret_cast<double2*>(&Bs[st][(e / (T / 2)) * L::KI + (e % (T / 2)) * 2]) = rb[slot][q];
      else *reinterpret_cast<double2*>(&Bs[st][(e / (TK / 2)) * L::IK + (e % (TK / 2)) * 2]) = rb[slot][q];
    }
  };

  // v_mfma_f64_16x16x4f64: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] of a 16 x 4 by
  // 4 x 16 product and holds D[4 r + l / 16][l % 16] in register r. A wave's (T/2) x (T/2) block is
  // FR x FC such 16 x 16 tiles.
  constexpr int FR = T / 32;
  constexpr int FC = T / 32;
#pragma unroll
  for (int p = 0; p < FR; ++p)
#pragma unroll
    for (int q = 0; q < FC; ++q) acc[p][q] = f64x4{0.0, 0.0, 0.0, 0.0};

  const int nk = (khi > klo) ? (khi - klo + TK - 1) / TK : 0;
  static_for_d<0, PD>([&](auto pc) {
    if (decltype(pc)::value < nk) gload(pc, klo + decltype(pc)::value * TK);
  });
  if (nk > 0) lstore(std::integral_constant<int, 0>{}, 0);
  __syncthreads();
  const int lk = lane >> 4, lc = lane & 15;
  // chunk kt sits in ring slot kt % PD until it is stored to LDS buffer kt % 2
  for (int kt0 = 0; kt0 < nk; kt0 += PD) {
    static_for_d<0, PD>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    const int kt = kt0 + p;
    if (kt >= nk) return;
    const int st = kt & 1;
    if (kt + PD < nk) gload(pc, klo + (kt + PD) * TK);
#pragma unroll
    for (int k4 = 0; k4 < TK; k4 += 4) {
      const int kr = k4 + lk;
      double fa[FR], fb[FC];
#pragma unroll
      for (int r = 0; r < FR; ++r) {
        const int i = wm * (T / 2) + r * 16 + lc;
        fa[r] = TA ? As[st][kr * L::KI + i] : As[st][i * L::IK + kr];
      }
#pragma unroll
      for (int q = 0; q < FC; ++q) {
        const int j = wn * (T / 2) + q * 16 + lc;
        fb[q] = TB ? Bs[st][j * L::IK + kr] : Bs[st][kr * L::KI + j];
      }
#pragma unroll
      for (int r = 0; r < FR; ++r)
#pragma unroll
        for (int q = 0; q < FC; ++q) acc[r][q] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[r], fb[q], acc[r][q], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(std::integral_constant<int, (p + 1) % PD>{}, st ^ 1);
    __syncthreads();
    });
  }
}

// Tile t of the lower triangle of an nt x nt tile grid: in row order (row I holds t = I(I+1)/2 ..
// I(I+1)/2 + I), or in column order (column J from row J down, then column J + 1), which is row order
// on the grid turned half a revolution.
__device__ __forceinline__ void tri_tile(int t, int nt, bool col_order, int& I, int& J) {
  const int s = col_order ? nt * (nt + 1) / 2 - 1 - t : t;
  int R = (int)((sqrt(8.0 * (double)s + 1.0) - 1.0) * 0.5);
  while ((R + 1) * (R + 2) / 2 <= s) ++R;
  while (R * (R + 1) / 2 > s) --R;
  const int C = s - R * (R + 1) / 2;
  I = col_order ? nt - 1 - C : R;
  J = col_order ? nt - 1 - R : C;
}

// T x T tile of C = alpha opA(A) opB(B) + beta C (see the file comment for the options).
template <bool TA, bool TB, int T>
__global__ __launch_bounds__(256) void k_dgemm(DgemmArgs a) {
  using L = Lds<T>;
  __shared__ __attribute__((aligned(16))) double As[2][L::SZ];
  __shared__ __attribute__((aligned(16))) double Bs[2][L::SZ];

  const int batch = blockIdx.y;
  int I, J;
  if (a.tri_tiles) {
    tri_tile((int)blockIdx.x + a.tile_first, (a.M + T - 1) / T, a.tri_tiles == 2, I, J);
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
  if (a.lower_only && I < J) return;
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

  constexpr int FR = T / 32;
  constexpr int FC = T / 32;
  f64x4 acc[FR][FC];
  tile_product<TA, TB, T>(a, A, B, M, N, K, i0, j0, klo, khi, As, Bs, acc);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lk = lane >> 4, lc = lane & 15;

  const bool diag_tile = (a.tri_tiles || a.lower_only) && I == J;
#pragma unroll
  for (int r = 0; r < FR; ++r)
#pragma unroll
    for (int q = 0; q < FC; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = i0 + wm * (T / 2) + r * 16 + 4 * e + lk;
        const int gj = j0 + wn * (T / 2) + q * 16 + lc;
        if (gi < M && gj < N) {
          double* ptr = C + (int64_t)gi * a.ldc + gj;
          const double v = a.alpha * acc[r][q][e];
          // a diagonal tile of a triangular update writes its lower triangle only
          if (!diag_tile || gj - j0 <= gi - i0) *ptr = (a.beta == 0.0) ? v : fma(a.beta, *ptr, v);
        }
      }
}

// Single-shot form of tile_product for the block-column step (A B^T, T = 64, K = 64): all operand loads
// in flight at once, one LDS store, one barrier, then the whole K, unrolled, on the matrix cores. The
// operands sit in LDS as [row][k] with rows of 68 doubles (a 16 x 4 fragment read touches each bank pair
// twice). k64_stage loads and stores them (rows i0.. of A to As, rows j0.. of B to Bs) and ends with a
// barrier; the products read them.
constexpr int K64S = 68;
// thread element e = tid + 256 v of a 64 x 64 operand block: row e / 32, column pair 2 (e % 32)
__device__ __forceinline__ void k64_load(const double* A, const double* B, int64_t lda, int64_t ldb, int M, int N,
                                         int i0, int j0, double2 (&ra)[8], double2 (&rb)[8]) {
  const int tid = threadIdx.x;
  const bool a_vec = ((lda & 1) == 0) && ((reinterpret_cast<uintptr_t>(A) & 15) == 0);
  const bool b_vec = ((ldb & 1) == 0) && ((reinterpret_cast<uintptr_t>(B) & 15) == 0);
  auto ld2 = [&](const double* P, int64_t ld, int r, int rlim, int c2, bool vec) {
    double2 v = make_double2(0.0, 0.0);
    if (r < rlim) {
      const double* q = P + (int64_t)r * ld + c2;
      if (vec) {
        v = *reinterpret_cast<const double2*>(q);
      } else {
        v.x = q[0];
        v.y = q[1];
      }
    }
    return v;
  };
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int e = tid + 256 * v, r = e >> 5, c2 = (e & 31) * 2;
    ra[v] = ld2(A, lda, i0 + r, M, c2, a_vec);
    rb[v] = ld2(B, ldb, j0 + r, N, c2, b_vec);
  }
}
// stores a loaded pair of operand blocks (A to As, B to Bs) and ends with a barrier
__device__ __forceinline__ void k64_store(const double2 (&ra)[8], const double2 (&rb)[8], double* As, double* Bs) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int e = tid + 256 * v, r = e >> 5, c2 = (e & 31) * 2;
    *reinterpret_cast<double2*>(&As[r * K64S + c2]) = ra[v];
    *reinterpret_cast<double2*>(&Bs[r * K64S + c2]) = rb[v];
  }
  __syncthreads();
}
__device__ __forceinline__ void k64_stage(const double* A, const double* B, int64_t lda, int64_t ldb, int M, int N,
                                          int i0, int j0, double* As, double* Bs) {
  double2 ra[8], rb[8];
  k64_load(A, B, lda, ldb, M, N, i0, j0, ra, rb);
  k64_store(ra, rb, As, Bs);
}

// acc = the T x T tile of A B^T over K = 64 nk (nk >= 1), staged 64 of K at a time; 4 waves in 2 x 2, each
// 32 x 32. Ends with a barrier.
__device__ __forceinline__ void tile_product_k64(const double* A, const double* B, int64_t lda, int64_t ldb, int M,
                                                 int N, int i0, int j0, double* As, double* Bs,
                                                 f64x4 (&acc)[2][2], const int nk = 1) {
  constexpr int T = 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lk = lane >> 4, lc = lane & 15;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[p][q] = f64x4{0.0, 0.0, 0.0, 0.0};
  // the next 64 of K is loaded into registers while the matrix cores work on the staged chunk
  double2 ra[8], rb[8];
  k64_load(A, B, lda, ldb, M, N, i0, j0, ra, rb);
  for (int kc = 0; kc < nk; ++kc) {
    k64_store(ra, rb, As, Bs);
    if (kc + 1 < nk) k64_load(A + T * (kc + 1), B + T * (kc + 1), lda, ldb, M, N, i0, j0, ra, rb);
#pragma unroll
    for (int k4 = 0; k4 < T; k4 += 4) {
      const int kr = k4 + lk;
      double fa[2], fb[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) fa[r] = As[(wm * (T / 2) + r * 16 + lc) * K64S + kr];
#pragma unroll
      for (int q = 0; q < 2; ++q) fb[q] = Bs[(wn * (T / 2) + q * 16 + lc) * K64S + kr];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          acc[r][q] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[r], fb[q], acc[r][q], 0, 0, 0);
    }
    __syncthreads();
  }
}

// The two products of a panel workgroup of the block-column step, over K = 64 nk (nk >= 1), from stagings of
// the previous panel's rows 64 of K at a time (this tile's rows i0.. as A, the diagonal block's rows 0.. as B):
//   dacc: the diagonal block's update B B^T, 2 x 2 waves of 32 x 32 as in tile_product_k64;
//   xt:   this tile's update A B^T, transposed: wave w forms the 64 x 16 strip (B A^T)[:, 16w .. 16w + 15],
//         so entry r of xt[jb] in lane l is (A B^T)[16w + l % 16][16 jb + 4 r + l / 16], exactly the A-operand
//         fragment of k-step 4 jb + r of a product whose left factor is that tile's rows 16w .. 16w + 15.
// Ends with a barrier.
__device__ __forceinline__ void panel_products_k64(const double* A, const double* B, int64_t lda, int64_t ldb,
                                                   int M, int N, int i0, double* As, double* Bs,
                                                   f64x4 (&dacc)[2][2], f64x4 (&xt)[4], int nk = 1) {
  constexpr int T = 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lk = lane >> 4, lc = lane & 15;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q) dacc[p][q] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) xt[jb] = f64x4{0.0, 0.0, 0.0, 0.0};
  // (no register prefetch of the next chunk here: the panel workgroup already holds its tile X and the
  // diagonal block's old values, and the extra 64 registers would spill)
  for (int kc = 0; kc < nk; ++kc) {
    k64_stage(A + T * kc, B + T * kc, lda, ldb, M, N, i0, 0, As, Bs);
#pragma unroll
    for (int k4 = 0; k4 < T; k4 += 4) {
      const int kr = k4 + lk;
      double fb[4], fo;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) fb[jb] = Bs[(jb * 16 + lc) * K64S + kr];
      fo = As[(wave * 16 + lc) * K64S + kr];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          dacc[r][q] = __builtin_amdgcn_mfma_f64_16x16x4f64(fb[2 * wm + r], fb[2 * wn + q], dacc[r][q], 0, 0, 0);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) xt[jb] = __builtin_amdgcn_mfma_f64_16x16x4f64(fb[jb], fo, xt[jb], 0, 0, 0);
    }
    __syncthreads();
  }
}

// C = alpha A B + beta C for one 64 x 64 tile with K = 64, A (64 x 64) and B (64 x 64) row-major: rows of A
// and C at or past mrows are zero / not stored, rows of B at or past krows are zero. A is staged as [i][k]
// with rows of 68 doubles, B as [k][j] with rows of 80 (as in k_dgemm_nn_smallk); 4 waves in 2 x 2. C may
// be B itself: all of B is in LDS before C is written. beta == 0 reads no C.
constexpr int NN_BS = 80;
constexpr int NN64_LDS = 64 * K64S + 64 * NN_BS;  // doubles
__device__ __forceinline__ void nn64(const double* A, int64_t lda, const double* B, int64_t ldb, double* C,
                                     int64_t ldc, int mrows, int krows, double alpha, double beta, double* As,
                                     double* Bs) {
  constexpr int T = 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lk = lane >> 4, lc = lane & 15;
  double2 ra[8], rb[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int e = tid + 256 * v, r = e >> 5, c2 = (e & 31) * 2;
    ra[v] = (r < mrows) ? make_double2(A[(int64_t)r * lda + c2], A[(int64_t)r * lda + c2 + 1]) : make_double2(0.0, 0.0);
    rb[v] = (r < krows) ? make_double2(B[(int64_t)r * ldb + c2], B[(int64_t)r * ldb + c2 + 1]) : make_double2(0.0, 0.0);
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int e = tid + 256 * v, r = e >> 5, c2 = (e & 31) * 2;
    *reinterpret_cast<double2*>(&As[r * K64S + c2]) = ra[v];
    *reinterpret_cast<double2*>(&Bs[r * NN_BS + c2]) = rb[v];
  }
  __syncthreads();
  f64x4 acc[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[p][q] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int k4 = 0; k4 < T; k4 += 4) {
    const int kr = k4 + lk;
    double fa[2], fb[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) fa[r] = As[(wm * 32 + r * 16 + lc) * K64S + kr];
#pragma unroll
    for (int q = 0; q < 2; ++q) fb[q] = Bs[kr * NN_BS + wn * 32 + q * 16 + lc];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[r][q] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[r], fb[q], acc[r][q], 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = wm * 32 + r * 16 + 4 * e + lk, j = wn * 32 + q * 16 + lc;
        if (i < mrows) {
          double* ptr = C + (int64_t)i * ldc + j;
          const double v = alpha * acc[r][q][e];
          *ptr = (beta == 0.0) ? v : fma(beta, *ptr, v);
        }
      }
}

}  // namespace

// Tiles of launch f.k of the inverse: G tiles of step k - 1, update tiles of step k - 2, scaling tiles of
// step k - 3 (see InvFill in dgemm.h).
__host__ __device__ inline void inv_fill_counts(const InvFill& f, int& na, int& nb, int& nc) {
  const int ta = f.k - 1, tb = f.k - 2, tc = f.k - 3;
  na = (ta >= 0 && ta < f.S - 1) ? f.S - 1 - ta : 0;               // blocks i > ta
  nb = (tb >= 0 && tb < f.S - 1) ? (f.S - 1 - tb) * (tb + 1) : 0;  // i > tb, j <= tb
  nc = (tc >= 0 && tc < f.S) ? tc + 1 : 0;                         // j <= tc
}

int inv_fill_tiles(const InvFill& f) {
  int na, nb, nc;
  inv_fill_counts(f, na, nb, nc);
  return na + nb + nc;
}

namespace {

__device__ __forceinline__ void inv_fill_tile(const InvFill& f, int t, double* lds) {
  constexpr int T = 64;
  int na, nb, nc;
  inv_fill_counts(f, na, nb, nc);
  double* As = lds;
  double* Bs = lds + 64 * K64S;
  const int d = f.d;
  if (t < na) {
    // G_{i,ta} = L_{i,ta} Dinv_ta, block row i > ta (rows past d skipped)
    const int ta = f.k - 1, i = ta + 1 + t;
    double* G = f.G[ta & 1] + (int64_t)i * T * T;
    nn64(f.L + (int64_t)i * T * d + (int64_t)ta * T, d, f.Dinv + (int64_t)ta * T * T, T, G, T, min(T, d - i * T), T,
         1.0, 0.0, As, Bs);
    return;
  }
  t -= na;
  if (t < nb) {
    // Z_{i,j} -= G_{i,tb} Z_{tb,j} (j < tb), Z_{i,tb} = -G_{i,tb}
    const int tb = f.k - 2, i = tb + 1 + t / (tb + 1), j = t % (tb + 1);
    const double* G = f.G[tb & 1] + (int64_t)i * T * T;
    double* Zij = f.Z + (int64_t)i * T * d + (int64_t)j * T;
    const int mrows = min(T, d - i * T);
    if (j < tb) {
      nn64(G, T, f.Z + (int64_t)tb * T * d + (int64_t)j * T, d, Zij, d, mrows, T, -1.0, 1.0, As, Bs);
    } else {
      for (int e = threadIdx.x; e < T * T; e += 256) {
        const int r = e / T, c = e % T;
        if (r < mrows) Zij[(int64_t)r * d + c] = -G[e];
      }
    }
    return;
  }
  t -= nb;
  // Z_{tc,j} = Dinv_tc Z_{tc,j} (j < tc, in place), Z_{tc,tc} = Dinv_tc
  const int tc = f.k - 3, j = t;
  const double* D = f.Dinv + (int64_t)tc * T * T;
  double* Ztj = f.Z + (int64_t)tc * T * d + (int64_t)j * T;
  const int rows = min(T, d - tc * T);
  if (j < tc) {
    nn64(D, T, Ztj, d, Ztj, d, rows, rows, 1.0, 0.0, As, Bs);
  } else {
    for (int e = threadIdx.x; e < T * T; e += 256) {
      const int r = e / T, c = e % T;
      if (r < rows && c < rows) Ztj[(int64_t)r * d + c] = D[e];
    }
  }
}

__global__ __launch_bounds__(256, 2) void k_inv_fill(InvFill f) {
  __shared__ __attribute__((aligned(16))) double lds[NN64_LDS];
  inv_fill_tile(f, (int)blockIdx.x, lds);
}

// Block-column step of the factorization (T = 64, C = A B^T update with beta = 1, kmode FULL). C is the
// region A[c1:, c1:c1 + N] of the matrix being factored, M x N with M >= N; its tile (0, 0) is the next
// 64 x 64 diagonal block and its column-0 tiles below are the next panel. Workgroup roles:
//  * tiles (I, J >= 1), I >= J: the update C -= A B^T, as k_dgemm with lower_only;
//  * tile (0, 0): the updated diagonal block D is factored; L goes to diag_Lstage[kb], L^-1 to
//    diag_Dinv[kb], bad pivots to diag_status. The block in C itself is not written in this launch;
//  * tiles (I >= 1, 0): the updated tile X and, again, D from the same inputs (so every one of these
//    workgroups gets the same factor as tile (0, 0) without waiting for it); X is then solved,
//    X (L^-1)^T on the matrix cores from X held in registers, and written in place: the panel of the
//    next step.
// K is 64 (the previous step's panel), 256 (the first step of an outer block: the previous outer block's
// whole panel, staged 64 of K at a time), or 0 (the very first step: the launch only factors the block and
// solves the panel). Further workgroups past the step's own tiles take tiles of a deferred update xa.
// NK: K / 64 when K > 0 (1 or 4), a compile-time count so that the K = 64 launches keep the register budget
// of a single staged product.
template <int T, int NK>
__global__ __launch_bounds__(256, 2) void k_colstep(DgemmArgs a, DgemmArgs xa, int x_first, int n_own,
                                                   int x_count, InvFill fl) {
  static_assert(T == diagblock::NB, "the diagonal block is one tile");
  using L = Lds<T>;
  // One LDS buffer, two uses in turn: the operands (2 x 64 rows of K64S for the step's own K = 64
  // products, or the ring of tile_product for the deferred tiles), then the diagonal block and its
  // inverse for the factorization (the products end with a barrier). About 70 KB, so two workgroups
  // share a CU.
  constexpr int AB_SZ = (2 * T * K64S > 4 * L::SZ) ? 2 * T * K64S : 4 * L::SZ;
  constexpr int BSM_SZ = (int)(sizeof(diagblock::BlockSmem) / sizeof(double));
  constexpr int SZ1 = AB_SZ > BSM_SZ ? AB_SZ : BSM_SZ;
  __shared__ __attribute__((aligned(16))) double ABs[SZ1 > NN64_LDS ? SZ1 : NN64_LDS];
  diagblock::BlockSmem& bsm = *reinterpret_cast<diagblock::BlockSmem*>(ABs);
  double(*As)[L::SZ] = reinterpret_cast<double(*)[L::SZ]>(ABs);
  double(*Bs)[L::SZ] = reinterpret_cast<double(*)[L::SZ]>(ABs + 2 * L::SZ);

  if ((int)blockIdx.x >= n_own + x_count) {
    // a tile of the inverse L^-1 (independent of this step's own work)
    inv_fill_tile(fl, (int)blockIdx.x - n_own - x_count, ABs);
    return;
  }
  if ((int)blockIdx.x >= n_own) {
    // a tile of the deferred trailing update xa (lower tiles of a square region from x_first, in column
    // order if xa.tri_tiles is 2, else in row order): independent of this step's own work, it fills CUs
    // the step leaves idle
    const int t = x_first + ((int)blockIdx.x - n_own);
    const int xnt = (xa.M + T - 1) / T;
    if (t >= xnt * (xnt + 1) / 2) return;
    int XI, XJ;
    tri_tile(t, xnt, xa.tri_tiles == 2, XI, XJ);
    const int xi0 = XI * T, xj0 = XJ * T;
    if (xi0 >= xa.M || xj0 >= xa.N) return;
    f64x4 xacc[T / 32][T / 32];
    tile_product<false, true, T>(xa, xa.A, xa.B, xa.M, xa.N, xa.K, xi0, xj0, 0, xa.K, As, Bs, xacc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int r = 0; r < T / 32; ++r)
#pragma unroll
      for (int q = 0; q < T / 32; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = xi0 + wm * (T / 2) + r * 16 + 4 * e + (lane >> 4);
          const int gj = xj0 + wn * (T / 2) + q * 16 + (lane & 15);
          if (gi < xa.M && gj < xa.N && (XI != XJ || gj - xj0 <= gi - xi0)) {
            double* ptr = xa.C + (int64_t)gi * xa.ldc + gj;
            *ptr = fma(xa.beta, *ptr, xa.alpha * xacc[r][q][e]);
          }
        }
    return;
  }
  const int ntn = (a.N + T - 1) / T;
  const int I = blockIdx.x / ntn, J = blockIdx.x - I * ntn;
  if (I < J) return;
  const int M = a.M, N = a.N, K = a.K;  // K is 0, 64 or 256
  const int i0 = I * T, j0 = J * T;
  if (i0 >= M || j0 >= N) return;
  const double* A = a.A;
  const double* B = a.B;
  double* C = a.C;
  constexpr int FR = T / 32;
  constexpr int FC = T / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lk = lane >> 4, lc = lane & 15;
  // element (r, q, e) of a 2 x 2-wave accumulator is tile entry (ti(r, e), tj(q))
  auto ti = [&](int r, int e) { return wm * (T / 2) + r * 16 + 4 * e + lk; };
  auto tj = [&](int q) { return wn * (T / 2) + q * 16 + lc; };
  const int m = min(T, N);  // size of the diagonal block

  if (J != 0) {
    // the update C -= A B^T of a tile to the right of the panel
    if (K == 0) return;
    f64x4 acc[FR][FC];
    tile_product_k64(A, B, a.lda, a.ldb, M, N, i0, j0, ABs, ABs + T * K64S, acc, NK);
    const bool diag_tile = (I == J);
#pragma unroll
    for (int r = 0; r < FR; ++r)
#pragma unroll
      for (int q = 0; q < FC; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = i0 + ti(r, e), gj = j0 + tj(q);
          if (gi < M && gj < N && (!diag_tile || gj - j0 <= gi - i0)) {
            double* ptr = C + (int64_t)gi * a.ldc + gj;
            *ptr = fma(a.beta, *ptr, a.alpha * acc[r][q][e]);
          }
        }
    return;
  }

  // column 0: the diagonal block's old values (2 x 2-wave layout) are loaded before the products, so
  // their latency overlaps them
  double cdiag[FR][FC][4];
#pragma unroll
  for (int r = 0; r < FR; ++r)
#pragma unroll
    for (int q = 0; q < FC; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = ti(r, e), j = tj(q);
        cdiag[r][q][e] = (i < m && j < m && j <= i) ? C[(int64_t)i * a.ldc + j] : 0.0;
      }
  // the updated diagonal block, staged for the factorization (lower part; identity past the edge)
  auto stage_diag = [&](const f64x4 (&d)[FR][FC]) {
#pragma unroll
    for (int r = 0; r < FR; ++r)
#pragma unroll
      for (int q = 0; q < FC; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = ti(r, e), j = tj(q);
          double v = (i == j) ? 1.0 : 0.0;
          if (i < m && j < m && j <= i) v = fma(a.beta, cdiag[r][q][e], a.alpha * d[r][q][e]);
          bsm.A[i][j] = v;
        }
  };
  if (I == 0) {
    f64x4 acc[FR][FC];
    if (K > 0) {
      tile_product_k64(A, B, a.lda, a.ldb, M, N, 0, 0, ABs, ABs + T * K64S, acc, NK);
    } else {
#pragma unroll
      for (int r = 0; r < FR; ++r)
#pragma unroll
        for (int q = 0; q < FC; ++q) acc[r][q] = f64x4{0.0, 0.0, 0.0, 0.0};
    }
    stage_diag(acc);
    __syncthreads();
    const unsigned flags = diagblock::factor_invert_blocked(bsm);
    double* Lout = a.diag_Lstage + (int64_t)a.diag_kb * T * T;
    double* Dout = a.diag_Dinv + (int64_t)a.diag_kb * T * T;
    for (int e = tid; e < T * T; e += 256) {
      const int i = e / T, j = e % T;
      if (i < m && j < m) Lout[i * T + j] = bsm.A[i][j];
      Dout[e] = bsm.M[i][j];  // the identity past the edge
    }
    if (flags && tid == 0) atomicOr(a.diag_status, flags);
    return;
  }
  // A panel tile X (rows i0 .. i0 + 63 of column 0): wave w holds rows 16w .. 16w + 15 of X in the
  // A-operand layout of the solve, x[jb][r] = X[16w + lc][16 jb + 4 r + lk] (see panel_products_k64).
  const int xrow = i0 + 16 * wave + lc;
  double x[4][4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * jb + 4 * r + lk;
      x[jb][r] = (xrow < M && j < m) ? C[(int64_t)xrow * a.ldc + j] : 0.0;
    }
  f64x4 dacc[FR][FC];
  if (K > 0) {
    f64x4 xt[4];
    panel_products_k64(A, B, a.lda, a.ldb, M, N, i0, ABs, ABs + T * K64S, dacc, xt, NK);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jb + 4 * r + lk;
        x[jb][r] = (xrow < M && j < m) ? fma(a.beta, x[jb][r], a.alpha * xt[jb][r]) : 0.0;
      }
  } else {
#pragma unroll
    for (int r = 0; r < FR; ++r)
#pragma unroll
      for (int q = 0; q < FC; ++q) dacc[r][q] = f64x4{0.0, 0.0, 0.0, 0.0};
  }
  // the diagonal block again from the same inputs (no waiting on tile (0, 0)), factored and inverted
  stage_diag(dacc);
  __syncthreads();
  diagblock::factor_invert_blocked(bsm);
  // the panel tile X L^-T = X (L^-1)^T: out[i][j'] = sum_j X[i][j] L^-1[j'][j], on the matrix cores, wave w
  // forming rows 16w .. 16w + 15
  f64x4 sol[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sol[q] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kr = 16 * jb + 4 * r + lk;
      double fb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) fb[q] = bsm.M[16 * q + lc][kr];
#pragma unroll
      for (int q = 0; q < 4; ++q) sol[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(x[jb][r], fb[q], sol[q], 0, 0, 0);
    }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int gi = i0 + 16 * wave + 4 * e + lk, gj = 16 * q + lc;
      if (gi < M && gj < m) C[(int64_t)gi * a.ldc + gj] = sol[q][e];
    }
}

}  // namespace

// Large plain products C = alpha A B + beta C (A M x K, B K x N, both row-major, no options): the quantize
// loop's updates by a whole outer block (K = 1024). 128 x 128 tiles, 4 waves of 64 x 64, on
// v_mfma_f64_4x4x4_4b: on gfx950 that instruction sustains about 70 TFLOP/s where v_mfma_f64_16x16x4f64
// stops near 45, and a wave tile this large keeps the LDS bytes per matrix-core cycle low enough for it
// (measured on the 4096 x 3072 x 1024 update: 53.5 TFLOP/s against 46.6-48.0 for k_dgemm's 64 x 64
// tiles). The fragments are those of the 16 x 16 form, lane l supplying A[l % 16][l / 16] and
// B[l / 16][l % 16]; one 4x4 instruction multiplies, for each lane group g = (l % 16) / 4, the 4 x 4 blocks
// the group holds in both operands (rows 4g.. of A, columns 4g.. of B) into lane l's entry (row
// 4g + l / 16, column 4g + l % 4). The other block pairings take B rotated by 4, 8 and 12 lanes within
// each row of 16 (DPP row_ror), so four instructions form a 16 x 16 product, entry t of lane l being
// D[bmrow(l)][bmcol(l, t)]. K runs in chunks of 16 through double-buffered LDS (A as [i][k] rows of 20, B as
// [k][j] rows of 144); fragments are read one k-step ahead.
template <int N>
__device__ __forceinline__ double bm_ror(double v) {  // lane i of a row of 16 takes lane (i - N) mod 16
  return __builtin_amdgcn_mov_dpp(v, 0x120 + N, 0xF, 0xF, false);
}
__device__ __forceinline__ int bmrow(int lane) { return 4 * ((lane & 15) >> 2) + (lane >> 4); }
__device__ __forceinline__ int bmcol(int lane, int t) { return 4 * ((((lane & 15) >> 2) + t) & 3) + (lane & 3); }
constexpr int BM_T = 128, BM_K = 16;
constexpr int BM_AS = BM_K + 4, BM_BS = BM_T + 16;
constexpr int BM_MIN_K = 256;  // products with less K stay on k_dgemm / the small-K kernels
constexpr int BM_MIN_TILES = 512;  // two rounds of 256 CUs at two workgroups each
// The launch guarantees K % 16 == 0, even N, even lda and ldb, 16-byte aligned A and B, and strides below
// 2^31, so every element pair a thread stages is one 16-byte load that lies wholly inside or outside the
// operand.
__global__ __launch_bounds__(256, 2) void k_dgemm_nn_big(const double* __restrict__ A, int lda,
                                                         const double* __restrict__ B, int ldb,
                                                         double* __restrict__ C, int ldc, int M, int N, int K,
                                                         double alpha, double beta) {
  __shared__ __attribute__((aligned(16))) double As[2][BM_T * BM_AS];
  __shared__ __attribute__((aligned(16))) double Bs[2][BM_K * BM_BS];
  const int ntn = (N + BM_T - 1) / BM_T;
  const int I = blockIdx.x / ntn, J = blockIdx.x - I * ntn;
  const int i0 = I * BM_T, j0 = J * BM_T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lk = lane >> 4, lc = lane & 15;
  // a chunk: A 128 x 16 and B 16 x 128, four element pairs of each per thread
  double2 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = tid + 256 * v;
      const int gi = i0 + (e >> 3), gj = j0 + (e & 63) * 2;
      ra[v] = gi < M ? *reinterpret_cast<const double2*>(A + (int64_t)gi * lda + k0 + (e & 7) * 2)
                     : make_double2(0.0, 0.0);
      rb[v] = gj < N ? *reinterpret_cast<const double2*>(B + (int64_t)(k0 + (e >> 6)) * ldb + gj)
                     : make_double2(0.0, 0.0);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = tid + 256 * v;
      *reinterpret_cast<double2*>(&As[st][(e >> 3) * BM_AS + (e & 7) * 2]) = ra[v];
      *reinterpret_cast<double2*>(&Bs[st][(e >> 6) * BM_BS + (e & 63) * 2]) = rb[v];
    }
  };
  // acc[4 q + r]: row block r (rows 64 wm + 16 r ..) x column block q (columns 64 wn + 16 q ..)
  f64x4 acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int nk = K / BM_K;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BM_K);
    double fa[2][4], fb[2][4];
    auto frag = [&](int s2, int k4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) fa[s2][r] = As[st][(64 * wm + 16 * r + lc) * BM_AS + k4 + lk];
#pragma unroll
      for (int q = 0; q < 4; ++q) fb[s2][q] = Bs[st][(k4 + lk) * BM_BS + 64 * wn + 16 * q + lc];
    };
    frag(0, 0);
#pragma unroll
    for (int ks = 0; ks < BM_K / 4; ++ks) {
      const int s2 = ks & 1;
      if (ks + 1 < BM_K / 4) frag(s2 ^ 1, 4 * (ks + 1));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double br[4] = {fb[s2][q], bm_ror<12>(fb[s2][q]), bm_ror<8>(fb[s2][q]), bm_ror<4>(fb[s2][q])};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[4 * q + r][t] = __builtin_amdgcn_mfma_f64_4x4x4f64(fa[s2][r], br[t], acc[4 * q + r][t], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }
  const int mr = bmrow(lane);
#pragma unroll
  for (int x = 0; x < 16; ++x)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int gi = i0 + 64 * wm + 16 * (x & 3) + mr, gj = j0 + 64 * wn + 16 * (x >> 2) + bmcol(lane, t);
      if (gi < M && gj < N) {
        double* ptr = C + (int64_t)gi * ldc + gj;
        const double v = alpha * acc[x][t];
        *ptr = (beta == 0.0) ? v : fma(beta, *ptr, v);
      }
    }
}

// Plain products with K <= 128 and both operands row-major, C = alpha A B + beta C (A M x K, B K x N): the
// quantize loop's updates within an outer block (K = 128). Every operand load of the 64 x 64 tile is in
// flight at once, then the old C values; per 64 of K one LDS store, one barrier and the MFMA sequence.
// A is staged as [i][k] with rows of 68 doubles, B as [k][j] with rows of 80 doubles, so a 16 x 4 fragment
// read touches each bank pair twice.
#ifndef GPTQ_DGEMM_SMALLK
#define GPTQ_DGEMM_SMALLK 1
#endif
constexpr int SK_MAX = 128;
#ifndef GPTQ_DGEMM_SMALLK_TILES
#define GPTQ_DGEMM_SMALLK_TILES 1024
#endif
constexpr int SK_TILES = GPTQ_DGEMM_SMALLK_TILES;  // at most this many 64 x 64 tiles per launch (0: never)
constexpr int SK_AS = 68, SK_BS = 80;
__global__ __launch_bounds__(256) void k_dgemm_nn_smallk(DgemmArgs a) {
  constexpr int T = 64, NH = SK_MAX / T;
  __shared__ __attribute__((aligned(16))) double As[T * SK_AS];
  __shared__ __attribute__((aligned(16))) double Bs[T * SK_BS];
  const int M = a.M, N = a.N, K = a.K;
  const int ntn = (N + T - 1) / T;
  const int I = blockIdx.x / ntn, J = blockIdx.x - I * ntn;
  const int i0 = I * T, j0 = J * T;
  if (i0 >= M || j0 >= N) return;
  const double* A = a.A;
  const double* B = a.B;
  double* C = a.C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lk = lane >> 4, lc = lane & 15;
  const bool a_vec = ((a.lda & 1) == 0) && ((reinterpret_cast<uintptr_t>(A) & 15) == 0);
  const bool b_vec = ((a.ldb & 1) == 0) && ((reinterpret_cast<uintptr_t>(B) & 15) == 0);
  // element pair (r, c..c+1) of a row-major P, zero outside [0, rlim) x [0, clim)
  auto ld2 = [](const double* P, int64_t ld, int r, int rlim, int c, int clim, bool vec) {
    double2 v = make_double2(0.0, 0.0);
    if (r < rlim) {
      const double* q = P + (int64_t)r * ld + c;
      if (vec && c + 1 < clim) {
        v = *reinterpret_cast<const double2*>(q);
      } else {
        if (c < clim) v.x = q[0];
        if (c + 1 < clim) v.y = q[1];
      }
    }
    return v;
  };
  // thread element e = tid + 256 v of a 64 x 64 block: row e / 32, column pair 2 (e % 32)
  double2 ra[NH][8], rb[NH][8];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int e = tid + 256 * v, r = e >> 5, c2 = (e & 31) * 2;
      ra[h][v] = ld2(A + h * T, a.lda, i0 + r, M, c2, K - h * T, a_vec);                      // A[i0 + r][hT + c2]
      rb[h][v] = ld2(B + (int64_t)h * T * a.ldb, a.ldb, r, K - h * T, j0 + c2, N, b_vec);   // B[hT + r][j0 + c2]
    }
  // the old values of the thread's C entries (entry (r, q, e) is row 4e + lk of 16 x 16 block (r, q))
  double cold[2][2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = i0 + wm * (T / 2) + r * 16 + 4 * e + lk;
        const int gj = j0 + wn * (T / 2) + q * 16 + lc;
        cold[r][q][e] = (a.beta != 0.0 && gi < M && gj < N) ? C[(int64_t)gi * a.ldc + gj] : 0.0;
      }
  f64x4 acc[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[r][q] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    if (h * T >= K) break;  // K is the same for the whole workgroup
    if (h > 0) __syncthreads();  // the previous half is read
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int e = tid + 256 * v, r = e >> 5, c2 = (e & 31) * 2;
      *reinterpret_cast<double2*>(&As[r * SK_AS + c2]) = ra[h][v];
      *reinterpret_cast<double2*>(&Bs[r * SK_BS + c2]) = rb[h][v];
    }
    __syncthreads();
#pragma unroll
    for (int k4 = 0; k4 < T; k4 += 4) {
      const int kr = k4 + lk;
      double fa[2], fb[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) fa[r] = As[(wm * (T / 2) + r * 16 + lc) * SK_AS + kr];
#pragma unroll
      for (int q = 0; q < 2; ++q) fb[q] = Bs[kr * SK_BS + wn * (T / 2) + q * 16 + lc];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[r][q] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[r], fb[q], acc[r][q], 0, 0, 0);
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = i0 + wm * (T / 2) + r * 16 + 4 * e + lk;
        const int gj = j0 + wn * (T / 2) + q * 16 + lc;
        if (gi < M && gj < N) {
          const double v = a.alpha * acc[r][q][e];
          C[(int64_t)gi * a.ldc + gj] = (a.beta == 0.0) ? v : fma(a.beta, cold[r][q][e], v);
        }
      }
}

template <int T>
static hipError_t dgemm_launch_t(const DgemmArgs& a, bool ta, bool tb, int batches, hipStream_t stream) {
  int tiles;
  if (a.tri_tiles) {
    const int nt = (a.M + T - 1) / T;
    tiles = nt * (nt + 1) / 2 - a.tile_first;
    if (tiles <= 0) return hipSuccess;
  } else {
    tiles = ((a.M + T - 1) / T) * ((a.N + T - 1) / T);
  }
  dim3 grid(tiles, batches);
  const bool plain = T == 64 && !ta && !a.tri_tiles && a.kmode == KMODE_FULL && batches == 1 && a.m_step == 0 &&
                     !a.k_by_m;
  // the small-K kernel runs two workgroups per CU; past about two rounds of tiles the chunked ring's four
  // per CU wins (measured: 11008-row quantize updates 1.2 % slower on the small-K kernel, 4096-row ones
  // 2-3 % faster)
  const bool few = tiles <= SK_TILES;
  const bool smallk = GPTQ_DGEMM_SMALLK && plain && few && !tb && a.K <= SK_MAX && !a.lower_only;
#ifndef GPTQ_DGEMM_BIG
#define GPTQ_DGEMM_BIG 1
#endif
  // large plain A B: 128 x 128 tiles on the 4x4 matrix-core form (at least one round of the chip's
  // two workgroups per CU, so the larger tile does not leave CUs idle)
  const int big_tiles = ((a.M + BM_T - 1) / BM_T) * ((a.N + BM_T - 1) / BM_T);
  const bool big = GPTQ_DGEMM_BIG && plain && !tb && !a.lower_only && a.K >= BM_MIN_K && a.K % BM_K == 0 &&
                   a.N % 2 == 0 && big_tiles >= BM_MIN_TILES && (a.lda & 1) == 0 && (a.ldb & 1) == 0 &&
                   a.lda < INT32_MAX && a.ldb < INT32_MAX && a.ldc < INT32_MAX &&
                   (reinterpret_cast<uintptr_t>(a.A) & 15) == 0 && (reinterpret_cast<uintptr_t>(a.B) & 15) == 0;
  if (big)
    k_dgemm_nn_big<<<dim3(big_tiles), dim3(256), 0, stream>>>(a.A, (int)a.lda, a.B, (int)a.ldb, a.C, (int)a.ldc,
                                                            a.M, a.N, a.K, a.alpha, a.beta);
  else if (smallk) k_dgemm_nn_smallk<<<grid, dim3(256), 0, stream>>>(a);
  else if (!ta && !tb) k_dgemm<false, false, T><<<grid, dim3(256), 0, stream>>>(a);
  else if (!ta && tb) k_dgemm<false, true, T><<<grid, dim3(256), 0, stream>>>(a);
  else if (ta && !tb) k_dgemm<true, false, T><<<grid, dim3(256), 0, stream>>>(a);
  else k_dgemm<true, true, T><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t dgemm_launch(const DgemmArgs& a, bool ta, bool tb, int batches, hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0 || batches <= 0) return hipSuccess;
  // 64 x 64 tiles: the triangular K-ranges rely on zeros above the diagonal inside the factorization's
  // 64 x 64 diagonal blocks, which is exactly one tile (128 x 128 tiles measured no faster here)
  return dgemm_launch_t<64>(a, ta, tb, batches, stream);
}

hipError_t colstep_launch(const DgemmArgs& a, const DgemmArgs* x, int x_first, int x_count, const InvFill* f,
                          hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0 || a.N > a.M || (a.K != 0 && a.K != 64 && a.K != 256) || !a.diag_Lstage ||
      !a.diag_Dinv || !a.diag_status)
    return hipErrorInvalidValue;
  const int tiles = ((a.M + 63) / 64) * ((a.N + 63) / 64);
  DgemmArgs none{};
  if (!x || x_count < 0) x_count = 0;
  if (x_count > 0 && (x->M != x->N || x->kmode != KMODE_FULL)) return hipErrorInvalidValue;
  const InvFill nof{};
  const int f_count = f ? inv_fill_tiles(*f) : 0;
  const dim3 grid(tiles + x_count + f_count);
  if (a.K == 256)
    k_colstep<64, 4><<<grid, dim3(256), 0, stream>>>(a, x_count > 0 ? *x : none, x_first, tiles, x_count, f ? *f : nof);
  else
    k_colstep<64, 1><<<grid, dim3(256), 0, stream>>>(a, x_count > 0 ? *x : none, x_first, tiles, x_count, f ? *f : nof);
  return hipGetLastError();
}

hipError_t inv_fill_launch(const InvFill& f, hipStream_t stream) {
  const int n = inv_fill_tiles(f);
  if (n <= 0) return hipSuccess;
  k_inv_fill<<<dim3(n), dim3(256), 0, stream>>>(f);
  return hipGetLastError();
}

}  // namespace gptq
