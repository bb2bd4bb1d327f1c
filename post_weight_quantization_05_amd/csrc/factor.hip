// Prepare step and the factor U of H^-1 (fp64) on gfx950.
//
// GPTQ guide ("GPTQ", herodthegreater.github.io/pigeon/guide/gptq/):
//  * "The code, line by line", _hessian_inverse_chol: H = 2 X^T X / n; inputs whose diagonal is zero are
//    dead and get H[i][i] = 1; damping adds damp * mean(diag H) to the diagonal; U is the transposed
//    Cholesky factor of H^-1.
//  * act_order bullet: columns by decreasing diag(X^T X); U is recomputed for that order (= P^T H P).
//  * "GPTQ's two tricks", trick 2: U upper with H^-1 = U^T U.
//
// Kernels:
//  k_prep_stats   one workgroup: dead mask, diag H, lambda = damp * mean(diag H) (fixed-order reduction),
//                 non-finite check on colsq.
//  k_perm         act_order permutation by ranks (descending key, ties by index): a stable sort.
//  k_gather       H_p = P^T H P (optionally index-reversed) from S's lower triangle, lower part only.
//  k_potrf_diag   one wave factors a 64 x 64 diagonal block in registers (lane = row) and inverts it
//                 (lane = column); flags pivots that are not > 0 or not finite.
//  panel / SYRK / triangular-inverse levels / H^-1 = L^-T L^-1 use the fp64 MFMA GEMM core (dgemm.hip).
// Routes (flags): INVERSE_RECHOL = potrf, trtri, lauum, potrf, transpose (the guide's order);
// REVERSED = potrf and trtri of J H J, then U = J L^-1 J (same unique U, half the work).
#include <type_traits>

#include "common.h"
#include "dgemm.h"

namespace gptq {

namespace {

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

__global__ void k_zero_u32(unsigned* p) { *p = 0u; }

__global__ __launch_bounds__(1024) void k_prep_stats(const double* __restrict__ colsq, int64_t n_total, int d,
                                                     double damp, double* __restrict__ diag_out,
                                                     uint8_t* __restrict__ dead, unsigned* status) {
  __shared__ double red[1024];
  const int tid = threadIdx.x;
  const double two_over_n = 2.0 / (double)n_total;
  double local = 0.0;
  bool bad = false;
  for (int i = tid; i < d; i += 1024) {
    const double c = colsq[i];
    if (!isfinite(c)) bad = true;
    const bool dd = (c == 0.0);
    dead[i] = dd ? 1 : 0;
    const double h = dd ? 1.0 : two_over_n * c;
    diag_out[i] = h;
    local += h;
  }
  if (bad) atomicOr(status, DEV_STATUS_NONFINITE);
  red[tid] = local;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double lam = damp * (red[0] / (double)d);
  for (int i = tid; i < d; i += 1024) diag_out[i] += lam;
}

// perm[rank(i)] = i with rank by (descending key, ascending index); NaN keys order as -inf so the ranks
// always form a permutation.
__global__ __launch_bounds__(256) void k_perm(const double* __restrict__ colsq, int d, int act_order,
                                              int32_t* __restrict__ perm) {
  __shared__ double keys[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (!act_order) {
    if (i < d) perm[i] = i;
    return;
  }
  double key = -INFINITY;
  if (i < d) {
    key = colsq[i];
    if (isnan(key)) key = -INFINITY;
  }
  int rank = 0;
  for (int c0 = 0; c0 < d; c0 += 256) {
    __syncthreads();
    const int c = c0 + threadIdx.x;
    double v = -INFINITY;
    if (c < d) {
      v = colsq[c];
      if (isnan(v)) v = -INFINITY;
    }
    keys[threadIdx.x] = v;
    __syncthreads();
    const int lim = min(256, d - c0);
    for (int q = 0; q < lim; ++q) {
      const double kq = keys[q];
      const int k = c0 + q;
      rank += (kq > key || (kq == key && k < i)) ? 1 : 0;
    }
  }
  if (i < d) perm[rank] = i;
}

// A[a][b] (a >= b) = H[perm[x]][perm[y]] with (x, y) = (a, b), or (d-1-a, d-1-b) when reversed; the
// strictly upper part of A is set to 0. H off-diagonal = (2/n) S[max][min]; diagonal = diag_h (dead
// fixed, damped).
__global__ __launch_bounds__(256) void k_gather(const double* __restrict__ S, const double* __restrict__ diag_h,
                                                const int32_t* __restrict__ perm, int64_t n_total, int d,
                                                int reversed, double* __restrict__ A) {
  const int nbx = (d + 255) / 256;
  const int a = blockIdx.x / nbx;
  const int b = (blockIdx.x - a * nbx) * 256 + threadIdx.x;
  if (b >= d) return;
  double v = 0.0;
  if (b <= a) {
    const int x = reversed ? d - 1 - a : a;
    const int y = reversed ? d - 1 - b : b;
    const int pi = min(max(perm[x], 0), d - 1);
    const int pj = min(max(perm[y], 0), d - 1);
    if (pi == pj) {
      v = diag_h[pi];
    } else {
      const int hi = max(pi, pj), lo = min(pi, pj);
      v = (2.0 / (double)n_total) * S[(int64_t)hi * d + lo];
    }
  }
  A[(int64_t)a * d + b] = v;
}

// Factor the diagonal block kb of A in place (lower, zeros above) and write its inverse to Dinv[kb].
// One wave. Cholesky: lane i holds row i of the block in registers (right-looking: after pivot k every
// lane updates its own entries j > k with column k, which goes through LDS). Inverse: lane j holds
// column j of L^-1 and eliminates right-looking as well (c[i] -= L[i][k] c[k] for i > k). In both
// phases a step's LDS values are read in chunks of 8 with three chunks in flight ahead of the
// multiply-adds that use them, so a step waits for one LDS round trip, not one per chunk.
// Rows/columns past the matrix edge act as the identity.
template <int K>
struct ChunkSpan {
  static constexpr int first = ((K + 1) & ~7);                // first chunk start with entries > K
  static constexpr int count = (NB - first) / 8;               // chunks of 8 from `first` to NB
};

__global__ __launch_bounds__(64) void k_potrf_diag(double* __restrict__ A, int64_t lda, int d, int kb,
                                                   double* __restrict__ Dinv, unsigned* status) {
  __shared__ double col[NB];
  __shared__ double Ls[NB][NB + 1];
  __shared__ double rdg[NB];
  const int o = kb * NB;
  const int m = min(NB, d - o);
  const int i = threadIdx.x;
  unsigned flags = 0;
  {
    double r[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      double v = (i == j) ? 1.0 : 0.0;
      if (i < m && j < m && j <= i) v = A[(int64_t)(o + i) * lda + o + j];
      r[j] = v;
    }
    static_for<0, NB>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      double piv = readlane_d(r[k], k);
      if (!(piv > 0.0)) {
        flags |= isfinite(piv) ? DEV_STATUS_NOT_SPD : DEV_STATUS_NONFINITE;
        piv = 1.0;
      } else if (!isfinite(piv)) {
        flags |= DEV_STATUS_NONFINITE;
        piv = 1.0;
      }
      const double lkk = sqrt(piv);
      const double inv = 1.0 / lkk;
      r[k] = (i == k) ? lkk : r[k] * inv;
      if (i == k) rdg[k] = inv;  // 1 / L[k][k] for the inverse
      if constexpr (k + 1 < NB) {
        col[i] = r[k];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int F = ChunkSpan<k>::first, NC = ChunkSpan<k>::count;
        double buf[4][8];
        auto rd = [&](auto cc) {
          constexpr int c = decltype(cc)::value;
#pragma unroll
          for (int q = 0; q < 8; ++q) buf[c & 3][q] = col[F + 8 * c + q];
        };
        static_for<0, (NC < 3 ? NC : 3)>(rd);
        static_for<0, NC>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if constexpr (c + 3 < NC) rd(std::integral_constant<int, c + 3>{});
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            constexpr int dummy = 0;
            (void)dummy;
            const int jj = F + 8 * c + q;
            if (jj > k) r[F + 8 * c + q] = fma(-r[k], buf[c & 3][q], r[F + 8 * c + q]);
          }
        });
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = k + 1; j < NB; ++j) asm volatile("" : "+v"(r[j]));
      }
    });
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const double v = (j <= i) ? r[j] : 0.0;
      Ls[i][j] = v;
      if (i < m && j < m) A[(int64_t)(o + i) * lda + o + j] = v;
    }
  }
  if (flags && i == 0) atomicOr(status, flags);
  __syncthreads();
  // inverse: lane j holds column j of L^-1 (starts as e_j), right-looking elimination
  const int jc = i;
  double c[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) c[k] = (k == jc) ? 1.0 : 0.0;
  static_for<0, NB>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    c[k] = c[k] * rdg[k];
    if constexpr (k + 1 < NB) {
      constexpr int F = ChunkSpan<k>::first, NC = ChunkSpan<k>::count;
      double buf[4][8];
      auto rd = [&](auto cc) {
        constexpr int cb = decltype(cc)::value;
#pragma unroll
        for (int q = 0; q < 8; ++q) buf[cb & 3][q] = Ls[F + 8 * cb + q][k];
      };
      static_for<0, (NC < 3 ? NC : 3)>(rd);
      static_for<0, NC>([&](auto cc) {
        constexpr int cb = decltype(cc)::value;
        if constexpr (cb + 3 < NC) rd(std::integral_constant<int, cb + 3>{});
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r2 = F + 8 * cb + q;
          if (r2 > k) c[F + 8 * cb + q] = fma(-buf[cb & 3][q], c[k], c[F + 8 * cb + q]);
        }
      });
#pragma unroll
      for (int j = k; j < NB; ++j) asm volatile("" : "+v"(c[j]));
    }
  });
  double* D = Dinv + (int64_t)kb * NB * NB;
#pragma unroll
  for (int k = 0; k < NB; ++k) D[k * NB + jc] = (k < m && jc < m) ? c[k] : ((k == jc) ? 1.0 : 0.0);
}

// Copy the inverted diagonal blocks into the diagonal of A (start of the triangular inverse).
__global__ __launch_bounds__(256) void k_place_dinv(const double* __restrict__ Dinv, double* __restrict__ A,
                                                    int64_t lda, int d) {
  const int kb = blockIdx.x;
  const int o = kb * NB;
  const int m = min(NB, d - o);
  const double* D = Dinv + (int64_t)kb * NB * NB;
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int k = e / NB, j = e % NB;
    if (k < m && j < m) A[(int64_t)(o + k) * lda + o + j] = D[e];
  }
}

// U = L^T in place: lower triangle moved to the upper, lower set to 0 (32 x 32 tiles through LDS).
__global__ __launch_bounds__(256) void k_transpose_lower_to_upper(double* __restrict__ U, int d) {
  __shared__ double t1[32][33];
  const int t = blockIdx.x;
  int I = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while ((I + 1) * (I + 2) / 2 <= t) ++I;
  while (I * (I + 1) / 2 > t) --I;
  const int J = t - I * (I + 1) / 2;  // tile (I, J), I >= J, of the lower triangle
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  // load lower tile (I, J) and, for off-diagonal tiles, the upper tile (J, I)
  for (int y = ty; y < 32; y += 8) {
    const int gi = I * 32 + y, gj = J * 32 + tx;
    t1[y][tx] = (gi < d && gj < d) ? U[(int64_t)gi * d + gj] : 0.0;
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    // write upper tile (J, I): element (J*32 + y, I*32 + tx) = L[I*32 + tx][J*32 + y]
    const int gi = J * 32 + y, gj = I * 32 + tx;
    if (gi < d && gj < d) {
      const bool upper_or_diag = gj >= gi;
      U[(int64_t)gi * d + gj] = upper_or_diag ? t1[tx][y] : 0.0;
    }
  }
  if (I != J) {
    for (int y = ty; y < 32; y += 8) {
      const int gi = I * 32 + y, gj = J * 32 + tx;
      if (gi < d && gj < d) U[(int64_t)gi * d + gj] = 0.0;
    }
  }
}

// U[a][b] = Li[d-1-a][d-1-b] for a <= b, 0 below the diagonal.
__global__ __launch_bounds__(256) void k_reverse_to_upper(const double* __restrict__ Li, int d,
                                                          double* __restrict__ U) {
  const int nbx = (d + 255) / 256;
  const int a = blockIdx.x / nbx;
  const int b = (blockIdx.x - a * nbx) * 256 + threadIdx.x;
  if (b >= d) return;
  U[(int64_t)a * d + b] = (b >= a) ? Li[(int64_t)(d - 1 - a) * d + (d - 1 - b)] : 0.0;
}

hipError_t potrf_lower(double* A, int d, double* Dinv, unsigned* status, hipStream_t stream) {
  const int nblk = (d + NB - 1) / NB;
  for (int kb = 0; kb < nblk; ++kb) {
    hipLaunchKernelGGL(k_potrf_diag, dim3(1), dim3(64), 0, stream, A, (int64_t)d, d, kb, Dinv, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int o = kb * NB;
    const int m = min(NB, d - o);
    const int rest = d - o - m;
    if (rest <= 0) break;
    double* panel = A + (int64_t)(o + m) * d + o;
    // panel <- panel * Dinv^T (solve X L_kk^T = panel)
    DgemmArgs p{};
    p.A = panel; p.lda = d;
    p.B = Dinv + (int64_t)kb * NB * NB; p.ldb = NB;
    p.C = panel; p.ldc = d;
    p.M = rest; p.N = m; p.K = m;
    p.alpha = 1.0; p.beta = 0.0;
    p.kmode = KMODE_FULL;
    e = dgemm_launch(p, false, true, 1, stream);
    if (e != hipSuccess) return e;
    // trailing update, lower tiles: A22 -= panel panel^T
    DgemmArgs s{};
    s.A = panel; s.lda = d;
    s.B = panel; s.ldb = d;
    s.C = A + (int64_t)(o + m) * d + (o + m); s.ldc = d;
    s.M = rest; s.N = rest; s.K = m;
    s.alpha = -1.0; s.beta = 1.0;
    s.tri_tiles = 1;
    s.kmode = KMODE_FULL;
    e = dgemm_launch(s, false, true, 1, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// L (lower, in A, diagonal blocks already replaced by their inverses) -> L^-1 in place. T is scratch of
// at least d*d doubles. Level s joins diagonal blocks of size s into 2s:
//   [L11 0; L21 L22]^-1 = [L11^-1 0; -L22^-1 L21 L11^-1  L22^-1]
hipError_t trtri_lower(double* A, int d, double* T, hipStream_t stream) {
  for (int s = NB; s < d; s *= 2) {
    const int pairs = (d - s + 2 * s - 1) / (2 * s);
    // T_p = L21_p * Li11_p  (Li11 lower: k >= j)
    DgemmArgs g1{};
    g1.A = A + (int64_t)s * d; g1.lda = d; g1.strideA = (int64_t)2 * s * d + 2 * s;
    g1.B = A; g1.ldb = d; g1.strideB = (int64_t)2 * s * d + 2 * s;
    g1.C = T; g1.ldc = s; g1.strideC = (int64_t)s * s;
    g1.M = s; g1.N = s; g1.K = s;
    g1.m_lim = d - s; g1.m_step = 2 * s;
    g1.alpha = 1.0; g1.beta = 0.0;
    g1.kmode = KMODE_GE_J;
    hipError_t e = dgemm_launch(g1, false, false, pairs, stream);
    if (e != hipSuccess) return e;
    // L21_p <- -Li22_p * T_p  (Li22 lower: k <= i; K limited to the block's rows)
    DgemmArgs g2{};
    g2.A = A + (int64_t)s * d + s; g2.lda = d; g2.strideA = (int64_t)2 * s * d + 2 * s;
    g2.B = T; g2.ldb = s; g2.strideB = (int64_t)s * s;
    g2.C = A + (int64_t)s * d; g2.ldc = d; g2.strideC = (int64_t)2 * s * d + 2 * s;
    g2.M = s; g2.N = s; g2.K = s;
    g2.m_lim = d - s; g2.m_step = 2 * s;
    g2.k_by_m = 1;
    g2.alpha = -1.0; g2.beta = 0.0;
    g2.kmode = KMODE_LT_I_END;
    e = dgemm_launch(g2, false, false, pairs, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t prepare_ws_bytes(int64_t in) {
  const int64_t d = in;
  const int64_t nblk = ceil_div(d, NB);
  size_t b = 0;
  b += align_up((size_t)d * d * sizeof(double), 256);          // A
  b += align_up((size_t)nblk * NB * NB * sizeof(double), 256);  // Dinv
  b += align_up((size_t)d * sizeof(double), 256);              // diag of H
  b += 256;                                                    // status
  return b;
}

hipError_t prepare_launch(const double* S, const double* colsq, int64_t n_total, int64_t in, double damp,
                          int act_order, unsigned flags, double* U, int32_t* perm, uint8_t* dead, void* ws,
                          hipStream_t stream, unsigned* host_status) {
  const int d = (int)in;
  const int64_t nblk = ceil_div(d, NB);
  char* w = reinterpret_cast<char*>(ws);
  double* A = reinterpret_cast<double*>(w);
  w += align_up((size_t)d * d * sizeof(double), 256);
  double* Dinv = reinterpret_cast<double*>(w);
  w += align_up((size_t)nblk * NB * NB * sizeof(double), 256);
  double* diag_h = reinterpret_cast<double*>(w);
  w += align_up((size_t)d * sizeof(double), 256);
  unsigned* status = reinterpret_cast<unsigned*>(w);
  const bool reversed = (flags & GPTQ_FACTOR_REVERSED) != 0;

  hipError_t e;
#define GPTQ_TRY(x)          \
  do {                       \
    e = (x);                 \
    if (e != hipSuccess) return e; \
  } while (0)

  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, stream, status);
  GPTQ_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_prep_stats, dim3(1), dim3(1024), 0, stream, colsq, n_total, d, damp, diag_h, dead, status);
  GPTQ_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_perm, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, stream, colsq, d, act_order, perm);
  GPTQ_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_gather, dim3((unsigned)(ceil_div(d, 256) * d)), dim3(256), 0, stream, S, diag_h, perm, n_total,
                     d, reversed ? 1 : 0, A);
  GPTQ_TRY(hipGetLastError());

  GPTQ_TRY(potrf_lower(A, d, Dinv, status, stream));
  hipLaunchKernelGGL(k_place_dinv, dim3((unsigned)nblk), dim3(256), 0, stream, Dinv, A, (int64_t)d, d);
  GPTQ_TRY(hipGetLastError());
  GPTQ_TRY(trtri_lower(A, d, U /* scratch */, stream));
  if (reversed) {
    hipLaunchKernelGGL(k_reverse_to_upper, dim3((unsigned)(ceil_div(d, 256) * d)), dim3(256), 0, stream, A, d, U);
    GPTQ_TRY(hipGetLastError());
  } else {
    // H^-1 = Li^T Li (lower tiles) into U, then its Cholesky factor, then U = Lu^T
    DgemmArgs g{};
    g.A = A; g.lda = d;
    g.B = A; g.ldb = d;
    g.C = U; g.ldc = d;
    g.M = d; g.N = d; g.K = d;
    g.alpha = 1.0; g.beta = 0.0;
    g.tri_tiles = 1;
    g.kmode = KMODE_GE_I;
    GPTQ_TRY(dgemm_launch(g, true, false, 1, stream));
    GPTQ_TRY(potrf_lower(U, d, Dinv, status, stream));
    const int nt = (d + 31) / 32;
    hipLaunchKernelGGL(k_transpose_lower_to_upper, dim3(nt * (nt + 1) / 2), dim3(256), 0, stream, U, d);
    GPTQ_TRY(hipGetLastError());
  }
  GPTQ_TRY(hipMemcpyAsync(host_status, status, sizeof(unsigned), hipMemcpyDeviceToHost, stream));
  GPTQ_TRY(hipStreamSynchronize(stream));
#undef GPTQ_TRY
  return hipSuccess;
}

}  // namespace gptq
