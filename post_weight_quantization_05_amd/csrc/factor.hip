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
//  k_colstep      (dgemm.hip) one 64-column step of the blocked factorization: block-column update,
//                 the next 64 x 64 diagonal block factored and inverted in 16-column sub-blocks
//                 (diagblock.h), the next panel solved on the matrix cores; flags pivots that are
//                 not > 0 or not finite. Its spare workgroups carry deferred trailing-update tiles and
//                 the tiles of L^-1 (InvFill in dgemm.h), two steps behind the factorization.
//  k_inv_fill     (dgemm.hip) the last tiles of L^-1, after the last step.
//  k_place_lblocks the staged factors of the diagonal blocks into A.
//  trailing SYRK updates and H^-1 = L^-T L^-1 use the fp64 MFMA GEMM core (dgemm.hip).
// Routes (flags): INVERSE_RECHOL = potrf with L^-1, lauum, potrf, transpose (the guide's order);
// REVERSED = potrf with L^-1 of J H J, then U = J L^-1 J (same unique U, half the work).
// R_FORM = potrf of J H J without L^-1, then R = J L J (= U^-1) and U's 128 x 128 diagonal blocks, the
// inverses of R's, from the steps' 64 x 64 diagonal inverses (k_rform_diag), for the R route of the loop.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "dgemm.h"
#include "diagblock.h"

namespace gptq {

namespace {

using diagblock::NB;

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
// fixed, damped). One 64 x 64 tile of A per workgroup, staged through LDS: without act_order the source
// of a tile is one 64 x 64 block of S, and threads walk along S's rows (along A's columns when A is in
// S's order, along A's rows when reversed), so reads and writes are both coalesced.
__global__ __launch_bounds__(256) void k_gather(const double* __restrict__ S, const double* __restrict__ diag_h,
                                                const int32_t* __restrict__ perm, int64_t n_total, int d,
                                                int reversed, double* __restrict__ A) {
  __shared__ double t[64][65];
  const int a0 = blockIdx.y * 64, b0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const double s2n = 2.0 / (double)n_total;
  if (b0 > a0) {  // strictly upper tile
    for (int aa = ty; aa < 64; aa += 4) {
      const int a = a0 + aa, b = b0 + tx;
      if (a < d && b < d) A[(int64_t)a * d + b] = 0.0;
    }
    return;
  }
  // the thread's 16 elements: (a0 + tx, b0 + ty + 4k) when reversed ((a, b) reads S[d-1-b][d-1-a], so
  // consecutive a are consecutive addresses), else (a0 + ty + 4k, b0 + tx). Every load is issued before
  // its values are needed (indices clamped into range, values selected afterwards): the permutation
  // entries of all 16, then their S and diagonal entries, two round trips to memory instead of two per
  // element.
  constexpr int NE = 16;
  int pi[NE], pj[NE];
  bool ok[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int a = reversed ? a0 + tx : a0 + ty + 4 * k;
    const int b = reversed ? b0 + ty + 4 * k : b0 + tx;
    ok[k] = a < d && b < d && b <= a;
    const int x = ok[k] ? (reversed ? d - 1 - a : a) : 0;
    const int y = ok[k] ? (reversed ? d - 1 - b : b) : 0;
    pi[k] = perm[x];
    pj[k] = perm[y];
  }
  double sv[NE], dv[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int p = min(max(pi[k], 0), d - 1), q = min(max(pj[k], 0), d - 1);
    pi[k] = p;
    pj[k] = q;
    sv[k] = S[(int64_t)max(p, q) * d + min(p, q)];
    dv[k] = diag_h[p];
  }
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const double v = ok[k] ? (pi[k] == pj[k] ? dv[k] : s2n * sv[k]) : 0.0;
    if (reversed) t[ty + 4 * k][tx] = v;
    else t[tx][ty + 4 * k] = v;
  }
  __syncthreads();
  for (int aa = ty; aa < 64; aa += 4) {
    const int a = a0 + aa, b = b0 + tx;
    if (a < d && b < d) A[(int64_t)a * d + b] = t[tx][aa];
  }
}

// Copy the staged factors of the diagonal blocks into the diagonal of A (lower part, zeros above).
__global__ __launch_bounds__(256) void k_place_lblocks(const double* __restrict__ Lst, double* __restrict__ A,
                                                       int64_t lda, int d) {
  const int kb = blockIdx.x;
  const int o = kb * NB;
  const int m = min(NB, d - o);
  const double* Lb = Lst + (int64_t)kb * NB * NB;
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int i = e / NB, j = e % NB;
    if (i < m && j < m) A[(int64_t)(o + i) * lda + o + j] = Lb[e];
  }
}

// Copy the inverted diagonal blocks into the diagonal of A (start of the level-wise triangular inverse).
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

// U[a][b] = Li[d-1-a][d-1-b] for a <= b, 0 below the diagonal. Grid: x = 256-column blocks of a row,
// y = rows in a grid-stride loop (the grid stays small at any d).
__global__ __launch_bounds__(256) void k_reverse_to_upper(const double* __restrict__ Li, int d,
                                                          double* __restrict__ U) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= d) return;
  for (int a = blockIdx.y; a < d; a += gridDim.y)
    U[(int64_t)a * d + b] = (b >= a) ? Li[(int64_t)(d - 1 - a) * d + (d - 1 - b)] : 0.0;
}

// Blocked right-looking Cholesky in two levels. Inside an outer block column of NBO columns, each
// 64-column step is one launch (k_colstep): the outer block's remaining columns get the previous
// panel's update (K = 64), the next diagonal block is factored and inverted, and the next panel is
// solved against it. The outer block's whole panel (K = NBO) updates the trailing matrix: the next outer
// block's columns in that block's first step launch (its own tiles, before its diagonal block is
// factored), the rest as deferred tiles inside the next outer block's steps. Near the end of the matrix
// (GPTQ_FACTOR_LOOKAHEAD_ROWS) an outer block's steps also update the next block's columns with each
// panel once it is solved, so that block's first step takes only the last 64 columns of the panel
// before it (K = 64); those steps run only after the deferred tiles of the same columns are done (they
// come first in column order and all go to the first step). The factors of the diagonal blocks are
// staged in Lst and copied into A at the end (A's diagonal block is read by several workgroups of the
// launch that factors it).
#ifndef GPTQ_FACTOR_NBO
#define GPTQ_FACTOR_NBO 256
#endif
constexpr int NBO = GPTQ_FACTOR_NBO;  // outer block width (a multiple of 64)
static_assert(NBO == 256, "an outer block's panel is the K of its successor's first step launch (64 or 256)");
// Deferred trailing tiles per block-column step: with L^-1 in the steps (two workgroups per CU carrying
// it) 640 (prepare at in = 4096: 2.92 ms against 3.00 with 160); without, 160 (in = 8192 / 11008: 13.7 /
// 29.0 ms against 14.0 / 29.9 with 640).
#ifndef GPTQ_FACTOR_DEFER
#define GPTQ_FACTOR_DEFER 160
#endif
// The R form's steps carry no L^-1: 640 deferred tiles per step up to in = 6144, 320 above (in = 4096:
// 2.49 ms with 640, 2.52 with 320; in = 11008: 18.3 ms with 320, 18.7 with 640, 18.6 with 160).
#ifndef GPTQ_FACTOR_DEFER_RFORM
#define GPTQ_FACTOR_DEFER_RFORM 640
#endif
#ifndef GPTQ_FACTOR_DEFER_RFORM_LARGE
#define GPTQ_FACTOR_DEFER_RFORM_LARGE 320
#endif
#ifndef GPTQ_FACTOR_DEFER_FILL
#define GPTQ_FACTOR_DEFER_FILL 640
#endif
// An outer block's steps also update the next outer block's columns (one 64-column panel per step, so
// that block's first step takes K = 64 instead of the whole panel before it) once at most this many
// rows lie below the next block's start: there the steps are bound by their chain of diagonal blocks
// and the extra K = 64 tiles fill idle CUs, while higher up the steps are bound by their tiles, which
// then read and write the next block's columns four times instead of once.
// Prepare (ms) at in = 4096 / 8192 / 11008, R form: 2.353 / 8.92 / 18.04 with 2048, 2.350 / 8.92 / 18.06
// with 3072, 2.358 / 9.25 / 18.45 with every block looking ahead, 2.449 / 9.02 / 18.06 with none.
#ifndef GPTQ_FACTOR_LOOKAHEAD_ROWS
#define GPTQ_FACTOR_LOOKAHEAD_ROWS 2048
#endif

// place_l: copy the diagonal blocks' factors into A at the end.
// Z, G (both null, or Z d x d and G two buffers of 64 rows per block x 64): also form Z = L^-1 (lower part)
// with the steps' idle CUs (InvFill in dgemm.h), finished by three launches after the last step.
hipError_t potrf_lower(double* A, int d, double* Dinv, double* Lst, unsigned* status, bool place_l, double* Z,
                       double* G, hipStream_t stream, int defer = -1) {
  const int S = (d + NB - 1) / NB;
  InvFill inv{};
  inv.L = A;
  inv.Dinv = Dinv;
  inv.Z = Z;
  inv.G[0] = G;
  inv.G[1] = G ? G + (int64_t)S * NB * NB : nullptr;
  inv.d = d;
  inv.S = S;
  const int defer_per_step = defer >= 0 ? defer : Z ? GPTQ_FACTOR_DEFER_FILL : GPTQ_FACTOR_DEFER;
  // The trailing update of an outer block is split in two: the next outer block's columns in that block's
  // first step (or panel by panel in this block's steps, near the end), the rest (columns from the block
  // after that on) as one K = NBO product deferred and spread over the next outer block's steps as extra
  // workgroups.
  // deferred part of the previous outer block's trailing update: its tiles in column order (tri_tiles = 2)
  // when the block that takes them looks ahead, else in row order (faster there: 18.06 against 18.20 ms
  // for the R form's prepare at in = 11008)
  DgemmArgs pend{};
  int pend_tiles = 0, pend_done = 0;
  // one block-column step: update C = A[c1:, c1:c1 + n] with the panel A[c1:, o:o + k] (k = 0: no
  // update), factor the diagonal block at (c1, c1), solve the panel below it; plus `share` deferred tiles
  auto colstep = [&](int c1, int n, int o, int k, int share) {
    DgemmArgs s{};
    const double* P = A + (int64_t)c1 * d + o;
    s.A = P; s.lda = d;
    s.B = P; s.ldb = d;
    s.C = A + (int64_t)c1 * d + c1; s.ldc = d;
    s.M = d - c1; s.N = n; s.K = k;
    s.alpha = -1.0; s.beta = 1.0;
    s.kmode = KMODE_FULL;
    s.diag_kb = c1 / NB; s.diag_Lstage = Lst; s.diag_Dinv = Dinv; s.diag_status = status;
    share = min(share, pend_tiles - pend_done);
    inv.k = c1 / NB;
    const hipError_t e = colstep_launch(s, &pend, pend_done, share, Z ? &inv : nullptr, stream);
    pend_done += share;
    return e;
  };
  hipError_t e;
  bool prev_look = false;
  for (int b0 = 0; b0 < d; b0 += NBO) {
    const int b1 = min(d, b0 + NBO);
    const int b2 = min(d, b1 + NBO);  // end of the next outer block's columns
    const bool look = b1 < d && d - b1 <= GPTQ_FACTOR_LOOKAHEAD_ROWS;  // steps update [b1, b2) too
    const int steps = (b1 - b0 + NB - 1) / NB;
    // the deferred tiles are shared out evenly over this outer block's steps (all of them by its end)
    int step = 0;
    auto share = [&]() {
      const int left = pend_tiles - pend_done, rem = steps - step++;
      return (left + rem - 1) / rem;
    };
    // with look, the deferred tiles of the next outer block's columns (the first tile columns in column
    // order) all go to the first step, since the steps after it update those columns themselves
    const int pend_nt = (pend.M + NB - 1) / NB, strip_cols = min(pend_nt, NBO / NB);
    const int strip = look && pend_tiles > 0
                          ? min(pend_tiles, strip_cols * pend_nt - strip_cols * (strip_cols - 1) / 2) : 0;
    // first block of the outer block column: the update of the whole outer block by the last panel of
    // the previous one (by the whole previous panel, K = NBO, if the previous block's steps did not look
    // ahead; none for the first outer block), its diagonal block and its panel
    if (b0 == 0) e = colstep(b0, min(NB, d - b0), b0, 0, share());
    else if (prev_look) e = colstep(b0, b1 - b0, b0 - NB, NB, max(share(), strip));
    else e = colstep(b0, b1 - b0, b0 - NBO, NBO, max(share(), strip));
    if (e != hipSuccess) return e;
    const int cend = look ? b2 : b1;
    for (int o = b0; o + NB < b1; o += NB) {
      // the outer block's remaining columns (and with look the next block's) get panel o; the next block
      // is factored and its panel solved
      const int c1 = o + NB;
      e = colstep(c1, cend - c1, o, NB, share());
      if (e != hipSuccess) return e;
    }
    prev_look = look;
    pend_tiles = pend_done = 0;
    pend = DgemmArgs{};
    if (b1 < d) {
      // trailing update with the whole outer panel Q = A[b1:, b0:b1]: A22 -= Q Q^T (lower part). The next
      // outer block's columns have it by the end of that block's first step; the rest is deferred.
      if (b2 < d) {  // the rest, deferred
        pend = DgemmArgs{};
        const double* Q2 = A + (int64_t)b2 * d + b0;
        pend.A = Q2; pend.lda = d;
        pend.B = Q2; pend.ldb = d;
        pend.C = A + (int64_t)b2 * d + b2; pend.ldc = d;
        pend.M = d - b2; pend.N = d - b2; pend.K = b1 - b0;
        pend.alpha = -1.0; pend.beta = 1.0;
        pend.kmode = KMODE_FULL;
        pend.tri_tiles = d - b2 <= GPTQ_FACTOR_LOOKAHEAD_ROWS ? 2 : 1;  // the look of the block [b1, b2)
        const int nt = (pend.M + NB - 1) / NB;
        const int all = nt * (nt + 1) / 2;
        // the next outer block's steps take as many as they can hide (about one tile per CU that a
        // step leaves idle); the remaining tiles are launched now as a product of their own
        const int next_steps = (b2 - b1 + NB - 1) / NB;
        pend_tiles = min(all, next_steps * defer_per_step);
        if (pend_tiles < all) {
          DgemmArgs r = pend;
          r.tile_first = pend_tiles;
          e = dgemm_launch(r, false, true, 1, stream);
          if (e != hipSuccess) return e;
        }
      }
    }
  }
  if (Z) {
    for (inv.k = S; inv.k < S + 3; ++inv.k) {
      e = inv_fill_launch(inv, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (!place_l) return hipSuccess;
  const int nblk = (d + NB - 1) / NB;
  hipLaunchKernelGGL(k_place_lblocks, dim3(nblk), dim3(256), 0, stream, Lst, A, (int64_t)d, d);
  return hipGetLastError();
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

// L^-1 two ways: for in <= FILL_MAX as tiles carried by the factorization's steps (their idle CUs hold
// it: d^2 of spare workgroup slots against d^3 / 3 flops), above it as the level-wise doubling after the
// factorization (its large products run nearer the GEMM core's rate, and the step launches would
// otherwise grow longer than they save). Measured prepare (ms), steps / levels: in = 2048 1.17 / 1.45,
// 4096 2.92 / 3.37, 6144 7.43 / 7.44, 8192 15.8 / 13.7, 11008 38.8 / 29.0.
#ifndef GPTQ_FACTOR_FILL_MAX
#define GPTQ_FACTOR_FILL_MAX 6144
#endif
constexpr int FILL_MAX = GPTQ_FACTOR_FILL_MAX;

}  // namespace

size_t prepare_ws_bytes(int64_t in) {
  const int64_t d = in;
  const int64_t nblk = ceil_div(d, NB);
  size_t b = 0;
  b += align_up((size_t)d * d * sizeof(double), 256);          // A
  b += align_up((size_t)d * d * sizeof(double), 256);          // Z = L^-1
  b += align_up((size_t)2 * nblk * NB * NB * sizeof(double), 256);  // G (two buffers)
  b += align_up((size_t)nblk * NB * NB * sizeof(double), 256);  // Dinv
  b += align_up((size_t)nblk * NB * NB * sizeof(double), 256);  // staged factors of the diagonal blocks
  b += align_up((size_t)d * sizeof(double), 256);              // diag of H
  b += 256;                                                    // status
  return b;
}

// The R form's diagonal blocks (see GPTQ_FACTOR_R_FORM): for the quantization panel [b0, b0 + pw) the inverse
// of L's diagonal block over the reversed rows [s, s + pw), s = in - b0 - pw, goes into the strictly lower part
// of the output's diagonal block, unreversed (output (b0 + r, b0 + c) = (L_ss^-1)[r][c], r > c): that is
// J U_PP J. With in % 64 == 0, s is a multiple of 64 and the block is one or two of the factorization's
// 64 x 64 diagonal blocks, whose inverses the steps left in Dinv; for two,
//   [A 0; B C]^-1 = [A^-1 0; -C^-1 B A^-1  C^-1],
// the off-diagonal part formed here in fp64 on the matrix cores (one workgroup per panel, B A^-1 and then
// C^-1 (B A^-1), the k-steps above C^-1's diagonal skipped).
__global__ __launch_bounds__(256) void k_rform_diag(const double* __restrict__ L, const double* __restrict__ Dinv,
                                                    int d, double* __restrict__ M) {
  __shared__ double Ai[NB][NB + 1], Ci[NB][NB + 1], Bb[NB][NB + 1], Y[NB][NB + 1];
  const int b0 = blockIdx.x * 128;
  const int pw = min(128, d - b0);
  const int s = d - b0 - pw;
  const int kb = s / NB;
  const int tid = threadIdx.x;
  double* out = M + (int64_t)b0 * d + b0;
  auto put = [&](int r, int c, double v) { out[(int64_t)r * d + c] = v; };
  // the diagonal 64 x 64 inverses, strictly lower parts (the blocks are lower; zeros are staged above).
  // All of a thread's loads are issued first (the second block's with clamped addresses when pw < 128).
  constexpr int NE = NB * NB / 256;
  const bool two = pw == 128;
  double av[NE], cv[NE], bv[NE];
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int e = tid + 256 * q, r = e / NB, c = e % NB;
    av[q] = Dinv[(int64_t)kb * NB * NB + e];
    cv[q] = Dinv[(int64_t)(two ? kb + 1 : kb) * NB * NB + e];
    bv[q] = L[(int64_t)(two ? s + NB + r : s + r) * d + s + c];
  }
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int e = tid + 256 * q, r = e / NB, c = e % NB;
    if (r > c) put(r, c, av[q]);
    Ai[r][c] = (r >= c) ? av[q] : 0.0;
    if (two) {
      if (r > c) put(NB + r, NB + c, cv[q]);
      Ci[r][c] = (r >= c) ? cv[q] : 0.0;
      Bb[r][c] = bv[q];
    }
  }
  if (!two) return;
  __syncthreads();
  // both 64 x 64 x 64 products on the matrix cores: wave wv forms the 16 rows 16 wv .. 16 wv + 15 of the
  // result in four 16 x 16 blocks (v_mfma_f64_16x16x4f64: lane l supplies the left operand's
  // [l % 16][k0 + l / 16] and the right operand's [k0 + l / 16][l % 16]; accumulator entry e of lane l is
  // row 4e + l / 16, column l % 16 of the block)
  const int lane = tid & 63, wv = tid >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  f64x4 acc[4];
  // Y = B A^-1
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < NB; k0 += 4) {
    const double av = Bb[16 * wv + lr][k0 + lk];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = diagblock::mfma16(av, Ai[k0 + lk][16 * q + lr], acc[q]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) Y[16 * wv + 4 * e + lk][16 * q + lr] = acc[q][e];
  __syncthreads();
  // X21 = -C^-1 Y (C^-1 lower: the wave's rows need k < 16 wv + 16)
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < 16 * wv + 16; k0 += 4) {
    const double av = Ci[16 * wv + lr][k0 + lk];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = diagblock::mfma16(av, Y[k0 + lk][16 * q + lr], acc[q]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) put(NB + 16 * wv + 4 * e + lk, 16 * q + lr, -acc[q][e]);
}

hipError_t prepare_launch(const double* S, const double* colsq, int64_t n_total, int64_t in, double damp,
                          int act_order, unsigned flags, double* U, int32_t* perm, uint8_t* dead, void* ws,
                          hipStream_t stream, unsigned* host_status) {
  const int d = (int)in;
  const int64_t nblk = ceil_div(d, NB);
  char* w = reinterpret_cast<char*>(ws);
  double* A = reinterpret_cast<double*>(w);
  w += align_up((size_t)d * d * sizeof(double), 256);
  double* Z = reinterpret_cast<double*>(w);
  w += align_up((size_t)d * d * sizeof(double), 256);
  double* G = reinterpret_cast<double*>(w);
  w += align_up((size_t)2 * nblk * NB * NB * sizeof(double), 256);
  double* Dinv = reinterpret_cast<double*>(w);
  w += align_up((size_t)nblk * NB * NB * sizeof(double), 256);
  double* Lst = reinterpret_cast<double*>(w);
  w += align_up((size_t)nblk * NB * NB * sizeof(double), 256);
  double* diag_h = reinterpret_cast<double*>(w);
  w += align_up((size_t)d * sizeof(double), 256);
  unsigned* status = reinterpret_cast<unsigned*>(w);
  const bool reversed = (flags & GPTQ_FACTOR_INVERSE_RECHOL) == 0;

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
  hipLaunchKernelGGL(k_gather, dim3((unsigned)ceil_div(d, 64), (unsigned)ceil_div(d, 64)), dim3(256), 0, stream, S, diag_h, perm, n_total,
                     d, reversed ? 1 : 0, A);
  GPTQ_TRY(hipGetLastError());

  if (flags == GPTQ_FACTOR_R_FORM) {
    // R = J L J (L placed in A), then the inverses of its 128 x 128 diagonal blocks in their lower parts
    GPTQ_TRY(potrf_lower(A, d, Dinv, Lst, status, true, nullptr, G, stream,
                         d <= FILL_MAX ? GPTQ_FACTOR_DEFER_RFORM : GPTQ_FACTOR_DEFER_RFORM_LARGE));
    hipLaunchKernelGGL(k_reverse_to_upper, dim3((unsigned)ceil_div(d, 256), (unsigned)std::min(d, 4096)), dim3(256),
                       0, stream, A, d, U);
    GPTQ_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_rform_diag, dim3((unsigned)ceil_div(d, 128)), dim3(256), 0, stream, A, Dinv, d, U);
    GPTQ_TRY(hipGetLastError());
    GPTQ_TRY(hipMemcpyAsync(host_status, status, sizeof(unsigned), hipMemcpyDeviceToHost, stream));
    GPTQ_TRY(hipStreamSynchronize(stream));
    return hipSuccess;
  }
  const bool fill = d <= FILL_MAX;
  GPTQ_TRY(potrf_lower(A, d, Dinv, Lst, status, false, fill ? Z : nullptr, G, stream));
  double* Li = Z;  // L^-1 (lower part)
  if (!fill) {
    hipLaunchKernelGGL(k_place_dinv, dim3((unsigned)nblk), dim3(256), 0, stream, Dinv, A, (int64_t)d, d);
    GPTQ_TRY(hipGetLastError());
    GPTQ_TRY(trtri_lower(A, d, Z /* scratch */, stream));
    Li = A;
  }
  if (reversed) {
    hipLaunchKernelGGL(k_reverse_to_upper, dim3((unsigned)ceil_div(d, 256), (unsigned)std::min(d, 4096)), dim3(256),
                       0, stream, Li, d, U);
    GPTQ_TRY(hipGetLastError());
  } else {
    // H^-1 = Li^T Li (lower tiles) into U, then its Cholesky factor, then U = Lu^T
    DgemmArgs g{};
    g.A = Li; g.lda = d;
    g.B = Li; g.ldb = d;
    g.C = U; g.ldc = d;
    g.M = d; g.N = d; g.K = d;
    g.alpha = 1.0; g.beta = 0.0;
    g.tri_tiles = 1;
    g.kmode = KMODE_GE_I;
    GPTQ_TRY(dgemm_launch(g, true, false, 1, stream));
    GPTQ_TRY(potrf_lower(U, d, Dinv, Lst, status, true, nullptr, nullptr, stream));
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
