// fp64 tiled GEMM core shared by the factorization and the quantize loop (see dgemm.hip).
#pragma once
#include "common.h"

namespace gptq {

enum : int {
  KMODE_FULL = 0,      // k in [0, K)
  KMODE_GE_J = 1,      // k >= first column of the tile (B lower triangular)
  KMODE_LT_I_END = 2,  // k < last row of the tile + 1 (A lower triangular)
  KMODE_GE_I = 3,      // k >= first row of the tile (opA = A^T with A lower triangular)
};

struct DgemmArgs {
  const double* A;
  int64_t lda, strideA;
  const double* B;
  int64_t ldb, strideB;
  double* C;
  int64_t ldc, strideC;
  int M, N, K;
  double alpha, beta;
  int tri_tiles;  // only tiles with I >= J (square C): 1 counted in row order, 2 in column order
  int tile_first; // tri_tiles: launch covers lower tiles tile_first, tile_first + 1, ... in that order
  int lower_only; // rectangular C whose origin lies on a diagonal: tiles with I < J are skipped
  int kmode;
  int m_lim, m_step;  // when m_step != 0: rows of batch b = min(M, m_lim - b * m_step)
  int k_by_m;         // K of each batch equals its row count (square triangular A)
  // Block-column step of the factorization (colstep_launch only): the next diagonal block is block
  // diag_kb; its L goes to diag_Lstage[diag_kb], its L^-1 to diag_Dinv[diag_kb] (64 x 64 each), bad
  // pivots to diag_status.
  int diag_kb;
  double* diag_Lstage;
  double* diag_Dinv;
  unsigned* diag_status;
};

// C = alpha op(A) op(B) + beta C on 64 x 64 tiles. Single plain products op(B) = B take kernels of their own:
// K <= 128 with at most 1024 tiles (no lower_only) a kernel that keeps a whole tile's operands in flight,
// K >= 256 (a multiple of 16, even N) with at least 512 tiles of 128 x 128 the 128 x 128 kernel. Everything
// else (batches, triangular K ranges, tile lists, op(A) = A^T, op(B) = B^T, other sizes) takes the
// chunked-ring GEMM.
hipError_t dgemm_launch(const DgemmArgs& a, bool ta, bool tb, int batches, hipStream_t stream);
// The inverse Z = L^-1 of the factor, formed by the block-column steps as work that fills the CUs their
// chain leaves idle (see inv_fill_tile in dgemm.hip). Row block t of L Z = I is eliminated right-looking:
//   G_{i,t} = L_{i,t} L_tt^-1 for the blocks i > t below step t (launch t + 1),
//   Z_{i,j} -= G_{i,t} Z_{t,j} for j < t, Z_{i,t} = -G_{i,t} (launch t + 2; Z holds unscaled rows),
//   Z_{t,j} = L_tt^-1 Z_{t,j} for j < t, Z_{t,t} = L_tt^-1 (launch t + 3),
// where launch k is the step that factors diagonal block k, and launches S .. S + 2 (S = number of
// 64-blocks) come after the last step. Every input of a launch's tiles is final by the end of the
// launch before it.
struct InvFill {
  const double* L;     // the matrix being factored (its lower part is L once the step has passed), ld d
  const double* Dinv;  // the steps' diagonal-block inverses, 64 x 64 row-major each
  double* Z;           // d x d, ld d; its lower part becomes L^-1
  double* G[2];        // d x 64 each, used in turn by steps of even and odd t
  int d, S;
  int k;               // the launch
};
int inv_fill_tiles(const InvFill& f);
// One block-column step of the blocked Cholesky factorization (see k_colstep in dgemm.hip): C -= A B^T
// on the lower tiles of the M x N region C, the diagonal block at its origin factored and inverted, and
// the column-0 tiles below it solved against that factor; K is 0, 64 or 256. The same launch also
// computes lower tiles x_first .. x_first + x_count - 1 (in column order if x->tri_tiles is 2, else in
// row order) of x, an independent A B^T update of a square region (x may be null when x_count is 0),
// and, when f is not null, the tiles of launch f->k of the inverse.
hipError_t colstep_launch(const DgemmArgs& a, const DgemmArgs* x, int x_first, int x_count, const InvFill* f,
                          hipStream_t stream);
// The inverse's tiles of a launch after the last step (f.k = S, S + 1, S + 2).
hipError_t inv_fill_launch(const InvFill& f, hipStream_t stream);

}  // namespace gptq
