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
  int tri_tiles;  // only tiles with I >= J (square C)
  int lower_only; // rectangular C whose origin lies on a diagonal: tiles with I < J are skipped
  int kmode;
  int m_lim, m_step;  // when m_step != 0: rows of batch b = min(M, m_lim - b * m_step)
  int k_by_m;         // K of each batch equals its row count (square triangular A)
  // When fuse_diag is set (A B^T products only), the workgroup of tile (0, 0) then factors the 64 x 64
  // diagonal block diag_kb of diag_A (which that tile has just written) and stores its inverse in
  // diag_Dinv, flagging bad pivots in diag_status, while the other tiles are still being computed.
  int fuse_diag;
  double* diag_A;
  int diag_d, diag_kb;
  double* diag_Dinv;
  unsigned* diag_status;
};

hipError_t dgemm_launch(const DgemmArgs& a, bool ta, bool tb, int batches, hipStream_t stream);

}  // namespace gptq
