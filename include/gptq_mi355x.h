/*
 * gptq_mi355x.h - C ABI of libgptq_mi355x.so: GPTQ per-layer weight quantization on one MI355X (gfx950).
 *
 * The layer problem (GPTQ guide, herodthegreater.github.io/pigeon/guide/gptq/, "How it works"; and the
 * lesson "GPTQ's error-compensation loop", herodthegreater.github.io/pigeon/school/gptq_loop/):
 * weights W (out x in), calibration inputs X (n x in), a symmetric b-bit grid with qmax = 2^(b-1) - 1,
 * optional groups of `group` input columns with their own scales, damping `damp`, optional act_order.
 * The path is three calls, each stream-ordered on the caller's HIP stream:
 *
 *   1. gptq_hessian_accumulate  S += X^T X, colsq += column sums of squares, n_total += rows
 *   2. gptq_prepare_chol        H = 2 S / n_total, dead inputs, damping, act_order permutation,
 *                               U = upper Cholesky factor of H^-1 (H^-1 = U^T U)
 *   3. gptq_quantize_layer      the column-by-column error-compensation loop -> integer codes,
 *                               scales and (optionally) g_idx and the per-row loss
 *
 * Conventions shared by every call
 *  - All matrices are row-major. Every pointer to matrix/vector data is a DEVICE pointer unless stated
 *    otherwise; `n_total` is the only host pointer.
 *  - The caller owns every buffer, workspace included. The library allocates no device memory, frees
 *    nothing and keeps no pointer after a call returns. Workspaces are sized by the *_workspace_bytes
 *    queries and need no initialisation. Their contents after a call are unspecified.
 *  - `stream` is a hipStream_t (NULL = the null stream). Call 1 is fully asynchronous; calls 2 and 3
 *    synchronise `stream` once, at their end, to read a 4-byte status word written by their kernels.
 *  - Every call returns a gptq_status. On an argument error nothing is launched and no output is
 *    written. Calls on different streams with disjoint buffers are independent; the library has no
 *    global mutable state.
 *  - W and X are read only. The library works on its own fp64 copy of W in the workspace.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = -1, /* bad size, pointer, dtype, bits, damp or leading dimension */
  GPTQ_ERR_UNSUPPORTED = -2, /* valid request this library does not implement (group size, see below) */
  GPTQ_ERR_NOT_SPD = -3,     /* the damped Hessian has no Cholesky factor (a pivot below 2^-1000) */
  GPTQ_ERR_NONFINITE = -4,   /* NaN or Inf met in S, colsq or during the factorization */
  GPTQ_ERR_WORKSPACE = -5,   /* ws is NULL or ws_bytes is below the size query's value */
  GPTQ_ERR_HIP = -6          /* a HIP runtime call or kernel launch failed */
} gptq_status;

typedef enum { GPTQ_F32 = 0, GPTQ_BF16 = 1 } gptq_dtype;

/* Factorization route for gptq_prepare_chol (`flags`).
 *  GPTQ_FACTOR_REVERSED (0, the default): U = J chol(J H J)^-1 J with J the index reversal: one Cholesky
 *    factorization and one triangular inverse. It is the unique U (upper, positive diagonal,
 *    U^T U = H^-1) because H = V V^T with V = U^-1 upper, and J V J is lower.
 *  GPTQ_FACTOR_INVERSE_RECHOL (1): L = chol(H); L^-1; H^-1 = L^-T L^-1; U = (chol(H^-1))^T, the order the
 *    guide's _hessian_inverse_chol takes ("The code, line by line"), at twice the flops. */
#define GPTQ_FACTOR_REVERSED 0u
#define GPTQ_FACTOR_INVERSE_RECHOL 1u
/* GPTQ_FACTOR_R_FORM (2): instead of U, the factor form that gptq_quantize_layer_r reads (the same route
 *    without the triangular inverse). R = U^-1 = J chol(J H J) J is upper triangular with R R^T = H (P^T H P
 *    with act_order): its upper triangle, diagonal included, holds R. The loop also needs U's 128 x 128
 *    diagonal blocks, which are the inverses of R's: for the block of columns [b, b + p) (b a multiple of
 *    128, p = min(128, in - b)) the strictly lower part of that diagonal block holds J U_bb J, i.e.
 *    element (b + r, b + c), r > c, is U[b + p - 1 - r][b + p - 1 - c]. Everything else is 0. Requires
 *    in % 64 == 0 (UNSUPPORTED otherwise); not combined with GPTQ_FACTOR_INVERSE_RECHOL. */
#define GPTQ_FACTOR_R_FORM 2u

/* ---------------------------------------------------------------------------------------------------
 * 1. Hessian accumulation. GPTQ guide, "The idea": H = 2 X^T X / n is the curvature of the layer's
 *    squared output error over n calibration inputs; the handbook page ("GPTQ > Implementation with
 *    AutoGPTQ", compute_hessian) flattens (samples, seq, hidden) inputs to (tokens, hidden), so a caller
 *    passes tokens as rows and may stream them in chunks with repeated calls.
 *
 *  X        n_rows x in, leading dimension ld_x >= in (elements), dtype x_dtype (GPTQ_F32 or GPTQ_BF16).
 *           Rows may start at any element offset; 16-byte aligned rows (ld_x*elem % 16 == 0 and X 16-byte
 *           aligned) take the fast load path.
 *  S        in x in fp64. Only the lower triangle (i >= j) is read and written: S[i][j] += sum_k
 *           X[k][i] X[k][j]. The first chunk (*n_total == 0 on entry) writes S[i][j] = sum_k X[k][i]
 *           X[k][j] instead, so S needs no zeroing; later chunks add to it. The products of bf16
 *           or fp32 inputs are formed on the matrix cores and summed in fp32 within a slice of rows;
 *           slices are summed in fp64 in a fixed order, so results are bitwise reproducible.
 *  colsq    fp64[in]: colsq[i] += sum_k X[k][i]^2, summed in fp64 (the act_order key and the exact
 *           dead-input test need it exact up to fp64 rounding); written, not added, on the first chunk.
 *  n_total  HOST pointer; rows accumulated so far (0 before the first chunk); incremented by n_rows
 *           when the call is accepted.
 *  ws       workspace of at least gptq_hessian_workspace_bytes(n_rows, in, x_dtype) bytes.
 *  Errors   INVALID_ARG (n_rows < 1, in < 1, ld_x < in, unknown dtype, NULL pointer), WORKSPACE, HIP.
 * ------------------------------------------------------------------------------------------------- */
size_t gptq_hessian_workspace_bytes(int64_t n_rows, int64_t in, int x_dtype);
int gptq_hessian_accumulate(const void* X, int x_dtype, int64_t n_rows, int64_t in, int64_t ld_x,
                            double* S, double* colsq, int64_t* n_total,
                            void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * 2. Damping, dead inputs, order and the factor U. GPTQ guide, "The code, line by line"
 *    (_hessian_inverse_chol and the act_order bullet), "How it works" (Damping; GPTQ's two tricks,
 *    trick 2) and "When it breaks" (bad H).
 *
 *  H = 2 S / n_total (S's lower triangle). Input i is dead when colsq[i] == 0 exactly; dead inputs get
 *  H[i][i] = 1 (diagonal only). Then lambda = damp * mean(diag H) is added to the diagonal.
 *  act_order != 0: perm sorts inputs by decreasing colsq (= diag X^T X, taken before the dead fix),
 *  equal keys by increasing index; otherwise perm is the identity. U is the factor for P^T H P.
 *
 *  S, colsq   as left by gptq_hessian_accumulate (in x in lower triangle; in).
 *  U          out: in x in fp64, upper triangular with positive diagonal, U^T U = (P^T H P)^-1, in
 *             quantization order; the strictly lower triangle is set to 0.
 *  perm       out: int32[in], perm[j] = original input index quantized at position j.
 *  dead       out: uint8[in], 1 for dead inputs (original order).
 *  flags      GPTQ_FACTOR_REVERSED (0), GPTQ_FACTOR_INVERSE_RECHOL or GPTQ_FACTOR_R_FORM (then U receives
 *             the R form described with that flag); other values -> INVALID_ARG.
 *  ws         at least gptq_prepare_workspace_bytes(in) bytes.
 *  Synchronises `stream` once. Errors: INVALID_ARG (in < 1, n_total < 1, damp < 0 or not finite, NULL
 *  pointer, unknown flags), UNSUPPORTED (GPTQ_FACTOR_R_FORM with in % 64 != 0), WORKSPACE, NOT_SPD (a
 *  Cholesky pivot below 2^-1000, in particular <= 0, e.g.
 *  damp = 0 with a rank-deficient X),
 *  NONFINITE (NaN/Inf in S or colsq, or met in a pivot), HIP. On NOT_SPD/NONFINITE, U is unspecified.
 * ------------------------------------------------------------------------------------------------- */
size_t gptq_prepare_workspace_bytes(int64_t in);
int gptq_prepare_chol(const double* S, const double* colsq, int64_t n_total, int64_t in,
                      double damp, int act_order, unsigned flags,
                      double* U, int32_t* perm, uint8_t* dead,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * 3. The error-compensation loop. Lesson "GPTQ's error-compensation loop" (its four steps: each column in
 *    turn is snapped to the grid in every row, the residual over the pivot U[j][j] is the row's error, and
 *    the later columns k of the row take off error * U[j][k]) and GPTQ guide,
 *    "The code, line by line" (per-row scales from the starting weights; with groups, scales from the
 *    already-updated weights at each group boundary; clip to +-qmax) and "When it breaks" (g_idx).
 *    The guide's "Simplifications" mentions lazy updates in 128-column blocks; this library quantizes
 *    128-column panels in registers and applies the panels' errors to the columns on their right as
 *    matrix products (two levels of lazy updates), which computes the same loop.
 *
 *  W          out x in, leading dimension ld_w >= in, dtype w_dtype (GPTQ_F32 or GPTQ_BF16).
 *  U, perm, dead  as produced by gptq_prepare_chol (or supplied by the caller with the same meaning).
 *  bits       2..8; codes lie in [-qmax, qmax], qmax = 2^(bits-1) - 1.
 *  group      0 = one scale per row from the starting (dead-zeroed) weights; otherwise scales for each
 *             run of `group` columns in quantization order. Supported: group divides 128 or is a multiple
 *             of 128 (group boundaries must fall on the 128-column panel grid); others -> UNSUPPORTED.
 *  codes      out: int8, out x in, ORIGINAL column order (codes[r][perm[j]] is position j's code).
 *  scales     out: fp32, out x G, G = group ? ceil(in/group) : 1; column g = g-th group in quantization
 *             order. The arithmetic is fp64; the stored scale is rounded to fp32.
 *  g_idx      out (may be NULL): int32[in], g_idx[perm[j]] = j / group (0 when group == 0).
 *  row_loss   out (may be NULL): fp64[out], sum over columns of err^2, which equals (q - w0) H (q - w0)^T
 *             for the row's dead-zeroed, permuted start w0 and result q.
 *  Dequantized weights: Q[r][c] = codes[r][c] * scales[r][g_idx[c]] (with fp64 scales: see row_loss).
 *  ws         at least gptq_quantize_workspace_bytes(out, in) bytes.
 *  Synchronises `stream` once at its end (the status word of the weight check).
 *  Errors: INVALID_ARG (out/in < 1, ld_w < in, bits outside 2..8, group < 0, unknown dtype, NULL required
 *  pointer), UNSUPPORTED (group), WORKSPACE, NONFINITE (a NaN or Inf weight in a live input column; the
 *  outputs are then unspecified; weights of dead columns are zeroed first and never read), HIP.
 * ------------------------------------------------------------------------------------------------- */
size_t gptq_quantize_workspace_bytes(int64_t out, int64_t in);
int gptq_quantize_layer(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ld_w,
                        const double* U, const int32_t* perm, const uint8_t* dead,
                        int bits, int group,
                        int8_t* codes, float* scales, int32_t* g_idx, double* row_loss,
                        void* ws, size_t ws_bytes, void* stream);

/* Quantization grid for gptq_quantize_layer_ex (`grid`). */
typedef enum { GPTQ_GRID_SYMMETRIC = 0, GPTQ_GRID_ASYMMETRIC = 1 } gptq_grid;

/* ---------------------------------------------------------------------------------------------------
 * 3'. The same loop on a chosen grid. GPTQ guide, "Simplifications": the paper's default quantizer is
 *    asymmetric (min/max plus a zero point). Handbook page "GPTQ > Implementation with AutoGPTQ",
 *    quantize_weight / dequantize_weight / gptq_quantize_row, gives the formulas used here.
 *
 *  grid       GPTQ_GRID_SYMMETRIC: exactly gptq_quantize_layer (zeros may be NULL and is not written).
 *             GPTQ_GRID_ASYMMETRIC: levels 0..L, L = 2^bits - 1. For each row (group == 0, from the
 *             starting weights) or each group (from the already-updated weights at the group's first
 *             column): scale = (max - min) / L, or 1 when max == min; zero = round(-min / scale) clipped
 *             to [0, L]. code = round(w / scale + zero) clipped to [0, L]; the loop's quantized value is
 *             scale * (code - zero). Every rounding is to nearest, ties to even; divisions are correctly
 *             rounded. min and max are of the weights themselves (0 is not added to the range).
 *  codes      asymmetric: values 0..L stored as their uint8 bit pattern (read the buffer as uint8 when
 *             bits == 8).
 *  zeros      out (required for the asymmetric grid): int32, out x G, the same layout as scales.
 *  Dequantized weights (asymmetric): Q[r][c] = scales[r][g] * (codes[r][c] - zeros[r][g]), g = g_idx[c].
 *  Everything else (arguments, layouts, workspace, errors) is as for gptq_quantize_layer; an unknown grid,
 *  or the asymmetric grid with zeros == NULL, is INVALID_ARG.
 * ------------------------------------------------------------------------------------------------- */
int gptq_quantize_layer_ex(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ld_w,
                           const double* U, const int32_t* perm, const uint8_t* dead,
                           int bits, int group, int grid,
                           int8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, double* row_loss,
                           void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * 3''. The same loop from the R form of the factor (gptq_prepare_chol with GPTQ_FACTOR_R_FORM), which
 *    prepare forms without the triangular inverse. Lesson "GPTQ's error-compensation loop": after the
 *    loop, every row's start minus its quantized values is its errors times U, W0 - Q = E U, so E = D R with
 *    D = W0 - Q and R = U^-1. The columns of a 128-column panel P, when P's turn comes, therefore hold
 *    W0_P + (D_A R_AP) U_PP, A the columns before P: the loop keeps T = D R up to date with the same
 *    lazy products as the U route (T += D R instead of W -= E U), and each panel starts from
 *    W0_P + T_P U_PP, U_PP being U's diagonal block (with one grid per row, T_P enters the loop's steps
 *    instead), its columns then quantized exactly as in gptq_quantize_layer_ex.
 *
 *  R          the R form written by gptq_prepare_chol with GPTQ_FACTOR_R_FORM (in x in, in quantization
 *             order), or the same layout built by the caller.
 *  Requires in % 64 == 0 and group == 0 or 128 % group == 0 (a wider group takes its scale from columns
 *  beyond the current panel, whose updated values the R form does not give): UNSUPPORTED otherwise.
 *  ws         at least gptq_quantize_r_workspace_bytes(out, in) bytes: gptq_quantize_workspace_bytes(out,
 *             in) plus out x in doubles for T (rounded up to 256 bytes). It returns 0 for out/in outside
 *             the accepted range.
 *  Everything else (arguments, grids, outputs, layouts, errors) is as for gptq_quantize_layer_ex; the results
 *  agree with it up to rounding (codes may differ only where a weight lies within rounding of a grid
 *  midpoint).
 * ------------------------------------------------------------------------------------------------- */
size_t gptq_quantize_r_workspace_bytes(int64_t out, int64_t in);
int gptq_quantize_layer_r(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ld_w,
                          const double* R, const int32_t* perm, const uint8_t* dead,
                          int bits, int group, int grid,
                          int8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, double* row_loss,
                          void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * 4. Packed codes and a consumer of the outputs. GPTQ guide, "When it breaks": the layer is stored as
 *    integer codes with per-group scales, and with act_order a consumer finds a column's group through
 *    g_idx. Handbook page "GPTQ > Implementation with AutoGPTQ": codes are stored packed at 4 bits each.
 *
 *  gptq_packed_words_per_row  ceil(in * bits / 32), the uint32 words of one packed row (0 for bad sizes).
 *  gptq_pack_codes   codes (int8, out x in, as gptq_quantize_layer[_ex] writes them) -> packed (uint32,
 *                    out x words_per_row, caller-allocated). Row r is a little-endian bit stream: code j
 *                    occupies bits [bits*j, bits*(j+1)), bit k of the stream being bit k % 32 of word
 *                    k / 32. Symmetric codes are stored as code + 2^(bits-1); asymmetric codes (0..2^b-1)
 *                    as they are. Unused high bits of a row's last word are 0.
 *  gptq_dequant_matmul  Y = X Q^T, Y n x out fp32 (leading dimension ld_y >= out), X n x in (GPTQ_BF16 or
 *                    GPTQ_F32, ld_x >= in). Q[r][c] = scales[r][g] * (code(r, c) - zero(r, g)) with
 *                    g = g_idx[c]; zero = zeros[r][g] on the asymmetric grid, 0 on the symmetric one.
 *                    scales / zeros are out x G as the quantize call writes them, G = group ?
 *                    ceil(in/group) : 1; g_idx is required (all zeros when group == 0). Q is formed in
 *                    fp32 (one rounding per element) and the products accumulate in fp32. Then, in the
 *                    same pass, Y += bias (fp32[out], nullable) and, when relu == 1, Y = max(Y, 0): the
 *                    forward of a quantized MLP layer, as the guide's layer-wise driver needs it to feed
 *                    the next layer ("How it works", apply_layerwise). relu must be 0 or 1.
 *  Errors: INVALID_ARG (NULL pointer, sizes, ld, dtype, bits outside 2..8, unknown grid, asymmetric grid
 *  without zeros), HIP. Both calls are asynchronous on `stream`.
 * ------------------------------------------------------------------------------------------------- */
int64_t gptq_packed_words_per_row(int64_t in, int bits);
int gptq_pack_codes(const int8_t* codes, int64_t out, int64_t in, int bits, int grid, uint32_t* packed,
                    void* stream);
int gptq_dequant_matmul(const void* X, int x_dtype, int64_t n, int64_t in, int64_t ld_x,
                        const uint32_t* packed, const float* scales, const int32_t* zeros,
                        const int32_t* g_idx, int64_t out, int bits, int grid, int group,
                        const float* bias, int relu, float* Y, int64_t ld_y, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * 1'. gptq_hessian_accumulate without a workspace argument, for callers that cannot allocate device
 *    memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 *  Arguments, layouts, results and errors are those of gptq_hessian_accumulate, without ws / ws_bytes.
 *  Its scratch (the per-slice partial sums) is a static 80 MiB device array inside the library, one copy
 *  per GPU, held from the first call on that GPU until the process ends; the call allocates nothing
 *  (no hipMalloc, no allocating library routine). To fit it the rows may be cut into fewer slices than
 *  gptq_hessian_accumulate uses, so S can differ from that call's in fp32 rounding (bf16: in <= 4096 runs
 *  with two slices at most). A size whose single slice does not fit (bf16 in > 6144, fp32 in > 6400)
 *  returns GPTQ_ERR_UNSUPPORTED without launching anything.
 *  Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (different
 *  streams or host threads of one process) race and give wrong results. Calls ordered on
 *  one stream are safe; nothing in the array needs clearing between calls.
 * ------------------------------------------------------------------------------------------------- */
int gptq_hessian_accumulate_noalloc(const void* X, int x_dtype, int64_t n_rows, int64_t in, int64_t ld_x,
                                    double* S, double* colsq, int64_t* n_total, void* stream);

/* Human-readable name of a gptq_status value (static storage). */
const char* gptq_status_string(int status);

/* Library version string (static storage). */
const char* gptq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
