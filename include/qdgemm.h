/*
 * qdgemm.h -- quad-double matrix product C = A·B on AMD Instinct MI355X
 * (gfx950) by exact 13-bit slicing on FP64 matrix cores.
 *
 * Method: "Multiple Double Arithmetic on NVIDIA Tensor Cores" §2 (quartering;
 * a quartered quad-double matrix is sixteen times the size of a matrix of
 * doubles), §3 (balancing), §1 (the algorithms carry over to general multiple
 * doubles), §4.2 Table 1 (quad-double runs).  The same three stages as the
 * double-double product (ddgemm.h), with sixteen slices per entry:
 *
 *   1. qd_split_balanced     -- one balancing exponent per row of A / column
 *                               of B, then sixteen 13-bit slices of every entry
 *                               (a 208-bit window);
 *   2+3. qd_sliced_gemm_renorm -- the 136 slice-pair products with s + t <= 15,
 *                               summed exactly per level l = s + t on FP64 MFMA,
 *                               and per output the exact total of the sixteen
 *                               level sums rounded to the nearest quad double;
 *   qd_gemm / qd_gemm_ws run 1 + 1 + (2+3); for k > QDGEMM_K_MAX they run
 *   the product in k-blocks that share the exponents of the whole k (below).
 *
 * Conventions (as in ddgemm.h, whose status codes these calls return)
 *   - A quad-double matrix X is four row-major float64 planes X[0..3] in device
 *     memory with one leading dimension; its value is X[0] + X[1] + X[2] + X[3].
 *     The entry points take a host array of four device pointers; X[1], X[2],
 *     X[3] may be NULL (all-zero planes), X[0] may not when the matrix has
 *     entries.  The pointer array is read during the call only.
 *   - Entries must be finite and normalised the way the quad-double library the
 *     pages build on keeps them: each component at most half an ulp of the one
 *     before it (|x1| <= ulp(x0)/2, |x2| <= ulp(x1)/2, |x3| <= ulp(x2)/2; a zero
 *     component is followed by zeros).  Double-double and double inputs
 *     (trailing components NULL) always are.  For other inputs the slices are
 *     unspecified (no error is reported).
 *   - Pointers stay owned by the caller; only qd_gemm allocates (stream-ordered).
 *     Every call only enqueues work on `stream` (a hipStream_t, NULL = default);
 *     argument errors are reported before anything is enqueued.
 */
#ifndef QDGEMM_H
#define QDGEMM_H

#include "ddgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define QDGEMM_NUM_SLICES 16 /* 208-bit window: four quarters of each component     */
#define QDGEMM_NUM_LEVELS 16 /* levels l = s + t = 0..15; 136 slice pairs           */
/* Largest k: level 15 holds 16 pairs per k, and the exact-sum bound of §2 eq. (5)
 * (67,108,865 products of 26-bit quantities) allows 67,108,865 / 16 terms. */
#define QDGEMM_K_MAX 4194304
/* Largest k of qd_gemm, qd_gemm_ws and qd_gemm_ws_kb.  Longer products run in
 * k-blocks of at most QDGEMM_K_MAX terms.  Every block slices its entries below
 * the exponents of the whole row of A / column of B, so all blocks' level sums
 * are integers on the same grids; they are added exactly in 64-bit integers
 * (|level sum| <= 16 k (2^13 - 1)^2 < 2^62 units for k <= 2^32), and the total
 * is rounded once: the result equals that of one unblocked product, bit for bit. */
#define QDGEMM_K_MAX_BLOCKED 4294967296LL

/* Packed slices: the layout of ddgemm.h with 16 slices per fragment, slice s of
 * entry (o, p) at ((((o/16)*KB + p/4)*16 + s)*64) + (p%4)*16 + o%16, value
 * sign(x) * d_s * 2^(-13(s+1)) with d_s the s-th 13-bit digit of
 * N = floor(|x| * 2^(208-E)).  Bytes for one operand: qd_split_slices_bytes;
 * 0 for negative sizes. */
size_t qd_split_slices_bytes(int64_t outer, int64_t k);

/* Workspace bytes qd_gemm_ws needs: slices of both operands for one k-block
 * and both exponent vectors (256-byte aligned regions), plus
 *   - for a product of one k-block with k <= 2^21 (the pair-packed schedule of
 *     ddgemm.h, dd_sliced_gemm_pairs, with 16 slices: 72 matrix products per
 *     k-block): 15 int64 m×n planes of group sums when k exceeds 2048, the most
 *     values whose FP64 group sums stay exact, and when its tiles from some
 *     tile on split over k (ddgemm_split_parts / ddgemm_split_first_row with 16
 *     slices: p parts from row r) p 15 int64 (m - r)×n part planes;
 *   - otherwise (the level schedule: 136 products per k-block): sixteen int64
 *     m×n level planes when k needs more than one block, and when the product
 *     splits over k, sixteen double (m - r)×n level planes (the blocks of a
 *     blocked product split all tiles or none: r = 0).
 * 0 for negative sizes, k > QDGEMM_K_MAX_BLOCKED, or a workspace past 2^62 bytes (which
 * qd_gemm_ws and qd_gemm reject with DDGEMM_ERROR_INVALID_VALUE).  The _kb form is for qd_gemm_ws_kb with k-blocks of
 * kblock terms (0 for kblock outside [1, QDGEMM_K_MAX] when k > 0). */
size_t qd_gemm_workspace_size(int64_t m, int64_t n, int64_t k);
size_t qd_gemm_workspace_size_kb(int64_t m, int64_t n, int64_t k, int64_t kblock);

/*
 * Balancing exponents and slices of one quad-double operand.
 *   X      : four component planes, rows×cols, row stride ldx >= max(1, cols).
 *   axis   : 0 = the A operand (one exponent per row, outer = rows, k = cols);
 *            1 = the B operand (one exponent per column, outer = cols, k = rows).
 *   exps   : the largest frexp exponent of RN(x0 + x1 + x2 + x3) over the
 *            nonzero entries of each row/column (so |x| < 2^E), 0 if all are zero.
 *   slices : qd_split_slices_bytes(outer, k) bytes, packed as above.
 * Errors: DDGEMM_ERROR_INVALID_VALUE for negative sizes, ldx < max(1, cols), axis
 * not 0/1, k > QDGEMM_K_MAX, NULL X / X[0] / exps / slices with a nonzero extent.
 */
ddgemm_status_t qd_split_balanced(int64_t rows, int64_t cols, const double* const X[4], int64_t ldx,
                                  int axis, int32_t* exps, double* slices, void* stream);

/*
 * The sixteen level sums S_l = sum_{s+t=l} sum_p A_s[i][p] B_t[p][j] (exact on the
 * matrix cores, §2 eqs. (3)-(5)) and, per output, their exact total T rounded
 * greedily: C[0] = RN(T), C[1] = RN(T - C[0]), C[2] = RN(T - C[0] - C[1]),
 * C[3] = RN(T - C[0] - C[1] - C[2]), scaled by 2^(E[i] + F[j]) (ties to even;
 * the nearest quad double of T; beyond the double range the words overflow as
 * ldexp does).  The pages' fifth step, adding the parts of each entry in
 * multiple-double arithmetic, done exactly.
 *   A_slices, E : qd_split_balanced output for A (outer = m); B_slices, F : for B.
 *   C           : four m×n planes, row stride ldc >= max(1, n), all non-NULL and
 *                 pairwise disjoint.  k = 0 writes zeros.
 * Errors: DDGEMM_ERROR_INVALID_VALUE for negative sizes, ldc < max(1, n),
 * k > QDGEMM_K_MAX, NULL or overlapping C planes, NULL slices/E/F.
 */
ddgemm_status_t qd_sliced_gemm_renorm(int64_t m, int64_t n, int64_t k,
                                      const double* A_slices, const int32_t* E,
                                      const double* B_slices, const int32_t* F,
                                      double* const C[4], int64_t ldc, void* stream);

/*
 * C = A·B for quad-double A (m×k) and B (k×n).  Overwrites C.  m = 0 or n = 0:
 * no-op; k = 0: C = 0.  Every entry is the nearest quad double of the exact
 * total of its window slice products (as qd_sliced_gemm_renorm rounds it),
 * whatever the schedule: up to k = 2^21 in one block the 136 slice pairs run as
 * 72 pair-packed matrix products (ddgemm.h, dd_sliced_gemm_pairs), beyond that
 * as sixteen exact levels.  Per entry the result is within
 *     2^-208 (2^F_j sum_p |a_ip| + 2^E_i sum_p |b_pj| + 16 k 2^(E_i+F_j))
 *     + 2^-200 (|A||B|)_ij
 * of the exact product (E_i, F_j the row/column exponents): the truncation of
 * the operands to 208 bits below their exponents, the slice pairs below the
 * window, and the final rounding.
 * k up to QDGEMM_K_MAX_BLOCKED: beyond QDGEMM_K_MAX the product runs in the
 * fewest equal k-blocks within it, with the same result (see that constant).
 *   qd_gemm       allocates its workspace with hipMallocAsync/hipFreeAsync on
 *                 `stream` (DDGEMM_ERROR_WORKSPACE if that fails).
 *   qd_gemm_ws    uses the caller's workspace of ws_bytes >= qd_gemm_workspace_size
 *                 (256-byte aligned), allocates nothing.
 *   qd_gemm_ws_kb the same with k-blocks of kblock terms (1 <= kblock <=
 *                 QDGEMM_K_MAX; any k > 0) and ws_bytes >= qd_gemm_workspace_size_kb:
 *                 block b covers k indices [b kblock, min(k, (b+1) kblock)).
 *                 The result does not depend on kblock.
 * Errors: as for the stage calls, plus lda < max(1, k), ldb < max(1, n), a C
 * plane overlapping A, B or another C plane, k > QDGEMM_K_MAX_BLOCKED, kblock
 * out of range.
 */
ddgemm_status_t qd_gemm(int64_t m, int64_t n, int64_t k,
                        const double* const A[4], int64_t lda,
                        const double* const B[4], int64_t ldb,
                        double* const C[4], int64_t ldc, void* stream);

ddgemm_status_t qd_gemm_ws(int64_t m, int64_t n, int64_t k,
                           const double* const A[4], int64_t lda,
                           const double* const B[4], int64_t ldb,
                           double* const C[4], int64_t ldc,
                           void* workspace, size_t ws_bytes, void* stream);

ddgemm_status_t qd_gemm_ws_kb(int64_t m, int64_t n, int64_t k, int64_t kblock,
                              const double* const A[4], int64_t lda,
                              const double* const B[4], int64_t ldb,
                              double* const C[4], int64_t ldc,
                              void* workspace, size_t ws_bytes, void* stream);

/* qd_gemm_ws recording the hipEvent_t `after_split` (NULL: none) on `stream`
 * once the operands of the first k-block are sliced, so that a caller can time
 * the slicing and the GEMM apart inside one product. */
ddgemm_status_t qd_gemm_ws_timed(int64_t m, int64_t n, int64_t k,
                                 const double* const A[4], int64_t lda,
                                 const double* const B[4], int64_t ldb,
                                 double* const C[4], int64_t ldc,
                                 void* workspace, size_t ws_bytes, void* after_split, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QDGEMM_H */
