/*
 * ddgemm.h -- double-double matrix product C = A·B on AMD Instinct MI355X
 * (gfx950) by exact 13-bit slicing on FP64 matrix cores.
 *
 * Method: "Multiple Double Arithmetic on NVIDIA Tensor Cores" (arXiv
 * 2607.06881v1).  §2 cuts every double into 13-bit quarters whose pairwise
 * products are exact, groups the quarter products by the sum of their indices
 * (eqs. (1)-(3)), writes the double-double product as one product of double
 * matrices (eq. (4)) and adds the parts of each output entry in double-double
 * arithmetic once at the end (the fifth step of the overview).  §3 keeps the
 * parts on a common exponent grid (balancing).  This library realises that as:
 *
 *   1. dd_split_balanced  -- one balancing exponent per row of A / column of B,
 *                            then eight 13-bit slices of every entry;
 *   2. dd_sliced_gemm     -- the 36 slice-pair products with s + t <= 7, summed
 *                            exactly per level l = s + t on FP64 MFMA;
 *   3. dd_renorm_levels   -- TwoSum cascade of the 8 level sums into (hi, lo);
 *   dd_sliced_gemm_renorm fuses 2 and 3.
 * The product entry points (dd_gemm, dd_gemm_ws, ...) run 1 for both operands
 * and then the same 36 slice-pair products grouped two to a matrix
 * instruction (dd_sliced_gemm_pairs: 20 instructions per k instead of 36),
 * with the epilogue fused: each entry's exact windowed total -- the same
 * total the level sums of 2 add up to -- rounded once to the nearest
 * double-double.  Outputs whose tiles leave the chip partly idle are split
 * over k for some or all output rows (dd_gemm_workspace_size).
 *
 * Conventions for every entry point
 *   - All matrices are row-major float64 planes in device memory; a
 *     double-double matrix X is the pair of planes (X_hi, X_lo) with value
 *     X_hi + X_lo.  Leading dimensions count elements; a rows×cols matrix
 *     needs max(1, cols) <= ld and rows·ld <= 2^58 (so that no extent or byte
 *     count overflows), else DDGEMM_ERROR_INVALID_VALUE.  A lo pointer may be
 *     NULL, meaning an all-zero lo plane.
 *   - Pointers are owned by the caller; the library keeps none after a call
 *     returns.  Only dd_gemm allocates (stream-ordered, freed on the stream);
 *     dd_gemm_noalloc works in a fixed device array the library holds.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work and returns; errors from the execution itself surface at
 *     the caller's next synchronisation, as with any HIP launch.  Argument
 *     errors are reported before anything is enqueued.
 *   - Inputs must be finite; pairs need not be normalised (the exact value
 *     hi + lo is sliced).  Outputs must not overlap inputs.
 *   - Calls are reentrant: no global state except a per-device capability
 *     check cached on first use (and dd_gemm_noalloc's per-device array).
 */
#ifndef DDGEMM_H
#define DDGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DDGEMM_SUCCESS = 0,
    DDGEMM_ERROR_INVALID_VALUE = 1, /* negative size, short leading dimension, NULL with a
                                       nonzero extent, bad axis, k > DDGEMM_K_MAX, overlap */
    DDGEMM_ERROR_WORKSPACE = 2,     /* workspace allocation failed or caller workspace too small */
    DDGEMM_ERROR_LAUNCH = 3,        /* a HIP launch or runtime call failed while enqueuing */
    DDGEMM_ERROR_DEVICE = 4         /* no current HIP device, or it is not gfx950 */
} ddgemm_status_t;

/* Slicing constants ("Multiple Double Arithmetic on NVIDIA Tensor Cores", §2). */
#define DDGEMM_SLICE_BITS 13 /* significant bits per slice: the pages' quarters   */
#define DDGEMM_NUM_SLICES 8  /* 104-bit window: four quarters of hi, four of lo    */
#define DDGEMM_NUM_LEVELS 8  /* levels l = s + t = 0..7; 36 slice pairs            */
/* The *_ns entry points take the number of slices n per operand entry instead:
 * a 13n-bit window, n levels, n(n+1)/2 slice pairs, DDGEMM_MIN_SLICES <= n <=
 * DDGEMM_MAX_SLICES.  n = 4 is §2 eqs. (1)-(3): the four quarters of a leading
 * double; n = 8 is the double-double product.  Fewer slices trade accuracy
 * (about 13n - 7 bits relative to the row/column maxima) for speed; more than
 * eight keep entries that lie up to 13(n - 8) bits below their row's (column's)
 * largest at full double-double precision -- the purpose of §3 Problem 3.2's
 * exponent classes, a class 13c bits down being the same digits c places
 * deeper -- for n(n+1)/2 pairs. */
#define DDGEMM_MIN_SLICES 4
#define DDGEMM_MAX_SLICES 16
/* Largest k: with every level holding at most 8 pairs, the exact-sum bound of §2
 * eq. (5) (67,108,865 products of 26-bit quantities) allows 67,108,865 / 8 terms.
 * With n > 8 slices the deepest level holds n pairs: k <= floor(67,108,865 / n)
 * (DDGEMM_K_MAX_NS(n)). */
#define DDGEMM_K_MAX 8388608
#define DDGEMM_K_MAX_NS(n) ((n) <= 8 ? DDGEMM_K_MAX : 67108865 / (n))

/* Packed slice layout (the output of dd_split_balanced, the input of the GEMMs).
 *
 * For one operand, "outer" is the row index i of A (axis 0) or the column index
 * j of B (axis 1) and p is the index along k.  Outer is padded to
 * Op = roundup(outer, DDGEMM_PACK_OUTER), k to Kp = roundup(k, DDGEMM_PACK_K),
 * KB = Kp / 4.  Slice s of entry (o, p) is the double at
 *
 *     ((((o / 16) * KB + p / 4) * 8 + s) * 64) + (p % 4) * 16 + (o % 16)
 *
 * i.e. 16×4 (A) or 4×16 (B) fragments of 64 doubles in the lane order of the
 * gfx950 FP64 16x16x4 matrix instruction, the eight slices of one fragment
 * adjacent.  The value stored is sign(x) * d_s * 2^(-13(s+1)) where d_s is the
 * s-th 13-bit digit of N = floor(|x| * 2^(104-E)), x = hi + lo exactly and E the
 * balancing exponent of the entry's row (A) or column (B); padding holds +0.0.
 * Total size: Op * Kp * 8 doubles (dd_split_slices_bytes). */
#define DDGEMM_PACK_OUTER 64  /* the tallest tile: padding rows beyond it are never read */
#define DDGEMM_PACK_K 16

/* Bytes of packed slices for one operand with `outer` rows (A) / columns (B) and
 * inner dimension k; 0 for negative sizes. */
size_t dd_split_slices_bytes(int64_t outer, int64_t k);

/* Workspace bytes dd_gemm_ws needs for an m×k by k×n product (slices of both
 * operands and both exponent vectors, each region 256-byte aligned, plus 7
 * int64 m×n planes of group sums when k exceeds 4096, the most values whose
 * FP64 group sums stay exact, see dd_sliced_gemm_pairs); 0 for
 * negative sizes, and for sizes whose workspace would pass 2^62 bytes (the
 * products reject those with DDGEMM_ERROR_INVALID_VALUE).  When the output tiles (64×64; 32×64 with 6 or 9..16 slices)
 * leave part of the chip idle -- a few tiles, or a last round of 256
 * workgroups far from full -- the output tiles from some first tile t on
 * (row-major; t = 0: all of them) may be split over k into p parts of at least
 * one stage each (a stage is 8 values of k, 4 from 14 slices on), p <= 256,
 * while the tiles before t, whole rounds of 256 workgroups, run unsplit; t and
 * p are chosen by a timing model of the rounds of workgroups and of the part
 * planes' traffic, and only where that saves at least 5 %; outputs that
 * fill whole rounds never split.  ddgemm_split_parts returns p,
 * ddgemm_split_first_tile t and ddgemm_split_first_row the first row r of t's
 * tile row.  Each part stores the exact int64 group sums of its outputs in
 * planes of its own (no atomics), and one more launch adds the parts and
 * rounds; the workspace also holds those p (nslices - 1) (m - r)×n int64
 * planes.  The split result is bit-identical to the unsplit one. */
size_t dd_gemm_workspace_size(int64_t m, int64_t n, int64_t k);

/*
 * Balancing exponents and slices of one operand ("Multiple Double Arithmetic on
 * NVIDIA Tensor Cores", §2 quartering with its worked example, §3 balancing).
 *
 *   X_hi, X_lo : rows×cols double-double matrix, row stride ldx >= max(1, cols).
 *   axis = 0   : X is the A operand (m×k): one exponent per row, outer = rows,
 *                k = cols; `exps` has rows entries.
 *   axis = 1   : X is the B operand (k×n): one exponent per column, outer = cols,
 *                k = rows; `exps` has cols entries.
 *   exps       : E = the largest frexp exponent of RN(hi + lo) over the nonzero
 *                entries of the row/column (so |hi + lo| < 2^E), 0 if all are zero.
 *   slices     : dd_split_slices_bytes(outer, k) bytes, packed as described above.
 * Errors: DDGEMM_ERROR_INVALID_VALUE for negative sizes, ldx < max(1, cols),
 * axis not 0/1, k > DDGEMM_K_MAX, or NULL X_hi/exps/slices with a nonzero extent.
 */
ddgemm_status_t dd_split_balanced(int64_t rows, int64_t cols,
                                  const double* X_hi, const double* X_lo, int64_t ldx,
                                  int axis, int32_t* exps, double* slices, void* stream);

/*
 * Level sums of the slice-pair products ("Multiple Double Arithmetic on NVIDIA
 * Tensor Cores", §2 eqs. (3)-(4); exactness: §2 eq. (5)).
 *
 *   A_slices : packed A operand (outer = m), B_slices : packed B operand (outer = n),
 *              both with the same k.
 *   levels   : 8 planes, plane l at levels + l*m*ldl, each m×n with row stride
 *              ldl >= max(1, n):  S_l[i][j] = sum_{s+t=l} sum_p A_s[i][p] * B_t[p][j]
 *              for l = 0..7, computed exactly (every partial sum is an integer
 *              multiple of 2^(-13(l+2)) below 2^53 units).  k = 0 writes zeros.
 *              Outputs that leave the chip partly idle are split over k, all
 *              rows at once (the rule of dd_gemm_workspace_size with r = 0):
 *              the planes are zeroed and the k-parts add into them with atomic
 *              adds, exact and so order-independent.
 * Errors: DDGEMM_ERROR_INVALID_VALUE for negative sizes, ldl < max(1, n),
 * k > DDGEMM_K_MAX, NULL pointers with a nonzero extent.
 */
ddgemm_status_t dd_sliced_gemm(int64_t m, int64_t n, int64_t k,
                               const double* A_slices, const double* B_slices,
                               double* levels, int64_t ldl, void* stream);

/*
 * Renormalisation of the level sums ("Multiple Double Arithmetic on NVIDIA
 * Tensor Cores", §2, the fifth step: the parts of each product entry are added
 * in double-double arithmetic on the regular cores; Problem 1.1 is why this is
 * done once per entry and not inside the product).
 *
 * Per entry, smallest level first: (h, t) = (S_7, 0); for l = 6..0:
 * (s, e) = TwoSum(h, S_l); t = t + e; (h, t) = TwoSum(s, t).  Then
 * C_hi = h * 2^(E[i] + F[j]), C_lo = t * 2^(E[i] + F[j]) (ldexp).
 *   levels : as written by dd_sliced_gemm (row stride ldl, plane stride m*ldl).
 *   E, F   : the exponents from dd_split_balanced for A (m) and B (n).
 *   C_hi, C_lo : m×n, row stride ldc >= max(1, n).
 */
ddgemm_status_t dd_renorm_levels(int64_t m, int64_t n, const double* levels, int64_t ldl,
                                 const int32_t* E, const int32_t* F,
                                 double* C_hi, double* C_lo, int64_t ldc, void* stream);

/* dd_sliced_gemm followed by dd_renorm_levels in one kernel: the level sums stay
 * in registers; bit-identical to the two-call sequence. */
ddgemm_status_t dd_sliced_gemm_renorm(int64_t m, int64_t n, int64_t k,
                                      const double* A_slices, const int32_t* E,
                                      const double* B_slices, const int32_t* F,
                                      double* C_hi, double* C_lo, int64_t ldc, void* stream);

/*
 * Group sums of the pair-packed schedule, the exact sums the product entry
 * points round (stage call, for bit-exact tests).  Slices 2u and 2u+1 of an
 * entry of A have its sign and sit 13 bits apart, so d_2u 2^13 + d_(2u+1) is
 * one exact 26-bit operand, and its product with a 13-bit slice of B covers the
 * window pairs (2u, t) and (2u+1, t) at once ("Multiple Double Arithmetic on
 * NVIDIA Tensor Cores", §2 eqs. (1)-(4); every product and partial sum stays
 * an exact FP64 integer of units, as in §2 eq. (5), for 39-bit products):
 * where only (2u, t) is in the window (2u + t = 7) it runs alone.  That covers
 * the 36 window pairs with 20 products per k (the fewest: a product covers at
 * most two pairs of opposite index-sum parity, and 20 of the 36 pairs have an
 * odd index sum).  Product (u, t) adds into group g = 2u + t, a single pair
 * into group 6; group g counts units 2^(-13(g+3)), so the exact windowed total
 * of entry (i, j) is 2^(E_i + F_j) sum_g G_g 2^(-13(g+3)) -- the same total as
 * sum_l S_l 2^(-13(l+2)) from dd_sliced_gemm.
 *   units : 7 int64 planes (n - 1 with the _ns variant), plane g at
 *           units + g*m*ldu, each m×n with row stride ldu >= max(1, n):
 *           G_g[i][j] exactly.  The kernels keep FP64 sums over at most 4096
 *           values of k (the most whose largest group sum stays below 2^53)
 *           and add them into the int64 planes; k <= dd_gemm_kblock_max(n)
 *           (2^22 for 8 slices) keeps every group sum below 2^63.
 * Errors: DDGEMM_ERROR_INVALID_VALUE for negative sizes, ldu < max(1, n),
 * k > dd_gemm_kblock_max(n), NULL pointers with a nonzero extent.
 */
ddgemm_status_t dd_sliced_gemm_pairs(int64_t m, int64_t n, int64_t k,
                                     const double* A_slices, const double* B_slices,
                                     int64_t* units, int64_t ldu, void* stream);

/*
 * C = A·B for double-double A (m×k) and B (k×n) ("Multiple Double Arithmetic on
 * NVIDIA Tensor Cores", §2 overview, steps 1-5).  Overwrites C (no alpha/beta).
 * m = 0 or n = 0: no-op.  k = 0: C = 0.  k beyond dd_gemm_kblock_max(8) =
 * 4,194,304 is processed in the fewest equal k-blocks within it, as
 * dd_gemm_ws_kb describes.  Result: the nearest double-double (C_hi = RN(x), C_lo =
 * RN(x - C_hi), gradual underflow honoured) of x = the exact sum of the 36
 * window slice-pair products, i.e. the product of the operands truncated to
 * 104 bits below their row/column exponents minus the pairs below the
 * window; on inputs whose entries sit within a few binades of their
 * row/column maximum this is within 1e-28 * (|A||B|)_ij of the exact product.
 * Beyond the double range C_hi is +-inf and C_lo rounds what is left after
 * C_hi's value with an unbounded exponent range.
 *   dd_gemm     allocates its workspace with hipMallocAsync/hipFreeAsync on
 *               `stream` (DDGEMM_ERROR_WORKSPACE if that fails).
 *   dd_gemm_ws  uses the caller's workspace of ws_bytes >= dd_gemm_workspace_size
 *               (256-byte aligned), allocates nothing.
 * Errors: as for the stage calls (except the k limit), plus lda < max(1, k),
 * ldb < max(1, n), ldc < max(1, n), C overlapping A or B.
 */
ddgemm_status_t dd_gemm(int64_t m, int64_t n, int64_t k,
                        const double* A_hi, const double* A_lo, int64_t lda,
                        const double* B_hi, const double* B_lo, int64_t ldb,
                        double* C_hi, double* C_lo, int64_t ldc, void* stream);

ddgemm_status_t dd_gemm_ws(int64_t m, int64_t n, int64_t k,
                           const double* A_hi, const double* A_lo, int64_t lda,
                           const double* B_hi, const double* B_lo, int64_t ldb,
                           double* C_hi, double* C_lo, int64_t ldc,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * The same operations with n slices per entry (see DDGEMM_MIN_SLICES).  The
 * packed layout is the one described above with n slices per fragment in place
 * of 8 (slice s of entry (o, p) at ((((o/16)*KB + p/4)*n + s)*64) + (p%4)*16 +
 * o%16); for n = 8 every call equals its counterpart without the suffix.  The
 * product C is the nearest double-double of the exact sum of the n(n+1)/2
 * window pairs (n - 1 groups, n^2/4 + n/2 matrix products per k rounded up:
 * 6 for n = 4, 20 for n = 8, 72 for n = 16); per entry it is within
 * 2^(-13n) (2^F_j sum_p |a_ip| + 2^E_i sum_p |b_pj| + n k 2^(E_i+F_j))
 * + 2^-104 |C_ij| of the exact product, E_i and F_j the row/column exponents.
 * The stage chain's cascade (dd_sliced_gemm_renorm_ns) adds at most 2^-104
 * of the level magnitudes instead.  Errors: as for the counterparts, plus
 * DDGEMM_ERROR_INVALID_VALUE for n outside [DDGEMM_MIN_SLICES, DDGEMM_MAX_SLICES]
 * and k > DDGEMM_K_MAX_NS(n) (the products: k-blocks beyond
 * dd_gemm_kblock_max(n)).
 */
size_t dd_split_slices_bytes_ns(int64_t outer, int64_t k, int nslices);
size_t dd_gemm_workspace_size_ns(int64_t m, int64_t n, int64_t k, int nslices);
ddgemm_status_t dd_split_balanced_ns(int64_t rows, int64_t cols,
                                     const double* X_hi, const double* X_lo, int64_t ldx,
                                     int axis, int nslices, int32_t* exps, double* slices,
                                     void* stream);
ddgemm_status_t dd_sliced_gemm_renorm_ns(int64_t m, int64_t n, int64_t k, int nslices,
                                         const double* A_slices, const int32_t* E,
                                         const double* B_slices, const int32_t* F,
                                         double* C_hi, double* C_lo, int64_t ldc, void* stream);
ddgemm_status_t dd_sliced_gemm_pairs_ns(int64_t m, int64_t n, int64_t k, int nslices,
                                        const double* A_slices, const double* B_slices,
                                        int64_t* units, int64_t ldu, void* stream);
ddgemm_status_t dd_gemm_ws_ns(int64_t m, int64_t n, int64_t k, int nslices,
                              const double* A_hi, const double* A_lo, int64_t lda,
                              const double* B_hi, const double* B_lo, int64_t ldb,
                              double* C_hi, double* C_lo, int64_t ldc,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * k-blocked product (§2 eq. (5) bounds how many slice products one level sum
 * holds exactly).  k is cut into consecutive blocks of kblock indices (the last
 * one shorter); block b is the sliced product of A[:, b kblock ...] and the
 * matching rows of B with its own balancing exponents, and the block results
 * are added into C in block order with the accurate double-word addition of
 * Joldes, Muller and Popescu (relative error < 3·2^-106 per addition).  With
 * kblock >= k this is dd_gemm_ws_ns bit for bit.  Smaller blocks also shrink the
 * workspace: slices are sized by kblock, plus two m×n planes when there is more
 * than one block (dd_gemm_workspace_size_kb).
 * Errors: as for dd_gemm_ws_ns, plus DDGEMM_ERROR_INVALID_VALUE for k > 0 and
 * kblock outside [1, dd_gemm_kblock_max(n)].
 */
size_t dd_gemm_workspace_size_kb(int64_t m, int64_t n, int64_t k, int nslices, int64_t kblock);
ddgemm_status_t dd_gemm_ws_kb(int64_t m, int64_t n, int64_t k, int nslices, int64_t kblock,
                              const double* A_hi, const double* A_lo, int64_t lda,
                              const double* B_hi, const double* B_lo, int64_t ldb,
                              double* C_hi, double* C_lo, int64_t ldc,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * The double-double product for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments (minus the workspace), kernels and result as
 * dd_gemm_ws -- bit for bit -- with the workspace taken from a device array
 * that the library holds itself: DDGEMM_NOALLOC_SCRATCH_BYTES bytes on every
 * GPU the call runs on, reserved from the first call on that GPU until the
 * process ends.  Calls nothing that allocates.
 *   - Products whose dd_gemm_workspace_size exceeds DDGEMM_NOALLOC_SCRATCH_BYTES
 *     are rejected with DDGEMM_ERROR_WORKSPACE before anything is enqueued
 *     (m = n = k = 1024 fits; 2048^3 does not).
 *   - All calls on one GPU share that GPU's array, which keeps what the last
 *     call left in it (no call depends on its contents).  Calls ordered on one
 *     stream are safe; calls whose execution overlaps on one GPU (different
 *     streams without ordering, or several host threads) race on the array and
 *     give undefined results.
 * Errors: as for dd_gemm_ws, plus DDGEMM_ERROR_WORKSPACE as above and
 * DDGEMM_ERROR_LAUNCH if the array's device address cannot be obtained.
 */
#define DDGEMM_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
ddgemm_status_t dd_gemm_noalloc(int64_t m, int64_t n, int64_t k,
                                const double* A_hi, const double* A_lo, int64_t lda,
                                const double* B_hi, const double* B_lo, int64_t ldb,
                                double* C_hi, double* C_lo, int64_t ldc, void* stream);

/*
 * dd_gemm_ws_ns with a measurement mark: `after_split` (a hipEvent_t, or NULL)
 * is recorded on `stream` once both operands of the first k-block are sliced,
 * so that the time from it to the end of the call is the product's
 * matrix-core part alone (with one k-block: k <= dd_gemm_kblock_max(n)).
 * Otherwise identical to dd_gemm_ws_ns, bit for bit.
 */
ddgemm_status_t dd_gemm_ws_timed(int64_t m, int64_t n, int64_t k, int nslices,
                                 const double* A_hi, const double* A_lo, int64_t lda,
                                 const double* B_hi, const double* B_lo, int64_t ldb,
                                 double* C_hi, double* C_lo, int64_t ldc,
                                 void* workspace, size_t ws_bytes, void* after_split, void* stream);

/* The largest k-block of the product entry points with n slices per entry
 * (longer k is cut into the fewest equal blocks within it): the smaller of
 * DDGEMM_K_MAX_NS(n) and the most values of k whose int64 group sums
 * (dd_sliced_gemm_pairs) stay below 2^63 -- 4,194,304 for 8 slices,
 * 2,097,152 for 16.  0 for n outside [DDGEMM_MIN_SLICES, DDGEMM_MAX_SLICES]. */
int64_t dd_gemm_kblock_max(int nslices);

/* Static, human-readable name of a status code. */
const char* ddgemm_status_string(ddgemm_status_t status);

/* Diagnostics: how the product entry points (dd_gemm*, and with nslices = 16
 * the quad-double ones) split an m×n×k product, or one k-block of k values,
 * with nslices slices over k: ddgemm_split_parts gives the number of k-parts
 * (1 = not split; 0 for invalid sizes or slice counts), ddgemm_split_first_tile
 * the first split output tile (tiles row-major; the tiles before it run unsplit;
 * the number of tiles when the product is not split) and ddgemm_split_first_row
 * the first row of that tile's tile row (m when not split); -1 for invalid
 * arguments.  dd_sliced_gemm
 * and the blocks of a blocked quad-double product split all rows or none, with
 * the part count of the plan whose first row is 0.  Host-only, needs no device. */
int64_t ddgemm_split_parts(int64_t m, int64_t n, int64_t k, int nslices);
int64_t ddgemm_split_first_row(int64_t m, int64_t n, int64_t k, int nslices);
int64_t ddgemm_split_first_tile(int64_t m, int64_t n, int64_t k, int nslices);
/* 1 when the product entry points compute an m×n×k product with nslices slices
 * (16: also the quad-double product) by the small-output kernel -- one 4-wave
 * workgroup per 16×16 output block, the waves sharing k, their exact group sums
 * added in LDS, no split and no second launch -- else 0 (also for invalid
 * sizes).  It is taken for at most 256 such blocks and k within one exact FP64
 * chunk (dd_sliced_gemm_pairs) where a timing model of it beats the tiled
 * kernel's plan. */
int ddgemm_small_product(int64_t m, int64_t n, int64_t k, int nslices);

/* Diagnostics: runs one FP64 16x16x4 matrix instruction on one wave with
 * a-operand lane value (lane + 1) and b-operand lane value 100 * (lane + 1) and
 * writes the four result doubles of every lane to out[lane * 4 + v]
 * (256 doubles, device memory).  Used to confirm the operand/result lane layout
 * the packed format assumes.  Errors: DDGEMM_ERROR_INVALID_VALUE for NULL out. */
ddgemm_status_t ddgemm_probe_mfma_f64(double* out, void* stream);

/* Diagnostics: the pair-packed products' exit rounding ("Multiple Double
 * Arithmetic on NVIDIA Tensor Cores", §2 overview, fifth step: the parts of an
 * entry added into a double-double; here the exact total rounded once) on
 * given group sums.  Entry i (0 <= i < count) has nslices - 1 int64 group sums
 * units[i * (nslices - 1) + g], group g counting units 2^(scale[i] - 13(g + 3)),
 * and gets out[2 i] = RN(x), out[2 i + 1] = RN(x - out[2 i]) for their exact
 * total x (ties to even, gradual underflow, overflow as the products give it).
 * Device pointers; the sums must stay below 2^63 in magnitude with the carries
 * between groups, as the products' own do.  Used to test the exit at ties and
 * at the ends of the exponent range.  Errors: DDGEMM_ERROR_INVALID_VALUE for
 * count < 0 or > 2^38, nslices outside [DDGEMM_MIN_SLICES, DDGEMM_MAX_SLICES],
 * or a NULL pointer with count > 0. */
ddgemm_status_t ddgemm_probe_pair_round(int64_t count, int nslices, const int64_t* units, const int32_t* scale,
                                        double* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DDGEMM_H */
