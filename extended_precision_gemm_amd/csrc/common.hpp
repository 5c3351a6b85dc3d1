// Shared host/device definitions of the gfx950 double-double GEMM library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ddgemm.h"
#include "qdgemm.h"

namespace ddg {

constexpr int kSliceBits = DDGEMM_SLICE_BITS;
constexpr int kSlices = DDGEMM_NUM_SLICES;  // slices of the double-double product
constexpr int kMinSlices = DDGEMM_MIN_SLICES;
constexpr int kMaxSlices = DDGEMM_MAX_SLICES;
constexpr int kLevels = DDGEMM_NUM_LEVELS;
constexpr int kWindowBits = kSliceBits * kSlices;  // 104
constexpr int kPackOuter = DDGEMM_PACK_OUTER;
constexpr int kPackK = DDGEMM_PACK_K;
constexpr int kFragDoubles = 64;                    // one 16x4 / 4x16 FP64 MFMA operand
constexpr int kFragSetDoubles = kFragDoubles * kSlices;  // all 8 slices of one fragment
constexpr int kQdSlices = QDGEMM_NUM_SLICES;         // slices of the quad-double product

typedef double double4_t __attribute__((ext_vector_type(4)));

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Packed-operand geometry for `outer` rows (A) / columns (B) and inner dimension k.
struct PackGeom {
    int64_t outer, k, Op, Kp, KB, RB;  // RB = Op / 16 fragment rows, KB = Kp / 4
    PackGeom(int64_t outer_, int64_t k_)
        : outer(outer_), k(k_), Op(round_up(outer_, kPackOuter)), Kp(round_up(k_, kPackK)),
          KB(round_up(k_, kPackK) / 4), RB(round_up(outer_, kPackOuter) / 16) {}
    int64_t doubles(int ns = kSlices) const { return Op * Kp * ns; }
};

// The component planes of one quad-double operand (x[1..3] may be null: zero).
struct QdPlanes {
    const double* x[4];
};

// Output planes of the fused product: c[0], c[1] = (hi, lo) for a double-double
// result; c[0..3] for a quad-double result.
struct OutPlanes {
    double* c[4];
};

// Phases of an operand's split: the exponent pass and the slice pass, so that
// the quad-double product can run both operands' exponent passes before either
// slice pass.  An operand sliced in one pass does it all in the slice phase.
enum SplitPhase { kSplitExps = 1, kSplitSlices = 2, kSplitAll = 3 };

// Columns per workgroup of the streaming column-exponent pass.
constexpr int64_t kExpColChunk = 512;
inline int64_t exp_col_chunks(int64_t cols) { return (cols + kExpColChunk - 1) / kExpColChunk; }

// Argument checks shared by the double-double product entry points: `status`
// is the error to report (DDGEMM_SUCCESS when the call may proceed), `empty`
// marks the no-op m = 0 or n = 0, `need` the workspace bytes otherwise.
struct ProductCheck {
    ddgemm_status_t status;
    bool empty;
    size_t need;
};
ProductCheck check_dd_product(int64_t m, int64_t n, int64_t k, int ns, int64_t kblock, const double* A_hi,
                              const double* A_lo, int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb,
                              const double* C_hi, const double* C_lo, int64_t ldc);
// The k-block the product uses when none is given: all of k when it fits the
// exact-sum bound for ns slices, else the fewest equal blocks that do.
int64_t default_kblock(int64_t k, int ns);
// DDGEMM_SUCCESS when the current device is a gfx950 (cached per device).
ddgemm_status_t check_current_device();

// Host-side launch helpers implemented next to their kernels.
// pairs: an A operand (axis 0) in the pair-packed layout the product's GEMM
// reads (plane 2u = slices 2u + 2u+1, plane 2u+1 = slice 2u).
hipError_t launch_split(int64_t rows, int64_t cols, const double* X_hi, const double* X_lo,
                        int64_t ldx, int axis, int ns, int32_t* exps, double* slices, hipStream_t stream,
                        int phases = kSplitAll, bool pairs = false);
// Both operands of a product: exponents and slices, A pair-packed.
hipError_t launch_split_operands(int64_t m, int64_t n, int64_t k, const double* A_hi, const double* A_lo,
                                 int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb, int ns, int32_t* E,
                                 double* A_slices, int32_t* F, double* B_slices, hipStream_t stream);
hipError_t launch_sliced_gemm(int64_t m, int64_t n, int64_t k, int ns, const double* A_slices,
                              const double* B_slices, double* levels, int64_t ldl,
                              const int32_t* E, const int32_t* F, double* C_hi, double* C_lo,
                              int64_t ldc, bool fused, hipStream_t stream, int64_t tile_count = -1);
hipError_t launch_renorm(int64_t m, int64_t n, const double* levels, int64_t ldl, const int32_t* E,
                         const int32_t* F, double* C_hi, double* C_lo, int64_t ldc,
                         hipStream_t stream);
hipError_t launch_probe_mfma(double* out, hipStream_t stream);
// Work geometry of the sliced GEMM for ns slices: one workgroup per output tile
// of tile_m x tile_n, k-blocks of 4 values of k, ks of them per stage; each wave
// issues mfma_per_stage 16x16x4 FP64 instructions per stage, waves_per_simd
// waves of a workgroup share a SIMD, and a workgroup holds lds_bytes of LDS.
// All zero for ns outside 4..16.
struct GemmGeometry {
    int tile_m, tile_n, ks, mfma_per_stage, waves_per_simd, lds_bytes;
};
GemmGeometry gemm_geometry(int ns);

// Split over k for outputs whose tiles leave the chip partly idle: the k-parts' level sums
// are added exactly (atomically, in any order) into zeroed level planes
// [ns][rows][ldl], then turned into the result.  A plan computes the output
// tiles [0, first_tile) (row-major) in one unsplit launch and the tiles from
// first_tile on in `parts` k-parts; first_row is the first row of first_tile's
// tile row, where the level planes start.  parts = 1: no split (first_tile =
// all tiles, first_row = m).  Without `tail` the plan splits the whole product
// or nothing; split_k_parts() is that plan's part count.
struct SplitPlan {
    int64_t first_tile, first_row, parts;
};
SplitPlan split_plan(int64_t m, int64_t n, int64_t k, int ns, bool tail);
int64_t split_k_parts(int64_t m, int64_t n, int64_t k, int ns);
hipError_t launch_zero_levels(int64_t m, int64_t n, int ns, double* levels, int64_t ldl, hipStream_t stream);
// The k-parts of the tiles from tile_first on; their level planes hold the rows
// from tile_first's tile row on (plane stride: those rows times ldl).
hipError_t launch_sliced_gemm_split(int64_t m, int64_t n, int64_t k, int ns, const double* A_slices,
                                    const double* B_slices, double* levels, int64_t ldl, int64_t parts,
                                    hipStream_t stream, int64_t tile_first = 0);
hipError_t launch_levels_to_qd(int64_t m, int64_t n, const double* levels, int64_t ldl, const int32_t* E,
                               const int32_t* F, const OutPlanes& C, int64_t ldc, hipStream_t stream,
                               int64_t plane = -1);
hipError_t launch_dd_accumulate(int64_t m, int64_t n, double* C_hi, double* C_lo, int64_t ldc, const double* T_hi,
                                const double* T_lo, int64_t ldt, hipStream_t stream);
// pairs: an A operand (axis 0) in the pair-packed layout (as launch_split).
hipError_t launch_qd_split(int64_t rows, int64_t cols, const QdPlanes& X, int64_t ldx, int axis, int32_t* exps,
                           double* slices, hipStream_t stream, int phases = kSplitAll, bool pairs = false);
hipError_t launch_qd_exps(int64_t rows, int64_t cols, const QdPlanes& X, int64_t ldx, int axis, int32_t* exps,
                          hipStream_t stream);
hipError_t launch_qd_slices(int64_t rows, int64_t cols, const QdPlanes& X, int64_t ldx, int axis,
                            const int32_t* exps, double* slices, hipStream_t stream, bool pairs = false);
// Quad-double k-blocks that share their balancing exponents: the 16 level sums
// of a block, in integer units, are stored into (first block) or added to
// (later blocks) int64 level planes [16][m][n]; the last block adds its own and
// rounds the exact total to C.
enum QdBlockStep { kQdFirstBlock = 0, kQdMiddleBlock = 1, kQdLastBlock = 2 };
hipError_t launch_qd_gemm_block(int64_t m, int64_t n, int64_t k, const double* A_slices, const double* B_slices,
                                int64_t* units, QdBlockStep step, const int32_t* E, const int32_t* F,
                                const OutPlanes& C, int64_t ldc, hipStream_t stream);
// The same step for a k-block that was split over k: its double level planes
// [16][m][n] (launch_sliced_gemm_split) into the int64 level planes.
hipError_t launch_qd_levels_to_units(int64_t m, int64_t n, const double* levels, int64_t* units, QdBlockStep step,
                                     const int32_t* E, const int32_t* F, const OutPlanes& C, int64_t ldc,
                                     hipStream_t stream);
hipError_t launch_qd_gemm(int64_t m, int64_t n, int64_t k, const double* A_slices, const double* B_slices,
                          const int32_t* E, const int32_t* F, const OutPlanes& C, int64_t ldc,
                          hipStream_t stream, int64_t tile_count = -1);

// The pair-packed schedule (include/ddgemm.h, dd_sliced_gemm_pairs): slices
// 2u and 2u+1 of an A entry as one exact 26-bit operand, so one product of
// 39-bit terms covers two window pairs; ns - 1 group sums per output entry,
// group g counting units 2^(-13(g+3)).
//   pair_products(ns)   matrix products per k-block and 16x16 block (20 for 8);
//   pair_term_max(ns)   the largest |group sum| one value of k can add (all digits 8191);
//   pair_chunk_k(ns)    the most values of k whose FP64 group sums stay below
//                       2^53 units, i.e. exact, in multiples of 16;
//   pair_k_max(ns)      the most values of k whose int64 group sums stay below 2^63.
constexpr int64_t pair_products(int ns) {
    int64_t c = 0;
    for (int u = 0; 2 * u < ns; ++u)
        for (int t = 0; t < ns; ++t)
            if ((2 * u + 1 < ns && 2 * u + 1 + t <= ns - 1) || 2 * u + t == ns - 1) ++c;
    return c;
}
constexpr int64_t pair_term_max(int ns) {
    constexpr int64_t d = (int64_t{1} << kSliceBits) - 1;
    int64_t worst = 0;
    for (int g = 0; g + 1 < ns; ++g) {
        int64_t sum = 0;
        for (int u = 0; 2 * u < ns; ++u)
            for (int t = 0; t < ns; ++t) {
                if (2 * u + 1 < ns && 2 * u + 1 + t <= ns - 1) {
                    if (2 * u + t == g) sum += ((d << kSliceBits) + d) * d;
                } else if (2 * u + t == ns - 1 && g == ns - 2) {
                    sum += d * d;
                }
            }
        worst = sum > worst ? sum : worst;
    }
    return worst;
}
constexpr int64_t pair_chunk_k(int ns) {
    return (((int64_t{1} << 53) - 1) / pair_term_max(ns)) / kPackK * kPackK;
}
constexpr int64_t pair_k_max(int ns) { return INT64_MAX / pair_term_max(ns); }
static_assert(pair_products(8) == 20 && pair_products(16) == 72, "pair-packed product counts");
static_assert(pair_chunk_k(8) == 4096 && pair_chunk_k(16) == 2048, "exact FP64 chunks");
static_assert(pair_k_max(8) == 4194304, "exact int64 group sums");

// What a pair-packed launch produces: the nearest double-double or quad double
// of each entry, or the group sums in int64 units (stage call, split parts).
enum PairOut { kPairToDD = 0, kPairToQD = 1, kPairToUnits = 2 };
// A_prepacked: A_slices in the pair-packed layout (launch_split with pairs),
// else the standard one (the sums of slice pairs are formed in registers).
hipError_t launch_pair_gemm(int64_t m, int64_t n, int64_t k, int ns, const double* A_slices, const double* B_slices,
                            PairOut out, const int32_t* E, const int32_t* F, const OutPlanes& C, int64_t ldc,
                            int64_t* units, int64_t ldu, int64_t plane, int64_t part_stride, int64_t tile_first,
                            int64_t count, int64_t parts, hipStream_t stream, bool A_prepacked = false);
// Geometry of the pair-packed launch for ns slices (mfma_per_stage counts its products).
GemmGeometry pair_geometry(int ns);
// Split parts of a pair-packed product -> results: for the rows x cols block of
// outputs whose group-sum cells start at `units` (group stride `plane`, row
// stride ldu, part stride part_stride), add the parts' sums and round the exact
// total to two (C.c[0..1]) or four words.
hipError_t launch_pair_parts(int64_t rows, int64_t cols, int ns, int words, const int64_t* units, int64_t ldu,
                             int64_t plane, int64_t part_stride, int64_t parts, const int32_t* E, const int32_t* F,
                             const OutPlanes& C, int64_t ldc, hipStream_t stream);
// Split plan of a pair-packed product: tiles [0, first_tile) unsplit, the rest
// in `parts` k-parts whose group sums go to part planes (no atomics).
SplitPlan pair_split_plan(int64_t m, int64_t n, int64_t k, int ns);
// A product of a few outputs and a short k (within one exact chunk) runs as one
// 4-wave workgroup per 16×16 output block when a timing model of that beats
// the tiled kernel's plan; pair_split_plan does not split such a product.
bool pair_small_product(int64_t m, int64_t n, int64_t k, int ns);
hipError_t launch_small_pair_gemm(int64_t m, int64_t n, int64_t k, int ns, int words, const double* A_slices,
                                  const double* B_slices, const int32_t* E, const int32_t* F, const OutPlanes& C,
                                  int64_t ldc, hipStream_t stream);

}  // namespace ddg
