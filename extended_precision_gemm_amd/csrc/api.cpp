// Host side of the C ABI declared in include/ddgemm.h: argument validation,
// device check, workspace layout and stream-ordered launches.  Every argument
// error is detected before any HIP call, so it is reported even on a machine
// without a GPU.
#include <atomic>
#include <cstring>

#include "common.hpp"

using namespace ddg;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// A workspace as a sum of 256-byte aligned regions, each a product of sizes in
// bytes.  The size bound of the arguments (2^58 elements per matrix) does not
// keep 16 level planes of 8-byte sums within 64 bits, so every product and the
// total are checked: past 2^62 bytes the workspace is reported as 0 bytes (no
// such workspace exists), and the entry points reject the sizes.
class Workspace {
  public:
    Workspace& add(uint64_t a, uint64_t b = 1, uint64_t c = 1) {
        uint64_t x = 0;
        if (__builtin_mul_overflow(a, b, &x) || __builtin_mul_overflow(x, c, &x) || x > kMaxBytes)
            ok_ = false;
        else if ((total_ += align_up(x)) > kMaxBytes)
            ok_ = false;
        return *this;
    }
    // Packed slices of one operand (dd_split_slices_bytes_ns or qd_split_slices_bytes):
    // those report 0 bytes for an empty operand and also for one too large to
    // size, which has no workspace.
    Workspace& add_slices(size_t slice_bytes, int64_t outer, int64_t k) {
        if (slice_bytes == 0 && outer > 0 && k > 0) ok_ = false;
        return add(slice_bytes);
    }
    size_t bytes() const { return ok_ ? total_ : 0; }

  private:
    static constexpr uint64_t kMaxBytes = uint64_t(1) << 62;
    uint64_t total_ = 0;
    bool ok_ = true;
};

// Elements spanned by a rows×cols matrix with row stride ld (0 when empty).
inline int64_t extent(int64_t rows, int64_t cols, int64_t ld) {
    return (rows == 0 || cols == 0) ? 0 : (rows - 1) * ld + cols;
}

inline bool overlaps(const void* a, int64_t a_elems, const void* b, int64_t b_elems) {
    if (!a || !b || a_elems == 0 || b_elems == 0) return false;
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + b_elems * 8 && pb < pa + a_elems * 8;
}

// Sizes beyond this would overflow the 64-bit byte counts below.
inline bool size_ok(int64_t a, int64_t b) {
    return a >= 0 && b >= 0 && (a == 0 || b <= (int64_t(1) << 58) / (a > 0 ? a : 1));
}

// A row stride for a rows×cols matrix: at least max(1, cols), and small enough
// that the extent rows·ld (and its bytes) cannot overflow.
inline bool ld_ok(int64_t ld, int64_t rows, int64_t cols) {
    return ld >= (cols > 1 ? cols : 1) && size_ok(rows, ld);
}

std::atomic<int> g_device_state[256];  // 0 unknown, 1 gfx950, 2 unsupported

ddgemm_status_t check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DDGEMM_ERROR_DEVICE;
    if (dev >= 256) return DDGEMM_ERROR_DEVICE;
    int st = g_device_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DDGEMM_ERROR_DEVICE;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? DDGEMM_SUCCESS : DDGEMM_ERROR_DEVICE;
}

inline ddgemm_status_t launched(hipError_t e) { return e == hipSuccess ? DDGEMM_SUCCESS : DDGEMM_ERROR_LAUNCH; }

inline bool ns_ok(int ns) { return ns >= kMinSlices && ns <= kMaxSlices; }

inline int64_t k_max(int ns) { return DDGEMM_K_MAX_NS(ns); }

ddgemm_status_t validate_split(int64_t rows, int64_t cols, const double* X_hi, int64_t ldx, int axis, int ns,
                               const int32_t* exps, const double* slices) {
    if (!size_ok(rows, cols) || !ld_ok(ldx, rows, cols) || (axis != 0 && axis != 1) || !ns_ok(ns))
        return DDGEMM_ERROR_INVALID_VALUE;
    const int64_t outer = axis == 0 ? rows : cols;
    const int64_t k = axis == 0 ? cols : rows;
    if (k > k_max(ns)) return DDGEMM_ERROR_INVALID_VALUE;
    if (rows * cols > 0 && !X_hi) return DDGEMM_ERROR_INVALID_VALUE;
    if (outer > 0 && !exps) return DDGEMM_ERROR_INVALID_VALUE;
    if (dd_split_slices_bytes_ns(outer, k, ns) > 0 && !slices) return DDGEMM_ERROR_INVALID_VALUE;
    return DDGEMM_SUCCESS;
}

ddgemm_status_t validate_sizes(int64_t m, int64_t n, int64_t k) {
    if (!size_ok(m, k) || !size_ok(k, n) || !size_ok(m, n)) return DDGEMM_ERROR_INVALID_VALUE;
    return DDGEMM_SUCCESS;
}

// One sliced product: k within the exact-sum bound.
ddgemm_status_t validate_gemm_dims(int64_t m, int64_t n, int64_t k) {
    if (validate_sizes(m, n, k) != DDGEMM_SUCCESS || k > DDGEMM_K_MAX) return DDGEMM_ERROR_INVALID_VALUE;
    return DDGEMM_SUCCESS;
}

// The product entry points run the pair-packed schedule on k-blocks of at most
// this many values: the slicer's limit and the int64 bound of the group sums.
inline int64_t product_k_max(int ns) { return k_max(ns) < pair_k_max(ns) ? k_max(ns) : pair_k_max(ns); }

bool kblock_ok(int64_t k, int ns, int64_t kblock) { return k == 0 || (kblock >= 1 && kblock <= product_k_max(ns)); }

int64_t block_count(int64_t k, int64_t kblock) { return k == 0 ? 1 : (k + kblock - 1) / kblock; }

// Quad-double operands: a host array of four device pointers per matrix.
ddgemm_status_t read_qd_planes(const double* const X[4], int64_t extent_elems, QdPlanes& out) {
    if (extent_elems == 0) {
        for (int c = 0; c < 4; ++c) out.x[c] = X ? X[c] : nullptr;
        return DDGEMM_SUCCESS;
    }
    if (!X || !X[0]) return DDGEMM_ERROR_INVALID_VALUE;
    for (int c = 0; c < 4; ++c) out.x[c] = X[c];
    return DDGEMM_SUCCESS;
}

// Four output planes: all present, pairwise disjoint.
ddgemm_status_t read_out_planes(double* const C[4], int64_t ce, OutPlanes& out) {
    if (!C) return DDGEMM_ERROR_INVALID_VALUE;
    for (int c = 0; c < 4; ++c) {
        if (!C[c]) return DDGEMM_ERROR_INVALID_VALUE;
        out.c[c] = C[c];
    }
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(C[a], ce, C[b], ce)) return DDGEMM_ERROR_INVALID_VALUE;
    return DDGEMM_SUCCESS;
}

ddgemm_status_t validate_qd_gemm_dims(int64_t m, int64_t n, int64_t k) {
    if (!size_ok(m, k) || !size_ok(k, n) || !size_ok(m, n)) return DDGEMM_ERROR_INVALID_VALUE;
    if (k > QDGEMM_K_MAX) return DDGEMM_ERROR_INVALID_VALUE;
    return DDGEMM_SUCCESS;
}

// The quad-double product in k-blocks: k up to QDGEMM_K_MAX_BLOCKED.
ddgemm_status_t validate_qd_blocked_dims(int64_t m, int64_t n, int64_t k, int64_t kblock) {
    if (!size_ok(m, k) || !size_ok(k, n) || !size_ok(m, n)) return DDGEMM_ERROR_INVALID_VALUE;
    if (k > QDGEMM_K_MAX_BLOCKED) return DDGEMM_ERROR_INVALID_VALUE;
    if (k > 0 && (kblock < 1 || kblock > QDGEMM_K_MAX)) return DDGEMM_ERROR_INVALID_VALUE;
    return DDGEMM_SUCCESS;
}

// All of k when it fits one sliced product, else the fewest equal blocks that do.
// The quad-double product takes the pair-packed schedule when k is one block
// within the group sums' int64 bound (k <= 2^21); longer k keeps the level
// schedule of R23, whose blocks share exponents and add exactly.
bool qd_pairs(int64_t k, int64_t kb) { return kb >= k && k <= pair_k_max(kQdSlices); }

int64_t qd_default_kblock(int64_t k) {
    if (k <= QDGEMM_K_MAX) return k;
    const int64_t blocks = (k + QDGEMM_K_MAX - 1) / QDGEMM_K_MAX;
    return (k + blocks - 1) / blocks;
}

// The split tiles of a plan, from plan.first_tile on, are the rest of the tile
// row holding it, from column c0, and every row below; their level planes
// [ns][m - first_row][n] start at plan.first_row.  `piece(rows, cols, r, c,
// levels)` renormalises the rows x cols block at output (r, c) whose level
// sums start at `levels` (row stride n, plane stride (m - first_row) n).
template <class T, class Piece>
hipError_t renorm_split_tiles(int64_t m, int64_t n, const GemmGeometry& g, const SplitPlan& plan, const T* L,
                              Piece&& piece) {
    const int64_t tiles_n = (n + g.tile_n - 1) / g.tile_n;
    const int64_t r0 = plan.first_row, mt = m - r0;
    const int64_t c0 = plan.first_tile % tiles_n * g.tile_n;
    int64_t done = 0;
    if (c0 > 0) {  // the split tiles of the partly unsplit tile row
        done = g.tile_m < mt ? g.tile_m : mt;
        const hipError_t e = piece(done, n - c0, r0, c0, L + c0);
        if (e != hipSuccess) return e;
    }
    return mt > done ? piece(mt - done, n, r0 + done, int64_t{0}, L + done * n) : hipSuccess;
}

// One k-block of a pair-packed product (A pre-packed) into `out` (words = 2:
// the nearest double-double; 4: the nearest quad double): the small-output
// kernel where pair_small_product picks it; otherwise, with the plan `plan`
// the tiles from plan.first_tile on run in k-parts whose int64 group sums go
// to the part planes P and are added and rounded by one more launch, the
// tiles before it unsplit; a plan that needs more part planes than
// `part_cells` (rows of n entries over all parts) runs unsplit.  U: the chunk
// planes when k exceeds one exact chunk.
hipError_t pair_block_gemm(int64_t m, int64_t n, int64_t kc, int ns, int words, const double* A_sl,
                           const double* B_sl, const int32_t* E, const int32_t* F, const OutPlanes& out, int64_t ldd,
                           int64_t* U, int64_t* P, int64_t part_cells, const SplitPlan& plan, hipStream_t st) {
    if (pair_small_product(m, n, kc, ns))  // a few outputs, a short k: 4-wave workgroups per 16×16 block
        return launch_small_pair_gemm(m, n, kc, ns, words, A_sl, B_sl, E, F, out, ldd, st);
    const PairOut kind = words == 4 ? kPairToQD : kPairToDD;
    const int64_t mn = m * n;
    if (plan.parts <= 1 || plan.parts * (m - plan.first_row) > part_cells)
        return launch_pair_gemm(m, n, kc, ns, A_sl, B_sl, kind, E, F, out, ldd, U, n, mn, 0, 0, -1, 1, st, true);
    hipError_t err = hipSuccess;
    if (plan.first_tile > 0)  // whole rounds of tiles, unsplit
        err = launch_pair_gemm(m, n, kc, ns, A_sl, B_sl, kind, E, F, out, ldd, U, n, mn, 0, 0, plan.first_tile, 1, st,
                               true);
    const int64_t plane = (m - plan.first_row) * n, part_stride = (ns - 1) * plane;
    if (err == hipSuccess)
        err = launch_pair_gemm(m, n, kc, ns, A_sl, B_sl, kPairToUnits, nullptr, nullptr, OutPlanes{}, 0, P, n, plane,
                               part_stride, plan.first_tile, -1, plan.parts, st, true);
    if (err != hipSuccess) return err;
    return renorm_split_tiles(m, n, pair_geometry(ns), plan, static_cast<const int64_t*>(P),
                              [&](int64_t rows, int64_t cols, int64_t r, int64_t c, const int64_t* cells) {
                                  OutPlanes piece = out;
                                  for (int q = 0; q < words; ++q) piece.c[q] = out.c[q] + r * ldd + c;
                                  return launch_pair_parts(rows, cols, ns, words, cells, n, plane, part_stride,
                                                           plan.parts, E + r, F + c, piece, ldd, st);
                              });
}


// Plane c of X advanced by `off` entries (a missing plane stays missing).
QdPlanes offset_planes(const QdPlanes& X, int64_t off) {
    QdPlanes r;
    for (int c = 0; c < 4; ++c) r.x[c] = X.x[c] ? X.x[c] + off : nullptr;
    return r;
}

}  // namespace

namespace ddg {

int64_t default_kblock(int64_t k, int ns) {
    const int64_t km = product_k_max(ns);
    if (k <= km) return k;
    const int64_t blocks = (k + km - 1) / km;
    return (k + blocks - 1) / blocks;
}

ProductCheck check_dd_product(int64_t m, int64_t n, int64_t k, int ns, int64_t kblock, const double* A_hi,
                              const double* A_lo, int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb,
                              const double* C_hi, const double* C_lo, int64_t ldc) {
    const ProductCheck bad{DDGEMM_ERROR_INVALID_VALUE, false, 0};
    if (validate_sizes(m, n, k) != DDGEMM_SUCCESS) return bad;
    if (!ns_ok(ns) || !kblock_ok(k, ns, kblock)) return bad;
    if (!ld_ok(lda, m, k) || !ld_ok(ldb, k, n) || !ld_ok(ldc, m, n)) return bad;
    if (m == 0 || n == 0) return ProductCheck{DDGEMM_SUCCESS, true, 0};
    if (!C_hi || !C_lo || (k > 0 && (!A_hi || !B_hi))) return bad;
    const int64_t ae = extent(m, k, lda), be = extent(k, n, ldb), ce = extent(m, n, ldc);
    for (const double* C : {C_hi, C_lo})
        if (overlaps(C, ce, A_hi, ae) || overlaps(C, ce, A_lo, ae) || overlaps(C, ce, B_hi, be) ||
            overlaps(C, ce, B_lo, be))
            return bad;
    if (overlaps(C_hi, ce, C_lo, ce)) return bad;
    const size_t need = dd_gemm_workspace_size_kb(m, n, k, ns, kblock);
    if (need == 0) return bad;  // the workspace would pass 2^62 bytes
    return ProductCheck{DDGEMM_SUCCESS, false, need};
}

ddgemm_status_t check_current_device() { return check_device(); }

}  // namespace ddg

extern "C" {

size_t dd_split_slices_bytes_ns(int64_t outer, int64_t k, int nslices) {
    if (!ns_ok(nslices) || !size_ok(outer, k) || !size_ok(outer, k * nslices)) return 0;
    return static_cast<size_t>(PackGeom(outer, k).doubles(nslices)) * sizeof(double);
}

size_t dd_split_slices_bytes(int64_t outer, int64_t k) { return dd_split_slices_bytes_ns(outer, k, kSlices); }

size_t dd_gemm_workspace_size_kb(int64_t m, int64_t n, int64_t k, int nslices, int64_t kblock) {
    if (validate_sizes(m, n, k) != DDGEMM_SUCCESS || !ns_ok(nslices) || !kblock_ok(k, nslices, kblock)) return 0;
    const int64_t kb = k < kblock ? k : kblock;
    Workspace ws;
    ws.add_slices(dd_split_slices_bytes_ns(m, kb, nslices), m, kb);
    ws.add_slices(dd_split_slices_bytes_ns(n, kb, nslices), n, kb);
    ws.add(m, 4).add(n, 4);
    if (block_count(k, kblock) > 1) ws.add(m, n, 8).add(m, n, 8);  // (hi, lo) of the blocks after the first
    if (kb > pair_chunk_k(nslices)) ws.add(nslices - 1, m * n, 8);   // int64 group sums between k-chunks
    const SplitPlan plan = pair_split_plan(m, n, kb, nslices);
    if (plan.parts > 1)  // int64 group sums of each k-part of the rows split over k
        ws.add(plan.parts * (nslices - 1), m - plan.first_row, n * 8);
    return ws.bytes();
}

size_t dd_gemm_workspace_size_ns(int64_t m, int64_t n, int64_t k, int nslices) {
    if (!ns_ok(nslices) || k < 0) return 0;
    return dd_gemm_workspace_size_kb(m, n, k, nslices, default_kblock(k, nslices));
}

size_t dd_gemm_workspace_size(int64_t m, int64_t n, int64_t k) { return dd_gemm_workspace_size_ns(m, n, k, kSlices); }

ddgemm_status_t dd_split_balanced_ns(int64_t rows, int64_t cols, const double* X_hi, const double* X_lo,
                                     int64_t ldx, int axis, int nslices, int32_t* exps, double* slices,
                                     void* stream) {
    ddgemm_status_t st = validate_split(rows, cols, X_hi, ldx, axis, nslices, exps, slices);
    if (st != DDGEMM_SUCCESS) return st;
    if ((axis == 0 ? rows : cols) == 0) return DDGEMM_SUCCESS;
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;
    return launched(launch_split(rows, cols, X_hi, X_lo, ldx, axis, nslices, exps, slices,
                                 static_cast<hipStream_t>(stream)));
}

ddgemm_status_t dd_split_balanced(int64_t rows, int64_t cols, const double* X_hi, const double* X_lo,
                                  int64_t ldx, int axis, int32_t* exps, double* slices, void* stream) {
    return dd_split_balanced_ns(rows, cols, X_hi, X_lo, ldx, axis, kSlices, exps, slices, stream);
}

ddgemm_status_t dd_sliced_gemm(int64_t m, int64_t n, int64_t k, const double* A_slices,
                               const double* B_slices, double* levels, int64_t ldl, void* stream) {
    ddgemm_status_t st = validate_gemm_dims(m, n, k);
    if (st != DDGEMM_SUCCESS || !ld_ok(ldl, m, n)) return DDGEMM_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) return DDGEMM_SUCCESS;
    if (!levels || (k > 0 && (!A_slices || !B_slices))) return DDGEMM_ERROR_INVALID_VALUE;
    if (!size_ok(m * ldl, DDGEMM_NUM_LEVELS)) return DDGEMM_ERROR_INVALID_VALUE;
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;
    const int64_t parts = split_k_parts(m, n, k, kSlices);
    if (parts > 1)  // tiles leave the chip partly idle: k-parts add into the zeroed planes
        return launched(launch_sliced_gemm_split(m, n, k, kSlices, A_slices, B_slices, levels, ldl, parts,
                                                 static_cast<hipStream_t>(stream)));
    return launched(launch_sliced_gemm(m, n, k, kSlices, A_slices, B_slices, levels, ldl, nullptr, nullptr,
                                       nullptr, nullptr, 0, false, static_cast<hipStream_t>(stream)));
}

ddgemm_status_t dd_renorm_levels(int64_t m, int64_t n, const double* levels, int64_t ldl,
                                 const int32_t* E, const int32_t* F, double* C_hi, double* C_lo,
                                 int64_t ldc, void* stream) {
    if (!size_ok(m, n) || !ld_ok(ldl, m, n) || !ld_ok(ldc, m, n) || !size_ok(m * ldl, DDGEMM_NUM_LEVELS))
        return DDGEMM_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) return DDGEMM_SUCCESS;
    if (!levels || !E || !F || !C_hi || !C_lo) return DDGEMM_ERROR_INVALID_VALUE;
    const int64_t ce = extent(m, n, ldc);
    if (overlaps(C_hi, ce, C_lo, ce) || overlaps(C_hi, ce, levels, 8 * m * ldl) ||
        overlaps(C_lo, ce, levels, 8 * m * ldl))
        return DDGEMM_ERROR_INVALID_VALUE;
    ddgemm_status_t st = check_device();
    if (st != DDGEMM_SUCCESS) return st;
    return launched(launch_renorm(m, n, levels, ldl, E, F, C_hi, C_lo, ldc, static_cast<hipStream_t>(stream)));
}

ddgemm_status_t dd_sliced_gemm_renorm_ns(int64_t m, int64_t n, int64_t k, int nslices, const double* A_slices,
                                         const int32_t* E, const double* B_slices, const int32_t* F,
                                         double* C_hi, double* C_lo, int64_t ldc, void* stream) {
    ddgemm_status_t st = validate_gemm_dims(m, n, k);
    if (st != DDGEMM_SUCCESS || !ld_ok(ldc, m, n) || !ns_ok(nslices) || k > k_max(nslices))
        return DDGEMM_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) return DDGEMM_SUCCESS;
    if (!E || !F || !C_hi || !C_lo || (k > 0 && (!A_slices || !B_slices))) return DDGEMM_ERROR_INVALID_VALUE;
    const int64_t ce = extent(m, n, ldc);
    if (overlaps(C_hi, ce, C_lo, ce)) return DDGEMM_ERROR_INVALID_VALUE;
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;
    return launched(launch_sliced_gemm(m, n, k, nslices, A_slices, B_slices, nullptr, 0, E, F, C_hi, C_lo, ldc,
                                       true, static_cast<hipStream_t>(stream)));
}

ddgemm_status_t dd_sliced_gemm_renorm(int64_t m, int64_t n, int64_t k, const double* A_slices,
                                      const int32_t* E, const double* B_slices, const int32_t* F,
                                      double* C_hi, double* C_lo, int64_t ldc, void* stream) {
    return dd_sliced_gemm_renorm_ns(m, n, k, kSlices, A_slices, E, B_slices, F, C_hi, C_lo, ldc, stream);
}

ddgemm_status_t dd_sliced_gemm_pairs_ns(int64_t m, int64_t n, int64_t k, int nslices, const double* A_slices,
                                        const double* B_slices, int64_t* units, int64_t ldu, void* stream) {
    if (validate_sizes(m, n, k) != DDGEMM_SUCCESS || !ns_ok(nslices) || k > product_k_max(nslices))
        return DDGEMM_ERROR_INVALID_VALUE;
    if (!ld_ok(ldu, m, n) || !size_ok(m * ldu, nslices - 1)) return DDGEMM_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) return DDGEMM_SUCCESS;
    if (!units || (k > 0 && (!A_slices || !B_slices))) return DDGEMM_ERROR_INVALID_VALUE;
    ddgemm_status_t st = check_device();
    if (st != DDGEMM_SUCCESS) return st;
    const int64_t plane = m * ldu;
    return launched(launch_pair_gemm(m, n, k, nslices, A_slices, B_slices, kPairToUnits, nullptr, nullptr,
                                     OutPlanes{}, 0, units, ldu, plane, 0, 0, -1, 1,
                                     static_cast<hipStream_t>(stream)));
}

ddgemm_status_t dd_sliced_gemm_pairs(int64_t m, int64_t n, int64_t k, const double* A_slices,
                                     const double* B_slices, int64_t* units, int64_t ldu, void* stream) {
    return dd_sliced_gemm_pairs_ns(m, n, k, kSlices, A_slices, B_slices, units, ldu, stream);
}

}  // extern "C"

namespace {

// dd_gemm_ws_kb, and with after_split an event recorded on the stream once the
// first k-block's operands are sliced (dd_gemm_ws_timed).
ddgemm_status_t product_kb(int64_t m, int64_t n, int64_t k, int nslices, int64_t kblock, const double* A_hi,
                           const double* A_lo, int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb,
                           double* C_hi, double* C_lo, int64_t ldc, void* workspace, size_t ws_bytes, void* stream,
                           void* after_split) {
    const ProductCheck chk =
        check_dd_product(m, n, k, nslices, kblock, A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi, C_lo, ldc);
    if (chk.status != DDGEMM_SUCCESS || chk.empty) return chk.status;
    const size_t need = chk.need;
    ddgemm_status_t st;
    if (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return DDGEMM_ERROR_WORKSPACE;
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;

    const int64_t kb = k < kblock ? k : kblock;
    const int64_t blocks = block_count(k, kb);
    char* w = static_cast<char*>(workspace);
    double* A_sl = reinterpret_cast<double*>(w);
    w += align_up(dd_split_slices_bytes_ns(m, kb, nslices));
    double* B_sl = reinterpret_cast<double*>(w);
    w += align_up(dd_split_slices_bytes_ns(n, kb, nslices));
    int32_t* E = reinterpret_cast<int32_t*>(w);
    w += align_up(static_cast<size_t>(m) * 4);
    int32_t* F = reinterpret_cast<int32_t*>(w);
    w += align_up(static_cast<size_t>(n) * 4);
    double* T_hi = reinterpret_cast<double*>(w);  // block results after the first (blocks > 1)
    double* T_lo = T_hi + (blocks > 1 ? align_up(static_cast<size_t>(m) * static_cast<size_t>(n) * 8) / 8 : 0);
    if (blocks > 1) w += 2 * align_up(static_cast<size_t>(m) * static_cast<size_t>(n) * 8);
    const int ns = nslices;
    int64_t* U = nullptr;  // int64 group sums [ns-1][m][n] between k-chunks
    if (kb > pair_chunk_k(ns)) {
        U = reinterpret_cast<int64_t*>(w);
        w += align_up(static_cast<size_t>(ns - 1) * static_cast<size_t>(m) * static_cast<size_t>(n) * 8);
    }
    int64_t* P = reinterpret_cast<int64_t*>(w);  // part planes [parts][ns-1][rows][n] of the rows split over k
    const SplitPlan plan_kb = pair_split_plan(m, n, kb, ns);
    const int64_t part_cells = plan_kb.parts > 1 ? plan_kb.parts * (m - plan_kb.first_row) : 0;

    // One block's product into (hi, lo) planes (see pair_block_gemm); a shorter
    // last block is planned for its own k.
    auto block_gemm = [&](int64_t kc, double* d_hi, double* d_lo, int64_t ldd, hipStream_t st) {
        const SplitPlan plan = kc == kb ? plan_kb : pair_split_plan(m, n, kc, ns);
        return pair_block_gemm(m, n, kc, ns, 2, A_sl, B_sl, E, F, OutPlanes{{d_hi, d_lo, nullptr, nullptr}}, ldd, U,
                               P, part_cells, plan, st);
    };

    // Block b covers k indices [b kb, min(k, (b+1) kb)): a separate sliced product
    // with its own exponents; blocks after the first are added into C in
    // double-double arithmetic, in order, on the caller's stream.
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    for (int64_t b = 0; b < blocks && e == hipSuccess; ++b) {
        const int64_t p0 = b * kb;
        const int64_t kc = k - p0 < kb ? k - p0 : kb;
        const double* a_hi = A_hi ? A_hi + p0 : nullptr;
        const double* a_lo = A_lo ? A_lo + p0 : nullptr;
        const double* b_hi = B_hi ? B_hi + p0 * ldb : nullptr;
        const double* b_lo = B_lo ? B_lo + p0 * ldb : nullptr;
        // A in the pair-packed layout the product's GEMM reads
        e = launch_split_operands(m, n, kc, a_hi, a_lo, lda, b_hi, b_lo, ldb, nslices, E, A_sl, F, B_sl, s);
        if (e == hipSuccess && b == 0 && after_split) e = hipEventRecord(static_cast<hipEvent_t>(after_split), s);
        if (e != hipSuccess) break;
        if (b == 0) {
            e = block_gemm(kc, C_hi, C_lo, ldc, s);
        } else {
            e = block_gemm(kc, T_hi, T_lo, n, s);
            if (e == hipSuccess) e = launch_dd_accumulate(m, n, C_hi, C_lo, ldc, T_hi, T_lo, n, s);
        }
    }
    return launched(e);
}

}  // namespace

extern "C" {

ddgemm_status_t dd_gemm_ws_kb(int64_t m, int64_t n, int64_t k, int nslices, int64_t kblock, const double* A_hi,
                              const double* A_lo, int64_t lda, const double* B_hi, const double* B_lo,
                              int64_t ldb, double* C_hi, double* C_lo, int64_t ldc, void* workspace,
                              size_t ws_bytes, void* stream) {
    return product_kb(m, n, k, nslices, kblock, A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi, C_lo, ldc, workspace,
                      ws_bytes, stream, nullptr);
}

ddgemm_status_t dd_gemm_ws_timed(int64_t m, int64_t n, int64_t k, int nslices, const double* A_hi,
                                 const double* A_lo, int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb,
                                 double* C_hi, double* C_lo, int64_t ldc, void* workspace, size_t ws_bytes,
                                 void* after_split, void* stream) {
    if (k < 0 || !ns_ok(nslices)) return DDGEMM_ERROR_INVALID_VALUE;
    return product_kb(m, n, k, nslices, default_kblock(k, nslices), A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi, C_lo,
                      ldc, workspace, ws_bytes, stream, after_split);
}

int64_t dd_gemm_kblock_max(int nslices) { return ns_ok(nslices) ? product_k_max(nslices) : 0; }

ddgemm_status_t dd_gemm_ws_ns(int64_t m, int64_t n, int64_t k, int nslices, const double* A_hi,
                              const double* A_lo, int64_t lda, const double* B_hi, const double* B_lo,
                              int64_t ldb, double* C_hi, double* C_lo, int64_t ldc, void* workspace,
                              size_t ws_bytes, void* stream) {
    if (!ns_ok(nslices) || k < 0) return DDGEMM_ERROR_INVALID_VALUE;
    return dd_gemm_ws_kb(m, n, k, nslices, default_kblock(k, nslices), A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi,
                         C_lo, ldc, workspace, ws_bytes, stream);
}

ddgemm_status_t dd_gemm_ws(int64_t m, int64_t n, int64_t k, const double* A_hi, const double* A_lo,
                           int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb,
                           double* C_hi, double* C_lo, int64_t ldc, void* workspace, size_t ws_bytes,
                           void* stream) {
    return dd_gemm_ws_ns(m, n, k, kSlices, A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi, C_lo, ldc, workspace,
                         ws_bytes, stream);
}

ddgemm_status_t dd_gemm(int64_t m, int64_t n, int64_t k, const double* A_hi, const double* A_lo,
                        int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb, double* C_hi,
                        double* C_lo, int64_t ldc, void* stream) {
    ddgemm_status_t st = validate_sizes(m, n, k);
    if (st != DDGEMM_SUCCESS) return st;
    if (!ld_ok(lda, m, k) || !ld_ok(ldb, k, n) || !ld_ok(ldc, m, n)) return DDGEMM_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) return DDGEMM_SUCCESS;
    if (!C_hi || !C_lo || (k > 0 && (!A_hi || !B_hi))) return DDGEMM_ERROR_INVALID_VALUE;
    const size_t need = dd_gemm_workspace_size(m, n, k);
    if (need == 0) return DDGEMM_ERROR_INVALID_VALUE;  // the workspace would pass 2^62 bytes
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, need, s) != hipSuccess || !ws) return DDGEMM_ERROR_WORKSPACE;
    st = dd_gemm_ws(m, n, k, A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi, C_lo, ldc, ws, need, stream);
    if (hipFreeAsync(ws, s) != hipSuccess && st == DDGEMM_SUCCESS) st = DDGEMM_ERROR_LAUNCH;
    return st;
}

size_t qd_split_slices_bytes(int64_t outer, int64_t k) {
    if (!size_ok(outer, k) || !size_ok(outer, k * kQdSlices)) return 0;
    return static_cast<size_t>(PackGeom(outer, k).doubles(kQdSlices)) * sizeof(double);
}

size_t qd_gemm_workspace_size_kb(int64_t m, int64_t n, int64_t k, int64_t kblock) {
    if (validate_qd_blocked_dims(m, n, k, kblock) != DDGEMM_SUCCESS) return 0;
    const int64_t kb = k < kblock ? k : kblock;
    const bool blocked = block_count(k, kb) > 1;
    Workspace ws;
    ws.add_slices(qd_split_slices_bytes(m, kb), m, kb).add_slices(qd_split_slices_bytes(n, kb), n, kb);
    ws.add(m, 4).add(n, 4);
    if (qd_pairs(k, kb)) {
        if (kb > pair_chunk_k(kQdSlices)) ws.add(kQdSlices - 1, m * n, 8);  // int64 group sums between k-chunks
        const SplitPlan plan = pair_split_plan(m, n, kb, kQdSlices);
        if (plan.parts > 1)  // int64 group sums of each k-part of the rows split over k
            ws.add(plan.parts * (kQdSlices - 1), m - plan.first_row, n * 8);
        return ws.bytes();
    }
    // a blocked product's blocks split whole or not at all; one block may split its later rows only
    const SplitPlan plan = split_plan(m, n, kb, kQdSlices, !blocked);
    if (blocked) ws.add(QDGEMM_NUM_LEVELS, m, n * 8);  // int64 level planes of a blocked product
    if (plan.parts > 1)                                // double level planes of the rows split over k
        ws.add(QDGEMM_NUM_LEVELS, m - plan.first_row, n * 8);
    return ws.bytes();
}

size_t qd_gemm_workspace_size(int64_t m, int64_t n, int64_t k) {
    if (k < 0) return 0;
    return qd_gemm_workspace_size_kb(m, n, k, qd_default_kblock(k));
}

ddgemm_status_t qd_split_balanced(int64_t rows, int64_t cols, const double* const X[4], int64_t ldx, int axis,
                                  int32_t* exps, double* slices, void* stream) {
    if (!size_ok(rows, cols) || !ld_ok(ldx, rows, cols) || (axis != 0 && axis != 1)) return DDGEMM_ERROR_INVALID_VALUE;
    const int64_t outer = axis == 0 ? rows : cols;
    const int64_t k = axis == 0 ? cols : rows;
    if (k > QDGEMM_K_MAX) return DDGEMM_ERROR_INVALID_VALUE;
    QdPlanes planes;
    ddgemm_status_t st = read_qd_planes(X, rows * cols, planes);
    if (st != DDGEMM_SUCCESS) return st;
    if (outer > 0 && !exps) return DDGEMM_ERROR_INVALID_VALUE;
    if (qd_split_slices_bytes(outer, k) > 0 && !slices) return DDGEMM_ERROR_INVALID_VALUE;
    if (outer == 0) return DDGEMM_SUCCESS;
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;
    return launched(launch_qd_split(rows, cols, planes, ldx, axis, exps, slices, static_cast<hipStream_t>(stream)));
}

ddgemm_status_t qd_sliced_gemm_renorm(int64_t m, int64_t n, int64_t k, const double* A_slices, const int32_t* E,
                                      const double* B_slices, const int32_t* F, double* const C[4], int64_t ldc,
                                      void* stream) {
    ddgemm_status_t st = validate_qd_gemm_dims(m, n, k);
    if (st != DDGEMM_SUCCESS || !ld_ok(ldc, m, n)) return DDGEMM_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) return DDGEMM_SUCCESS;
    OutPlanes out;
    if ((st = read_out_planes(C, extent(m, n, ldc), out)) != DDGEMM_SUCCESS) return st;
    if (!E || !F || (k > 0 && (!A_slices || !B_slices))) return DDGEMM_ERROR_INVALID_VALUE;
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;
    return launched(launch_qd_gemm(m, n, k, A_slices, B_slices, E, F, out, ldc, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The quad-double product; `after_split` (a hipEvent_t, or null) is recorded
// on the stream once the first k-block's operands are sliced.
ddgemm_status_t qd_product_kb(int64_t m, int64_t n, int64_t k, int64_t kblock, const double* const A[4],
                              int64_t lda, const double* const B[4], int64_t ldb, double* const C[4], int64_t ldc,
                              void* workspace, size_t ws_bytes, void* stream, void* after_split) {
    ddgemm_status_t st = validate_qd_blocked_dims(m, n, k, kblock);
    if (st != DDGEMM_SUCCESS) return st;
    if (!ld_ok(lda, m, k) || !ld_ok(ldb, k, n) || !ld_ok(ldc, m, n)) return DDGEMM_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) return DDGEMM_SUCCESS;
    const int64_t ae = extent(m, k, lda), be = extent(k, n, ldb), ce = extent(m, n, ldc);
    QdPlanes pa, pb;
    OutPlanes out;
    if ((st = read_qd_planes(A, m * k, pa)) != DDGEMM_SUCCESS) return st;
    if ((st = read_qd_planes(B, k * n, pb)) != DDGEMM_SUCCESS) return st;
    if ((st = read_out_planes(C, ce, out)) != DDGEMM_SUCCESS) return st;
    for (int c = 0; c < 4; ++c)
        for (int q = 0; q < 4; ++q)
            if (overlaps(out.c[c], ce, pa.x[q], ae) || overlaps(out.c[c], ce, pb.x[q], be))
                return DDGEMM_ERROR_INVALID_VALUE;
    const size_t need = qd_gemm_workspace_size_kb(m, n, k, kblock);
    if (need == 0) return DDGEMM_ERROR_INVALID_VALUE;  // the workspace would pass 2^62 bytes
    if (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return DDGEMM_ERROR_WORKSPACE;
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;

    const int64_t kb = k < kblock ? k : kblock;
    const int64_t blocks = block_count(k, kb);
    const bool split = split_k_parts(m, n, kb, kQdSlices) > 1;
    char* w = static_cast<char*>(workspace);
    double* A_sl = reinterpret_cast<double*>(w);
    w += align_up(qd_split_slices_bytes(m, kb));
    double* B_sl = reinterpret_cast<double*>(w);
    w += align_up(qd_split_slices_bytes(n, kb));
    int32_t* E = reinterpret_cast<int32_t*>(w);
    w += align_up(static_cast<size_t>(m) * 4);
    int32_t* F = reinterpret_cast<int32_t*>(w);
    w += align_up(static_cast<size_t>(n) * 4);
    int64_t* units = reinterpret_cast<int64_t*>(w);  // [16][m][n] int64 level sums of the blocks (blocks > 1)
    if (blocks > 1) w += align_up(static_cast<size_t>(m) * static_cast<size_t>(n) * 8 * QDGEMM_NUM_LEVELS);
    double* L = reinterpret_cast<double*>(w);        // [16][m][n] double level planes of a split product

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (qd_pairs(k, kb)) {
        // the pair-packed schedule (R25) with the nearest quad double of each
        // entry's exact total; A sliced pre-packed
        int64_t* U = reinterpret_cast<int64_t*>(w);  // [15][m][n] group sums between k-chunks
        if (k > pair_chunk_k(kQdSlices))
            w += align_up(static_cast<size_t>(kQdSlices - 1) * static_cast<size_t>(m) * static_cast<size_t>(n) * 8);
        int64_t* P = reinterpret_cast<int64_t*>(w);  // part planes of the rows split over k
        const SplitPlan plan = pair_split_plan(m, n, k, kQdSlices);
        const int64_t part_cells = plan.parts > 1 ? plan.parts * (m - plan.first_row) : 0;
        hipError_t e = launch_qd_split(m, k, pa, lda, 0, E, A_sl, s, kSplitExps);  // both exponent passes first
        if (e == hipSuccess) e = launch_qd_split(k, n, pb, ldb, 1, F, B_sl, s, kSplitExps);
        if (e == hipSuccess) e = launch_qd_split(k, n, pb, ldb, 1, F, B_sl, s, kSplitSlices);
        if (e == hipSuccess) e = launch_qd_split(m, k, pa, lda, 0, E, A_sl, s, kSplitSlices, true);
        if (e == hipSuccess && after_split) e = hipEventRecord(static_cast<hipEvent_t>(after_split), s);
        if (e == hipSuccess)
            e = pair_block_gemm(m, n, k, kQdSlices, 4, A_sl, B_sl, E, F, out, ldc, U, P, part_cells, plan, s);
        return launched(e);
    }
    if (blocks == 1) {
        hipError_t e = launch_qd_split(m, k, pa, lda, 0, E, A_sl, s, kSplitExps);  // both exponent passes first
        if (e == hipSuccess) e = launch_qd_split(k, n, pb, ldb, 1, F, B_sl, s, kSplitExps);
        if (e == hipSuccess) e = launch_qd_split(k, n, pb, ldb, 1, F, B_sl, s, kSplitSlices);
        if (e == hipSuccess) e = launch_qd_split(m, k, pa, lda, 0, E, A_sl, s, kSplitSlices);
        if (e == hipSuccess && after_split) e = hipEventRecord(static_cast<hipEvent_t>(after_split), s);
        const SplitPlan plan = split_plan(m, n, k, kQdSlices, true);
        if (e == hipSuccess && plan.parts > 1) {  // tiles leave the chip partly idle: the last ones split over k
            if (plan.first_tile > 0) e = launch_qd_gemm(m, n, k, A_sl, B_sl, E, F, out, ldc, s, plan.first_tile);
            if (e == hipSuccess)
                e = launch_sliced_gemm_split(m, n, k, kQdSlices, A_sl, B_sl, L, n, plan.parts, s, plan.first_tile);
            const int64_t plane = (m - plan.first_row) * n;
            if (e == hipSuccess)
                e = renorm_split_tiles(m, n, gemm_geometry(kQdSlices), plan, L, [&](int64_t rows, int64_t cols, int64_t r,
                                                                     int64_t c, const double* lv) {
                    OutPlanes piece_out = out;
                    for (int q = 0; q < 4; ++q) piece_out.c[q] = out.c[q] + r * ldc + c;
                    return launch_levels_to_qd(rows, cols, lv, n, E + r, F + c, piece_out, ldc, s, plane);
                });
        } else if (e == hipSuccess) {
            e = launch_qd_gemm(m, n, k, A_sl, B_sl, E, F, out, ldc, s);
        }
        return launched(e);
    }
    // Exponents of the whole rows of A / columns of B; block b covers k indices
    // [b kb, min(k, (b+1) kb)) and is sliced below them, so the blocks' level
    // sums add exactly; the last block rounds the total.
    hipError_t e = launch_qd_exps(m, k, pa, lda, 0, E, s);
    if (e == hipSuccess) e = launch_qd_exps(k, n, pb, ldb, 1, F, s);
    for (int64_t b = 0; b < blocks && e == hipSuccess; ++b) {
        const int64_t p0 = b * kb;
        const int64_t kc = k - p0 < kb ? k - p0 : kb;
        e = launch_qd_slices(m, kc, offset_planes(pa, p0), lda, 0, E, A_sl, s);
        if (e == hipSuccess) e = launch_qd_slices(kc, n, offset_planes(pb, p0 * ldb), ldb, 1, F, B_sl, s);
        if (e == hipSuccess && b == 0 && after_split) e = hipEventRecord(static_cast<hipEvent_t>(after_split), s);
        if (e != hipSuccess) break;
        const QdBlockStep step = b == 0 ? kQdFirstBlock : (b + 1 == blocks ? kQdLastBlock : kQdMiddleBlock);
        const int64_t parts = split ? split_k_parts(m, n, kc, kQdSlices) : 1;
        if (parts > 1) {  // this block split over k, then its exact level sums into the int64 planes
            e = launch_sliced_gemm_split(m, n, kc, kQdSlices, A_sl, B_sl, L, n, parts, s);
            if (e == hipSuccess) e = launch_qd_levels_to_units(m, n, L, units, step, E, F, out, ldc, s);
        } else {
            e = launch_qd_gemm_block(m, n, kc, A_sl, B_sl, units, step, E, F, out, ldc, s);
        }
    }
    return launched(e);
}

}  // namespace

extern "C" {

ddgemm_status_t qd_gemm_ws_kb(int64_t m, int64_t n, int64_t k, int64_t kblock, const double* const A[4],
                              int64_t lda, const double* const B[4], int64_t ldb, double* const C[4], int64_t ldc,
                              void* workspace, size_t ws_bytes, void* stream) {
    return qd_product_kb(m, n, k, kblock, A, lda, B, ldb, C, ldc, workspace, ws_bytes, stream, nullptr);
}

ddgemm_status_t qd_gemm_ws_timed(int64_t m, int64_t n, int64_t k, const double* const A[4], int64_t lda,
                                 const double* const B[4], int64_t ldb, double* const C[4], int64_t ldc,
                                 void* workspace, size_t ws_bytes, void* after_split, void* stream) {
    if (k < 0) return DDGEMM_ERROR_INVALID_VALUE;
    return qd_product_kb(m, n, k, qd_default_kblock(k), A, lda, B, ldb, C, ldc, workspace, ws_bytes, stream,
                         after_split);
}

ddgemm_status_t qd_gemm_ws(int64_t m, int64_t n, int64_t k, const double* const A[4], int64_t lda,
                           const double* const B[4], int64_t ldb, double* const C[4], int64_t ldc,
                           void* workspace, size_t ws_bytes, void* stream) {
    if (k < 0) return DDGEMM_ERROR_INVALID_VALUE;
    return qd_gemm_ws_kb(m, n, k, qd_default_kblock(k), A, lda, B, ldb, C, ldc, workspace, ws_bytes, stream);
}

ddgemm_status_t qd_gemm(int64_t m, int64_t n, int64_t k, const double* const A[4], int64_t lda,
                        const double* const B[4], int64_t ldb, double* const C[4], int64_t ldc, void* stream) {
    if (k < 0) return DDGEMM_ERROR_INVALID_VALUE;
    ddgemm_status_t st = validate_qd_blocked_dims(m, n, k, qd_default_kblock(k));
    if (st != DDGEMM_SUCCESS) return st;
    if (!ld_ok(lda, m, k) || !ld_ok(ldb, k, n) || !ld_ok(ldc, m, n)) return DDGEMM_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) return DDGEMM_SUCCESS;
    QdPlanes pa, pb;
    OutPlanes out;
    if ((st = read_qd_planes(A, m * k, pa)) != DDGEMM_SUCCESS) return st;
    if ((st = read_qd_planes(B, k * n, pb)) != DDGEMM_SUCCESS) return st;
    if ((st = read_out_planes(C, extent(m, n, ldc), out)) != DDGEMM_SUCCESS) return st;
    const size_t need = qd_gemm_workspace_size(m, n, k);
    if (need == 0) return DDGEMM_ERROR_INVALID_VALUE;  // the workspace would pass 2^62 bytes
    if ((st = check_device()) != DDGEMM_SUCCESS) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, need, s) != hipSuccess || !ws) return DDGEMM_ERROR_WORKSPACE;
    st = qd_gemm_ws(m, n, k, A, lda, B, ldb, C, ldc, ws, need, stream);
    if (hipFreeAsync(ws, s) != hipSuccess && st == DDGEMM_SUCCESS) st = DDGEMM_ERROR_LAUNCH;
    return st;
}

const char* ddgemm_status_string(ddgemm_status_t status) {
    switch (status) {
        case DDGEMM_SUCCESS: return "DDGEMM_SUCCESS";
        case DDGEMM_ERROR_INVALID_VALUE: return "DDGEMM_ERROR_INVALID_VALUE: invalid argument";
        case DDGEMM_ERROR_WORKSPACE: return "DDGEMM_ERROR_WORKSPACE: workspace missing, too small or misaligned";
        case DDGEMM_ERROR_LAUNCH: return "DDGEMM_ERROR_LAUNCH: a HIP launch or runtime call failed";
        case DDGEMM_ERROR_DEVICE: return "DDGEMM_ERROR_DEVICE: no current gfx950 device";
    }
    return "unknown ddgemm status";
}

}  // extern "C"

namespace {
// The split plan a product entry point takes: the pair-packed schedule's, but
// for 16 slices beyond the pair-packed int64 bound, where the quad-double
// product keeps the level schedule.
SplitPlan product_plan(int64_t m, int64_t n, int64_t k, int ns) {
    return ns == kQdSlices && k > pair_k_max(ns) ? split_plan(m, n, k, ns, true) : pair_split_plan(m, n, k, ns);
}
}  // namespace

extern "C" {

int64_t ddgemm_split_parts(int64_t m, int64_t n, int64_t k, int nslices) {
    if (!ns_ok(nslices) || validate_sizes(m, n, k) != DDGEMM_SUCCESS) return 0;
    return product_plan(m, n, k, nslices).parts;
}

int64_t ddgemm_split_first_row(int64_t m, int64_t n, int64_t k, int nslices) {
    if (!ns_ok(nslices) || validate_sizes(m, n, k) != DDGEMM_SUCCESS) return -1;
    const SplitPlan plan = product_plan(m, n, k, nslices);
    return plan.parts > 1 ? plan.first_row : m;
}

int ddgemm_small_product(int64_t m, int64_t n, int64_t k, int nslices) {
    if (!ns_ok(nslices) || validate_sizes(m, n, k) != DDGEMM_SUCCESS) return 0;
    return pair_small_product(m, n, k, nslices) ? 1 : 0;
}

int64_t ddgemm_split_first_tile(int64_t m, int64_t n, int64_t k, int nslices) {
    if (!ns_ok(nslices) || validate_sizes(m, n, k) != DDGEMM_SUCCESS) return -1;
    return product_plan(m, n, k, nslices).first_tile;
}

ddgemm_status_t ddgemm_probe_mfma_f64(double* out, void* stream) {
    if (!out) return DDGEMM_ERROR_INVALID_VALUE;
    ddgemm_status_t st = check_device();
    if (st != DDGEMM_SUCCESS) return st;
    return launched(launch_probe_mfma(out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
