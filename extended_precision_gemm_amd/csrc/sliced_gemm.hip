// Sliced GEMM on gfx950 FP64 matrix cores ("Multiple Double Arithmetic on NVIDIA
// Tensor Cores", §2 eqs. (1)-(4); exactness from §2 eq. (5)).
//
// Level l = s + t of output entry (i, j) is S_l = sum_{s+t=l} sum_p A_s[i][p] B_t[p][j]
// for l = 0..7: the 36 slice pairs inside the double-double window.  Instead of
// the pages' single product with a block-Toeplitz right operand (28 of whose 64
// blocks are zero), each k step issues exactly the 36 nonzero pair products, one
// v_mfma_f64_16x16x4_f64 per pair and 16x16 output block, into one accumulator
// per level.  Slices are 13-bit integers times powers of two, so every product
// is exact and every partial sum is an integer multiple of 2^(-13(l+2)) below
// 2^53 units: the matrix-core accumulation is exact in any order.
//
// Work split: each wave computes a (16 RPW)x16 strip (RPW 16x16 blocks stacked;
// RPW = 2 for 4, 5, 7 and 8 slices, 1 for 6 and for 9 to 16) with one accumulator
// per level and block; a workgroup of WM x WN waves owns a (16 RPW WM) x (16 WN)
// output tile; at least two waves share each SIMD (with six slices a workgroup
// takes 72 KB of LDS and two fit a CU, four waves per SIMD).  The same kernel serves the quad-double product:
// sixteen slices, 136 pairs, sixteen levels, and the exact four-double
// epilogue (or, for a k-block of a longer product, the level sums in integer
// units added into int64 planes).  The operand panels move through LDS in stages
// of KS k-blocks (4 values of k each): every (16x4 or 4x16) fragment of one
// slice is 64 consecutive doubles in the packed planes, so a stage of one
// 16-row (16-column) block is a contiguous KS x 4 KB run, copied with 16-byte
// direct-to-LDS loads and read back by the waves as conflict-free
// 8-byte-per-lane fragment reads straight into the matrix-instruction operand
// registers.  NBUF stages are in flight; one workgroup barrier per stage.
#include "common.hpp"
#include "dispatch_ns.hpp"
#include "eft.hpp"
#include "pair_levels.hpp"
#include "qd_levels.hpp"

namespace ddg {
namespace {

// Result layout of the FP64 16x16x4 instruction, as measured with the probe
// entry point on gfx950: lane L holds rows L/16 + 4v, v = 0..3, of column L % 16.
__device__ __forceinline__ int frag_row(int lane, int v) { return (lane >> 4) + 4 * v; }
__device__ __forceinline__ int frag_col(int lane) { return lane & 15; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_void_t;

// A value the whole wave holds, moved to scalar registers (a 64-bit division of
// uniform operands is otherwise left in vector registers).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Order the compiler's memory operations around a hardware barrier or wait
// without adding any instruction.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ISSUE: where a stage's copy of a later stage is issued -- 0 after the first
// k-block's fragment reads (halfway through a stage of two k-blocks), 1 right
// after the stage's barrier, before any fragment read.
// DEFER (pair-packed schedule only): the last DEFER products of a stage's last
// k-block are issued after the next stage's barrier, beside its first fragment
// reads, so that the matrix pipe has work while those reads are in flight.
template <int WM, int WN, int KS, int NBUF, int WGS, int NS, int RPW = 2, int ISSUE = 0, int DEFER = 0>
struct GemmConfig {
    static constexpr int kIssueEarly = ISSUE;
    static constexpr int kDefer = DEFER;
    static constexpr int kWaves = WM * WN;
    static constexpr int kRPW = RPW;                                 // 16-row blocks per wave
    static constexpr int kNBuf = NBUF;
    static constexpr int kWGS = WGS;
    static constexpr int kNS = NS;                                   // slices per operand entry
    static constexpr int kSetDoubles = NS * kFragDoubles;            // one fragment, all slices
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kTBM = RPW * WM;                            // 16-row blocks per tile
    static constexpr int kTBN = WN;                                  // 16-column blocks per tile
    static constexpr int kKS = KS;
    static constexpr int kBlockStage = KS * kSetDoubles;             // one block, one stage
    static constexpr int kStageDoubles = (kTBM + kTBN) * kBlockStage;
    static constexpr int kPieces = kStageDoubles / 128;               // 1 KB pieces per stage
    static constexpr int kPiecesPerWave = (kPieces + kWaves - 1) / kWaves;
    static constexpr bool kEvenPieces = kPieces % kWaves == 0;
    static_assert(kStageDoubles % 128 == 0, "a stage is whole 1 KB pieces");
    static_assert(kEvenPieces || NBUF == 2, "uneven copies rely on the full wait of two stages");
    static_assert(NBUF >= 2 && WGS * NBUF * kStageDoubles * 8 <= 160 * 1024, "LDS budget");
    static_assert(kPackOuter % (16 * kTBM) == 0 && kPackOuter % (16 * kTBN) == 0, "tile divides the packing");
    static_assert(kPackK % (4 * KS) == 0, "stage divides the k packing");
};

// What the epilogue does with the NS level sums of an output entry.
enum Epilogue : int {
    kEpiLevels = 0,    // store them as doubles to level planes
    kEpiDD = 1,        // cascade them into (hi, lo)
    kEpiQD = 2,        // round their exact total to four doubles
    kEpiUnitsSet = 3,  // store them in integer units to int64 planes
    kEpiUnitsAdd = 4,  // add them in integer units to the int64 planes
    kEpiUnitsQD = 5,   // add them to the int64 planes' values and round that total
    kEpiAtomicLevels = 6,  // add them, as doubles, into level planes (one k-part of a split product)
    kEpiPairUnits = 7,     // pair-packed schedule: store its group sums in integer units to int64 planes
};

// One product of the pair-packed schedule: A operand u (slices 2u and 2u+1
// packed, or slice 2u alone), B slice t, into accumulator acc.
struct PairProduct {
    int u, t, acc;
    bool packed;
};

// The products of one k-block for NS slices, in issue order: round i holds
// the i-th product of every accumulator that has one, accumulators 0..NS-2
// being the groups 2u + t of the packed products and NS - 1 the single ones.
template <int NS>
struct PairSchedule {
    static constexpr int kMax = NS * NS;
    PairProduct order[kMax] = {};
    int count = 0;
    constexpr PairSchedule() {
        PairProduct all[kMax] = {};
        int per_acc[NS] = {};
        int n = 0;
        for (int u = 0; 2 * u < NS; ++u)
            for (int t = 0; t < NS; ++t) {
                if (2 * u + 1 < NS && 2 * u + 1 + t <= NS - 1)
                    all[n++] = PairProduct{u, t, 2 * u + t, true};
                else if (2 * u + t == NS - 1)
                    all[n++] = PairProduct{u, t, NS - 1, false};
            }
        for (int i = 0; i < n; ++i) ++per_acc[all[i].acc];
        int most = 0;
        for (int g = 0; g < NS; ++g) most = per_acc[g] > most ? per_acc[g] : most;
        for (int round = 0; round < most; ++round)
            for (int g = 0; g < NS; ++g) {
                int seen = 0;
                for (int i = 0; i < n; ++i)
                    if (all[i].acc == g && seen++ == round) order[count++] = all[i];
            }
    }
};

// Extra arguments of the pair-packed schedule.  Every chunk_stages stages of
// k (0: never) the exact group sums leave the accumulators for int64 planes,
// so that no FP64 sum ever holds more than the terms it adds exactly;
// `units` + blockIdx.y part_stride + g plane + (row - row_off) ldl + col is
// the cell of group g of output (row, col) in those planes (k-part blockIdx.y
// of a split product).
struct PairArgs {
    int64_t chunk_stages, part_stride, row_off;
};

// The second launch bound is the minimum number of waves per SIMD (four SIMDs
// per CU): kWGS workgroups of kWaves waves.
//
// PAIRED selects the pair-packed schedule (include/ddgemm.h,
// dd_sliced_gemm_pairs): slices 2u and 2u+1 of A are added into one exact
// 26-bit operand in registers, and each product covers two window pairs, NS - 1
// group accumulators in place of NS levels (20 products per k-block for eight
// slices instead of 36).
// PREPACKED (pair-packed schedule only): A_slices come in the pair-packed
// layout (plane 2u = slices 2u + 2u+1, plane 2u+1 = slice 2u), so no sum is
// formed in the k loop.
template <class C, int EPI, bool PAIRED = false, bool PREPACKED = false>
__global__ void __launch_bounds__(C::kThreads, C::kWGS * C::kWaves / 4)
sliced_gemm_kernel(int64_t m, int64_t n, int64_t KB, int64_t tiles_n, int64_t tile0,
                   const double* __restrict__ Ap, const double* __restrict__ Bp,
                   double* __restrict__ levels, int64_t* __restrict__ units, int64_t ldl, int64_t plane,
                   const int32_t* __restrict__ E, const int32_t* __restrict__ F,
                   OutPlanes out, int64_t ldc, PairArgs pair) {
    constexpr int KS = C::kKS;
    constexpr int RPW = C::kRPW;
    constexpr int NBUF = C::kNBuf;
    constexpr int NS = C::kNS;
    // accumulators per 16x16 block: NS levels, or for the pair-packed schedule
    // its NS - 1 groups with the single products of the deepest group apart
    // (accumulator NS - 1), so that no FP64 sum chains more than half the
    // products of a k-block
    constexpr int NACC = NS;

    __shared__ __attribute__((aligned(1024))) double lds[NBUF * C::kStageDoubles];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wr = wave / C::kTBN;  // block rows RPW*wr .. RPW*wr+RPW-1 of the tile
    const int wc = wave % C::kTBN;  // block column wc of the tile
    // the launch covers tiles tile0 .. tile0 + gridDim.x - 1, row-major over the output
    const int64_t tile = static_cast<int64_t>(blockIdx.x) + tile0;
    const int64_t tm = tile / tiles_n;
    const int64_t tn = tile % tiles_n;
    const int64_t rb0 = tm * C::kTBM, cb0 = tn * C::kTBN;
    // stages of KS k-blocks: KB <= 2^21 (k within the exact-sum bound), so the
    // stage counters are 32-bit and compare in scalar registers
    const int nstages = static_cast<int>(KB / KS);  // KB is a multiple of 4 (k is packed to 16)

    // A stage in LDS is the runs of its blocks back to back (A blocks first,
    // then B blocks), kBlockStage doubles each.  1 KB piece q of it is copied by
    // wave q % waves; lane L moves the 16 bytes at stage offset 1024 q + 16 L,
    // which lie in block (128 q + 2 L) / kBlockStage (a piece may straddle two
    // runs).  When the pieces do not split evenly the last round is issued by
    // the first kPieces % waves waves only.
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const double* src[C::kPiecesPerWave];
    int dst[C::kPiecesPerWave];
#pragma unroll
    for (int i = 0; i < C::kPiecesPerWave; ++i) {
        if constexpr (C::kEvenPieces && C::kBlockStage % 128 == 0) {
            // every piece inside one block's run: the block is uniform per piece,
            // so the piece's base and LDS offset live in scalar registers and a
            // copy is a scalar base plus the lane's 16-byte offset
            const int q = i * C::kWaves + uwave;
            const int blk = q / (C::kBlockStage / 128), pc = q % (C::kBlockStage / 128);
            const double* base = blk < C::kTBM ? Ap + (rb0 + blk) * KB * C::kSetDoubles
                                               : Bp + (cb0 + blk - C::kTBM) * KB * C::kSetDoubles;
            src[i] = base + pc * 128;
            dst[i] = blk * C::kBlockStage + pc * 128;
        } else {
            int q = i * C::kWaves + uwave;
            if (q >= C::kPieces) q = 0;  // not issued; keeps the address in range
            const int g = q * 128 + lane * 2;
            const int blk = g / C::kBlockStage, off = g % C::kBlockStage;
            const double* base = blk < C::kTBM ? Ap + (rb0 + blk) * KB * C::kSetDoubles
                                               : Bp + (cb0 + blk - C::kTBM) * KB * C::kSetDoubles;
            src[i] = base + off;
            dst[i] = q * 128;
        }
    }
    // the lane's part of a piece's address (the uneven path keeps it in src)
    constexpr bool kScalarBase = C::kEvenPieces && C::kBlockStage % 128 == 0;
    const int lane_off = kScalarBase ? lane * 2 : 0;
    auto issue = [&](int64_t st, int buf) {
#pragma unroll
        for (int i = 0; i < C::kPiecesPerWave; ++i)
            if (C::kEvenPieces || i + 1 < C::kPiecesPerWave || i * C::kWaves + uwave < C::kPieces)
                __builtin_amdgcn_global_load_lds((global_void_t*)(src[i] + st * C::kBlockStage + lane_off),
                                                 (lds_void_t*)(lds + buf * C::kStageDoubles + dst[i]), 16, 0, 0);
    };

    double4_t acc[NACC][RPW];
#pragma unroll
    for (int l = 0; l < NACC; ++l)
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[l][r] = double4_t{0.0, 0.0, 0.0, 0.0};

    // Stages [s0, s1): all of them, or this workgroup's k-part of a split product
    // (blockIdx.y of gridDim.y parts).
    int s0 = 0, s1 = nstages;
    if constexpr (EPI == kEpiAtomicLevels || EPI == kEpiPairUnits) {
        s0 = static_cast<int>(uniform64(static_cast<int64_t>(nstages) * blockIdx.y / gridDim.y));
        s1 = static_cast<int>(uniform64(static_cast<int64_t>(nstages) * (blockIdx.y + 1) / gridDim.y));
    }

    const int64_t col = (cb0 + wc) * 16 + frag_col(lane);
    // The int64 cell of group g = 0 of output (row, col); group g is g planes on.
    int64_t* const part_units = units + static_cast<int64_t>(blockIdx.y) * pair.part_stride;
    auto unit_cell = [&](int64_t row) { return part_units + (row - pair.row_off) * ldl + col; };
    // Pair-packed schedule: move the group sums into the int64 planes (store
    // the first time, add later) and restart the accumulators from zero.
    bool flushed = false;
    auto flush = [&]() {
        // Row offset of this lane's cells, opaque to the compiler so that the
        // cell addresses are formed here, at a flush, rather than hoisted out of
        // the k loop into registers the matrix operands need.
        int64_t row_lane = (rb0 + RPW * wr) * 16 + frag_row(lane, 0);
        asm volatile("" : "+v"(row_lane));
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = row_lane + r * 16 + 4 * v;
                if (row < m && col < n) {
                    int64_t* u = unit_cell(row);
#pragma unroll
                    for (int g = 0; g < NS - 1; ++g) {
                        int64_t x = pair_group_units(acc[g][r][v], g);
                        if (g == NS - 2) x += pair_group_units(acc[NS - 1][r][v], g);
                        if (flushed) x += u[g * plane];
                        u[g * plane] = x;
                    }
                }
            }
#pragma unroll
        for (int l = 0; l < NACC; ++l)
#pragma unroll
            for (int r = 0; r < RPW; ++r) acc[l][r] = double4_t{0.0, 0.0, 0.0, 0.0};
        flushed = true;
        // the stage waits count vector-memory operations: drain these stores here
        wait_vmcnt<0>();
    };
    int since_flush = 0;
    // The products a stage's last k-block defers to the next stage (DEFER): their
    // operands wait in dx, db, which hold zeros before the first stage and after
    // a flush.  A product of zeros changes an accumulator at most from -0 to +0,
    // and the pair-packed schedule reads its accumulators only as integers
    // (pair_group_units), so the results are those of the undeferred order.
    constexpr int kDefer = PAIRED ? C::kDefer : 0;
    constexpr PairSchedule<NS> dsched{};
    static_assert(kDefer >= 0 && kDefer <= dsched.count, "deferred products of one k-block");
    constexpr int kDeferSlots = kDefer > 0 ? kDefer : 1;
    double dx[kDeferSlots][RPW] = {}, db[kDeferSlots] = {};
    auto run_deferred = [&]() {
        if constexpr (kDefer > 0) {
#pragma unroll
            for (int d = 0; d < kDefer; ++d)
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    const PairProduct p = dsched.order[dsched.count - kDefer + d];
                    acc[p.acc][r] = __builtin_amdgcn_mfma_f64_16x16x4f64(dx[d][r], db[d], acc[p.acc][r], 0, 0, 0);
                }
        }
    };
    const int chunk_stages = static_cast<int>(pair.chunk_stages);

    if (s1 > s0) {
#pragma unroll
        for (int j = 0; j < NBUF - 1; ++j) issue(s0 + j < s1 ? s0 + j : s1 - 1, j);
        for (int st = s0; st < s1; ++st) {
            // Stage st has landed once at most NBUF-2 younger stages are pending.
            wait_vmcnt<(NBUF - 2) * C::kPiecesPerWave>();
            compiler_fence();
            __builtin_amdgcn_s_barrier();  // every wave's copy of stage st is in LDS, and
            compiler_fence();               // every wave is done reading stage st-1
            // The copy of stage st + NBUF - 1 goes into the buffer every wave has
            // finished reading (certified by the barrier above); it is issued
            // after the first fragment reads of this stage rather than before
            // them, so the matrix instructions start sooner (measured: +2-3 %).
            const int nxt = st + NBUF - 1;
            const int nxt_c = nxt < s1 ? nxt : s1 - 1;

            const double* stage = lds + ((st - s0) % NBUF) * C::kStageDoubles + lane;
            if (C::kIssueEarly) issue(nxt_c, static_cast<int>((nxt - s0) % NBUF));
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                if (!C::kIssueEarly && KS > 1 && j == KS / 2) issue(nxt_c, static_cast<int>((nxt - s0) % NBUF));
                const double* sa = stage + (RPW * wr) * C::kBlockStage + j * C::kSetDoubles;
                const double* sb = stage + (C::kTBM + wc) * C::kBlockStage + j * C::kSetDoubles;
                double a[NS][RPW], b[NS];
#pragma unroll
                for (int s = 0; s < NS; ++s) {
#pragma unroll
                    for (int r = 0; r < RPW; ++r) a[s][r] = sa[r * C::kBlockStage + s * kFragDoubles];
                    b[s] = sb[s * kFragDoubles];
                }
                if (!C::kIssueEarly && KS == 1) issue(nxt_c, static_cast<int>((nxt - s0) % NBUF));
                if constexpr (PAIRED) {
                    // Slices 2u and 2u+1 of an entry share its sign and sit 13
                    // bits apart: their sum is an exact 26-bit operand.  Product
                    // (u, t) covers pairs (2u, t), (2u+1, t) into group 2u + t;
                    // where only (2u, t) is in the window it runs alone, into the
                    // single products' accumulator.  The products are issued in
                    // rounds -- round i holds the i-th product of every
                    // accumulator -- so that two products into one accumulator
                    // are never adjacent.
                    constexpr int NU = (NS + 1) / 2;
                    double ap[NU][RPW];  // packed operands (pair-packed layout: the planes themselves)
#pragma unroll
                    for (int u = 0; u < NU; ++u)
#pragma unroll
                        for (int r = 0; r < RPW; ++r) {
                            if constexpr (PREPACKED)
                                ap[u][r] = a[2 * u][r];
                            else
                                ap[u][r] = 2 * u + 1 < NS ? a[2 * u][r] + a[2 * u + 1][r] : a[2 * u][r];
                        }
                    // slice 2u alone: plane 2u + 1 of the pair-packed layout (the
                    // last plane itself for an odd count), else plane 2u
                    auto single = [&](int u, int r) {
                        if constexpr (PREPACKED) return 2 * u + 1 < NS ? a[2 * u + 1][r] : a[2 * u][r];
                        return a[2 * u][r];
                    };
                    constexpr PairSchedule<NS> sched{};
                    // the previous stage's deferred products, beside this stage's
                    // first fragment reads
                    if (j == 0) run_deferred();
#pragma unroll
                    for (int i = 0; i < sched.count; ++i)
#pragma unroll
                        for (int r = 0; r < RPW; ++r) {
                            const PairProduct p = sched.order[i];
                            const double x = p.packed ? ap[p.u][r] : single(p.u, r);
                            if (j == KS - 1 && i >= sched.count - kDefer) {
                                dx[i - (sched.count - kDefer)][r] = x;
                                db[i - (sched.count - kDefer)] = b[p.t];
                            } else {
                                acc[p.acc][r] = __builtin_amdgcn_mfma_f64_16x16x4f64(x, b[p.t], acc[p.acc][r], 0, 0, 0);
                            }
                        }
                } else {
                    // Triangular schedule: pair (s, t) feeds level s + t < NS.
#pragma unroll
                    for (int s = 0; s < NS; ++s)
#pragma unroll
                        for (int t = 0; s + t < NS; ++t)
#pragma unroll
                            for (int r = 0; r < RPW; ++r)
                                acc[s + t][r] =
                                    __builtin_amdgcn_mfma_f64_16x16x4f64(a[s][r], b[t], acc[s + t][r], 0, 0, 0);
                }
            }
            if constexpr (PAIRED) {
                if (chunk_stages > 0 && ++since_flush == chunk_stages && st + 1 < s1) {
                    run_deferred();
#pragma unroll
                    for (int d = 0; d < kDeferSlots; ++d) {
#pragma unroll
                        for (int r = 0; r < RPW; ++r) dx[d][r] = 0.0;
                        db[d] = 0.0;
                    }
                    flush();
                    since_flush = 0;
                }
            }
        }
        run_deferred();  // the last stage's
        // No direct-to-LDS copy may still be in flight when the workgroup ends.
        wait_vmcnt<0>();
    }

    if constexpr (PAIRED) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = (rb0 + RPW * wr + r) * 16 + frag_row(lane, v);
                if (row < m && col < n) {
                    int64_t N[NS - 1];
                    int64_t* u = flushed || EPI == kEpiPairUnits ? unit_cell(row) : nullptr;
#pragma unroll
                    for (int g = 0; g < NS - 1; ++g) {
                        N[g] = pair_group_units(acc[g][r][v], g);
                        if (g == NS - 2) N[g] += pair_group_units(acc[NS - 1][r][v], g);
                        if (flushed) N[g] += u[g * plane];
                    }
                    if constexpr (EPI == kEpiPairUnits) {
#pragma unroll
                        for (int g = 0; g < NS - 1; ++g) u[g * plane] = N[g];
                    } else if constexpr (EPI == kEpiDD) {
                        double c[2];
                        pair_units_round<NS, 2>(N, E[row] + F[col], c);
                        out.c[0][row * ldc + col] = c[0];
                        out.c[1][row * ldc + col] = c[1];
                    } else {
                        static_assert(EPI == kEpiQD, "pair-packed epilogues: units, dd, qd");
                        double c[4];
                        pair_units_round<NS, 4>(N, E[row] + F[col], c);
#pragma unroll
                        for (int q = 0; q < 4; ++q) out.c[q][row * ldc + col] = c[q];
                    }
                }
            }
        }
        return;
    } else {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t row = (rb0 + RPW * wr + r) * 16 + frag_row(lane, v);
            if (row < m && col < n) {
                double S[NS];
#pragma unroll
                for (int l = 0; l < NS; ++l) S[l] = acc[l][r][v];
                if constexpr (EPI == kEpiLevels) {
#pragma unroll
                    for (int l = 0; l < NS; ++l) levels[l * plane + row * ldl + col] = S[l];
                } else if constexpr (EPI == kEpiAtomicLevels) {
                    // Every part's level sum is a multiple of 2^(-13(l+2)) and their
                    // total stays below 2^53 such units (the exact-sum bound on the
                    // whole k), so the additions are exact in any order.  The planes
                    // start at the first tile row of the launch.
                    const int64_t lrow = row - (tile0 / tiles_n) * (C::kTBM * 16);
#pragma unroll
                    for (int l = 0; l < NS; ++l) atomicAdd(levels + l * plane + lrow * ldl + col, S[l]);
                } else if constexpr (EPI == kEpiDD || EPI == kEpiQD) {
                    const int sc = E[row] + F[col];
                    const int64_t idx = row * ldc + col;
                    if constexpr (EPI == kEpiDD) {
                        double hi, lo;
                        renorm_levels<NS>(S, sc, hi, lo);
                        out.c[0][idx] = hi;
                        out.c[1][idx] = lo;
                    } else {
                        double c[4];
                        qd_from_levels<NS>(S, sc, c);
#pragma unroll
                        for (int q = 0; q < 4; ++q) out.c[q][idx] = c[q];
                    }
                } else {
                    // Level l is an integer number of units 2^(-13(l+2)) below
                    // 2^53 per block, so int64 holds the sum of up to 1023 blocks.
                    int64_t N[NS];
#pragma unroll
                    for (int l = 0; l < NS; ++l) {
                        N[l] = static_cast<int64_t>(ldexp(S[l], kSliceBits * (l + 2)));
                        int64_t* u = units + l * plane + row * ldl + col;
                        if constexpr (EPI != kEpiUnitsSet) N[l] += *u;
                        if constexpr (EPI != kEpiUnitsQD) *u = N[l];
                    }
                    if constexpr (EPI == kEpiUnitsQD) {
                        double c[4];
                        qd_from_level_units<NS>(N, E[row] + F[col], c);
                        const int64_t idx = row * ldc + col;
#pragma unroll
                        for (int q = 0; q < 4; ++q) out.c[q][idx] = c[q];
                    }
                }
            }
        }
    }
    }
}

__global__ void __launch_bounds__(64) probe_mfma_kernel(double* __restrict__ out) {
    const int lane = threadIdx.x;
    const double a = static_cast<double>(lane + 1);
    const double b = 100.0 * static_cast<double>(lane + 1);
    double4_t c = {0.0, 0.0, 0.0, 0.0};
    c = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) out[lane * 4 + v] = c[v];
}

// Launch configuration per slice count: 32x16 wave strips, 2 x 4 waves per
// workgroup (64x64 tile, one workgroup per CU), two k-blocks per LDS stage (at
// most 64 KB), two stages; measured best among the stage depths and strip
// shapes that fit.
template <int NS> struct ConfigFor;
template <> struct ConfigFor<4> { using type = GemmConfig<2, 4, 2, 2, 1, 4>; };
template <> struct ConfigFor<5> { using type = GemmConfig<2, 4, 2, 2, 1, 5>; };
// Six slices: one 16x16 block per wave (32x64 tile) measured faster than two
// (73.2 vs 71.6 TFLOP/s at 4096^3; slower for 4, 5 and 7 slices).
// DEFER, for the pair-packed products of 6, 7, 9, 11, 12 and 13 slices: GEMM
// at 4096^3 22.80 -> 22.50, 30.11 -> 29.91, 49.79 -> 47.86, 69.92 -> 67.98,
// 79.59 -> 78.87, 93.43 -> 92.03 ms; with 4 or 5 slices (four waves per SIMD
// no longer fit), 10, 14 and 15 it measured slower.
template <> struct ConfigFor<6> { using type = GemmConfig<2, 4, 2, 2, 1, 6, 1, 0, 3>; };
template <> struct ConfigFor<7> { using type = GemmConfig<2, 4, 2, 2, 1, 7, 2, 0, 4>; };
template <> struct ConfigFor<8> { using type = GemmConfig<2, 4, 2, 2, 1, 8>; };
// Nine to sixteen slices (wide double-double windows, the quad-double product):
// up to 16 level accumulators of one 16x16 block per wave (at most 128
// registers) and a 32x64 tile.  Two k-blocks per stage while two stages fit
// the 160 KB of LDS (up to 13 slices: 78 KB a stage; measured at 4096^3 with
// 9..13 slices: 69.5-72.8 -> 74.2-75.7 TFLOP/s), one from 14 slices on.
template <> struct ConfigFor<9> { using type = GemmConfig<2, 4, 2, 2, 1, 9, 1, 0, 6>; };
template <> struct ConfigFor<10> { using type = GemmConfig<2, 4, 2, 2, 1, 10, 1>; };
template <> struct ConfigFor<11> { using type = GemmConfig<2, 4, 2, 2, 1, 11, 1, 0, 6>; };
template <> struct ConfigFor<12> { using type = GemmConfig<2, 4, 2, 2, 1, 12, 1, 0, 6>; };
template <> struct ConfigFor<13> { using type = GemmConfig<2, 4, 2, 2, 1, 13, 1, 0, 6>; };
template <> struct ConfigFor<14> { using type = GemmConfig<2, 4, 1, 2, 1, 14, 1>; };
template <> struct ConfigFor<15> { using type = GemmConfig<2, 4, 1, 2, 1, 15, 1>; };
template <> struct ConfigFor<16> { using type = GemmConfig<2, 4, 1, 2, 1, 16, 1>; };

// Launch configuration of the pair-packed schedule per slice count.  Eight
// slices: sixteen waves of one 16x16 block each (64x64 tile, four waves per
// SIMD), two k-blocks per stage -- measured at 4096^3 against two-block strips
// of eight waves (68.5 TFLOP/s), two 32x64 workgroups per CU (67.2), one or
// more k-blocks per stage with two to four stages (65.2-69.4): 70.3 TFLOP/s.
// Five slices take the same shape (4096^3: 17.63 against 18.12 ms for the
// 32x16 strips of eight waves); for four, six and seven slices the strips stay
// faster (11.40 / 22.91 / 30.22 against 12.73 / 23.08 / 30.37 ms), and from
// nine slices on sixteen waves would spill.  With eight slices the last six
// of a stage's 40 products wait for the next stage's barrier (DEFER; 122
// VGPRs, four waves per SIMD still): GEMM 4096^3 37.33 -> 36.93-36.96 ms,
// 65536x512x512 9.60 -> 9.48, 1024^3 0.601 -> 0.592 (two, eight, ten or
// twelve deferred: less), every output unchanged.  Sixteen slices (the quad
// double's 72 products, two waves per SIMD) defer eight: qd 2048^3 17.77 ->
// 17.62 ms, the 16-slice double-double GEMM at 2048^3 17.35 -> 17.23 (four:
// less, twelve: the same with more registers; 248 of 256 VGPRs).
template <int NS> struct PairConfigFor { using type = typename ConfigFor<NS>::type; };
template <> struct PairConfigFor<5> { using type = GemmConfig<4, 4, 2, 2, 1, 5, 1>; };
template <> struct PairConfigFor<8> { using type = GemmConfig<4, 4, 2, 2, 1, 8, 1, 0, 6>; };
template <> struct PairConfigFor<16> { using type = GemmConfig<2, 4, 1, 2, 1, 16, 1, 0, 8>; };

template <int NS>
hipError_t launch_gemm_ns(int64_t m, int64_t n, int64_t k, const double* A_slices, const double* B_slices,
                          double* levels, int64_t ldl, const int32_t* E, const int32_t* F, double* C_hi,
                          double* C_lo, int64_t ldc, bool fused, hipStream_t stream, int64_t tile_count) {
    using Cfg = typename ConfigFor<NS>::type;
    const PackGeom ga(m, k);
    constexpr int BM = Cfg::kTBM * 16, BN = Cfg::kTBN * 16;
    const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    int64_t tiles = tiles_m * tiles_n;
    if (tile_count >= 0 && tile_count < tiles) tiles = tile_count;  // the first tile_count tiles only
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (tiles == 0) return hipSuccess;
    const int64_t plane = m * ldl;
    if (fused)
        sliced_gemm_kernel<Cfg, kEpiDD><<<static_cast<unsigned>(tiles), Cfg::kThreads, 0, stream>>>(
            m, n, ga.KB, tiles_n, 0, A_slices, B_slices, nullptr, nullptr, 0, 0, E, F,
            OutPlanes{{C_hi, C_lo, nullptr, nullptr}}, ldc, PairArgs{});
    else if constexpr (NS == kSlices)
        sliced_gemm_kernel<Cfg, kEpiLevels><<<static_cast<unsigned>(tiles), Cfg::kThreads, 0, stream>>>(
            m, n, ga.KB, tiles_n, 0, A_slices, B_slices, levels, nullptr, ldl, plane, nullptr, nullptr,
            OutPlanes{{nullptr, nullptr, nullptr, nullptr}}, 0, PairArgs{});
    else
        return hipErrorInvalidValue;  // level planes are offered for the double-double product only
    return hipGetLastError();
}

template <int NS>
hipError_t launch_split_ns(int64_t m, int64_t n, int64_t k, const double* A_slices, const double* B_slices,
                           double* levels, int64_t ldl, int64_t parts, hipStream_t stream, int64_t tile_first) {
    using Cfg = typename ConfigFor<NS>::type;
    const PackGeom ga(m, k);
    constexpr int BM = Cfg::kTBM * 16;
    const int64_t tiles_n = (n + Cfg::kTBN * 16 - 1) / (Cfg::kTBN * 16);
    const int64_t tiles = (m + BM - 1) / BM * tiles_n;
    if (tiles > 0x7FFFFFFF || parts < 1 || parts > 65535 || tile_first < 0 || tile_first >= tiles)
        return hipErrorInvalidValue;
    // the level planes hold rows row0 .. m-1, row0 the first row of tile_first's tile row
    const int64_t row0 = tile_first / tiles_n * BM;
    const int64_t plane = (m - row0) * ldl;
    hipError_t err = launch_zero_levels(m - row0, n, NS, levels, ldl, stream);
    if (err != hipSuccess) return err;
    const dim3 grid(static_cast<unsigned>(tiles - tile_first), static_cast<unsigned>(parts));
    sliced_gemm_kernel<Cfg, kEpiAtomicLevels><<<grid, Cfg::kThreads, 0, stream>>>(
        m, n, ga.KB, tiles_n, tile_first, A_slices, B_slices, levels, nullptr, ldl, plane, nullptr, nullptr,
        OutPlanes{}, 0, PairArgs{});
    return hipGetLastError();
}

// The pair-packed schedule over the output tiles [tile_first, tile_first +
// count) (count < 0: to the last tile), row-major, in `parts` k-parts.
//   epi = kEpiDD / kEpiQD: one part; the nearest double-double / quad double
//         of each entry's exact total into C.  When k needs more than one
//         chunk, `units` holds the chunk planes [NS-1][m][ldu] (absolute rows).
//   epi = kEpiPairUnits: each part stores its group sums into its own planes,
//         part p at units + p part_stride, rows from tile_first's tile row on.
template <int NS, bool PREPACKED>
hipError_t launch_pair_ns(int64_t m, int64_t n, int64_t k, const double* A_slices, const double* B_slices, int epi,
                          const int32_t* E, const int32_t* F, const OutPlanes& C, int64_t ldc, int64_t* units,
                          int64_t ldu, int64_t plane, int64_t part_stride, int64_t tile_first, int64_t count,
                          int64_t parts, hipStream_t stream) {
    using Cfg = typename PairConfigFor<NS>::type;
    const PackGeom ga(m, k);
    constexpr int BM = Cfg::kTBM * 16, BN = Cfg::kTBN * 16;
    const int64_t tiles_n = (n + BN - 1) / BN;
    const int64_t tiles = (m + BM - 1) / BM * tiles_n;
    if (tile_first < 0 || tile_first > tiles || parts < 1 || parts > 65535) return hipErrorInvalidValue;
    const int64_t launch = count < 0 || tile_first + count > tiles ? tiles - tile_first : count;
    if (launch > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (launch == 0) return hipSuccess;
    if (epi != kEpiPairUnits && parts != 1) return hipErrorInvalidValue;
    constexpr int64_t kStageK = 4 * Cfg::kKS;
    const int64_t chunk_stages = pair_chunk_k(NS) / kStageK;
    const int64_t part_stages = (ga.KB / Cfg::kKS + parts - 1) / parts;
    if (epi != kEpiPairUnits && part_stages > chunk_stages && !units) return hipErrorInvalidValue;
    const PairArgs pa{chunk_stages, part_stride, epi == kEpiPairUnits ? tile_first / tiles_n * BM : 0};
    const dim3 grid(static_cast<unsigned>(launch), static_cast<unsigned>(parts));
    // the products read pre-packed A; the group sums also serve the stage call,
    // which takes the standard layout
    if (epi == kEpiDD && PREPACKED)
        sliced_gemm_kernel<Cfg, kEpiDD, true, true><<<grid, Cfg::kThreads, 0, stream>>>(
            m, n, ga.KB, tiles_n, tile_first, A_slices, B_slices, nullptr, units, ldu, plane, E, F, C, ldc, pa);
    else if (epi == kEpiQD && PREPACKED) {
        if constexpr (NS == kQdSlices)
            sliced_gemm_kernel<Cfg, kEpiQD, true, true><<<grid, Cfg::kThreads, 0, stream>>>(
                m, n, ga.KB, tiles_n, tile_first, A_slices, B_slices, nullptr, units, ldu, plane, E, F, C, ldc, pa);
        else
            return hipErrorInvalidValue;  // four words: the quad-double product only
    } else if (epi == kEpiPairUnits)
        sliced_gemm_kernel<Cfg, kEpiPairUnits, true, PREPACKED><<<grid, Cfg::kThreads, 0, stream>>>(
            m, n, ga.KB, tiles_n, tile_first, A_slices, B_slices, nullptr, units, ldu, plane, nullptr, nullptr,
            OutPlanes{}, 0, pa);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

namespace {

// The pair-packed product of a few outputs: one workgroup of four waves per
// 16×16 output block, wave w taking the k-blocks w, w + 4, ... with the
// fragments of the next two of them loaded while the current one's products
// issue; no LDS staging (every fragment is read once, straight into
// registers).  The four waves' group sums are added through LDS -- exactly,
// as every one is an integer multiple of its group's unit and k is within one
// exact chunk -- and wave w rounds the entries of accumulator component w (a
// quarter of the block's rows) as the tiled kernel does.  A pre-packed.
template <int NS, int W>
__global__ void __launch_bounds__(256) small_pair_gemm_kernel(int64_t m, int64_t n, int64_t KB, int64_t blocks_n,
                                                              const double* __restrict__ Ap,
                                                              const double* __restrict__ Bp,
                                                              const int32_t* __restrict__ E,
                                                              const int32_t* __restrict__ F, OutPlanes out,
                                                              int64_t ldc) {
    constexpr int kSet = NS * kFragDoubles;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t bi = blockIdx.x / blocks_n, bj = blockIdx.x % blocks_n;  // uniform
    const double* a0 = Ap + bi * KB * kSet + lane;
    const double* b0 = Bp + bj * KB * kSet + lane;
    double4_t acc[NS];
#pragma unroll
    for (int l = 0; l < NS; ++l) acc[l] = double4_t{0.0, 0.0, 0.0, 0.0};
    // k-block kb's fragments (kb clamped to the last one: a load past the end
    // refetches it and is never used)
    auto load = [&](double (&a)[NS], double (&b)[NS], int64_t kb) {
        const int64_t c = kb < KB ? kb : KB - 1;
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            a[q] = a0[c * kSet + q * kFragDoubles];
            b[q] = b0[c * kSet + q * kFragDoubles];
        }
    };
    constexpr PairSchedule<NS> sched{};
    auto issue = [&](const double (&a)[NS], const double (&b)[NS]) {
#pragma unroll
        for (int i = 0; i < sched.count; ++i) {
            const PairProduct pr = sched.order[i];
            // packed: plane 2u; alone: plane 2u + 1 (the last plane itself for an odd count)
            const double x = pr.packed ? a[2 * pr.u] : a[2 * pr.u + 1 < NS ? 2 * pr.u + 1 : 2 * pr.u];
            acc[pr.acc] = __builtin_amdgcn_mfma_f64_16x16x4f64(x, b[pr.t], acc[pr.acc], 0, 0, 0);
        }
    };
    double a_0[NS], b_0[NS], a_1[NS], b_1[NS];
    int64_t kb = w;  // < KB: k >= 1 pads to at least 4 k-blocks
    load(a_0, b_0, kb);
    load(a_1, b_1, kb + 4);
    for (; kb < KB; kb += 8) {  // uniform over the wave
        issue(a_0, b_0);
        load(a_0, b_0, kb + 8);
        if (kb + 4 < KB) issue(a_1, b_1);
        load(a_1, b_1, kb + 12);
    }
    __shared__ double4_t red[4][NS][kFragDoubles];
#pragma unroll
    for (int l = 0; l < NS; ++l) red[w][l][lane] = acc[l];
    __syncthreads();
    // wave w: component w of every accumulator, i.e. rows 4 w' + (lane >> 4)... of its lanes
    double sum[NS];
#pragma unroll
    for (int l = 0; l < NS; ++l) {
        sum[l] = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) sum[l] += red[j][l][lane][w];
    }
    const int64_t col = bj * 16 + frag_col(lane);
    const int64_t row = bi * 16 + frag_row(lane, w);
    if (row < m && col < n) {
        int64_t N[NS - 1];
#pragma unroll
        for (int g = 0; g < NS - 1; ++g) {
            N[g] = pair_group_units(sum[g], g);
            if (g == NS - 2) N[g] += pair_group_units(sum[NS - 1], g);
        }
        double c[W];
        pair_units_round<NS, W>(N, E[row] + F[col], c);
#pragma unroll
        for (int q = 0; q < W; ++q) out.c[q][row * ldc + col] = c[q];
    }
}

}  // namespace

hipError_t launch_small_pair_gemm(int64_t m, int64_t n, int64_t k, int ns, int words, const double* A_slices,
                                  const double* B_slices, const int32_t* E, const int32_t* F, const OutPlanes& C,
                                  int64_t ldc, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (ns < kMinSlices || ns > kMaxSlices || k > pair_chunk_k(ns) || (words != 2 && words != 4))
        return hipErrorInvalidValue;
    const PackGeom ga(m, k);
    const int64_t blocks_m = (m + 15) / 16, blocks_n = (n + 15) / 16;
    if (blocks_m * blocks_n > 0x7FFFFFFF) return hipErrorInvalidValue;
    const unsigned grid = static_cast<unsigned>(blocks_m * blocks_n);
    return dispatch_ns(ns, [&](auto c) -> hipError_t {
        constexpr int NS = decltype(c)::value;
        if (words == 2)
            small_pair_gemm_kernel<NS, 2><<<grid, 256, 0, stream>>>(m, n, ga.KB, blocks_n, A_slices, B_slices, E, F,
                                                                    C, ldc);
        else if constexpr (NS == kQdSlices)
            small_pair_gemm_kernel<NS, 4><<<grid, 256, 0, stream>>>(m, n, ga.KB, blocks_n, A_slices, B_slices, E, F,
                                                                    C, ldc);
        else
            return hipErrorInvalidValue;  // four words: the quad-double product only
        return hipGetLastError();
    });
}

hipError_t launch_pair_gemm(int64_t m, int64_t n, int64_t k, int ns, const double* A_slices, const double* B_slices,
                            PairOut out, const int32_t* E, const int32_t* F, const OutPlanes& C, int64_t ldc,
                            int64_t* units, int64_t ldu, int64_t plane, int64_t part_stride, int64_t tile_first,
                            int64_t count, int64_t parts, hipStream_t stream, bool A_prepacked) {
    if (m == 0 || n == 0) return hipSuccess;
    if (ns < kMinSlices || ns > kMaxSlices) return hipErrorInvalidValue;
    const int epi = out == kPairToDD ? kEpiDD : out == kPairToQD ? kEpiQD : kEpiPairUnits;
    return dispatch_ns(ns, [&](auto c) {
        constexpr int NS = decltype(c)::value;
        if (A_prepacked)
            return launch_pair_ns<NS, true>(m, n, k, A_slices, B_slices, epi, E, F, C, ldc, units, ldu, plane,
                                            part_stride, tile_first, count, parts, stream);
        return launch_pair_ns<NS, false>(m, n, k, A_slices, B_slices, epi, E, F, C, ldc, units, ldu, plane,
                                         part_stride, tile_first, count, parts, stream);
    });
}

GemmGeometry pair_geometry(int ns) {
    return dispatch_ns(ns, [&](auto c) {
        using Cfg = typename PairConfigFor<decltype(c)::value>::type;
        return GemmGeometry{Cfg::kTBM * 16, Cfg::kTBN * 16, Cfg::kKS,
                            static_cast<int>(pair_products(decltype(c)::value)) * Cfg::kRPW * Cfg::kKS,
                            Cfg::kWGS * Cfg::kWaves / 4, Cfg::kWGS * Cfg::kNBuf * Cfg::kStageDoubles * 8};
    });
}

hipError_t launch_sliced_gemm(int64_t m, int64_t n, int64_t k, int ns, const double* A_slices,
                              const double* B_slices, double* levels, int64_t ldl,
                              const int32_t* E, const int32_t* F, double* C_hi, double* C_lo,
                              int64_t ldc, bool fused, hipStream_t stream, int64_t tile_count) {
    if (m == 0 || n == 0) return hipSuccess;
    if (ns < kMinSlices || ns > kMaxSlices) return hipErrorInvalidValue;
    return dispatch_ns(ns, [&](auto c) {
        return launch_gemm_ns<decltype(c)::value>(m, n, k, A_slices, B_slices, levels, ldl, E, F, C_hi, C_lo, ldc,
                                                  fused, stream, tile_count);
    });
}

hipError_t launch_qd_gemm(int64_t m, int64_t n, int64_t k, const double* A_slices, const double* B_slices,
                          const int32_t* E, const int32_t* F, const OutPlanes& C, int64_t ldc,
                          hipStream_t stream, int64_t tile_count) {
    if (m == 0 || n == 0) return hipSuccess;
    using Cfg = ConfigFor<kQdSlices>::type;
    const PackGeom ga(m, k);
    const int64_t tiles_n = (n + Cfg::kTBN * 16 - 1) / (Cfg::kTBN * 16);
    int64_t tiles = (m + Cfg::kTBM * 16 - 1) / (Cfg::kTBM * 16) * tiles_n;
    if (tile_count >= 0 && tile_count < tiles) tiles = tile_count;  // the first tile_count tiles only
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (tiles == 0) return hipSuccess;
    sliced_gemm_kernel<Cfg, kEpiQD><<<static_cast<unsigned>(tiles), Cfg::kThreads, 0, stream>>>(
        m, n, ga.KB, tiles_n, 0, A_slices, B_slices, nullptr, nullptr, 0, 0, E, F, C, ldc, PairArgs{});
    return hipGetLastError();
}

hipError_t launch_qd_gemm_block(int64_t m, int64_t n, int64_t k, const double* A_slices, const double* B_slices,
                                int64_t* units, QdBlockStep step, const int32_t* E, const int32_t* F,
                                const OutPlanes& C, int64_t ldc, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    using Cfg = ConfigFor<kQdSlices>::type;
    const PackGeom ga(m, k);
    const int64_t tiles_n = (n + Cfg::kTBN * 16 - 1) / (Cfg::kTBN * 16);
    const int64_t tiles = (m + Cfg::kTBM * 16 - 1) / (Cfg::kTBM * 16) * tiles_n;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const unsigned g = static_cast<unsigned>(tiles);
    const int64_t plane = m * n;  // level plane l of the int64 sums: units[l][row][col], row stride n
    if (step == kQdFirstBlock)
        sliced_gemm_kernel<Cfg, kEpiUnitsSet><<<g, Cfg::kThreads, 0, stream>>>(
            m, n, ga.KB, tiles_n, 0, A_slices, B_slices, nullptr, units, n, plane, nullptr, nullptr, OutPlanes{}, 0, PairArgs{});
    else if (step == kQdMiddleBlock)
        sliced_gemm_kernel<Cfg, kEpiUnitsAdd><<<g, Cfg::kThreads, 0, stream>>>(
            m, n, ga.KB, tiles_n, 0, A_slices, B_slices, nullptr, units, n, plane, nullptr, nullptr, OutPlanes{}, 0, PairArgs{});
    else
        sliced_gemm_kernel<Cfg, kEpiUnitsQD><<<g, Cfg::kThreads, 0, stream>>>(
            m, n, ga.KB, tiles_n, 0, A_slices, B_slices, nullptr, units, n, plane, E, F, C, ldc, PairArgs{});
    return hipGetLastError();
}

GemmGeometry gemm_geometry(int ns) {
    return dispatch_ns(ns, [&](auto c) {
        using Cfg = typename ConfigFor<decltype(c)::value>::type;
        constexpr int pairs = decltype(c)::value * (decltype(c)::value + 1) / 2;
        return GemmGeometry{Cfg::kTBM * 16, Cfg::kTBN * 16, Cfg::kKS, pairs * Cfg::kRPW * Cfg::kKS,
                            Cfg::kWGS * Cfg::kWaves / 4, Cfg::kWGS * Cfg::kNBuf * Cfg::kStageDoubles * 8};
    });
}

hipError_t launch_sliced_gemm_split(int64_t m, int64_t n, int64_t k, int ns, const double* A_slices,
                                    const double* B_slices, double* levels, int64_t ldl, int64_t parts,
                                    hipStream_t stream, int64_t tile_first) {
    if (m == 0 || n == 0) return hipSuccess;
    if (ns < kMinSlices || ns > kMaxSlices) return hipErrorInvalidValue;
    return dispatch_ns(ns, [&](auto c) {
        return launch_split_ns<decltype(c)::value>(m, n, k, A_slices, B_slices, levels, ldl, parts, stream,
                                                   tile_first);
    });
}

hipError_t launch_probe_mfma(double* out, hipStream_t stream) {
    probe_mfma_kernel<<<1, 64, 0, stream>>>(out);
    return hipGetLastError();
}

}  // namespace ddg
