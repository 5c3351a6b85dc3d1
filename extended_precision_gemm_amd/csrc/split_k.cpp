// Host-side rule for splitting a sliced product over k.  The integer level sums
// of the method make the split exact: each part's level sums are multiples of
// 2^-13(l+2) whose total over the whole k stays below 2^53 units (eq. (5) of
// "Multiple Double Arithmetic on NVIDIA Tensor Cores", §2), so adding the parts
// in any order gives the unsplit sums bit for bit.  Only the speed depends on
// the part count, which this file chooses.
#include <algorithm>

#include "common.hpp"

namespace ddg {

namespace {

constexpr int64_t kComputeUnits = 256;
constexpr int64_t kLdsBytesPerCu = 160 * 1024;
constexpr double kCoResidentShare = 0.95;     // two workgroups on one CU: 0.95 of twice the time of one
constexpr int64_t kMinStagesPerPart = 16;
constexpr int64_t kMaxParts = 256;
constexpr double kClockHz = 2.38e9;           // sustained MFMA clock under load
constexpr double kMfmaEfficiency = 0.96;      // measured MFMA busy fraction of the GEMM
constexpr double kMfmaCycles = 64.0;          // one 16x16x4 FP64 MFMA on one SIMD
constexpr double kAtomicAddsPerSecond = 2e11; // FP64 atomic adds into the level planes
constexpr double kPlaneBytesPerSecond = 5e12; // zeroing and re-reading the level planes
constexpr double kSplitLaunchSeconds = 15e-6; // the zeroing and renormalising launches
constexpr double kMinSaving = 0.95;           // a split must save at least 5 %

}  // namespace

// The modelled time of one launch over `tiles` output tiles holding `outputs`
// outputs, k cut into p parts of ceil(stages / p) stages:
//     T = c(L) ceil(stages / p) t_stage
//         + [p > 1] (ns outputs p / atomic rate + 2 ns outputs 8 B / plane rate + launches),
// where t_stage is one stage of one workgroup alone on its CU (mfma_per_stage
// MFMAs of 64 cycles for each of the waves sharing a SIMD: one 8-wave workgroup
// already keeps the MFMA pipes of its CU busy), L = ceil(tiles p / 256) is the
// most workgroups any CU runs, and c(L) = L, or 0.95 L when two workgroups fit a
// CU's LDS (4..6 slices, whose waves also stay within the 128 VGPRs of four
// waves per SIMD) and L >= 2: two co-resident workgroups hide a little of each
// other's waiting.  The constants were fitted to timings of split products of 1
// to 640 output tiles with 4..8 and 16 slices.
namespace {

struct CostModel {
    GemmGeometry g;
    int ns;
    int64_t stages;
    bool two_per_cu;
    double t_stage;

    CostModel(int64_t m, int64_t k, int ns_, const GemmGeometry& geom) : g(geom), ns(ns_), stages(0) {
        stages = g.ks > 0 ? PackGeom(m, k).KB / g.ks : 0;
        // a second workgroup fits where its LDS does and the first leaves its
        // waves room: workgroups of four waves per SIMD take a SIMD's registers
        two_per_cu = g.lds_bytes > 0 && 2 * static_cast<int64_t>(g.lds_bytes) <= kLdsBytesPerCu &&
                     g.waves_per_simd <= 2;
        t_stage = static_cast<double>(g.mfma_per_stage) * g.waves_per_simd * kMfmaCycles / kClockHz / kMfmaEfficiency;
    }
    double time(int64_t tiles, double outputs, int64_t p) const {
        if (tiles <= 0) return 0.0;
        const int64_t L = (tiles * p + kComputeUnits - 1) / kComputeUnits;
        const double load = two_per_cu && L >= 2 ? kCoResidentShare * static_cast<double>(L) : static_cast<double>(L);
        const double t = load * static_cast<double>((stages + p - 1) / p) * t_stage;
        if (p == 1) return t;
        return t + ns * outputs * static_cast<double>(p) / kAtomicAddsPerSecond +
               2.0 * ns * outputs * 8.0 / kPlaneBytesPerSecond + kSplitLaunchSeconds;
    }
};

}  // namespace

// The plan with the least modelled time: the output tiles [0, first_tile)
// (row-major) in one unsplit launch, the tiles from first_tile on split into
// `parts` k-parts; first_tile = 0 splits the whole product.  Candidates:
// first_tile = 0, and with `tail` the tiles of exactly 1..4 rounds of 256
// workgroups fewer than the unsplit product takes, so that the unsplit launch
// ends on a round boundary and only the last, partly idle rounds are split.
// Each part keeps at least 16 stages; at most 256 parts; the plan must save 5 %
// against the unsplit product, else no split.  Outputs whose tiles fill whole
// rounds never split.
SplitPlan split_plan(int64_t m, int64_t n, int64_t k, int ns, bool tail) {
    const GemmGeometry g = gemm_geometry(ns);
    if (g.tile_m <= 0 || g.tile_n <= 0 || m <= 0 || n <= 0 || k <= 0) return SplitPlan{0, m, 1};
    const int64_t tiles_m = (m + g.tile_m - 1) / g.tile_m, tiles_n = (n + g.tile_n - 1) / g.tile_n;
    const int64_t tiles = tiles_m * tiles_n;
    const SplitPlan none{tiles, m, 1};
    // whole rounds: a split could only trade the co-residency of two workgroups
    // on a CU (4..6 slices) for atomics, measured under 2 % (1024² x 100000, 4 slices)
    if (tiles % kComputeUnits == 0) return none;
    const CostModel cm(m, k, ns, g);
    const int64_t pmax = cm.stages / kMinStagesPerPart < kMaxParts ? cm.stages / kMinStagesPerPart : kMaxParts;
    if (pmax < 2) return none;
    const double outputs = static_cast<double>(m) * static_cast<double>(n);
    const double t1 = cm.time(tiles, outputs, 1);
    const int64_t rounds = (tiles + kComputeUnits - 1) / kComputeUnits;
    int64_t heads[5] = {0, -1, -1, -1, -1};
    if (tail)
        for (int r = 1; r <= 4; ++r)
            if (rounds > r) heads[r] = kComputeUnits * (rounds - r);  // < tiles
    SplitPlan best = none;
    double best_t = t1;
    for (int64_t h : heads) {
        if (h < 0) continue;
        const int64_t row0 = h / tiles_n * g.tile_m;
        const double tile_outputs = static_cast<double>(g.tile_m) * static_cast<double>(g.tile_n);
        const double tail_outputs = std::min(static_cast<double>(tiles - h) * tile_outputs,
                                             static_cast<double>(m - row0) * static_cast<double>(n));
        const double t_head =
            h > 0 ? cm.time(h, outputs - tail_outputs, 1) + kSplitLaunchSeconds : 0.0;
        for (int64_t p = 2; p <= pmax; ++p) {
            const double t = t_head + cm.time(tiles - h, tail_outputs, p);
            if (t < best_t) {
                best_t = t;
                best = SplitPlan{h, row0, p};
            }
        }
    }
    return best.parts > 1 && best_t < kMinSaving * t1 ? best : none;
}

int64_t split_k_parts(int64_t m, int64_t n, int64_t k, int ns) { return split_plan(m, n, k, ns, false).parts; }

// The pair-packed product splits the same way, with other costs for the split
// tiles: no atomics and no zeroing; each k-part stores the ns - 1 int64 group
// sums of its outputs, and one more launch adds the parts and rounds:
//     T = c(L) ceil(stages / p) t_stage
//         + [p > 1] (2 p (ns - 1) outputs 8 B / plane rate + launches),
// t_stage from the pair-packed product count.  The plan must save 5 %.
// Its parts may be as short as one stage: with no atomics a part costs only its
// planes, and a product of a few tiles and a short k (64^3: one tile, 8 stages)
// then spreads over as many workgroups as it has stages.
namespace {
constexpr double kPairMinSaving = 0.95;
constexpr int64_t kPairMinStagesPerPart = 1;
}  // namespace

namespace {

struct PairPlanCost {
    SplitPlan plan;
    double seconds;
};

PairPlanCost pair_plan_cost(int64_t m, int64_t n, int64_t k, int ns) {
    const GemmGeometry g = pair_geometry(ns);
    if (g.tile_m <= 0 || g.tile_n <= 0 || m <= 0 || n <= 0 || k <= 0) return PairPlanCost{SplitPlan{0, m, 1}, 0.0};
    const int64_t tiles_m = (m + g.tile_m - 1) / g.tile_m, tiles_n = (n + g.tile_n - 1) / g.tile_n;
    const int64_t tiles = tiles_m * tiles_n;
    const SplitPlan none{tiles, m, 1};
    const CostModel cm(m, k, ns, g);
    const int64_t pmax = cm.stages / kPairMinStagesPerPart < kMaxParts ? cm.stages / kPairMinStagesPerPart : kMaxParts;
    if (tiles % kComputeUnits == 0 || pmax < 2) return PairPlanCost{none, cm.time(tiles, 0.0, 1)};
    auto cost = [&](int64_t t, double outputs, int64_t p) {
        const double base = cm.time(t, outputs, 1);  // the rounds of one part's stages, below
        if (p == 1) return base;
        const int64_t L = (t * p + kComputeUnits - 1) / kComputeUnits;
        const double load = cm.two_per_cu && L >= 2 ? kCoResidentShare * static_cast<double>(L) : static_cast<double>(L);
        return load * static_cast<double>((cm.stages + p - 1) / p) * cm.t_stage +
               2.0 * p * (ns - 1) * outputs * 8.0 / kPlaneBytesPerSecond + kSplitLaunchSeconds;
    };
    const double outputs = static_cast<double>(m) * static_cast<double>(n);
    const double t1 = cost(tiles, outputs, 1);
    const int64_t rounds = (tiles + kComputeUnits - 1) / kComputeUnits;
    int64_t heads[5] = {0, -1, -1, -1, -1};
    for (int r = 1; r <= 4; ++r)
        if (rounds > r) heads[r] = kComputeUnits * (rounds - r);
    SplitPlan best = none;
    double best_t = t1;
    for (int64_t h : heads) {
        if (h < 0) continue;
        const int64_t row0 = h / tiles_n * g.tile_m;
        const double tile_outputs = static_cast<double>(g.tile_m) * static_cast<double>(g.tile_n);
        const double tail_outputs = std::min(static_cast<double>(tiles - h) * tile_outputs,
                                             static_cast<double>(m - row0) * static_cast<double>(n));
        const double t_head = h > 0 ? cost(h, outputs - tail_outputs, 1) + kSplitLaunchSeconds : 0.0;
        for (int64_t p = 2; p <= pmax; ++p) {
            const double t = t_head + cost(tiles - h, tail_outputs, p);
            if (t < best_t) {
                best_t = t;
                best = SplitPlan{h, row0, p};
            }
        }
    }
    return best.parts > 1 && best_t < kPairMinSaving * t1 ? PairPlanCost{best, best_t} : PairPlanCost{none, t1};
}

// The small-output kernel: every 16×16 block on its own CU (at most 256 of
// them), each of its four waves working through a quarter of the k-blocks.  A
// wave's k-block costs its products' MFMA time, but no less than the latency
// of its 2 ns fragment loads with two k-blocks in flight (measured: 1.4 us per
// k-block with 8 slices, 64x64 to 128x128 outputs); plus the fixed cost of a
// launch and the rounding.
constexpr int64_t kSmallBlocksMax = 256;
constexpr double kSmallLaunchSeconds = 4e-6;
constexpr double kSmallKBlockSeconds8 = 1.4e-6;

double small_seconds(int64_t m, int64_t n, int64_t k, int ns) {
    const int64_t blocks = ((m + 15) / 16) * ((n + 15) / 16);
    if (blocks > kSmallBlocksMax || k > pair_chunk_k(ns)) return 1e30;
    const int64_t kb = PackGeom(m, k).KB;
    const double mfma = static_cast<double>(pair_products(ns)) * kMfmaCycles / kClockHz / kMfmaEfficiency;
    const double latency = kSmallKBlockSeconds8 * ns / 8.0;
    return static_cast<double>((kb + 3) / 4) * (mfma > latency ? mfma : latency) + kSmallLaunchSeconds;
}

}  // namespace

bool pair_small_product(int64_t m, int64_t n, int64_t k, int ns) {
    if (m <= 0 || n <= 0 || k <= 0) return false;
    const double t_small = small_seconds(m, n, k, ns);
    if (t_small >= 1e30) return false;
    const PairPlanCost c = pair_plan_cost(m, n, k, ns);
    // the tiled plan's time counts its split launches but not its own launch
    return t_small < c.seconds + kSmallLaunchSeconds;
}

SplitPlan pair_split_plan(int64_t m, int64_t n, int64_t k, int ns) {
    if (pair_small_product(m, n, k, ns)) {
        const GemmGeometry g = pair_geometry(ns);
        const int64_t tiles = ((m + g.tile_m - 1) / g.tile_m) * ((n + g.tile_n - 1) / g.tile_n);
        return SplitPlan{tiles, m, 1};
    }
    return pair_plan_cost(m, n, k, ns).plan;
}

}  // namespace ddg
