// Host-side rule for splitting a sliced product over k.  The integer level sums
// of the method make the split exact: each part's level sums are multiples of
// 2^-13(l+2) whose total over the whole k stays below 2^53 units (eq. (5) of
// "Multiple Double Arithmetic on NVIDIA Tensor Cores", §2), so adding the parts
// in any order gives the unsplit sums bit for bit.  Only the speed depends on
// the part count, which this file chooses.
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

// The modelled time of one launch over `tiles` output tiles of `rows` x n
// outputs, k cut into p parts of ceil(stages / p) stages:
//     T = c(L) ceil(stages / p) t_stage
//         + [p > 1] (ns rows n p / atomic rate + 2 ns rows n 8 B / plane rate + launches),
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
    int64_t n, stages;
    bool two_per_cu;
    double t_stage;

    CostModel(int64_t n_, int64_t m, int64_t k, int ns_) : g(gemm_geometry(ns_)), ns(ns_), n(n_), stages(0) {
        stages = g.ks > 0 ? PackGeom(m, k).KB / g.ks : 0;
        two_per_cu = g.lds_bytes > 0 && 2 * static_cast<int64_t>(g.lds_bytes) <= kLdsBytesPerCu;
        t_stage = static_cast<double>(g.mfma_per_stage) * g.waves_per_simd * kMfmaCycles / kClockHz / kMfmaEfficiency;
    }
    double time(int64_t tiles, int64_t rows, int64_t p) const {
        if (tiles <= 0) return 0.0;
        const int64_t L = (tiles * p + kComputeUnits - 1) / kComputeUnits;
        const double load = two_per_cu && L >= 2 ? kCoResidentShare * static_cast<double>(L) : static_cast<double>(L);
        const double t = load * static_cast<double>((stages + p - 1) / p) * t_stage;
        if (p == 1) return t;
        const double outputs = static_cast<double>(rows) * static_cast<double>(n);
        return t + ns * outputs * static_cast<double>(p) / kAtomicAddsPerSecond +
               2.0 * ns * outputs * 8.0 / kPlaneBytesPerSecond + kSplitLaunchSeconds;
    }
};

}  // namespace

// The plan with the least modelled time: rows [0, first_row) of C in one
// unsplit launch (whole tile rows, ending on or before a round boundary of 256
// workgroups), rows [first_row, m) split into `parts` k-parts; first_row = 0
// splits the whole product.  Candidates: first_row = 0, and with `tail` the
// most tile rows that fit 1..4 rounds fewer than the unsplit product takes.
// Each part keeps at least 16 stages; at most 256 parts; the plan must save
// 5 % against the unsplit product, else {m, 1}: no split.  Outputs whose
// tiles fill whole rounds never split.
SplitPlan split_plan(int64_t m, int64_t n, int64_t k, int ns, bool tail) {
    const SplitPlan none{m, 1};
    const GemmGeometry g = gemm_geometry(ns);
    if (g.tile_m <= 0 || g.tile_n <= 0 || m <= 0 || n <= 0 || k <= 0) return none;
    const CostModel cm(n, m, k, ns);
    const int64_t pmax = cm.stages / kMinStagesPerPart < kMaxParts ? cm.stages / kMinStagesPerPart : kMaxParts;
    if (pmax < 2) return none;
    const int64_t tiles_m = (m + g.tile_m - 1) / g.tile_m, tiles_n = (n + g.tile_n - 1) / g.tile_n;
    const double t1 = cm.time(tiles_m * tiles_n, m, 1);
    const int64_t rounds = (tiles_m * tiles_n + kComputeUnits - 1) / kComputeUnits;
    int64_t firsts[5] = {0, -1, -1, -1, -1};
    if (tail)
        for (int r = 1; r <= 4; ++r)
            if (rounds > r) {
                int64_t d = kComputeUnits * (rounds - r) / tiles_n;  // tile rows of the unsplit launch
                firsts[r] = d < tiles_m ? d : -1;
            }
    SplitPlan best = none;
    double best_t = t1;
    for (int64_t d : firsts) {
        if (d < 0) continue;
        const int64_t r0 = d * g.tile_m;
        const double t_head = d > 0 ? cm.time(d * tiles_n, r0, 1) + kSplitLaunchSeconds : 0.0;
        for (int64_t p = 2; p <= pmax; ++p) {
            const double t = t_head + cm.time((tiles_m - d) * tiles_n, m - r0, p);
            if (t < best_t) {
                best_t = t;
                best = SplitPlan{r0, p};
            }
        }
    }
    return best.parts > 1 && best_t < kMinSaving * t1 ? best : none;
}

int64_t split_k_parts(int64_t m, int64_t n, int64_t k, int ns) { return split_plan(m, n, k, ns, false).parts; }

}  // namespace ddg
