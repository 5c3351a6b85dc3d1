// Helpers shared by the double-double and quad-double slicers: exponent
// encoding for max-reductions, exact decomposition of a double, and two small
// utility kernels.
#pragma once

#include "common.hpp"

namespace ddg {
namespace {

constexpr int kNoExp = 0;          // encoded "no nonzero entry seen"
constexpr int kExpBias = 4096;     // encoded exponent = frexp exponent + bias (>= 1)
constexpr uint64_t kMant = (1ull << 52) - 1;
// A balancing exponent replaced by this value marks its row (column) for the
// exact pass: it holds a pair whose leading word is not RN(hi + lo).
constexpr int32_t kUnnormalised = INT32_MIN;

// frexp exponent of a nonzero finite double: smallest e with |x| < 2^e.
__device__ __forceinline__ int frexp_exponent(double x) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x)) & 0x7FFFFFFFFFFFFFFFull;
    const int be = static_cast<int>(b >> 52);
    if (be != 0) return be - 1022;
    return (64 - __clzll(static_cast<long long>(b & kMant))) - 1074;
}

__device__ __forceinline__ int decode_exp(int code) { return code == kNoExp ? 0 : code - kExpBias; }

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
    return v;
}

// |x| = mant * 2^exp for a finite double (sign ignored); mant < 2^53.
__device__ __forceinline__ void decompose(double x, uint64_t& mant, int& exp) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x)) & 0x7FFFFFFFFFFFFFFFull;
    const int be = static_cast<int>(b >> 52);
    mant = b & kMant;
    if (be != 0) {
        mant |= 1ull << 52;
        exp = be - 1075;
    } else {
        exp = -1074;
    }
}

__global__ void fill_int_kernel(int32_t* __restrict__ p, int64_t count, int32_t v) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = v;
}

__global__ void decode_exps_kernel(int32_t* __restrict__ exps, int64_t count) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        exps[i] = decode_exp(exps[i]);
}

// Row parts for the column-exponent kernels: enough workgroups of 16 columns
// to fill the chip, each part at least kMinRowsPerPart rows long (one part,
// and so no clearing and decoding launches, from kExpColMinWorkgroups column
// blocks up).
constexpr int64_t kExpColMinWorkgroups = 256;
constexpr int64_t kMinRowsPerPart = 256;
inline int64_t exp_col_parts(int64_t rows, int64_t cols) {
    const int64_t blocks = (cols + 15) / 16;
    int64_t parts = (kExpColMinWorkgroups + blocks - 1) / blocks;
    const int64_t most = rows / kMinRowsPerPart > 1 ? rows / kMinRowsPerPart : 1;
    if (parts > most) parts = most;
    if (parts > 65535) parts = 65535;
    return parts;
}

// k-parts for the row-exponent kernels (one wave per row and part): enough
// waves to fill the chip when the rows are few, each part at least
// kMinColsPerPart values long (one part, and so no clearing and decoding
// launches, from kExpRowMinWaves rows up).
constexpr int64_t kExpRowMinWaves = 2048;
constexpr int64_t kMinColsPerPart = 2048;
inline int64_t exp_row_parts(int64_t rows, int64_t cols) {
    int64_t parts = (kExpRowMinWaves + rows - 1) / rows;
    const int64_t most = cols / kMinColsPerPart > 1 ? cols / kMinColsPerPart : 1;
    if (parts > most) parts = most;
    if (parts > 65535) parts = 65535;
    return parts;
}

inline unsigned grid_for(int64_t work, int64_t per_block, int64_t cap) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return static_cast<unsigned>(g);
}

}  // namespace
}  // namespace ddg
