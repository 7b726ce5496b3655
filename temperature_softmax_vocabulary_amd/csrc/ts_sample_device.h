// Integer arithmetic of the inverse-CDF token draw (draw_kernels.hip).
//
// The pull-request page "fix(kernel): avoid nan in triton sampling softmax
// when a chunk starts with -inf" feeds the softmax into a draw of token ids
// (scope paragraph) that must land on allowed ids only (results table,
// sampling row). The rule used: with u clamped to [0, 1] (NaN -> 0) and C the
// row's inclusive prefix sums in id order, the id is the smallest j with
// C[j] > u * C[V-1].
//
// Prefix sums are formed in 64-bit integers, where addition is exact and does
// not depend on its order: a value w > 0 becomes q = rint(w * 2^s) at a
// power-of-two scale 2^s (exact scaling), and a value that is not > 0 becomes
// 0, so it can never hold a target: with T = min(floor(u Q), Q - 1) and Q the
// integer total, the smallest j whose integer prefix exceeds T has q[j] >= 1.
#pragma once

#include "ts_device.h"

namespace tsk {

// q = rint(w * 2^s) for w > 0, else 0 (zero, negative and NaN values).
__device__ __forceinline__ uint64_t fixed_point(float w, int s) {
    if (!(w > 0.0f)) return 0;
    return static_cast<uint64_t>(rintf(ldexpf(w, s)));
}

// Scale exponent for values whose sum is `total` (> 0, finite): each value is
// <= total < 2^e, so each q <= 2^61 and a sum of them stays below 2^62 (up to
// the float rounding of `total`).
__device__ __forceinline__ int scale_exponent(float total) {
    int e = 0;
    frexpf(total, &e);
    return 61 - e;
}

// Target for a uniform: clamp to [0, 1] (NaN -> 0), T = min(floor(u Q), Q - 1).
__device__ __forceinline__ uint64_t target_of(float u, uint64_t Q) {
    u = (u == u) ? fminf(fmaxf(u, 0.0f), 1.0f) : 0.0f;
    const uint64_t T = static_cast<uint64_t>(floor(static_cast<double>(u) * static_cast<double>(Q)));
    return T < Q ? T : Q - 1;
}

// Lane `src`'s value of a 64-bit variable, on every lane (src wave-uniform).
__device__ __forceinline__ uint64_t lane_value_u64(uint64_t v, int src) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), src);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), src);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// A 64-bit DPP lane move (two 32-bit moves); 0 where the source lane lies
// outside its row or the row is masked off. All 64 lanes must be active.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64_or0(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, ROW_MASK, 0xF,
                                               false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, ROW_MASK,
                                               0xF, false);
    return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// Inclusive prefix sum over the lanes of a wave, in lane order, with DPP moves
// only (no LDS): shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then the
// last lane of rows 0 and 2 into rows 1 and 3 (row_bcast15), then lane 31 into
// rows 2 and 3 (row_bcast31). All 64 lanes must be active.
__device__ __forceinline__ uint64_t wave_inclusive_scan_u64(uint64_t v) {
    v += dpp_u64_or0<0x111>(v);        // row_shr:1
    v += dpp_u64_or0<0x112>(v);        // row_shr:2
    v += dpp_u64_or0<0x114>(v);        // row_shr:4
    v += dpp_u64_or0<0x118>(v);        // row_shr:8
    v += dpp_u64_or0<0x142, 0xA>(v);   // row_bcast15 -> rows 1, 3
    v += dpp_u64_or0<0x143, 0xC>(v);   // row_bcast31 -> rows 2, 3
    return v;
}

// Sum over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) { return lane_value_u64(wave_inclusive_scan_u64(v), 63); }

// A group's weight from its probability partials (a float4 per group): the
// sum of its four parts, added in one fixed order (the fused softmax leaves one
// part per wave; the draw's partials kernel the whole sum and three zeros).
__device__ __forceinline__ float group_prob_sum(float4 v) { return (v.x + v.y) + (v.z + v.w); }

// Block sums of one group held in the layout of load_chunk with 256 lanes and
// F = 4: block b = 16 j + t / 16 is the 4 entries of each of the 16 lanes of
// one row of lanes in chunk group j. The last lane of each row of lanes writes
// the block's sum to blocks[b] (LDS); the caller synchronises before reading.
template <int F>
__device__ __forceinline__ void block_sums_to_lds(const float (&x)[4 * F], float* blocks) {
    static_assert(F == 4, "a group of 4096 columns is four float4 per lane");
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < F; ++j) {
        const float b = row16_reduce<SumOp>((x[4 * j] + x[4 * j + 1]) + (x[4 * j + 2] + x[4 * j + 3]));
        if ((t & 15) == 15) blocks[j * 16 + (t >> 4)] = b;
    }
}

}  // namespace tsk
