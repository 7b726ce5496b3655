// Inverse-CDF token draws: HIP kernels for gfx950.
//
// The pull-request page "fix(kernel): avoid nan in triton sampling softmax
// when a chunk starts with -inf" (FreeToken pull request 654) feeds the
// temperature softmax into a token draw (scope paragraph) and requires every
// draw to land on an allowed id (results table, sampling row). The draw rule:
// for u clamped to [0, 1] (NaN -> 0) and the row's inclusive prefix sums C of
// the probabilities, the id is the smallest j with C[j] > u * C[V-1].
//
// A row is cut into groups of 4096 columns, each of 64 blocks of 64 columns,
// and the draw takes two short kernels:
//  ts_draw_partials: one read of the row, no exchange between workgroups. Each
//    group gets a float partial: from logits, the method's chunk partial
//    (pm, pl) -- the group's max and the sum of exp2((x - shift) k) with the
//    -inf guard of the fix paragraph; from probabilities, the sum of the
//    positive entries (one share per wave). Each block gets its sum of the
//    same terms: the exponentials at its group's max, or the probabilities.
//  ts_draw_resolve: one wave per (row, target), three levels. At each level
//    the 64 lanes hold 64 float weights -- the row's groups (for logits, their
//    pl rescaled to the row's max as in the finalize, so that a fully masked
//    group weighs exactly 0), then the chosen group's blocks, then the chosen
//    block's entries -- which become integers at one power-of-two scale; an
//    integer prefix sum over the lanes gives each its range, and the lane whose
//    range holds the target is chosen. The target is carried into the next
//    level's integer units in double precision and clamped to its total.
// Every wave computes the same integers from the same partials, so at each
// level the ranges tile the total exactly. The draw follows the rule up to the
// float rounding of the group and block weights (about 1e-7 of the row total);
// with dyadic probabilities whose float sums are exact it is exact. The id
// always has an entry whose integer weight is >= 1: a masked id (a -inf logit,
// a cleared allowed bit, a probability that is not > 0) is never drawn.
#include "ts_device.h"
#include "ts_launch.h"
#include "ts_sample_device.h"

namespace tsk {

namespace {

constexpr int DT = 256;                  // lanes per workgroup
constexpr int DW = DT / kWave;
static_assert(DT * 4 * 4 == kDrawGroup, "a group is four float4 per lane");
static_assert(kBlocksPerGroup == kWave && kDrawBlock == kWave, "one lane per block, one lane per entry");

__device__ __forceinline__ const uint32_t* draw_mask_row(const DrawArgs& a, int64_t row) {
    return a.allowed ? a.allowed + row * a.mwords : nullptr;
}

// N sums (or maxima) over the workgroup at once: one LDS round for all of
// them, combined in a fixed order; every lane gets every result.
template <class Op, int NW, int N>
__device__ __forceinline__ void block_reduce_n(float (&v)[N], float (*lds)[NW]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float w = wave_reduce<Op>(v[i]);
        if ((threadIdx.x & (kWave - 1)) == 0) lds[i][threadIdx.x / kWave] = w;
    }
    __syncthreads();
    Op op;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float r = lds[i][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) r = op(r, lds[i][w]);
        v[i] = r;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// ts_draw_partials: workgroup (row, h) reads groups G = GPW h + d, d < GPW, in
// the layout of load_chunk (F = 4 GPW: chunk group j = columns
// GPW h 4096 + j 1024 + [0, 1024), lane t holding 4 consecutive columns of
// each), so group G = GPW h + j / 4 and its block b = 16 (j % 4) + t / 16 is
// one row of 16 lanes.
// ---------------------------------------------------------------------------
template <int LD, int KIND, int GPW>
__global__ __launch_bounds__(DT) void ts_draw_partials(DrawArgs a) {
    __shared__ float red[GPW][DW];   // (logits only)
    constexpr int F = 4 * GPW;
    const int t = threadIdx.x;
    const int64_t nh = (a.ngroups + GPW - 1) / GPW;
    const int64_t row = blockIdx.x / nh;
    const int64_t h = blockIdx.x - row * nh;
    const int64_t G0 = h * GPW;
    const bool holder = (t & 15) == 15;
    float x[4 * F];
    if constexpr (KIND == kDrawLogits) {
        {
            const int64_t c0 = G0 * kDrawGroup;
            const uint32_t* mrow = draw_mask_row(a, row);
            uint32_t mw[2];
            issue_chunk_loads<DT, F, LD, true>(a.x + row * a.V, c0, a.V, x);
            if (mrow) load_mask_words<DT, F>(mrow, c0, a.V, mw);
            if constexpr (LD == kLdUnaligned) shift_tail_group<DT, F>(c0, a.V, x);
            fill_past_end<DT, F>(c0, a.V, x, kNegInf);
            if (mrow) apply_mask_words<DT, F>(c0, a.V, mw, x);
        }
        const float k = exp2_scale(a.temps[row]);
        // each group's max over the workgroup; then its exponentials at that max,
        // summed per block and per group as probabilities are
        float gm[GPW];
#pragma unroll
        for (int d = 0; d < GPW; ++d) {
            float m = kNegInf;
#pragma unroll
            for (int i = 16 * d; i < 16 * d + 16; ++i) m = fmaxf(m, x[i]);
            gm[d] = m;
        }
        block_reduce_n<MaxOp, DW, GPW>(gm, red);
        float gl[GPW];
#pragma unroll
        for (int d = 0; d < GPW; ++d) {
            const float gsh = guarded_shift(gm[d]);
#pragma unroll
            for (int i = 16 * d; i < 16 * d + 16; ++i) x[i] = exp2_hw((x[i] - gsh) * k);
            const int64_t G = G0 + d;   // (workgroup-uniform test: a group past the row's end writes nothing)
            gl[d] = G < a.ngroups ? prob_block_sums<F>(x, 4 * d, a.bpart + (row * a.ngroups + G) * kBlocksPerGroup)
                                  : 0.0f;
        }
        block_reduce_n<SumOp, DW, GPW>(gl, red);
#pragma unroll
        for (int d = 0; d < GPW; ++d)
            if (t == 0 && G0 + d < a.ngroups) a.gpart[row * a.ngroups + G0 + d] = make_float4(gm[d], gl[d], 0.0f, 0.0f);
    } else {
        issue_chunk_loads<DT, F, LD, true>(a.x + row * a.V, G0 * kDrawGroup, a.V, x);
        if constexpr (LD == kLdUnaligned) shift_tail_group<DT, F>(G0 * kDrawGroup, a.V, x);
        fill_past_end<DT, F>(G0 * kDrawGroup, a.V, x, 0.0f);
        float gs[GPW];
#pragma unroll
        for (int d = 0; d < GPW; ++d) {
            const int64_t G = G0 + d;   // (workgroup-uniform test: a group past the row's end writes nothing)
            gs[d] = G < a.ngroups ? prob_block_sums<F>(x, 4 * d, a.bpart + (row * a.ngroups + G) * kBlocksPerGroup)
                                  : 0.0f;
        }
        // each wave's share of each group sum (kernel-wide no barrier)
#pragma unroll
        for (int d = 0; d < GPW; ++d) {
            const float w = wave_reduce<SumOp>(gs[d]);
            if ((t & (kWave - 1)) == 0 && G0 + d < a.ngroups)
                reinterpret_cast<float*>(a.gpart + row * a.ngroups + G0 + d)[t / kWave] = w;
        }
    }
}

// ---------------------------------------------------------------------------
// ts_draw_resolve: wave w of the grid draws target w % K of row w / K.
// ---------------------------------------------------------------------------

// The lane whose integer range [base + incl - q, base + incl) holds T (incl:
// the lane's inclusive prefix of q); -1 if none. Wave-uniform.
__device__ __forceinline__ int find_lane(uint64_t q, uint64_t incl, uint64_t base, uint64_t T) {
    const uint64_t lo = base + incl - q;
    const bool hit = T >= lo && T - lo < q;
    const uint64_t hits = __ballot(hit);
    return hits ? __ffsll(static_cast<unsigned long long>(hits)) - 1 : -1;
}

// T, a place in [P, P + q) of the level above, carried into this level's
// integer units (total L >= 1) in double precision and clamped to [0, L - 1].
__device__ __forceinline__ uint64_t carry_target(uint64_t T, uint64_t P, uint64_t q, uint64_t L) {
    const double f = static_cast<double>(T - P) * (static_cast<double>(L) / static_cast<double>(q));
    const uint64_t Tc = f < static_cast<double>(L) ? static_cast<uint64_t>(f) : L - 1;
    return Tc < L ? Tc : L - 1;
}

template <int KIND>
__global__ __launch_bounds__(DT) void ts_draw_resolve(DrawArgs a) {
    const int ln = threadIdx.x & (kWave - 1);
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * DW + threadIdx.x / kWave;
    if (wid >= a.B * a.K) return;   // the whole wave
    const int64_t row = wid / a.K;
    const int64_t ng = a.ngroups;
    const float4* grow = a.gpart + row * ng;
    int32_t* out = a.out_ids + wid;
    // independent loads first
    const float u = a.uniforms[wid];
    const float k = KIND == kDrawLogits ? exp2_scale(a.temps[row]) : 0.0f;

    // level 1: the row's groups, 64 per tile, lane l holding group b0 + l
    const float4 gv = ln < ng ? grow[ln] : make_float4(kNegInf, 0.0f, 0.0f, 0.0f);
    float gsh = 0.0f;
    if constexpr (KIND == kDrawLogits) {
        float mm = gv.x;
        for (int64_t b0 = kWave; b0 < ng; b0 += kWave) mm = fmaxf(mm, b0 + ln < ng ? grow[b0 + ln].x : kNegInf);
        gsh = guarded_shift(wave_reduce<MaxOp>(mm));
    }
    auto group_weight = [&](float4 v, int64_t i) -> float {
        if (i >= ng) return 0.0f;
        if constexpr (KIND == kDrawLogits) return masked_term(v.x, v.y * exp2_hw((v.x - gsh) * k));
        else return group_prob_sum(v);
    };
    const float gw0 = group_weight(gv, ln);
    float tl = gw0;
    for (int64_t b0 = kWave; b0 < ng; b0 += kWave)
        tl += b0 + ln < ng ? group_weight(grow[b0 + ln], b0 + ln) : 0.0f;
    const float tot = wave_reduce<SumOp>(tl);
    if (!(tot > 0.0f) || !(tot < __builtin_huge_valf())) {   // nothing can be drawn
        if (ln == 0) *out = -1;
        return;
    }
    const int s1 = scale_exponent(tot);
    const uint64_t q0 = fixed_point(gw0, s1);
    const uint64_t incl0 = wave_inclusive_scan_u64(q0);
    uint64_t Q = lane_value_u64(incl0, kWave - 1);
    if (ng > kWave) {   // the row's integer total over every tile
        uint64_t ql = 0;
        for (int64_t b0 = kWave; b0 < ng; b0 += kWave)
            ql += b0 + ln < ng ? fixed_point(group_weight(grow[b0 + ln], b0 + ln), s1) : 0;
        Q += wave_sum_u64(ql);
    }
    const uint64_t T = target_of(u, Q);
    int64_t G = -1;
    uint64_t PG = 0, qG = 0, carry = 0;
    for (int64_t b0 = 0; b0 < ng; b0 += kWave) {
        uint64_t q = q0, incl = incl0;
        if (b0 > 0) {
            q = b0 + ln < ng ? fixed_point(group_weight(grow[b0 + ln], b0 + ln), s1) : 0;
            incl = wave_inclusive_scan_u64(q);
        }
        const int src = find_lane(q, incl, carry, T);
        if (src >= 0) {
            G = b0 + src;
            PG = carry + lane_value_u64(incl - q, src);
            qG = lane_value_u64(q, src);
            break;
        }
        carry += lane_value_u64(incl, kWave - 1);
    }
    // (the ranges tile [0, Q) and T < Q, so this and the two checks below
    // never fire; they keep every index in bounds regardless)
    if (G < 0) {
        if (ln == 0) *out = -1;
        return;
    }

    // level 2: the group's 64 blocks, lane l holding block l
    // (block weights: sums of the group's exponentials at its max, or of probabilities)
    const float bw = a.bpart[(row * ng + G) * kBlocksPerGroup + ln].x;
    const int s2 = scale_exponent(wave_reduce<SumOp>(bw));   // > 0: qG >= 1 needs a positive group
    const uint64_t qb = fixed_point(bw, s2);
    const uint64_t incl2 = wave_inclusive_scan_u64(qb);
    const uint64_t T2 = carry_target(T, PG, qG, lane_value_u64(incl2, kWave - 1));
    const int b = find_lane(qb, incl2, 0, T2);
    if (b < 0) {
        if (ln == 0) *out = -1;
        return;
    }
    const uint64_t Pb = lane_value_u64(incl2 - qb, b);
    const uint64_t qbb = lane_value_u64(qb, b);
    const float bx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bw), b));   // > 0

    // level 3: the block's 64 entries, lane l holding column G 4096 + 64 b + l
    const int64_t col = G * kDrawGroup + static_cast<int64_t>(b) * kDrawBlock + ln;
    const float* xr = a.x + row * a.V;
    float v = col < a.V ? xr[col] : (KIND == kDrawLogits ? kNegInf : 0.0f);
    if constexpr (KIND == kDrawLogits) {
        if (const uint32_t* mrow = draw_mask_row(a, row)) {
            if (col < a.V && !((mrow[col >> 5] >> (col & 31)) & 1u)) v = kNegInf;
        }
        v = exp2_hw((v - guarded_shift(grow[G].x)) * k);   // as the partials kernel formed them
    }
    const int s3 = scale_exponent(bx);   // each entry <= the block's sum
    const uint64_t qe = fixed_point(v, s3);
    const uint64_t incl3 = wave_inclusive_scan_u64(qe);
    const uint64_t T3 = carry_target(T2, Pb, qbb, lane_value_u64(incl3, kWave - 1));
    const int e = find_lane(qe, incl3, 0, T3);
    if (e < 0 && ln == 0) *out = -1;
    if (ln == e) *out = static_cast<int32_t>(col);
}

// Groups per workgroup of the partials kernel: two (32 KiB of reads) once the
// call fills the device, else one.
constexpr int kPartialsGPW = 2;

template <int LD, int GPW>
hipError_t partials_impl(const DrawArgs& a, int kind, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(a.B * ((a.ngroups + GPW - 1) / GPW)));
    if (kind == kDrawLogits) hipLaunchKernelGGL((ts_draw_partials<LD, kDrawLogits, GPW>), grid, dim3(DT), 0, s, a);
    else hipLaunchKernelGGL((ts_draw_partials<LD, kDrawProbs, GPW>), grid, dim3(DT), 0, s, a);
    return hipGetLastError();
}

template <int GPW>
hipError_t partials_ld(const DrawArgs& a, int ld, int kind, hipStream_t s) {
    switch (ld) {
        case kLdAligned: return partials_impl<kLdAligned, GPW>(a, kind, s);
        case kLdUnaligned: return partials_impl<kLdUnaligned, GPW>(a, kind, s);
        case kLdScalar: return partials_impl<kLdScalar, GPW>(a, kind, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_draw_partials(const DrawArgs& a, int ld, int kind, hipStream_t s) {
    // the unaligned loads need a row of at least 4 columns
    if (ld == kLdUnaligned && a.V < 4) ld = kLdScalar;
    const bool wide = a.B * a.ngroups >= 2048;
    return wide ? partials_ld<kPartialsGPW>(a, ld, kind, s) : partials_ld<1>(a, ld, kind, s);
}

hipError_t launch_draw_resolve(const DrawArgs& a, int kind, hipStream_t s) {
    const int64_t waves = a.B * a.K;
    const dim3 grid(static_cast<uint32_t>((waves + DW - 1) / DW));
    if (kind == kDrawLogits) hipLaunchKernelGGL((ts_draw_resolve<kDrawLogits>), grid, dim3(DT), 0, s, a);
    else hipLaunchKernelGGL((ts_draw_resolve<kDrawProbs>), grid, dim3(DT), 0, s, a);
    return hipGetLastError();
}

}  // namespace tsk
