// Inverse-CDF token draws: HIP kernels for gfx950.
//
// The pull-request page "fix(kernel): avoid nan in triton sampling softmax
// when a chunk starts with -inf" (FreeToken pull request 654) feeds the
// temperature softmax into a token draw (scope paragraph) and requires every
// draw to land on an allowed id (results table, sampling row). The draw rule:
// for u clamped to [0, 1] (NaN -> 0) and the row's inclusive prefix sums C of
// the probabilities, the id is the smallest j with C[j] > u * C[V-1].
//
// The row is cut into groups of kDrawGroup = 1024 columns, and the draw takes
// two short kernels:
//  ts_group_partials: one read of the row, no exchange between workgroups.
//    Each group gets a float partial: from logits, the method's chunk partial
//    (pm, pl) -- max, and sum of exp2((x - shift) k) with the -inf guard of the
//    fix paragraph -- taken at the group's own max; from probabilities, the
//    sum of the positive entries.
//  ts_draw_resolve: one wave per (row, target). The wave turns the row's group
//    partials into one float weight per group (for logits, pl rescaled to the
//    row max as in the finalize: a fully masked group weighs exactly 0), the
//    weights into integers at one power-of-two scale, and finds the group
//    whose integer range holds the target. It then reloads that group's 1024
//    entries, forms their exact integer prefix sums at a scale of the group,
//    carries the target into the group's units and walks to the id.
// Every wave of a row computes the same integers from the same partials, so
// the groups' ranges tile [0, Q) exactly and any two draws of a row agree on
// them. The draw follows the rule up to the float rounding of the group
// weights (about 1e-7 of the row total); with dyadic probabilities whose float
// sums are exact, it is exact. The id always has an entry with q >= 1: a
// masked id (a -inf logit, a cleared allowed bit, a probability that is not
// > 0) is never drawn.
#include "ts_device.h"
#include "ts_launch.h"
#include "ts_sample_device.h"

namespace tsk {

namespace {

constexpr int DT = 256;                  // lanes per workgroup
constexpr int DW = DT / kWave;
static_assert(DT * 4 == kDrawGroup, "a group is one float4 per lane");
constexpr int GL = kDrawGroup / kWave;   // columns per lane when one wave holds a group (16)

__device__ __forceinline__ const uint32_t* draw_mask_row(const DrawArgs& a, int64_t row) {
    return a.allowed ? a.allowed + row * a.mwords : nullptr;
}

// ---------------------------------------------------------------------------
// ts_group_partials: workgroup (row, c) reads columns [c C, (c + 1) C), C =
// F groups, in the layout of load_chunk (group j = columns c C + j 1024 +
// [0, 1024), lane t holding 4 consecutive columns of each), and writes the F
// group partials part[row nsub + c F + j].
// ---------------------------------------------------------------------------
template <int F, bool VEC, int KIND>
__global__ __launch_bounds__(DT) void ts_group_partials(DrawArgs a) {
    __shared__ float red[2][F][DW];
    constexpr int C = kDrawGroup * F;
    const int t = threadIdx.x, ln = t & (kWave - 1), wv = t / kWave;
    const int64_t row = blockIdx.x / a.nch;
    const int64_t c = blockIdx.x - row * a.nch;
    float x[4 * F];
    if constexpr (KIND == kDrawLogits) {
        load_chunk<DT, F, VEC, true>(a.x + row * a.V, c * C, a.V, x, kNegInf, draw_mask_row(a, row));
        const float k = exp2_scale(a.temps[row]);
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const float m = fmaxf(fmaxf(x[4 * j], x[4 * j + 1]), fmaxf(x[4 * j + 2], x[4 * j + 3]));
            const float wm = wave_reduce<MaxOp>(m);
            if (ln == 0) red[0][j][wv] = wm;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < F; ++j) {
            float gm = red[0][j][0];
#pragma unroll
            for (int w = 1; w < DW; ++w) gm = fmaxf(gm, red[0][j][w]);
            const float sh = guarded_shift(gm);
            float l = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) l += exp2_hw((x[4 * j + e] - sh) * k);
            const float wl = wave_reduce<SumOp>(l);
            if (ln == 0) red[1][j][wv] = wl;
        }
        __syncthreads();
        if (t < F && c * F + t < a.nsub) {
            float gm = red[0][t][0], gl = red[1][t][0];
#pragma unroll
            for (int w = 1; w < DW; ++w) {
                gm = fmaxf(gm, red[0][t][w]);
                gl += red[1][t][w];
            }
            a.part[row * a.nsub + c * F + t] = make_float2(gm, gl);
        }
    } else {
        load_chunk<DT, F, VEC, true>(a.x + row * a.V, c * C, a.V, x, 0.0f);
#pragma unroll
        for (int j = 0; j < F; ++j) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (x[4 * j + e] > 0.0f) ? x[4 * j + e] : 0.0f;
            // the order the fused softmax sums its written probabilities in, so
            // that both give the same group sums for the same probabilities
            const float wl = wave_reduce<SumOp>((y[0] + y[1]) + (y[2] + y[3]));
            if (ln == 0) red[1][j][wv] = wl;
        }
        __syncthreads();
        if (t < F && c * F + t < a.nsub) {
            float gl = red[1][t][0];
#pragma unroll
            for (int w = 1; w < DW; ++w) gl += red[1][t][w];
            a.part[row * a.nsub + c * F + t] = make_float2(gl, 0.0f);
        }
    }
}

// ---------------------------------------------------------------------------
// ts_draw_resolve: wave g of the grid draws target g % K of row g / K.
// Lane l looks at groups b0 + 4 l + [0, 4) of each tile of 256 groups. With
// ONE (a row of at most 256 groups) the lane's 4 partials are loaded once and
// kept in registers; otherwise each pass reloads them tile by tile.
// ---------------------------------------------------------------------------
template <int KIND>
struct GroupWeights {
    const float2* prow;
    int64_t nsub;
    float gsh, k;
    // the 4 weights (shares of the row) of lane `ln` in tile b0: 0 past the row's end
    __device__ __forceinline__ void tile(int64_t b0, int ln, float (&w)[4]) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = b0 + 4 * ln + e;
            w[e] = i < nsub ? weight(prow[i]) : 0.0f;
        }
    }
    __device__ __forceinline__ float weight(float2 v) const {
        if constexpr (KIND == kDrawLogits) return masked_term(v.x, v.y * exp2_hw((v.x - gsh) * k));
        else return v.x;
    }
};

template <int KIND, bool VEC, bool ONE>
__global__ __launch_bounds__(DT) void ts_draw_resolve(DrawArgs a) {
    const int ln = threadIdx.x & (kWave - 1);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * DW + threadIdx.x / kWave;
    if (g >= a.B * a.K) return;   // the whole wave
    const int64_t row = g / a.K;
    const int64_t nsub = a.nsub;
    constexpr int64_t TILE = 4 * kWave;
    GroupWeights<KIND> gw{a.part + row * nsub, nsub, 0.0f, 0.0f};
    // independent loads first: the uniform, the temperature, the partials
    const float u = a.uniforms[g];
    if constexpr (KIND == kDrawLogits) gw.k = exp2_scale(a.temps[row]);
    float2 pv[4];
    if constexpr (ONE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = 4 * ln + e;
            pv[e] = i < nsub ? gw.prow[i] : make_float2(kNegInf, 0.0f);
        }
    }
    float w[4];   // ONE: the lane's weights, computed once

    if constexpr (KIND == kDrawLogits) {
        // the row max of the group maxima, as the finalize takes it
        float mm = kNegInf;
        if constexpr (ONE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) mm = fmaxf(mm, pv[e].x);
        } else {
            for (int64_t b0 = 0; b0 < nsub; b0 += TILE)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t i = b0 + 4 * ln + e;
                    if (i < nsub) mm = fmaxf(mm, gw.prow[i].x);
                }
        }
        gw.gsh = guarded_shift(wave_reduce<MaxOp>(mm));
    }
    if constexpr (ONE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = 4 * ln + e < nsub ? gw.weight(pv[e]) : 0.0f;
    }

    // float total of the weights (fixed order) -> the scale of the integer weights
    float tl = 0.0f;
    if constexpr (ONE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) tl += w[e];
    } else {
        for (int64_t b0 = 0; b0 < nsub; b0 += TILE) {
            gw.tile(b0, ln, w);
#pragma unroll
            for (int e = 0; e < 4; ++e) tl += w[e];
        }
    }
    const float tot = wave_reduce<SumOp>(tl);
    int32_t* out = a.out_ids + g;
    if (!(tot > 0.0f) || !(tot < __builtin_huge_valf())) {   // nothing can be drawn
        if (ln == 0) *out = -1;
        return;
    }
    const int s = scale_exponent(tot);
    uint64_t ql = 0;
    if constexpr (ONE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ql += fixed_point(w[e], s);
    } else {
        for (int64_t b0 = 0; b0 < nsub; b0 += TILE) {
            gw.tile(b0, ln, w);
#pragma unroll
            for (int e = 0; e < 4; ++e) ql += fixed_point(w[e], s);
        }
    }
    const uint64_t Q = wave_sum_u64(ql);
    const uint64_t T = target_of(u, Q);

    // the group whose integer range [P, P + q) holds T
    int64_t m = 0;
    uint64_t Pm = 0, qm = 0, carry = 0;
    for (int64_t b0 = 0; b0 < nsub; b0 += TILE) {
        if constexpr (!ONE) gw.tile(b0, ln, w);
        uint64_t q[4], lsum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            q[e] = fixed_point(w[e], s);
            lsum += q[e];
        }
        const uint64_t incl = wave_inclusive_scan_u64(lsum);
        const uint64_t lo = carry + incl - lsum;
        const bool hit = T >= lo && T - lo < lsum;
        const uint64_t hits = __ballot(hit);
        if (hits) {
            const int src = __ffsll(static_cast<unsigned long long>(hits)) - 1;
            int64_t mi = 0;
            uint64_t p0 = 0, q0 = 0;
            if (hit) {
                uint64_t acc = lo;   // <= T throughout
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (T - acc < q[e] && q0 == 0) {
                        mi = b0 + 4 * ln + e;
                        p0 = acc;
                        q0 = q[e];
                    }
                    acc += q[e];
                }
            }
            m = static_cast<int64_t>(lane_value_u64(static_cast<uint64_t>(mi), src));
            Pm = lane_value_u64(p0, src);
            qm = lane_value_u64(q0, src);
            break;
        }
        carry += lane_value_u64(incl, kWave - 1);
    }

    // the group's entries: lane l holds columns m 1024 + 16 l + [0, 16)
    const int64_t col0 = m * kDrawGroup + static_cast<int64_t>(GL) * ln;
    const float* xr = a.x + row * a.V;
    const float fill = KIND == kDrawLogits ? kNegInf : 0.0f;
    float v[GL];
    if constexpr (VEC) {
#pragma unroll
        for (int u = 0; u < GL / 4; ++u) {
            const int64_t col = col0 + 4 * u;
            f4 w4 = {fill, fill, fill, fill};
            if (col < a.V) w4 = *reinterpret_cast<const f4*>(xr + col);
            v[4 * u + 0] = w4.x; v[4 * u + 1] = w4.y; v[4 * u + 2] = w4.z; v[4 * u + 3] = w4.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < GL; ++i) v[i] = (col0 + i < a.V) ? xr[col0 + i] : fill;
    }
    int se;
    if constexpr (KIND == kDrawLogits) {
        if (const uint32_t* mrow = draw_mask_row(a, row)) {
            // 16 columns = half a mask word; the index is clamped to the row
            const int64_t last = (a.V - 1) >> 5;
            const int64_t wi = col0 >> 5;
            const uint32_t bits = mrow[wi < last ? wi : last] >> (col0 & 31);
#pragma unroll
            for (int i = 0; i < GL; ++i)
                if (col0 + i < a.V && !((bits >> i) & 1u)) v[i] = kNegInf;
        }
        // e = exp2((x - shift) k) <= 1 at the group's own max (the partial's pm)
        const float sh = guarded_shift(gw.prow[m].x);
#pragma unroll
        for (int i = 0; i < GL; ++i) v[i] = exp2_hw((v[i] - sh) * gw.k);
        se = 61 - 10;   // 1024 entries <= 1: integer total <= 2^61
    } else {
        se = scale_exponent(gw.prow[m].x);   // > 0: the group's q weight is >= 1
    }
    uint64_t gsum = 0;
#pragma unroll
    for (int i = 0; i < GL; ++i) gsum += fixed_point(v[i], se);
    const uint64_t gincl = wave_inclusive_scan_u64(gsum);
    const uint64_t L = lane_value_u64(gincl, kWave - 1);   // >= 1: the group holds its max entry
    // T carried into the group's units, clamped to its total
    const double f = static_cast<double>(T - Pm) * (static_cast<double>(L) / static_cast<double>(qm));
    uint64_t Tc = f < static_cast<double>(L) ? static_cast<uint64_t>(f) : L - 1;
    if (Tc > L - 1) Tc = L - 1;
    const uint64_t glo = gincl - gsum;
    if (Tc >= glo && Tc - glo < gsum) {   // exactly one lane
        uint64_t acc = glo;
        int i = 0;
        for (; i < GL - 1; ++i) {
            acc += fixed_point(v[i], se);
            if (acc > Tc) break;
        }
        *out = static_cast<int32_t>(col0 + i);
    }
}

template <int F, bool VEC>
hipError_t partials_impl(const DrawArgs& a, int kind, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(a.B * a.nch));
    if (kind == kDrawLogits) hipLaunchKernelGGL((ts_group_partials<F, VEC, kDrawLogits>), grid, dim3(DT), 0, s, a);
    else hipLaunchKernelGGL((ts_group_partials<F, VEC, kDrawProbs>), grid, dim3(DT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_group_partials(const DrawArgs& a, int F, bool vec, int kind, hipStream_t s) {
    switch (F) {
        case 1: return vec ? partials_impl<1, true>(a, kind, s) : partials_impl<1, false>(a, kind, s);
        case 4: return vec ? partials_impl<4, true>(a, kind, s) : partials_impl<4, false>(a, kind, s);
        case 8: return vec ? partials_impl<8, true>(a, kind, s) : partials_impl<8, false>(a, kind, s);
        default: return hipErrorInvalidValue;
    }
}

template <int KIND, bool ONE>
hipError_t resolve_impl(const DrawArgs& a, bool vec, dim3 grid, hipStream_t s) {
    if (vec) hipLaunchKernelGGL((ts_draw_resolve<KIND, true, ONE>), grid, dim3(DT), 0, s, a);
    else hipLaunchKernelGGL((ts_draw_resolve<KIND, false, ONE>), grid, dim3(DT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_draw_resolve(const DrawArgs& a, bool vec, int kind, hipStream_t s) {
    const int64_t waves = a.B * a.K;
    const dim3 grid(static_cast<uint32_t>((waves + DW - 1) / DW));
    const bool one = a.nsub <= 4 * kWave;
    if (kind == kDrawLogits)
        return one ? resolve_impl<kDrawLogits, true>(a, vec, grid, s) : resolve_impl<kDrawLogits, false>(a, vec, grid, s);
    return one ? resolve_impl<kDrawProbs, true>(a, vec, grid, s) : resolve_impl<kDrawProbs, false>(a, vec, grid, s);
}

}  // namespace tsk
