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
//  ts_draw_partials: one read of the row, one workgroup per group, no
//    exchange between workgroups. Each group gets a float partial: from
//    logits, the method's chunk partial (pm, pl) -- the group's max and the sum
//    of exp2((x - shift) k) with the -inf guard of the fix paragraph; from
//    probabilities, the sum of the positive entries. Each block gets its sum of
//    the same terms: the exponentials at its group's max, or the
//    probabilities; the group's sum is the sum of its block sums.
//  the resolve: one wave per (row, target), three levels. At each level the
//    64 lanes hold 64 float weights -- the row's groups (for logits, their pl
//    rescaled to the row's max as in the finalize, so that a fully masked
//    group weighs exactly 0), then the chosen group's blocks, then the chosen
//    block's entries -- which become integers at one power-of-two scale; an
//    integer prefix sum over the lanes gives each its range, and the lane whose
//    range holds the target is chosen. The target is carried into the next
//    level's integer units in double precision and clamped to its total.
//    Level 1 is the same for all targets of a row: ts_draw_resolve_rows
//    computes it once per 16 waves and shares it through LDS (each wave then
//    takes 1 or 2 targets, their loads issued together: resolve_row_batch;
//    for rows of few groups level 2 of every group is shared the same way),
//    ts_draw_resolve_waves in every wave (resolve_shares_rows picks).
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
static_assert(DT * 4 * 4 == kDrawGroup && DW == 4, "a group is four float4 per lane of four waves");
static_assert(kBlocksPerGroup == kWave && kDrawBlock == kWave, "one lane per block, one lane per entry");

__device__ __forceinline__ const uint32_t* draw_mask_row(const DrawArgs& a, int64_t row) {
    return a.allowed ? a.allowed + row * a.mwords : nullptr;
}

// ---------------------------------------------------------------------------
// ts_draw_partials: one workgroup per group of 4096 columns (item = row
// ngroups + group). Lane t holds the float4 at column 1024 j + 4 t of the
// group (the layout of load_chunk, j < 4), so block 16 j + t / 16 is one row
// of 16 lanes. The block sums meet in LDS and leave in one 256-byte store;
// the group's sum is the sum of its block sums.
// ---------------------------------------------------------------------------
template <int LD, int KIND>
__global__ __launch_bounds__(DT) void ts_draw_partials(DrawArgs a) {
    constexpr int F = kDrawGroup / (DT * 4);
    __shared__ float red[DW];                 // (logits: the group's max)
    __shared__ float blocks[kBlocksPerGroup];
    const int t = threadIdx.x;
    // (32-bit: the grid is; a 64-bit division would hold up the first loads)
    const uint32_t ng = static_cast<uint32_t>(a.ngroups);
    const uint32_t row32 = blockIdx.x / ng;
    const int64_t item = blockIdx.x;
    const int64_t row = row32;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x - row32 * ng) * kDrawGroup;
    const bool masked = KIND == kDrawLogits && a.allowed;
    float x[4 * F];
    uint32_t mw[2];
    issue_chunk_loads<DT, F, LD, true>(a.x + row * a.V, c0, a.V, x);
    if (masked) load_mask_words<DT, F>(draw_mask_row(a, row), c0, a.V, mw);
    if (c0 + kDrawGroup > a.V) {   // (workgroup-uniform: the row's last, partial group)
        if constexpr (LD == kLdUnaligned) shift_tail_group<DT, F>(c0, a.V, x);
        fill_past_end<DT, F>(c0, a.V, x, KIND == kDrawLogits ? kNegInf : 0.0f);
    }
    float gm = 0.0f;
    if constexpr (KIND == kDrawLogits) {
        if (masked) apply_mask_words<DT, F>(c0, a.V, mw, x);
        // the method's chunk partial for the group: its max, then the sum of
        // exp2((x - shift) k) with the -inf guard; the blocks sum the same terms
        float m = kNegInf;
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) m = fmaxf(m, x[i]);
        m = wave_reduce<MaxOp>(m);
        if ((t & (kWave - 1)) == 0) red[t / kWave] = m;
        __syncthreads();   // (red is written once: no barrier after its reads)
        gm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const float gsh = guarded_shift(gm);
        const float k = exp2_scale(a.temps[row]);
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) x[i] = exp2_hw((x[i] - gsh) * k);
    } else {
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) x[i] = fmaxf(x[i], 0.0f);   // NaN and negatives hold no mass
    }
    block_sums_to_lds<F>(x, blocks);
    __syncthreads();
    if (t < kWave) {
        const float b = blocks[t];
        a.bpart[item * kBlocksPerGroup + t] = b;
        const float g = wave_reduce<SumOp>(b);
        if (t == 0) a.gpart[item] = KIND == kDrawLogits ? make_float4(gm, g, 0.0f, 0.0f) : make_float4(g, 0.0f, 0.0f, 0.0f);
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

// Level 1 of a row, common to all its targets. The row's groups, 64 per tile,
// lane l holding group b0 + l, get float weights (from logits: pl rescaled to
// the row's max, as in the finalize, so that a fully masked group weighs
// exactly 0; from probabilities: the waves' sums), then integers at one
// power-of-two scale 2^s1.
template <int KIND>
struct RowGroups {
    const float4* grow;   // the row's group partials
    int64_t ng;
    float k;              // exp2 scale (logits)
    float gsh;            // the row's guarded max (logits)
    int s1;

    __device__ __forceinline__ float weight(float4 v, int64_t i) const {
        if (i >= ng) return 0.0f;
        if constexpr (KIND == kDrawLogits) return masked_term(v.x, v.y * exp2_hw((v.x - gsh) * k));
        else return group_prob_sum(v);
    }
    __device__ __forceinline__ float4 part(int64_t i) const {
        return i < ng ? grow[i] : make_float4(kNegInf, 0.0f, 0.0f, 0.0f);
    }
    // group b0 + ln's integer weight (0 past the row's end)
    __device__ __forceinline__ uint64_t q(int64_t b0, int ln) const {
        return fixed_point(weight(part(b0 + ln), b0 + ln), s1);
    }
};

// Fills r for `row` and returns the row's integer total Q, or 0 when nothing
// can be drawn (no positive weight, or a total that is not finite). q0 and
// incl0: the first tile's integers and their inclusive scan. Called by all
// lanes of one wave.
template <int KIND>
__device__ __forceinline__ uint64_t row_level1(const DrawArgs& a, int64_t row, float k, int ln, RowGroups<KIND>& r,
                                               uint64_t& q0, uint64_t& incl0) {
    r.grow = a.gpart + row * a.ngroups;
    r.ng = a.ngroups;
    r.k = k;
    r.gsh = 0.0f;
    const float4 gv = r.part(ln);
    if constexpr (KIND == kDrawLogits) {
        float mm = gv.x;
        for (int64_t b0 = kWave; b0 < r.ng; b0 += kWave) mm = fmaxf(mm, r.part(b0 + ln).x);
        r.gsh = guarded_shift(wave_reduce<MaxOp>(mm));
    }
    const float gw0 = r.weight(gv, ln);
    float tl = gw0;
    for (int64_t b0 = kWave; b0 < r.ng; b0 += kWave) tl += r.weight(r.part(b0 + ln), b0 + ln);
    const float tot = wave_reduce<SumOp>(tl);
    if (!(tot > 0.0f) || !(tot < __builtin_huge_valf())) return 0;
    r.s1 = scale_exponent(tot);
    q0 = fixed_point(gw0, r.s1);
    incl0 = wave_inclusive_scan_u64(q0);
    uint64_t Q = lane_value_u64(incl0, kWave - 1);
    if (r.ng > kWave) {   // the row's integer total over every tile
        uint64_t ql = 0;
        for (int64_t b0 = kWave; b0 < r.ng; b0 += kWave) ql += r.q(b0, ln);
        Q += wave_sum_u64(ql);
    }
    return Q;   // >= 1: the largest group's integer is at least 2^60 / ng
}

// Levels 2 and 3 of one target, by one wave: the target T lies in
// [PG, PG + qG) of the level-1 integers, in group G. Writes the id (or -1).
template <int KIND>
__device__ __forceinline__ void resolve_in_group(const DrawArgs& a, int64_t row, float k, int64_t G, uint64_t T,
                                                 uint64_t PG, uint64_t qG, int32_t* out, int ln) {
    const int64_t ng = a.ngroups;
    // level 2: the group's 64 blocks, lane l holding block l
    // (block weights: sums of the group's exponentials at its max, or of probabilities)
    const float bw = a.bpart[(row * ng + G) * kBlocksPerGroup + ln];
    const int s2 = scale_exponent(wave_reduce<SumOp>(bw));   // > 0: qG >= 1 needs a positive group
    const uint64_t qb = fixed_point(bw, s2);
    const uint64_t incl2 = wave_inclusive_scan_u64(qb);
    const uint64_t T2 = carry_target(T, PG, qG, lane_value_u64(incl2, kWave - 1));
    const int b = find_lane(qb, incl2, 0, T2);
    // (the ranges tile each level's total and the target lies below it, so
    // this and the check below never fire; they keep every index in bounds)
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
        v = exp2_hw((v - guarded_shift(a.gpart[row * ng + G].x)) * k);   // as the partials kernel formed them
    }
    const int s3 = scale_exponent(bx);   // each entry <= the block's sum
    const uint64_t qe = fixed_point(v, s3);
    const uint64_t incl3 = wave_inclusive_scan_u64(qe);
    const uint64_t T3 = carry_target(T2, Pb, qbb, lane_value_u64(incl3, kWave - 1));
    const int e = find_lane(qe, incl3, 0, T3);
    if (e < 0 && ln == 0) *out = -1;
    if (ln == e) *out = static_cast<int32_t>(col);
}

// Levels 2 and 3 of M targets of one row, by one wave: resolve_in_group's
// integers for each, with every target's loads at a level issued before any
// of them is used, so that a wave waits on memory once per level rather than
// once per level and target. live[j] is wave-uniform and cleared for a target
// that is done (its id, or -1, written). SH: every group's level-2 integers
// (inclusive scan, lane l for block l) and block weights are already in LDS
// at l2i and l2w, computed by the same code, so they are the same integers.
template <int KIND, int M, bool SH>
__device__ __forceinline__ void resolve_in_group_batch(const DrawArgs& a, int64_t row, float k, const int64_t (&G)[M],
                                                       const uint64_t (&T)[M], const uint64_t (&PG)[M],
                                                       const uint64_t (&qG)[M], bool (&live)[M],
                                                       int32_t* const (&out)[M], int ln,
                                                       const uint64_t* l2i, const float* l2w) {
    const int64_t ng = a.ngroups;
    float bw[M], gx[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {   // level 2 weights (and, from logits, the group's kept max)
        if constexpr (SH) bw[j] = live[j] ? l2w[G[j] * kWave + ln] : 0.0f;
        else bw[j] = live[j] ? a.bpart[(row * ng + G[j]) * kBlocksPerGroup + ln] : 0.0f;
        gx[j] = KIND == kDrawLogits && live[j] ? a.gpart[row * ng + G[j]].x : 0.0f;
    }
    uint64_t T2[M], Pb[M], qbb[M];
    int64_t col[M];
    int s3[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        T2[j] = 0; Pb[j] = 0; qbb[j] = 0; col[j] = 0; s3[j] = 0;
        if (!live[j]) continue;
        uint64_t qb, incl2;
        if constexpr (SH) {
            incl2 = l2i[G[j] * kWave + ln];
            qb = incl2 - (ln > 0 ? l2i[G[j] * kWave + ln - 1] : 0);
        } else {
            const int s2 = scale_exponent(wave_reduce<SumOp>(bw[j]));
            qb = fixed_point(bw[j], s2);
            incl2 = wave_inclusive_scan_u64(qb);
        }
        T2[j] = carry_target(T[j], PG[j], qG[j], lane_value_u64(incl2, kWave - 1));
        const int b = find_lane(qb, incl2, 0, T2[j]);
        if (b < 0) {   // (never, as in resolve_in_group)
            if (ln == 0) *out[j] = -1;
            live[j] = false;
            continue;
        }
        Pb[j] = lane_value_u64(incl2 - qb, b);
        qbb[j] = lane_value_u64(qb, b);
        s3[j] = scale_exponent(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(bw[j]), b)));
        col[j] = G[j] * kDrawGroup + static_cast<int64_t>(b) * kDrawBlock + ln;
    }
    const float* xr = a.x + row * a.V;
    const uint32_t* mrow = KIND == kDrawLogits ? draw_mask_row(a, row) : nullptr;
    float v[M];
    uint32_t mw[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {   // level 3 entries (and their allowed words)
        const bool in = live[j] && col[j] < a.V;
        v[j] = in ? xr[col[j]] : (KIND == kDrawLogits ? kNegInf : 0.0f);
        mw[j] = mrow && in ? mrow[col[j] >> 5] : ~0u;
    }
#pragma unroll
    for (int j = 0; j < M; ++j) {
        if (!live[j]) continue;
        float e3 = v[j];
        if constexpr (KIND == kDrawLogits) {
            if (!((mw[j] >> (col[j] & 31)) & 1u)) e3 = kNegInf;
            e3 = exp2_hw((e3 - guarded_shift(gx[j])) * k);   // as the partials kernel formed them
        }
        const uint64_t qe = fixed_point(e3, s3[j]);
        const uint64_t incl3 = wave_inclusive_scan_u64(qe);
        const uint64_t T3 = carry_target(T2[j], Pb[j], qbb[j], lane_value_u64(incl3, kWave - 1));
        const int e = find_lane(qe, incl3, 0, T3);
        if (e < 0 && ln == 0) *out[j] = -1;
        if (ln == e) *out[j] = static_cast<int32_t>(col[j]);
    }
}

// ts_draw_resolve_rows: workgroup (row, tile) draws targets tile TW M + j TW + w
// (w < TW, j < M) of the row, M per wave. Wave 0 does level 1 once for all of them
// and leaves the groups' inclusive integer prefix sums in LDS (incl[0, ng),
// then the row's total Q at incl[ng]); each wave then finds its target's group
// as the first with a prefix above the target, which is the group whose range
// holds it. The integers are those of ts_draw_resolve_waves, so are the ids.
// Dynamic LDS: 8 (ngroups + 1) bytes.
template <int KIND, int M, bool SH>
__global__ __launch_bounds__(kWave * kResolveRowTargets) void ts_draw_resolve_rows(DrawArgs a) {
    constexpr int TW = kResolveRowTargets;
    extern __shared__ uint64_t incl[];
    const int ln = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int64_t ntiles = (a.K + TW * M - 1) / (TW * M);
    const int64_t row = blockIdx.x / ntiles;
    const int64_t k0 = (blockIdx.x - row * ntiles) * (TW * M) + w;
    const int64_t ng = a.ngroups;
    bool live[M];
    float u[M];
    int32_t* out[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const int64_t kk = k0 + static_cast<int64_t>(j) * TW;
        live[j] = kk < a.K;   // wave-uniform
        u[j] = live[j] ? a.uniforms[row * a.K + kk] : 0.0f;
        out[j] = a.out_ids + row * a.K + (live[j] ? kk : 0);
    }
    const float k = KIND == kDrawLogits ? exp2_scale(a.temps[row]) : 0.0f;
    if (w == 0) {
        RowGroups<KIND> r;
        uint64_t q0 = 0, incl0 = 0;
        const uint64_t Q = row_level1<KIND>(a, row, k, ln, r, q0, incl0);
        if (Q > 0) {
            if (ln < ng) incl[ln] = incl0;
            uint64_t carry = lane_value_u64(incl0, kWave - 1);
            for (int64_t b0 = kWave; b0 < ng; b0 += kWave) {
                const uint64_t t = wave_inclusive_scan_u64(r.q(b0, ln));
                if (b0 + ln < ng) incl[b0 + ln] = carry + t;
                carry += lane_value_u64(t, kWave - 1);
            }
        }
        if (ln == 0) incl[ng] = Q;
    }
    uint64_t* l2i = incl + ng + 1;
    float* l2w = reinterpret_cast<float*>(l2i + (SH ? ng * kWave : 0));
    if constexpr (SH) {   // wave 1 + g: group g's level 2, for every target of the workgroup
        const int64_t g = w - 1;
        if (w >= 1 && g < ng) {
            const float bw = a.bpart[(row * ng + g) * kBlocksPerGroup + ln];
            const int s2 = scale_exponent(wave_reduce<SumOp>(bw));
            l2i[g * kWave + ln] = wave_inclusive_scan_u64(fixed_point(bw, s2));
            l2w[g * kWave + ln] = bw;
        }
    }
    __syncthreads();
    const uint64_t Q = incl[ng];
    int64_t G[M];
    uint64_t T[M], PG[M], qG[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        G[j] = 0; T[j] = 0; PG[j] = 0; qG[j] = 0;
        if (!live[j]) continue;
        if (Q == 0) {   // nothing can be drawn
            if (ln == 0) *out[j] = -1;
            live[j] = false;
            continue;
        }
        T[j] = target_of(u[j], Q);
        int64_t g = -1;
        for (int64_t b0 = 0; b0 < ng && g < 0; b0 += kWave) {
            const uint64_t hits = __ballot(b0 + ln < ng && incl[b0 + ln] > T[j]);
            if (hits) g = b0 + __ffsll(static_cast<unsigned long long>(hits)) - 1;
        }
        if (g < 0) {   // (never: incl[ng - 1] = Q > T)
            if (ln == 0) *out[j] = -1;
            live[j] = false;
            continue;
        }
        G[j] = g;
        PG[j] = g > 0 ? incl[g - 1] : 0;
        qG[j] = incl[g] - PG[j];
    }
    if constexpr (M == 1 && !SH) {
        if (live[0]) resolve_in_group<KIND>(a, row, k, G[0], T[0], PG[0], qG[0], out[0], ln);
    } else {
        resolve_in_group_batch<KIND, M, SH>(a, row, k, G, T, PG, qG, live, out, ln, l2i, l2w);
    }
}

// ts_draw_resolve_waves (rows whose prefix sums do not fit LDS): wave w of the
// grid draws target w % K of row w / K and does level 1 itself, finding the
// target's group tile by tile.
template <int KIND>
__global__ __launch_bounds__(DT) void ts_draw_resolve_waves(DrawArgs a) {
    const int ln = threadIdx.x & (kWave - 1);
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * DW + threadIdx.x / kWave;
    if (wid >= a.B * a.K) return;   // the whole wave
    const int64_t row = wid / a.K;
    int32_t* out = a.out_ids + wid;
    const float u = a.uniforms[wid];
    const float k = KIND == kDrawLogits ? exp2_scale(a.temps[row]) : 0.0f;
    RowGroups<KIND> r;
    uint64_t q0 = 0, incl0 = 0;
    const uint64_t Q = row_level1<KIND>(a, row, k, ln, r, q0, incl0);
    if (Q == 0) {   // nothing can be drawn
        if (ln == 0) *out = -1;
        return;
    }
    const uint64_t T = target_of(u, Q);
    int64_t G = -1;
    uint64_t PG = 0, qG = 0, carry = 0;
    for (int64_t b0 = 0; b0 < r.ng; b0 += kWave) {
        uint64_t q = q0, incl = incl0;
        if (b0 > 0) {
            q = r.q(b0, ln);
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
    if (G < 0) {   // (never: the ranges tile [0, Q) and T < Q)
        if (ln == 0) *out = -1;
        return;
    }
    resolve_in_group<KIND>(a, row, k, G, T, PG, qG, out, ln);
}

template <int LD>
hipError_t partials_impl(const DrawArgs& a, int kind, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(a.B * a.ngroups));
    if (kind == kDrawLogits) hipLaunchKernelGGL((ts_draw_partials<LD, kDrawLogits>), grid, dim3(DT), 0, s, a);
    else hipLaunchKernelGGL((ts_draw_partials<LD, kDrawProbs>), grid, dim3(DT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_draw_partials(const DrawArgs& a, int ld, int kind, hipStream_t s) {
    // the unaligned loads need a row of at least 4 columns
    if (ld == kLdUnaligned && a.V < 4) ld = kLdScalar;
    switch (ld) {
        case kLdAligned: return partials_impl<kLdAligned>(a, kind, s);
        case kLdUnaligned: return partials_impl<kLdUnaligned>(a, kind, s);
        case kLdScalar: return partials_impl<kLdScalar>(a, kind, s);
        default: return hipErrorInvalidValue;
    }
}

namespace {

// Targets per wave of ts_draw_resolve_rows: a wave that resolves two targets
// issues both targets' loads together, but the grid halves; two only while
// the grid keeps at least 4 workgroups per compute unit (two rounds of the
// device's resident workgroups of 1024 lanes). The resolve is bound by issue
// more than by memory waits, so four (at 5-6 waves per SIMD) was slower.
// Rows of at most this many groups (32768 columns) have every group's level 2
// computed once per workgroup, by waves 1..ng beside wave 0's level 1, and
// shared through LDS (12 bytes per block); longer rows compute it per target.
constexpr int64_t kShareLevel2Groups = 8;
static_assert(kShareLevel2Groups < kResolveRowTargets, "one wave per group besides wave 0");

int resolve_row_batch(int64_t B, int64_t K, int64_t cus) {
    const int64_t per = 2 * static_cast<int64_t>(kResolveRowTargets);
    return B * ((K + per - 1) / per) >= 4 * cus ? 2 : 1;
}

template <int KIND>
hipError_t resolve_impl(const DrawArgs& a, hipStream_t s) {
    if (resolve_shares_rows(a.B, a.K, a.ngroups, a.cus)) {
        const int M = resolve_row_batch(a.B, a.K, a.cus);
        const int64_t per = static_cast<int64_t>(kResolveRowTargets) * M;
        const dim3 grid(static_cast<uint32_t>(a.B * ((a.K + per - 1) / per)));
        const dim3 block(kWave * kResolveRowTargets);
        const bool sh = a.ngroups <= kShareLevel2Groups;
        const size_t lds = static_cast<size_t>(a.ngroups + 1) * sizeof(uint64_t) +
                           (sh ? static_cast<size_t>(a.ngroups) * kWave * (sizeof(uint64_t) + sizeof(float)) : 0);
        if (sh) {
            if (M == 2) hipLaunchKernelGGL((ts_draw_resolve_rows<KIND, 2, true>), grid, block, lds, s, a);
            else hipLaunchKernelGGL((ts_draw_resolve_rows<KIND, 1, true>), grid, block, lds, s, a);
        } else {
            if (M == 2) hipLaunchKernelGGL((ts_draw_resolve_rows<KIND, 2, false>), grid, block, lds, s, a);
            else hipLaunchKernelGGL((ts_draw_resolve_rows<KIND, 1, false>), grid, block, lds, s, a);
        }
    } else {
        const dim3 grid(static_cast<uint32_t>((a.B * a.K + DW - 1) / DW));
        hipLaunchKernelGGL((ts_draw_resolve_waves<KIND>), grid, dim3(DT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

// Sharing level 1 saves each row's redundant level-1 work but puts 16 targets
// on one compute unit; measured on MI355X at B=64 (µs per ts_sample call,
// cold), it wins once the grid still gives every compute unit a workgroup:
// K=16 +1.0, K=32 +0.7, K=64 -0.3, K=128 -0.6, K=256 -0.9.
bool resolve_shares_rows(int64_t B, int64_t K, int64_t ngroups, int64_t cus) {
    if ((ngroups + 1) * static_cast<int64_t>(sizeof(uint64_t)) > kResolveLdsMax) return false;
    return K >= kResolveRowTargets && B * ((K + kResolveRowTargets - 1) / kResolveRowTargets) >= cus;
}

hipError_t launch_draw_resolve(const DrawArgs& a, int kind, hipStream_t s) {
    return kind == kDrawLogits ? resolve_impl<kDrawLogits>(a, s) : resolve_impl<kDrawProbs>(a, s);
}

}  // namespace tsk
