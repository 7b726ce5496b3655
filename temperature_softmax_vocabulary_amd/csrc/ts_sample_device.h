// Device-side pieces of the inverse-CDF token draw, shared by ts_sample and the
// fused softmax-and-sample kernel.
//
// The pull-request page "fix(kernel): avoid nan in triton sampling softmax
// when a chunk starts with -inf" feeds the softmax into a draw of token ids
// (scope paragraph) that must land on allowed ids only (results table,
// sampling row). The rule used: with u clamped to [0, 1] (NaN -> 0) and C the
// row's inclusive prefix sums in id order, the id is the smallest j with
// C[j] > u * C[V-1].
//
// How the chunked kernels form the prefix sums, with one exchange per row:
//  * Across chunks. Every chunk publishes one float weight (its share of the
//    row). Each workgroup of the row turns the row's weights into integers at
//    one power-of-two scale (chunk_range) and takes exact integer prefix sums:
//    all of them compute the same integers from the same slot values, so the
//    chunks' ranges [base, base + width) tile [0, Q) with no gap or overlap,
//    and the chunk whose range holds the target T = min(floor(u Q), Q - 1)
//    resolves it. A chunk with no positive entry has width 0 and never does.
//  * Inside a chunk. Each entry e > 0 becomes q = rint(e * 2^s) at a
//    power-of-two scale of the chunk, and the integer prefix sums of the q are
//    exact whatever the order of addition. T is carried into the chunk's units
//    in double precision and clamped to its integer total L; the id is the
//    smallest column whose prefix exceeds it. That column always has q >= 1,
//    so an entry that is not > 0 (a masked id) is never drawn.
// The draw therefore follows the rule up to the float rounding of the chunk
// weights (about 1e-7 of the row total). When the weights and entries are
// dyadic and their float sums exact, every step is exact and the ids are the
// rule's ids exactly.
#pragma once

#include "ts_device.h"

namespace tsk {

// q = rint(p * 2^s) for p > 0, else 0 (zero, negative and NaN entries).
__device__ __forceinline__ uint64_t fixed_point(float p, int s) {
    if (!(p > 0.0f)) return 0;
    return static_cast<uint64_t>(rintf(ldexpf(p, s)));
}

// Scale exponent for a row whose positive entries sum to `total` (> 0, finite):
// every entry is <= total < 2^e, so each q < 2^61 (1 + rounding) and Q < 2^62.
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

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// A chunk's share of its row's integer CDF.
struct ChunkRange {
    uint64_t base;    // integer prefix of the chunks before it
    uint64_t width;   // its own integer weight
    uint64_t total;   // the row's integer total Q (0: nothing can be drawn)
};

// Called by the 64 lanes of one wave with w[j] = float weight of chunk
// lane + 64 j (0 for chunks past the row's end or without a positive entry);
// returns chunk c's range to every lane. The scale comes from the float total
// (each integer weight < 2^61, so the total < 2^62); reductions run in a fixed
// order, so every workgroup of the row gets the same integers.
template <int N>
__device__ __forceinline__ ChunkRange chunk_range(const float (&w)[N], int64_t c) {
    const int lane = threadIdx.x & (kWave - 1);
    float tot = 0.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) tot += w[j];
    tot = wave_reduce<SumOp>(tot);
    ChunkRange r = {0, 0, 0};
    if (!(tot > 0.0f) || !(tot < __builtin_huge_valf())) return r;
    const int s = scale_exponent(tot);
    uint64_t before = 0, mine = 0, all = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const int64_t i = lane + static_cast<int64_t>(j) * kWave;
        const uint64_t q = fixed_point(w[j], s);
        all += q;
        before += (i < c) ? q : 0;
        mine += (i == c) ? q : 0;
    }
    r.base = wave_sum_u64(before);
    r.width = wave_sum_u64(mine);
    r.total = wave_sum_u64(all);
    return r;
}

// LDS bytes resolve_chunk needs for NT lanes and chunks of F groups.
template <int NT, int F>
constexpr size_t resolve_lds_bytes() {
    return static_cast<size_t>(F) * NT * sizeof(uint64_t)          // column-order prefix per (group, lane)
           + static_cast<size_t>(NT / kWave) * F * sizeof(uint64_t);   // wave totals per group
}

// Resolve every target of the row that falls in chunk range r.
//
// e[] holds the chunk's entries in the layout of load_chunk: F groups of
// NT * 4 consecutive columns, lane t holding columns (j NT + t) 4 + e of group
// j, so (group, lane) order is column order. Lane t takes targets t, t + NT,
// ... of the row; u0 is its uniform for target t (loaded ahead by the caller).
// Only when some target lands in the chunk are the lanes' per-group integer
// sums at scale 2^s scanned into an LDS table pre[j NT + t] of column-order
// exclusive prefixes (all groups in one pass: wave shuffles, then one LDS round
// for the wave totals). The owner of chunk-relative target Tc is the largest m
// with pre[m] <= Tc (binary search; an entry whose sum is 0 has the same prefix
// as the next one, so the largest is never empty), and fetch(j, t, v) reloads
// the owner's 4 entries -- bitwise the values summed here -- for a walk to the
// smallest column whose running sum exceeds Tc. `lds` points at
// resolve_lds_bytes<NT, F>() bytes; all lanes must call; r.width > 0 implies
// that the chunk holds an entry e with rint(e 2^s) >= 1.
template <int NT, int F, class Fetch>
__device__ __forceinline__ void resolve_chunk(const float (&e)[4 * F], unsigned char* lds, int s, ChunkRange r,
                                              int64_t c0, float u0, const float* __restrict__ urow, int64_t K,
                                              int32_t* __restrict__ idrow, const Fetch& fetch) {
    constexpr int NW = NT / kWave;
    uint64_t* pre = reinterpret_cast<uint64_t*>(lds);
    uint64_t* wt = pre + F * NT;
    const int t = threadIdx.x;
    const int ln = t & (kWave - 1), wv = t / kWave;
    bool scanned = false;
    uint64_t L = 0;   // the chunk's integer total
    for (int64_t kb = 0; kb < K; kb += NT) {
        const int64_t k = kb + t;
        uint64_t T = 0;
        bool own = false;
        if (k < K) {
            T = target_of(kb == 0 ? u0 : urow[k], r.total);
            own = T >= r.base && T - r.base < r.width;
        }
        if (!__syncthreads_or(own)) continue;
        if (!scanned) {
            // one group at a time (few live registers): wave-inclusive scans of
            // the lanes' 4-entry sums, kept in pre[] as wave-exclusive prefixes,
            // and the wave totals in wt[]; then one LDS round adds the offsets
#pragma unroll
            for (int j = 0; j < F; ++j) {
                const uint64_t sg = fixed_point(e[4 * j], s) + fixed_point(e[4 * j + 1], s) +
                                    fixed_point(e[4 * j + 2], s) + fixed_point(e[4 * j + 3], s);
                uint64_t x = sg;
#pragma unroll
                for (int d = 1; d < kWave; d <<= 1) {
                    const uint64_t y = __shfl_up(x, d, kWave);
                    if (ln >= d) x += y;
                }
                pre[j * NT + t] = x - sg;
                if (ln == kWave - 1) wt[wv * F + j] = x;
            }
            __syncthreads();
            uint64_t run = 0;
#pragma unroll
            for (int j = 0; j < F; ++j) {
                uint64_t before = 0, total = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const uint64_t v = wt[w * F + j];
                    total += v;
                    before += (w < wv) ? v : 0;
                }
                pre[j * NT + t] += run + before;
                run += total;
            }
            L = run;
            __syncthreads();   // pre complete before any lane searches it
            scanned = true;
        }
        if (!own) continue;
        // the target's place inside the chunk, in the chunk's own units
        const double f = static_cast<double>(T - r.base) * (static_cast<double>(L) / static_cast<double>(r.width));
        uint64_t Tc = f < static_cast<double>(L) ? static_cast<uint64_t>(f) : L - 1;
        if (Tc > L - 1) Tc = L - 1;
        int lo = 0, hi = F * NT - 1;             // largest m with pre[m] <= Tc (pre[0] = 0)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= Tc) lo = mid; else hi = mid - 1;
        }
        const int j = lo / NT, o = lo - j * NT;
        float v[4];
        fetch(j, o, v);
        uint64_t acc = pre[lo];
        int ee = 0;
        for (; ee < 3; ++ee) {
            acc += fixed_point(v[ee], s);
            if (acc > Tc) break;
        }
        idrow[k] = static_cast<int32_t>(c0 + (static_cast<int64_t>(j) * NT + o) * 4 + ee);
    }
}

// Reload of the 4 entries a lane holds for group j of a chunk: probabilities
// read back from memory (ts_sample), or recomputed from the logits with the
// same instructions that produced them in registers (fused softmax-and-draw).
template <int NT>
__device__ __forceinline__ void load_group4(const float* __restrict__ row, int64_t c0, int64_t V, int j, int o,
                                            float fill, float (&v)[4], const uint32_t* __restrict__ mrow = nullptr) {
    const int64_t col = c0 + (static_cast<int64_t>(j) * NT + o) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (col + e < V) ? row[col + e] : fill;
    if (mrow && col < V) apply_allowed(mrow, col, v);
}

}  // namespace tsk
