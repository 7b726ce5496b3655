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
// Exactness: each entry p > 0 becomes the integer q = rint(p * 2^s), with one
// power of two 2^s per row, chosen so that the row's integer total Q stays
// below 2^62. Scaling by a power of two is exact, so q depends only on p and s;
// integer sums do not depend on the order of addition. With the target
// T = min(floor(u * Q), Q - 1) the id is the smallest j with Q[j] > T, and
// Q[j] > T >= Q[j-1] forces q[j] >= 1: an entry that is not > 0 (a masked id)
// is never drawn, whichever lanes and workgroups add which parts.
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

// Sum over the workgroup (NW waves); lds holds NW values. Returned to all lanes.
template <int NW>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* lds) {
    v = wave_sum_u64(v);
    if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
    __syncthreads();
    uint64_t r = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) r += lds[i];
    __syncthreads();
    return r;
}

// Exclusive prefix over lanes in threadIdx order; lds holds NW values.
template <int NW>
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* lds) {
    const int ln = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    uint64_t x = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint64_t y = __shfl_up(x, d, kWave);
        if (ln >= d) x += y;
    }
    if (ln == kWave - 1) lds[wv] = x;
    __syncthreads();
    uint64_t before = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) before += (i < wv) ? lds[i] : 0;
    __syncthreads();
    return before + x - v;
}

// Targets per batch held in LDS by resolve_chunk.
constexpr int kTargetBatch = 256;

// LDS bytes resolve_chunk needs for NT lanes and chunks of F groups.
template <int NT, int F>
constexpr size_t resolve_lds_bytes() {
    return kTargetBatch * sizeof(uint64_t)              // targets of a batch
           + static_cast<size_t>(F) * NT * sizeof(uint64_t)   // column-order prefix per (group, lane)
           + static_cast<size_t>(NT / kWave) * F * sizeof(uint64_t);   // wave totals per group
}

// Resolve, inside one chunk, every target of the row that falls in it.
//
// The chunk's entries p (the probabilities) sit in registers in the layout of
// load_chunk: F groups of NT * 4 consecutive columns, lane t holding columns
// (j NT + t) 4 + e of group j, so (group, lane) order is column order. The
// lanes' per-group integer sums are scanned across the workgroup into an LDS
// table pre[j NT + t] of column-order exclusive prefixes (all groups in one
// pass: wave shuffles, then one LDS round for the wave totals). The row's
// uniforms become integer targets a batch at a time (one per lane, loads in
// parallel) in LDS. Each lane then takes its own share of the batch's targets
// that fall in [base, base + Qc): the owner of chunk-relative target Tc is the
// largest m with pre[m] <= Tc (binary search; an entry whose sum is 0 has the
// same prefix as the next one, so the largest is never empty), and
// fetch(j, t, v) reloads the owner's 4 entries -- bitwise the values summed
// here -- for a walk to the smallest column whose running sum exceeds Tc.
// `lds` points at resolve_lds_bytes<NT, F>() bytes; all lanes must call.
template <int NT, int F, class Fetch>
__device__ __forceinline__ void resolve_chunk(const float (&p)[4 * F], unsigned char* lds, int s,
                                              uint64_t base, uint64_t Qc, uint64_t Q, int64_t c0,
                                              const float* __restrict__ urow, int64_t K,
                                              int32_t* __restrict__ idrow, const Fetch& fetch) {
    constexpr int NW = NT / kWave;
    uint64_t* tgt = reinterpret_cast<uint64_t*>(lds);
    uint64_t* pre = tgt + kTargetBatch;
    uint64_t* wt = pre + F * NT;
    const int t = threadIdx.x;
    const int ln = t & (kWave - 1), wv = t / kWave;
    bool scanned = false;
    for (int64_t kb = 0; kb < K; kb += kTargetBatch) {
        const int n = static_cast<int>(K - kb < kTargetBatch ? K - kb : kTargetBatch);
        int hit = 0;
        for (int i = t; i < n; i += NT) {
            const uint64_t T = target_of(urow[kb + i], Q);
            tgt[i] = T;
            hit |= (T >= base && T - base < Qc) ? 1 : 0;
        }
        if (!__syncthreads_or(hit)) continue;      // also orders the tgt writes
        if (!scanned) {
            // all groups at once: wave scans, one LDS round for the wave totals
            uint64_t sg[F], x[F];
#pragma unroll
            for (int j = 0; j < F; ++j) {
                sg[j] = fixed_point(p[4 * j], s) + fixed_point(p[4 * j + 1], s) + fixed_point(p[4 * j + 2], s) +
                        fixed_point(p[4 * j + 3], s);
                x[j] = sg[j];
            }
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
#pragma unroll
                for (int j = 0; j < F; ++j) {
                    const uint64_t y = __shfl_up(x[j], d, kWave);
                    if (ln >= d) x[j] += y;
                }
            }
            if (ln == kWave - 1)
#pragma unroll
                for (int j = 0; j < F; ++j) wt[wv * F + j] = x[j];
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
                pre[j * NT + t] = run + before + x[j] - sg[j];
                run += total;
            }
            __syncthreads();   // pre complete before any lane searches it
            scanned = true;
        }
        for (int i = t; i < n; i += NT) {
            const uint64_t T = tgt[i];
            if (T < base || T - base >= Qc) continue;
            const uint64_t Tc = T - base;
            int lo = 0, hi = F * NT - 1;             // largest m with pre[m] <= Tc (pre[0] = 0)
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pre[mid] <= Tc) lo = mid; else hi = mid - 1;
            }
            const int j = lo / NT, o = lo - j * NT;
            float v[4];
            fetch(j, o, v);
            uint64_t acc = pre[lo];
            int e = 0;
            for (; e < 3; ++e) {
                acc += fixed_point(v[e], s);
                if (acc > Tc) break;
            }
            idrow[kb + i] = static_cast<int32_t>(c0 + (static_cast<int64_t>(j) * NT + o) * 4 + e);
        }
        __syncthreads();   // tgt is rewritten by the next batch
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
