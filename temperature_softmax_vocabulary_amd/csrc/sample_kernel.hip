// Inverse-CDF token draws from softmax rows: HIP kernel for gfx950.
//
// The pull-request page "fix(kernel): avoid nan in triton sampling softmax
// when a chunk starts with -inf" (FreeToken pull request 654) feeds the
// softmax into a token draw (scope paragraph) and requires every draw to be an
// allowed id (results table, sampling row). The draw rule used here is the
// inverse CDF on caller-supplied uniforms: for u clamped to [0, 1] (NaN -> 0)
// and the row's inclusive prefix sums C, the id is the smallest j with
// C[j] > u * C[V-1].
//
// Exactness: the prefix sums are formed in 64-bit fixed point. Each entry p > 0
// becomes q = rint(p * 2^s), where 2^s is a per-row power of two chosen from
// the row's float sum so that sum(q) < 2^62. Scaling by a power of two is
// exact, integer addition is associative, and an entry that is not > 0 gives
// q = 0; with Q[j] the integer prefix sums and T = min(floor(u * Q[V-1]),
// Q[V-1] - 1), the id is the smallest j with Q[j] > T. That j always has
// q[j] >= 1, so a masked (zero-probability) id can never be drawn, whatever
// the order in which lanes add. Rounding is <= 0.5 * 2^-s per entry, i.e.
// about 2^-62 of the row total.
//
// One workgroup per row, three sweeps over the row: float sum (scale), exact
// integer total, then a tile walk with an integer carry that resolves every
// target inside the tile that holds it.
#include "ts_device.h"
#include "ts_launch.h"

namespace tsk {

namespace {

constexpr int ST = 256;                 // lanes per workgroup
constexpr int SW = ST / kWave;
constexpr int STILE = ST * 4;           // columns per tile: 4 consecutive per lane
constexpr int KPL = 4;                  // targets held per lane per walk

template <bool VEC>
__device__ __forceinline__ void load4(const float* __restrict__ row, int64_t col, int64_t V, float (&v)[4]) {
    if constexpr (VEC) {
        f4 t = {0.0f, 0.0f, 0.0f, 0.0f};
        if (col < V) t = *reinterpret_cast<const f4*>(row + col);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (col + e < V) ? row[col + e] : 0.0f;
    }
}

// q = rint(p * 2^s) for p > 0, else 0 (NaN, zero and negative entries).
__device__ __forceinline__ uint64_t fixed_point(float p, int s) {
    if (!(p > 0.0f)) return 0;
    return static_cast<uint64_t>(rintf(ldexpf(p, s)));
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

template <bool VEC>
__global__ __launch_bounds__(ST) void ts_sample_rows(SampleArgs a) {
    __shared__ float redf[SW];
    __shared__ uint64_t wtot[SW];
    __shared__ uint64_t incl[ST];
    __shared__ uint64_t qtile[STILE];

    const int t = threadIdx.x;
    const int wv = t / kWave;
    const int ln = t & (kWave - 1);
    const int64_t row = blockIdx.x;
    const float* pr = a.probs + row * a.V;
    const float* ur = a.uniforms + row * a.K;
    int32_t* idr = a.out_ids + row * a.K;

    // sweep 1: float sum of the positive entries, to pick the scale
    float fs = 0.0f;
    for (int64_t c0 = 0; c0 < a.V; c0 += STILE) {
        float v[4];
        load4<VEC>(pr, c0 + 4 * t, a.V, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) fs += (v[e] > 0.0f) ? v[e] : 0.0f;
    }
    const float total = block_reduce<SumOp, SW>(fs, redf);
    if (!(total > 0.0f) || !(total < __builtin_huge_valf())) {
        for (int64_t k = t; k < a.K; k += ST) idr[k] = -1;
        return;
    }
    int ex = 0;
    frexpf(total, &ex);           // total < 2^ex
    const int s = 61 - ex;        // every p <= row total, so each q < 2^61 (1 + 2^-20)

    // sweep 2: exact integer total
    uint64_t qs = 0;
    for (int64_t c0 = 0; c0 < a.V; c0 += STILE) {
        float v[4];
        load4<VEC>(pr, c0 + 4 * t, a.V, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) qs += fixed_point(v[e], s);
    }
    qs = wave_sum_u64(qs);
    if (ln == 0) wtot[wv] = qs;
    __syncthreads();
    uint64_t qtotal = 0;
#pragma unroll
    for (int i = 0; i < SW; ++i) qtotal += wtot[i];
    __syncthreads();
    if (qtotal == 0) {            // every positive entry rounded to 0: cannot happen for p <= total
        for (int64_t k = t; k < a.K; k += ST) idr[k] = -1;
        return;
    }

    // sweep 3, once per group of ST * KPL targets: tile walk with integer carry
    for (int64_t kbase = 0; kbase < a.K; kbase += static_cast<int64_t>(ST) * KPL) {
        uint64_t tgt[KPL];
        bool mine[KPL];
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const int64_t k = kbase + t + static_cast<int64_t>(m) * ST;
            mine[m] = k < a.K;
            float u = mine[m] ? ur[k] : 0.0f;
            u = (u == u) ? fminf(fmaxf(u, 0.0f), 1.0f) : 0.0f;
            uint64_t T = static_cast<uint64_t>(floor(static_cast<double>(u) * static_cast<double>(qtotal)));
            tgt[m] = T < qtotal ? T : qtotal - 1;
        }
        uint64_t carry = 0;
        for (int64_t c0 = 0; c0 < a.V; c0 += STILE) {
            float v[4];
            load4<VEC>(pr, c0 + 4 * t, a.V, v);
            uint64_t q[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) q[e] = fixed_point(v[e], s);
            uint64_t x = q[0] + q[1] + q[2] + q[3];
            // inclusive scan across the wave, then across waves
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const uint64_t y = __shfl_up(x, d, kWave);
                if (ln >= d) x += y;
            }
            if (ln == kWave - 1) wtot[wv] = x;
#pragma unroll
            for (int e = 0; e < 4; ++e) qtile[4 * t + e] = q[e];
            __syncthreads();
            uint64_t before = 0, tile_total = 0;
#pragma unroll
            for (int i = 0; i < SW; ++i) {
                before += (i < wv) ? wtot[i] : 0;
                tile_total += wtot[i];
            }
            incl[t] = x + before;
            __syncthreads();
#pragma unroll
            for (int m = 0; m < KPL; ++m) {
                if (!mine[m] || tgt[m] < carry || tgt[m] - carry >= tile_total) continue;
                const uint64_t T = tgt[m] - carry;
                // smallest lane i with incl[i] > T (incl is non-decreasing)
                int lo = 0, hi = ST - 1;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (incl[mid] > T) hi = mid; else lo = mid + 1;
                }
                uint64_t acc = lo ? incl[lo - 1] : 0;
                int e = 0;
                for (; e < 3; ++e) {
                    acc += qtile[4 * lo + e];
                    if (acc > T) break;
                }
                idr[kbase + t + static_cast<int64_t>(m) * ST] = static_cast<int32_t>(c0 + 4 * lo + e);
            }
            carry += tile_total;
            __syncthreads();      // LDS is rewritten by the next tile
        }
    }
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, bool vec, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(a.B));
    if (vec) hipLaunchKernelGGL((ts_sample_rows<true>), grid, dim3(ST), 0, s, a);
    else hipLaunchKernelGGL((ts_sample_rows<false>), grid, dim3(ST), 0, s, a);
    return hipGetLastError();
}

}  // namespace tsk
