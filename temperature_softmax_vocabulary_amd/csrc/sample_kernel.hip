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
// Two kernels:
//  ts_sample_chunks: (row, chunk) items over a persistent grid, one read of the
//    probabilities. Each chunk's positive-entry float sum travels between the
//    row's workgroups through the tagged slots of ts_exchange.h; every
//    workgroup turns the sums into the row's integer chunk ranges, and the
//    chunk whose range holds a target resolves it in its own exact fixed point
//    (ts_sample_device.h). Used while a row has at most kSlotStride chunks.
//  ts_sample_rows: one workgroup per row, three sweeps over the row (float
//    sum for the scale, exact integer total, then a tile walk with an integer
//    carry). Any V. Its prefix sums are exact over the whole row: each entry
//    p > 0 becomes q = rint(p * 2^s) at one power-of-two scale per row with
//    sum(q) < 2^62, and the id is the smallest j whose integer prefix exceeds
//    T = min(floor(u * Q), Q - 1); that j always has q >= 1.
#include "ts_device.h"
#include "ts_exchange.h"
#include "ts_launch.h"
#include "ts_sample_device.h"

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
    const int s = scale_exponent(total);

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
            tgt[m] = target_of(mine[m] ? ur[k] : 0.0f, qtotal);
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


// ---------------------------------------------------------------------------
// chunked: one read of the probabilities
// ---------------------------------------------------------------------------
constexpr int CT = 256;
constexpr int CW = CT / kWave;

template <int F>
constexpr size_t sample_chunk_lds() {
    return resolve_lds_bytes<CT, F>();
}

template <int F, bool VEC>
__global__ __launch_bounds__(CT) void ts_sample_chunks(SampleArgs a) {
    extern __shared__ __align__(16) float dyn[];
    __shared__ float redf[CW];
    __shared__ ChunkRange row_range;
    constexpr int C = CT * 4 * F;
    const int lane = threadIdx.x;
    int64_t item = blockIdx.x;
    if (item >= a.items) return;
    // the next item's chunk (and the lane's uniform of its row) is loaded while
    // this one waits on its row
    float p[4 * F], np[4 * F];
    unsigned long long own_f = 0, next_f = 0;
    float u0 = 0.0f, nu0 = 0.0f;
    {
        const int64_t row = item / a.nch, c = item - row * a.nch;
        load_chunk<CT, F, VEC, true>(a.probs + row * a.V, c * C, a.V, p, 0.0f);
        if (lane < a.K) u0 = a.uniforms[row * a.K + lane];
        if (lane == 0) own_f = slot_load(a.fslots + row * kSlotStride + c);
    }
    for (; item < a.items; item += gridDim.x) {
        const int64_t row = item / a.nch;
        const int64_t c = item - row * a.nch;
        unsigned long long* fs = a.fslots + row * kSlotStride;
        const int64_t nitem = item + gridDim.x;
        if (nitem < a.items) {
            const int64_t nr = nitem / a.nch, nc = nitem - nr * a.nch;
            load_chunk<CT, F, VEC, true>(a.probs + nr * a.V, nc * C, a.V, np, 0.0f);
            if (lane < a.K) nu0 = a.uniforms[nr * a.K + lane];
            if (lane == 0) next_f = slot_load(a.fslots + nr * kSlotStride + nc);
        }
        // the chunk's weight: the float sum of its positive entries
        float fsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) fsum += (p[i] > 0.0f) ? p[i] : 0.0f;
        fsum = block_reduce<SumOp, CW>(fsum, redf);
        if (lane < kWave) {
            const unsigned long long tf = next_tag(own_f);
            publish(fs, c, a.nch, tf, __float_as_uint(fsum) & 0x7fffffffu);   // a sum of positives
            unsigned long long v[kSlotsPerLane];
            wait_row(fs, a.nch, tf, 0ull, v, a.spin_limit, a.err);
            float w[kSlotsPerLane];
#pragma unroll
            for (int j = 0; j < kSlotsPerLane; ++j) w[j] = __uint_as_float(static_cast<uint32_t>(v[j]));
            const ChunkRange r = chunk_range(w, c);
            if (lane == 0) row_range = r;
        }
        __syncthreads();
        const ChunkRange r = row_range;
        const float* urow = a.uniforms + row * a.K;
        int32_t* idrow = a.out_ids + row * a.K;
        if (r.total == 0) {   // no positive entry (or a sum that is not finite)
            if (c == 0)
                for (int64_t kk = lane; kk < a.K; kk += CT) idrow[kk] = -1;
        } else if (r.width > 0) {
            // the chunk's own scale: each entry <= fsum < 2^e, chunk total < 2^62
            const float* pr = a.probs + row * a.V;
            const int64_t c0 = c * C;
            const int64_t V = a.V;
            auto fetch = [=](int j, int o, float (&v)[4]) { load_group4<CT>(pr, c0, V, j, o, 0.0f, v); };
            resolve_chunk<CT, F>(p, reinterpret_cast<unsigned char*>(dyn), scale_exponent(fsum), r, c0, u0, urow,
                                 a.K, idrow, fetch);
        }
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) p[i] = np[i];
        own_f = next_f;
        u0 = nu0;
        __syncthreads();   // the row range and the resolve table are rewritten by the next item
    }
}

template <int F, bool VEC>
hipError_t sample_chunks_impl(const SampleArgs& a, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((ts_sample_chunks<F, VEC>), dim3(static_cast<uint32_t>(grid)), dim3(CT),
                       sample_chunk_lds<F>(), s, a);
    return hipGetLastError();
}

template <int F, bool VEC>
hipError_t sample_cap_impl(int64_t* cap) {
    int dev = 0, per_cu = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&ts_sample_chunks<F, VEC>),
                                                     CT, sample_chunk_lds<F>());
    if (e != hipSuccess) return e;
    *cap = static_cast<int64_t>(per_cu) * cus;
    return hipSuccess;
}

#define TS_SAMPLE_DISPATCH(IMPL, F, VEC, ...)                                                   \
    do {                                                                                        \
        switch (F) {                                                                            \
            case 4: return VEC ? IMPL<4, true>(__VA_ARGS__) : IMPL<4, false>(__VA_ARGS__);     \
            case 8: return VEC ? IMPL<8, true>(__VA_ARGS__) : IMPL<8, false>(__VA_ARGS__);     \
            default: return hipErrorInvalidValue;                                               \
        }                                                                                       \
    } while (0)

}  // namespace

hipError_t launch_sample_chunks(const SampleArgs& a, int F, bool vec, int64_t grid, hipStream_t s) {
    TS_SAMPLE_DISPATCH(sample_chunks_impl, F, vec, a, grid, s);
}

hipError_t sample_resident_capacity(int F, bool vec, int64_t* cap) {
    TS_SAMPLE_DISPATCH(sample_cap_impl, F, vec, cap);
}

hipError_t launch_sample_rows(const SampleArgs& a, bool vec, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(a.B));
    if (vec) hipLaunchKernelGGL((ts_sample_rows<true>), grid, dim3(ST), 0, s, a);
    else hipLaunchKernelGGL((ts_sample_rows<false>), grid, dim3(ST), 0, s, a);
    return hipGetLastError();
}

}  // namespace tsk
