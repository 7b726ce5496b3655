// Temperature softmax over the vocabulary: HIP kernels for gfx950.
//
// Method: the pull-request page "fix(kernel): avoid nan in triton sampling
// softmax when a chunk starts with -inf" (FreeToken pull request 654).
//  - Test paragraph: probs[b, :] = softmax(logits[b, :] / t[b]).
//  - Bug paragraph: the work is split by row and column chunk; each chunk
//    keeps a running max m and a sum of exponentials l relative to it, and a
//    finalize step combines the chunk partials with a global rescale.
//  - Fix paragraph: while a max is still -inf the shift is 0, so an all -inf
//    block adds 0, a fully masked chunk stores pl = 0, and its rescale term
//    0 * exp(-inf - gm) is 0 whenever the row has a finite logit.
//
// Three ways to split the work, all with the same per-element arithmetic:
//  split   : ts_split_partials writes (pm, pl) per (row, chunk); then
//            ts_split_finalize_write combines a row's partials and writes the
//            chunk's probs (finalize fused into the write; logits read twice).
//  fused   : one kernel; each workgroup keeps its chunk's exponentials in
//            registers, publishes (pm, pl) in the row's tagged slots, waits
//            for the row's other chunks, then writes (logits read once).
//  rowwise : one workgroup per row; the row sits in registers when it fits
//            (read once), else an online (m, l) sweep and a write sweep.
#include <map>
#include <mutex>

#include "ts_device.h"
#include "ts_exchange.h"
#include "ts_launch.h"

namespace tsk {

// Scratch of the allocation-free entry point (ts_softmax_noalloc): flags,
// fused-kernel slots, split partials, as ts_launch.h lays them out. Zero when
// the library loads, so every slot starts with tag 0 (the exchange needs only
// that a row's slots carry one tag between kernels, which every kernel keeps).
// Each GPU holds its own copy until the process ends. Host code uses the
// address static_scratch returns, never this name.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
    static std::mutex mu;
    static std::map<int, void*> addr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu);
    auto it = addr.find(dev);
    if (it == addr.end()) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        it = addr.emplace(dev, p).first;
    }
    *ptr = it->second;
    return hipSuccess;
}

namespace {

constexpr int NT = kChunkThreads;      // 256 lanes = 4 waves
constexpr int NW = NT / kWave;

__device__ __forceinline__ float2 load_partial(const float2* p) { return *p; }

__device__ __forceinline__ const uint32_t* mask_row(const SoftmaxArgs& a, int64_t row) {
    return a.allowed ? a.allowed + row * a.mwords : nullptr;
}

// ---------------------------------------------------------------------------
// split, kernel 1: one workgroup per (row, chunk) -> (pm, pl)
// ---------------------------------------------------------------------------
template <int F, bool VEC>
__global__ __launch_bounds__(NT) void ts_split_partials(SoftmaxArgs a) {
    __shared__ float red[NW];
    constexpr int C = NT * 4 * F;
    const int64_t item = blockIdx.x;
    const int64_t row = item / a.nch;
    const int64_t c = item - row * a.nch;
    const float k = exp2_scale(a.temps[row]);

    float x[4 * F];
    load_chunk<NT, F, VEC, false>(a.logits + row * a.V, c * C, a.V, x, kNegInf, mask_row(a, row));

    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < 4 * F; ++i) m = fmaxf(m, x[i]);
    const float pm = block_reduce<MaxOp, NW>(m, red);
    const float sh = guarded_shift(pm);
    float l = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * F; ++i) l += exp2_hw((x[i] - sh) * k);
    const float pl = block_reduce<SumOp, NW>(l, red);
    if (threadIdx.x == 0) a.part[item] = make_float2(pm, pl);
}

// Combine a row's partials: gm = max pm, gl = sum pl * exp2((pm - gm) k), with
// a fully masked chunk (pm = -inf, pl = 0) contributing exactly 0.
__device__ __forceinline__ void combine_row(const float2* __restrict__ part, int64_t nch, float k,
                                            float* red, float& gsh, float& r) {
    float m = kNegInf;
    for (int64_t i = threadIdx.x; i < nch; i += NT) m = fmaxf(m, load_partial(part + i).x);
    const float gm = block_reduce<MaxOp, NW>(m, red);
    gsh = guarded_shift(gm);
    float l = 0.0f;
    for (int64_t i = threadIdx.x; i < nch; i += NT) {
        const float2 p = load_partial(part + i);
        l += masked_term(p.x, p.y * exp2_hw((p.x - gsh) * k));
    }
    const float gl = block_reduce<SumOp, NW>(l, red);
    r = 1.0f / gl;
}

// ---------------------------------------------------------------------------
// split, rows of more than kSplitRowCombineMin chunks: one workgroup per row
// combines its partials once into (shift, 1 / sum) for the write pass
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void ts_split_row_combine(SoftmaxArgs a) {
    __shared__ float red[NW];
    const int64_t row = blockIdx.x;
    float gsh, r;
    combine_row(a.part + row * a.nch, a.nch, exp2_scale(a.temps[row]), red, gsh, r);
    if (threadIdx.x == 0) a.part[a.items + row] = make_float2(gsh, r);
}

// ---------------------------------------------------------------------------
// split, kernel 2: finalize fused into the write of the probs (ROWSTAT: the
// row's (shift, 1 / sum) from ts_split_row_combine; else combined here)
// ---------------------------------------------------------------------------
template <int F, bool VEC, bool ROWSTAT>
__global__ __launch_bounds__(NT) void ts_split_finalize_write(SoftmaxArgs a) {
    __shared__ float red[NW];
    constexpr int C = NT * 4 * F;
    const int64_t item = blockIdx.x;
    const int64_t row = item / a.nch;
    const int64_t c = item - row * a.nch;
    const float k = exp2_scale(a.temps[row]);

    float x[4 * F];
    load_chunk<NT, F, VEC, true>(a.logits + row * a.V, c * C, a.V, x, kNegInf, mask_row(a, row));   // last use of logits

    float gsh, r;
    if constexpr (ROWSTAT) {
        const float2 st = a.part[a.items + row];
        gsh = st.x;
        r = st.y;
    } else {
        combine_row(a.part + row * a.nch, a.nch, k, red, gsh, r);
    }
#pragma unroll
    for (int i = 0; i < 4 * F; ++i) x[i] = exp2_hw((x[i] - gsh) * k) * r;
    store_chunk<NT, F, VEC, true>(a.out + row * a.V, c * C, a.V, x);
}

// The payload a chunk publishes: pm in the low word, pl in the high word. pl
// >= 0; clearing its sign bit keeps a NaN (possible only outside the method's
// domain) from reaching the tag bit.
__device__ __forceinline__ unsigned long long pack_partial(float pm, float pl) {
    return (static_cast<unsigned long long>(__float_as_uint(pl) & 0x7fffffffu) << 32) | __float_as_uint(pm);
}

// One column of a chunk, as the chunk's loads and the allowed-id mask give it
// to its lane: base = the chunk's first column, mbase = the mask word holding
// it (or null), left = columns from base to the row's end, off = the column's
// offset from base (-inf at or past the row's end, or where not allowed).
__device__ __forceinline__ float chunk_value(const float* base, const uint32_t* mbase, int64_t left, uint32_t off) {
    float v = kNegInf;
    if (off < left) {
        v = base[off];
        if (mbase && !((mbase[off >> 5] >> (off & 31)) & 1u)) v = kNegInf;
    }
    return v;
}

// Chunk c's partial (pm, pl), formed by one wave alone and bit for bit as the
// chunk's own workgroup forms it: the wave takes the parts of the workgroup's
// NW waves in turn (lane l as lane 64 w + l: the same values, summed in the
// same order), reduces each part with the same wave reduction, and combines
// the NW sums in block_reduce's order. One column at a time and two reads of
// the chunk (max, then sum), to keep its registers few: it runs only when a
// wait ran out, beside the registers that hold this chunk and the next.
template <int F>
__device__ __forceinline__ unsigned long long chunk_partial_by_wave(const SoftmaxArgs& a, int64_t row, int64_t c,
                                                                    float k) {
    constexpr int C = NT * 4 * F;
    const int l = threadIdx.x & (kWave - 1);
    const int64_t c0 = c * C;
    const float* base = a.logits + row * a.V + c0;
    const uint32_t* mbase = a.allowed ? a.allowed + row * a.mwords + (c0 >> 5) : nullptr;
    const int64_t left = a.V - c0;
    // column of value i (group i / 4, element i % 4) of lane 64 w + l
#define TS_LANE_COL(w, i) static_cast<uint32_t>((((i) >> 2) * NT + (w) * kWave + l) * 4 + ((i) & 3))
    float m = kNegInf;
#pragma unroll 1
    for (int w = 0; w < NW; ++w) {
#pragma unroll 1
        for (int i = 0; i < 4 * F; ++i) m = fmaxf(m, chunk_value(base, mbase, left, TS_LANE_COL(w, i)));
    }
    const float pm = wave_reduce<MaxOp>(m);
    const float sh = guarded_shift(pm);
    float pl = 0.0f;
#pragma unroll 1
    for (int w = 0; w < NW; ++w) {
        float s = 0.0f;
#pragma unroll 1
        for (int i = 0; i < 4 * F; ++i) s += exp2_hw((chunk_value(base, mbase, left, TS_LANE_COL(w, i)) - sh) * k);
        const float r = wave_reduce<SumOp>(s);
        pl = w == 0 ? r : pl + r;
    }
#undef TS_LANE_COL
    return pack_partial(pm, pl);
}

// Wave 0, after a wait that ran out: the chunks whose slots were still
// unpublished (bit j of `missing` on lane l: chunk l + 64 j) get their partial
// from chunk_partial_by_wave, so the row combines exactly what the exchange
// would have given it. Each slot is read once more after that chunk's loads
// have completed, and a partial published meanwhile is taken instead: in place,
// its owner may since have written its probabilities over the logits just read
// (it publishes before it writes, and it writes only after a poll of its own).
// v is parked in `park` (LDS) meanwhile, to keep registers free.
template <int F>
__device__ __forceinline__ void recover_missing(const SoftmaxArgs& a, int64_t row, float k,
                                                const unsigned long long* rs, unsigned long long tag, uint32_t missing,
                                                unsigned long long (&v)[kSlotsPerLane], unsigned long long* park) {
    const int l = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int j = 0; j < kSlotsPerLane; ++j) park[l + j * kWave] = v[j];
#pragma unroll 1
    for (int j = 0; j < kSlotsPerLane; ++j) {
        unsigned long long lanes = __ballot((missing >> j) & 1u);
        while (lanes) {
            const int src = __ffsll(lanes) - 1;
            lanes &= lanes - 1;
            const int64_t c = src + static_cast<int64_t>(j) * kWave;
            unsigned long long p = chunk_partial_by_wave<F>(a, row, c, k);
            // (the loads above are complete: their values are in p; the fence
            // keeps the slot's read from moving ahead of them)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            const unsigned long long x = slot_load(rs + c);
            if ((x & kTagBit) == tag) p = x & ~kTagBit;
            if (l == src) park[c] = p;
        }
    }
#pragma unroll
    for (int j = 0; j < kSlotsPerLane; ++j) v[j] = park[l + j * kWave];
}

// ---------------------------------------------------------------------------
// fused: one read of the logits, one kernel.
//
// Work items are (row, chunk) pairs, item = row * nch + chunk. Workgroup w
// handles items w, w + gridDim.x, ... in order, and issues the loads of its
// next item before it waits on the current row, so a workgroup's waits and
// stores overlap its next reads. The chunk partials (pm, pl) travel through
// the tagged slots of ts_exchange.h (no fence, no contended read-modify-write:
// either costs microseconds per workgroup on a multi-XCD part). The host
// launches no more workgroups than the device holds at once and at least nch.
// Should a wait run out all the same (the device shared with work that keeps
// some of a row's workgroups from running), recover_missing forms the missing
// partials from the logits, so the result never depends on the wait.
//
// MODE kFusedProbs writes the probabilities; kFusedProbsSums also writes the
// sums of the probabilities per group of 4096 columns (one share per wave) and
// per block of 64, for a token draw that follows (draw_kernels.hip). They are
// formed from the exponentials while the kernel waits on its row, then
// multiplied by the chunk's scale: within float rounding of the sums of the
// written probabilities.
// ---------------------------------------------------------------------------
template <int F, int MODE>
struct FusedOcc {
    // registers hold the current and the next chunk (8 F floats per lane)
    static constexpr int probs = F <= 2 ? 8 : (F == 4 ? 6 : (F == 8 ? 4 : 2));
    // the draw sums need a few more: at 4096 columns one wave per SIMD less
    // keeps them in registers (the sums run at 4096 only for small calls,
    // B V <= 2^21, whose grid is far below the device's capacity either way)
    static constexpr int waves_per_eu = MODE != kFusedProbsSums ? probs : (F == 4 ? 5 : probs);
};

template <int F, bool VEC, int MODE>
__global__ __launch_bounds__(NT, (FusedOcc<F, MODE>::waves_per_eu)) void ts_fused(SoftmaxArgs a) {
    static_assert(MODE != kFusedProbsSums || F % 4 == 0, "draw sums need whole 4096-column groups");
    __shared__ float red[NW];
    __shared__ float chunk_scale;
    __shared__ unsigned long long park[kSlotStride];   // a row's partials, when a wait ran out
    __shared__ float bsum[MODE == kFusedProbsSums ? F : 1][16];   // draw sums: per block of a chunk
    constexpr int C = NT * 4 * F;
    const int lane = threadIdx.x;
    int64_t item = blockIdx.x;
    if (item >= a.items) return;

    float x[4 * F], nx[4 * F];
    // mask words of the current and the next chunk: applied only when the
    // chunk's values are used, so the prefetch below never waits on its loads
    uint32_t mw[2] = {0u, 0u}, nmw[2] = {0u, 0u};
    // lane 0: old high word of the item's own slot (and of the next item's)
    uint32_t own = 0, next_own = 0;
    {
        const int64_t row = item / a.nch, c = item - row * a.nch;
        load_chunk<NT, F, VEC, true>(a.logits + row * a.V, c * C, a.V, x, kNegInf);
        if (a.allowed) load_mask_words<NT, F>(mask_row(a, row), c * C, a.V, mw);
        if (lane == 0) own = slot_load_hi(a.slots + row * kSlotStride + c);
    }
    for (; item < a.items; item += gridDim.x) {
        const int64_t row = item / a.nch;
        const int64_t c = item - row * a.nch;
        const float k = exp2_scale(a.temps[row]);
        unsigned long long* rs = a.slots + row * kSlotStride;
        if (a.allowed) apply_mask_words<NT, F>(c * C, a.V, mw, x);

        // chunk partial: pm = max, pl = sum exp2((x - shift) k); x keeps the exponentials
        float m = kNegInf;
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) m = fmaxf(m, x[i]);
        const float pm = block_reduce<MaxOp, NW>(m, red);
        const float sh = guarded_shift(pm);
        float l = 0.0f;
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) {
            x[i] = exp2_hw((x[i] - sh) * k);
            l += x[i];
        }
        const float pl = block_reduce<SumOp, NW>(l, red);

        const unsigned long long tag = next_tag(own);   // wave-uniform, all lanes
        if (lane < kWave)
            publish(rs, c, a.nch, tag, pack_partial(pm, pl));

        // prefetch the next item (a later row: gridDim.x >= nch)
        const int64_t nitem = item + gridDim.x;
        if (nitem < a.items) {
            const int64_t nr = nitem / a.nch, nc = nitem - nr * a.nch;
            load_chunk<NT, F, VEC, true>(a.logits + nr * a.V, nc * C, a.V, nx, kNegInf);
            if (a.allowed) load_mask_words<NT, F>(mask_row(a, nr), nc * C, a.V, nmw);
            if (lane == 0) next_own = slot_load_hi(a.slots + nr * kSlotStride + nc);
        }

        // draw sums: block sums of the exponentials, formed while the row's
        // other chunks arrive and parked in LDS; after the wait they are scaled
        // to probabilities and written (with each wave's share of each group)
        if constexpr (MODE == kFusedProbsSums) {
#pragma unroll
            for (int j = 0; j < F; ++j) {
                const float b = row16_reduce<SumOp>((x[4 * j] + x[4 * j + 1]) + (x[4 * j + 2] + x[4 * j + 3]));
                if ((lane & 15) == 15) bsum[j][lane >> 4] = b;
            }
        }

        // wave 0 waits for the row's partials and combines them: gm = max pm,
        // gl = sum pl exp2((pm - gm) k), a fully masked chunk adding exactly 0
        if (lane < kWave) {
            unsigned long long v[kSlotsPerLane];
            const unsigned long long absent = __float_as_uint(kNegInf);   // pm = -inf, pl = 0
            const uint32_t missing = wait_row(rs, a.nch, tag, absent, v, a.spin_limit, a.err);
            if (__ballot(missing != 0u)) recover_missing<F>(a, row, k, rs, tag, missing, v, park);
            float mm = kNegInf;
#pragma unroll
            for (int j = 0; j < kSlotsPerLane; ++j) mm = fmaxf(mm, __uint_as_float(static_cast<uint32_t>(v[j])));
            const float gsh = guarded_shift(wave_reduce<MaxOp>(mm));
            float ll = 0.0f;
#pragma unroll
            for (int j = 0; j < kSlotsPerLane; ++j) {
                const float vm = __uint_as_float(static_cast<uint32_t>(v[j]));
                const float vl = __uint_as_float(static_cast<uint32_t>(v[j] >> 32));
                ll += masked_term(vm, vl * exp2_hw((vm - gsh) * k));
            }
            const float gl = wave_reduce<SumOp>(ll);
            if (lane == 0) chunk_scale = masked_term(pm, exp2_hw((pm - gsh) * k) * (1.0f / gl));
        }
        __syncthreads();
        const float scale = chunk_scale;
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) x[i] *= scale;    // the probabilities
        store_chunk<NT, F, VEC, true>(a.out + row * a.V, c * C, a.V, x);
        if constexpr (MODE == kFusedProbsSums) {
            // bsum is complete: the barrier after the wait follows every write.
            // Block (j, r) of the chunk is block 16 j + r of the row counted from
            // the chunk's first group, so lane t < 16 F writes block t; lane
            // t < 4 NG writes wave t % 4's share of group t / 4, the sum of its
            // blocks in that wave's 4 rows of lanes. (Offsets from a uniform
            // base: no per-lane 64-bit index is kept across the loop.)
            constexpr int NG = F / 4;
            const int64_t g0 = c * NG;   // the chunk's first group
            const int64_t gbase = row * a.ngroups + g0;
            if (lane < 16 * F && g0 + (lane >> 6) < a.ngroups)
                a.bpart[gbase * kBlocksPerGroup + lane] = (&bsum[0][0])[lane] * scale;
            if (lane < NG * NW) {
                const int d = lane / NW, w = lane % NW;
                if (g0 + d < a.ngroups) {
                    float h = 0.0f;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        h += (bsum[4 * d + jj][4 * w] + bsum[4 * d + jj][4 * w + 1]) +
                             (bsum[4 * d + jj][4 * w + 2] + bsum[4 * d + jj][4 * w + 3]);
                    reinterpret_cast<float*>(a.gpart + gbase)[lane] = h * scale;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4 * F; ++i) x[i] = nx[i];
        mw[0] = nmw[0];
        mw[1] = nmw[1];
        own = next_own;
        __syncthreads();   // chunk_scale (and the draw sums) are rewritten by the next item
    }
}

// ---------------------------------------------------------------------------
// rowwise, resident: one workgroup of RT lanes holds the whole row (V <= C).
// ---------------------------------------------------------------------------
template <int RT, int F, bool VEC>
__global__ __launch_bounds__(RT) void ts_rowwise_resident(SoftmaxArgs a) {
    constexpr int RW = RT / kWave;
    __shared__ float red[RW];
    const int64_t row = blockIdx.x;
    const float k = exp2_scale(a.temps[row]);
    float x[4 * F];
    load_chunk<RT, F, VEC, true>(a.logits + row * a.V, 0, a.V, x, kNegInf, mask_row(a, row));
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < 4 * F; ++i) m = fmaxf(m, x[i]);
    const float gsh = guarded_shift(block_reduce<MaxOp, RW>(m, red));
    float l = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * F; ++i) {
        x[i] = exp2_hw((x[i] - gsh) * k);
        l += x[i];
    }
    const float r = 1.0f / block_reduce<SumOp, RW>(l, red);
#pragma unroll
    for (int i = 0; i < 4 * F; ++i) x[i] *= r;
    store_chunk<RT, F, VEC, true>(a.out + row * a.V, 0, a.V, x);
}

// ---------------------------------------------------------------------------
// rowwise, streaming: online (m, l) per lane over the row, a workgroup
// combine, then a write sweep. Tile = RT lanes x U float4.
// ---------------------------------------------------------------------------
template <int RT, bool VEC>
__global__ __launch_bounds__(RT) void ts_rowwise_stream(SoftmaxArgs a) {
    constexpr int RW = RT / kWave;
    constexpr int U = 4;
    constexpr int TILE = RT * 4 * U;
    __shared__ float red[RW];
    const int64_t row = blockIdx.x;
    const float k = exp2_scale(a.temps[row]);
    const float* xr = a.logits + row * a.V;
    float* yr = a.out + row * a.V;
    const uint32_t* mrow = mask_row(a, row);

    float m = kNegInf, l = 0.0f;
    for (int64_t c0 = 0; c0 < a.V; c0 += TILE) {
        float x[4 * U];
        load_chunk<RT, U, VEC, false>(xr, c0, a.V, x, kNegInf, mrow);
        float bm = kNegInf;
#pragma unroll
        for (int i = 0; i < 4 * U; ++i) bm = fmaxf(bm, x[i]);
        const float nm = fmaxf(m, bm);
        const float sh = guarded_shift(nm);
        // m = -inf gives exp2(-inf) = 0 with l = 0; sh is always finite.
        float s = l * exp2_hw((m - sh) * k);
#pragma unroll
        for (int i = 0; i < 4 * U; ++i) s += exp2_hw((x[i] - sh) * k);
        l = s;
        m = nm;
    }
    const float gsh = guarded_shift(block_reduce<MaxOp, RW>(m, red));
    const float mine = masked_term(m, l * exp2_hw((m - gsh) * k));
    const float r = 1.0f / block_reduce<SumOp, RW>(mine, red);
    for (int64_t c0 = 0; c0 < a.V; c0 += TILE) {
        float x[4 * U];
        load_chunk<RT, U, VEC, true>(xr, c0, a.V, x, kNegInf, mrow);
#pragma unroll
        for (int i = 0; i < 4 * U; ++i) x[i] = exp2_hw((x[i] - gsh) * k) * r;
        store_chunk<RT, U, VEC, true>(yr, c0, a.V, x);
    }
}

template <int F, bool VEC>
hipError_t split_impl(const SoftmaxArgs& a, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(a.items));
    hipLaunchKernelGGL((ts_split_partials<F, VEC>), grid, dim3(NT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.nch > kSplitRowCombineMin) {
        hipLaunchKernelGGL(ts_split_row_combine, dim3(static_cast<uint32_t>(a.B)), dim3(NT), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ts_split_finalize_write<F, VEC, true>), grid, dim3(NT), 0, s, a);
    } else {
        hipLaunchKernelGGL((ts_split_finalize_write<F, VEC, false>), grid, dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

template <int F, bool VEC>
hipError_t fused_impl(const SoftmaxArgs& a, int mode, int64_t grid, hipStream_t s) {
    const dim3 g(static_cast<uint32_t>(grid));
    if (mode == kFusedProbs) {
        hipLaunchKernelGGL((ts_fused<F, VEC, kFusedProbs>), g, dim3(NT), 0, s, a);
    } else if constexpr (F % 4 == 0) {
        hipLaunchKernelGGL((ts_fused<F, VEC, kFusedProbsSums>), g, dim3(NT), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int F, bool VEC>
hipError_t fused_cap_impl(int mode, int64_t* cap) {
    int dev = 0, per_cu = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const void* fn = reinterpret_cast<const void*>(&ts_fused<F, VEC, kFusedProbs>);
    if (mode != kFusedProbs) {
        if constexpr (F % 4 == 0) fn = reinterpret_cast<const void*>(&ts_fused<F, VEC, kFusedProbsSums>);
        else return hipErrorInvalidValue;
    }
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, 0);
    if (e != hipSuccess) return e;
    *cap = static_cast<int64_t>(per_cu) * cus;
    return hipSuccess;
}

#define TS_DISPATCH_F(IMPL, F, VEC, ...)                                       \
    do {                                                                       \
        switch (F) {                                                           \
            case 1: return VEC ? IMPL<1, true>(__VA_ARGS__) : IMPL<1, false>(__VA_ARGS__);   \
            case 2: return VEC ? IMPL<2, true>(__VA_ARGS__) : IMPL<2, false>(__VA_ARGS__);   \
            case 4: return VEC ? IMPL<4, true>(__VA_ARGS__) : IMPL<4, false>(__VA_ARGS__);   \
            case 8: return VEC ? IMPL<8, true>(__VA_ARGS__) : IMPL<8, false>(__VA_ARGS__);   \
            case 16: return VEC ? IMPL<16, true>(__VA_ARGS__) : IMPL<16, false>(__VA_ARGS__); \
            default: return hipErrorInvalidValue;                              \
        }                                                                      \
    } while (0)

}  // namespace

hipError_t launch_split(const SoftmaxArgs& a, int F, bool vec, hipStream_t s) {
    TS_DISPATCH_F(split_impl, F, vec, a, s);
}

hipError_t launch_fused(const SoftmaxArgs& a, int F, bool vec, int mode, int64_t grid, hipStream_t s) {
    TS_DISPATCH_F(fused_impl, F, vec, a, mode, grid, s);
}

hipError_t fused_resident_capacity(int F, bool vec, int mode, int64_t* cap) {
    TS_DISPATCH_F(fused_cap_impl, F, vec, mode, cap);
}

hipError_t launch_rowwise(const SoftmaxArgs& a, bool vec, hipStream_t s) {
    constexpr int RT = kRowwiseThreads;
    const dim3 grid(static_cast<uint32_t>(a.B));
    if (a.V <= RT * 4 * 1) {
        if (vec) hipLaunchKernelGGL((ts_rowwise_resident<RT, 1, true>), grid, dim3(RT), 0, s, a);
        else hipLaunchKernelGGL((ts_rowwise_resident<RT, 1, false>), grid, dim3(RT), 0, s, a);
    } else if (a.V <= RT * 4 * 2) {
        if (vec) hipLaunchKernelGGL((ts_rowwise_resident<RT, 2, true>), grid, dim3(RT), 0, s, a);
        else hipLaunchKernelGGL((ts_rowwise_resident<RT, 2, false>), grid, dim3(RT), 0, s, a);
    } else if (a.V <= RT * 4 * 4) {
        if (vec) hipLaunchKernelGGL((ts_rowwise_resident<RT, 4, true>), grid, dim3(RT), 0, s, a);
        else hipLaunchKernelGGL((ts_rowwise_resident<RT, 4, false>), grid, dim3(RT), 0, s, a);
    } else if (a.V <= kRowwiseRegisterMaxV) {
        if (vec) hipLaunchKernelGGL((ts_rowwise_resident<RT, 8, true>), grid, dim3(RT), 0, s, a);
        else hipLaunchKernelGGL((ts_rowwise_resident<RT, 8, false>), grid, dim3(RT), 0, s, a);
    } else {
        if (vec) hipLaunchKernelGGL((ts_rowwise_stream<RT, true>), grid, dim3(RT), 0, s, a);
        else hipLaunchKernelGGL((ts_rowwise_stream<RT, false>), grid, dim3(RT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace tsk
