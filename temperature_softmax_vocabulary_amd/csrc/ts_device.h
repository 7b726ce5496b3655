// Device-side building blocks shared by the tsoftmax kernels (gfx950, wave64).
//
// Notation follows the pull-request page "fix(kernel): avoid nan in triton
// sampling softmax when a chunk starts with -inf" (FreeToken pull request 654,
// bug and fix paragraphs): m is a running max, l a sum of exponentials taken
// relative to it, (pm, pl) a chunk's partial, gm the row's global max.
//
// The exponentials are evaluated as exp2((x - shift) * k) with k = log2(e) / T:
// subtracting the shift in the raw-logit domain keeps the exponent's rounding
// error proportional to |x - shift|, and exp2 maps to one v_exp_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ts_launch.h"   // kLd*: how a one-shot kernel loads a chunk

namespace tsk {

typedef float f4 __attribute__((ext_vector_type(4)));
// A float4 at a 4-byte aligned address: gfx950 serves one unaligned 16-byte
// global load or store for it (loads at full speed, stores within a few per
// cent of aligned ones, measured on MI355X).
typedef float f4u __attribute__((ext_vector_type(4))) __attribute__((aligned(4)));

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_inff();
constexpr double kLog2eD = 1.4426950408889634073599246810019;

// k = log2(e) / T, formed in double and rounded once to float. A temperature
// so small (denormal) that k would overflow takes the largest float instead:
// (x - max) k is then 0 at the row's max and -inf or far below -126 elsewhere,
// the one-hot limit of the softmax, where an infinite k would give 0 * inf =
// NaN at the max. Every normal temperature is unaffected.
__device__ __forceinline__ float exp2_scale(float T) {
    constexpr double kFltMax = 3.4028234663852886e38;
    const double k = kLog2eD / static_cast<double>(T);
    return static_cast<float>(k < kFltMax ? k : kFltMax);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// The fix (fix paragraph): while a max is still -inf the shift is 0, so an all
// -inf block contributes exp2(-inf) = 0 instead of exp2(-inf - -inf) = NaN.
// For a finite max this is the plain max: a pure select, no change to the
// arithmetic of rows without -inf. A library built with TS_NO_INF_GUARD drops
// the selects (the arithmetic before the fix); it exists only so that tests
// can show both that finite rows are bitwise unchanged by the guard (A/B list
// of the page) and that masked chunk starts give NaN without it (bug paragraph).
#ifdef TS_NO_INF_GUARD
constexpr bool kInfGuard = false;
#else
constexpr bool kInfGuard = true;
#endif

__device__ __forceinline__ float guarded_shift(float m) { return (kInfGuard && m == kNegInf) ? 0.0f : m; }

// A chunk (or lane) whose max is -inf adds exactly 0 to a rescaled sum, even
// when the row's own max is -inf too; `term` is the rescaled value otherwise.
__device__ __forceinline__ float masked_term(float m, float term) {
    return (kInfGuard && m == kNegInf) ? 0.0f : term;
}

// ---------------------------------------------------------------------------
// Wave64 reductions with DPP. Steps: two quad permutes (sum of 4 lanes), half
// row mirror (8), row mirror (16), then row_bcast15 and row_bcast31 fold the
// four rows of 16 into lane 63, which readlane returns to every lane.
// Must be called with all 64 lanes active.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_or(float v, float fill) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL,
                                                      ROW_MASK, 0xF, false));
}

struct MaxOp {
    static constexpr float identity = kNegInf;
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumOp {
    static constexpr float identity = 0.0f;
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

template <class Op>
__device__ __forceinline__ float wave_reduce(float v) {
    Op op;
    v = op(v, dpp_or<0xB1>(v, Op::identity));          // quad_perm [1,0,3,2]
    v = op(v, dpp_or<0x4E>(v, Op::identity));          // quad_perm [2,3,0,1]
    v = op(v, dpp_or<0x141>(v, Op::identity));         // row_half_mirror
    v = op(v, dpp_or<0x140>(v, Op::identity));         // row_mirror
    v = op(v, dpp_or<0x142, 0xA>(v, Op::identity));    // row_bcast15 -> rows 1, 3
    v = op(v, dpp_or<0x143, 0xC>(v, Op::identity));    // row_bcast31 -> rows 2, 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Reduction over each row of 16 lanes (lanes 16 r .. 16 r + 15), returned to
// all 16 lanes of the row: the first four steps of wave_reduce.
template <class Op>
__device__ __forceinline__ float row16_reduce(float v) {
    Op op;
    v = op(v, dpp_or<0xB1>(v, Op::identity));          // quad_perm [1,0,3,2]
    v = op(v, dpp_or<0x4E>(v, Op::identity));          // quad_perm [2,3,0,1]
    v = op(v, dpp_or<0x141>(v, Op::identity));         // row_half_mirror
    v = op(v, dpp_or<0x140>(v, Op::identity));         // row_mirror
    return v;
}

// Workgroup reduction: wave64 DPP reduce, then a fixed-order combine of the
// NW wave results through LDS. The order never depends on timing, so results
// are bitwise reproducible. `lds` holds NW floats; the trailing barrier lets
// the caller reuse it immediately.
template <class Op, int NW>
__device__ __forceinline__ float block_reduce(float v, float* lds) {
    v = wave_reduce<Op>(v);
    if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
    __syncthreads();
    Op op;
    float r = lds[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r = op(r, lds[i]);
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------------------
// Chunk access. A chunk is C = NT * 4 * F consecutive columns of one row, in F
// groups of NT * 4 columns. Lane t of the workgroup owns the 4 consecutive
// columns c0 + (j * NT + t) * 4 + e, e in [0, 4), of every group j, held in
// x[4 j + e]; within a group, lane order is column order. One float4 load per
// group, so each wave64 load instruction covers 1 KiB of contiguous memory:
// aligned (VEC: a 16-byte aligned row start and V % 4 == 0) or unaligned (any
// 4-byte aligned row, e.g. an odd V), where the row's last float4, when V % 4
// != 0, is partial and is read element by element. Columns at or past V read
// as `fill` (-inf for logits: they add nothing to a max or to a sum of
// exponentials).
// ---------------------------------------------------------------------------
// allowed-id bitmask of one row: bit (j % 32) of word j / 32, 1 = allowed. A
// lane's 4 columns of a group share one word (4 divides 32), so the mask costs
// one 4-byte load per group.
__device__ __forceinline__ void apply_allowed(const uint32_t* __restrict__ mrow, int64_t col, float (&v)[4]) {
    const uint32_t bits = mrow[col >> 5] >> (col & 31);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (!((bits >> e) & 1u)) v[e] = kNegInf;
}

// The mask words of a whole chunk. Lane t = 64 w + l of the workgroup needs,
// for group j, word (j NT + t) / 8 = j NT/8 + 8 w + l/8 of the chunk's words:
// per wave, 8 consecutive words per group. With at most 8 groups, lane l loads
// the word of group l / 8 at index l % 8 (one word per lane covers every group
// of the wave); with up to 16, the words of groups 2 (l / 8) and 2 (l / 8) + 1.
// A group's word is thus always in the same register of another lane of the
// same wave, fetched by one cross-lane read (ds_bpermute) when the mask is
// applied. The loads carry no branch (the index is clamped to the row's last
// word), so they stay in flight with the data loads until the values are used.
template <int F>
constexpr int kMaskWordsPerLane = F <= 8 ? 1 : 2;

template <int NT, int F>
__device__ __forceinline__ void load_mask_words(const uint32_t* __restrict__ mrow, int64_t c0, int64_t V,
                                                uint32_t (&mw)[2]) {
    static_assert(F <= 16, "two words per lane cover at most 16 groups");
    constexpr int MW = kMaskWordsPerLane<F>;
    const int l = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    // a uniform base and 32-bit lane offsets (a row has at most 2^26 words)
    const uint32_t* __restrict__ base = mrow + (c0 >> 5);
    const uint32_t last = static_cast<uint32_t>(((V - 1) >> 5) - (c0 >> 5));
    mw[1] = 0u;
#pragma unroll
    for (int h = 0; h < MW; ++h) {
        // (with fewer than 8 groups, the lanes past them repeat the last group's
        // words, so they add no memory requests)
        const int j = MW == 1 ? ((l >> 3) < F ? (l >> 3) : F - 1) : MW * (l >> 3) + h;
        const uint32_t off = static_cast<uint32_t>(j * (NT / 8) + 8 * w + (l & 7));
        mw[h] = base[off < last ? off : last];
    }
}

// x[4 j + e] = -inf where the id is not allowed (bits past V count as allowed:
// those columns already hold the fill value).
template <int NT, int F>
__device__ __forceinline__ void apply_mask_words(int64_t c0, int64_t V, const uint32_t (&mw)[2],
                                                 float (&x)[4 * F]) {
    constexpr int MW = kMaskWordsPerLane<F>;
    const int t = threadIdx.x, l = t & (kWave - 1);
#pragma unroll
    for (int j = 0; j < F; ++j) {
        const uint32_t word = static_cast<uint32_t>(
            __shfl(static_cast<int>(mw[j % MW]), (j / MW) * 8 + (l >> 3), kWave));
        const int64_t col = c0 + (static_cast<int64_t>(j) * NT + t) * 4;
        const uint32_t bits = (col < V) ? (word >> (col & 31)) : 0xFu;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (!((bits >> e) & 1u)) x[4 * j + e] = kNegInf;
    }
}

// Columns at or past V take `fill` (a separate step, so that a prefetch can
// put it off until the values are used: replacing a value waits for its load).
template <int NT, int F>
__device__ __forceinline__ void fill_past_end(int64_t c0, int64_t V, float (&x)[4 * F], float fill) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < F; ++j) {
        const int64_t col = c0 + (static_cast<int64_t>(j) * NT + t) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (col + e >= V) x[4 * j + e] = fill;
    }
}

// Issues the chunk's loads: every one before any value is used, none under a
// branch (a branch around a load makes the compiler wait for it at the join).
// Addresses are the chunk's start (uniform) plus a 32-bit lane offset.
//  kLdAligned: a lane past V reads the chunk's first float4 instead, which
//    always exists, and holds garbage until fill_past_end replaces it.
//  kLdUnaligned (V >= 4): a float4 that is not wholly inside the row is read
//    from the row's last 4 columns instead (the float4 ending at V, which may
//    start in the chunk before); shift_tail_group then moves the lane's own
//    columns into place, and fill_past_end replaces the rest.
//  kLdScalar: each column alone, at the chunk's first column when past V.
template <int NT, int F, int LD, bool NT_LOAD>
__device__ __forceinline__ void issue_chunk_loads(const float* __restrict__ row, int64_t c0, int64_t V,
                                                  float (&x)[4 * F]) {
    const int t = threadIdx.x;
    const float* __restrict__ base = row + c0;
    const int64_t left = V - c0;   // columns from the chunk's start to the row's end (> 0)
    if constexpr (LD == kLdAligned) {
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const uint32_t off = static_cast<uint32_t>((j * NT + t) * 4);
            const f4* p = reinterpret_cast<const f4*>(base + (off < left ? off : 0u));
            f4 v;
            if constexpr (NT_LOAD) v = __builtin_nontemporal_load(p);
            else v = *p;
            x[4 * j + 0] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
        }
    } else if constexpr (LD == kLdUnaligned) {
        const int64_t last = left - 4;   // start of the row's last 4 columns, from c0 (>= -c0: V >= 4)
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const int64_t off = (j * NT + t) * 4;
            const f4u* p = reinterpret_cast<const f4u*>(base + (off < last ? off : last));
            f4u v;
            if constexpr (NT_LOAD) v = __builtin_nontemporal_load(p);
            else v = *p;
            x[4 * j + 0] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < F; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t off = static_cast<uint32_t>((j * NT + t) * 4 + e);
                const float* p = base + (off < left ? off : 0u);
                if constexpr (NT_LOAD) x[4 * j + e] = __builtin_nontemporal_load(p);
                else x[4 * j + e] = *p;
            }
        }
    }
}

// After kLdUnaligned loads: the lane whose float4 straddles V read the row's
// last 4 columns, starting d = 1..3 columns before its own first column; its
// columns below V are elements d .. 3 of what it read. (Columns at or past V
// are left for fill_past_end.)
template <int NT, int F>
__device__ __forceinline__ void shift_tail_group(int64_t c0, int64_t V, float (&x)[4 * F]) {
    const int t = threadIdx.x;
    const int64_t last = V - c0 - 4;
#pragma unroll
    for (int j = 0; j < F; ++j) {
        const int64_t off = (j * NT + t) * 4;
        const int64_t d = off < last ? 0 : off - last;
        const float w0 = x[4 * j], w1 = x[4 * j + 1], w2 = x[4 * j + 2], w3 = x[4 * j + 3];
        x[4 * j + 0] = d == 0 ? w0 : (d == 1 ? w1 : (d == 2 ? w2 : w3));
        x[4 * j + 1] = d == 0 ? w1 : (d == 1 ? w2 : w3);
        x[4 * j + 2] = d == 0 ? w2 : w3;
    }
}

// A whole chunk, ready to use: loads, `fill` past V, and the allowed-id mask
// (mrow, or none). Every load is issued before any value is used; each sits
// under its own bounds test, which suits kernels that load the next chunk
// while working on this one (issue_chunk_loads suits one-shot kernels).
template <int NT, int F, bool VEC, bool NT_LOAD>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int64_t c0, int64_t V,
                                           float (&x)[4 * F], float fill = kNegInf,
                                           const uint32_t* __restrict__ mrow = nullptr) {
    const int t = threadIdx.x;
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const int64_t col = c0 + (static_cast<int64_t>(j) * NT + t) * 4;
            f4 v = {fill, fill, fill, fill};
            if (col < V) {
                const f4* p = reinterpret_cast<const f4*>(row + col);
                if constexpr (NT_LOAD) v = __builtin_nontemporal_load(p);
                else v = *p;
            }
            x[4 * j + 0] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const int64_t col = c0 + (static_cast<int64_t>(j) * NT + t) * 4;
            float v[4] = {fill, fill, fill, fill};
            if (col + 3 < V) {   // wholly inside the row: one unaligned 16-byte load
                const f4u* p = reinterpret_cast<const f4u*>(row + col);
                f4u q;
                if constexpr (NT_LOAD) q = __builtin_nontemporal_load(p);
                else q = *p;
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            } else {             // the row's last, partial float4 (or past V)
#pragma unroll
                for (int e = 0; e < 3; ++e) {
                    if (col + e < V) {
                        if constexpr (NT_LOAD) v[e] = __builtin_nontemporal_load(row + col + e);
                        else v[e] = row[col + e];
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * j + e] = v[e];
        }
    }
    if (mrow) {
        uint32_t mw[2];
        load_mask_words<NT, F>(mrow, c0, V, mw);
        apply_mask_words<NT, F>(c0, V, mw, x);
    }
}

template <int NT, int F, bool VEC, bool NT_STORE>
__device__ __forceinline__ void store_chunk(float* __restrict__ row, int64_t c0, int64_t V,
                                            const float (&y)[4 * F]) {
    const int t = threadIdx.x;
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const int64_t col = c0 + (static_cast<int64_t>(j) * NT + t) * 4;
            if (col < V) {
                f4 v = {y[4 * j + 0], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]};
                f4* p = reinterpret_cast<f4*>(row + col);
                if constexpr (NT_STORE) __builtin_nontemporal_store(v, p);
                else *p = v;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const int64_t col = c0 + (static_cast<int64_t>(j) * NT + t) * 4;
            if (col + 3 < V) {   // wholly inside the row: one unaligned 16-byte store
                f4u v = {y[4 * j + 0], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]};
                f4u* p = reinterpret_cast<f4u*>(row + col);
                if constexpr (NT_STORE) __builtin_nontemporal_store(v, p);
                else *p = v;
            } else {             // the row's last, partial float4 (or past V)
#pragma unroll
                for (int e = 0; e < 3; ++e) {
                    if (col + e < V) {
                        if constexpr (NT_STORE) __builtin_nontemporal_store(y[4 * j + e], row + col + e);
                        else row[col + e] = y[4 * j + e];
                    }
                }
            }
        }
    }
}

}  // namespace tsk
