// Exchange of per-chunk values between the workgroups of one row, inside one
// kernel, with no fence and no contended read-modify-write.
//
// The method splits each row into column chunks and combines per-chunk values
// in a finalize step (pull-request page "fix(kernel): avoid nan in triton
// sampling softmax when a chunk starts with -inf", bug and fix paragraphs).
// Here the chunks of a row are workgroups of one kernel, and they trade their
// values through slots in device memory.
//
// Protocol. A slot set gives every row kSlotStride 64-bit slots. A slot holds
// a 63-bit payload and, in bit 63, a parity tag. Between kernels every slot of
// a row carries the same tag t. In a kernel, the workgroup of chunk c
//   1. reads its own slot rs[c] (it is that slot's only writer, so it sees t),
//   2. stores payload | (t ^ 1) into rs[c] with one 64-bit atomic store, and
//      tag t ^ 1 into the row's unused slots c + nch, c + 2 nch, ...,
//   3. polls the row's nch slots until each carries t ^ 1. The value that
//      carries the new tag is the payload itself.
// Only per-location coherence of relaxed agent-scope atomics is relied on (and
// the ordering of launches on a stream). After the kernel every slot of the
// row carries t ^ 1 again, whatever nch the next kernel uses.
//
// Progress: a row's wait ends once all of its nch workgroups have published.
// Kernels using this launch no more workgroups than the device holds at once
// and at least nch, and visit items in order, so the lowest unfinished row
// always completes. Each wait is also bounded by spin_limit polls (should the
// device be shared with other work that keeps some of a row's workgroups from
// running): running out raises bit 0 of *err, and wait_row reports the slots
// still unpublished so that the caller can form their values itself.
#pragma once

#include "ts_device.h"
#include "ts_launch.h"

namespace tsk {

constexpr unsigned long long kTagBit = 1ull << 63;
constexpr int kSlotsPerLane = static_cast<int>(kSlotStride / kWave);

__device__ __forceinline__ unsigned long long slot_load(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_store(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The high word of a slot (where its tag bit sits): enough for a workgroup to
// read the tag of its own slot, which nothing else writes.
__device__ __forceinline__ uint32_t slot_load_hi(const unsigned long long* p) {
    return __hip_atomic_load(reinterpret_cast<const uint32_t*>(p) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The tag to publish, from the old high word of the caller's own slot (read by
// lane 0 before it published anything in this kernel). Wave-uniform.
__device__ __forceinline__ unsigned long long next_tag(uint32_t own_old_hi) {
    const uint32_t hi = __builtin_amdgcn_readfirstlane(own_old_hi);
    return static_cast<unsigned long long>((hi >> 31) ^ 1u) << 63;
}

// Step 2, called by all lanes of wave 0. payload must have bit 63 clear.
__device__ __forceinline__ void publish(unsigned long long* rs, int64_t c, int64_t nch,
                                        unsigned long long tag, unsigned long long payload) {
    const int lane = threadIdx.x;
    if (lane == 0) slot_store(rs + c, tag | payload);
    for (int64_t j = c + nch * (1 + lane); j < kSlotStride; j += nch * kWave) slot_store(rs + j, tag);
}

// Step 3, called by all lanes of wave 0: v[j] receives slot lane + 64 j
// (payload only) for lane + 64 j < nch, else `absent`. Returns, per lane, bit j
// set for each of its slots that still carried the old tag when the lane's
// polls ran out (v[j] is then `absent`, not a value of the row).
__device__ __forceinline__ uint32_t wait_row(const unsigned long long* rs, int64_t nch, unsigned long long tag,
                                             unsigned long long absent, unsigned long long (&v)[kSlotsPerLane],
                                             uint32_t spin_limit, uint32_t* err) {
    const int lane = threadIdx.x;
    uint32_t polls = 0, missing = 0;
#pragma unroll
    for (int j = 0; j < kSlotsPerLane; ++j) {
        const int64_t i = lane + static_cast<int64_t>(j) * kWave;
        v[j] = absent;
        if (i < nch) {
            unsigned long long x = slot_load(rs + i);
            while ((x & kTagBit) != tag) {
                if (++polls > spin_limit) {
                    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    missing |= 1u << j;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                x = slot_load(rs + i);
            }
            if (!((missing >> j) & 1u)) v[j] = x & ~kTagBit;
        }
    }
    return missing;
}

}  // namespace tsk
