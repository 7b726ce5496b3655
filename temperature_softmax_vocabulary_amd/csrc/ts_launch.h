// Internal host-side launch interface between the C-ABI layer and the HIP
// kernels. Not installed, not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsk {

// Columns per chunk for the split and fused kernels: 1024 * F, F in {1,2,4,8,16}
// (256 lanes x F float4 each).
constexpr int kChunkThreads = 256;
constexpr int kMinChunk = 1024;
constexpr int kMaxChunk = 16384;

// Slots per row for the in-kernel exchange (ts_exchange.h): the chunked
// kernels run only when a row has at most this many chunks. Each stream's
// workspace holds two slot sets: the fused kernel's chunk partials (pm, pl),
// and the chunked sampler's float sums.
constexpr int64_t kSlotStride = 256;
constexpr int kSlotSets = 2;
constexpr int kSetPartials = 0, kSetFloatSums = 1;

// Largest row the resident one-workgroup-per-row kernel holds in registers.
constexpr int kRowwiseThreads = 1024;
constexpr int64_t kRowwiseResidentMaxV = 16384;

struct SoftmaxArgs {
    const float* logits;   // [B, V]
    const float* temps;    // [B]
    const uint32_t* allowed;  // [B, mwords] allowed-id bitmask, or null (no mask)
    int64_t mwords;        // ceil(V / 32)
    float* out;            // [B, V]
    int64_t B;
    int64_t V;
    int64_t nch;           // chunks per row (split, fused)
    int64_t items;         // B * nch
    float2* part;          // [B * nch] chunk partials (pm, pl) of the split kernels
    unsigned long long* slots;   // [B * kSlotStride] tagged (pm, pl) slots of the fused kernel
    uint32_t* err;         // device error flags (bit 0: a bounded wait ran out)
    uint32_t spin_limit;   // polls before a fused wait gives up
    // fused softmax-and-sample only
    const float* uniforms; // [B, K]
    int32_t* out_ids;      // [B, K]
    int64_t K;
};

// Fused kernel modes: probabilities only; probabilities and ids; ids only.
constexpr int kFusedProbs = 0, kFusedProbsIds = 1, kFusedIds = 2;

hipError_t launch_split(const SoftmaxArgs& a, int F, bool vec, hipStream_t s);
hipError_t launch_fused(const SoftmaxArgs& a, int F, bool vec, int mode, int64_t grid, hipStream_t s);
// Workgroups of the fused kernel that one device holds at once (occupancy x CUs).
hipError_t fused_resident_capacity(int F, bool vec, int mode, int64_t* cap);
hipError_t launch_rowwise(const SoftmaxArgs& a, bool vec, hipStream_t s);

struct SampleArgs {
    const float* probs;      // [B, V]
    const float* uniforms;   // [B, K]
    int32_t* out_ids;        // [B, K]
    int64_t B;
    int64_t V;
    int64_t K;
    // chunked kernel only
    int64_t nch;
    int64_t items;
    unsigned long long* fslots;  // [B * kSlotStride] tagged float-sum slots
    uint32_t* err;
    uint32_t spin_limit;
};
// One workgroup per row, three sweeps (any V).
hipError_t launch_sample_rows(const SampleArgs& a, bool vec, hipStream_t s);
// Chunked, one read: (row, chunk) items over a persistent grid (nch <= kSlotStride).
hipError_t launch_sample_chunks(const SampleArgs& a, int F, bool vec, int64_t grid, hipStream_t s);
hipError_t sample_resident_capacity(int F, bool vec, int64_t* cap);

hipError_t launch_copy(const float* src, float* dst, int64_t n, bool vec, hipStream_t s);

}  // namespace tsk
