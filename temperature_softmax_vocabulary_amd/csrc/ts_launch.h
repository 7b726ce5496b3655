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
// Rows of more chunks than this get a row-combine kernel between the split's
// two passes, so that each finalize workgroup reads its row's (shift, 1 / sum)
// instead of combining all nch partials itself (nch^2 reads per row).
constexpr int64_t kSplitRowCombineMin = 256;
constexpr int kMaxChunk = 16384;

// Slots per row for the in-kernel exchange (ts_exchange.h): the fused kernel
// runs only when a row has at most this many chunks. Each stream's workspace
// holds one slot set (the fused kernel's chunk partials (pm, pl)).
constexpr int64_t kSlotStride = 256;
constexpr int kSlotSets = 1;
constexpr int kSetPartials = 0;

// Token draws (draw_kernels.hip) work on blocks of kDrawBlock columns and
// groups of kDrawGroup columns (64 blocks): float partials per group and per
// block, then one wave per target.
constexpr int kDrawBlock = 64;
constexpr int kDrawGroup = 4096;
constexpr int kBlocksPerGroup = kDrawGroup / kDrawBlock;

// One workgroup per row: rows of up to kRowwiseRegisterMaxV columns sit in
// its registers (read once); longer rows are streamed twice. The work-split
// table picks this kernel by default for rows of up to kRowwiseResidentMaxV.
constexpr int kRowwiseThreads = 1024;
constexpr int64_t kRowwiseRegisterMaxV = 32768;
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
    float2* part;          // split: [B * nch] chunk partials (pm, pl), then for rows of
                           // more than kSplitRowCombineMin chunks [B] (shift, 1 / sum)
    float4* gpart;         // fused with draw sums: [B * ngroups] per group, the sums of
                           // its probabilities held by each of the 4 waves
    float* bpart;          // fused with draw sums: [B * ngroups * 64] sum of probs per block
    int64_t ngroups;       // groups of kDrawGroup columns per row (fused with draw sums)
    unsigned long long* slots;   // [B * kSlotStride] tagged (pm, pl) slots of the fused kernel
    uint32_t* err;         // device error flags (bit 0: a bounded wait ran out)
    uint32_t spin_limit;   // polls before a fused wait gives up
};

// Fused kernel modes: probabilities only; probabilities and the group and
// block sums of the probabilities (for a token draw that follows; chunks of a
// whole number of groups, F in {4, 8, 16}).
constexpr int kFusedProbs = 0, kFusedProbsSums = 1;

hipError_t launch_split(const SoftmaxArgs& a, int F, bool vec, hipStream_t s);
hipError_t launch_fused(const SoftmaxArgs& a, int F, bool vec, int mode, int64_t grid, hipStream_t s);
// Workgroups of the fused kernel that one device holds at once (occupancy x CUs).
hipError_t fused_resident_capacity(int F, bool vec, int mode, int64_t* cap);
hipError_t launch_rowwise(const SoftmaxArgs& a, bool vec, hipStream_t s);

// How a one-shot kernel loads a chunk (issue_chunk_loads in ts_device.h):
// four 4-byte loads per group of 4 columns (rows of fewer than 4 columns), one
// unaligned float4 per group (any other row), one aligned float4 per group (a
// 16-byte aligned row start and V % 4 == 0).
constexpr int kLdScalar = 0, kLdUnaligned = 1, kLdAligned = 2;

// Token draws (draw_kernels.hip).
constexpr int kDrawLogits = 0, kDrawProbs = 1;
struct DrawArgs {
    const float* x;           // [B, V] logits (kDrawLogits) or probabilities (kDrawProbs)
    const float* temps;       // [B] (kDrawLogits)
    const uint32_t* allowed;  // [B, mwords] allowed-id bitmask or null (kDrawLogits)
    int64_t mwords;
    const float* uniforms;    // [B, K]
    int32_t* out_ids;         // [B, K]
    float4* gpart;            // [B, ngroups] group partials: (max, sum exp2, 0, 0) from logits,
                              // or the positive sums held by each of the 4 waves
    float* bpart;             // [B, ngroups, 64] block partials: sum of the exponentials at the
                              // group's max, or of the positive probabilities
    int64_t B;
    int64_t V;
    int64_t K;
    int64_t ngroups;          // ceil(V / kDrawGroup)
    int64_t cus;              // compute units of the device (the resolve's choice of kernel)
};
// Group and block partials over the whole of x (one read), one group per
// workgroup; ld: a kLd* for x's rows.
hipError_t launch_draw_partials(const DrawArgs& a, int ld, int kind, hipStream_t s);
// One wave per (row, target): the target's group, then its block, then its id.
// With resolve_shares_rows, 16 targets of a row share a workgroup, whose
// first wave computes the row's level 1 once into LDS; otherwise every wave
// does level 1 itself.
constexpr int kResolveRowTargets = 16;
constexpr int64_t kResolveLdsMax = 65536;   // 8 (ngroups + 1) bytes must fit
hipError_t launch_draw_resolve(const DrawArgs& a, int kind, hipStream_t s);
bool resolve_shares_rows(int64_t B, int64_t K, int64_t ngroups, int64_t cus);

hipError_t launch_copy(const float* src, float* dst, int64_t n, bool vec, hipStream_t s);

// The allocation-free entry point's scratch: one device array per GPU, laid
// out as a workspace with kStaticRows rows of fused-kernel slots and
// kStaticParts split partials (flags, then slots, then partials).
constexpr int64_t kStaticRows = 1024;
constexpr int64_t kStaticParts = 262144;
constexpr int64_t kStaticScratchBytes = 256 + 8 * kSlotStride * kStaticRows * kSlotSets + 8 * kStaticParts;
// The array's device address on the current device (looked up once per
// device, with that device current).
hipError_t static_scratch(void** ptr);

}  // namespace tsk
