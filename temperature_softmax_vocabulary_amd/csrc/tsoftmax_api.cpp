// C-ABI layer of libtsoftmax: argument checks, the (B, V) -> work-split table,
// the per-stream workspace, and kernel dispatch. Host code only; every step of
// the computation runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <array>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <map>
#include <tuple>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/tsoftmax.h"
#include "../../include/tsoftmax_measure.h"
#include "ts_launch.h"

#define TS_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint32_t kDefaultSpinLimit = 1u << 18;
std::atomic<uint32_t> g_spin_limit{kDefaultSpinLimit};
// Upper bound on the co-resident workgroups the planner counts on (0: none).
std::atomic<int64_t> g_cap_limit{0};

// ----------------------------------------------------------------------------
// argument checks (host only: no device reads)
// ----------------------------------------------------------------------------
bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// B * V * 4 bytes must be addressable and the element count must fit int64.
bool sizes_ok(int64_t B, int64_t V) {
    if (B < 0 || V < 1 || V > INT32_MAX) return false;
    return B <= (INT64_MAX / 8) / V;
}

// ----------------------------------------------------------------------------
// workspace: one per (device, stream), grow-only, zeroed when allocated.
// Layout is fixed by the allocation's capacity, never by the call, so row r's
// slots stay at the same address whatever B and V the calls use (their tags
// carry over from call to call, ts_exchange.h):
//   [0, 256)                                   flags (uint32 at offset 0)
//   [256, 256 + 8 kSlotStride Bcap kSlotSets)  slots[kSlotSets][Bcap][kSlotStride]
//   [aligned 256, + 8 Pcap)                    part[Pcap] (float2, split)
// An outgrown allocation is retired, never freed: a graph captured on the
// stream may still point at it, and work queued before the growth may still
// use it. Growth is geometric, so a stream retires only a few.
// ----------------------------------------------------------------------------
struct Alloc {
    void* base = nullptr;
    int64_t bcap = 0;   // rows
    int64_t pcap = 0;   // partials
};

struct Workspace : Alloc {
    std::vector<Alloc> retired;
};

struct WsView {
    uint32_t* err;
    unsigned long long* sets[tsk::kSlotSets];
    float2* part;
};

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int64_t slot_bytes(int64_t bcap) { return 8 * tsk::kSlotStride * bcap * tsk::kSlotSets; }

int64_t ws_bytes(int64_t bcap, int64_t pcap) {
    return align256(256 + slot_bytes(bcap)) + 8 * pcap;
}

WsView ws_view(const Alloc& w) {
    char* b = static_cast<char*>(w.base);
    WsView v;
    v.err = reinterpret_cast<uint32_t*>(b);
    for (int k = 0; k < tsk::kSlotSets; ++k)
        v.sets[k] = reinterpret_cast<unsigned long long*>(b + 256) + static_cast<int64_t>(k) * tsk::kSlotStride * w.bcap;
    v.part = reinterpret_cast<float2*>(b + align256(256 + slot_bytes(w.bcap)));
    return v;
}

std::mutex g_mu;   // guards g_ws and is held across each launch that uses it
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

ts_status hip_status(hipError_t e) {
    if (e == hipSuccess) return TS_OK;
    if (e == hipErrorOutOfMemory) return TS_ERR_OUT_OF_MEMORY;
    return TS_ERR_HIP;
}

// Called with g_mu held. Makes the stream's workspace hold >= need_b rows and
// need_p partials, allocating (outside capture only) and zeroing if it grows.
ts_status ws_get(hipStream_t stream, int64_t need_b, int64_t need_p, Workspace** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return TS_ERR_HIP;
    Workspace& w = g_ws[{dev, stream}];
    if (w.base && w.bcap >= need_b && w.pcap >= need_p) {
        *out = &w;
        return TS_OK;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return TS_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return TS_ERR_NOT_RESERVED;
    // at least double what grows, so that few allocations are ever retired
    int64_t nb = w.bcap, np = w.pcap;
    if (need_b > nb) nb = need_b > 2 * w.bcap ? need_b : 2 * w.bcap;
    if (need_p > np) np = need_p > 2 * w.pcap ? need_p : 2 * w.pcap;
    void* p = nullptr;
    const int64_t bytes = ws_bytes(nb, np);
    e = hipMalloc(&p, static_cast<size_t>(bytes));
    if (e != hipSuccess) return e == hipErrorOutOfMemory ? TS_ERR_OUT_OF_MEMORY : TS_ERR_HIP;
    // cleared in stream order, before any later call on the stream uses it
    e = hipMemsetAsync(p, 0, static_cast<size_t>(bytes), stream);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return TS_ERR_HIP;
    }
    if (w.base) w.retired.push_back(Alloc{w.base, w.bcap, w.pcap});
    w.base = p;
    w.bcap = nb;
    w.pcap = np;
    *out = &w;
    return TS_OK;
}

// ----------------------------------------------------------------------------
// work-split table (a7): variant and chunk from (B, V)
// ----------------------------------------------------------------------------
constexpr int kFs[] = {1, 2, 4, 8, 16};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
    int variant;
    int F;   // chunk = 1024 * F (split, fused)
};

// Workgroups one device holds at once, per kernel (cached per device):
// kind = the fused kernel's mode.
ts_status resident_cap(int kind, int F, bool vec, int64_t* cap) {
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, bool>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TS_ERR_HIP;
    std::lock_guard<std::mutex> lk(mu);
    const auto key = std::make_tuple(dev, kind, F, vec);
    auto it = cache.find(key);
    if (it == cache.end()) {
        int64_t c = 0;
        const hipError_t e = tsk::fused_resident_capacity(F, vec, kind, &c);
        if (e != hipSuccess) return TS_ERR_HIP;
        it = cache.emplace(key, c).first;
    }
    *cap = it->second;
    const int64_t lim = g_cap_limit.load(std::memory_order_relaxed);
    if (lim > 0 && *cap > lim) *cap = lim;
    return TS_OK;
}

// Compute units of the current device (cached per device).
ts_status device_cus(int64_t* cus) {
    static std::mutex mu;
    static std::map<int, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TS_ERR_HIP;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it == cache.end()) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return TS_ERR_HIP;
        it = cache.emplace(dev, n).first;
    }
    *cus = it->second;
    return TS_OK;
}

// A fused split needs every chunk of a row resident at once (ts_exchange.h),
// so rows of more chunks than the row's slots or than the device holds at
// once cannot take it. Without `on_device` only the slots are checked.
ts_status fused_fits(int F, bool vec, int64_t V, bool on_device, bool* fits) {
    *fits = false;
    const int64_t nch = cdiv(V, 1024 * F);
    if (nch > tsk::kSlotStride) return TS_OK;
    if (!on_device) {
        *fits = true;
        return TS_OK;
    }
    int64_t cap = 0;
    const ts_status st = resident_cap(tsk::kFusedProbs, F, vec, &cap);
    if (st != TS_OK) return st;
    *fits = nch <= cap;
    return TS_OK;
}

// The work-split table, from cold timings on MI355X of every variant and
// chunk size over B in {1, 3, 8, 16, 32, 64, 128, 256} and V in {151936,
// 201088, 262144}, and by graph replay around each edge (B in 2..16 for those
// V; B in 16..256 for V of 32000..65536; B in 16..4096 for V of 4096..32768):
//  - a row that fits one workgroup's registers: one workgroup per row (single
//    read, no partials), but the fused split for 768..2048 such rows of at
//    least 4096 columns; for rows of 16385..32768 columns only where it was
//    measured faster;
//  - B*V <= 2^20 elements, or 2^21 for rows of at most 65536 columns: fused,
//    4096-column chunks (the call is bound by latency; more, smaller
//    workgroups; beyond that 8192 columns are as fast or faster, by graph
//    replay at B in 2..256);
//  - larger: fused, 8192-column chunks (four workgroups per CU hide the waits
//    better than two of 16384 columns, and a short last chunk wastes less:
//    at B=64 it is 22.7 against 23.2 us for V=262144 and 14.7 against 17.6 us
//    for V=151936);
//  - rows of more chunks than the fused split can hold (kSlotStride, or
//    what the device holds at once): the next larger chunk while that fits,
//    else the split pair, which never waits.
ts_status choose_plan(int64_t B, int64_t V, bool vec, bool on_device, Plan* p) {
    if (V <= tsk::kRowwiseResidentMaxV) {
        // except for 768..2048 rows of 4096..16384 columns: there the row
        // kernel's 1024-lane workgroups fill the device in uneven rounds, and
        // the fused split was 1-12 % faster (by graph replay)
        if (V >= 4096 && B >= 768 && B <= 2048) {
            const int F = V > 4096 ? 8 : 4;
            bool fits = false;
            const ts_status st = fused_fits(F, vec, V, on_device, &fits);
            if (st != TS_OK) return st;
            if (fits) {
                *p = Plan{TS_VARIANT_FUSED, F};
                return TS_OK;
            }
        }
        *p = Plan{TS_VARIANT_ROWWISE, 0};
        return TS_OK;
    }
    // rows of 16385..32768 columns still fit the row kernel's registers (8
    // values a lane); it was 2-21 % faster than the fused split for at least
    // 128 rows of up to 20480 columns and for at least 2048 rows of any such
    // length, and up to 13 % slower elsewhere (rows of 3 or 4 whole
    // 8192-column chunks at 512..1536 rows), by graph replay
    if (V <= tsk::kRowwiseRegisterMaxV && (B >= 2048 || (V <= 20480 && B >= 128))) {
        *p = Plan{TS_VARIANT_ROWWISE, 0};
        return TS_OK;
    }
    const int64_t small = V <= 65536 ? (int64_t(1) << 21) : (int64_t(1) << 20);
    for (int F = B * V <= small ? 4 : 8; F <= 16; F *= 2) {
        bool fits = false;
        const ts_status st = fused_fits(F, vec, V, on_device, &fits);
        if (st != TS_OK) return st;
        if (fits) {
            *p = Plan{TS_VARIANT_FUSED, F};
            return TS_OK;
        }
    }
    *p = Plan{TS_VARIANT_SPLIT, 16};
    return TS_OK;
}

// The softmax ahead of a draw that also writes the probabilities: the fused
// split leaves the draw's group sums of the probabilities, which the draw
// otherwise reads the probabilities once more to form, so rows the table
// gives the row kernel take the fused split here when it fits.
ts_status choose_draw_plan(int64_t B, int64_t V, bool vec, Plan* p) {
    ts_status st = choose_plan(B, V, vec, true, p);
    if (st != TS_OK || p->variant != TS_VARIANT_ROWWISE) return st;
    const int64_t small = V <= 65536 ? (int64_t(1) << 21) : (int64_t(1) << 20);
    const int F = B * V <= small || V <= 4096 ? 4 : 8;
    bool fits = false;
    st = fused_fits(F, vec, V, true, &fits);
    if (st == TS_OK && fits) *p = Plan{TS_VARIANT_FUSED, F};
    return st;
}

// Fused grid: one workgroup per item while the device holds them all at once;
// beyond that the grid is the device's capacity and each workgroup loops over
// items, loading its next chunk while it waits on the current row. Never
// fewer workgroups than chunks per row.
int64_t fused_grid(int64_t items, int64_t nch, int64_t cap) {
    int64_t g = items < cap ? items : cap;
    if (g < nch) g = nch;
    return g;
}

int64_t mask_words(int64_t V) { return (V + 31) / 32; }

// A softmax call, checked and planned, ready to launch on a workspace.
struct SoftmaxCall {
    tsk::SoftmaxArgs a{};
    Plan plan{};
    bool vec = false;
    int64_t grid = 0;
    int64_t need_b = 0;   // workspace rows (fused slots)
    int64_t need_p = 0;   // workspace partials (split)
};

// Argument checks and the work split; launches nothing. B > 0.
ts_status prepare_softmax(const float* logits, const float* temps, const uint32_t* allowed, int64_t B, int64_t V,
                          float* out, int variant, int chunk, SoftmaxCall* call, bool for_draw = false) {
    if (!logits || !temps || !out) return TS_ERR_INVALID_ARGUMENT;
    const int64_t xbytes = B * V * 4;
    if (out != logits && overlaps(out, xbytes, logits, xbytes)) return TS_ERR_INVALID_ARGUMENT;
    if (overlaps(out, xbytes, temps, B * 4)) return TS_ERR_INVALID_ARGUMENT;
    if (allowed && overlaps(out, xbytes, allowed, B * mask_words(V) * 4)) return TS_ERR_INVALID_ARGUMENT;
    if (variant < TS_VARIANT_AUTO || variant > TS_VARIANT_FUSED) return TS_ERR_INVALID_ARGUMENT;
    int F = 0;
    if (chunk != 0) {
        if (chunk % 1024 != 0) return TS_ERR_INVALID_ARGUMENT;
        F = chunk / 1024;
        if (F != 1 && F != 2 && F != 4 && F != 8 && F != 16) return TS_ERR_INVALID_ARGUMENT;
    }
    const bool vec = aligned16(logits) && aligned16(out) && (V % 4 == 0);

    Plan plan{variant, F};
    if (variant == TS_VARIANT_AUTO) {
        ts_status st = for_draw ? choose_draw_plan(B, V, vec, &plan) : choose_plan(B, V, vec, true, &plan);
        if (st != TS_OK) return st;
        if (F != 0 && plan.variant != TS_VARIANT_ROWWISE) plan.F = F;
    }
    if (plan.variant != TS_VARIANT_ROWWISE && plan.F == 0) {
        // the smallest chunk giving at least ~2 workgroups per CU, else 16K
        plan.F = 16;
        for (int f : kFs) {
            if (B * cdiv(V, 1024 * f) <= 2048) { plan.F = f; break; }
        }
    }

    tsk::SoftmaxArgs& a = call->a;
    a = tsk::SoftmaxArgs{};
    a.logits = logits;
    a.temps = temps;
    a.allowed = allowed;
    a.mwords = mask_words(V);
    a.out = out;
    a.B = B;
    a.V = V;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    call->plan = plan;
    call->vec = vec;

    if (plan.variant == TS_VARIANT_ROWWISE) {
        if (B > INT32_MAX) return TS_ERR_INVALID_ARGUMENT;
        return TS_OK;
    }
    a.nch = cdiv(V, 1024 * plan.F);
    a.items = B * a.nch;
    call->grid = a.items;
    if (plan.variant == TS_VARIANT_FUSED) {
        int64_t cap = 0;
        ts_status st = resident_cap(tsk::kFusedProbs, plan.F, vec, &cap);
        if (st != TS_OK) return st;
        // The lowest unfinished row must fit the device at once (ts_exchange.h).
        if (a.nch > tsk::kSlotStride || a.nch > cap) return TS_ERR_INVALID_ARGUMENT;
        call->grid = fused_grid(a.items, a.nch, cap);
        call->need_b = B;
    } else {
        if (a.items > INT32_MAX) return TS_ERR_INVALID_ARGUMENT;
        call->need_p = a.items + (a.nch > tsk::kSplitRowCombineMin ? B : 0);   // (+ per-row (shift, 1 / sum))
    }
    return TS_OK;
}

// Called with g_mu held and a workspace sized for the call. With group_sums
// and the fused split, the kernel also writes the per-group sums of the
// probabilities to the workspace partials (*sums = true).
ts_status launch_softmax(SoftmaxCall& call, const WsView& v, bool group_sums, bool* sums, hipStream_t stream) {
    tsk::SoftmaxArgs& a = call.a;
    if (sums) *sums = false;
    if (call.plan.variant == TS_VARIANT_ROWWISE) return hip_status(tsk::launch_rowwise(a, call.vec, stream));
    a.part = v.part;
    a.slots = v.sets[tsk::kSetPartials];
    a.err = v.err;
    if (call.plan.variant == TS_VARIANT_FUSED) {
        int mode = tsk::kFusedProbs;
        int64_t grid = call.grid;
        if (group_sums && call.plan.F % 4 == 0) {   // chunks of whole draw groups
            // (at the plan's chunk: at 8192 columns the sums keep the plain
            // mode's four waves per SIMD without spills, which beats 16384
            // columns, two waves, at every batch measured)
            // this mode has its own occupancy: the grid must fit it too
            int64_t cap = 0;
            ts_status st = resident_cap(tsk::kFusedProbsSums, call.plan.F, call.vec, &cap);
            if (st != TS_OK) return st;
            if (a.nch <= cap) {   // else: the plain mode as planned, and a partials kernel later
                mode = tsk::kFusedProbsSums;
                grid = fused_grid(a.items, a.nch, cap);
                a.ngroups = cdiv(a.V, tsk::kDrawGroup);
                a.gpart = reinterpret_cast<float4*>(v.part);
                a.bpart = reinterpret_cast<float*>(v.part + 2 * a.B * a.ngroups);
                *sums = true;
            }
        }
        return hip_status(tsk::launch_fused(a, call.plan.F, call.vec, mode, grid, stream));
    }
    return hip_status(tsk::launch_split(a, call.plan.F, call.vec, stream));
}

ts_status run_softmax(const float* logits, const float* temps, const uint32_t* allowed, int64_t B, int64_t V,
                      float* out, int variant, int chunk, hipStream_t stream) {
    if (!sizes_ok(B, V)) return TS_ERR_INVALID_ARGUMENT;
    if (B == 0) return TS_OK;
    SoftmaxCall call;
    ts_status st = prepare_softmax(logits, temps, allowed, B, V, out, variant, chunk, &call);
    if (st != TS_OK) return st;
    if (call.plan.variant == TS_VARIANT_ROWWISE) return launch_softmax(call, WsView{}, false, nullptr, stream);
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace* w = nullptr;
    st = ws_get(stream, call.need_b, call.need_p, &w);
    if (st != TS_OK) return st;
    return launch_softmax(call, ws_view(*w), false, nullptr, stream);
}

// Workspace partials of a draw, in float2 units: one float4 per group of 4096
// columns, then 64 floats per group (its blocks of 64 columns).
int64_t draw_parts(int64_t B, int64_t V) { return B * cdiv(V, tsk::kDrawGroup) * (2 + tsk::kBlocksPerGroup / 2); }

// The draw's two kernels (draw_kernels.hip) on x = logits (kDrawLogits) or
// probabilities (kDrawProbs); partials_done: the partials are already in the
// workspace (written by the fused softmax). Called with g_mu held.
ts_status launch_draw(int kind, const float* x, const float* temps, const uint32_t* allowed, const float* uniforms,
                      int64_t B, int64_t V, int64_t K, int32_t* out_ids, const WsView& v, bool partials_done,
                      hipStream_t stream) {
    tsk::DrawArgs d{};
    d.x = x;
    d.temps = temps;
    d.allowed = allowed;
    d.mwords = mask_words(V);
    d.uniforms = uniforms;
    d.out_ids = out_ids;
    d.B = B;
    d.V = V;
    d.K = K;
    d.ngroups = cdiv(V, tsk::kDrawGroup);
    ts_status st = device_cus(&d.cus);
    if (st != TS_OK) return st;
    d.gpart = reinterpret_cast<float4*>(v.part);
    d.bpart = reinterpret_cast<float*>(v.part + 2 * B * d.ngroups);
    const int ld = aligned16(x) && (V % 4 == 0) ? tsk::kLdAligned : tsk::kLdUnaligned;
    if (!partials_done) {
        hipError_t e = tsk::launch_draw_partials(d, ld, kind, stream);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(tsk::launch_draw_resolve(d, kind, stream));
}

// Size limits of the draw's grids (32-bit grid dimensions).
// (the resolve's grid is at most the one-wave-per-target grid)
bool draw_sizes_ok(int64_t B, int64_t V, int64_t K) {
    return B * cdiv(V, tsk::kDrawGroup) <= INT32_MAX && cdiv(B * K, 4) <= INT32_MAX;
}

}  // namespace

TS_API ts_status ts_softmax(const float* logits, const float* temps, int64_t B, int64_t V, float* out,
                            hipStream_t stream) {
    return run_softmax(logits, temps, nullptr, B, V, out, TS_VARIANT_AUTO, 0, stream);
}

TS_API ts_status ts_softmax_noalloc(const float* logits, const float* temps, int64_t B, int64_t V, float* out,
                                    hipStream_t stream) {
    if (!sizes_ok(B, V)) return TS_ERR_INVALID_ARGUMENT;
    if (B == 0) return TS_OK;
    SoftmaxCall call;
    ts_status st = prepare_softmax(logits, temps, nullptr, B, V, out, TS_VARIANT_AUTO, 0, &call);
    if (st != TS_OK) return st;
    if (call.plan.variant == TS_VARIANT_ROWWISE) return launch_softmax(call, WsView{}, false, nullptr, stream);
    if (call.need_b > tsk::kStaticRows || call.need_p > tsk::kStaticParts) return TS_ERR_INVALID_ARGUMENT;
    void* base = nullptr;
    if (tsk::static_scratch(&base) != hipSuccess) return TS_ERR_HIP;
    static_assert(tsk::kStaticScratchBytes == 256 + 8 * tsk::kSlotStride * tsk::kStaticRows * tsk::kSlotSets +
                                                  8 * tsk::kStaticParts,
                  "the scratch is laid out as a workspace of kStaticRows rows and kStaticParts partials");
    return launch_softmax(call, ws_view(Alloc{base, tsk::kStaticRows, tsk::kStaticParts}), false, nullptr, stream);
}

TS_API ts_status ts_softmax_masked(const float* logits, const float* temps, const uint32_t* allowed, int64_t B,
                                   int64_t V, float* out, hipStream_t stream) {
    if (B > 0 && !allowed) return TS_ERR_INVALID_ARGUMENT;
    return run_softmax(logits, temps, allowed, B, V, out, TS_VARIANT_AUTO, 0, stream);
}

TS_API ts_status ts_softmax_variant(const float* logits, const float* temps, const uint32_t* allowed, int64_t B,
                                    int64_t V, float* out, int32_t variant, int32_t chunk, hipStream_t stream) {
    return run_softmax(logits, temps, allowed, B, V, out, variant, chunk, stream);
}

TS_API ts_status ts_plan(int64_t B, int64_t V, int32_t* variant, int32_t* chunk) {
    if (!sizes_ok(B, V) || !variant || !chunk) return TS_ERR_INVALID_ARGUMENT;
    // with no HIP device (host-only use) the table alone: no call can run there
    int ndev = 0;
    const bool on_device = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0;
    Plan p{};
    ts_status st = choose_plan(B, V, true, on_device, &p);
    if (st != TS_OK) return st;
    *variant = p.variant;
    *chunk = p.F * 1024;
    return TS_OK;
}

TS_API ts_status ts_sample(const float* probs, const float* uniforms, int64_t B, int64_t V, int64_t K,
                           int32_t* out_ids, hipStream_t stream) {
    if (!sizes_ok(B, V) || K < 0 || (K > 0 && B > (INT64_MAX / 8) / K)) return TS_ERR_INVALID_ARGUMENT;
    if (B == 0 || K == 0) return TS_OK;
    if (!probs || !uniforms || !out_ids) return TS_ERR_INVALID_ARGUMENT;
    if (!draw_sizes_ok(B, V, K)) return TS_ERR_INVALID_ARGUMENT;
    if (overlaps(out_ids, B * K * 4, probs, B * V * 4) || overlaps(out_ids, B * K * 4, uniforms, B * K * 4))
        return TS_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace* w = nullptr;
    ts_status st = ws_get(stream, 0, draw_parts(B, V), &w);
    if (st != TS_OK) return st;
    return launch_draw(tsk::kDrawProbs, probs, nullptr, nullptr, uniforms, B, V, K, out_ids, ws_view(*w), false,
                       stream);
}

TS_API ts_status ts_softmax_sample(const float* logits, const float* temps, const uint32_t* allowed,
                                   const float* uniforms, int64_t B, int64_t V, int64_t K, float* probs_out,
                                   int32_t* out_ids, hipStream_t stream) {
    if (!sizes_ok(B, V) || K < 0 || (K > 0 && B > (INT64_MAX / 8) / K)) return TS_ERR_INVALID_ARGUMENT;
    if (B == 0) return TS_OK;
    if (!logits || !temps || (K > 0 && (!uniforms || !out_ids))) return TS_ERR_INVALID_ARGUMENT;
    const int64_t xbytes = B * V * 4, kbytes = B * K * 4;
    if (probs_out) {
        if (probs_out != logits && overlaps(probs_out, xbytes, logits, xbytes)) return TS_ERR_INVALID_ARGUMENT;
        if (overlaps(probs_out, xbytes, temps, B * 4) || overlaps(probs_out, xbytes, uniforms, kbytes) ||
            overlaps(probs_out, xbytes, out_ids, kbytes))
            return TS_ERR_INVALID_ARGUMENT;
    }
    if (overlaps(out_ids, kbytes, logits, xbytes) || overlaps(out_ids, kbytes, temps, B * 4) ||
        overlaps(out_ids, kbytes, uniforms, kbytes))
        return TS_ERR_INVALID_ARGUMENT;
    const int64_t mbytes = B * mask_words(V) * 4;
    if (allowed && (overlaps(out_ids, kbytes, allowed, mbytes) || (probs_out && overlaps(probs_out, xbytes, allowed, mbytes))))
        return TS_ERR_INVALID_ARGUMENT;
    if (K == 0)
        return probs_out ? run_softmax(logits, temps, allowed, B, V, probs_out, TS_VARIANT_AUTO, 0, stream) : TS_OK;
    if (!draw_sizes_ok(B, V, K)) return TS_ERR_INVALID_ARGUMENT;
    const int64_t nparts = draw_parts(B, V);
    if (!probs_out) {
        // ids only: group partials straight from the logits (one read), then the draw
        std::lock_guard<std::mutex> lk(g_mu);
        Workspace* w = nullptr;
        ts_status st = ws_get(stream, 0, nparts, &w);
        if (st != TS_OK) return st;
        return launch_draw(tsk::kDrawLogits, logits, temps, allowed, uniforms, B, V, K, out_ids, ws_view(*w), false,
                           stream);
    }
    // probabilities and ids: the softmax (the fused split also leaves the group
    // sums of the probabilities), then the draw on the written probabilities
    SoftmaxCall call;
    ts_status st = prepare_softmax(logits, temps, allowed, B, V, probs_out, TS_VARIANT_AUTO, 0, &call, true);
    if (st != TS_OK) return st;
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace* w = nullptr;
    st = ws_get(stream, call.need_b, call.need_p > nparts ? call.need_p : nparts, &w);
    if (st != TS_OK) return st;
    const WsView v = ws_view(*w);
    bool sums = false;
    st = launch_softmax(call, v, true, &sums, stream);
    if (st != TS_OK) return st;
    return launch_draw(tsk::kDrawProbs, probs_out, nullptr, nullptr, uniforms, B, V, K, out_ids, v, sums, stream);
}

TS_API ts_status ts_reserve(int64_t max_B, int64_t max_V, hipStream_t stream) {
    if (!sizes_ok(max_B, max_V)) return TS_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace* w = nullptr;
    const int64_t split_parts = max_B * cdiv(max_V, tsk::kMinChunk) + max_B;
    const int64_t parts = draw_parts(max_B, max_V);
    return ws_get(stream, max_B, split_parts > parts ? split_parts : parts, &w);
}

TS_API ts_status ts_device_errors(hipStream_t stream, uint32_t* flags) {
    if (!flags) return TS_ERR_INVALID_ARGUMENT;
    *flags = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TS_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_ws.find({dev, stream});
    if (it == g_ws.end() || !it->second.base) return TS_OK;
    if (hipStreamSynchronize(stream) != hipSuccess) return TS_ERR_HIP;
    uint32_t all = 0;
    std::vector<Alloc> allocs = it->second.retired;   // (graphs may still write to these)
    allocs.push_back(it->second);
    for (const Alloc& a : allocs) {
        uint32_t f = 0;
        if (hipMemcpy(&f, a.base, 4, hipMemcpyDeviceToHost) != hipSuccess) return TS_ERR_HIP;
        // (a wait that ran out still leaves every slot of its row with the
        // kernel's new tag: each workgroup publishes before it waits)
        if (f != 0 && hipMemset(a.base, 0, sizeof(uint32_t)) != hipSuccess) return TS_ERR_HIP;
        all |= f;
    }
    *flags = all;
    return (all & 1u) ? TS_ERR_SYNC_TIMEOUT : TS_OK;
}

TS_API const char* ts_status_string(ts_status s) {
    switch (s) {
        case TS_OK: return "TS_OK";
        case TS_ERR_INVALID_ARGUMENT: return "TS_ERR_INVALID_ARGUMENT: a pointer, size or alias rule was broken";
        case TS_ERR_HIP: return "TS_ERR_HIP: the HIP runtime reported an error";
        case TS_ERR_OUT_OF_MEMORY: return "TS_ERR_OUT_OF_MEMORY: workspace allocation failed";
        case TS_ERR_NOT_RESERVED:
            return "TS_ERR_NOT_RESERVED: the stream is capturing and the workspace is too small; call ts_reserve first";
        case TS_ERR_SYNC_TIMEOUT:
            return "TS_ERR_SYNC_TIMEOUT: a fused kernel's bounded wait ran out (the missing partials were formed "
                   "in place of it: the results are exact)";
    }
    return "unknown ts_status";
}

TS_API int32_t ts_abi_version(void) { return TSOFTMAX_ABI_VERSION; }

TS_API ts_status ts_copy_f32(const float* src, float* dst, int64_t n, hipStream_t stream) {
    if (n < 0 || n > INT64_MAX / 8) return TS_ERR_INVALID_ARGUMENT;
    if (n == 0) return TS_OK;
    if (!src || !dst || overlaps(src, n * 4, dst, n * 4)) return TS_ERR_INVALID_ARGUMENT;
    const bool vec = aligned16(src) && aligned16(dst);
    return hip_status(tsk::launch_copy(src, dst, n, vec, stream));
}

TS_API ts_status ts_debug_set_spin_limit(uint32_t polls) {
    g_spin_limit.store(polls == 0 ? kDefaultSpinLimit : polls, std::memory_order_relaxed);
    return TS_OK;
}

TS_API ts_status ts_device_memory_params(int32_t device, int32_t* clock_khz, int32_t* bus_bits) {
    if (!clock_khz || !bus_bits) return TS_ERR_INVALID_ARGUMENT;
    int c = 0, w = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMemoryClockRate, device) != hipSuccess) return TS_ERR_HIP;
    if (hipDeviceGetAttribute(&w, hipDeviceAttributeMemoryBusWidth, device) != hipSuccess) return TS_ERR_HIP;
    *clock_khz = c;
    *bus_bits = w;
    return TS_OK;
}

TS_API ts_status ts_debug_set_resident_cap(int64_t workgroups) {
    if (workgroups < 0) return TS_ERR_INVALID_ARGUMENT;
    g_cap_limit.store(workgroups, std::memory_order_relaxed);
    return TS_OK;
}
