/*
 * Measurement and failure-path hooks of libtsoftmax. Not part of the method:
 * they exist so that the softmax's bandwidth can be put next to a plain copy
 * of the same bytes, and so that the bounded wait of the fused kernel can be
 * exercised from the host without any kernel faulting or hanging.
 */
#ifndef TSOFTMAX_MEASURE_H_
#define TSOFTMAX_MEASURE_H_

#include "tsoftmax.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dst[i] = src[i] for i in [0, n): a streaming float32 copy on `stream`
 * (16-byte loads and stores when both pointers are 16-byte aligned). It reads
 * n*4 bytes and writes n*4 bytes, the same algorithmic traffic as ts_softmax
 * on n = B*V elements, and serves as the practical bandwidth ceiling and as
 * the calibration kernel for the HBM byte counters.
 * Errors: TS_ERR_INVALID_ARGUMENT for n < 0, NULL pointers with n > 0, or
 * overlapping ranges.
 */
ts_status ts_copy_f32(const float* src, float* dst, int64_t n, hipStream_t stream);

/*
 * The memory clock (kHz) and memory bus width (bits) that HIP reports for
 * `device`, from which a peak HBM bandwidth can be recomputed beside the
 * nominal one: clock x transfers per pin per clock x width / 8 bytes, where
 * the transfers per clock depend on the memory type (4 for HBM3E).
 * Host only: launches nothing.
 * Errors: TS_ERR_INVALID_ARGUMENT for NULL pointers, TS_ERR_HIP if the query
 * fails (e.g. no such device).
 */
ts_status ts_device_memory_params(int32_t device, int32_t* clock_khz, int32_t* bus_bits);

/*
 * Number of polls (each a short sleep plus one load) a fused-kernel
 * workgroup makes while waiting for the rest of its row before it gives up,
 * raises bit 0 of the device error flags and forms the missing chunk partials
 * from the logits itself (the result stays exact). 0 restores the default
 * (about 2^18 polls, far beyond any wait on a device the call has to itself).
 * Takes effect for launches made after the call, on every device. For
 * failure-path tests only.
 */
ts_status ts_debug_set_spin_limit(uint32_t polls);

/*
 * Make the planner count on at most `workgroups` co-resident workgroups of a
 * fused kernel per device, as on a device with fewer compute units (e.g. one
 * partition of a partitioned GPU). 0 restores the queried capacity. It never
 * raises the capacity, so every fused grid still fits the device at once.
 * With a bound below a row's chunk count the default plan takes a larger
 * chunk or the split pair (ts_plan reports it) and a forced FUSED split
 * returns TS_ERR_INVALID_ARGUMENT; with one between them, each workgroup
 * loops over more (row, chunk) items. Takes effect for calls made after it,
 * on every device. For tests only.
 * Errors: TS_ERR_INVALID_ARGUMENT for workgroups < 0.
 */
ts_status ts_debug_set_resident_cap(int64_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* TSOFTMAX_MEASURE_H_ */
