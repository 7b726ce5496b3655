// Plain streaming float32 copy: the practical bandwidth ceiling for a kernel
// that reads n*4 bytes and writes n*4 bytes, and the calibration kernel for
// the HBM byte counters. Not part of the softmax method.
#include "ts_device.h"
#include "ts_launch.h"

namespace tsk {

namespace {

constexpr int CT = 256;
constexpr int CU = 4;      // float4 per lane per iteration

__global__ __launch_bounds__(CT) void ts_copy_vec(const f4* __restrict__ src, f4* __restrict__ dst, int64_t n4) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * CT * CU;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * CT * CU + threadIdx.x; base < n4; base += stride) {
        f4 v[CU];
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * CT;
            if (i < n4) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * CT;
            if (i < n4) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

__global__ __launch_bounds__(CT) void ts_copy_scalar(const float* __restrict__ src, float* __restrict__ dst,
                                                     int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * CT;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * CT + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy(const float* src, float* dst, int64_t n, bool vec, hipStream_t s) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (vec) {
        const int64_t n4 = n / 4;
        int64_t blocks = (n4 + CT * CU - 1) / (CT * CU);
        const int64_t cap = static_cast<int64_t>(cus) * 16;
        if (blocks > cap) blocks = cap;
        if (blocks > 0)
            hipLaunchKernelGGL(ts_copy_vec, dim3(static_cast<uint32_t>(blocks)), dim3(CT), 0, s,
                               reinterpret_cast<const f4*>(src), reinterpret_cast<f4*>(dst), n4);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t tail = n - n4 * 4;
        if (tail > 0) {
            hipLaunchKernelGGL(ts_copy_scalar, dim3(1), dim3(CT), 0, s, src + n4 * 4, dst + n4 * 4, tail);
            e = hipGetLastError();
        }
        return e;
    }
    int64_t blocks = (n + CT - 1) / CT;
    const int64_t cap = static_cast<int64_t>(cus) * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(ts_copy_scalar, dim3(static_cast<uint32_t>(blocks)), dim3(CT), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace tsk
