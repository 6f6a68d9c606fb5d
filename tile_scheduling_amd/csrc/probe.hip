// Empirical MFMA throughput probe: the rate the matrix cores sustain on this
// device with no memory traffic, the ceiling a GEMM kernel's MFMA stream could
// reach at the clock it is given.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tsgemm.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;   // 8 waves, two per SIMD, as the 256x256x64 GEMM tile
constexpr int kChains = 8;      // independent accumulators per wave

__global__ void __launch_bounds__(kThreads) mfma_loop_kernel(int iters, float* sink) {
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)((threadIdx.x & 7) * 0.125f + i);
        b[i] = (_Float16)(i * 0.25f);
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[(long long)blockIdx.x * kThreads + threadIdx.x] = s;   // keeps every MFMA live
}

}  // namespace

extern "C" ts_status ts_mfma_loop_probe(int32_t iters, float* sink, int64_t sink_elems, double* flops,
                                        void* stream) {
    if (iters <= 0 || !sink || !flops) return TS_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return TS_ERR_NO_DEVICE;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return TS_ERR_NO_DEVICE;
    }
    if (sink_elems < (int64_t)cus * kThreads) return TS_ERR_INVALID_ARG;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(cus), dim3(kThreads), 0, (hipStream_t)stream, (int)iters, sink);
    if (hipGetLastError() != hipSuccess) return TS_ERR_HIP;
    *flops = 2.0 * 32 * 32 * 16 * kChains * (double)iters * (kThreads / 64) * cus;
    return TS_OK;
}
