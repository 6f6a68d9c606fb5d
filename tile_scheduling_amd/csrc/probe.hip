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

// Barrier-phase probe: the same MFMA stream, interrupted by workgroup barriers in
// the patterns a K loop can use.  Per iteration every wave issues 16 MFMAs
// (PATTERN 3: 32):
//   0  no barrier;
//   1  8 MFMAs, barrier, 8 MFMAs, barrier (every wave, as one mid-step barrier per
//      half K step);
//   2  ping-pong: waves 0-3 issue 16 MFMAs while waves 4-7 wait, barrier, then the
//      other way round, barrier (two phases of 16 MFMAs per SIMD);
//   3  ping-pong with phases of 32 MFMAs.
template <int PATTERN>
__global__ void __launch_bounds__(kThreads) mfma_phase_kernel(int iters, float* sink) {
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
    const bool first_half = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) < kThreads / 128;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
            constexpr int ROUNDS = PATTERN == 3 ? 4 : PATTERN == 2 ? 2 : 1;
            if (PATTERN < 2 || (ph == 0) == first_half) {
#pragma unroll
                for (int r = 0; r < ROUNDS; ++r)
#pragma unroll
                    for (int j = 0; j < kChains; ++j)
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (PATTERN != 0) __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[(long long)blockIdx.x * kThreads + threadIdx.x] = s;
}

ts_status device_cus(int* cus) {
    int dev = 0;
    *cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return TS_ERR_NO_DEVICE;
    }
    if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *cus <= 0) {
        (void)hipGetLastError();
        return TS_ERR_NO_DEVICE;
    }
    return TS_OK;
}

}  // namespace

extern "C" ts_status ts_mfma_phase_probe(int32_t iters, int32_t pattern, float* sink, int64_t sink_elems,
                                         double* flops, void* stream) {
    if (iters <= 0 || pattern < 0 || pattern > 3 || !sink || !flops) return TS_ERR_INVALID_ARG;
    int cus = 0;
    const ts_status st = device_cus(&cus);
    if (st != TS_OK) return st;
    if (sink_elems < (int64_t)cus * kThreads) return TS_ERR_INVALID_ARG;
    void (*k)(int, float*) = pattern == 0   ? mfma_phase_kernel<0>
                             : pattern == 1 ? mfma_phase_kernel<1>
                             : pattern == 2 ? mfma_phase_kernel<2>
                                            : mfma_phase_kernel<3>;
    hipLaunchKernelGGL(k, dim3(cus), dim3(kThreads), 0, (hipStream_t)stream, (int)iters, sink);
    if (hipGetLastError() != hipSuccess) return TS_ERR_HIP;
    const int per_wave = pattern == 3 ? 32 : 16;   // MFMAs per wave per iteration
    *flops = 2.0 * 32 * 32 * 16 * per_wave * (double)iters * (kThreads / 64) * cus;
    return TS_OK;
}

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
