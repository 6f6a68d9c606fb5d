// The compiler's resource report for every kernel of the library (registers,
// spills, LDS, occupancy), recorded by the build from hipcc's
// -Rpass-analysis=kernel-resource-usage remarks and compiled into the library.
// The HIP runtime reports only a kernel's total vector registers and private
// bytes; the split into architectural VGPRs and accumulation registers (AGPRs),
// the scalar registers and the spill counts come from here.
#pragma once

namespace ts {

struct KernelResources {
    const char* name;   // mangled kernel name (the symbol of its launch handle)
    int vgprs;          // architectural vector registers per lane
    int agprs;          // accumulation registers per lane
    int sgprs;          // scalar registers per wave
    int scratch;        // private (spill) bytes per lane
    int vgpr_spill;     // vector registers spilled
    int sgpr_spill;     // scalar registers spilled
    int occupancy;      // waves per SIMD the compiler computed
    int lds;            // static LDS bytes per workgroup
};

extern const KernelResources kKernelResources[];
extern const int kNumKernelResources;

}  // namespace ts
