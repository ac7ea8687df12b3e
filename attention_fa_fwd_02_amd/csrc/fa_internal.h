// Internal interface between the C ABI (fa_api.cpp) and the kernels (fa_fwd.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Kernel arguments, passed by value.
struct FwdArgs {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;
    int32_t N;      // keys = queries per (batch, head) slice
    int32_t n_qblk; // query blocks per slice: ceil(N / kQueryBlock)
    float c;        // |scale| * log2(e): scores enter exp2 through one FMA
    uint32_t qneg;  // sign-bit mask XORed onto Q words when scale < 0 (0 otherwise)
};

// Query rows per workgroup for every path (8 waves x 32 rows).
constexpr int kQueryBlock = 256;

// Enqueue the forward pass; arguments are already validated.
hipError_t launch_fwd(int dtype, int D, bool causal, int64_t BH, const FwdArgs &args,
                      hipStream_t stream);

} // namespace fa
