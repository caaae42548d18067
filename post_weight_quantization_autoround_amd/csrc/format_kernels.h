// Tensor-level fake quantization to FP8 E4M3 and MXFP4 (format_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

struct FloatQdqArgs {
    int32_t format;            // 1 = FP8 E4M3 (per group), 2 = MXFP4 (E2M1, blocks of 32)
    const void* W; bool w_bf16;
    int64_t N, K;
    int32_t group;             // group / block size along K (a multiple of 8)
    const float* mx; const float* mn;   // zero-inclusive group range [N, K/group]
    const float* alpha;        // [N, K/group] clip factor on the group maximum, nullable (= 1)
    void* w_hat; int out_kind; // 0 none, 1 fp32, 2 bf16
    uint8_t* codes;            // [N, K] E4M3 byte / E2M1 nibble, nullable
    float* scale;              // [N, K/group], nullable
    uint8_t* zero;             // [N, K/group]: 0 (FP8) or the block scale's biased exponent (MXFP4)
};

hipError_t launch_float_qdq(const FloatQdqArgs& a, hipStream_t stream);

}  // namespace ar
