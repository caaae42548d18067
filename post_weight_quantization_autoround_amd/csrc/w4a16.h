// Launch interface of the INT4-weight GEMM (w4a16_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

struct W4A16Args {
    const uint16_t* X;        // bf16 [M, ldx], rows 16-byte aligned
    int64_t ldx;
    int64_t M, N, K;          // K a multiple of 64
    const uint32_t* packed;   // [N, K/8] dwords = [N, K/2] bytes, low nibble = even k
    const float* scale;       // [N, G]
    const uint8_t* zero;      // [N, G]
    int32_t g;                // group size, a multiple of 8 dividing K
    int64_t G;                // K / g
    void* Y;                  // [M, ldy] fp32 or bf16
    int64_t ldy;
    bool y_bf16;
};

hipError_t launch_w4a16_gemm(const W4A16Args& a, hipStream_t stream);

}  // namespace ar
