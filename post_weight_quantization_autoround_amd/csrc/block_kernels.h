// Elementwise kernels of the SwiGLU MLP block step (block_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

// Gated activation Hh = silu(A) * B from the pre-activations A^T, B^T
// (fp32 [F, ld], columns [0, ncols)); writes Hh^T [F, ld] and Hh [ncols, F]
// (ld F) in fp32 or, with out_bf16, their bf16 rounding.
hipError_t launch_swiglu_fwd(const float* At, const float* Bt, int64_t F, int64_t ncols, int64_t ld, void* Hht,
                             void* Hh, bool out_bf16, hipStream_t stream);
// Backward of the gated activation: dA = dHh * B * silu'(A), dB = dHh * silu(A),
// all [F, ld] (columns [0, ncols)), outputs fp32 or bf16.
hipError_t launch_swiglu_bwd(const float* dHt, const float* At, const float* Bt, int64_t F, int64_t ncols,
                             int64_t ld, void* dAt, void* dBt, bool out_bf16, hipStream_t stream);
// launch_swiglu_bwd in bf16 that also writes [dA dB] [ncols, 2F] (row
// stride 2F, dA in columns [0, F), dB in [F, 2F)).  F, ncols and ld
// multiples of 8 and 16-byte aligned pointers, else hipErrorInvalidValue.
hipError_t launch_swiglu_bwd_ab(const float* dHt, const float* At, const float* Bt, int64_t F, int64_t ncols,
                                int64_t ld, uint16_t* dAt, uint16_t* dBt, uint16_t* dAB, hipStream_t stream);
// y[i] = bf16(x[i]) (round to nearest even), n elements.
hipError_t launch_narrow_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream);

}  // namespace ar
