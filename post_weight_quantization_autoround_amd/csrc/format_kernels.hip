// Tensor-level fake quantization to low-bit float formats: the AutoRound
// blog (sec. 4, "data-type decoupling") evaluates a new data type such as
// FP8 or MXFP4 by registering a tensor-level QDQ function for it.
//   FP8 E4M3 : per group, s = alpha * max|W_g| / 448 (1 for an all-zero
//              group), code = E4M3 value of W/s, w^ = s * code;
//   MXFP4    : blocks of 32 along K share s = 2^e, e = floor(log2(alpha *
//              max|W_b|)) - 2, elements are E2M1 values of W/s, w^ = s * code.
// Rounding is to the nearest value of the format, ties to the even code,
// saturating at the largest finite magnitude (448, 6).  On the grid this is
// rint(|x| / step) * step with step the spacing of x's binade (a power of
// two, so both operations are exact), which puts ties on even multiples,
// i.e. even mantissa codes.
#include "ar_internal.h"
#include "format_kernels.h"

namespace ar {
namespace {

constexpr int kThreads = 256;

// floor(log2(a)) for finite a > 0 (exact, from the exponent)
__device__ __forceinline__ int ilog2f(float a) {
    int k;
    (void)frexpf(a, &k);   // a = m 2^k, m in [0.5, 1)
    return k - 1;
}

// E4M3: returns the rounded value, *code = sign | exponent field | mantissa
__device__ __forceinline__ float e4m3_round(float x, uint32_t* code) {
    const float a = __builtin_fabsf(x);
    float v;
    if (a >= 448.0f) {
        v = 448.0f;
    } else if (a == 0.0f) {
        v = 0.0f;
    } else {
        const int e = ilog2f(a) > -6 ? ilog2f(a) : -6;
        const float step = ldexpf(1.0f, e - 3);
        v = __builtin_rintf(a / step) * step;
    }
    uint32_t c = 0;
    if (v > 0.0f) {
        const int k = ilog2f(v);
        if (k < -6) c = (uint32_t)(v * 512.0f);                                   // subnormal: m 2^-9
        else c = ((uint32_t)(k + 7) << 3) | (uint32_t)(ldexpf(v, -k) * 8.0f - 8.0f);
    }
    const bool neg = __builtin_signbit(x) && v != 0.0f;
    *code = c | (neg ? 0x80u : 0u);
    return neg ? -v : v;
}

// E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
__device__ __forceinline__ float e2m1_round(float x, uint32_t* code) {
    const float a = __builtin_fabsf(x);
    float v;
    if (a >= 6.0f) {
        v = 6.0f;
    } else {
        const float step = a < 2.0f ? 0.5f : ldexpf(1.0f, ilog2f(a) - 1);
        v = __builtin_rintf(a / step) * step;
    }
    uint32_t c = 0;
    if (v >= 1.0f) {
        const int k = ilog2f(v);
        c = ((uint32_t)(k + 1) << 1) | (uint32_t)(ldexpf(v, -k) * 2.0f - 2.0f);
    } else if (v > 0.0f) {
        c = 1;
    }
    const bool neg = __builtin_signbit(x) && v != 0.0f;
    *code = c | (neg ? 0x8u : 0u);
    return neg ? -v : v;
}

template <int FMT>
__global__ void __launch_bounds__(kThreads) float_qdq_kernel(FloatQdqArgs a) {
    const int64_t chunks_per_row = a.K >> 3;
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= a.N * chunks_per_row) return;
    const int64_t n = c / chunks_per_row;
    const int64_t k0 = (c - n * chunks_per_row) << 3;
    const int64_t G = a.K / a.group;
    const int64_t gi = n * G + k0 / a.group;
    const float al = a.alpha ? a.alpha[gi] : 1.0f;
    const float amax = al * fmaxf(a.mx[gi], -a.mn[gi]);
    float s;
    uint32_t sbits = 0;
    if (FMT == 1) {
        s = amax == 0.0f ? 1.0f : amax / 448.0f;
    } else {
        const int e = amax == 0.0f ? 0 : ilog2f(amax) - 2;
        s = ldexpf(1.0f, e);
        sbits = (uint32_t)(e + 127);
    }
    const int64_t idx = n * a.K + k0;
    float wh[8];
    uint32_t cd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float w = a.w_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.W)[idx + i])
                                 : static_cast<const float*>(a.W)[idx + i];
        const float x = w / s;
        const float v = FMT == 1 ? e4m3_round(x, &cd[i]) : e2m1_round(x, &cd[i]);
        wh[i] = s * v;
    }
    if (a.out_kind == 1) {
        float* o = static_cast<float*>(a.w_hat) + idx;
        *reinterpret_cast<float4*>(o) = make_float4(wh[0], wh[1], wh[2], wh[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(wh[4], wh[5], wh[6], wh[7]);
    } else if (a.out_kind == 2) {
        uint16_t* o = static_cast<uint16_t*>(a.w_hat) + idx;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = f32_to_bf16(wh[i]);
    }
    if (a.codes) {
#pragma unroll
        for (int i = 0; i < 8; ++i) a.codes[idx + i] = (uint8_t)cd[i];
    }
    if ((k0 % a.group) == 0) {
        if (a.scale) a.scale[gi] = s;
        if (a.zero) a.zero[gi] = (uint8_t)sbits;
    }
}

}  // namespace

hipError_t launch_float_qdq(const FloatQdqArgs& a, hipStream_t stream) {
    const int64_t chunks = a.N * (a.K >> 3);
    const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads));
    if (a.format == 1)
        hipLaunchKernelGGL(float_qdq_kernel<1>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(float_qdq_kernel<2>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ar
