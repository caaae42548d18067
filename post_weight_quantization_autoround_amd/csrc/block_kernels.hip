// Elementwise kernels of the SwiGLU MLP block step: the gated activation of
// Llama-style MLPs, Hh = silu(A) * B with silu(a) = a / (1 + exp(-a)), and
// its backward.  The blog's block-wise tuning (sec. 3) back-propagates the
// block's output error through this activation to the gate and up weights.
// Both are bound by HBM (fp32 pre-activations in, GEMM operands out).
#include <initializer_list>

#include "ar_internal.h"
#include "block_kernels.h"

namespace ar {
namespace {

constexpr int kTile = 64;

template <bool BF16>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
    if constexpr (BF16)
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else
        static_cast<float*>(p)[i] = v;
}

// 64 x 64 tile (features f x columns m): read and write Hh^T along m, then
// write Hh along f from an LDS copy of the tile.
template <bool BF16>
__global__ void __launch_bounds__(256) swiglu_fwd_kernel(const float* __restrict__ At, const float* __restrict__ Bt,
                                                         int64_t F, int64_t ncols, int64_t ld, void* Hht, void* Hh) {
    __shared__ float tile[kTile][kTile + 1];
    const int64_t m0 = (int64_t)blockIdx.x * kTile, f0 = (int64_t)blockIdx.y * kTile;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < kTile; r += 4) {
        const int64_t f = f0 + r, m = m0 + tx;
        float h = 0.0f;
        if (f < F && m < ncols) {
            const float a = At[f * ld + m], b = Bt[f * ld + m];
            h = a / (1.0f + expf(-a)) * b;
            store_elem<BF16>(Hht, f * ld + m, h);
        }
        tile[r][tx] = h;
    }
    __syncthreads();
    for (int r = ty; r < kTile; r += 4) {
        const int64_t m = m0 + r, f = f0 + tx;
        if (f < F && m < ncols) store_elem<BF16>(Hh, m * F + f, tile[tx][r]);
    }
}

template <bool BF16>
__global__ void __launch_bounds__(256) swiglu_bwd_kernel(const float* __restrict__ dHt, const float* __restrict__ At,
                                                         const float* __restrict__ Bt, int64_t F, int64_t ncols,
                                                         int64_t ld, void* dAt, void* dBt) {
    const int64_t total = F * ncols;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t f = i / ncols, m = i - f * ncols, o = f * ld + m;
        const float a = At[o], b = Bt[o], dh = dHt[o];
        const float sg = 1.0f / (1.0f + expf(-a));
        store_elem<BF16>(dAt, o, dh * b * (sg * (1.0f + a * (1.0f - sg))));
        store_elem<BF16>(dBt, o, dh * (a * sg));
    }
}

// 16-byte forms for bf16 outputs (F, ncols and ld multiples of 8, 16-byte
// aligned rows): 8 consecutive columns per thread, the transposed tile
// leaves as 16-byte pieces of 8 features.  Same arithmetic per element.
typedef uint32_t vu32x4 __attribute__((ext_vector_type(4)));
typedef float vf32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void ld8f(const float* p, float v[8]) {
    const vf32x4 a = *reinterpret_cast<const vf32x4*>(p), b = *reinterpret_cast<const vf32x4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ vu32x4 pack8h(const float v[8]) {
    return vu32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}

__global__ void __launch_bounds__(256) swiglu_fwd_vec_kernel(const float* __restrict__ At,
                                                             const float* __restrict__ Bt, int64_t F, int64_t ncols,
                                                             int64_t ld, uint16_t* Hht, uint16_t* Hh) {
    constexpr int P = kTile + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Tr[kTile * P];   // [f][m]
    const int64_t m0 = (int64_t)blockIdx.x * kTile, f0 = (int64_t)blockIdx.y * kTile;
#pragma unroll
    for (int it = 0; it < kTile * kTile / 8 / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int r = p / 8, g = p % 8;
        const int64_t f = f0 + r, m = m0 + 8 * g;
        vu32x4 u = {0u, 0u, 0u, 0u};
        if (f < F && m < ncols) {
            float a8[8], b8[8], h8[8];
            ld8f(At + f * ld + m, a8);
            ld8f(Bt + f * ld + m, b8);
#pragma unroll
            for (int e = 0; e < 8; ++e) h8[e] = a8[e] / (1.0f + expf(-a8[e])) * b8[e];
            u = pack8h(h8);
            *reinterpret_cast<vu32x4*>(Hht + f * ld + m) = u;
        }
        *reinterpret_cast<vu32x4*>(Tr + r * P + 8 * g) = u;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kTile * kTile / 8 / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int mm = p / 8, g = p % 8;
        const int64_t m = m0 + mm, f = f0 + 8 * g;
        if (m < ncols && f < F) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)Tr[(8 * g + 2 * e) * P + mm] | ((uint32_t)Tr[(8 * g + 2 * e + 1) * P + mm] << 16);
            *reinterpret_cast<vu32x4*>(Hh + m * F + f) = vu32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

// dA, dB of 8 consecutive elements at offset o of the [F, ld] layouts, bf16
__device__ __forceinline__ void swiglu_bwd8(const float* __restrict__ dHt, const float* __restrict__ At,
                                            const float* __restrict__ Bt, int64_t o, vu32x4& ua, vu32x4& ub) {
    float a8[8], b8[8], d8[8], ga[8], gb[8];
    ld8f(At + o, a8);
    ld8f(Bt + o, b8);
    ld8f(dHt + o, d8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float sg = 1.0f / (1.0f + expf(-a8[e]));
        ga[e] = d8[e] * b8[e] * (sg * (1.0f + a8[e] * (1.0f - sg)));
        gb[e] = d8[e] * (a8[e] * sg);
    }
    ua = pack8h(ga);
    ub = pack8h(gb);
}

// one feature row per blockIdx.y, 8 consecutive columns per thread
__global__ void __launch_bounds__(256) swiglu_bwd_vec_kernel(const float* __restrict__ dHt,
                                                             const float* __restrict__ At,
                                                             const float* __restrict__ Bt, int64_t ncols, int64_t ld,
                                                             uint16_t* dAt, uint16_t* dBt) {
    const int64_t f = blockIdx.y;
    for (int64_t m = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; m < ncols; m += (int64_t)gridDim.x * 256 * 8) {
        const int64_t o = f * ld + m;
        vu32x4 ua, ub;
        swiglu_bwd8(dHt, At, Bt, o, ua, ub);
        *reinterpret_cast<vu32x4*>(dAt + o) = ua;
        *reinterpret_cast<vu32x4*>(dBt + o) = ub;
    }
}

// swiglu_bwd_vec_kernel on 64 x 64 tiles (features f, columns m) that also
// writes [dA dB] [ncols, 2F] row-major, the operand of the decoder's dh2
// GEMM, through a transpose of the tile in LDS: 16-byte pieces both ways.
__global__ void __launch_bounds__(256) swiglu_bwd_ab_kernel(const float* __restrict__ dHt,
                                                            const float* __restrict__ At,
                                                            const float* __restrict__ Bt, int64_t F, int64_t ncols,
                                                            int64_t ld, uint16_t* dAt, uint16_t* dBt,
                                                            uint16_t* dAB) {
    constexpr int P = kTile + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Ta[kTile * P];   // [f][m]
    __shared__ __attribute__((aligned(16))) uint16_t Tb[kTile * P];
    const int64_t m0 = (int64_t)blockIdx.x * kTile, f0 = (int64_t)blockIdx.y * kTile;
#pragma unroll
    for (int it = 0; it < kTile * kTile / 8 / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int r = p / 8, g = p % 8;
        const int64_t f = f0 + r, m = m0 + 8 * g;
        vu32x4 ua = {0u, 0u, 0u, 0u}, ub = {0u, 0u, 0u, 0u};
        if (f < F && m < ncols) {
            swiglu_bwd8(dHt, At, Bt, f * ld + m, ua, ub);
            *reinterpret_cast<vu32x4*>(dAt + f * ld + m) = ua;
            *reinterpret_cast<vu32x4*>(dBt + f * ld + m) = ub;
        }
        *reinterpret_cast<vu32x4*>(Ta + r * P + 8 * g) = ua;
        *reinterpret_cast<vu32x4*>(Tb + r * P + 8 * g) = ub;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kTile * kTile / 8 / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int mm = p / 8, g = p % 8;
        const int64_t m = m0 + mm, f = f0 + 8 * g;
        if (m < ncols && f < F) {
            uint32_t wa[4], wb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wa[e] = (uint32_t)Ta[(8 * g + 2 * e) * P + mm] | ((uint32_t)Ta[(8 * g + 2 * e + 1) * P + mm] << 16);
                wb[e] = (uint32_t)Tb[(8 * g + 2 * e) * P + mm] | ((uint32_t)Tb[(8 * g + 2 * e + 1) * P + mm] << 16);
            }
            *reinterpret_cast<vu32x4*>(dAB + m * 2 * F + f) = vu32x4{wa[0], wa[1], wa[2], wa[3]};
            *reinterpret_cast<vu32x4*>(dAB + m * 2 * F + F + f) = vu32x4{wb[0], wb[1], wb[2], wb[3]};
        }
    }
}

bool vec_ok(int64_t F, int64_t ncols, int64_t ld, std::initializer_list<const void*> ptrs) {
    if (F % 8 || ncols % 8 || ld % 8) return false;
    for (const void* q : ptrs)
        if (reinterpret_cast<uintptr_t>(q) % 16) return false;
    return true;
}

__global__ void narrow_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) y[i] = f32_to_bf16(x[i]);
}

unsigned grid_1d(int64_t n) {
    int64_t b = (n + 1023) / 1024;
    if (b > 16384) b = 16384;
    return (unsigned)(b > 0 ? b : 1);
}

}  // namespace

hipError_t launch_swiglu_fwd(const float* At, const float* Bt, int64_t F, int64_t ncols, int64_t ld, void* Hht,
                             void* Hh, bool out_bf16, hipStream_t stream) {
    const dim3 grid((unsigned)((ncols + kTile - 1) / kTile), (unsigned)((F + kTile - 1) / kTile));
    if (out_bf16 && vec_ok(F, ncols, ld, {At, Bt, Hht, Hh}))
        hipLaunchKernelGGL(swiglu_fwd_vec_kernel, grid, dim3(256), 0, stream, At, Bt, F, ncols, ld,
                           static_cast<uint16_t*>(Hht), static_cast<uint16_t*>(Hh));
    else if (out_bf16)
        hipLaunchKernelGGL(swiglu_fwd_kernel<true>, grid, dim3(256), 0, stream, At, Bt, F, ncols, ld, Hht, Hh);
    else
        hipLaunchKernelGGL(swiglu_fwd_kernel<false>, grid, dim3(256), 0, stream, At, Bt, F, ncols, ld, Hht, Hh);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* dHt, const float* At, const float* Bt, int64_t F, int64_t ncols,
                             int64_t ld, void* dAt, void* dBt, bool out_bf16, hipStream_t stream) {
    if (out_bf16 && F <= 65535 && vec_ok(F, ncols, ld, {dHt, At, Bt, dAt, dBt})) {
        int64_t gx = (ncols + 256 * 8 - 1) / (256 * 8);
        if (gx > 64) gx = 64;
        hipLaunchKernelGGL(swiglu_bwd_vec_kernel, dim3((unsigned)gx, (unsigned)F), dim3(256), 0, stream, dHt, At, Bt,
                           ncols, ld, static_cast<uint16_t*>(dAt), static_cast<uint16_t*>(dBt));
        return hipGetLastError();
    }
    const unsigned grid = grid_1d(F * ncols);
    if (out_bf16)
        hipLaunchKernelGGL(swiglu_bwd_kernel<true>, dim3(grid), dim3(256), 0, stream, dHt, At, Bt, F, ncols, ld, dAt,
                           dBt);
    else
        hipLaunchKernelGGL(swiglu_bwd_kernel<false>, dim3(grid), dim3(256), 0, stream, dHt, At, Bt, F, ncols, ld, dAt,
                           dBt);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd_ab(const float* dHt, const float* At, const float* Bt, int64_t F, int64_t ncols,
                                int64_t ld, uint16_t* dAt, uint16_t* dBt, uint16_t* dAB, hipStream_t stream) {
    if (!vec_ok(F, ncols, ld, {dHt, At, Bt, dAt, dBt, dAB})) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((ncols + kTile - 1) / kTile), (unsigned)((F + kTile - 1) / kTile));
    hipLaunchKernelGGL(swiglu_bwd_ab_kernel, grid, dim3(256), 0, stream, dHt, At, Bt, F, ncols, ld, dAt, dBt, dAB);
    return hipGetLastError();
}

hipError_t launch_narrow_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(narrow_kernel, dim3(grid_1d(n)), dim3(256), 0, stream, x, y, n);
    return hipGetLastError();
}

}  // namespace ar
