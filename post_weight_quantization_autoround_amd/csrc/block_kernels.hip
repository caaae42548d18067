// Elementwise kernels of the SwiGLU MLP block step: the gated activation of
// Llama-style MLPs, Hh = silu(A) * B with silu(a) = a / (1 + exp(-a)), and
// its backward.  The blog's block-wise tuning (sec. 3) back-propagates the
// block's output error through this activation to the gate and up weights.
// Both are bound by HBM (fp32 pre-activations in, GEMM operands out).
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
    if (out_bf16)
        hipLaunchKernelGGL(swiglu_fwd_kernel<true>, grid, dim3(256), 0, stream, At, Bt, F, ncols, ld, Hht, Hh);
    else
        hipLaunchKernelGGL(swiglu_fwd_kernel<false>, grid, dim3(256), 0, stream, At, Bt, F, ncols, ld, Hht, Hh);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* dHt, const float* At, const float* Bt, int64_t F, int64_t ncols,
                             int64_t ld, void* dAt, void* dBt, bool out_bf16, hipStream_t stream) {
    const unsigned grid = grid_1d(F * ncols);
    if (out_bf16)
        hipLaunchKernelGGL(swiglu_bwd_kernel<true>, dim3(grid), dim3(256), 0, stream, dHt, At, Bt, F, ncols, ld, dAt,
                           dBt);
    else
        hipLaunchKernelGGL(swiglu_bwd_kernel<false>, dim3(grid), dim3(256), 0, stream, dHt, At, Bt, F, ncols, ld, dAt,
                           dBt);
    return hipGetLastError();
}

hipError_t launch_narrow_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(narrow_kernel, dim3(grid_1d(n)), dim3(256), 0, stream, x, y, n);
    return hipGetLastError();
}

}  // namespace ar
