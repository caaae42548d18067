// Measured peaks of the GPU (include/ar_peaks.h): a streaming copy, a
// read-only stream and a register-only MFMA loop, each timed with HIP events.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/ar_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // eight independent 16-byte loads in flight per thread and round
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) r[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) __builtin_nontemporal_store(r[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// Read-only stream the way the GEMM main loops read their operands: global
// loads straight into LDS (global_load_lds_dwordx4), one 512-thread
// workgroup per compute unit, each streaming its own run of 64 KB pieces, two
// pieces in flight per workgroup.  Nothing reads the LDS and nothing is written.
__global__ void __launch_bounds__(512) read_lds_kernel(const uint8_t* __restrict__ src, int64_t npieces) {
    __shared__ __attribute__((aligned(1024))) char buf0[65536];
    __shared__ __attribute__((aligned(1024))) char buf1[65536];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = (int)(threadIdx.x & 63);
    // workgroup b reads the run of pieces [b * per, (b + 1) * per), then
    // the leftover pieces round-robin
    const int64_t per = npieces / gridDim.x;
    const int64_t total = per + ((int64_t)blockIdx.x < npieces - per * gridDim.x ? 1 : 0);
    int s = 0;
    for (int64_t k = 0; k < total; ++k, s ^= 1) {
        const int64_t c = k < per ? (int64_t)blockIdx.x * per + k : per * gridDim.x + blockIdx.x;
        const uint8_t* g = src + c * 65536 + wave * 8192 + lane * 16;
        char* l = (s ? buf1 : buf0) + wave * 8192;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            __builtin_amdgcn_global_load_lds((gbl_void*)(g + q * 1024), (lds_void*)(l + q * 1024), 16, 0, 0);
        // the previous piece into the other buffer has landed before that
        // buffer is filled again
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

constexpr int kChains = 4;

// Every wavefront runs `iters` rounds of kChains independent MFMAs on
// operands derived from its lane id; one float per lane is stored at the
// end so the loop cannot be removed.
__global__ void __launch_bounds__(256) mfma_loop_kernel(int32_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(0.001f * (float)(lane + j));
        b[j] = (__bf16)(0.002f * (float)(lane - j));
    }
    f32x16 acc[kChains];
    for (int c = 0; c < kChains; ++c)
        for (int j = 0; j < 16; ++j) acc[c][j] = 0.0f;
    for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
    for (int c = 0; c < kChains; ++c)
        for (int j = 0; j < 16; ++j) s += acc[c][j];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

struct Timer {
    hipStream_t s = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t init() {
        hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreate(&e0);
        if (e == hipSuccess) e = hipEventCreate(&e1);
        return e;
    }
    ~Timer() {
        if (e0) (void)hipEventDestroy(e0);
        if (e1) (void)hipEventDestroy(e1);
        if (s) (void)hipStreamDestroy(s);
    }
};

int num_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

}  // namespace

extern "C" {

int ar_peak_copy_gbs(int64_t bytes, int32_t reps, double* gbs) {
    if (!gbs || bytes <= 0 || bytes % 4096 != 0 || reps < 1) return (int)hipErrorInvalidValue;
    Timer t;
    hipError_t e = t.init();
    void *src = nullptr, *dst = nullptr;
    if (e == hipSuccess) e = hipMalloc(&src, (size_t)bytes);
    if (e == hipSuccess) e = hipMalloc(&dst, (size_t)bytes);
    if (e == hipSuccess) e = hipMemsetAsync(src, 1, (size_t)bytes, t.s);
    const int64_t n16 = bytes / 16;
    const dim3 grid((unsigned)(num_cus() * 16)), block(256);
    float ms = 0.0f;
    if (e == hipSuccess) {
        hipLaunchKernelGGL(copy16_kernel, grid, block, 0, t.s, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                           n16);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(t.e0, t.s);
    for (int32_t r = 0; r < reps && e == hipSuccess; ++r) {
        hipLaunchKernelGGL(copy16_kernel, grid, block, 0, t.s, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                           n16);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(t.e1, t.s);
    if (e == hipSuccess) e = hipEventSynchronize(t.e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.e0, t.e1);
    if (src) (void)hipFree(src);
    if (dst) (void)hipFree(dst);
    if (e != hipSuccess) return (int)e;
    *gbs = 2.0 * (double)bytes * reps / ((double)ms * 1e-3) / 1e9;
    return 0;
}

int ar_peak_read_gbs(int64_t bytes, int32_t reps, double* gbs) {
    if (!gbs || bytes <= 0 || bytes % 65536 != 0 || reps < 1) return (int)hipErrorInvalidValue;
    Timer t;
    hipError_t e = t.init();
    void* src = nullptr;
    if (e == hipSuccess) e = hipMalloc(&src, (size_t)bytes);
    if (e == hipSuccess) e = hipMemsetAsync(src, 1, (size_t)bytes, t.s);
    const int64_t npieces = bytes / 65536;
    const dim3 grid((unsigned)num_cus()), block(512);
    float ms = 0.0f;
    if (e == hipSuccess) {
        hipLaunchKernelGGL(read_lds_kernel, grid, block, 0, t.s, static_cast<const uint8_t*>(src), npieces);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(t.e0, t.s);
    for (int32_t r = 0; r < reps && e == hipSuccess; ++r) {
        hipLaunchKernelGGL(read_lds_kernel, grid, block, 0, t.s, static_cast<const uint8_t*>(src), npieces);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(t.e1, t.s);
    if (e == hipSuccess) e = hipEventSynchronize(t.e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.e0, t.e1);
    if (src) (void)hipFree(src);
    if (e != hipSuccess) return (int)e;
    *gbs = (double)bytes * reps / ((double)ms * 1e-3) / 1e9;
    return 0;
}

int ar_peak_mfma_tflops(int32_t iters, double* tflops) {
    if (!tflops || iters < 1) return (int)hipErrorInvalidValue;
    Timer t;
    hipError_t e = t.init();
    // two wavefronts per SIMD: 4 SIMDs x 2 = 8 wavefronts = 2 workgroups of 256 per CU
    const int blocks = num_cus() * 2;
    float* out = nullptr;
    if (e == hipSuccess) e = hipMalloc(&out, (size_t)blocks * 256 * sizeof(float));
    float ms = 0.0f;
    if (e == hipSuccess) {
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, t.s, iters < 64 ? iters : 64, out);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(t.e0, t.s);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, t.s, iters, out);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(t.e1, t.s);
    if (e == hipSuccess) e = hipEventSynchronize(t.e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.e0, t.e1);
    if (out) (void)hipFree(out);
    if (e != hipSuccess) return (int)e;
    const double waves = (double)blocks * 4.0;
    const double flops = waves * (double)iters * kChains * (32.0 * 32.0 * 16.0 * 2.0);
    *tflops = flops / ((double)ms * 1e-3) / 1e12;
    return 0;
}

}  // extern "C"
