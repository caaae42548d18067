// Fake quantizer, INT4 packing and data-preparation kernels (gfx950).
//
// The quantizer follows the AutoRound blog (sec. 2 "Essence": a scale from
// the range, then rounding to the integer grid; sec. 3: a per-weight offset
// v added before rounding and per-group clip bounds; sec. 4: zero-point added
// after rounding, q = round(w/s) + z clamped to [0, 15], w^ = (q - z) s).
// All arithmetic is fp32 in a fixed order with IEEE division and
// round-half-to-even; the library is built without FMA contraction so the
// codes are reproducible bit for bit.
//
// These kernels stream HBM: one thread handles 8 consecutive weights of a row
// (one 16-byte bf16 load or two 16-byte fp32 loads), so each wavefront moves
// contiguous 1-2 KiB per access.  Groups are multiples of 8, so a thread's 8
// weights share one group's scale and zero-point.
#include "ar_internal.h"

namespace ar {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8(const void* W, bool bf16, int64_t idx, float w[8]) {
    if (bf16) {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + idx);
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = __uint_as_float(p[i] << 16);
            w[2 * i + 1] = __uint_as_float(p[i] & 0xFFFF0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx + 4);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
}

__global__ void __launch_bounds__(kThreads) group_range_kernel(const void* __restrict__ W, bool bf16,
                                                               int64_t ngroups, int32_t g,
                                                               float* __restrict__ mx, float* __restrict__ mn) {
    // One wavefront per group; lanes stride over the group's g weights.
    const int lane = threadIdx.x & 63;
    const int64_t grp = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (grp >= ngroups) return;
    const int64_t base = grp * g;
    float hi = 0.0f, lo = 0.0f;     // the range always contains 0
    for (int32_t e = lane; e < g; e += 64) {
        const float v = bf16 ? bf16_to_f32(static_cast<const uint16_t*>(W)[base + e])
                             : static_cast<const float*>(W)[base + e];
        hi = fmaxf(hi, v);
        lo = fminf(lo, v);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        hi = fmaxf(hi, __shfl_xor(hi, off, 64));
        lo = fminf(lo, __shfl_xor(lo, off, 64));
    }
    if (lane == 0) {
        mx[grp] = hi;
        mn[grp] = lo;
    }
}

__global__ void __launch_bounds__(kThreads) qdq_kernel(QdqArgs a) {
    if (a.state && a.state->halted) return;
    const int64_t chunks_per_row = a.K >> 3;
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= a.N * chunks_per_row) return;
    const int64_t n = c / chunks_per_row;
    const int64_t k0 = (c - n * chunks_per_row) << 3;
    const int64_t G = a.K / a.qp.group;
    const int64_t gi = n * G + k0 / a.qp.group;
    const int buf = a.state ? a.state->cur : 0;
    const float* V = a.V[buf];
    const float al = a.alpha[buf] ? a.alpha[buf][gi] : 1.0f;
    const float be = a.beta[buf] ? a.beta[buf][gi] : 1.0f;
    const float Q = a.qp.qmax;
    const GroupQ gq = group_quant(a.mx[gi], a.mn[gi], al, be, a.qp);

    const int64_t idx = n * a.K + k0;
    float w[8], v[8];
    load8(a.W, a.w_bf16, idx, w);
    if (V) {
        const float4 v0 = *reinterpret_cast<const float4*>(V + idx);
        const float4 v1 = *reinterpret_cast<const float4*>(V + idx + 4);
        v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
        v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float q[8], wh[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float t;
        q[i] = quant_code(w[i], v[i], gq, Q, t);
        wh[i] = gq.s * (q[i] - gq.z);
    }
    if (a.out_kind == 1) {
        float* o = static_cast<float*>(a.w_hat) + idx;
        *reinterpret_cast<float4*>(o) = make_float4(wh[0], wh[1], wh[2], wh[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(wh[4], wh[5], wh[6], wh[7]);
    } else if (a.out_kind == 3) {
        // w^ - W in fp32: the rounding error the loss measures, formed before
        // any product (half an ulp of the difference at most)
        float* o = static_cast<float*>(a.w_hat) + idx;
        *reinterpret_cast<float4*>(o) = make_float4(wh[0] - w[0], wh[1] - w[1], wh[2] - w[2], wh[3] - w[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(wh[4] - w[4], wh[5] - w[5], wh[6] - w[6], wh[7] - w[7]);
    } else if (a.out_kind == 2) {
        uint4 o;
        o.x = pack_bf16x2(wh[0], wh[1]);
        o.y = pack_bf16x2(wh[2], wh[3]);
        o.z = pack_bf16x2(wh[4], wh[5]);
        o.w = pack_bf16x2(wh[6], wh[7]);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.w_hat) + idx) = o;
    }
    if (a.codes) {
        uint2 o;
        o.x = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
        o.y = (uint32_t)q[4] | ((uint32_t)q[5] << 8) | ((uint32_t)q[6] << 16) | ((uint32_t)q[7] << 24);
        *reinterpret_cast<uint2*>(a.codes + idx) = o;
    }
    if (a.packed) {
        uint32_t p = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) p |= ((uint32_t)q[i] & 0xFu) << (4 * i);
        *reinterpret_cast<uint32_t*>(a.packed + (idx >> 1)) = p;
    }
    if ((k0 % a.qp.group) == 0) {
        if (a.scale) a.scale[gi] = gq.s;
        if (a.zero) a.zero[gi] = (uint8_t)gq.z;
    }
}

__global__ void __launch_bounds__(kThreads) nonfinite_kernel(const void* __restrict__ x, bool bf16, int64_t n,
                                                             int32_t* flag) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    bool bad = false;
    if (bf16) {
        const uint16_t* p = static_cast<const uint16_t*>(x);
        for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
            bad |= (p[i] & 0x7F80u) == 0x7F80u;
    } else {
        const uint32_t* p = static_cast<const uint32_t*>(x);
        for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
            bad |= (p[i] & 0x7F800000u) == 0x7F800000u;
    }
    if (bad) atomicOr(flag, 1);
}

template <typename T>
__global__ void __launch_bounds__(kThreads) transpose_pool_kernel(const T* __restrict__ x, T* __restrict__ xt,
                                                                  int64_t T_, int64_t K) {
    // 64 x 64 tile of one sample: read along k, write along t.
    __shared__ T tile[64][65];
    const int64_t s = blockIdx.z;
    const int64_t k0 = (int64_t)blockIdx.x * 64;
    const int64_t t0 = (int64_t)blockIdx.y * 64;
    const T* src = x + s * T_ * K;
    T* dst = xt + s * T_ * K;
    const int tx = threadIdx.x & 63;
    const int ty = threadIdx.x >> 6;   // 0..3
    for (int r = ty; r < 64; r += 4) {
        const int64_t t = t0 + r, k = k0 + tx;
        if (t < T_ && k < K) tile[r][tx] = src[t * K + k];
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t k = k0 + r, t = t0 + tx;
        if (t < T_ && k < K) dst[k * T_ + t] = tile[tx][r];
    }
}

// 16-bit transpose with 16-byte accesses: dst[b][c][r] = src[b][r][c] for
// r < rows, c < cols, one 64 x 64 tile per workgroup.  Each thread loads two
// 8-element row vectors (8 threads cover one 128-byte tile row) and stores
// two 8-element vectors of the transposed tile.  Needs rows, cols, lds, ldd
// multiples of 8 and 16-byte aligned bases (the launcher checks).
constexpr int kStrip = 4;   // 64 x 64 tiles per workgroup, along the columns

__global__ void __launch_bounds__(kThreads) transpose_b16_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                                 int64_t sst, uint16_t* __restrict__ dst,
                                                                 int64_t ldd, int64_t dstr, int64_t rows,
                                                                 int64_t cols) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
    const int64_t b = blockIdx.z;
    const int64_t cbase = (int64_t)blockIdx.x * 64 * kStrip, r0 = (int64_t)blockIdx.y * 64;
    src += b * sst;
    dst += b * dstr;
    const int v8 = threadIdx.x & 7, vr = threadIdx.x >> 3;   // vr 0..31 for 256 threads
    uint4 v[2];
    auto load = [&](int64_t c0) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int64_t r = r0 + vr + pass * 32, c = c0 + v8 * 8;
            v[pass] = (r < rows && c < cols) ? *reinterpret_cast<const uint4*>(src + r * lds + c)
                                             : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    load(cbase);
    for (int st = 0; st < kStrip; ++st) {
        const int64_t c0 = cbase + 64 * st;
        if (c0 >= cols) break;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) *reinterpret_cast<uint4*>(&tile[vr + pass * 32][v8 * 8]) = v[pass];
        __syncthreads();
        if (st + 1 < kStrip && c0 + 64 < cols) load(c0 + 64);   // in flight during the stores below
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int oc = vr + pass * 32;
            const int64_t c = c0 + oc, r = r0 + v8 * 8;
            if (c < cols && r < rows) {
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[i] = (uint32_t)tile[v8 * 8 + 2 * i][oc] | ((uint32_t)tile[v8 * 8 + 2 * i + 1][oc] << 16);
                *reinterpret_cast<uint4*>(dst + c * ldd + r) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        __syncthreads();
    }
}

__global__ void widen_kernel(const uint16_t* __restrict__ x, float* __restrict__ y, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) y[i] = bf16_to_f32(x[i]);
}

__global__ void fill_kernel(float* __restrict__ p, float v, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

__global__ void copy_kernel(float* __restrict__ d, const float* __restrict__ s, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) d[i] = s[i];
}

__global__ void state_init_kernel(StepState* s, int32_t step0, double best0) {
    s->step = step0;
    s->cur = 0;
    s->src = 0;
    s->dst = 0;
    s->best_idx = -1;
    s->best_step = -1;
    s->halted = 0;
    s->t_eval = 0;
    s->best_loss = best0;
}

int grid_for(int64_t n, int per_block, int cap) {
    int64_t b = (n + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

}  // namespace

hipError_t launch_group_range(const void* W, bool w_bf16, int64_t N, int64_t K, int32_t g, float* mx, float* mn,
                              hipStream_t stream) {
    const int64_t ngroups = N * (K / g);
    const int blocks = (int)((ngroups + (kThreads / 64) - 1) / (kThreads / 64));
    hipLaunchKernelGGL(group_range_kernel, dim3(blocks), dim3(kThreads), 0, stream, W, w_bf16, ngroups, g, mx, mn);
    return hipGetLastError();
}

hipError_t launch_qdq(const QdqArgs& a, hipStream_t stream) {
    const int64_t chunks = a.N * (a.K >> 3);
    const int blocks = (int)((chunks + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(qdq_kernel, dim3(blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_nonfinite_scan(const void* x, bool bf16, int64_t n, int32_t* flag, hipStream_t stream) {
    hipLaunchKernelGGL(nonfinite_kernel, dim3(grid_for(n, kThreads * 8, 4096)), dim3(kThreads), 0, stream, x, bf16, n,
                       flag);
    return hipGetLastError();
}

bool transpose_b16_fits(const void* src, int64_t lds, const void* dst, int64_t ldd, int64_t rows, int64_t cols) {
    return rows % 8 == 0 && cols % 8 == 0 && lds % 8 == 0 && ldd % 8 == 0 &&
           reinterpret_cast<uintptr_t>(src) % 16 == 0 && reinterpret_cast<uintptr_t>(dst) % 16 == 0;
}

hipError_t launch_transpose_b16(const uint16_t* src, int64_t lds, int64_t sst, uint16_t* dst, int64_t ldd,
                                int64_t dstr, int64_t rows, int64_t cols, int64_t batch, hipStream_t stream) {
    const dim3 grid((unsigned)((cols + 64 * kStrip - 1) / (64 * kStrip)), (unsigned)((rows + 63) / 64),
                    (unsigned)batch);
    hipLaunchKernelGGL(transpose_b16_kernel, grid, dim3(kThreads), 0, stream, src, lds, sst, dst, ldd, dstr, rows,
                       cols);
    return hipGetLastError();
}

hipError_t launch_transpose_pool(const void* x, void* xt, int elem_bytes, int64_t S, int64_t T, int64_t K,
                                 hipStream_t stream) {
    dim3 grid((unsigned)((K + 63) / 64), (unsigned)((T + 63) / 64), (unsigned)S);
    if (elem_bytes == 2 && transpose_b16_fits(x, K, xt, T, T, K))
        return launch_transpose_b16(static_cast<const uint16_t*>(x), K, T * K, static_cast<uint16_t*>(xt), T, T * K,
                                    T, K, S, stream);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(transpose_pool_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(x), static_cast<uint16_t*>(xt), T, K);
    else
        hipLaunchKernelGGL(transpose_pool_kernel<float>, grid, dim3(kThreads), 0, stream,
                           static_cast<const float*>(x), static_cast<float*>(xt), T, K);
    return hipGetLastError();
}

hipError_t launch_widen_bf16(const uint16_t* x, float* y, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(widen_kernel, dim3(grid_for(n, kThreads * 4, 8192)), dim3(kThreads), 0, stream, x, y, n);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n, kThreads * 4, 8192)), dim3(kThreads), 0, stream, p, v, n);
    return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n, kThreads * 4, 8192)), dim3(kThreads), 0, stream, dst, src, n);
    return hipGetLastError();
}

hipError_t launch_state_init(StepState* s, int32_t step0, double best0, hipStream_t stream) {
    hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(1), 0, stream, s, step0, best0);
    return hipGetLastError();
}

}  // namespace ar
