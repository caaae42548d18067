// Kernels of the Llama decoder block step: RMSNorm forward/backward with the
// residual, the rotary embedding, causal softmax attention and its backward,
// and the layout moves around them.  The block-wise tuning of the AutoRound
// blog (sec. 3) back-propagates the block output's error through all of
// these to the seven quantized linears.
//
// Attention runs per sample (T <= 256 tokens) and head on
// v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16 and k-chunk l / 16 of
// the A and B tiles; accumulator r of lane l is row 4 (l / 16) + r, column
// l % 16.  A wavefront owns 16 query rows (forward, dQ) or 16 key rows (dK,
// dV); a row's scores live in registers, P and dS pass through the
// wavefront's own LDS rows to become A operands.  The backward is two kernels
// (dQ over query blocks, dK/dV over key blocks with the GQA heads of a group
// summed in order), so nothing is accumulated atomically and results are
// deterministic.
#include <cmath>

#include "decoder_kernels.h"

namespace ar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t map_row(const RowMap& mp, int64_t m) {
    if (!mp.sched) return m;
    int64_t row = 0;
    if (mp.state) row = mp.after_decide ? mp.state->t_eval : mp.state->step;
    const int32_t* ids = mp.sched + row * mp.nseg;
    return (int64_t)ids[m / mp.T] * mp.T + m % mp.T;
}

__device__ __forceinline__ float load_elem(const void* p, bool bf16, int64_t i) {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_elem(void* p, bool bf16, int64_t i, float v) {
    if (bf16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else static_cast<float*>(p)[i] = v;
}

__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float t = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return t;
}

__global__ void __launch_bounds__(256) rmsnorm_fwd_kernel(const void* x, bool x_bf16, RowMap mp, const float* add,
                                                          int64_t H, const float* w, float eps, float* h_out,
                                                          float* r_out, void* out, bool out_bf16) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const int64_t src = map_row(mp, m);
    float ss = 0.0f;
    for (int64_t c = threadIdx.x; c < H; c += 256) {
        float v = load_elem(x, x_bf16, src * H + c);
        if (add) v += add[m * H + c];
        if (h_out) h_out[m * H + c] = v;
        ss += v * v;
    }
    const float r = 1.0f / sqrtf(block_sum256(ss, red) / (float)H + eps);
    if (threadIdx.x == 0 && r_out) r_out[m] = r;
    for (int64_t c = threadIdx.x; c < H; c += 256) {
        float v = load_elem(x, x_bf16, src * H + c);
        if (add) v += add[m * H + c];
        store_elem(out, out_bf16, m * H + c, v * r * (w ? w[c] : 1.0f));
    }
}

__global__ void __launch_bounds__(256) rmsnorm_bwd_kernel(const float* dh2, const float* dh2b, const float* h,
                                                          const float* r, const float* w, const void* dy,
                                                          bool dy_bf16, int64_t H, void* dh, bool dh_bf16) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    auto g = [&](int64_t c) { return dh2b ? dh2[m * H + c] + dh2b[m * H + c] : dh2[m * H + c]; };
    float s = 0.0f;
    for (int64_t c = threadIdx.x; c < H; c += 256) s += h[m * H + c] * g(c) * (w ? w[c] : 1.0f);
    s = block_sum256(s, red);
    const float rr = r[m];
    const float coef = rr * rr * rr * s / (float)H;
    for (int64_t c = threadIdx.x; c < H; c += 256) {
        const float u = g(c) * (w ? w[c] : 1.0f);
        store_elem(dh, dh_bf16, m * H + c, load_elem(dy, dy_bf16, m * H + c) + u * rr - h[m * H + c] * coef);
    }
}

// ------------------------------------------------ 16-byte vector forms ----
// The row kernels below move 8 consecutive elements per thread and access:
// 16 bytes of bf16 or 32 bytes of fp32, so a wavefront's load or store is
// 1-2 KB of contiguous memory.
typedef uint32_t vu32x4 __attribute__((ext_vector_type(4)));
typedef float vf32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void ld8f(const float* p, float v[8]) {
    const vf32x4 a = *reinterpret_cast<const vf32x4*>(p), b = *reinterpret_cast<const vf32x4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void st8f(float* p, const float v[8]) {
    *reinterpret_cast<vf32x4*>(p) = vf32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<vf32x4*>(p + 4) = vf32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void ld8h(const uint16_t* p, float v[8]) {
    const vu32x4 u = *reinterpret_cast<const vu32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ vu32x4 pack8h(const float v[8]) {
    return vu32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}

constexpr int kRowChunks = 4;   // 8-element chunks per thread: rows of up to 256 * 8 * 4 = 8192

// rmsnorm_fwd_kernel for bf16 x and output, H % 8 == 0, H <= 8192: the row
// stays in registers between the sum of squares and the scaling.
__global__ void __launch_bounds__(256) rmsnorm_fwd_vec_kernel(const uint16_t* x, RowMap mp, const float* add,
                                                              int64_t H, const float* w, float eps, float* h_out,
                                                              float* r_out, uint16_t* out) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const int64_t src = map_row(mp, m);
    float v[kRowChunks][8];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kRowChunks; ++j) {
        const int64_t c = ((int64_t)threadIdx.x + 256 * j) * 8;
        if (c < H) {
            ld8h(x + src * H + c, v[j]);
            if (add) {
                float a8[8];
                ld8f(add + m * H + c, a8);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[j][e] += a8[e];
            }
            if (h_out) st8f(h_out + m * H + c, v[j]);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
        }
    }
    const float r = 1.0f / sqrtf(block_sum256(ss, red) / (float)H + eps);
    if (threadIdx.x == 0 && r_out) r_out[m] = r;
#pragma unroll
    for (int j = 0; j < kRowChunks; ++j) {
        const int64_t c = ((int64_t)threadIdx.x + 256 * j) * 8;
        if (c < H) {
            float w8[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
            if (w) ld8f(w + c, w8);
            float o8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = v[j][e] * r * w8[e];
            *reinterpret_cast<vu32x4*>(out + m * H + c) = pack8h(o8);
        }
    }
}

// rmsnorm_bwd_kernel for bf16 dy and dh, H % 8 == 0, H <= 8192.
__global__ void __launch_bounds__(256) rmsnorm_bwd_vec_kernel(const float* dh2, const float* dh2b, const float* h,
                                                              const float* r, const float* w, const uint16_t* dy,
                                                              int64_t H, uint16_t* dh) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    float u[kRowChunks][8], hv[kRowChunks][8];
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kRowChunks; ++j) {
        const int64_t c = ((int64_t)threadIdx.x + 256 * j) * 8;
        if (c < H) {
            ld8f(dh2 + m * H + c, u[j]);
            if (dh2b) {
                float b8[8];
                ld8f(dh2b + m * H + c, b8);
#pragma unroll
                for (int e = 0; e < 8; ++e) u[j][e] += b8[e];
            }
            ld8f(h + m * H + c, hv[j]);
            if (w) {
                float w8[8];
                ld8f(w + c, w8);
#pragma unroll
                for (int e = 0; e < 8; ++e) u[j][e] *= w8[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) s += hv[j][e] * u[j][e];
        }
    }
    s = block_sum256(s, red);
    const float rr = r[m];
    const float coef = rr * rr * rr * s / (float)H;
#pragma unroll
    for (int j = 0; j < kRowChunks; ++j) {
        const int64_t c = ((int64_t)threadIdx.x + 256 * j) * 8;
        if (c < H) {
            float d8[8];
            ld8h(dy + m * H + c, d8);
#pragma unroll
            for (int e = 0; e < 8; ++e) d8[e] = d8[e] + u[j][e] * rr - hv[j][e] * coef;
            *reinterpret_cast<vu32x4*>(dh + m * H + c) = pack8h(d8);
        }
    }
}

// yref_combine_kernel with 32-byte pieces (H, T multiples of 8, 16-byte
// aligned rows): h is read along c into the LDS tile, y and out along t.
__global__ void __launch_bounds__(256) yref_combine_vec_kernel(const float* y, RowMap mp, int64_t s0, const float* h,
                                                               int64_t H, int64_t T, float ca, float ch, float* out) {
    __shared__ float tile[64][65];   // [t][c]
    const int64_t t0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64, j = blockIdx.z;
    int64_t sj = s0 + j;
    if (mp.sched) {
        int64_t row = 0;
        if (mp.state) row = mp.after_decide ? mp.state->t_eval : mp.state->step;
        sj = mp.sched[row * mp.nseg + j];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int rr = p / 8, g = p % 8;
        const int64_t t = t0 + rr, c = c0 + 8 * g;
        float h8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (t < T && c < H) ld8f(h + (j * T + t) * H + c, h8);
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[rr][8 * g + e] = h8[e];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int cc = p / 8, g = p % 8;
        const int64_t c = c0 + cc, t = t0 + 8 * g;
        if (c < H && t < T) {
            float y8[8], o8[8];
            ld8f(y + (sj * H + c) * T + t, y8);
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = ca * y8[e] + ch * tile[8 * g + e][cc];
            st8f(out + (j * H + c) * T + t, o8);
        }
    }
}

// A 64-token x D tile of bf16 values staged row-major in LDS ([token][D + 8])
// and written transposed ([dim][token]) with 16-byte stores: each piece is 8
// tokens of one dim, read as 8 LDS halves.
template <int D>
__device__ __forceinline__ void store_tile_transposed(const uint16_t* Tr, uint16_t* dst, int64_t ld) {
    constexpr int P = D + 8;
#pragma unroll
    for (int it = 0; it < D * 8 / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int dim = p / 8, g = p % 8;
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            u[e] = (uint32_t)Tr[(8 * g + 2 * e) * P + dim] | ((uint32_t)Tr[(8 * g + 2 * e + 1) * P + dim] << 16);
        *reinterpret_cast<vu32x4*>(dst + dim * ld + 8 * g) = vu32x4{u[0], u[1], u[2], u[3]};
    }
}

// 64 x 64 tiles of (hidden c, token t) for one sample
__global__ void __launch_bounds__(256) yref_combine_kernel(const float* y, RowMap mp, int64_t s0, const float* h,
                                                           int64_t H, int64_t T, float ca, float ch, float* out) {
    __shared__ float tile[64][65];
    const int64_t t0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64, j = blockIdx.z;
    int64_t sj = s0 + j;
    if (mp.sched) {
        int64_t row = 0;
        if (mp.state) row = mp.after_decide ? mp.state->t_eval : mp.state->step;
        sj = mp.sched[row * mp.nseg + j];
    }
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int rr = ty; rr < 64; rr += 4) {
        const int64_t t = t0 + rr, c = c0 + tx;
        tile[rr][tx] = (t < T && c < H) ? h[(j * T + t) * H + c] : 0.0f;
    }
    __syncthreads();
    for (int rr = ty; rr < 64; rr += 4) {
        const int64_t c = c0 + rr, t = t0 + tx;
        if (c < H && t < T) out[(j * H + c) * T + t] = ca * y[(sj * H + c) * T + t] + ch * tile[tx][rr];
    }
}

template <typename E>
__global__ void __launch_bounds__(256) transpose2d_kernel(const E* src, int64_t lds, E* dst, int64_t ldd,
                                                          int64_t rows, int64_t cols) {
    __shared__ uint32_t tile[64][65];
    const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int rr = ty; rr < 64; rr += 4) {
        const int64_t r = r0 + rr, c = c0 + tx;
        if (r < rows && c < cols) {
            const E v = src[r * lds + c];
            uint32_t u;
            if constexpr (sizeof(E) == 2) u = v;
            else u = __float_as_uint(v);
            tile[rr][tx] = u;
        }
    }
    __syncthreads();
    for (int rr = ty; rr < 64; rr += 4) {
        const int64_t c = c0 + rr, r = r0 + tx;
        if (r < rows && c < cols) {
            const uint32_t u = tile[tx][rr];
            if constexpr (sizeof(E) == 2) dst[c * ldd + r] = (E)u;
            else dst[c * ldd + r] = __uint_as_float(u);
        }
    }
}

__global__ void add_rows_kernel(const float* a, const float* b, int64_t n, void* y, bool y_bf16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        store_elem(y, y_bf16, i, a[i] + b[i]);
}

// ---------------------------------------------------------------- RoPE ----
// Head slot hh of qkv: q heads, then k heads, then v heads.
struct HeadSlot {
    int kind;      // 0 q, 1 k, 2 v
    int head;
    int nheads;
    int64_t col0;  // column of the head in qkv
};

__device__ __forceinline__ HeadSlot head_slot(int hh, const AttnShape& s) {
    HeadSlot h;
    if (hh < s.nq) {
        h.kind = 0; h.head = hh; h.nheads = s.nq; h.col0 = (int64_t)hh * s.d;
    } else if (hh < s.nq + s.nkv) {
        h.kind = 1; h.head = hh - s.nq; h.nheads = s.nkv; h.col0 = (int64_t)s.nq * s.d + (int64_t)h.head * s.d;
    } else {
        h.kind = 2; h.head = hh - s.nq - s.nkv; h.nheads = s.nkv;
        h.col0 = (int64_t)(s.nq + s.nkv) * s.d + (int64_t)h.head * s.d;
    }
    return h;
}

template <int D>
__global__ void __launch_bounds__(256) rope_fwd_kernel(const float* qkv, const float* cosT, const float* sinT,
                                                       AttnShape s, uint16_t* q, uint16_t* qT, uint16_t* k,
                                                       uint16_t* kT, uint16_t* v, uint16_t* vT) {
    constexpr int P = D + 8, Q = D / 8;   // LDS pitch; 4-element groups per half row
    __shared__ __attribute__((aligned(16))) uint16_t Tr[64 * P];
    const int64_t t0 = (int64_t)blockIdx.x * 64, b = blockIdx.z;
    const HeadSlot hs = head_slot(blockIdx.y, s);
    const int64_t ldqkv = (int64_t)(s.nq + 2 * s.nkv) * D;
    uint16_t* rm = hs.kind == 0 ? q : (hs.kind == 1 ? k : v);
    uint16_t* tr = hs.kind == 0 ? qT : (hs.kind == 1 ? kT : vT);
    const int64_t ldo = (int64_t)hs.nheads * D;
#pragma unroll
    for (int it = 0; it < 64 * Q / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int rr = p / Q, i4 = (p % Q) * 4;
        const int64_t t = t0 + rr, m = b * s.T + t;
        const float* row = qkv + m * ldqkv + hs.col0;
        const vf32x4 a = *reinterpret_cast<const vf32x4*>(row + i4);
        const vf32x4 bb = *reinterpret_cast<const vf32x4*>(row + D / 2 + i4);
        vf32x4 ra = a, rb = bb;
        if (hs.kind < 2) {
            const vf32x4 c = *reinterpret_cast<const vf32x4*>(cosT + t * (D / 2) + i4);
            const vf32x4 sn = *reinterpret_cast<const vf32x4*>(sinT + t * (D / 2) + i4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ra[e] = a[e] * c[e] - bb[e] * sn[e];
                rb[e] = bb[e] * c[e] + a[e] * sn[e];
            }
        }
        const uint2 ua = make_uint2(pack_bf16x2(ra[0], ra[1]), pack_bf16x2(ra[2], ra[3]));
        const uint2 ub = make_uint2(pack_bf16x2(rb[0], rb[1]), pack_bf16x2(rb[2], rb[3]));
        uint16_t* orow = rm + m * ldo + (int64_t)hs.head * D;
        *reinterpret_cast<uint2*>(orow + i4) = ua;
        *reinterpret_cast<uint2*>(orow + D / 2 + i4) = ub;
        *reinterpret_cast<uint2*>(Tr + rr * P + i4) = ua;
        *reinterpret_cast<uint2*>(Tr + rr * P + D / 2 + i4) = ub;
    }
    __syncthreads();
    store_tile_transposed<D>(Tr, tr + ((b * hs.nheads + hs.head) * D) * s.T + t0, s.T);
}

template <int D>
__global__ void __launch_bounds__(256) rope_bwd_kernel(const float* dq, const float* dk, const float* dv,
                                                       int parts, int64_t part_stride, const float* cosT,
                                                       const float* sinT, AttnShape s, uint16_t* dqkvT) {
    constexpr int P = D + 8, Q = D / 8;
    __shared__ __attribute__((aligned(16))) uint16_t Tr[64 * P];
    const int64_t t0 = (int64_t)blockIdx.x * 64, b = blockIdx.z;
    const HeadSlot hs = head_slot(blockIdx.y, s);
    const float* src = hs.kind == 0 ? dq : (hs.kind == 1 ? dk : dv);
    const int64_t lds = (int64_t)hs.nheads * D;
    const int64_t M = s.B * s.T;
    // K and V gradients: the query heads' partial sums, added in order
    const int np = hs.kind == 0 ? 1 : parts;
#pragma unroll
    for (int it = 0; it < 64 * Q / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int rr = p / Q, i4 = (p % Q) * 4;
        const int64_t t = t0 + rr, m = b * s.T + t;
        vf32x4 ga = {0.0f, 0.0f, 0.0f, 0.0f}, gb = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int q = 0; q < np; ++q) {
            const float* row = src + q * part_stride + m * lds + (int64_t)hs.head * D;
            const vf32x4 xa = *reinterpret_cast<const vf32x4*>(row + i4);
            const vf32x4 xb = *reinterpret_cast<const vf32x4*>(row + D / 2 + i4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ga[e] += xa[e];
                gb[e] += xb[e];
            }
        }
        vf32x4 ra = ga, rb = gb;
        if (hs.kind < 2) {
            const vf32x4 c = *reinterpret_cast<const vf32x4*>(cosT + t * (D / 2) + i4);
            const vf32x4 sn = *reinterpret_cast<const vf32x4*>(sinT + t * (D / 2) + i4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ra[e] = ga[e] * c[e] + gb[e] * sn[e];
                rb[e] = gb[e] * c[e] - ga[e] * sn[e];
            }
        }
        *reinterpret_cast<uint2*>(Tr + rr * P + i4) = make_uint2(pack_bf16x2(ra[0], ra[1]), pack_bf16x2(ra[2], ra[3]));
        *reinterpret_cast<uint2*>(Tr + rr * P + D / 2 + i4) =
            make_uint2(pack_bf16x2(rb[0], rb[1]), pack_bf16x2(rb[2], rb[3]));
    }
    __syncthreads();
    store_tile_transposed<D>(Tr, dqkvT + hs.col0 * M + b * s.T + t0, M);
}

// ----------------------------------------------------------- attention ----
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float rowmax16(float v) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float rowsum16(float v) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

constexpr int kMaxT = 256;
constexpr int kPitch = kMaxT + 8;   // bf16 elements per LDS row (16-byte aligned rows)
constexpr int kCh = 32;             // tokens per staged chunk of the streamed operand

// R x C bf16 tile (C a multiple of 8, R C a multiple of 2048) moved between
// global memory, registers and LDS in 16-byte pieces by the 256 threads of a
// workgroup: piece p = tid + 256 i is row p / (C/8), columns 8 (p % (C/8)).
// A chunk is loaded into registers while the previous one is in use, then
// stored to LDS between two barriers.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <int R, int C>
struct StagedTile {
    static constexpr int PER = R * C / 8 / 256;
    static_assert(PER * 256 * 8 == R * C, "tile must split evenly over the workgroup");
    u32x4_t v[PER];
    __device__ __forceinline__ void load(const uint16_t* g, int64_t ld, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + 256 * i;
            v[i] = *reinterpret_cast<const u32x4_t*>(g + (int64_t)(p / (C / 8)) * ld + (p % (C / 8)) * 8);
        }
    }
    __device__ __forceinline__ void store(uint16_t* l, int pitch, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + 256 * i;
            *reinterpret_cast<u32x4_t*>(l + (p / (C / 8)) * pitch + (p % (C / 8)) * 8) = v[i];
        }
    }
};

// Causal attention forward for one (sample, head, 64-query tile): four
// wavefronts of 16 query rows.  K (32 keys at a time, rows [key][dim]) and
// then V^T (rows [dim][key]) pass through LDS once per workgroup; each row's
// scores stay in registers, its probabilities go through the wavefront's LDS
// rows into P V.  The output tile is staged in LDS so that o and its
// transpose are written with 16-byte stores.
template <int D>
__global__ void __launch_bounds__(256) attn_fwd_kernel(const uint16_t* q, const uint16_t* k, const uint16_t* vT,
                                                       AttnShape s, uint16_t* o, uint16_t* oT, float* lse) {
    constexpr int KC = D / 32, DT = D / 16, KT = kMaxT / 16;
    constexpr int KP = D + 8, VP = kCh + 8, OTP = 64 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Pl[4][16][kPitch];
    // streamed chunk (K [32][KP] or V^T [D][VP]); then the output tile o [64][KP] and o^T [D][OTP]
    constexpr int STAGE = (kCh * KP > D * VP ? kCh * KP : D * VP);
    constexpr int OUT = 64 * KP + D * OTP;
    __shared__ __attribute__((aligned(16))) uint16_t Sm[STAGE > OUT ? STAGE : OUT];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, c4 = lane >> 4;
    // grid (heads, samples, query tiles), the longest (last) query tiles first
    const int64_t b = blockIdx.y, h = blockIdx.x, g = h / (s.nq / s.nkv);
    const int64_t qt0 = (int64_t)(gridDim.z - 1 - blockIdx.z) * 64, q0 = qt0 + w * 16;
    const int64_t ldq = (int64_t)s.nq * D, ldk = (int64_t)s.nkv * D, M = s.B * s.T, base = b * s.T;
    const float sc = 1.0f / sqrtf((float)D);
    bf16x8 qf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qf[kc] = ld8(q + (base + q0 + r16) * ldq + h * D + kc * 32 + c4 * 8);
    const int nkt = (int)(q0 / 16) + 1;          // 16-key tiles this wavefront needs
    const int nch = (int)(qt0 / kCh) + 2;        // 32-key chunks the workgroup needs
    floatx4 S[KT];
    float mrow[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    {
        StagedTile<kCh, D> kt_regs;
        const uint16_t* kg = k + base * ldk + g * D;
        kt_regs.load(kg, ldk, tid);
#pragma unroll
        for (int c = 0; c < KT / 2; ++c) {
            if (c < nch) {
                kt_regs.store(Sm, KP, tid);
                __syncthreads();
                if (c + 1 < nch) kt_regs.load(kg + (int64_t)(c + 1) * kCh * ldk, ldk, tid);
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    const int kt = 2 * c + sub;
                    if (kt < nkt) {
                        floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int kc = 0; kc < KC; ++kc)
                            acc = mfma16(qf[kc], *reinterpret_cast<const bf16x8*>(&Sm[(sub * 16 + r16) * KP + kc * 32 + c4 * 8]),
                                         acc);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int64_t qi = q0 + 4 * c4 + r, key = kt * 16 + r16;
                            acc[r] = key <= qi ? acc[r] * sc : -INFINITY;
                            mrow[r] = fmaxf(mrow[r], acc[r]);
                        }
                        S[kt] = acc;
                    }
                }
                __syncthreads();
            }
        }
    }
    float srow[4], lrow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        mrow[r] = rowmax16(mrow[r]);
        srow[r] = 0.0f;
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
        if (kt < nkt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                S[kt][r] = expf(S[kt][r] - mrow[r]);
                srow[r] += S[kt][r];
            }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        srow[r] = rowsum16(srow[r]);
        lrow[r] = mrow[r] + logf(srow[r]);
        srow[r] = 1.0f / srow[r];
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        if (kt < nkt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Pl[w][4 * c4 + r][kt * 16 + r16] = f32_to_bf16(S[kt][r] * srow[r]);
        } else if (kt == nkt && (nkt & 1)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Pl[w][4 * c4 + r][kt * 16 + r16] = 0;
        }
    }
    wave_lds_fence();
    const int nkc = (nkt * 16 + 31) / 32;       // 32-key chunks with non-zero P for this wavefront
    floatx4 O[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    {
        StagedTile<D, kCh> vt_regs;
        const uint16_t* vg = vT + (b * s.nkv + g) * D * s.T;
        vt_regs.load(vg, s.T, tid);
#pragma unroll
        for (int c = 0; c < kMaxT / 32; ++c) {
            if (c < nch) {
                vt_regs.store(Sm, VP, tid);
                __syncthreads();
                if (c + 1 < nch) vt_regs.load(vg + (c + 1) * kCh, s.T, tid);
                if (c < nkc) {
                    const bf16x8 pf = *reinterpret_cast<const bf16x8*>(&Pl[w][r16][c * 32 + c4 * 8]);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        O[dt] = mfma16(pf, *reinterpret_cast<const bf16x8*>(&Sm[(dt * 16 + r16) * VP + c4 * 8]), O[dt]);
                }
                __syncthreads();
            }
        }
    }
    // output tile: o rows [64][KP] then o^T rows [D][OTP]
    uint16_t* Os = Sm;
    uint16_t* OsT = Sm + 64 * KP;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = w * 16 + 4 * c4 + r, col = dt * 16 + r16;
            const uint16_t val = f32_to_bf16(O[dt][r]);
            Os[row * KP + col] = val;
            OsT[col * OTP + row] = val;
        }
    if (r16 == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) lse[(b * s.nq + h) * s.T + q0 + 4 * c4 + r] = lrow[r];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 64 * D / 8 / 256; ++i) {
        const int p = tid + 256 * i;
        const int row = p / (D / 8), c8 = p % (D / 8);
        *reinterpret_cast<u32x4_t*>(o + (base + qt0 + row) * ldq + h * D + c8 * 8) =
            *reinterpret_cast<const u32x4_t*>(&Os[row * KP + c8 * 8]);
        const int dim = p / 8, part = p % 8;
        *reinterpret_cast<u32x4_t*>(oT + (h * D + dim) * M + base + qt0 + part * 8) =
            *reinterpret_cast<const u32x4_t*>(&OsT[dim * OTP + part * 8]);
    }
}

// Di = rowsum(bf16(dO) * o) per (sample, head, token); dO in bf16 row-major
// and per head transposed.
template <int D>
__global__ void __launch_bounds__(256) attn_prep_bwd_kernel(const float* dO, const uint16_t* o, AttnShape s,
                                                            float* Di, uint16_t* dOb, uint16_t* dOT) {
    constexpr int P = D + 8, C8 = D / 8;   // LDS pitch; lanes per token row (an aligned lane group)
    __shared__ __attribute__((aligned(16))) uint16_t Tr[64 * P];
    const int64_t t0 = (int64_t)blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
    const int64_t ld = (int64_t)s.nq * D, base = b * s.T;
#pragma unroll
    for (int it = 0; it < 64 * C8 / 256; ++it) {
        const int p = threadIdx.x + 256 * it;
        const int rr = p / C8, c = (p % C8) * 8;
        const int64_t e = (base + t0 + rr) * ld + h * D + c;
        float d8[8], o8[8];
        ld8f(dO + e, d8);
        const vu32x4 u = pack8h(d8);
        *reinterpret_cast<vu32x4*>(dOb + e) = u;
        *reinterpret_cast<vu32x4*>(Tr + rr * P + c) = u;
        ld8h(o + e, o8);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc += __uint_as_float(u[i] << 16) * o8[2 * i] + __uint_as_float(u[i] & 0xFFFF0000u) * o8[2 * i + 1];
#pragma unroll
        for (int off = 1; off < C8; off <<= 1) acc += __shfl_xor(acc, off, 64);
        if (p % C8 == 0) Di[(b * s.nq + h) * s.T + t0 + rr] = acc;
    }
    __syncthreads();
    store_tile_transposed<D>(Tr, dOT + ((b * s.nq + h) * D) * s.T + t0, s.T);
}

// dQ for one (sample, head, 64-query tile), four wavefronts of 16 query rows:
// K and V (32 keys at a time, rows [key][dim]) pass through LDS once per
// workgroup for S and dP, then K^T (rows [dim][key]) for dS K.  dS goes
// through the wavefront's LDS rows.
template <int D>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(const uint16_t* q, const uint16_t* k, const uint16_t* kT,
                                                          const uint16_t* v, const uint16_t* dOb, const float* lse,
                                                          const float* Di, AttnShape s, float* dq) {
    constexpr int KC = D / 32, DT = D / 16, KT = kMaxT / 16;
    constexpr int KP = D + 8, VP = kCh + 8;
    constexpr int STAGE = (2 * kCh * KP > D * VP ? 2 * kCh * KP : D * VP);
    __shared__ __attribute__((aligned(16))) uint16_t Sl[4][16][kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Sm[STAGE];   // K and V chunks, later a K^T chunk
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, c4 = lane >> 4;
    // grid (heads, samples, query tiles), the longest (last) query tiles first
    const int64_t b = blockIdx.y, h = blockIdx.x, g = h / (s.nq / s.nkv);
    const int64_t qt0 = (int64_t)(gridDim.z - 1 - blockIdx.z) * 64, q0 = qt0 + w * 16;
    const int64_t ldq = (int64_t)s.nq * D, ldk = (int64_t)s.nkv * D, base = b * s.T;
    const float sc = 1.0f / sqrtf((float)D);
    bf16x8 qf[KC], df[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        qf[kc] = ld8(q + (base + q0 + r16) * ldq + h * D + kc * 32 + c4 * 8);
        df[kc] = ld8(dOb + (base + q0 + r16) * ldq + h * D + kc * 32 + c4 * 8);
    }
    float lr[4], dr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        lr[r] = lse[(b * s.nq + h) * s.T + q0 + 4 * c4 + r];
        dr[r] = Di[(b * s.nq + h) * s.T + q0 + 4 * c4 + r];
    }
    const int nkt = (int)(q0 / 16) + 1;
    const int nch = (int)(qt0 / kCh) + 2;
    {
        StagedTile<kCh, D> kr, vr;
        const uint16_t* kg = k + base * ldk + g * D;
        const uint16_t* vg = v + base * ldk + g * D;
        kr.load(kg, ldk, tid);
        vr.load(vg, ldk, tid);
#pragma unroll
        for (int c = 0; c < KT / 2; ++c) {
            if (c < nch) {
                kr.store(Sm, KP, tid);
                vr.store(Sm + kCh * KP, KP, tid);
                __syncthreads();
                if (c + 1 < nch) {
                    kr.load(kg + (int64_t)(c + 1) * kCh * ldk, ldk, tid);
                    vr.load(vg + (int64_t)(c + 1) * kCh * ldk, ldk, tid);
                }
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    const int kt = 2 * c + sub;
                    if (kt < nkt) {
                        floatx4 S = {0.0f, 0.0f, 0.0f, 0.0f}, dP = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int kc = 0; kc < KC; ++kc) {
                            const int off = (sub * 16 + r16) * KP + kc * 32 + c4 * 8;
                            S = mfma16(qf[kc], *reinterpret_cast<const bf16x8*>(&Sm[off]), S);
                            dP = mfma16(df[kc], *reinterpret_cast<const bf16x8*>(&Sm[kCh * KP + off]), dP);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int64_t qi = q0 + 4 * c4 + r, key = kt * 16 + r16;
                            const float p = key <= qi ? expf(S[r] * sc - lr[r]) : 0.0f;
                            Sl[w][4 * c4 + r][kt * 16 + r16] = f32_to_bf16(p * (dP[r] - dr[r]) * sc);
                        }
                    } else if (kt == nkt && (nkt & 1)) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) Sl[w][4 * c4 + r][kt * 16 + r16] = 0;
                    }
                }
                __syncthreads();
            }
        }
    }
    wave_lds_fence();
    const int nkc = (nkt * 16 + 31) / 32;
    floatx4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    {
        StagedTile<D, kCh> ktr;
        const uint16_t* ktg = kT + (b * s.nkv + g) * D * s.T;
        ktr.load(ktg, s.T, tid);
#pragma unroll
        for (int c = 0; c < kMaxT / 32; ++c) {
            if (c < nch) {
                ktr.store(Sm, VP, tid);
                __syncthreads();
                if (c + 1 < nch) ktr.load(ktg + (c + 1) * kCh, s.T, tid);
                if (c < nkc) {
                    const bf16x8 af = *reinterpret_cast<const bf16x8*>(&Sl[w][r16][c * 32 + c4 * 8]);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        acc[dt] = mfma16(af, *reinterpret_cast<const bf16x8*>(&Sm[(dt * 16 + r16) * VP + c4 * 8]), acc[dt]);
                }
                __syncthreads();
            }
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[(base + q0 + 4 * c4 + r) * ldq + h * D + dt * 16 + r16] = acc[dt][r];
}

// dK, dV for one (sample, KV head, 64-key tile), four wavefronts of 16 key
// rows, over the query heads [hs hper, (hs + 1) hper) of the KV head's group
// in order: Q and dO (rows [query][dim]) and their transposes (rows
// [dim][query]) pass through LDS 32 queries at a time, once per workgroup.
// P^T and dS^T go through the wavefront's LDS rows.  Workgroup part hs
// writes its sums at hs * part_stride.
template <int D>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_kernel(const uint16_t* q, const uint16_t* qT, const uint16_t* k,
                                                            const uint16_t* v, const uint16_t* dOb,
                                                            const uint16_t* dOT, const float* lse, const float* Di,
                                                            AttnShape s, int hper, int64_t part_stride, float* dk,
                                                            float* dv) {
    constexpr int KC = D / 32, DT = D / 16;
    constexpr int KP = D + 8, VP = kCh + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Pl[4][16][40];
    __shared__ __attribute__((aligned(16))) uint16_t Dl[4][16][40];
    // Q and dO chunks [32][KP], then Q^T and dO^T chunks [D][VP]
    __shared__ __attribute__((aligned(16))) uint16_t Sm[2 * kCh * KP + 2 * D * VP];
    uint16_t* Qs = Sm;
    uint16_t* dOs = Sm + kCh * KP;
    uint16_t* QTs = Sm + 2 * kCh * KP;
    uint16_t* dOTs = QTs + D * VP;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, c4 = lane >> 4;
    const int rep = s.nq / s.nkv;
    const int nsplit = rep / hper;                 // workgroups per (sample, KV head, key tile)
    // grid (KV heads, samples x head splits, key tiles), the longest (first) key tiles first
    const int64_t b = blockIdx.y / nsplit, hs = blockIdx.y % nsplit, g = blockIdx.x;
    const int64_t kt0 = (int64_t)blockIdx.z * 64, k0 = kt0 + w * 16;
    const int64_t ldq = (int64_t)s.nq * D, ldk = (int64_t)s.nkv * D, base = b * s.T;
    const float sc = 1.0f / sqrtf((float)D);
    bf16x8 kf[KC], vf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        kf[kc] = ld8(k + (base + k0 + r16) * ldk + g * D + kc * 32 + c4 * 8);
        vf[kc] = ld8(v + (base + k0 + r16) * ldk + g * D + kc * 32 + c4 * 8);
    }
    floatx4 dK[DT], dV[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dK[dt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        dV[dt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int64_t c0 = kt0 / kCh, nqc = s.T / kCh;   // query chunks of the workgroup: [c0, nqc)
    const int64_t cw = k0 / kCh;                       // first chunk with queries >= this wavefront's keys
    for (int hq = (int)g * rep + (int)hs * hper; hq < (int)g * rep + ((int)hs + 1) * hper; ++hq) {
        const uint16_t* qg = q + base * ldq + hq * D;
        const uint16_t* dg = dOb + base * ldq + hq * D;
        const uint16_t* qtg = qT + ((b * s.nq + hq) * D) * s.T;
        const uint16_t* dtg = dOT + ((b * s.nq + hq) * D) * s.T;
        StagedTile<kCh, D> qr, dr;
        StagedTile<D, kCh> qtr, dtr;
        qr.load(qg + c0 * kCh * ldq, ldq, tid);
        dr.load(dg + c0 * kCh * ldq, ldq, tid);
        qtr.load(qtg + c0 * kCh, s.T, tid);
        dtr.load(dtg + c0 * kCh, s.T, tid);
        for (int64_t qc = c0; qc < nqc; ++qc) {
            qr.store(Qs, KP, tid);
            dr.store(dOs, KP, tid);
            qtr.store(QTs, VP, tid);
            dtr.store(dOTs, VP, tid);
            __syncthreads();
            if (qc + 1 < nqc) {
                qr.load(qg + (qc + 1) * kCh * ldq, ldq, tid);
                dr.load(dg + (qc + 1) * kCh * ldq, ldq, tid);
                qtr.load(qtg + (qc + 1) * kCh, s.T, tid);
                dtr.load(dtg + (qc + 1) * kCh, s.T, tid);
            }
            if (qc >= cw) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int64_t qq = qc * kCh + half * 16 + r16;   // this lane's query column
                    floatx4 St = {0.0f, 0.0f, 0.0f, 0.0f}, dPt = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        const int off = (half * 16 + r16) * KP + kc * 32 + c4 * 8;
                        St = mfma16(kf[kc], *reinterpret_cast<const bf16x8*>(&Qs[off]), St);
                        dPt = mfma16(vf[kc], *reinterpret_cast<const bf16x8*>(&dOs[off]), dPt);
                    }
                    const float lq = lse[(b * s.nq + hq) * s.T + qq], dq_ = Di[(b * s.nq + hq) * s.T + qq];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t key = k0 + 4 * c4 + r;
                        const float p = qq >= key ? expf(St[r] * sc - lq) : 0.0f;
                        Pl[w][4 * c4 + r][half * 16 + r16] = f32_to_bf16(p);
                        Dl[w][4 * c4 + r][half * 16 + r16] = f32_to_bf16(p * (dPt[r] - dq_) * sc);
                    }
                }
                wave_lds_fence();
                const bf16x8 pa = *reinterpret_cast<const bf16x8*>(&Pl[w][r16][c4 * 8]);
                const bf16x8 da = *reinterpret_cast<const bf16x8*>(&Dl[w][r16][c4 * 8]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int off = (dt * 16 + r16) * VP + c4 * 8;
                    dV[dt] = mfma16(pa, *reinterpret_cast<const bf16x8*>(&dOTs[off]), dV[dt]);
                    dK[dt] = mfma16(da, *reinterpret_cast<const bf16x8*>(&QTs[off]), dK[dt]);
                }
                wave_lds_fence();
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t e = hs * part_stride + (base + k0 + 4 * c4 + r) * ldk + g * D + dt * 16 + r16;
            dk[e] = dK[dt][r];
            dv[e] = dV[dt][r];
        }
}

unsigned grid_1d(int64_t n) {
    int64_t b = (n + 1023) / 1024;
    if (b > 16384) b = 16384;
    return (unsigned)(b > 0 ? b : 1);
}

dim3 attn_grid(const AttnShape& s, int heads) { return dim3((unsigned)(s.T / 64), (unsigned)heads, (unsigned)s.B); }
// Causal attention tiles differ up to T/64-fold in work; with the tile index
// the slowest grid dimension, every sample's and head's longest tiles are
// dispatched first and the short ones fill in behind them.
dim3 attn_grid_by_tile(const AttnShape& s, int heads, int per_sample) {
    return dim3((unsigned)heads, (unsigned)(s.B * per_sample), (unsigned)(s.T / 64));
}

}  // namespace

hipError_t launch_rmsnorm_fwd(const void* x, bool x_bf16, RowMap map, const float* add, int64_t M, int64_t H,
                              const float* w, float eps, float* h_out, float* r_out, void* out, bool out_bf16,
                              hipStream_t stream) {
    const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(add) |
                           reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(h_out) |
                           reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    if (x_bf16 && out_bf16 && H % 8 == 0 && H <= 256 * 8 * kRowChunks && aligned)
        hipLaunchKernelGGL(rmsnorm_fwd_vec_kernel, dim3((unsigned)M), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), map, add, H, w, eps, h_out, r_out,
                           static_cast<uint16_t*>(out));
    else
        hipLaunchKernelGGL(rmsnorm_fwd_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, x_bf16, map, add, H, w, eps,
                           h_out, r_out, out, out_bf16);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const float* dh2, const float* dh2b, const float* h, const float* r, const float* w,
                              const void* dy, bool dy_bf16, int64_t M, int64_t H, void* dh, bool dh_bf16,
                              hipStream_t stream) {
    const bool aligned = ((reinterpret_cast<uintptr_t>(dh2) | reinterpret_cast<uintptr_t>(dh2b) |
                           reinterpret_cast<uintptr_t>(h) |
                           reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(dy) |
                           reinterpret_cast<uintptr_t>(dh)) & 15) == 0;
    if (dy_bf16 && dh_bf16 && H % 8 == 0 && H <= 256 * 8 * kRowChunks && aligned)
        hipLaunchKernelGGL(rmsnorm_bwd_vec_kernel, dim3((unsigned)M), dim3(256), 0, stream, dh2, dh2b, h, r, w,
                           static_cast<const uint16_t*>(dy), H, static_cast<uint16_t*>(dh));
    else
        hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3((unsigned)M), dim3(256), 0, stream, dh2, dh2b, h, r, w, dy,
                           dy_bf16, H, dh, dh_bf16);
    return hipGetLastError();
}

hipError_t launch_yref_combine(const float* y, RowMap map, int64_t s0, const float* h, int64_t nb, int64_t H,
                               int64_t T, float ca, float ch, float* out, hipStream_t stream) {
    const dim3 grid((unsigned)((T + 63) / 64), (unsigned)((H + 63) / 64), (unsigned)nb);
    const bool aligned = ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(h) |
                           reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    if (H % 8 == 0 && T % 8 == 0 && aligned)
        hipLaunchKernelGGL(yref_combine_vec_kernel, grid, dim3(256), 0, stream, y, map, s0, h, H, T, ca, ch, out);
    else
        hipLaunchKernelGGL(yref_combine_kernel, grid, dim3(256), 0, stream, y, map, s0, h, H, T, ca, ch, out);
    return hipGetLastError();
}

hipError_t launch_transpose2d(const void* src, int64_t lds, void* dst, int64_t ldd, int64_t rows, int64_t cols,
                              int elem_bytes, hipStream_t stream) {
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
    if (elem_bytes == 2 && transpose_b16_fits(src, lds, dst, ldd, rows, cols))
        return launch_transpose_b16(static_cast<const uint16_t*>(src), lds, 0, static_cast<uint16_t*>(dst), ldd, 0,
                                    rows, cols, 1, stream);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(transpose2d_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(src), lds, static_cast<uint16_t*>(dst), ldd, rows, cols);
    else
        hipLaunchKernelGGL(transpose2d_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(src), lds,
                           static_cast<float*>(dst), ldd, rows, cols);
    return hipGetLastError();
}

hipError_t launch_add_rows(const float* a, const float* b, int64_t n, void* y, bool y_bf16, hipStream_t stream) {
    hipLaunchKernelGGL(add_rows_kernel, dim3(grid_1d(n)), dim3(256), 0, stream, a, b, n, y, y_bf16);
    return hipGetLastError();
}

#define AR_BY_D(s, launch)                                           \
    do {                                                             \
        if ((s).d == 128) { constexpr int D = 128; launch; }        \
        else if ((s).d == 64) { constexpr int D = 64; launch; }     \
        else return hipErrorInvalidValue;                            \
    } while (0)

hipError_t launch_rope_fwd(const float* qkv, const float* cosT, const float* sinT, AttnShape s, uint16_t* q,
                           uint16_t* qT, uint16_t* k, uint16_t* kT, uint16_t* v, uint16_t* vT, hipStream_t stream) {
    AR_BY_D(s, hipLaunchKernelGGL(rope_fwd_kernel<D>, attn_grid(s, s.nq + 2 * s.nkv), dim3(256), 0, stream, qkv, cosT,
                                  sinT, s, q, qT, k, kT, v, vT));
    return hipGetLastError();
}

hipError_t launch_rope_bwd(const float* dq, const float* dk, const float* dv, int parts, int64_t part_stride,
                           const float* cosT, const float* sinT, AttnShape s, uint16_t* dqkvT, hipStream_t stream) {
    AR_BY_D(s, hipLaunchKernelGGL(rope_bwd_kernel<D>, attn_grid(s, s.nq + 2 * s.nkv), dim3(256), 0, stream, dq, dk, dv,
                                  parts, part_stride, cosT, sinT, s, dqkvT));
    return hipGetLastError();
}

hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* vT, AttnShape s, uint16_t* o,
                           uint16_t* oT, float* lse, hipStream_t stream) {
    AR_BY_D(s, hipLaunchKernelGGL(attn_fwd_kernel<D>, attn_grid_by_tile(s, s.nq, 1), dim3(256), 0, stream, q, k, vT, s, o, oT,
                                  lse));
    return hipGetLastError();
}

hipError_t launch_attn_prep_bwd(const float* dO, const uint16_t* o, AttnShape s, float* Di, uint16_t* dOb,
                                uint16_t* dOT, hipStream_t stream) {
    AR_BY_D(s, hipLaunchKernelGGL(attn_prep_bwd_kernel<D>, attn_grid(s, s.nq), dim3(256), 0, stream, dO, o, s, Di, dOb,
                                  dOT));
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* kT, const uint16_t* v,
                              const uint16_t* dOb, const float* lse, const float* Di, AttnShape s, float* dq,
                              hipStream_t stream) {
    AR_BY_D(s, hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, attn_grid_by_tile(s, s.nq, 1), dim3(256), 0, stream, q, k, kT, v, dOb,
                                  lse, Di, s, dq));
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(const uint16_t* q, const uint16_t* qT, const uint16_t* k, const uint16_t* v,
                                const uint16_t* dOb, const uint16_t* dOT, const float* lse, const float* Di,
                                AttnShape s, int hper, int64_t part_stride, float* dk, float* dv,
                                hipStream_t stream) {
    const int rep = s.nq / s.nkv;
    if (hper < 1 || rep % hper != 0) return hipErrorInvalidValue;
    const dim3 grid = attn_grid_by_tile(s, s.nkv, rep / hper);
    AR_BY_D(s, hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, grid, dim3(256), 0, stream, q, qT, k, v, dOb, dOT, lse, Di, s,
                                  hper, part_stride, dk, dv));
    return hipGetLastError();
}

}  // namespace ar
