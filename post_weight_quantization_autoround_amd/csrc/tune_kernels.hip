// Loss decision, straight-through backward and SignSGD update (gfx950).
//
// Straight-through estimator (AutoRound blog sec. 3 "SignSGD": the quantizer
// is a step function, its gradient is approximated by passing through the
// rounding): with t = rint(W/s + V) + z, q = clamp(t, 0, Q), w^ = s (q - z),
// m = [0 <= t <= Q] and both roundings taken as the identity,
//   dw^/dV     = s m
//   dw^/ds     = c = (q - z) - m W/s + (m - 1) wmin/s
//   dw^/dwmax  = c / Q,  dw^/dwmin = (1 - m) - c / Q
// so with G = dL/dw^:  dV = G s m,  dalpha = mx/Q sum_g G c,
// dbeta = mn sum_g G ((1 - m) - c/Q).  Symmetric groups (fixed zero-point,
// s = alpha amax/(2^(b-1) - 1)): c = (q - z) - m W/s,
// dalpha = amax/(2^(b-1) - 1) sum_g G c, dbeta = 0 (ste_terms, ste_group_grads).
//
// SignSGD (blog sec. 3 update rule, descending): p <- clamp(p - lr_t sign(g)),
// sign(0) = 0, V in [-0.5, 0.5], alpha and beta in the clip box.  The best-loss
// snapshot costs no copy: when the loss improves, the update writes into the
// other of two parameter buffers, so the evaluated state stays intact.
#include "ar_internal.h"

namespace ar {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8w(const void* W, bool bf16, int64_t idx, float w[8]) {
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

__device__ __forceinline__ void load8f(const float* p, float v[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Gradient terms of 8 consecutive weights of one group; returns the two
// group-sum contributions and writes dV.
__device__ __forceinline__ void ste_chunk(const SteArgs& a, int buf, int64_t idx, const GroupQ& gq, float& sa,
                                          float& sb) {
    const float Q = a.qp.qmax;
    float w[8], v[8], g[8], dv[8];
    load8w(a.W, a.w_bf16, idx, w);
    load8f(a.V[buf] + idx, v);
    load8f(a.G + idx, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float u, ru;
        const float ws = scaled_weight(w[i], v[i], gq.s, gq.r, gq.thr, u, ru);
        const float t = ru + gq.z;
        const float q = __builtin_amdgcn_fmed3f(t, 0.0f, Q);
        const bool m = q == t;
        dv[i] = m ? g[i] * gq.s : 0.0f;
        ste_terms(g[i], q, gq.z, ws, gq.wmin_s, m, sa, sb);
    }
    if (a.dV) {
        *reinterpret_cast<float4*>(a.dV + idx) = make_float4(dv[0], dv[1], dv[2], dv[3]);
        *reinterpret_cast<float4*>(a.dV + idx + 4) = make_float4(dv[4], dv[5], dv[6], dv[7]);
    }
}

// Groups of g <= 512 weights: g/8 consecutive lanes own one group; a segmented
// butterfly over those lanes reduces the group sums.
__global__ void __launch_bounds__(kThreads) ste_seg_kernel(SteArgs a) {
    if (a.state && a.state->halted) return;
    const int64_t nchunks = a.N * (a.K >> 3);
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int lpg = a.qp.group >> 3;              // lanes per group (1..64, power of two)
    const int buf = a.state ? a.state->src : 0;
    float sa = 0.0f, sb = 0.0f;
    int64_t gi = 0;
    float mx = 0.0f, mn = 0.0f;
    if (c < nchunks) {
        gi = c / lpg;                             // flattened group index (groups never cross rows)
        mx = a.mx[gi];
        mn = a.mn[gi];
        const float al = a.alpha[buf] ? a.alpha[buf][gi] : 1.0f;
        const float be = a.beta[buf] ? a.beta[buf][gi] : 1.0f;
        ste_chunk(a, buf, c << 3, group_quant(mx, mn, al, be, a.qp), sa, sb);
    }
    for (int off = 1; off < lpg; off <<= 1) {
        sa += __shfl_xor(sa, off, 64);
        sb += __shfl_xor(sb, off, 64);
    }
    if (c < nchunks && (c % lpg) == 0) ste_group_grads(mx, mn, a.qp, sa, sb, a.dalpha[gi], a.dbeta[gi]);
}

// Groups larger than 512 weights: one workgroup per group.
__global__ void __launch_bounds__(kThreads) ste_group_kernel(SteArgs a) {
    if (a.state && a.state->halted) return;
    __shared__ float ra[kThreads / 64], rb[kThreads / 64];
    const int64_t gi = blockIdx.x;
    const int64_t G = a.K / a.qp.group;
    const int64_t n = gi / G;
    const int64_t kbase = n * a.K + (gi - n * G) * a.qp.group;
    const int buf = a.state ? a.state->src : 0;
    const float mx = a.mx[gi], mn = a.mn[gi];
    const float al = a.alpha[buf] ? a.alpha[buf][gi] : 1.0f;
    const float be = a.beta[buf] ? a.beta[buf][gi] : 1.0f;
    const GroupQ gq = group_quant(mx, mn, al, be, a.qp);
    float sa = 0.0f, sb = 0.0f;
    for (int64_t e = (int64_t)threadIdx.x * 8; e < a.qp.group; e += kThreads * 8)
        ste_chunk(a, buf, kbase + e, gq, sa, sb);
    for (int off = 32; off > 0; off >>= 1) {
        sa += __shfl_xor(sa, off, 64);
        sb += __shfl_xor(sb, off, 64);
    }
    if ((threadIdx.x & 63) == 0) {
        ra[threadIdx.x >> 6] = sa;
        rb[threadIdx.x >> 6] = sb;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float ta = 0.0f, tb = 0.0f;
        for (int w = 0; w < kThreads / 64; ++w) {
            ta += ra[w];
            tb += rb[w];
        }
        ste_group_grads(mx, mn, a.qp, ta, tb, a.dalpha[gi], a.dbeta[gi]);
    }
}

__global__ void __launch_bounds__(kThreads) signsgd_kernel(UpdateArgs a) {
    if (a.state && a.state->halted) return;
    const int src = a.state ? a.state->src : 0;
    const int dst = a.state ? a.state->dst : 0;
    const int t = a.state ? a.state->t_eval : 0;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nv4 = a.nV >> 2;
    if (i < nv4) {
        const float lr = a.lr[t];
        const float4 p = reinterpret_cast<const float4*>(a.V[src])[i];
        const float4 g = reinterpret_cast<const float4*>(a.dV)[i];
        float4 o;
        o.x = sign_step(p.x, g.x, lr, -0.5f, 0.5f);
        o.y = sign_step(p.y, g.y, lr, -0.5f, 0.5f);
        o.z = sign_step(p.z, g.z, lr, -0.5f, 0.5f);
        o.w = sign_step(p.w, g.w, lr, -0.5f, 0.5f);
        reinterpret_cast<float4*>(a.V[dst])[i] = o;
    } else if (i < nv4 + a.nG) {
        const int64_t j = i - nv4;
        const float lr = a.lr_clip[t];
        a.alpha[dst][j] = sign_step(a.alpha[src][j], a.dalpha[j], lr, a.clip_lo, a.clip_hi);
        a.beta[dst][j] = sign_step(a.beta[src][j], a.dbeta[j], lr, a.clip_lo, a.clip_hi);
    }
}

__global__ void __launch_bounds__(64) loss_decide_kernel(const double* __restrict__ partials, int32_t np,
                                                        double inv_count, StepState* st, double* trace, int32_t iters) {
    if (st->halted) return;
    block_loss_decide(partials, np, inv_count, st, trace, iters);
}

}  // namespace

hipError_t launch_loss_decide(const double* partials, int32_t np, double inv_count, StepState* st,
                              double* loss_trace, int32_t iters, hipStream_t stream) {
    hipLaunchKernelGGL(loss_decide_kernel, dim3(1), dim3(64), 0, stream, partials, np, inv_count, st, loss_trace,
                       iters);
    return hipGetLastError();
}

hipError_t launch_ste_bwd(const SteArgs& a, hipStream_t stream) {
    const int32_t g = a.qp.group;
    if (g <= 512 && (512 % g) == 0) {
        const int64_t nchunks = a.N * (a.K >> 3);
        hipLaunchKernelGGL(ste_seg_kernel, dim3((unsigned)((nchunks + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                           stream, a);
    } else {
        const int64_t ngroups = a.N * (a.K / g);
        hipLaunchKernelGGL(ste_group_kernel, dim3((unsigned)ngroups), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_signsgd_update(const UpdateArgs& a, hipStream_t stream) {
    const int64_t n = (a.nV >> 2) + a.nG;
    hipLaunchKernelGGL(signsgd_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ar
