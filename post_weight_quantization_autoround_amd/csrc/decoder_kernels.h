// Kernels of the Llama decoder block step (decoder_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ar_internal.h"

namespace ar {

// Row map of a minibatch: row m of the step is pool row
// ids[m / T] * T + m % T, ids = sched + (state ? row of the step : 0) * nseg
// (identity when sched is NULL).
struct RowMap {
    const int32_t* sched;
    int32_t nseg;
    const StepState* state;
    int32_t after_decide;
    int64_t T;
};

// out[m] = (x[map(m)] (+ add[m])) * r_m * w with r_m = 1/sqrt(mean(h^2) + eps);
// x bf16 or fp32 [*, H]; add fp32 [M, H] nullable; h_out fp32 [M, H] (the
// sum) nullable; r_out [M] nullable; w [H] nullable (= 1); out bf16 or fp32.
hipError_t launch_rmsnorm_fwd(const void* x, bool x_bf16, RowMap map, const float* add, int64_t M, int64_t H,
                              const float* w, float eps, float* h_out, float* r_out, void* out, bool out_bf16,
                              hipStream_t stream);
// dh = dy + u r - h r^3 (sum_j h_j u_j) / H, u = dh2 * w; dy bf16 or fp32.
// dh2b (nullable): the second half of a reduction-split dh2, which is then
// dh2 + dh2b.
hipError_t launch_rmsnorm_bwd(const float* dh2, const float* dh2b, const float* h, const float* r, const float* w,
                              const void* dy, bool dy_bf16, int64_t M, int64_t H, void* dh, bool dh_bf16,
                              hipStream_t stream);
// out[j][c][t] = ca * y[s_j][c][t] + ch * h[j T + t][c] for j < nb samples,
// c < H, t < T (y, out: per-sample transposed [*, H, T]; h: [nb T, H]).
// s_j = map ids (RowMap, T ignored) or s0 + j when map.sched is NULL.
hipError_t launch_yref_combine(const float* y, RowMap map, int64_t s0, const float* h, int64_t nb, int64_t H,
                               int64_t T, float ca, float ch, float* out, hipStream_t stream);
// dst[c * ldd + r] = src[r * lds + c] (r < rows, c < cols), element size 2 or 4.
hipError_t launch_transpose2d(const void* src, int64_t lds, void* dst, int64_t ldd, int64_t rows, int64_t cols,
                              int elem_bytes, hipStream_t stream);
// y = a + b, fp32 [n] -> fp32 or bf16
hipError_t launch_add_rows(const float* a, const float* b, int64_t n, void* y, bool y_bf16, hipStream_t stream);

struct AttnShape {
    int64_t B;          // samples in the batch
    int64_t T;          // tokens per sample (a multiple of 64, at most 256)
    int32_t nq, nkv, d; // heads and head size (d = 64 or 128)
};

// RoPE on q, k of qkv fp32 [B T, (nq + 2 nkv) d] (rotate-half pairs, cos/sin
// [T, d/2]); writes the bf16 rotated q, k and v row-major ([B T, nq d] and
// [B T, nkv d]) and per head transposed ([B, heads, d, T]).
hipError_t launch_rope_fwd(const float* qkv, const float* cosT, const float* sinT, AttnShape s, uint16_t* q,
                           uint16_t* qT, uint16_t* k, uint16_t* kT, uint16_t* v, uint16_t* vT, hipStream_t stream);
// Inverse rotation of dq, dk (fp32 [B T, nq d], [B T, nkv d]) and dv; writes
// the bf16 transposed gradient [(nq + 2 nkv) d, B T].  dk and dv are the sum
// of `parts` partials part_stride elements apart, added in order.
hipError_t launch_rope_bwd(const float* dq, const float* dk, const float* dv, int parts, int64_t part_stride,
                           const float* cosT, const float* sinT, AttnShape s, uint16_t* dqkvT, hipStream_t stream);
// Causal attention per sample and head: o bf16 [B T, nq d] and [nq d, B T],
// lse fp32 [B, nq, T].
hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* vT, AttnShape s, uint16_t* o,
                           uint16_t* oT, float* lse, hipStream_t stream);
// Di = rowsum(bf16(dO) * o); dO rounded to bf16 in both layouts.
hipError_t launch_attn_prep_bwd(const float* dO, const uint16_t* o, AttnShape s, float* Di, uint16_t* dOb,
                                uint16_t* dOT, hipStream_t stream);
hipError_t launch_attn_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* kT, const uint16_t* v,
                              const uint16_t* dOb, const float* lse, const float* Di, AttnShape s, float* dq,
                              hipStream_t stream);
// dK, dV per KV head: hper query heads of its group per workgroup (hper
// divides nq / nkv); workgroup part p of a group writes at p * part_stride,
// so with hper < nq / nkv the caller sums the nq / (nkv hper) partials.
hipError_t launch_attn_bwd_dkdv(const uint16_t* q, const uint16_t* qT, const uint16_t* k, const uint16_t* v,
                                const uint16_t* dOb, const uint16_t* dOT, const float* lse, const float* Di,
                                AttnShape s, int hper, int64_t part_stride, float* dk, float* dv, hipStream_t stream);

}  // namespace ar
