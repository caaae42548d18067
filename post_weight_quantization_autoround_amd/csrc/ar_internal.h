// Internal declarations shared by the libautoround translation units.
// Device code targets gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

// ---------------------------------------------------------------- bf16 ----
// bf16 is stored as uint16_t bit patterns; conversions are written out so the
// rounding (nearest, ties to even) is explicit and identical everywhere.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Element loads that widen bf16 or pass fp32 through.
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float to_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
};

// ----------------------------------------------------- tuning loop state ----
// Lives in device memory so that one captured step serves every step.
struct StepState {
    int32_t step;       // index of the step being evaluated next
    int32_t cur;        // parameter buffer (0/1) holding the state to evaluate
    int32_t src;        // buffer read by this step's backward and update
    int32_t dst;        // buffer written by this step's update
    int32_t best_idx;   // buffer holding the best-loss snapshot (-1: none yet)
    int32_t best_step;  // step of the snapshot
    int32_t halted;     // set when a loss was non-finite: later steps do nothing
    int32_t t_eval;     // step evaluated by the latest loss decision
    double best_loss;   // +inf initially
};

// Group quantizer constants: Q = 2^bits - 1 as float, and the divisor of a
// group's range with its rounded reciprocal (set on the host).
struct QParams {
    int32_t bits;
    int32_t group;      // group size g (multiple of 8)
    float qmax;         // Q
    int32_t sym;        // 1: symmetric scale, zero-point fixed at 2^(b-1)
    float qdiv;         // Q (asymmetric) or 2^(b-1) - 1 (symmetric)
    float qdiv_inv;     // fl(1 / qdiv)
};

// x / qdiv rounded to nearest (the IEEE quotient) for finite x >= 0, without
// a division: q0 = fl(x y) with y = fl(1/qdiv) is within an ulp of the
// quotient, the residual x - q0 qdiv is exact in one fused multiply-add, and
// fl(q0 + residual y) is the correctly rounded quotient.  The identity was
// checked against the IEEE quotient for every non-negative finite fp32 x and
// every divisor that bit widths 2..8 give (2^b - 1 and 2^(b-1) - 1); an
// infinite x returns x, as the division does.
__device__ __forceinline__ float div_qdiv(float x, float qd, float y) {
    const float q0 = x * y;
    const float res = __builtin_fmaf(-q0, qd, x);
    const float q1 = __builtin_fmaf(res, y, q0);
    return (x < __builtin_inff()) ? q1 : x;
}

// Near-tie bound of the quantizer's rounding (see scaled_weight): u, computed
// from an approximate reciprocal of s, rounds like the exactly divided value
// when |u - rint(u)| < 1/2 - 2^-18 max(|w/s|, |u|, 1).  Every weight of a
// group lies in [mn, mx] (zero-inclusive range) and |v| <= 1/2, so
// max(mx, -mn) r + 1 bounds the magnitude for the whole group.  A reciprocal
// outside the normal range (a range near the fp32 limits) gives a bound no
// distance meets, so every element of such a group takes the division.
__device__ __forceinline__ float tie_threshold(float mx, float mn, float r) {
    const bool normal = r >= 0x1p-125f && r <= 0x1p125f;
    return normal ? 0.5f - (fmaxf(mx, -mn) * r + 1.0f) * 3.814697265625e-06f : -1.0f;
}

// Per-group quantities of the fake quantizer (fp32, fixed operation order,
// ties-to-even rounding, no contraction); every kernel that quantizes uses
// this one definition.
//   asymmetric (AutoRound blog sec. 2-4): wmax = alpha*mx, wmin = beta*mn,
//     s = (wmax - wmin)/Q (1 for an empty range), z = rint(-wmin/s) in [0, Q];
//   symmetric (coordinates page sec. 1.2): wmax = alpha*max(mx, -mn),
//     s = wmax/(2^(b-1) - 1) (1 for an empty range), z = 2^(b-1), wmin = -wmax.
// s is the IEEE quotient bit for bit (div_qdiv).  r is v_rcp_f32's
// reciprocal of s (within an ulp); z is rint(-wmin r) unless -wmin r lies
// near a rounding tie, where the IEEE quotient -wmin/s decides, so z is the
// one the division gives.  wmin_s = wmin/s, to the same precision (only the
// straight-through gradient uses it).  thr is the group's near-tie bound.
struct GroupQ {
    float s, z, r, wmin_s, thr;
};
__device__ __forceinline__ GroupQ group_quant(float mx, float mn, float al, float be, const QParams& qp) {
    GroupQ g;
    if (qp.sym) {
        const float wmax = al * fmaxf(mx, -mn);
        g.s = (wmax == 0.0f) ? 1.0f : div_qdiv(wmax, qp.qdiv, qp.qdiv_inv);
        g.z = (qp.qmax + 1.0f) * 0.5f;
        g.r = __builtin_amdgcn_rcpf(g.s);
        g.wmin_s = 0.0f;   // c = q - z where the code is clamped (the zero-point is fixed)
        g.thr = tie_threshold(mx, mn, g.r);
        return g;
    }
    const float wmax = al * mx;
    const float wmin = be * mn;
    const float d = wmax - wmin;
    g.s = (d == 0.0f) ? 1.0f : div_qdiv(d, qp.qdiv, qp.qdiv_inv);
    g.r = __builtin_amdgcn_rcpf(g.s);
    g.thr = tie_threshold(mx, mn, g.r);
    // -wmin/s lies in [0, Q(1 + 2^-23)]; the bound uses |u| + 1 as magnitude
    float u = -wmin * g.r;
    float ru = __builtin_rintf(u);
    const bool normal = g.thr > -1.0f;
    if (!(normal && __builtin_fabsf(u - ru) < 0.5f - (__builtin_fabsf(u) + 1.0f) * 3.814697265625e-06f)) {
        u = -wmin / g.s;
        ru = __builtin_rintf(u);
    }
    g.z = __builtin_amdgcn_fmed3f(ru, 0.0f, qp.qmax) + 0.0f;
    g.wmin_s = -u;
    return g;
}

// Straight-through terms of one element with t = rint(w/s + v) + z,
// q = clamp(t, 0, Q) and m = [0 <= t <= Q] (= [q == t]):
//   c = dw^/ds = (q - z) - m w/s + (m - 1) wmin/s = (q - z) - (m ? w/s : wmin/s)
// (symmetric groups: the zero-point is fixed and wmin_s is 0), accumulated
// per group as sa = sum G c and s0 = sum (1 - m) G.  The group finishes
//   asymmetric: dalpha = mx/Q sa, dbeta = mn sum G ((1 - m) - c/Q) = mn (s0 - sa/Q)
//   symmetric : dalpha = max(mx, -mn)/(2^(b-1) - 1) sa, dbeta = 0.
__device__ __forceinline__ void ste_terms(float g, float q, float z, float ws, float wmin_s, bool m, float& sa,
                                          float& s0) {
    const float c = (q - z) - (m ? ws : wmin_s);
    sa += g * c;
    s0 += m ? 0.0f : g;
}

__device__ __forceinline__ void ste_group_grads(float mx, float mn, const QParams& qp, float sa, float s0,
                                                float& dalpha, float& dbeta) {
    if (qp.sym) {
        dalpha = div_qdiv(fmaxf(mx, -mn), qp.qdiv, qp.qdiv_inv) * sa;
        dbeta = 0.0f;
    } else {
        dalpha = div_qdiv(mx, qp.qdiv, qp.qdiv_inv) * sa;
        dbeta = mn * (s0 - sa * qp.qdiv_inv);
    }
}

// SignSGD move of V with dV = m G s: the sign of G s where the code is
// unclamped and G s is non-zero, else no move (as sign_step(v, m ? G s : 0)).
__device__ __forceinline__ float v_step(float v, float g, float s, bool m, float lr) {
    const float gs = g * s;
    const float step = (m && __builtin_fabsf(gs) > 0.0f) ? __builtin_copysignf(lr, gs) : 0.0f;
    return __builtin_amdgcn_fmed3f(v - step, -0.5f, 0.5f);
}

// w/s for the rounding u = w/s + v, computed as w * r with r within an ulp
// of 1/s (one multiply instead of an IEEE division), falling back to the
// correctly rounded w/s whenever u lies near a rounding tie.
// |w r - w/s| <= 3 * 2^-24 |w/s| (reciprocal and product), fl(w/s) is within
// 2^-24 |w/s|, and the two sums with v add 2^-24 |u| each, so fl(w*r + v)
// and fl(fl(w/s) + v) are within 6 * 2^-24 max(|w/s|, |u|) of each other.
// When u is farther than 2^-18 max(|w/s|, |u|, 1) from every half-integer
// both round to the same integer, so rint(u) is the IEEE-division code bit
// for bit.  The test is false for a NaN u (an unusable reciprocal), which
// also takes the division.  Returns the w/s value used (w*r, or fl(w/s) near
// a tie) and u.
__device__ __forceinline__ float scaled_weight(float w, float v, float s, float r, float thr, float& u, float& ru) {
    float ws = w * r;
    u = ws + v;
    ru = __builtin_rintf(u);
    if (!(__builtin_fabsf(u - ru) < thr)) {
        ws = w / s;
        u = ws + v;
        ru = __builtin_rintf(u);
    }
    return ws;
}

// scaled_weight on eight elements of one group, with one branch for the
// chunk: the products w * r are tested for near-ties first, and only a chunk
// that has one redoes those elements with the division (rare: a near-tie
// needs u within about 2^-18 of a half-integer).  Same values as eight
// scaled_weight calls.
__device__ __forceinline__ void scaled_weights8(const float w[8], const float v[8], float s, float r, float thr,
                                                float ws[8], float ru[8]) {
    bool near = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ws[i] = w[i] * r;
        const float u = ws[i] + v[i];
        ru[i] = __builtin_rintf(u);
        near |= !(__builtin_fabsf(u - ru[i]) < thr);
    }
    if (__builtin_expect(near, 0)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float u = ws[i] + v[i];
            if (!(__builtin_fabsf(u - ru[i]) < thr)) {
                ws[i] = w[i] / s;
                ru[i] = __builtin_rintf(ws[i] + v[i]);
            }
        }
    }
}

// Integer code of one element: t = rint(w/s + v) + z, q = clamp(t, 0, Q)
// (t is finite and never -0, so the median equals the clamp).
__device__ __forceinline__ float quant_code(float w, float v, const GroupQ& gq, float Q, float& t) {
    float u, ru;
    scaled_weight(w, v, gq.s, gq.r, gq.thr, u, ru);
    t = ru + gq.z;
    return __builtin_amdgcn_fmed3f(t, 0.0f, Q);
}

// Two floats to packed bf16 (round to nearest even, v_cvt_pk_bf16_f32): the
// same bits as f32_to_bf16 for every finite value.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// One SignSGD move: p - lr*sign(g), sign(0) = 0 (also for NaN), then clamp
// to [lo, hi].  p - (-lr) equals p + lr exactly.
__device__ __forceinline__ float sign_step(float p, float g, float lr, float lo, float hi) {
    const float step = (g < 0.0f || g > 0.0f) ? __builtin_copysignf(lr, g) : 0.0f;
    return fminf(fmaxf(p - step, lo), hi);
}

// Sum of the forward GEMM's per-tile loss partials by one wavefront in a
// fixed order: lane l adds partials l, l + 64, ... in turn, then an xor
// butterfly over the 64 lanes, which gives every lane the same bits.  Every
// wavefront that computes it, in any kernel, gets the same value, so the
// loss decision can be taken redundantly.
__device__ __forceinline__ double wave_loss_sum(const double* partials, int32_t np) {
    const int lane = (int)__lane_id();
    double acc = 0.0;
    for (int i = lane; i < np; i += 64) acc += partials[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    return acc;
}

// The best-loss snapshot decision of step t = st->step with loss L,
// written to the state: L is recorded, a non-finite loss halts the loop;
// on improvement (strict <) the evaluated buffer becomes the snapshot and
// the update writes the other one, otherwise it updates in place.
__device__ __forceinline__ void commit_decision(StepState* st, double* trace, int32_t iters, double L) {
    const int t = st->step;
    if (trace && t < iters) trace[t] = L;
    if (!__builtin_isfinite(L)) {
        st->halted = 1;
        return;
    }
    const int cur = st->cur;
    st->src = cur;
    if (L < st->best_loss) {
        st->best_loss = L;
        st->best_idx = cur;
        st->best_step = t;
        st->dst = 1 - cur;
    } else {
        st->dst = cur;
    }
    st->cur = st->dst;
    st->t_eval = t;
    st->step = t + 1;
}

// Loss of one step (L = sum of partials / (M N)) and its decision, by the
// first wavefront of the calling workgroup.
__device__ __forceinline__ void block_loss_decide(const double* partials, int32_t np, double inv_count,
                                                  StepState* st, double* trace, int32_t iters) {
    if (threadIdx.x >= 64) return;
    const double L = wave_loss_sum(partials, np) * inv_count;
    if (threadIdx.x == 0) commit_decision(st, trace, iters, L);
}

// ----------------------------------------------------------- launchers ----
// Every launcher enqueues on `stream` and returns the launch status.

// mx = max(0, max W_g), mn = min(0, min W_g) per group.
hipError_t launch_group_range(const void* W, bool w_bf16, int64_t N, int64_t K, int32_t g,
                              float* mx, float* mn, hipStream_t stream);

// Fused fake quantizer.  Parameters may be NULL (V = 0, alpha = beta = 1).
// When `state` is non-NULL the parameter pointers are two-buffer arrays
// (V0,V1 etc.) and the buffer index is state->cur; otherwise buffer 0.
struct QdqArgs {
    const void* W; bool w_bf16;
    int64_t N, K;
    QParams qp;
    const float* mx; const float* mn;
    const float* V[2]; const float* alpha[2]; const float* beta[2];
    const StepState* state;
    void* w_hat; int out_kind;        // 0 none, 1 fp32, 2 bf16, 3 fp32 w^ - W
    uint8_t* codes;                   // [N, K] or NULL
    float* scale; uint8_t* zero;      // [N, G] or NULL
    uint8_t* packed;                  // [N, K/2] int4 pairs or NULL
};
hipError_t launch_qdq(const QdqArgs& a, hipStream_t stream);

// Non-finite scan: sets *flag to 1 if any element of x is NaN/Inf.
hipError_t launch_nonfinite_scan(const void* x, bool bf16, int64_t n, int32_t* flag, hipStream_t stream);

// [S, T, K] -> [S, K, T] per-sample transpose (element size 2 or 4 bytes).
// dst[b][c][r] = src[b][r][c] for 16-bit elements with 16-byte accesses
// (transpose_b16_fits: rows, cols, lds, ldd multiples of 8, aligned bases).
bool transpose_b16_fits(const void* src, int64_t lds, const void* dst, int64_t ldd, int64_t rows, int64_t cols);
hipError_t launch_transpose_b16(const uint16_t* src, int64_t lds, int64_t sst, uint16_t* dst, int64_t ldd,
                                int64_t dstr, int64_t rows, int64_t cols, int64_t batch, hipStream_t stream);
hipError_t launch_transpose_pool(const void* x, void* xt, int elem_bytes, int64_t S, int64_t T, int64_t K,
                                 hipStream_t stream);

// bf16 -> fp32 widening copy.
hipError_t launch_widen_bf16(const uint16_t* x, float* y, int64_t n, hipStream_t stream);

// Fill kernels (used instead of memset so captured graphs stay plain).
hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t stream);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t stream);
// Step counter at step0, no snapshot yet, best loss best0 (+inf for a fresh run).
hipError_t launch_state_init(StepState* s, int32_t step0, double best0, hipStream_t stream);

// ---------------------------------------------------------------- GEMM ----
// C[i, j] = sum_r A[i, r] * B[j, r]  ("NT": both operands reduction-contiguous).
// Operand rows or reduction columns may be segmented by calibration sample:
// segment `seg` of length seg_len maps to sample ids[seg] at seg_stride.
// An unsegmented bf16 operand may instead be stored transposed (trans = 1):
// element (i, r) at base[r * ld + i], contiguous along the output index, as
// a weight read by a data-gradient GEMM is (plain-store GEMMs only).
struct Operand {
    const void* base;
    int64_t ld;           // elements between rows
    int64_t seg_stride;   // elements between samples
    int32_t seg_len;      // rows (or columns) per segment; 0 = not segmented
    int32_t seg_cols;     // 1: columns (reduction) segmented, 0: rows segmented
    int32_t trans;        // 1: stored [R, rows] (see above)
};

enum EpilogueKind {
    EPI_STORE = 0,        // C -> out fp32 [I, J] (row stride ldc)
    EPI_STE = 2,          // C = G = dL/dw^ [N, K]: straight-through backward, SignSGD
                          // update of V/alpha/beta and fake quantization of the
                          // updated state for the next step (see FusedUpdate)
    EPI_LOSS = 1,         // rows n, columns m: D = C - Yref^T[sample of m, n, token of m];
                          // partial sum of D^2; dY^T[n, m] = dscale * D
};

// Parameters of the fused wgrad epilogue (EPI_STE).  Rows of C are output
// rows n of the weight, columns are input columns k; a tile holds whole
// groups (the group size divides the tile width).
struct FusedUpdate {
    const void* W; bool w_bf16;
    QParams qp;
    int64_t K, G;
    const float* mx; const float* mn;
    float* V[2]; float* alpha[2]; float* beta[2];
    const float* lr; const float* lr_clip;   // per-step tables
    float clip_lo, clip_hi;
    uint16_t* what_next;                     // bf16 [N, K]
};

struct GemmArgs {
    Operand A, B;
    int64_t I, J, R;      // C is I x J, reduction length R
    const int32_t* sched; // sample table [*, nseg]; row chosen from `state`
    int32_t nseg;         // samples per step (B)
    const StepState* state; // NULL: schedule row 0
    int32_t after_decide; // 1: row state->t_eval (after the loss decision), 0: state->step
    int epi;
    float* out; int64_t ldc;          // EPI_STORE
    float* out2;                      // EPI_STORE split over the reduction (launch_gemm_bf16_split2):
                                      // out = the first half's sum, out2 = the second half's
    const float* yref; int32_t yref_T; int64_t yref_ld; int64_t yref_seg_stride;
                                      // EPI_LOSS: Yref^T per sample [S, N, T] (ld T, stride N*T)
    void* dyt; int64_t lddyt; bool dyt_bf16; float dscale;  // EPI_LOSS: dY^T [N, M]
    double* partials;                 // EPI_LOSS: one per workgroup
    FusedUpdate fu;                   // EPI_STE
    // EPI_STE with the loss decision of the step folded in (dec_partials
    // non-NULL; `state` must then be NULL): every wavefront sums the forward
    // GEMM's loss partials and takes the decision on dec_state itself, and
    // the last workgroup to arrive (dec_arrivals, zero between launches)
    // commits it, so no workgroup can read a committed state.
    const double* dec_partials; int32_t dec_np; double dec_inv;
    StepState* dec_state; double* dec_trace; int32_t dec_iters;
    int32_t* dec_arrivals;
};
// bf16 operands, v_mfma_f32_32x32x16_bf16.  Returns the number of workgroups
// (partials written) through *nblocks when non-NULL.
hipError_t launch_gemm_bf16(const GemmArgs& a, int32_t* nblocks, hipStream_t stream);
// fp32 operands, v_mfma_f32_32x32x2_f32.
hipError_t launch_gemm_f32(const GemmArgs& a, int32_t* nblocks, hipStream_t stream);
int32_t gemm_grid_blocks(bool bf16, int64_t I, int64_t J, int64_t R, int epi);
// A plain-store GEMM whose 256 x 256 tiles fill only half of the 256 CUs but
// whose reduction is long: both halves of the reduction run as their own
// tiles in one launch, writing a.out and a.out2 (the caller adds them; with
// two terms the sum does not depend on order).  Needs operands that are not
// gathered by sample and R a multiple of 128; gemm_split2_fits says whether
// the split pays and applies.
bool gemm_split2_fits(const GemmArgs& a);
hipError_t launch_gemm_bf16_split2(const GemmArgs& a, hipStream_t stream);
// Column width of the tile the bf16 launcher uses for this GEMM (a fused
// EPI_STE launch needs the group size to divide it); 0 if EPI_STE is not
// available for these sizes.
int32_t gemm_fused_tile_cols(int64_t I, int64_t J, int64_t R);


// ---------------------------------------------------------- tuning step ----
// Sum the partials in a fixed order, decide the snapshot, advance the step.
hipError_t launch_loss_decide(const double* partials, int32_t np, double inv_count, StepState* st,
                              double* loss_trace, int32_t iters, hipStream_t stream);

struct SteArgs {
    const float* G;       // [N, K]
    const void* W; bool w_bf16;
    int64_t N, K;
    QParams qp;
    const float* mx; const float* mn;
    const float* V[2]; const float* alpha[2]; const float* beta[2];
    const StepState* state;           // NULL: buffer 0
    float* dV;                        // [N, K]
    float* dalpha; float* dbeta;      // [N, G]
};
hipError_t launch_ste_bwd(const SteArgs& a, hipStream_t stream);

struct UpdateArgs {
    float* V[2]; float* alpha[2]; float* beta[2];
    const float* dV; const float* dalpha; const float* dbeta;
    int64_t nV, nG;
    const float* lr; const float* lr_clip;   // per-step tables
    float clip_lo, clip_hi;
    const StepState* state;
};
hipError_t launch_signsgd_update(const UpdateArgs& a, hipStream_t stream);

}  // namespace ar
