// Block-wise tuning of a SwiGLU MLP block (AutoRound blog sec. 3: the
// linears of a block are tuned jointly on the MSE of the block output, with
// one snapshot, and the quantized block's output feeds the next block).
//
// One step, all on the library stream, every kernel reading the step index,
// parameter buffers and minibatch row from the device step state:
//   [qdq gate/up/down]                  (unfused steps; fused ones get w^ from the previous update)
//   [transpose w^_down -> [F, H]]       (fp32 GEMM mode: operand of the dHh GEMM)
//   A^T = w^_g X_b^T, B^T = w^_u X_b^T  (fp32 [F, M])
//   Hh = silu(A) * B                    (GEMM type, [M, F] and [F, M])
//   Y^T = w^_d Hh^T, loss epilogue      (dY^T [H, M], loss partials)
//   loss decision                       (one workgroup; snapshot, next buffers)
//   transpose dY^T -> dY [M, H]
//   dHh^T = w^_d^T dY^T                 (fp32 [F, M])
//   dA^T, dB^T                          (gated-activation backward)
//   G_d = dY^T Hh, G_g = dA^T X_b, G_u = dB^T X_b
//                                       (fused: straight-through backward, SignSGD and the
//                                        next fake quantization in the GEMM epilogue)
//   [ste + update per linear]           (unfused steps)
// The GEMMs are the tuning GEMMs of the layer path (C[i, j] = sum_r A[i, r]
// B[j, r], both operands reduction-contiguous), which is why dY is also kept
// transposed; the bf16 dHh GEMM reads w^_down in place as a transposed
// operand (fragments by ds_read_b64_tr_b16), the fp32 one a transposed copy.
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/libautoround.h"
#include "ar_internal.h"
#include "block_kernels.h"
#include "tuner.h"

using namespace ar;
using namespace ar::rt;

namespace ar {
namespace rt {
namespace {

enum BlockKernel {
    KB_QDQ0 = 0, KB_QDQ1, KB_QDQ2,
    KB_WDT, KB_GATE_UP, KB_SWIGLU, KB_DOWN_LOSS, KB_DECIDE, KB_DYT, KB_DH, KB_SWIGLU_BWD,
    KB_WG0, KB_WG1, KB_WG2,          // weight gradients stored (unfused)
    KB_WGF0, KB_WGF1, KB_WGF2,       // weight gradients with the fused backward + update + next QDQ
    KB_STE0, KB_STE1, KB_STE2,
    KB_UPD0, KB_UPD1, KB_UPD2,
    KB_COUNT
};
const char* const kBlockNames[KB_COUNT] = {
    "qdq_gate", "qdq_up", "qdq_down",
    "transpose_down_what", "gemm_gate_up_fwd", "swiglu_fwd", "gemm_down_fwd_loss", "loss_decide",
    "transpose_dy", "gemm_dh", "swiglu_bwd",
    "gemm_wgrad_gate", "gemm_wgrad_up", "gemm_wgrad_down",
    "gemm_wgrad_gate_ste_update", "gemm_wgrad_up_ste_update", "gemm_wgrad_down_ste_update",
    "ste_bwd_gate", "ste_bwd_up", "ste_bwd_down",
    "signsgd_update_gate", "signsgd_update_up", "signsgd_update_down"};

std::vector<int> block_sequence(bool fused, bool with_update, bool bf16) {
    std::vector<int> q;
    if (!fused) q.insert(q.end(), {KB_QDQ0, KB_QDQ1, KB_QDQ2});
    if (!bf16) q.push_back(KB_WDT);
    q.insert(q.end(), {KB_GATE_UP, KB_SWIGLU, KB_DOWN_LOSS, KB_DECIDE, KB_DYT, KB_DH, KB_SWIGLU_BWD});
    if (fused) {
        // down first: its epilogue overwrites w^_down only after the dHh GEMM read it
        q.insert(q.end(), {KB_WGF2, KB_WGF0, KB_WGF1});
    } else {
        q.insert(q.end(), {KB_WG2, KB_STE2, KB_WG0, KB_STE0, KB_WG1, KB_STE1});
        if (with_update) q.insert(q.end(), {KB_UPD0, KB_UPD1, KB_UPD2});
    }
    return q;
}

size_t op_bytes(const ar_tuner* t) { return t->bf16 ? 2 : 4; }

QdqArgs qdq_args(const ar_tuner* t, const BlockLinear& L) {
    QdqArgs a{};
    a.W = L.W; a.w_bf16 = t->w_bf16;
    a.N = L.N; a.K = L.K; a.qp = t->qp;
    a.mx = L.mx; a.mn = L.mn;
    for (int b = 0; b < 2; ++b) { a.V[b] = L.V[b]; a.alpha[b] = L.al[b]; a.beta[b] = L.be[b]; }
    a.state = t->state;
    a.w_hat = L.what; a.out_kind = t->bf16 ? 2 : 1;
    return a;
}

hipError_t gemm(const ar_tuner* t, const GemmArgs& a, hipStream_t s) {
    return t->bf16 ? launch_gemm_bf16(a, nullptr, s) : launch_gemm_f32(a, nullptr, s);
}

// Weight-gradient GEMM of linear i: gate/up reduce dA^T / dB^T against the
// transposed pool gathered by the step's samples, down reduces dY^T against Hh^T.
GemmArgs wgrad_args(const ar_tuner* t, int i, bool fused) {
    const BlockPart& b = *t->blk;
    const BlockLinear& L = b.lin[i];
    GemmArgs a{};
    if (i == 2) {
        a.A.base = t->dyt; a.A.ld = t->M;
        a.B.base = b.Hht; a.B.ld = t->M;
    } else {
        a.A.base = i == 0 ? b.dAt : b.dBt; a.A.ld = t->M;
        a.B.base = t->XT; a.B.ld = t->T; a.B.seg_stride = b.H * t->T; a.B.seg_len = (int32_t)t->T; a.B.seg_cols = 1;
    }
    a.I = L.N; a.J = L.K; a.R = t->M;
    a.sched = t->sched; a.nseg = t->B; a.state = t->state; a.after_decide = 1;
    if (fused) {
        a.epi = EPI_STE;
        FusedUpdate& f = a.fu;
        f.W = L.W; f.w_bf16 = t->w_bf16; f.qp = t->qp; f.K = L.K; f.G = L.G;
        f.mx = L.mx; f.mn = L.mn;
        for (int k = 0; k < 2; ++k) { f.V[k] = L.V[k]; f.alpha[k] = L.al[k]; f.beta[k] = L.be[k]; }
        f.lr = t->lr; f.lr_clip = t->lrc; f.clip_lo = t->clip_lo; f.clip_hi = t->clip_hi;
        f.what_next = static_cast<uint16_t*>(L.what);
    } else {
        a.epi = EPI_STORE; a.out = L.Gb; a.ldc = L.K;
    }
    return a;
}

}  // namespace

const char* block_kernel_name(int k) { return (k >= 0 && k < KB_COUNT) ? kBlockNames[k] : "?"; }

void block_release(ar_tuner* t) {
    if (t && t->blk) {
        delete t->blk;
        t->blk = nullptr;
    }
}

ar_status block_enqueue_kernel(ar_tuner* t, int k) {
    hipStream_t s = t->ts;
    BlockPart& b = *t->blk;
    const int64_t M = t->M, H = b.H, F = b.F;
    const int eo = (int)op_bytes(t);
    switch (k) {
        case KB_QDQ0: case KB_QDQ1: case KB_QDQ2:
            HIPCHK(launch_qdq(qdq_args(t, b.lin[k - KB_QDQ0]), s));
            break;
        case KB_WDT:
            HIPCHK(launch_transpose_pool(b.lin[2].what, b.wdt, eo, 1, H, F, s));
            break;
        case KB_GATE_UP: {
            // w^_gate and w^_up are stacked [2F, H] and A^T, B^T stacked [2F, M]:
            // one GEMM (more tiles than the CUs, fewer idle in the last round)
            GemmArgs a{};
            a.A.base = b.lin[0].what; a.A.ld = H;
            a.B.base = t->Xop; a.B.ld = H; a.B.seg_stride = t->T * H; a.B.seg_len = (int32_t)t->T; a.B.seg_cols = 0;
            a.I = 2 * F; a.J = M; a.R = H;
            a.sched = t->sched; a.nseg = t->B; a.state = t->state; a.after_decide = 0;
            a.epi = EPI_STORE; a.out = b.At; a.ldc = M;
            HIPCHK(gemm(t, a, s));
            break;
        }
        case KB_SWIGLU:
            HIPCHK(launch_swiglu_fwd(b.At, b.Bt, F, M, M, b.Hht, b.Hh, t->bf16, s));
            break;
        case KB_DOWN_LOSS: {
            GemmArgs a{};
            a.A.base = b.lin[2].what; a.A.ld = F;
            a.B.base = b.Hh; a.B.ld = F;
            a.I = H; a.J = M; a.R = F;
            a.sched = t->sched; a.nseg = t->B; a.state = t->state; a.after_decide = 0;
            a.epi = EPI_LOSS;
            a.yref = t->Yref; a.yref_T = (int32_t)t->T; a.yref_ld = t->T; a.yref_seg_stride = H * t->T;
            a.dyt = t->dyt; a.lddyt = M; a.dyt_bf16 = t->bf16;
            a.dscale = (float)(2.0 / ((double)M * (double)H));
            a.partials = t->partials;
            HIPCHK(gemm(t, a, s));
            break;
        }
        case KB_DECIDE:
            HIPCHK(launch_loss_decide(t->partials, t->nparts, 1.0 / ((double)M * (double)H), t->state, t->trace,
                                      t->iters, s));
            break;
        case KB_DYT:
            HIPCHK(launch_transpose_pool(t->dyt, b.dy, eo, 1, H, M, s));
            break;
        case KB_DH: {
            // dHh^T [F, M] = w^_d^T dY^T: bf16 reads w^_down [H, F] as a
            // transposed operand, fp32 its transposed copy
            GemmArgs a{};
            if (t->bf16) {
                a.A.base = b.lin[2].what; a.A.ld = F; a.A.trans = 1;
            } else {
                a.A.base = b.wdt; a.A.ld = H;
            }
            a.B.base = b.dy; a.B.ld = H;
            a.I = F; a.J = M; a.R = H;
            a.state = t->state;
            a.epi = EPI_STORE; a.out = b.dHt; a.ldc = M;
            HIPCHK(gemm(t, a, s));
            break;
        }
        case KB_SWIGLU_BWD:
            HIPCHK(launch_swiglu_bwd(b.dHt, b.At, b.Bt, F, M, M, b.dAt, b.dBt, t->bf16, s));
            break;
        case KB_WG0: case KB_WG1: case KB_WG2: {
            const GemmArgs a = wgrad_args(t, k - KB_WG0, false);
            HIPCHK(gemm(t, a, s));
            break;
        }
        case KB_WGF0: case KB_WGF1: case KB_WGF2: {
            const GemmArgs a = wgrad_args(t, k - KB_WGF0, true);
            HIPCHK(launch_gemm_bf16(a, nullptr, s));
            break;
        }
        case KB_STE0: case KB_STE1: case KB_STE2: {
            const BlockLinear& L = b.lin[k - KB_STE0];
            SteArgs a{};
            a.G = L.Gb; a.W = L.W; a.w_bf16 = t->w_bf16;
            a.N = L.N; a.K = L.K; a.qp = t->qp; a.mx = L.mx; a.mn = L.mn;
            for (int i = 0; i < 2; ++i) { a.V[i] = L.V[i]; a.alpha[i] = L.al[i]; a.beta[i] = L.be[i]; }
            a.state = t->state; a.dV = L.dV; a.dalpha = L.dal; a.dbeta = L.dbe;
            HIPCHK(launch_ste_bwd(a, s));
            break;
        }
        case KB_UPD0: case KB_UPD1: case KB_UPD2: {
            const BlockLinear& L = b.lin[k - KB_UPD0];
            UpdateArgs a{};
            for (int i = 0; i < 2; ++i) { a.V[i] = L.V[i]; a.alpha[i] = L.al[i]; a.beta[i] = L.be[i]; }
            a.dV = L.dV; a.dalpha = L.dal; a.dbeta = L.dbe;
            a.nV = L.N * L.K; a.nG = L.N * L.G;
            a.lr = t->lr; a.lr_clip = t->lrc;
            a.clip_lo = t->clip_lo; a.clip_hi = t->clip_hi;
            a.state = t->state;
            HIPCHK(launch_signsgd_update(a, s));
            break;
        }
        default:
            return fail(AR_ERR_INVALID_ARG, "unknown block kernel %d", k);
    }
    return AR_OK;
}

namespace {

ar_status validate_block(const ar_block_desc* d, const void* X, ar_dtype xt, int64_t S, int64_t T,
                         const ar_qconfig* qcfg, ar_gemm_mode mode, int32_t* g) {
    if (!d) return fail(AR_ERR_INVALID_ARG, "block descriptor is NULL");
    if (d->kind != AR_BLOCK_MLP_SWIGLU) return fail(AR_ERR_INVALID_ARG, "unknown block kind %d", d->kind);
    if (!d->weights[0] || !d->weights[1] || !d->weights[2])
        return fail(AR_ERR_INVALID_ARG, "the gate, up and down weights must be non-NULL");
    if (!X) return fail(AR_ERR_INVALID_ARG, "X_pool is NULL");
    if (d->hidden <= 0 || d->ffn <= 0) return fail(AR_ERR_INVALID_ARG, "hidden and ffn must be positive");
    if (S <= 0 || T <= 0) return fail(AR_ERR_INVALID_ARG, "S and T must be positive");
    if (!dtype_ok(d->weight_dtype) || !dtype_ok(xt)) return fail(AR_ERR_INVALID_ARG, "unknown dtype");
    int32_t g1 = 0, g2 = 0;
    ar_status st = check_qcfg(qcfg, d->hidden, &g1);
    if (st != AR_OK) return st;
    st = check_qcfg(qcfg, d->ffn, &g2);
    if (st != AR_OK) return st;
    st = require_int_format(qcfg);
    if (st != AR_OK) return st;
    if (qcfg->group_size == -1)
        return fail(AR_ERR_UNSUPPORTED, "per-channel groups (-1) differ between the block's linears; give a size");
    if (mode != AR_GEMM_BF16 && mode != AR_GEMM_F32) return fail(AR_ERR_INVALID_ARG, "unknown gemm_mode %d", (int)mode);
    if (mode == AR_GEMM_BF16 && (d->weight_dtype != AR_BF16 || xt != AR_BF16))
        return fail(AR_ERR_UNSUPPORTED, "bf16 GEMM mode needs bf16 weights and X (fp32 inputs: use AR_GEMM_F32)");
    if (T % 64 != 0) return fail(AR_ERR_UNSUPPORTED, "tokens per sample T must be a multiple of 64, got %lld", (long long)T);
    if (d->hidden > (int64_t)1 << 20 || d->ffn > (int64_t)1 << 20 || S * T > (int64_t)1 << 28)
        return fail(AR_ERR_UNSUPPORTED, "problem too large");
    *g = g1;
    return AR_OK;
}

void carve_block(ar_tuner* t, Carve& c, bool need_w32, bool need_x32) {
    BlockPart& b = *t->blk;
    const size_t eo = op_bytes(t);
    const int64_t M = t->M, H = b.H, F = b.F;
    if (need_x32) t->Xop = c.take<float>(t->S * t->T * H);
    t->XT = c.take<char>(t->S * t->T * H * eo);
    t->Yref = c.take<float>(t->S * t->T * H);
    char* gu = c.take<char>(2 * F * H * eo);     // w^_gate over w^_up
    b.lin[0].what = gu;
    b.lin[1].what = gu ? gu + F * H * eo : nullptr;
    for (BlockLinear& L : b.lin) {
        if (need_w32) L.Wop = c.take<float>(L.N * L.K);
        L.mx = c.take<float>(L.N * L.G);
        L.mn = c.take<float>(L.N * L.G);
        for (int k = 0; k < 2; ++k) {
            L.V[k] = c.take<float>(L.N * L.K);
            L.al[k] = c.take<float>(L.N * L.G);
            L.be[k] = c.take<float>(L.N * L.G);
        }
        if (&L == &b.lin[2]) L.what = c.take<char>(L.N * L.K * eo);
        if (!L.fused) {
            L.Gb = c.take<float>(L.N * L.K);
            L.dV = c.take<float>(L.N * L.K);
            L.dal = c.take<float>(L.N * L.G);
            L.dbe = c.take<float>(L.N * L.G);
        }
    }
    float* ab = c.take<float>(2 * F * M);        // A^T over B^T
    b.At = ab;
    b.Bt = ab ? ab + F * M : nullptr;
    b.Hh = c.take<char>(M * F * eo);
    b.Hht = c.take<char>(F * M * eo);
    t->dyt = c.take<char>(H * M * eo);
    b.dy = c.take<char>(M * H * eo);
    b.wdt = t->bf16 ? nullptr : c.take<char>(F * H * eo);
    b.dHt = c.take<float>(F * M);
    b.dAt = c.take<char>(F * M * eo);
    b.dBt = c.take<char>(F * M * eo);
    b.yq = c.take<float>(M * H);
    t->partials = c.take<double>(t->nparts);
    t->state = c.take<StepState>(1);
    const int64_t it = t->iters > 0 ? t->iters : 1;
    t->trace = c.take<double>(it);
    t->sched = c.take<int32_t>(it * t->B);
    t->lr = c.take<float>(it);
    t->lrc = c.take<float>(it);
    t->flag = c.take<int32_t>(1);
}

// Block forward over the pool samples [s0, s0 + nb) with the GEMM operands
// w[0..2] (original weights for the reference, fake-quantized ones for the
// output): A^T, B^T, Hh into the step buffers, then either the reference
// Y_ref^T per sample (yref_mode) or the output rows Y [nb T, H] into `yrows`.
ar_status block_forward_chunk(ar_tuner* t, const void* const w[3], int64_t s0, int64_t nb, bool yref_mode,
                              float* yrows) {
    BlockPart& b = *t->blk;
    hipStream_t s = t->ts;
    const int64_t H = b.H, F = b.F, T = t->T, cols = nb * T;
    const size_t xe = op_bytes(t);
    for (int i = 0; i < 2; ++i) {
        GemmArgs a{};
        a.A.base = w[i]; a.A.ld = H;
        a.B.base = static_cast<const char*>(t->Xop) + (size_t)(s0 * T * H) * xe; a.B.ld = H;
        a.I = F; a.J = cols; a.R = H;
        a.epi = EPI_STORE; a.out = i == 0 ? b.At : b.Bt; a.ldc = t->M;
        HIPCHK(gemm(t, a, s));
    }
    HIPCHK(launch_swiglu_fwd(b.At, b.Bt, F, cols, t->M, b.Hht, b.Hh, t->bf16, s));
    if (yref_mode) {
        for (int64_t j = 0; j < nb; ++j) {
            GemmArgs a{};
            a.A.base = w[2]; a.A.ld = F;
            a.B.base = static_cast<const char*>(b.Hh) + (size_t)(j * T * F) * xe; a.B.ld = F;
            a.I = H; a.J = T; a.R = F;
            a.epi = EPI_STORE; a.out = t->Yref + (s0 + j) * H * T; a.ldc = T;
            HIPCHK(gemm(t, a, s));
        }
    } else {
        GemmArgs a{};
        a.A.base = b.Hh; a.A.ld = F;
        a.B.base = w[2]; a.B.ld = F;
        a.I = cols; a.J = H; a.R = F;
        a.epi = EPI_STORE; a.out = yrows; a.ldc = H;
        HIPCHK(gemm(t, a, s));
    }
    return AR_OK;
}

ar_status block_create_impl(ar_tuner** out, const ar_block_desc* d, const void* X, ar_dtype xt, int64_t S, int64_t T,
                            const ar_qconfig* qcfg, const ar_tune_opts* o, const float* const V0[],
                            const float* const al0[], const float* const be0[], void* stream,
                            const int32_t* ids_override) {
    if (!out) return fail(AR_ERR_INVALID_ARG, "out is NULL");
    int32_t g = 0;
    ar_status st = validate_block(d, X, xt, S, T, qcfg, o ? o->gemm_mode : AR_GEMM_BF16, &g);
    if (st != AR_OK) return st;
    st = validate_opts(o, S);
    if (st != AR_OK) return st;
    if (!V0 || !al0 || !be0) return fail(AR_ERR_INVALID_ARG, "V, alpha and beta arrays must be non-NULL");
    for (int i = 0; i < 3; ++i)
        if (!V0[i] || !al0[i] || !be0[i]) return fail(AR_ERR_INVALID_ARG, "V/alpha/beta of linear %d is NULL", i);

    ar_tuner* t = new (std::nothrow) ar_tuner();
    BlockPart* bp = new (std::nothrow) BlockPart();
    if (!t || !bp) {
        delete t;
        delete bp;
        return fail(AR_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    t->blk = bp;
    BlockPart& b = *bp;
    b.kind = d->kind;
    b.xt = xt;
    b.H = d->hidden;
    b.F = d->ffn;
    const int64_t dims[3][2] = {{b.F, b.H}, {b.F, b.H}, {b.H, b.F}};
    t->S = S; t->T = T; t->g = g;
    t->B = o->batch_samples; t->M = (int64_t)t->B * T; t->iters = o->iters;
    t->qp = make_qp(qcfg, g);
    t->bf16 = (o->gemm_mode == AR_GEMM_BF16);
    t->w_bf16 = (d->weight_dtype == AR_BF16);
    t->return_last = o->return_last;
    t->clip_lo = o->clip_lo;
    t->clip_hi = o->clip_hi;
    t->host_trace = o->loss_trace;
    set_resume(t, o);
    t->user = static_cast<hipStream_t>(stream);
    bool all_fused = t->bf16 && !o->unfused;
    for (int i = 0; i < 3; ++i) {
        BlockLinear& L = b.lin[i];
        L.N = dims[i][0]; L.K = dims[i][1]; L.G = L.K / g;
        L.W = d->weights[i];
        if (all_fused) {
            const int32_t cols = gemm_fused_tile_cols(L.N, L.K, t->M);
            all_fused = cols > 0 && g <= cols && cols % g == 0;
        }
    }
    for (BlockLinear& L : b.lin) L.fused = all_fused;
    t->fused = all_fused;
    t->nparts = gemm_grid_blocks(t->bf16, b.H, t->M, b.F, EPI_LOSS);
    t->seq = block_sequence(all_fused, true, t->bf16);
    const bool need_w32 = !t->bf16 && d->weight_dtype == AR_BF16;
    const bool need_x32 = !t->bf16 && xt == AR_BF16;

    Carve sizing;
    carve_block(t, sizing, need_w32, need_x32);
    t->ws_bytes = sizing.off + 256;
    if (o->max_workspace_bytes && t->ws_bytes > o->max_workspace_bytes) {
        const size_t need = t->ws_bytes;
        destroy_tuner(t);
        return fail(AR_ERR_OUT_OF_MEMORY, "workspace of %zu bytes exceeds max_workspace_bytes = %zu", need,
                    o->max_workspace_bytes);
    }
    // --- first HIP call ---
    hipError_t e = hipStreamCreateWithFlags(&t->ts, hipStreamNonBlocking);
    if (e != hipSuccess) {
        t->ts = nullptr;
        destroy_tuner(t);
        return fail(AR_ERR_HIP, "hipStreamCreate: %s", hipGetErrorString(e));
    }
    // stream-ordered on the caller's stream; the library's stream waits for
    // it through the event below, and destroy_tuner frees it on the same stream
    e = hipMallocAsync(&t->ws, t->ws_bytes, t->user);
    if (e != hipSuccess) {
        const size_t need = t->ws_bytes;
        (void)hipGetLastError();
        t->ws = nullptr;
        destroy_tuner(t);
        return fail(AR_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) failed: %s", need, hipGetErrorString(e));
    }
    Carve c;
    c.base = static_cast<char*>(t->ws);
    carve_block(t, c, need_w32, need_x32);
    for (BlockLinear& L : b.lin)
        if (!need_w32) L.Wop = L.W;
    if (!need_x32) t->Xop = X;

#define TCHK(expr)                                                                   \
    do {                                                                             \
        hipError_t e_ = (expr);                                                      \
        if (e_ != hipSuccess) {                                                      \
            ar_status r_ = fail(AR_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
            destroy_tuner(t);                                                        \
            return r_;                                                               \
        }                                                                            \
    } while (0)
#define SCHK(expr)                  \
    do {                            \
        ar_status s_ = (expr);      \
        if (s_ != AR_OK) {          \
            destroy_tuner(t);       \
            return s_;              \
        }                           \
    } while (0)

    hipEvent_t ev;
    TCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    TCHK(hipEventRecord(ev, t->user));
    TCHK(hipStreamWaitEvent(t->ts, ev, 0));
    TCHK(hipEventDestroy(ev));

    // minibatch rows and lr_t = lr (1 - t/T) (fp64, stored fp32)
    SCHK(upload_tables(t, o, ids_override));

    // non-finite inputs
    TCHK(hipMemsetAsync(t->flag, 0, sizeof(int32_t), t->ts));
    for (const BlockLinear& L : b.lin) TCHK(launch_nonfinite_scan(L.W, t->w_bf16, L.N * L.K, t->flag, t->ts));
    TCHK(launch_nonfinite_scan(X, xt == AR_BF16, S * T * b.H, t->flag, t->ts));
    int32_t bad = 0;
    TCHK(hipMemcpyAsync(&bad, t->flag, sizeof(int32_t), hipMemcpyDeviceToHost, t->ts));
    TCHK(hipStreamSynchronize(t->ts));
    if (bad) {
        destroy_tuner(t);
        return fail(AR_ERR_NONFINITE, "a weight or X_pool holds NaN or Inf");
    }

    if (need_x32) TCHK(launch_widen_bf16(static_cast<const uint16_t*>(X), const_cast<float*>(static_cast<const float*>(t->Xop)), S * T * b.H, t->ts));
    TCHK(launch_transpose_pool(t->Xop, t->XT, (int)op_bytes(t), S, T, b.H, t->ts));
    for (int i = 0; i < 3; ++i) {
        BlockLinear& L = b.lin[i];
        if (need_w32)
            TCHK(launch_widen_bf16(static_cast<const uint16_t*>(L.W), const_cast<float*>(static_cast<const float*>(L.Wop)), L.N * L.K, t->ts));
        TCHK(launch_group_range(L.W, t->w_bf16, L.N, L.K, g, L.mx, L.mn, t->ts));
        TCHK(hipMemcpyAsync(L.V[0], V0[i], (size_t)(L.N * L.K) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
        TCHK(hipMemcpyAsync(L.al[0], al0[i], (size_t)(L.N * L.G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
        TCHK(hipMemcpyAsync(L.be[0], be0[i], (size_t)(L.N * L.G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    }
    TCHK(launch_state_init(t->state, t->start_step, t->best_in, t->ts));
    if (all_fused)
        for (int i = 0; i < 3; ++i) SCHK(block_enqueue_kernel(t, KB_QDQ0 + i));

    // Reference output of every sample with the original weights (blog sec. 3
    // step 2), stored fp32 per sample as Y_ref^T [S, H, T].
    const void* w0[3] = {b.lin[0].Wop, b.lin[1].Wop, b.lin[2].Wop};
    for (int64_t s0 = 0; s0 < S; s0 += t->B) {
        const int64_t nb = (S - s0) < t->B ? (S - s0) : t->B;
        SCHK(block_forward_chunk(t, w0, s0, nb, true, nullptr));
    }
    TCHK(hipStreamSynchronize(t->ts));
#undef TCHK
#undef SCHK
    *out = t;
    return AR_OK;
}

ar_status block_finish_impl(ar_tuner* t, float* const V[], float* const al[], float* const be[], void* Yq,
                            ar_dtype yt, float* best_loss, int32_t* best_step) {
    if (!t) return fail(AR_ERR_INVALID_ARG, "tuner is NULL");
    if (!t->blk) return fail(AR_ERR_INVALID_ARG, "not a block tuner (use ar_tuner_finish)");
    if (!V || !al || !be) return fail(AR_ERR_INVALID_ARG, "V, alpha and beta arrays must be non-NULL");
    for (int i = 0; i < 3; ++i)
        if (!V[i] || !al[i] || !be[i]) return fail(AR_ERR_INVALID_ARG, "V/alpha/beta of linear %d is NULL", i);
    BlockPart& b = *t->blk;
    StepState hs;
    HIPCHK(hipMemcpyAsync(&hs, t->state, sizeof(StepState), hipMemcpyDeviceToHost, t->ts));
    std::vector<double> tr((size_t)(t->iters > 0 ? t->iters : 1));
    HIPCHK(hipMemcpyAsync(tr.data(), t->trace, tr.size() * sizeof(double), hipMemcpyDeviceToHost, t->ts));
    HIPCHK(hipStreamSynchronize(t->ts));
    int src = hs.best_idx;
    if (t->return_last || src < 0) src = hs.cur;
    for (int i = 0; i < 3; ++i) {
        const BlockLinear& L = b.lin[i];
        HIPCHK(hipMemcpyAsync(V[i], L.V[src], (size_t)(L.N * L.K) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
        HIPCHK(hipMemcpyAsync(al[i], L.al[src], (size_t)(L.N * L.G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
        HIPCHK(hipMemcpyAsync(be[i], L.be[src], (size_t)(L.N * L.G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    }
    if (Yq) {
        // the chosen state's fake-quantized weights, then the block forward of
        // every sample (the next block's input, blog sec. 3 step 7); this ends
        // the run: the step buffers and w^ are overwritten
        for (int i = 0; i < 3; ++i) {
            BlockLinear& L = b.lin[i];
            QdqArgs a = qdq_args(t, L);
            a.state = nullptr;
            a.V[0] = L.V[src]; a.alpha[0] = L.al[src]; a.beta[0] = L.be[src];
            HIPCHK(launch_qdq(a, t->ts));
        }
        const void* wq[3] = {b.lin[0].what, b.lin[1].what, b.lin[2].what};
        for (int64_t s0 = 0; s0 < t->S; s0 += t->B) {
            const int64_t nb = (t->S - s0) < t->B ? (t->S - s0) : t->B;
            const int64_t rows = nb * t->T, off = s0 * t->T * b.H;
            float* dst = yt == AR_F32 ? static_cast<float*>(Yq) + off : b.yq;
            ar_status st = block_forward_chunk(t, wq, s0, nb, false, dst);
            if (st != AR_OK) return st;
            if (yt == AR_BF16) HIPCHK(launch_narrow_bf16(b.yq, static_cast<uint16_t*>(Yq) + off, rows * b.H, t->ts));
        }
        t->steps_enqueued = t->iters - t->start_step;
    }
    HIPCHK(hipStreamSynchronize(t->ts));
    write_host_trace(t, hs, tr);
    if (best_loss) *best_loss = (float)hs.best_loss;
    if (best_step) *best_step = hs.best_step;
    ar_status st = join_user(t);
    if (st != AR_OK) return st;
    if (hs.halted) return fail(AR_ERR_NONFINITE, "the loss became non-finite at step %d; best state written", hs.step);
    return AR_OK;
}

}  // namespace

ar_status block_validate(const ar_block_desc* d, const void* X, ar_dtype xt, int64_t S, int64_t T,
                         const ar_qconfig* qcfg, ar_gemm_mode mode, int32_t* g) {
    return validate_block(d, X, xt, S, T, qcfg, mode, g);
}

}  // namespace rt
}  // namespace ar

// ============================================================ C ABI =======
extern "C" {

ar_status ar_block_tuner_create(ar_tuner** out, const ar_block_desc* desc, const void* X_pool, ar_dtype xt, int64_t S,
                                int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* opts, const float* const V0[],
                                const float* const alpha0[], const float* const beta0[], void* stream) {
    if (desc && desc->kind == AR_BLOCK_LLAMA_DECODER)
        return decoder_create_impl(out, desc, X_pool, xt, S, T, qcfg, opts, V0, alpha0, beta0, stream, nullptr);
    return block_create_impl(out, desc, X_pool, xt, S, T, qcfg, opts, V0, alpha0, beta0, stream, nullptr);
}

ar_status ar_block_tuner_finish(ar_tuner* t, float* const V[], float* const alpha[], float* const beta[],
                                void* Y_q_out, float* final_best_loss, int32_t* best_step) {
    if (t && t->dec) return decoder_finish_impl(t, V, alpha, beta, Y_q_out, final_best_loss, best_step);
    // the block output takes the dtype of the pool
    const ar_dtype yt = (t && t->blk) ? t->blk->xt : AR_F32;
    return block_finish_impl(t, V, alpha, beta, Y_q_out, yt, final_best_loss, best_step);
}

ar_status ar_tune_block(const ar_block_desc* desc, const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                        const ar_qconfig* qcfg, const ar_tune_opts* opts, float* const V[], float* const alpha[],
                        float* const beta[], void* Y_q_out, float* final_best_loss, int32_t* best_step, void* stream) {
    if (!V || !alpha || !beta) return fail(AR_ERR_INVALID_ARG, "V, alpha and beta arrays must be non-NULL");
    const bool dec = desc && desc->kind == AR_BLOCK_LLAMA_DECODER;
    const int nl = dec ? 7 : 3;
    const float* V0[7] = {};
    const float* a0[7] = {};
    const float* b0[7] = {};
    for (int i = 0; i < nl; ++i) {
        V0[i] = V[i];
        a0[i] = alpha[i];
        b0[i] = beta[i];
    }
    ar_tuner* t = nullptr;
    ar_status st = dec ? decoder_create_impl(&t, desc, X_pool, xt, S, T, qcfg, opts, V0, a0, b0, stream, nullptr)
                       : block_create_impl(&t, desc, X_pool, xt, S, T, qcfg, opts, V0, a0, b0, stream, nullptr);
    if (st != AR_OK) return st;
    st = run_impl(t, opts->iters - opts->start_step, AR_RUN_GRAPH);
    if (st == AR_OK || st == AR_ERR_NONFINITE) {
        ar_status st2 = dec ? decoder_finish_impl(t, V, alpha, beta, Y_q_out, final_best_loss, best_step)
                            : block_finish_impl(t, V, alpha, beta, Y_q_out, xt, final_best_loss, best_step);
        if (st == AR_OK) st = st2;
    }
    destroy_tuner(t);
    return st;
}

ar_status ar_block_grads(const ar_block_desc* desc, const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                         const int32_t* ids, int32_t B, const ar_qconfig* qcfg, ar_gemm_mode mode,
                         const float* const V[], const float* const alpha[], const float* const beta[], double* loss,
                         float* const G[], float* const dV[], float* const dalpha[], float* const dbeta[],
                         void* stream) {
    if (!ids) return fail(AR_ERR_INVALID_ARG, "ids is NULL");
    if (!loss) return fail(AR_ERR_INVALID_ARG, "loss is NULL");
    if (B < 1 || B > S) return fail(AR_ERR_INVALID_ARG, "B must be in [1, S]");
    for (int32_t j = 0; j < B; ++j)
        if (ids[j] < 0 || ids[j] >= S) return fail(AR_ERR_INVALID_ARG, "ids[%d] = %d is outside [0, S)", j, ids[j]);
    if (desc && desc->kind == AR_BLOCK_LLAMA_DECODER)
        return decoder_grads_impl(desc, X_pool, xt, S, T, ids, B, qcfg, mode, V, alpha, beta, loss, G, dV, dalpha,
                                  dbeta, stream);
    ar_tune_opts o;
    ar_tune_opts_init(&o, AR_PRESET_DEFAULT);
    o.iters = 1;
    o.batch_samples = B;
    o.gemm_mode = mode;
    o.lr = 0.0f;
    o.lr_clip = 0.0f;
    o.unfused = 1;
    ar_tuner* t = nullptr;
    ar_status st = block_create_impl(&t, desc, X_pool, xt, S, T, qcfg, &o, V, alpha, beta, stream, ids);
    if (st != AR_OK) return st;
    const std::vector<int> seq = block_sequence(false, false, t->bf16);
    for (size_t k = 0; k < seq.size() && st == AR_OK; ++k) st = block_enqueue_kernel(t, seq[k]);
    StepState hs;
    double L = 0.0;
    if (st == AR_OK && hipMemcpyAsync(&hs, t->state, sizeof(StepState), hipMemcpyDeviceToHost, t->ts) != hipSuccess)
        st = fail(AR_ERR_HIP, "state copy");
    if (st == AR_OK && hipMemcpyAsync(&L, t->trace, sizeof(double), hipMemcpyDeviceToHost, t->ts) != hipSuccess)
        st = fail(AR_ERR_HIP, "loss copy");
    for (int i = 0; i < 3 && st == AR_OK; ++i) {
        const BlockLinear& Ln = t->blk->lin[i];
        const size_t nk = (size_t)(Ln.N * Ln.K) * sizeof(float), ng = (size_t)(Ln.N * Ln.G) * sizeof(float);
        struct { float* dst; const float* src; size_t n; } cp[4] = {
            {G ? G[i] : nullptr, Ln.Gb, nk}, {dV ? dV[i] : nullptr, Ln.dV, nk},
            {dalpha ? dalpha[i] : nullptr, Ln.dal, ng}, {dbeta ? dbeta[i] : nullptr, Ln.dbe, ng}};
        for (auto& c : cp)
            if (st == AR_OK && c.dst && hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, t->ts) != hipSuccess)
                st = fail(AR_ERR_HIP, "gradient copy");
    }
    if (st == AR_OK && hipStreamSynchronize(t->ts) != hipSuccess) st = fail(AR_ERR_HIP, "synchronize");
    if (st == AR_OK) {
        *loss = L;
        if (hs.halted) st = fail(AR_ERR_NONFINITE, "loss is not finite");
    }
    if (st == AR_OK) st = join_user(t);
    destroy_tuner(t);
    return st;
}

}  // extern "C"
