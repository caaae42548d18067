// Block-wise tuning of a Llama decoder block (AutoRound blog sec. 3: all
// linears of a Transformer decoder block tuned jointly on the MSE of the
// block output; one snapshot; the quantized output feeds the next block).
//
// One step (bf16 GEMM operands, fp32 accumulation and elementwise math):
//   qkv = h1_b w^_qkv^T            h1 = rmsnorm(x) of the pool, computed once
//   rope; attention                 q, k, v bf16 row-major and per head transposed; o, o^T, lse
//   attn = o w^_o^T; h = x_b + attn; h2 = rmsnorm(h); h2^T; tgt = y_ref^T - h^T
//   A^T, B^T = w^_{g,u} h2^T; Hh = silu(A) B; Y^T = w^_d Hh^T with the loss epilogue against tgt
//   loss decision
//   dY; dHh^T = w^_d^T dY^T; dA^T, dB^T and [dA dB]; dh2 = [dA dB] [w^_g; w^_u]; dh = dY + rmsnorm backward
//   dO = dh w^_o; attention backward (Di, dK/dV, dQ); inverse rope -> [dq dk dv]^T
//   weight gradients of down, gate, up, o, q, k, v, each with the fused
//   straight-through backward, SignSGD and next fake quantization (or the
//   separate kernels in the unfused form).
// The data-gradient GEMMs read w^_down, [w^_gate; w^_up] and w^_o in place
// as transposed operands, before the fused updates overwrite them.
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/libautoround.h"
#include "ar_internal.h"
#include "block_kernels.h"
#include "decoder_kernels.h"
#include "tuner.h"

using namespace ar;
using namespace ar::rt;

namespace ar {
namespace rt {
namespace {

enum { LQ = 0, LK, LV, LO, LG, LU, LD, NLIN };

enum DecoderKernel {
    KD_QDQ = 0,                                   // + linear index (7)
    KD_QKV = KD_QDQ + NLIN, KD_ROPE, KD_ATTN, KD_OPROJ, KD_NORM2, KD_H2T, KD_TGT, KD_GATE_UP, KD_SWIGLU,
    KD_DOWN_LOSS, KD_DECIDE, KD_DYT, KD_DH, KD_SWIGLU_BWD, KD_DH2, KD_NORM2_BWD, KD_DHT,
    KD_DA, KD_ATTN_PREP, KD_ATTN_DKDV, KD_ATTN_DQ, KD_ROPE_BWD,
    KD_WG,                                        // + linear index: stored gradient (unfused)
    KD_WGF = KD_WG + NLIN,                        // + linear index: fused backward + update + next QDQ
    KD_STE = KD_WGF + NLIN,
    KD_UPD = KD_STE + NLIN,
    KD_COUNT = KD_UPD + NLIN
};
const char* const kLinNames[NLIN] = {"q", "k", "v", "o", "gate", "up", "down"};
const char* const kStepNames[] = {"gemm_qkv", "rope_fwd", "attn_fwd", "gemm_oproj", "rmsnorm_residual",
                                  "transpose_h2", "loss_target", "gemm_gate_up_fwd", "swiglu_fwd",
                                  "gemm_down_fwd_loss", "loss_decide", "transpose_dy",
                                  "gemm_dh", "swiglu_bwd", "gemm_dh2",
                                  "rmsnorm_bwd", "transpose_dh", "gemm_do", "attn_bwd_prep",
                                  "attn_bwd_dkdv", "attn_bwd_dq", "rope_bwd"};
thread_local char g_name[64];

// Backward order: the MLP first (down before gate/up), then o, then q, k, v.
const int kWgradOrder[NLIN] = {LD, LG, LU, LO, LQ, LK, LV};

std::vector<int> decoder_sequence(bool fused, bool with_update) {
    std::vector<int> q;
    if (!fused)
        for (int i = 0; i < NLIN; ++i) q.push_back(KD_QDQ + i);
    for (int k = KD_QKV; k <= KD_ROPE_BWD; ++k) q.push_back(k);
    for (int j = 0; j < NLIN; ++j) {
        const int i = kWgradOrder[j];
        if (fused) {
            q.push_back(KD_WGF + i);
        } else {
            q.push_back(KD_WG + i);
            q.push_back(KD_STE + i);
        }
    }
    if (!fused && with_update)
        for (int i = 0; i < NLIN; ++i) q.push_back(KD_UPD + i);
    return q;
}

GemmArgs plain_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t I, int64_t J, int64_t R,
                    float* out, int64_t ldc, StepState* st) {
    GemmArgs a{};
    a.A.base = A; a.A.ld = lda;
    a.B.base = B; a.B.ld = ldb;
    a.I = I; a.J = J; a.R = R;
    a.state = st;
    a.epi = EPI_STORE; a.out = out; a.ldc = ldc;
    return a;
}

// dh2 [M, H] = [dA dB] [w^_gate; w^_up]: the stacked weights [2F, H] are the
// B operand read in place (transposed storage)
GemmArgs dh2_gemm(const ar_tuner* t) {
    const DecoderPart& d = *t->dec;
    GemmArgs a = plain_gemm(d.dAB, 2 * d.F, d.lin[LG].what, d.H, t->M, d.H, 2 * d.F, d.dh2, d.H, t->state);
    a.B.trans = 1;
    return a;
}

AttnShape attn_shape(const ar_tuner* t, int64_t nb) {
    const DecoderPart& d = *t->dec;
    AttnShape s;
    s.B = nb; s.T = t->T; s.nq = d.nq; s.nkv = d.nkv; s.d = d.d;
    return s;
}

RowMap step_map(const ar_tuner* t, int32_t after_decide) {
    RowMap m;
    m.sched = t->sched; m.nseg = t->B; m.state = t->state; m.after_decide = after_decide; m.T = t->T;
    return m;
}

RowMap identity_map() {
    RowMap m{};
    return m;
}

QdqArgs qdq_args(const ar_tuner* t, const BlockLinear& L) {
    QdqArgs a{};
    a.W = L.W; a.w_bf16 = t->w_bf16;
    a.N = L.N; a.K = L.K; a.qp = t->qp;
    a.mx = L.mx; a.mn = L.mn;
    for (int b = 0; b < 2; ++b) { a.V[b] = L.V[b]; a.alpha[b] = L.al[b]; a.beta[b] = L.be[b]; }
    a.state = t->state;
    a.w_hat = L.what; a.out_kind = 2;
    return a;
}

int64_t nqkv(const DecoderPart& d) { return (int64_t)(d.nq + 2 * d.nkv) * d.d; }

GemmArgs wgrad_args(const ar_tuner* t, int i, bool fused) {
    const DecoderPart& d = *t->dec;
    const BlockLinear& L = d.lin[i];
    const int64_t M = t->M;
    GemmArgs a{};
    switch (i) {
        case LQ: case LK: case LV: {
            const int64_t row0 = i == LQ ? 0 : (i == LK ? (int64_t)d.nq * d.d : (int64_t)(d.nq + d.nkv) * d.d);
            a.A.base = d.dqkvT + row0 * M; a.A.ld = M;
            a.B.base = d.h1T; a.B.ld = t->T; a.B.seg_stride = d.H * t->T; a.B.seg_len = (int32_t)t->T; a.B.seg_cols = 1;
            break;
        }
        case LO:
            a.A.base = d.dhT; a.A.ld = M;
            a.B.base = d.oT; a.B.ld = M;
            break;
        case LG: case LU:
            a.A.base = i == LG ? d.dAt : d.dBt; a.A.ld = M;
            a.B.base = d.h2T; a.B.ld = M;
            break;
        default:  // LD
            a.A.base = t->dyt; a.A.ld = M;
            a.B.base = d.Hht; a.B.ld = M;
            break;
    }
    a.I = L.N; a.J = L.K; a.R = M;
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

const char* decoder_kernel_name(int k) {
    if (k >= KD_QDQ && k < KD_QDQ + NLIN) snprintf(g_name, sizeof(g_name), "qdq_%s", kLinNames[k - KD_QDQ]);
    else if (k >= KD_QKV && k <= KD_ROPE_BWD) return kStepNames[k - KD_QKV];
    else if (k >= KD_WG && k < KD_WG + NLIN) snprintf(g_name, sizeof(g_name), "gemm_wgrad_%s", kLinNames[k - KD_WG]);
    else if (k >= KD_WGF && k < KD_WGF + NLIN)
        snprintf(g_name, sizeof(g_name), "gemm_wgrad_%s_ste_update", kLinNames[k - KD_WGF]);
    else if (k >= KD_STE && k < KD_STE + NLIN) snprintf(g_name, sizeof(g_name), "ste_bwd_%s", kLinNames[k - KD_STE]);
    else if (k >= KD_UPD && k < KD_UPD + NLIN)
        snprintf(g_name, sizeof(g_name), "signsgd_update_%s", kLinNames[k - KD_UPD]);
    else return "?";
    return g_name;
}

void decoder_release(ar_tuner* t) {
    if (t && t->dec) {
        delete t->dec;
        t->dec = nullptr;
    }
}

namespace {
ar_status enqueue_on(ar_tuner* t, int k, hipStream_t s);
}

ar_status decoder_enqueue_kernel(ar_tuner* t, int k) { return enqueue_on(t, k, t->ts); }

namespace {
ar_status enqueue_on(ar_tuner* t, int k, hipStream_t s) {
    DecoderPart& d = *t->dec;
    const int64_t M = t->M, H = d.H, F = d.F, T = t->T;
    const int64_t NQ = (int64_t)d.nq * d.d, NKV = (int64_t)d.nkv * d.d, NQKV = nqkv(d);
    if (k >= KD_QDQ && k < KD_QDQ + NLIN) {
        HIPCHK(launch_qdq(qdq_args(t, d.lin[k - KD_QDQ]), s));
        return AR_OK;
    }
    if (k >= KD_WG && k < KD_WG + NLIN) {
        HIPCHK(launch_gemm_bf16(wgrad_args(t, k - KD_WG, false), nullptr, s));
        return AR_OK;
    }
    if (k >= KD_WGF && k < KD_WGF + NLIN) {
        HIPCHK(launch_gemm_bf16(wgrad_args(t, k - KD_WGF, true), nullptr, s));
        return AR_OK;
    }
    if (k >= KD_STE && k < KD_STE + NLIN) {
        const BlockLinear& L = d.lin[k - KD_STE];
        SteArgs a{};
        a.G = L.Gb; a.W = L.W; a.w_bf16 = t->w_bf16;
        a.N = L.N; a.K = L.K; a.qp = t->qp; a.mx = L.mx; a.mn = L.mn;
        for (int i = 0; i < 2; ++i) { a.V[i] = L.V[i]; a.alpha[i] = L.al[i]; a.beta[i] = L.be[i]; }
        a.state = t->state; a.dV = L.dV; a.dalpha = L.dal; a.dbeta = L.dbe;
        HIPCHK(launch_ste_bwd(a, s));
        return AR_OK;
    }
    if (k >= KD_UPD && k < KD_UPD + NLIN) {
        const BlockLinear& L = d.lin[k - KD_UPD];
        UpdateArgs a{};
        for (int i = 0; i < 2; ++i) { a.V[i] = L.V[i]; a.alpha[i] = L.al[i]; a.beta[i] = L.be[i]; }
        a.dV = L.dV; a.dalpha = L.dal; a.dbeta = L.dbe;
        a.nV = L.N * L.K; a.nG = L.N * L.G;
        a.lr = t->lr; a.lr_clip = t->lrc; a.clip_lo = t->clip_lo; a.clip_hi = t->clip_hi;
        a.state = t->state;
        HIPCHK(launch_signsgd_update(a, s));
        return AR_OK;
    }
    const AttnShape as = attn_shape(t, t->B);
    switch (k) {
        case KD_QKV: {
            GemmArgs a{};
            a.A.base = d.h1; a.A.ld = H; a.A.seg_stride = T * H; a.A.seg_len = (int32_t)T; a.A.seg_cols = 0;
            a.B.base = d.what_qkv; a.B.ld = H;
            a.I = M; a.J = NQKV; a.R = H;
            a.sched = t->sched; a.nseg = t->B; a.state = t->state; a.after_decide = 0;
            a.epi = EPI_STORE; a.out = d.qkv; a.ldc = NQKV;
            HIPCHK(launch_gemm_bf16(a, nullptr, s));
            break;
        }
        case KD_ROPE:
            HIPCHK(launch_rope_fwd(d.qkv, d.cosT, d.sinT, as, d.qr, d.qT, d.kr, d.kT, d.vv, d.vT, s));
            break;
        case KD_ATTN:
            HIPCHK(launch_attn_fwd(d.qr, d.kr, d.vT, as, d.o, d.oT, d.lse, s));
            break;
        case KD_OPROJ:
            HIPCHK(launch_gemm_bf16(plain_gemm(d.o, NQ, d.lin[LO].what, NQ, M, H, NQ, d.attn, H, t->state), nullptr, s));
            break;
        case KD_NORM2:
            HIPCHK(launch_rmsnorm_fwd(d.X, d.xt == AR_BF16, step_map(t, 0), d.attn, M, H, d.w2, d.eps, d.h, d.r2, d.h2,
                                      true, s));
            break;
        case KD_H2T:
            HIPCHK(launch_transpose2d(d.h2, H, d.h2T, M, M, H, 2, s));
            break;
        case KD_TGT:
            HIPCHK(launch_yref_combine(t->Yref, step_map(t, 0), 0, d.h, t->B, H, T, 1.0f, -1.0f, d.tgt, s));
            break;
        case KD_GATE_UP:   // stacked w^_gate, w^_up [2F, H] -> A^T over B^T [2F, M]
            HIPCHK(launch_gemm_bf16(plain_gemm(d.lin[LG].what, H, d.h2, H, 2 * F, M, H, d.At, M, t->state), nullptr, s));
            break;
        case KD_SWIGLU:
            HIPCHK(launch_swiglu_fwd(d.At, d.Bt, F, M, M, d.Hht, d.Hh, true, s));
            break;
        case KD_DOWN_LOSS: {
            GemmArgs a{};
            a.A.base = d.lin[LD].what; a.A.ld = F;
            a.B.base = d.Hh; a.B.ld = F;
            a.I = H; a.J = M; a.R = F;
            a.state = t->state;
            a.epi = EPI_LOSS;
            a.yref = d.tgt; a.yref_T = (int32_t)T; a.yref_ld = T; a.yref_seg_stride = H * T;
            a.dyt = t->dyt; a.lddyt = M; a.dyt_bf16 = true;
            a.dscale = (float)(2.0 / ((double)M * (double)H));
            a.partials = t->partials;
            HIPCHK(launch_gemm_bf16(a, nullptr, s));
            break;
        }
        case KD_DECIDE:
            HIPCHK(launch_loss_decide(t->partials, t->nparts, 1.0 / ((double)M * (double)H), t->state, t->trace,
                                      t->iters, s));
            break;
        case KD_DYT:
            HIPCHK(launch_transpose2d(t->dyt, M, d.dy, H, H, M, 2, s));
            break;
        case KD_DH: {      // dHh^T [F, M] = w^_down^T dY^T, w^_down [H, F] read in place
            GemmArgs a = plain_gemm(d.lin[LD].what, F, d.dy, H, F, M, H, d.dHt, M, t->state);
            a.A.trans = 1;
            HIPCHK(launch_gemm_bf16(a, nullptr, s));
            break;
        }
        case KD_SWIGLU_BWD:   // dA^T over dB^T [2F, M] for the weight gradients, [dA dB] [M, 2F] for dh2
            HIPCHK(launch_swiglu_bwd_ab(d.dHt, d.At, d.Bt, F, M, M, d.dAt, d.dBt, d.dAB, s));
            break;
        case KD_DH2:
        {
            // dh2 = [dA dB] [w^_g; w^_u], the stacked weights [2F, H] read in
            // place: a long reduction (2F) on a grid of 256 x 256 tiles that
            // fills half the CUs, so both reduction halves run in one launch
            GemmArgs a = dh2_gemm(t);
            if (d.dh2b) {
                a.out2 = d.dh2b;
                HIPCHK(launch_gemm_bf16_split2(a, s));
            } else {
                HIPCHK(launch_gemm_bf16(a, nullptr, s));
            }
            break;
        }
        case KD_NORM2_BWD:
            HIPCHK(launch_rmsnorm_bwd(d.dh2, d.dh2b, d.h, d.r2, d.w2, d.dy, true, M, H, d.dh, true, s));
            break;
        case KD_DHT:
            HIPCHK(launch_transpose2d(d.dh, H, d.dhT, M, M, H, 2, s));
            break;
        case KD_DA: {      // dO [M, NQ] = dh w^_o, w^_o [H, NQ] read in place
            GemmArgs a = plain_gemm(d.dh, H, d.lin[LO].what, NQ, M, NQ, H, d.da, NQ, t->state);
            a.B.trans = 1;
            HIPCHK(launch_gemm_bf16(a, nullptr, s));
            break;
        }
        case KD_ATTN_PREP:
            HIPCHK(launch_attn_prep_bwd(d.da, d.o, as, d.Di, d.dOb, d.dOT, s));
            break;
        case KD_ATTN_DKDV:
            // one query head per workgroup: the nq / nkv partials of a KV head
            // are summed by the inverse rotation
            HIPCHK(launch_attn_bwd_dkdv(d.qr, d.qT, d.kr, d.vv, d.dOb, d.dOT, d.lse, d.Di, as, 1, M * NKV, d.dk, d.dv, s));
            break;
        case KD_ATTN_DQ:
            HIPCHK(launch_attn_bwd_dq(d.qr, d.kr, d.kT, d.vv, d.dOb, d.lse, d.Di, as, d.dq, s));
            break;
        case KD_ROPE_BWD:
            HIPCHK(launch_rope_bwd(d.dq, d.dk, d.dv, d.nq / d.nkv, M * NKV, d.cosT, d.sinT, as, d.dqkvT, s));
            break;
        default:
            return fail(AR_ERR_INVALID_ARG, "unknown decoder kernel %d", k);
    }
    return AR_OK;
}

ar_status validate_decoder(const ar_block_desc* d, const void* X, ar_dtype xt, int64_t S, int64_t T,
                           const ar_qconfig* qcfg, ar_gemm_mode mode, int32_t* g) {
    for (int i = 0; i < NLIN; ++i)
        if (!d->weights[i]) return fail(AR_ERR_INVALID_ARG, "weight %d (%s) is NULL", i, kLinNames[i]);
    if (!X) return fail(AR_ERR_INVALID_ARG, "X_pool is NULL");
    if (d->hidden <= 0 || d->ffn <= 0 || d->heads <= 0 || d->kv_heads <= 0 || d->head_dim <= 0)
        return fail(AR_ERR_INVALID_ARG, "hidden, ffn, heads, kv_heads and head_dim must be positive");
    if (d->heads % d->kv_heads != 0) return fail(AR_ERR_INVALID_ARG, "heads must be a multiple of kv_heads");
    if (S <= 0 || T <= 0) return fail(AR_ERR_INVALID_ARG, "S and T must be positive");
    if (!dtype_ok(d->weight_dtype) || !dtype_ok(xt)) return fail(AR_ERR_INVALID_ARG, "unknown dtype");
    if (!(d->norm_eps > 0.0f) || !(d->rope_theta > 0.0f)) return fail(AR_ERR_INVALID_ARG, "norm_eps and rope_theta must be > 0");
    if (mode != AR_GEMM_BF16)
        return fail(AR_ERR_UNSUPPORTED, "the decoder block runs bf16 GEMMs and attention only (AR_GEMM_BF16)");
    if (d->weight_dtype != AR_BF16 || xt != AR_BF16)
        return fail(AR_ERR_UNSUPPORTED, "the decoder block needs bf16 weights and X");
    if (d->head_dim != 64 && d->head_dim != 128) return fail(AR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (T % 64 != 0 || T > 256)
        return fail(AR_ERR_UNSUPPORTED, "tokens per sample T must be a multiple of 64 and at most 256, got %lld",
                    (long long)T);
    const int64_t nq = d->heads * d->head_dim;
    if (d->hidden % 64 || d->ffn % 64 || nq % 64)
        return fail(AR_ERR_UNSUPPORTED, "hidden, ffn and heads*head_dim must be multiples of 64");
    int32_t g1 = 0, g2 = 0, g3 = 0;
    ar_status st = check_qcfg(qcfg, d->hidden, &g1);
    if (st != AR_OK) return st;
    if ((st = check_qcfg(qcfg, d->ffn, &g2)) != AR_OK) return st;
    if ((st = check_qcfg(qcfg, nq, &g3)) != AR_OK) return st;
    if ((st = require_int_format(qcfg)) != AR_OK) return st;
    if (qcfg->group_size == -1)
        return fail(AR_ERR_UNSUPPORTED, "per-channel groups (-1) differ between the block's linears; give a size");
    if (d->hidden > (int64_t)1 << 20 || d->ffn > (int64_t)1 << 20 || S * T > (int64_t)1 << 28)
        return fail(AR_ERR_UNSUPPORTED, "problem too large");
    *g = g1;
    return AR_OK;
}

void carve_decoder(ar_tuner* t, Carve& c) {
    DecoderPart& d = *t->dec;
    const int64_t M = t->M, H = d.H, F = d.F, S = t->S, T = t->T;
    const int64_t NQ = (int64_t)d.nq * d.d, NKV = (int64_t)d.nkv * d.d, NQKV = nqkv(d);
    d.h1 = c.take<uint16_t>(S * T * H);
    d.h1T = c.take<uint16_t>(S * T * H);
    t->Yref = c.take<float>(S * T * H);
    d.cosT = c.take<float>(T * d.d / 2);
    d.sinT = c.take<float>(T * d.d / 2);
    d.what_qkv = c.take<uint16_t>(NQKV * H);
    d.what_gu = c.take<uint16_t>(2 * F * H);     // w^_gate over w^_up
    for (int i = 0; i < NLIN; ++i) {
        BlockLinear& L = d.lin[i];
        L.mx = c.take<float>(L.N * L.G);
        L.mn = c.take<float>(L.N * L.G);
        for (int b = 0; b < 2; ++b) {
            L.V[b] = c.take<float>(L.N * L.K);
            L.al[b] = c.take<float>(L.N * L.G);
            L.be[b] = c.take<float>(L.N * L.G);
        }
        if (i == LO || i == LD) L.what = c.take<uint16_t>(L.N * L.K);
        if (!L.fused) {
            L.Gb = c.take<float>(L.N * L.K);
            L.dV = c.take<float>(L.N * L.K);
            L.dal = c.take<float>(L.N * L.G);
            L.dbe = c.take<float>(L.N * L.G);
        }
    }
    {
        uint16_t* gu = d.what_gu;
        d.lin[LG].what = gu;
        d.lin[LU].what = gu ? gu + F * H : nullptr;
    }
    {
        uint16_t* base = static_cast<uint16_t*>(d.what_qkv);
        d.lin[LQ].what = base;
        d.lin[LK].what = base + NQ * H;
        d.lin[LV].what = base + (NQ + NKV) * H;
    }
    d.qkv = c.take<float>(M * NQKV);
    d.qr = c.take<uint16_t>(M * NQ);
    d.qT = c.take<uint16_t>(M * NQ);
    d.kr = c.take<uint16_t>(M * NKV);
    d.kT = c.take<uint16_t>(M * NKV);
    d.vv = c.take<uint16_t>(M * NKV);
    d.vT = c.take<uint16_t>(M * NKV);
    d.o = c.take<uint16_t>(M * NQ);
    d.oT = c.take<uint16_t>(M * NQ);
    d.lse = c.take<float>(M * d.nq);
    d.attn = c.take<float>(M * H);
    d.h = c.take<float>(M * H);
    d.r2 = c.take<float>(M);
    d.h2 = c.take<uint16_t>(M * H);
    d.h2T = c.take<uint16_t>(M * H);
    d.tgt = c.take<float>(M * H);
    d.At = c.take<float>(2 * F * M);              // A^T over B^T
    d.Bt = d.At ? d.At + F * M : nullptr;
    d.Hh = c.take<uint16_t>(M * F);
    d.Hht = c.take<uint16_t>(M * F);
    t->dyt = c.take<uint16_t>(H * M);
    d.dy = c.take<uint16_t>(M * H);
    d.dHt = c.take<float>(F * M);
    d.dAt = c.take<uint16_t>(2 * F * M);          // dA^T over dB^T
    d.dBt = d.dAt ? d.dAt + F * M : nullptr;
    d.dAB = c.take<uint16_t>(M * 2 * F);
    d.dh2 = c.take<float>(M * H);
    d.dh2b = gemm_split2_fits(dh2_gemm(t)) ? c.take<float>(M * H) : nullptr;
    d.dh = c.take<uint16_t>(M * H);
    d.dhT = c.take<uint16_t>(M * H);
    d.da = c.take<float>(M * NQ);
    d.Di = c.take<float>(M * d.nq);
    d.dOb = c.take<uint16_t>(M * NQ);
    d.dOT = c.take<uint16_t>(M * NQ);
    d.dq = c.take<float>(M * NQ);
    d.dk = c.take<float>((int64_t)(d.nq / d.nkv) * M * NKV);    // per query head of a group
    d.dv = c.take<float>((int64_t)(d.nq / d.nkv) * M * NKV);
    d.dqkvT = c.take<uint16_t>(NQKV * M);
    d.yq = c.take<float>(M * H);
    t->partials = c.take<double>(t->nparts);
    t->state = c.take<StepState>(1);
    const int64_t it = t->iters > 0 ? t->iters : 1;
    t->trace = c.take<double>(it);
    t->sched = c.take<int32_t>(it * t->B);
    t->lr = c.take<float>(it);
    t->lrc = c.take<float>(it);
    t->flag = c.take<int32_t>(1);
}

// Block forward over the pool samples [s0, s0 + nb) with GEMM operands w[7]
// (original weights, or the fake-quantized ones).  Reference mode adds the
// residual into Y_ref^T per sample; output mode writes rows y = h + mlp.
ar_status decoder_forward_chunk(ar_tuner* t, const void* const w[NLIN], int64_t s0, int64_t nb, bool yref_mode,
                                void* yrows, bool y_bf16) {
    DecoderPart& d = *t->dec;
    hipStream_t s = t->ts;
    const int64_t H = d.H, F = d.F, T = t->T, cols = nb * T;
    const int64_t NQ = (int64_t)d.nq * d.d, NKV = (int64_t)d.nkv * d.d, NQKV = nqkv(d);
    const uint16_t* h1c = static_cast<const uint16_t*>(d.h1) + s0 * T * H;
    const int64_t ncol[3] = {NQ, NKV, NKV};
    int64_t off = 0;
    for (int i = 0; i < 3; ++i) {
        HIPCHK(launch_gemm_bf16(plain_gemm(h1c, H, w[i], H, cols, ncol[i], H, d.qkv + off, NQKV, nullptr), nullptr, s));
        off += ncol[i];
    }
    const AttnShape as = attn_shape(t, nb);
    HIPCHK(launch_rope_fwd(d.qkv, d.cosT, d.sinT, as, d.qr, d.qT, d.kr, d.kT, d.vv, d.vT, s));
    HIPCHK(launch_attn_fwd(d.qr, d.kr, d.vT, as, d.o, d.oT, d.lse, s));
    HIPCHK(launch_gemm_bf16(plain_gemm(d.o, NQ, w[LO], NQ, cols, H, NQ, d.attn, H, nullptr), nullptr, s));
    const uint16_t* xc = static_cast<const uint16_t*>(d.X) + s0 * T * H;
    HIPCHK(launch_rmsnorm_fwd(xc, true, identity_map(), d.attn, cols, H, d.w2, d.eps, d.h, d.r2, d.h2, true, s));
    HIPCHK(launch_gemm_bf16(plain_gemm(w[LG], H, d.h2, H, F, cols, H, d.At, t->M, nullptr), nullptr, s));
    HIPCHK(launch_gemm_bf16(plain_gemm(w[LU], H, d.h2, H, F, cols, H, d.Bt, t->M, nullptr), nullptr, s));
    HIPCHK(launch_swiglu_fwd(d.At, d.Bt, F, cols, t->M, d.Hht, d.Hh, true, s));
    if (yref_mode) {
        for (int64_t j = 0; j < nb; ++j)
            HIPCHK(launch_gemm_bf16(plain_gemm(w[LD], F, d.Hh + j * T * F, F, H, T, F, t->Yref + (s0 + j) * H * T, T,
                                               nullptr), nullptr, s));
        HIPCHK(launch_yref_combine(t->Yref, identity_map(), s0, d.h, nb, H, T, 1.0f, 1.0f, t->Yref + s0 * H * T, s));
    } else {
        HIPCHK(launch_gemm_bf16(plain_gemm(d.Hh, F, w[LD], F, cols, H, F, d.yq, H, nullptr), nullptr, s));
        const int64_t o = s0 * T * H;
        void* dst = y_bf16 ? static_cast<void*>(static_cast<uint16_t*>(yrows) + o)
                           : static_cast<void*>(static_cast<float*>(yrows) + o);
        HIPCHK(launch_add_rows(d.yq, d.h, cols * H, dst, y_bf16, s));
    }
    return AR_OK;
}

}  // namespace

ar_status decoder_validate(const ar_block_desc* d, const void* X, ar_dtype xt, int64_t S, int64_t T,
                           const ar_qconfig* qcfg, ar_gemm_mode mode, int32_t* g) {
    if (!d) return fail(AR_ERR_INVALID_ARG, "block descriptor is NULL");
    return validate_decoder(d, X, xt, S, T, qcfg, mode, g);
}

ar_status decoder_create_impl(ar_tuner** out, const ar_block_desc* dsc, const void* X, ar_dtype xt, int64_t S,
                              int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* o, const float* const V0[],
                              const float* const al0[], const float* const be0[], void* stream,
                              const int32_t* ids_override) {
    if (!out) return fail(AR_ERR_INVALID_ARG, "out is NULL");
    int32_t g = 0;
    ar_status st = validate_decoder(dsc, X, xt, S, T, qcfg, o ? o->gemm_mode : AR_GEMM_BF16, &g);
    if (st != AR_OK) return st;
    if ((st = validate_opts(o, S)) != AR_OK) return st;
    if (!V0 || !al0 || !be0) return fail(AR_ERR_INVALID_ARG, "V, alpha and beta arrays must be non-NULL");
    for (int i = 0; i < NLIN; ++i)
        if (!V0[i] || !al0[i] || !be0[i]) return fail(AR_ERR_INVALID_ARG, "V/alpha/beta of linear %d is NULL", i);

    ar_tuner* t = new (std::nothrow) ar_tuner();
    DecoderPart* dp = new (std::nothrow) DecoderPart();
    if (!t || !dp) {
        delete t;
        delete dp;
        return fail(AR_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    t->dec = dp;
    DecoderPart& d = *dp;
    d.H = dsc->hidden; d.F = dsc->ffn; d.nq = (int32_t)dsc->heads; d.nkv = (int32_t)dsc->kv_heads;
    d.d = (int32_t)dsc->head_dim; d.eps = dsc->norm_eps; d.theta = dsc->rope_theta; d.xt = xt; d.X = X;
    d.w1 = static_cast<const float*>(dsc->norm_weights[0]);
    d.w2 = static_cast<const float*>(dsc->norm_weights[1]);
    const int64_t NQ = (int64_t)d.nq * d.d, NKV = (int64_t)d.nkv * d.d;
    const int64_t dims[NLIN][2] = {{NQ, d.H}, {NKV, d.H}, {NKV, d.H}, {d.H, NQ}, {d.F, d.H}, {d.F, d.H}, {d.H, d.F}};
    t->S = S; t->T = T; t->g = g;
    t->B = o->batch_samples; t->M = (int64_t)t->B * T; t->iters = o->iters;
    t->qp = make_qp(qcfg, g);
    t->bf16 = true;
    t->w_bf16 = true;
    t->return_last = o->return_last;
    t->clip_lo = o->clip_lo;
    t->clip_hi = o->clip_hi;
    t->host_trace = o->loss_trace;
    set_resume(t, o);
    t->user = static_cast<hipStream_t>(stream);
    bool fused = !o->unfused;
    for (int i = 0; i < NLIN; ++i) {
        BlockLinear& L = d.lin[i];
        L.N = dims[i][0]; L.K = dims[i][1]; L.G = L.K / g;
        L.W = dsc->weights[i];
        if (fused) {
            const int32_t cols = gemm_fused_tile_cols(L.N, L.K, t->M);
            fused = cols > 0 && g <= cols && cols % g == 0;
        }
    }
    for (BlockLinear& L : d.lin) L.fused = fused;
    t->fused = fused;
    t->nparts = gemm_grid_blocks(true, d.H, t->M, d.F, EPI_LOSS);
    t->seq = decoder_sequence(fused, true);

    Carve sizing;
    carve_decoder(t, sizing);
    t->ws_bytes = sizing.off + 256;
    if (o->max_workspace_bytes && t->ws_bytes > o->max_workspace_bytes) {
        const size_t need = t->ws_bytes;
        destroy_tuner(t);
        return fail(AR_ERR_OUT_OF_MEMORY, "workspace of %zu bytes exceeds max_workspace_bytes = %zu", need,
                    o->max_workspace_bytes);
    }
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
    carve_decoder(t, c);

#define TCHK(expr)                                                                   \
    do {                                                                             \
        hipError_t e_ = (expr);                                                      \
        if (e_ != hipSuccess) {                                                      \
            ar_status r_ = fail(AR_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
            destroy_tuner(t);                                                        \
            return r_;                                                               \
        }                                                                            \
    } while (0)
#define SCHK(expr)             \
    do {                       \
        ar_status s_ = (expr); \
        if (s_ != AR_OK) {     \
            destroy_tuner(t);  \
            return s_;         \
        }                      \
    } while (0)

    hipEvent_t ev;
    TCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    TCHK(hipEventRecord(ev, t->user));
    TCHK(hipStreamWaitEvent(t->ts, ev, 0));
    TCHK(hipEventDestroy(ev));

    SCHK(upload_tables(t, o, ids_override));
    // rotary tables: angle t * theta^(-2i/d), fp64 on the host
    std::vector<float> cs((size_t)(T * d.d / 2)), sn((size_t)(T * d.d / 2));
    for (int64_t tt = 0; tt < T; ++tt)
        for (int i = 0; i < d.d / 2; ++i) {
            const double ang = (double)tt * std::pow((double)d.theta, -2.0 * i / d.d);
            cs[(size_t)(tt * d.d / 2 + i)] = (float)std::cos(ang);
            sn[(size_t)(tt * d.d / 2 + i)] = (float)std::sin(ang);
        }
    TCHK(hipMemcpyAsync(d.cosT, cs.data(), cs.size() * sizeof(float), hipMemcpyHostToDevice, t->ts));
    TCHK(hipMemcpyAsync(d.sinT, sn.data(), sn.size() * sizeof(float), hipMemcpyHostToDevice, t->ts));

    TCHK(hipMemsetAsync(t->flag, 0, sizeof(int32_t), t->ts));
    for (const BlockLinear& L : d.lin) TCHK(launch_nonfinite_scan(L.W, true, L.N * L.K, t->flag, t->ts));
    TCHK(launch_nonfinite_scan(X, true, S * T * d.H, t->flag, t->ts));
    int32_t bad = 0;
    TCHK(hipMemcpyAsync(&bad, t->flag, sizeof(int32_t), hipMemcpyDeviceToHost, t->ts));
    TCHK(hipStreamSynchronize(t->ts));
    if (bad) {
        destroy_tuner(t);
        return fail(AR_ERR_NONFINITE, "a weight or X_pool holds NaN or Inf");
    }

    // h1 = rmsnorm(x) of the whole pool (the same for the reference and every
    // step), and its per-sample transpose for the q/k/v weight gradients
    TCHK(launch_rmsnorm_fwd(X, true, identity_map(), nullptr, S * T, d.H, d.w1, d.eps, nullptr, nullptr, d.h1, true,
                            t->ts));
    TCHK(launch_transpose_pool(d.h1, d.h1T, 2, S, T, d.H, t->ts));
    for (int i = 0; i < NLIN; ++i) {
        BlockLinear& L = d.lin[i];
        TCHK(launch_group_range(L.W, true, L.N, L.K, g, L.mx, L.mn, t->ts));
        TCHK(hipMemcpyAsync(L.V[0], V0[i], (size_t)(L.N * L.K) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
        TCHK(hipMemcpyAsync(L.al[0], al0[i], (size_t)(L.N * L.G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
        TCHK(hipMemcpyAsync(L.be[0], be0[i], (size_t)(L.N * L.G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    }
    TCHK(launch_state_init(t->state, t->start_step, t->best_in, t->ts));
    if (fused)
        for (int i = 0; i < NLIN; ++i) SCHK(decoder_enqueue_kernel(t, KD_QDQ + i));

    const void* w0[NLIN];
    for (int i = 0; i < NLIN; ++i) w0[i] = d.lin[i].W;
    for (int64_t s0 = 0; s0 < S; s0 += t->B) {
        const int64_t nb = (S - s0) < t->B ? (S - s0) : t->B;
        SCHK(decoder_forward_chunk(t, w0, s0, nb, true, nullptr, false));
    }
    TCHK(hipStreamSynchronize(t->ts));
#undef TCHK
#undef SCHK
    *out = t;
    return AR_OK;
}

ar_status decoder_finish_impl(ar_tuner* t, float* const V[], float* const al[], float* const be[], void* Yq,
                              float* best_loss, int32_t* best_step) {
    if (!V || !al || !be) return fail(AR_ERR_INVALID_ARG, "V, alpha and beta arrays must be non-NULL");
    for (int i = 0; i < NLIN; ++i)
        if (!V[i] || !al[i] || !be[i]) return fail(AR_ERR_INVALID_ARG, "V/alpha/beta of linear %d is NULL", i);
    DecoderPart& d = *t->dec;
    StepState hs;
    HIPCHK(hipMemcpyAsync(&hs, t->state, sizeof(StepState), hipMemcpyDeviceToHost, t->ts));
    std::vector<double> tr((size_t)(t->iters > 0 ? t->iters : 1));
    HIPCHK(hipMemcpyAsync(tr.data(), t->trace, tr.size() * sizeof(double), hipMemcpyDeviceToHost, t->ts));
    HIPCHK(hipStreamSynchronize(t->ts));
    int src = hs.best_idx;
    if (t->return_last || src < 0) src = hs.cur;
    for (int i = 0; i < NLIN; ++i) {
        const BlockLinear& L = d.lin[i];
        HIPCHK(hipMemcpyAsync(V[i], L.V[src], (size_t)(L.N * L.K) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
        HIPCHK(hipMemcpyAsync(al[i], L.al[src], (size_t)(L.N * L.G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
        HIPCHK(hipMemcpyAsync(be[i], L.be[src], (size_t)(L.N * L.G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    }
    if (Yq) {
        for (int i = 0; i < NLIN; ++i) {
            BlockLinear& L = d.lin[i];
            QdqArgs a = qdq_args(t, L);
            a.state = nullptr;
            a.V[0] = L.V[src]; a.alpha[0] = L.al[src]; a.beta[0] = L.be[src];
            HIPCHK(launch_qdq(a, t->ts));
        }
        const void* wq[NLIN];
        for (int i = 0; i < NLIN; ++i) wq[i] = d.lin[i].what;
        for (int64_t s0 = 0; s0 < t->S; s0 += t->B) {
            const int64_t nb = (t->S - s0) < t->B ? (t->S - s0) : t->B;
            ar_status st = decoder_forward_chunk(t, wq, s0, nb, false, Yq, d.xt == AR_BF16);
            if (st != AR_OK) return st;
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

ar_status decoder_grads_impl(const ar_block_desc* desc, const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                             const int32_t* ids, int32_t B, const ar_qconfig* qcfg, ar_gemm_mode mode,
                             const float* const V[], const float* const alpha[], const float* const beta[],
                             double* loss, float* const G[], float* const dV[], float* const dalpha[],
                             float* const dbeta[], void* stream) {
    ar_tune_opts o;
    ar_tune_opts_init(&o, AR_PRESET_DEFAULT);
    o.iters = 1;
    o.batch_samples = B;
    o.gemm_mode = mode;
    o.lr = 0.0f;
    o.lr_clip = 0.0f;
    o.unfused = 1;
    ar_tuner* t = nullptr;
    ar_status st = decoder_create_impl(&t, desc, X_pool, xt, S, T, qcfg, &o, V, alpha, beta, stream, ids);
    if (st != AR_OK) return st;
    const std::vector<int> seq = decoder_sequence(false, false);
    for (size_t k = 0; k < seq.size() && st == AR_OK; ++k) st = decoder_enqueue_kernel(t, seq[k]);
    StepState hs;
    double L = 0.0;
    if (st == AR_OK && hipMemcpyAsync(&hs, t->state, sizeof(StepState), hipMemcpyDeviceToHost, t->ts) != hipSuccess)
        st = fail(AR_ERR_HIP, "state copy");
    if (st == AR_OK && hipMemcpyAsync(&L, t->trace, sizeof(double), hipMemcpyDeviceToHost, t->ts) != hipSuccess)
        st = fail(AR_ERR_HIP, "loss copy");
    for (int i = 0; i < NLIN && st == AR_OK; ++i) {
        const BlockLinear& Ln = t->dec->lin[i];
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

}  // namespace rt
}  // namespace ar
