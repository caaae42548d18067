// libautoround C ABI: argument checks, workspace, the tuning loop.
//
// The loop follows the AutoRound blog's per-block algorithm flow (sec. 3):
// wrap the layer with a fake quantizer, run the reference forward once, then
// repeat {QDQ forward, MSE + backward, SignSGD update} and keep the best state.
// One step is six kernels on one stream, all reading the step index, the
// parameter-buffer indices and the minibatch row from device memory, so the
// host enqueues (or replays a captured graph of) identical launches and never
// waits inside the loop.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/libautoround.h"
#include "ar_internal.h"
#include "format_kernels.h"
#include "tuner.h"
#include "w4a16.h"

using namespace ar;

namespace ar {
namespace rt {

thread_local std::string g_err;

ar_status fail(ar_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

// ------------------------------------------------------------ validation --
ar_status check_qcfg(const ar_qconfig* q, int64_t K, int32_t* g_out) {
    if (!q) return fail(AR_ERR_INVALID_ARG, "qconfig is NULL");
    if (q->bits < 2 || q->bits > 8) return fail(AR_ERR_INVALID_ARG, "bits must be in [2, 8], got %d", q->bits);
    if (q->sym != 0 && q->sym != 1) return fail(AR_ERR_INVALID_ARG, "sym must be 0 or 1, got %d", q->sym);
    if (q->format < AR_FMT_INT || q->format > AR_FMT_MXFP4)
        return fail(AR_ERR_INVALID_ARG, "unknown format %d", q->format);
    int64_t g = q->group_size == -1 ? K : q->group_size;
    if (g <= 0) return fail(AR_ERR_INVALID_ARG, "group_size must be > 0 or -1, got %d", q->group_size);
    if (K % g != 0) return fail(AR_ERR_INVALID_ARG, "group_size %lld does not divide K = %lld", (long long)g, (long long)K);
    if (g % 8 != 0) return fail(AR_ERR_UNSUPPORTED, "group_size must be a multiple of 8, got %lld", (long long)g);
    if (g > (int64_t)1 << 30) return fail(AR_ERR_UNSUPPORTED, "group_size too large");
    *g_out = (int32_t)g;
    return AR_OK;
}

ar_status require_int_format(const ar_qconfig* q) {
    if (q->format != AR_FMT_INT)
        return fail(AR_ERR_UNSUPPORTED, "format %d is a tensor-level QDQ (ar_qdq_rtn) only; tuning and packing "
                                        "run on the integer grid", q->format);
    return AR_OK;
}

bool dtype_ok(ar_dtype d) { return d == AR_F32 || d == AR_BF16; }
size_t esize(ar_dtype d) { return d == AR_BF16 ? 2 : 4; }

QParams make_qp(const ar_qconfig* q, int32_t g) {
    QParams p;
    p.bits = q->bits;
    p.group = g;
    p.qmax = (float)((1 << q->bits) - 1);
    p.sym = q->sym;
    p.qdiv = q->sym ? (float)((1 << (q->bits - 1)) - 1) : p.qmax;
    volatile float num = 1.0f;   // fl(1 / qdiv), divided at run time in IEEE fp32
    p.qdiv_inv = num / p.qdiv;
    return p;
}

}  // namespace rt
}  // namespace ar

using namespace ar::rt;


namespace ar {
namespace rt {

// Kernels of one step.  Unfused: fake quantization, loss GEMM, loss decision,
// weight-gradient GEMM, backward, update.  Fused (bf16 with the group size
// dividing the weight-gradient tile): the weight-gradient GEMM also runs the
// backward, the update and the next fake quantization.  The decision stays a
// one-workgroup kernel: folding it into the loss GEMM's last workgroup needs
// device-scope fences in every workgroup, which on this multi-XCD GPU write
// back each XCD's L2 and cost far more than the launch they save.
enum KernelId { K_QDQ = 0, K_FWD = 1, K_DECIDE = 2, K_WGRAD = 3, K_STE = 4, K_UPDATE = 5, K_WGRAD_FUSED = 6 };
const char* const kKernelNames[] = {"qdq_fwd", "gemm_fwd_loss", "loss_decide", "gemm_wgrad", "ste_bwd",
                                    "signsgd_update", "gemm_wgrad_ste_update"};

std::vector<int> step_sequence(const ar_tuner* t, bool fused, bool with_update) {
    std::vector<int> q;
    if (!fused) q.push_back(K_QDQ);
    q.push_back(K_FWD);
    if (fused) {
        q.push_back(K_WGRAD_FUSED);   // takes the loss decision itself
    } else {
        q.push_back(K_DECIDE);
        q.push_back(K_WGRAD);
        q.push_back(K_STE);
        if (with_update) q.push_back(K_UPDATE);
    }
    return q;
}

int num_kernels(const ar_tuner* t) { return (int)t->seq.size(); }
int kernel_at(const ar_tuner* t, int i) { return t->seq[(size_t)i]; }

ar_status enqueue_kernel(ar_tuner* t, int k) {
    if (t->blk) return block_enqueue_kernel(t, k);
    if (t->dec) return decoder_enqueue_kernel(t, k);
    hipStream_t s = t->ts;
    switch (k) {
        case 0: {
            QdqArgs a{};
            a.W = t->W; a.w_bf16 = t->w_bf16;
            a.N = t->N; a.K = t->K; a.qp = t->qp;
            a.mx = t->mx; a.mn = t->mn;
            for (int b = 0; b < 2; ++b) { a.V[b] = t->V[b]; a.alpha[b] = t->al[b]; a.beta[b] = t->be[b]; }
            a.state = t->state;
            // bf16 GEMMs take bf16(w^) and subtract the stored reference
            // output; fp32 validation GEMMs take w^ - W, so the loss GEMM
            // yields D = X (w^ - W)^T directly instead of the difference of
            // two fp32 GEMM outputs that agree in their leading digits
            a.w_hat = t->what; a.out_kind = t->bf16 ? 2 : 3;
            HIPCHK(launch_qdq(a, s));
            break;
        }
        case 1: {
            GemmArgs a{};
            a.A.base = t->what; a.A.ld = t->K;
            a.B.base = t->Xop; a.B.ld = t->K; a.B.seg_stride = t->T * t->K; a.B.seg_len = (int32_t)t->T; a.B.seg_cols = 0;
            a.I = t->N; a.J = t->M; a.R = t->K;
            a.sched = t->sched; a.nseg = t->B; a.state = t->state; a.after_decide = 0;
            a.epi = EPI_LOSS;
            a.yref = t->bf16 ? t->Yref : nullptr;
            a.yref_T = (int32_t)t->T; a.yref_ld = t->T; a.yref_seg_stride = t->N * t->T;
            a.dyt = t->dyt; a.lddyt = t->M; a.dyt_bf16 = t->bf16;
            a.dscale = (float)(2.0 / ((double)t->M * (double)t->N));
            a.partials = t->partials;
            HIPCHK(t->bf16 ? launch_gemm_bf16(a, nullptr, s) : launch_gemm_f32(a, nullptr, s));
            break;
        }
        case 2:
            HIPCHK(launch_loss_decide(t->partials, t->nparts, 1.0 / ((double)t->M * (double)t->N), t->state, t->trace,
                                      t->iters, s));
            break;
        case 3: {
            GemmArgs a{};
            a.A.base = t->dyt; a.A.ld = t->M;
            a.B.base = t->XT; a.B.ld = t->T; a.B.seg_stride = t->K * t->T; a.B.seg_len = (int32_t)t->T; a.B.seg_cols = 1;
            a.I = t->N; a.J = t->K; a.R = t->M;
            a.sched = t->sched; a.nseg = t->B; a.state = t->state; a.after_decide = 1;
            a.epi = EPI_STORE; a.out = t->Gb; a.ldc = t->K;
            HIPCHK(t->bf16 ? launch_gemm_bf16(a, nullptr, s) : launch_gemm_f32(a, nullptr, s));
            break;
        }
        case 4: {
            SteArgs a{};
            a.G = t->Gb; a.W = t->W; a.w_bf16 = t->w_bf16;
            a.N = t->N; a.K = t->K; a.qp = t->qp; a.mx = t->mx; a.mn = t->mn;
            for (int b = 0; b < 2; ++b) { a.V[b] = t->V[b]; a.alpha[b] = t->al[b]; a.beta[b] = t->be[b]; }
            a.state = t->state; a.dV = t->dV; a.dalpha = t->dal; a.dbeta = t->dbe;
            HIPCHK(launch_ste_bwd(a, s));
            break;
        }
        case K_WGRAD_FUSED: {
            GemmArgs a{};
            a.A.base = t->dyt; a.A.ld = t->M;
            a.B.base = t->XT; a.B.ld = t->T; a.B.seg_stride = t->K * t->T; a.B.seg_len = (int32_t)t->T; a.B.seg_cols = 1;
            a.I = t->N; a.J = t->K; a.R = t->M;
            a.sched = t->sched; a.nseg = t->B;
            a.dec_partials = t->partials; a.dec_np = t->nparts; a.dec_inv = 1.0 / ((double)t->M * (double)t->N);
            a.dec_state = t->state; a.dec_trace = t->trace; a.dec_iters = t->iters; a.dec_arrivals = t->arrivals;
            a.epi = EPI_STE;
            FusedUpdate& f = a.fu;
            f.W = t->W; f.w_bf16 = t->w_bf16; f.qp = t->qp; f.K = t->K; f.G = t->G;
            f.mx = t->mx; f.mn = t->mn;
            for (int b = 0; b < 2; ++b) { f.V[b] = t->V[b]; f.alpha[b] = t->al[b]; f.beta[b] = t->be[b]; }
            f.lr = t->lr; f.lr_clip = t->lrc; f.clip_lo = t->clip_lo; f.clip_hi = t->clip_hi;
            f.what_next = static_cast<uint16_t*>(t->what);
            HIPCHK(launch_gemm_bf16(a, nullptr, s));
            break;
        }
        case 5: {
            UpdateArgs a{};
            for (int b = 0; b < 2; ++b) { a.V[b] = t->V[b]; a.alpha[b] = t->al[b]; a.beta[b] = t->be[b]; }
            a.dV = t->dV; a.dalpha = t->dal; a.dbeta = t->dbe;
            a.nV = t->N * t->K; a.nG = t->N * t->G;
            a.lr = t->lr; a.lr_clip = t->lrc;
            a.clip_lo = t->clip_lo; a.clip_hi = t->clip_hi;
            a.state = t->state;
            HIPCHK(launch_signsgd_update(a, s));
            break;
        }
    }
    return AR_OK;
}

ar_status enqueue_step(ar_tuner* t) {
    for (int i = 0; i < num_kernels(t); ++i) {
        ar_status st = enqueue_kernel(t, kernel_at(t, i));
        if (st != AR_OK) return st;
    }
    return AR_OK;
}

ar_status validate_problem(const void* W, ar_dtype wt, int64_t N, int64_t K, const void* X, ar_dtype xt, int64_t S,
                           int64_t T, const ar_qconfig* qcfg, ar_gemm_mode mode, int32_t* g) {
    if (!W) return fail(AR_ERR_INVALID_ARG, "W is NULL");
    if (!X) return fail(AR_ERR_INVALID_ARG, "X_pool is NULL");
    if (N <= 0 || K <= 0) return fail(AR_ERR_INVALID_ARG, "N and K must be positive (N=%lld, K=%lld)", (long long)N, (long long)K);
    if (S <= 0 || T <= 0) return fail(AR_ERR_INVALID_ARG, "S and T must be positive (S=%lld, T=%lld)", (long long)S, (long long)T);
    if (!dtype_ok(wt) || !dtype_ok(xt)) return fail(AR_ERR_INVALID_ARG, "unknown dtype");
    ar_status st = check_qcfg(qcfg, K, g);
    if (st != AR_OK) return st;
    st = require_int_format(qcfg);
    if (st != AR_OK) return st;
    if (mode != AR_GEMM_BF16 && mode != AR_GEMM_F32) return fail(AR_ERR_INVALID_ARG, "unknown gemm_mode %d", (int)mode);
    if (mode == AR_GEMM_BF16 && (wt != AR_BF16 || xt != AR_BF16))
        return fail(AR_ERR_UNSUPPORTED, "bf16 GEMM mode needs bf16 W and X (fp32 inputs: use AR_GEMM_F32)");
    if (T % 64 != 0) return fail(AR_ERR_UNSUPPORTED, "tokens per sample T must be a multiple of 64, got %lld", (long long)T);
    if (N > (int64_t)1 << 24 || K > (int64_t)1 << 24 || S * T > (int64_t)1 << 28)
        return fail(AR_ERR_UNSUPPORTED, "problem too large");
    return AR_OK;
}

ar_status validate_opts(const ar_tune_opts* o, int64_t S) {
    if (!o) return fail(AR_ERR_INVALID_ARG, "opts is NULL");
    if (o->iters < 0) return fail(AR_ERR_INVALID_ARG, "iters must be >= 0");
    if (!(o->lr >= 0.0f) || !(o->lr_clip >= 0.0f) || !std::isfinite(o->lr) || !std::isfinite(o->lr_clip))
        return fail(AR_ERR_INVALID_ARG, "lr and lr_clip must be finite and >= 0");
    if (!(o->clip_lo >= 0.0f) || !(o->clip_lo <= o->clip_hi) || !std::isfinite(o->clip_hi))
        return fail(AR_ERR_INVALID_ARG, "clip box must satisfy 0 <= clip_lo <= clip_hi");
    if (o->lr_decay != 0 && o->lr_decay != 1) return fail(AR_ERR_INVALID_ARG, "lr_decay must be 0 or 1");
    if (o->start_step < 0 || o->start_step > o->iters)
        return fail(AR_ERR_INVALID_ARG, "start_step must be in [0, iters = %d], got %d", o->iters, o->start_step);
    if (!(o->best_loss_in >= 0.0f))
        return fail(AR_ERR_INVALID_ARG, "best_loss_in must be >= 0 (+inf: no earlier snapshot)");
    if (o->batch_samples < 1 || o->batch_samples > S)
        return fail(AR_ERR_INVALID_ARG, "batch_samples must be in [1, S=%lld], got %d", (long long)S, o->batch_samples);
    if (o->schedule) {
        const int64_t n = (int64_t)o->iters * o->batch_samples;
        for (int64_t i = 0; i < n; ++i)
            if (o->schedule[i] < 0 || o->schedule[i] >= S)
                return fail(AR_ERR_INVALID_ARG, "schedule[%lld] = %d is outside [0, %lld)", (long long)i,
                            o->schedule[i], (long long)S);
    }
    return AR_OK;
}

void destroy_tuner(ar_tuner* t) {
    if (!t) return;
    if (t->gexec) hipGraphExecDestroy(t->gexec);
    if (t->gexec_multi) hipGraphExecDestroy(t->gexec_multi);
    if (t->ts) hipStreamSynchronize(t->ts);
    // nothing on the library's stream uses the workspace any more; the caller's
    // stream, which it was allocated on, returns it in its own order
    if (t->ws) hipFreeAsync(t->ws, t->user);
    if (t->ts) hipStreamDestroy(t->ts);
    block_release(t);
    decoder_release(t);
    delete t;
}

// Lay out (or, with base == nullptr, size) the workspace.
void carve(ar_tuner* t, Carve& c, bool need_w32, bool need_x32) {
    const size_t eo = t->bf16 ? 2 : 4;
    if (need_w32) t->Wop = c.take<float>(t->N * t->K);
    if (need_x32) t->Xop = c.take<float>(t->S * t->T * t->K);
    t->XT = c.take<char>(t->S * t->T * t->K * eo);
    if (t->bf16) t->Yref = c.take<float>(t->S * t->T * t->N);   // fp32 mode forms D from w^ - W
    t->mx = c.take<float>(t->N * t->G);
    t->mn = c.take<float>(t->N * t->G);
    for (int b = 0; b < 2; ++b) {
        t->V[b] = c.take<float>(t->N * t->K);
        t->al[b] = c.take<float>(t->N * t->G);
        t->be[b] = c.take<float>(t->N * t->G);
    }
    t->what = c.take<char>(t->N * t->K * eo);
    t->dyt = c.take<char>(t->N * t->M * eo);
    t->Gb = c.take<float>(t->N * t->K);
    t->dV = c.take<float>(t->N * t->K);
    t->dal = c.take<float>(t->N * t->G);
    t->dbe = c.take<float>(t->N * t->G);
    t->partials = c.take<double>(t->nparts);
    t->state = c.take<StepState>(1);
    const int64_t it = t->iters > 0 ? t->iters : 1;
    t->trace = c.take<double>(it);
    t->sched = c.take<int32_t>(it * t->B);
    t->lr = c.take<float>(it);
    t->lrc = c.take<float>(it);
    t->flag = c.take<int32_t>(1);
    t->arrivals = c.take<int32_t>(1);
}

// Minibatch rows and step sizes of every step index 0..iters-1, uploaded to
// the tuner's tables; the step counter starts at opts->start_step and reads
// from there.  lr_t = fp32(fp32(lr) * (1 - t/T)) with the product in fp64
// (linear decay), or fp32(lr) constant.
ar_status upload_tables(ar_tuner* t, const ar_tune_opts* o, const int32_t* ids_override) {
    const int64_t it = t->iters > 0 ? t->iters : 1;
    std::vector<int32_t> sched((size_t)(it * t->B));
    for (int64_t s = 0; s < it; ++s)
        for (int32_t b = 0; b < t->B; ++b) {
            int32_t v = b;
            if (ids_override) v = ids_override[b];
            else if (o->schedule && s < o->iters) v = o->schedule[s * t->B + b];
            sched[(size_t)(s * t->B + b)] = v;
        }
    std::vector<float> lrs((size_t)it), lrcs((size_t)it);
    for (int64_t s = 0; s < it; ++s) {
        const double f = o->lr_decay ? 1.0 - (double)s / (double)(t->iters > 0 ? t->iters : 1) : 1.0;
        lrs[(size_t)s] = (float)((double)o->lr * f);
        lrcs[(size_t)s] = (float)((double)o->lr_clip * f);
    }
    HIPCHK(hipMemcpyAsync(t->sched, sched.data(), sched.size() * sizeof(int32_t), hipMemcpyHostToDevice, t->ts));
    HIPCHK(hipMemcpyAsync(t->lr, lrs.data(), lrs.size() * sizeof(float), hipMemcpyHostToDevice, t->ts));
    HIPCHK(hipMemcpyAsync(t->lrc, lrcs.data(), lrcs.size() * sizeof(float), hipMemcpyHostToDevice, t->ts));
    // the host vectors go out of scope: make the copies complete first
    HIPCHK(hipStreamSynchronize(t->ts));
    return AR_OK;
}

// Per-step losses of the evaluated steps into the caller's trace; entries of
// steps before start_step and of steps not run are left alone / NaN.
void write_host_trace(const ar_tuner* t, const StepState& hs, const std::vector<double>& tr) {
    if (!t->host_trace) return;
    for (int32_t i = t->start_step; i < t->iters; ++i)
        t->host_trace[i] = (i < hs.step || (hs.halted && i == hs.step)) ? (float)tr[(size_t)i] : NAN;
}

void set_resume(ar_tuner* t, const ar_tune_opts* o) {
    t->start_step = o->start_step;
    t->best_in = (double)o->best_loss_in;
}

ar_status create_impl(ar_tuner** out, const void* W, ar_dtype wt, int64_t N, int64_t K, const void* X, ar_dtype xt,
                      int64_t S, int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* o, const float* V0,
                      const float* al0, const float* be0, void* stream, const int32_t* ids_override) {
    if (!out) return fail(AR_ERR_INVALID_ARG, "out is NULL");
    int32_t g = 0;
    ar_status st = validate_problem(W, wt, N, K, X, xt, S, T, qcfg, o ? o->gemm_mode : AR_GEMM_BF16, &g);
    if (st != AR_OK) return st;
    st = validate_opts(o, S);
    if (st != AR_OK) return st;
    if (!V0 || !al0 || !be0) return fail(AR_ERR_INVALID_ARG, "V, alpha and beta must be non-NULL");

    ar_tuner* t = new (std::nothrow) ar_tuner();
    if (!t) return fail(AR_ERR_OUT_OF_MEMORY, "host allocation failed");
    t->N = N; t->K = K; t->S = S; t->T = T; t->g = g; t->G = K / g;
    t->B = o->batch_samples; t->M = (int64_t)t->B * T; t->iters = o->iters;
    t->qp = make_qp(qcfg, g);
    t->bf16 = (o->gemm_mode == AR_GEMM_BF16);
    t->w_bf16 = (wt == AR_BF16);
    t->return_last = o->return_last;
    t->clip_lo = o->clip_lo;
    t->clip_hi = o->clip_hi;
    t->host_trace = o->loss_trace;
    set_resume(t, o);
    t->user = static_cast<hipStream_t>(stream);
    t->nparts = gemm_grid_blocks(t->bf16, t->N, t->M, t->K, EPI_LOSS);
    if (t->bf16 && !o->unfused) {
        const int32_t cols = gemm_fused_tile_cols(t->N, t->K, t->M);
        t->fused = cols > 0 && g <= cols && cols % g == 0;
    }
    t->seq = step_sequence(t, t->fused, true);
    const bool need_w32 = !t->bf16 && wt == AR_BF16;
    const bool need_x32 = !t->bf16 && xt == AR_BF16;

    Carve sizing;
    carve(t, sizing, need_w32, need_x32);
    t->ws_bytes = sizing.off + 256;
    if (o->max_workspace_bytes && t->ws_bytes > o->max_workspace_bytes) {
        size_t need = t->ws_bytes;
        delete t;
        return fail(AR_ERR_OUT_OF_MEMORY, "workspace of %zu bytes exceeds max_workspace_bytes = %zu", need,
                    o->max_workspace_bytes);
    }
    // --- first HIP call ---
    hipError_t e = hipStreamCreateWithFlags(&t->ts, hipStreamNonBlocking);
    if (e != hipSuccess) {
        delete t;
        return fail(AR_ERR_HIP, "hipStreamCreate: %s", hipGetErrorString(e));
    }
    // stream-ordered on the caller's stream; the library's stream waits for
    // it through the event below, and destroy_tuner frees it on the same stream
    e = hipMallocAsync(&t->ws, t->ws_bytes, t->user);
    if (e != hipSuccess) {
        size_t need = t->ws_bytes;
        (void)hipGetLastError();
        destroy_tuner(t);
        return fail(AR_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) failed: %s", need, hipGetErrorString(e));
    }
    Carve c;
    c.base = static_cast<char*>(t->ws);
    carve(t, c, need_w32, need_x32);
    t->W = W;
    if (!need_w32) t->Wop = W;
    if (!need_x32) t->Xop = X;

#define TCHK(expr)                                                                                \
    do {                                                                                          \
        hipError_t e_ = (expr);                                                                   \
        if (e_ != hipSuccess) {                                                                   \
            ar_status r_ = fail(AR_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_));              \
            destroy_tuner(t);                                                                     \
            return r_;                                                                            \
        }                                                                                         \
    } while (0)

    // Order the library stream after the caller's stream.
    hipEvent_t ev;
    TCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    TCHK(hipEventRecord(ev, t->user));
    TCHK(hipStreamWaitEvent(t->ts, ev, 0));
    TCHK(hipEventDestroy(ev));

    {
        const ar_status st_t = upload_tables(t, o, ids_override);
        if (st_t != AR_OK) {
            destroy_tuner(t);
            return st_t;
        }
    }

    // Non-finite scan of W and X.
    TCHK(hipMemsetAsync(t->flag, 0, sizeof(int32_t), t->ts));
    TCHK(launch_nonfinite_scan(W, wt == AR_BF16, N * K, t->flag, t->ts));
    TCHK(launch_nonfinite_scan(X, xt == AR_BF16, S * T * K, t->flag, t->ts));
    int32_t bad = 0;
    TCHK(hipMemcpyAsync(&bad, t->flag, sizeof(int32_t), hipMemcpyDeviceToHost, t->ts));
    TCHK(hipStreamSynchronize(t->ts));
    if (bad) {
        destroy_tuner(t);
        return fail(AR_ERR_NONFINITE, "W or X_pool holds NaN or Inf");
    }

    // Operands in the GEMM precision.
    if (need_w32) TCHK(launch_widen_bf16(static_cast<const uint16_t*>(W), const_cast<float*>(static_cast<const float*>(t->Wop)), N * K, t->ts));
    if (need_x32) TCHK(launch_widen_bf16(static_cast<const uint16_t*>(X), const_cast<float*>(static_cast<const float*>(t->Xop)), S * T * K, t->ts));
    TCHK(launch_transpose_pool(t->Xop, t->XT, t->bf16 ? 2 : 4, S, T, K, t->ts));

    // Group ranges of the frozen weight, initial parameters into buffer 0.
    TCHK(launch_group_range(W, wt == AR_BF16, N, K, g, t->mx, t->mn, t->ts));
    TCHK(hipMemcpyAsync(t->V[0], V0, (size_t)(N * K) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    TCHK(hipMemcpyAsync(t->al[0], al0, (size_t)(N * t->G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    TCHK(hipMemcpyAsync(t->be[0], be0, (size_t)(N * t->G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    TCHK(launch_state_init(t->state, t->start_step, t->best_in, t->ts));
    TCHK(hipMemsetAsync(t->arrivals, 0, sizeof(int32_t), t->ts));
    if (t->fused) {
        // the first step's fake-quantized weight; later ones come from the fused update
        ar_status q = enqueue_kernel(t, K_QDQ);
        if (q != AR_OK) {
            destroy_tuner(t);
            return q;
        }
    }

    // Reference output with the original weight (blog sec. 3 step 2), fp32
    // accumulate, stored fp32 per sample as Y_ref[s] = W X_s^T ([S, N, T]).
    // The fp32 validation mode needs none: its loss GEMM multiplies w^ - W.
    const size_t xe = t->bf16 ? 2 : 4;
    for (int64_t s = 0; s < (t->bf16 ? S : 0); ++s) {
        GemmArgs a{};
        a.A.base = t->Wop; a.A.ld = K;
        a.B.base = static_cast<const char*>(t->Xop) + (size_t)(s * T * K) * xe; a.B.ld = K;
        a.I = N; a.J = T; a.R = K;
        a.epi = EPI_STORE; a.out = t->Yref + s * N * T; a.ldc = T;
        TCHK(t->bf16 ? launch_gemm_bf16(a, nullptr, t->ts) : launch_gemm_f32(a, nullptr, t->ts));
    }
    TCHK(hipStreamSynchronize(t->ts));
#undef TCHK
    *out = t;
    return AR_OK;
}

ar_status join_user(ar_tuner* t) {
    hipEvent_t ev;
    HIPCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    HIPCHK(hipEventRecord(ev, t->ts));
    HIPCHK(hipStreamWaitEvent(t->user, ev, 0));
    HIPCHK(hipEventDestroy(ev));
    return AR_OK;
}

constexpr int32_t kGraphSteps = 8;   // steps per graph launch in long runs

ar_status run_impl(ar_tuner* t, int32_t nsteps, int32_t flags) {
    if (!t) return fail(AR_ERR_INVALID_ARG, "tuner is NULL");
    if (nsteps < 0) return fail(AR_ERR_INVALID_ARG, "nsteps must be >= 0");
    if (t->steps_enqueued + (int64_t)nsteps > (int64_t)t->iters - t->start_step)
        return fail(AR_ERR_INVALID_ARG, "run would exceed iters (%d enqueued from step %d, %d requested, iters %d)",
                    t->steps_enqueued, t->start_step, nsteps, t->iters);
    {
        hipEvent_t ev;
        HIPCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
        HIPCHK(hipEventRecord(ev, t->user));
        HIPCHK(hipStreamWaitEvent(t->ts, ev, 0));
        HIPCHK(hipEventDestroy(ev));
    }
    if (flags & AR_RUN_KERNEL_GRAPHS) {
        // Per-kernel durations as a step graph runs them: for each kernel of
        // the step in turn, a graph of nsteps launches of that kernel alone,
        // replayed once between two HIP events on the tuner's stream.  The
        // launches of the kernel that takes the loss decision advance the
        // step counter nsteps times; kernels after it read the evaluated
        // step.  Timing only: the weight-gradient launches reuse the last
        // forward's outputs, so these steps are not a tuning trajectory.
        const int nk = num_kernels(t);
        if (t->kms_sum.empty()) t->kms_sum.assign(nk, 0.0);
        if (nsteps > 0) {
            hipEvent_t e0 = nullptr, e1 = nullptr;
            ar_status st = AR_OK;
            if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
                st = fail(AR_ERR_HIP, "hipEventCreate");
            for (int k = 0; k < nk && st == AR_OK; ++k) {
                hipGraph_t graph = nullptr;
                hipGraphExec_t exec = nullptr;
                if (hipStreamBeginCapture(t->ts, hipStreamCaptureModeThreadLocal) != hipSuccess) {
                    st = fail(AR_ERR_HIP, "hipStreamBeginCapture");
                    break;
                }
                for (int32_t i = 0; i < nsteps && st == AR_OK; ++i) st = enqueue_kernel(t, kernel_at(t, k));
                const hipError_t ec = hipStreamEndCapture(t->ts, &graph);
                if (st == AR_OK && ec != hipSuccess) st = fail(AR_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(ec));
                if (st == AR_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess)
                    st = fail(AR_ERR_HIP, "hipGraphInstantiate");
                if (graph) hipGraphDestroy(graph);
                float ms = 0.0f;
                if (st == AR_OK && (hipEventRecord(e0, t->ts) != hipSuccess || hipGraphLaunch(exec, t->ts) != hipSuccess ||
                                    hipEventRecord(e1, t->ts) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                                    hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
                    st = fail(AR_ERR_HIP, "kernel graph timing");
                if (exec) hipGraphExecDestroy(exec);
                if (st == AR_OK) t->kms_sum[(size_t)k] += ms;
            }
            if (e0) hipEventDestroy(e0);
            if (e1) hipEventDestroy(e1);
            if (st != AR_OK) return st;
            t->kms_count += nsteps;
        }
    } else if (flags & AR_RUN_EVENTS) {
        // Eager launches bracketed by events: per-kernel durations on the
        // stream the kernels run on.
        const int nk = num_kernels(t);
        const int per = nk + 1;
        const int chunk = 64;
        std::vector<hipEvent_t> evs((size_t)chunk * per);
        for (auto& e : evs) HIPCHK(hipEventCreate(&e));
        if (t->kms_sum.empty()) t->kms_sum.assign(nk, 0.0);
        ar_status st = AR_OK;
        for (int32_t base = 0; base < nsteps && st == AR_OK; base += chunk) {
            const int n = (nsteps - base) < chunk ? (nsteps - base) : chunk;
            for (int s = 0; s < n && st == AR_OK; ++s) {
                for (int k = 0; k < nk && st == AR_OK; ++k) {
                    if (hipEventRecord(evs[(size_t)(s * per + k)], t->ts) != hipSuccess) st = fail(AR_ERR_HIP, "hipEventRecord");
                    if (st == AR_OK) st = enqueue_kernel(t, kernel_at(t, k));
                }
                if (st == AR_OK && hipEventRecord(evs[(size_t)(s * per + nk)], t->ts) != hipSuccess)
                    st = fail(AR_ERR_HIP, "hipEventRecord");
            }
            if (st == AR_OK && hipStreamSynchronize(t->ts) != hipSuccess) st = fail(AR_ERR_HIP, "hipStreamSynchronize");
            for (int s = 0; s < n && st == AR_OK; ++s) {
                for (int k = 0; k < nk; ++k) {
                    float ms = 0.0f;
                    if (hipEventElapsedTime(&ms, evs[(size_t)(s * per + k)], evs[(size_t)(s * per + k + 1)]) != hipSuccess) {
                        st = fail(AR_ERR_HIP, "hipEventElapsedTime");
                        break;
                    }
                    t->kms_sum[(size_t)k] += ms;
                }
                t->kms_count += 1;
            }
        }
        for (auto& e : evs) hipEventDestroy(e);
        if (st != AR_OK) return st;
    } else if (flags & AR_RUN_GRAPH) {
        // One graph of a single step and, for a layer tuner that runs at
        // least kGraphSteps steps, one of kGraphSteps steps: every step reads
        // its index and buffers from device state, so a graph replays any run
        // of steps, and fewer graph launches leave fewer gaps between them
        // (1-2% per step on the 4096 x 4096 layer).  Both are captured on the
        // first graph run.  The block tuners keep one step per launch: their
        // multi-step graphs measured slower.
        auto capture = [&](int32_t n, hipGraphExec_t* out) -> ar_status {
            hipGraph_t graph;
            HIPCHK(hipStreamBeginCapture(t->ts, hipStreamCaptureModeThreadLocal));
            ar_status st = AR_OK;
            for (int32_t i = 0; i < n && st == AR_OK; ++i) st = enqueue_step(t);
            hipError_t e = hipStreamEndCapture(t->ts, &graph);
            if (st != AR_OK) return st;
            if (e != hipSuccess) return fail(AR_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
            e = hipGraphInstantiate(out, graph, nullptr, nullptr, 0);
            hipGraphDestroy(graph);
            if (e != hipSuccess) {
                *out = nullptr;
                return fail(AR_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
            }
            return AR_OK;
        };
        const bool multi = !t->blk && !t->dec && t->iters >= kGraphSteps;
        if (!t->gexec) {
            const ar_status st = capture(1, &t->gexec);
            if (st != AR_OK) return st;
        }
        if (multi && !t->gexec_multi) {
            const ar_status st = capture(kGraphSteps, &t->gexec_multi);
            if (st != AR_OK) return st;
        }
        int32_t s = 0;
        if (multi)
            for (; s + kGraphSteps <= nsteps; s += kGraphSteps) HIPCHK(hipGraphLaunch(t->gexec_multi, t->ts));
        for (; s < nsteps; ++s) HIPCHK(hipGraphLaunch(t->gexec, t->ts));
    } else {
        for (int32_t s = 0; s < nsteps; ++s) {
            ar_status st = enqueue_step(t);
            if (st != AR_OK) return st;
        }
    }
    t->steps_enqueued += nsteps;
    return join_user(t);
}

ar_status finish_impl(ar_tuner* t, float* V, float* al, float* be, float* best_loss, int32_t* best_step) {
    if (!t) return fail(AR_ERR_INVALID_ARG, "tuner is NULL");
    if (t->blk || t->dec) return fail(AR_ERR_INVALID_ARG, "a block tuner is finished with ar_block_tuner_finish");
    if (!V || !al || !be) return fail(AR_ERR_INVALID_ARG, "V, alpha and beta must be non-NULL");
    StepState hs;
    HIPCHK(hipMemcpyAsync(&hs, t->state, sizeof(StepState), hipMemcpyDeviceToHost, t->ts));
    std::vector<double> tr((size_t)(t->iters > 0 ? t->iters : 1));
    HIPCHK(hipMemcpyAsync(tr.data(), t->trace, tr.size() * sizeof(double), hipMemcpyDeviceToHost, t->ts));
    HIPCHK(hipStreamSynchronize(t->ts));
    int src = hs.best_idx;
    if (t->return_last || src < 0) src = hs.cur;   // nothing evaluated yet: the initial state
    HIPCHK(hipMemcpyAsync(V, t->V[src], (size_t)(t->N * t->K) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    HIPCHK(hipMemcpyAsync(al, t->al[src], (size_t)(t->N * t->G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    HIPCHK(hipMemcpyAsync(be, t->be[src], (size_t)(t->N * t->G) * sizeof(float), hipMemcpyDeviceToDevice, t->ts));
    HIPCHK(hipStreamSynchronize(t->ts));
    write_host_trace(t, hs, tr);
    if (best_loss) *best_loss = (float)hs.best_loss;
    if (best_step) *best_step = hs.best_step;
    if (hs.halted) return fail(AR_ERR_NONFINITE, "the loss became non-finite at step %d; best state written", hs.step);
    return AR_OK;
}

// Host-side checks shared by the fake-quantizer entry points.
ar_status qdq_check(const void* W, ar_dtype wt, int64_t N, int64_t K, const ar_qconfig* qcfg, const float* V,
                    const float* beta, const void* W_qdq, ar_dtype out_dt, int32_t* g) {
    if (!W) return fail(AR_ERR_INVALID_ARG, "W is NULL");
    if (N <= 0 || K <= 0) return fail(AR_ERR_INVALID_ARG, "N and K must be positive");
    if (!dtype_ok(wt)) return fail(AR_ERR_INVALID_ARG, "unknown W dtype");
    if (W_qdq && !dtype_ok(out_dt)) return fail(AR_ERR_INVALID_ARG, "unknown output dtype");
    ar_status st = check_qcfg(qcfg, K, g);
    if (st != AR_OK) return st;
    if (N * K > ((int64_t)1 << 34)) return fail(AR_ERR_UNSUPPORTED, "problem too large");
    if (qcfg->format != AR_FMT_INT) {
        if (V || beta) return fail(AR_ERR_UNSUPPORTED, "float formats take no rounding offset V or beta");
        if (qcfg->format == AR_FMT_FP8_E4M3 && qcfg->bits != 8)
            return fail(AR_ERR_INVALID_ARG, "FP8 E4M3 needs bits = 8, got %d", qcfg->bits);
        if (qcfg->format == AR_FMT_MXFP4 && (qcfg->bits != 4 || *g != 32))
            return fail(AR_ERR_INVALID_ARG, "MXFP4 needs bits = 4 and group_size = 32");
    }
    return AR_OK;
}

// Group ranges into mm (mx = mm[0 .. N G), mn = mm[N G .. 2 N G)), then the
// integer or float fake quantizer, all on `s`.
hipError_t qdq_launch(const void* W, ar_dtype wt, int64_t N, int64_t K, int32_t g, const ar_qconfig* qcfg,
                      const float* V, const float* alpha, const float* beta, void* W_qdq, ar_dtype out_dt,
                      uint8_t* codes, float* scale, uint8_t* zero, float* mm, hipStream_t s) {
    const int64_t G = K / g;
    hipError_t e = launch_group_range(W, wt == AR_BF16, N, K, g, mm, mm + N * G, s);
    if (e != hipSuccess) return e;
    if (qcfg->format != AR_FMT_INT) {
        FloatQdqArgs a{};
        a.format = qcfg->format;
        a.W = W; a.w_bf16 = (wt == AR_BF16); a.N = N; a.K = K; a.group = g;
        a.mx = mm; a.mn = mm + N * G; a.alpha = alpha;
        a.w_hat = W_qdq; a.out_kind = W_qdq ? (out_dt == AR_BF16 ? 2 : 1) : 0;
        a.codes = codes; a.scale = scale; a.zero = zero;
        return launch_float_qdq(a, s);
    }
    QdqArgs a{};
    a.W = W; a.w_bf16 = (wt == AR_BF16); a.N = N; a.K = K; a.qp = make_qp(qcfg, g);
    a.mx = mm; a.mn = mm + N * G;
    a.V[0] = V; a.alpha[0] = alpha; a.beta[0] = beta;
    a.w_hat = W_qdq; a.out_kind = W_qdq ? (out_dt == AR_BF16 ? 2 : 1) : 0;
    a.codes = codes; a.scale = scale; a.zero = zero;
    return launch_qdq(a, s);
}

// Static group-range buffer of ar_qdq_rtn_noalloc: 64 MiB of device memory
// per GPU for the callers that cannot allocate (graph capture, serving
// loops).  Host code never uses the symbol itself as an address: each
// device's copy is looked up once with hipGetSymbolAddress (with that device
// current) and the pointer kept per device.
constexpr int64_t kScratchFloats = (int64_t)16 << 20;   // 2 N G floats at most: 8 Mi groups
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

ar_status scratch_for_current_device(float** out) {
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(AR_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return AR_OK;
}

}  // namespace rt
}  // namespace ar

// ============================================================ C ABI =======
extern "C" {

ar_status ar_tune_opts_init(ar_tune_opts* o, int32_t preset) {
    if (!o) return fail(AR_ERR_INVALID_ARG, "opts is NULL");
    int32_t batch, iters;
    switch (preset) {
        case AR_PRESET_DEFAULT: batch = 8; iters = 200; break;
        case AR_PRESET_BEST: batch = 8; iters = 1000; break;
        case AR_PRESET_LIGHT: batch = 8; iters = 50; break;
        case AR_PRESET_FAST: batch = 4; iters = 200; break;
        default: return fail(AR_ERR_INVALID_ARG, "unknown preset %d", preset);
    }
    std::memset(o, 0, sizeof(*o));
    o->iters = iters;
    o->lr = 5e-3f;
    o->lr_clip = 5e-3f;
    o->lr_decay = 1;
    o->clip_lo = 0.5f;
    o->clip_hi = 1.0f;
    o->batch_samples = batch;
    o->schedule = nullptr;
    o->gemm_mode = AR_GEMM_BF16;
    o->return_last = 0;
    o->loss_trace = nullptr;
    o->max_workspace_bytes = 0;
    o->unfused = 0;
    o->start_step = 0;
    o->best_loss_in = INFINITY;
    return AR_OK;
}

ar_status ar_qdq_rtn(const void* W, ar_dtype wt, int64_t N, int64_t K, const ar_qconfig* qcfg, const float* V,
                     const float* alpha, const float* beta, void* W_qdq, ar_dtype out_dt, uint8_t* codes, float* scale,
                     uint8_t* zero, void* stream) {
    int32_t g = 0;
    ar_status st = qdq_check(W, wt, N, K, qcfg, V, beta, W_qdq, out_dt, &g);
    if (st != AR_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t G = K / g;
    float* mm = nullptr;
    HIPCHK(hipMallocAsync(reinterpret_cast<void**>(&mm), (size_t)(2 * N * G) * sizeof(float), s));
    hipError_t e = qdq_launch(W, wt, N, K, g, qcfg, V, alpha, beta, W_qdq, out_dt, codes, scale, zero, mm, s);
    hipError_t e2 = hipFreeAsync(mm, s);
    if (e != hipSuccess) return fail(AR_ERR_HIP, "qdq launch: %s", hipGetErrorString(e));
    if (e2 != hipSuccess) return fail(AR_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e2));
    return AR_OK;
}

ar_status ar_qdq_rtn_noalloc(const void* W, ar_dtype wt, int64_t N, int64_t K, const ar_qconfig* qcfg,
                             const float* V, const float* alpha, const float* beta, void* W_qdq, ar_dtype out_dt,
                             uint8_t* codes, float* scale, uint8_t* zero, void* stream) {
    int32_t g = 0;
    ar_status st = qdq_check(W, wt, N, K, qcfg, V, beta, W_qdq, out_dt, &g);
    if (st != AR_OK) return st;
    const int64_t G = K / g;
    if (2 * N * G > kScratchFloats)
        return fail(AR_ERR_OUT_OF_MEMORY,
                    "ar_qdq_rtn_noalloc: N * K / group_size = %lld groups exceeds its static buffer of %lld groups "
                    "(use ar_qdq_rtn)", (long long)(N * G), (long long)(kScratchFloats / 2));
    float* mm = nullptr;
    st = scratch_for_current_device(&mm);
    if (st != AR_OK) return st;
    hipError_t e = qdq_launch(W, wt, N, K, g, qcfg, V, alpha, beta, W_qdq, out_dt, codes, scale, zero, mm,
                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(AR_ERR_HIP, "qdq launch: %s", hipGetErrorString(e));
    return AR_OK;
}

ar_status ar_pack_int4(const void* W, ar_dtype wt, int64_t N, int64_t K, const ar_qconfig* qcfg, const float* V,
                       const float* alpha, const float* beta, uint8_t* packed, float* scale, uint8_t* zero,
                       void* stream) {
    if (!W || !packed || !scale || !zero) return fail(AR_ERR_INVALID_ARG, "W, packed, scale and zero must be non-NULL");
    if (N <= 0 || K <= 0) return fail(AR_ERR_INVALID_ARG, "N and K must be positive");
    if (!dtype_ok(wt)) return fail(AR_ERR_INVALID_ARG, "unknown W dtype");
    int32_t g = 0;
    ar_status st = check_qcfg(qcfg, K, &g);
    if (st != AR_OK) return st;
    st = require_int_format(qcfg);
    if (st != AR_OK) return st;
    if (qcfg->bits != 4) return fail(AR_ERR_INVALID_ARG, "INT4 packing needs bits = 4, got %d", qcfg->bits);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t G = K / g;
    float* mm = nullptr;
    HIPCHK(hipMallocAsync(reinterpret_cast<void**>(&mm), (size_t)(2 * N * G) * sizeof(float), s));
    hipError_t e = launch_group_range(W, wt == AR_BF16, N, K, g, mm, mm + N * G, s);
    if (e == hipSuccess) {
        QdqArgs a{};
        a.W = W; a.w_bf16 = (wt == AR_BF16); a.N = N; a.K = K; a.qp = make_qp(qcfg, g);
        a.mx = mm; a.mn = mm + N * G;
        a.V[0] = V; a.alpha[0] = alpha; a.beta[0] = beta;
        a.packed = packed; a.scale = scale; a.zero = zero;
        e = launch_qdq(a, s);
    }
    hipError_t e2 = hipFreeAsync(mm, s);
    if (e != hipSuccess) return fail(AR_ERR_HIP, "pack launch: %s", hipGetErrorString(e));
    if (e2 != hipSuccess) return fail(AR_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e2));
    return AR_OK;
}

ar_status ar_w4a16_gemm(const void* X, ar_dtype xt, int64_t M, int64_t K, const uint8_t* packed, const float* scale,
                        const uint8_t* zero, int64_t N, int32_t group_size, void* Y, ar_dtype yt, void* stream) {
    if (M < 0 || N <= 0 || K <= 0) return fail(AR_ERR_INVALID_ARG, "need M >= 0 and N, K > 0");
    if (!packed || !scale || !zero || (M > 0 && (!X || !Y)))
        return fail(AR_ERR_INVALID_ARG, "packed, scale, zero (and X, Y when M > 0) must be non-NULL");
    if (!dtype_ok(xt) || !dtype_ok(yt)) return fail(AR_ERR_INVALID_ARG, "unknown dtype");
    ar_qconfig q{4, group_size, 0, AR_FMT_INT};
    int32_t g = 0;
    ar_status st = check_qcfg(&q, K, &g);
    if (st != AR_OK) return st;
    if (xt != AR_BF16) return fail(AR_ERR_UNSUPPORTED, "the INT4-weight GEMM takes bf16 activations");
    if (K % 64 != 0) return fail(AR_ERR_UNSUPPORTED, "K must be a multiple of 64, got %lld", (long long)K);
    if (K >= ((int64_t)1 << 30)) return fail(AR_ERR_UNSUPPORTED, "K must be below 2^30");
    if (reinterpret_cast<uintptr_t>(X) % 16 != 0 || reinterpret_cast<uintptr_t>(packed) % 4 != 0)
        return fail(AR_ERR_UNSUPPORTED, "X must be 16-byte and packed 4-byte aligned");
    if (M == 0) return AR_OK;
    W4A16Args a{};
    a.X = static_cast<const uint16_t*>(X);
    a.ldx = K;
    a.M = M; a.N = N; a.K = K;
    a.packed = reinterpret_cast<const uint32_t*>(packed);
    a.scale = scale; a.zero = zero;
    a.g = g; a.G = K / g;
    a.Y = Y; a.ldy = N; a.y_bf16 = (yt == AR_BF16);
    hipError_t e = launch_w4a16_gemm(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(AR_ERR_HIP, "INT4-weight GEMM launch: %s", hipGetErrorString(e));
    return AR_OK;
}

ar_status ar_layer_grads(const void* W, ar_dtype wt, int64_t N, int64_t K, const void* X_pool, ar_dtype xt, int64_t S,
                         int64_t T, const int32_t* ids, int32_t B, const ar_qconfig* qcfg, ar_gemm_mode mode,
                         const float* V, const float* alpha, const float* beta, double* loss, float* G, float* dV,
                         float* dalpha, float* dbeta, void* stream) {
    if (!ids) return fail(AR_ERR_INVALID_ARG, "ids is NULL");
    if (!loss) return fail(AR_ERR_INVALID_ARG, "loss is NULL");
    if (B < 1 || B > S) return fail(AR_ERR_INVALID_ARG, "B must be in [1, S]");
    for (int32_t b = 0; b < B; ++b)
        if (ids[b] < 0 || ids[b] >= S) return fail(AR_ERR_INVALID_ARG, "ids[%d] = %d is outside [0, S)", b, ids[b]);
    ar_tune_opts o;
    ar_tune_opts_init(&o, AR_PRESET_DEFAULT);
    o.iters = 1;
    o.batch_samples = B;
    o.gemm_mode = mode;
    o.lr = 0.0f;
    o.lr_clip = 0.0f;
    o.unfused = 1;
    ar_tuner* t = nullptr;
    ar_status st = create_impl(&t, W, wt, N, K, X_pool, xt, S, T, qcfg, &o, V, alpha, beta, stream, ids);
    if (st != AR_OK) return st;
    st = AR_OK;
    const std::vector<int> seq = step_sequence(t, false, false);   // through the STE backward
    for (size_t k = 0; k < seq.size() && st == AR_OK; ++k) st = enqueue_kernel(t, seq[k]);
    StepState hs;
    if (st == AR_OK && hipMemcpyAsync(&hs, t->state, sizeof(StepState), hipMemcpyDeviceToHost, t->ts) != hipSuccess)
        st = fail(AR_ERR_HIP, "state copy");
    double L = 0.0;
    if (st == AR_OK && hipMemcpyAsync(&L, t->trace, sizeof(double), hipMemcpyDeviceToHost, t->ts) != hipSuccess)
        st = fail(AR_ERR_HIP, "loss copy");
    const size_t nk = (size_t)(N * K) * sizeof(float), ng = (size_t)(N * t->G) * sizeof(float);
    if (st == AR_OK && G && hipMemcpyAsync(G, t->Gb, nk, hipMemcpyDeviceToDevice, t->ts) != hipSuccess) st = fail(AR_ERR_HIP, "G copy");
    if (st == AR_OK && dV && hipMemcpyAsync(dV, t->dV, nk, hipMemcpyDeviceToDevice, t->ts) != hipSuccess) st = fail(AR_ERR_HIP, "dV copy");
    if (st == AR_OK && dalpha && hipMemcpyAsync(dalpha, t->dal, ng, hipMemcpyDeviceToDevice, t->ts) != hipSuccess) st = fail(AR_ERR_HIP, "dalpha copy");
    if (st == AR_OK && dbeta && hipMemcpyAsync(dbeta, t->dbe, ng, hipMemcpyDeviceToDevice, t->ts) != hipSuccess) st = fail(AR_ERR_HIP, "dbeta copy");
    if (st == AR_OK && hipStreamSynchronize(t->ts) != hipSuccess) st = fail(AR_ERR_HIP, "synchronize");
    if (st == AR_OK) {
        *loss = L;
        if (hs.halted) st = fail(AR_ERR_NONFINITE, "loss is not finite");
    }
    if (st == AR_OK) st = join_user(t);
    destroy_tuner(t);
    return st;
}

ar_status ar_tuner_create(ar_tuner** out, const void* W, ar_dtype wt, int64_t N, int64_t K, const void* X_pool,
                          ar_dtype xt, int64_t S, int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* opts,
                          const float* V0, const float* alpha0, const float* beta0, void* stream) {
    return create_impl(out, W, wt, N, K, X_pool, xt, S, T, qcfg, opts, V0, alpha0, beta0, stream, nullptr);
}

ar_status ar_tuner_run(ar_tuner* t, int32_t nsteps, int32_t flags) { return run_impl(t, nsteps, flags); }

ar_status ar_tuner_finish(ar_tuner* t, float* V, float* alpha, float* beta, float* final_best_loss,
                          int32_t* best_step) {
    return finish_impl(t, V, alpha, beta, final_best_loss, best_step);
}

ar_status ar_tuner_destroy(ar_tuner* t) {
    destroy_tuner(t);
    return AR_OK;
}

int32_t ar_tuner_num_kernels(const ar_tuner* t) { return t ? num_kernels(t) : 0; }

const char* ar_tuner_kernel_name(const ar_tuner* t, int32_t i) {
    if (!t || i < 0 || i >= num_kernels(t)) return nullptr;
    if (t->blk) return block_kernel_name(kernel_at(t, i));
    if (t->dec) return decoder_kernel_name(kernel_at(t, i));
    return kKernelNames[kernel_at(t, i)];
}

ar_status ar_tuner_kernel_ms(const ar_tuner* t, float* mean_ms) {
    if (!t || !mean_ms) return fail(AR_ERR_INVALID_ARG, "NULL argument");
    if (t->kms_count == 0) return fail(AR_ERR_INVALID_ARG, "no AR_RUN_EVENTS run yet");
    for (int k = 0; k < num_kernels(t); ++k) mean_ms[k] = (float)(t->kms_sum[(size_t)k] / (double)t->kms_count);
    return AR_OK;
}

ar_status ar_tune_layer(const void* W, ar_dtype wt, int64_t N, int64_t K, const void* X_pool, ar_dtype xt, int64_t S,
                        int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* opts, float* V, float* alpha,
                        float* beta, float* final_best_loss, int32_t* best_step, void* stream) {
    ar_tuner* t = nullptr;
    ar_status st = create_impl(&t, W, wt, N, K, X_pool, xt, S, T, qcfg, opts, V, alpha, beta, stream, nullptr);
    if (st != AR_OK) return st;
    st = run_impl(t, opts->iters - opts->start_step, AR_RUN_GRAPH);
    if (st == AR_OK || st == AR_ERR_NONFINITE) {
        ar_status st2 = finish_impl(t, V, alpha, beta, final_best_loss, best_step);
        if (st == AR_OK) st = st2;
    }
    destroy_tuner(t);
    return st;
}

const char* ar_last_error(void) { return g_err.c_str(); }

const char* ar_version(void) { return "libautoround 0.1.0 (gfx950)"; }

}  // extern "C"
