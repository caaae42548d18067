// Internal interface between the C-ABI translation units: the tuner object,
// the shared argument checks and the workspace carver.
#pragma once

#include <string>
#include <vector>

#include "../../include/libautoround.h"
#include "ar_internal.h"

namespace ar {
namespace rt {

// Sets the thread's error string (ar_last_error) and returns `st`.
ar_status fail(ar_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

#define HIPCHK(expr)                                                                           \
    do {                                                                                       \
        hipError_t e_ = (expr);                                                                \
        if (e_ != hipSuccess) return ::ar::rt::fail(AR_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

ar_status check_qcfg(const ar_qconfig* q, int64_t K, int32_t* g_out);
ar_status require_int_format(const ar_qconfig* q);
bool dtype_ok(ar_dtype d);
size_t esize(ar_dtype d);
QParams make_qp(const ar_qconfig* q, int32_t g);
ar_status validate_opts(const ar_tune_opts* o, int64_t S);

// Bump allocator over one device allocation (256-byte aligned pieces); with
// base == nullptr it only sizes.
struct Carve {
    size_t off = 0;
    char* base = nullptr;
    template <typename T>
    T* take(size_t count) {
        off = (off + 255) & ~(size_t)255;
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

// One quantized linear of a block: weight [N, K], its parameters in two
// buffers (the best-loss snapshot needs no copy), the fake-quantized GEMM
// operand, and the buffers of the unfused backward.
struct BlockLinear {
    int64_t N = 0, K = 0, G = 0;
    const void* W = nullptr;       // caller's weight (quantizer input)
    const void* Wop = nullptr;     // reference GEMM operand (W, or a widened copy)
    float *mx = nullptr, *mn = nullptr;
    float *V[2] = {nullptr, nullptr}, *al[2] = {nullptr, nullptr}, *be[2] = {nullptr, nullptr};
    void* what = nullptr;          // fake-quantized weight [N, K] in the GEMM type (gate's and up's adjacent)
    float* Gb = nullptr;           // [N, K]
    float* dV = nullptr;           // [N, K]
    float *dal = nullptr, *dbe = nullptr;
    bool fused = false;            // the weight-gradient GEMM carries backward + update + next QDQ
};

// SwiGLU MLP block: gate [F, H], up [F, H], down [H, F].
struct BlockPart {
    int32_t kind = 0;
    ar_dtype xt = AR_BF16;         // dtype of the pool, and of the block output written at finish
    int64_t H = 0, F = 0;
    BlockLinear lin[3];
    float* At = nullptr;           // gate pre-activation^T [F, M] fp32, followed by
    float* Bt = nullptr;           // up pre-activation^T   [F, M] fp32 (one [2F, M] buffer)
    void* Hh = nullptr;            // gated activation      [M, F] GEMM type
    void* Hht = nullptr;           //                       [F, M]
    void* dy = nullptr;            // dY                    [M, H]
    void* wdt = nullptr;           // fake-quantized down^T [F, H] (fp32 GEMM mode only)
    float* dHt = nullptr;          // dL/dHh^T              [F, M] fp32
    void* dAt = nullptr;           // dL/dA^T               [F, M] GEMM type
    void* dBt = nullptr;           // dL/dB^T               [F, M]
    float* yq = nullptr;           // block output rows     [M, H] fp32 (final forward)
};

// Llama decoder block: linears q, k, v, o, gate, up, down (indices 0..6).
struct DecoderPart {
    int64_t H = 0, F = 0;
    int32_t nq = 0, nkv = 0, d = 0;
    float eps = 1e-5f, theta = 10000.0f;
    ar_dtype xt = AR_BF16;
    const float* w1 = nullptr;     // norm weights [H] (caller's, nullable = 1)
    const float* w2 = nullptr;
    const void* X = nullptr;       // caller's pool [S, T, H]
    BlockLinear lin[7];
    void* what_qkv = nullptr;      // w^ of q, k, v stacked [(nq + 2 nkv) d, H]
    uint16_t* what_gu = nullptr;   // w^ of gate, up stacked [2F, H]
    // persistent
    void* h1 = nullptr;            // rmsnorm(x) [S T, H] bf16
    void* h1T = nullptr;           // [S, H, T]
    float *cosT = nullptr, *sinT = nullptr;   // [T, d/2]
    // step buffers
    float* qkv = nullptr;          // [M, Nqkv] fp32
    uint16_t *qr = nullptr, *qT = nullptr, *kr = nullptr, *kT = nullptr, *vv = nullptr, *vT = nullptr;
    uint16_t *o = nullptr, *oT = nullptr;
    float* lse = nullptr;
    float* attn = nullptr;         // o-projection output [M, H]
    float* h = nullptr;            // residual stream after attention [M, H]
    float* r2 = nullptr;           // [M]
    uint16_t *h2 = nullptr, *h2T = nullptr;
    float* tgt = nullptr;          // y_ref - h, per sample transposed [B, H, T]
    float *At = nullptr, *Bt = nullptr;          // adjacent: A^T over B^T [2F, M]
    uint16_t *Hh = nullptr, *Hht = nullptr, *dy = nullptr;
    float* dHt = nullptr;
    uint16_t *dAt = nullptr, *dBt = nullptr, *dAB = nullptr;   // dA^T over dB^T [2F, M]
    float* dh2 = nullptr;
    float* dh2b = nullptr;       // second reduction half of dh2 (split GEMM), or NULL
    uint16_t *dh = nullptr, *dhT = nullptr;
    float* da = nullptr;
    float* Di = nullptr;
    uint16_t *dOb = nullptr, *dOT = nullptr;
    float *dq = nullptr, *dk = nullptr, *dv = nullptr;
    uint16_t* dqkvT = nullptr;
    float* yq = nullptr;           // [M, H]
};

}  // namespace rt
}  // namespace ar

// A tuning run in progress: one linear layer, or (blk != nullptr) the
// linears of a block.  All per-step state lives in device memory so one
// captured step serves every step.
struct ar_tuner {
    // problem
    int64_t N = 0, K = 0, S = 0, T = 0, G = 0, M = 0;
    int32_t B = 0, iters = 0, g = 0;
    ar::QParams qp{};
    bool bf16 = true;            // GEMM operand type
    bool w_bf16 = true;          // storage type of the W the quantizer reads
    int32_t return_last = 0;
    bool fused = false;          // wgrad GEMM carries backward + update + next QDQ
    std::vector<int> seq;        // kernels of one step
    float clip_lo = 0.5f, clip_hi = 1.0f;
    float* host_trace = nullptr;
    hipStream_t user = nullptr;
    hipStream_t ts = nullptr;    // the library's stream for all tuning work
    // workspace
    void* ws = nullptr;
    size_t ws_bytes = 0;
    const void* W = nullptr;     // quantizer input (caller's)
    const void* Wop = nullptr;   // GEMM operand of the reference (caller's or widened copy)
    const void* Xop = nullptr;   // pool operand [S, T, K]
    void* XT = nullptr;          // [S, K, T]
    float* Yref = nullptr;       // [S, N, T]
    float *mx = nullptr, *mn = nullptr;
    float *V[2] = {nullptr, nullptr}, *al[2] = {nullptr, nullptr}, *be[2] = {nullptr, nullptr};
    void* what = nullptr;        // [N, K]
    void* dyt = nullptr;         // [N, M]
    float* Gb = nullptr;         // [N, K]
    float* dV = nullptr;         // [N, K]
    float *dal = nullptr, *dbe = nullptr;
    double* partials = nullptr;
    ar::StepState* state = nullptr;
    double* trace = nullptr;
    int32_t* sched = nullptr;    // [max(iters,1), B]
    float *lr = nullptr, *lrc = nullptr;
    int32_t* flag = nullptr;
    int32_t* arrivals = nullptr; // workgroups of the fused weight-gradient launch that took the decision
    int32_t nparts = 0;
    int32_t steps_enqueued = 0; // steps enqueued by run() calls, counted from start_step
    int32_t start_step = 0;      // index of the first step this tuner evaluates
    double best_in = __builtin_inf();   // best loss of the steps before start_step
    // graph
    hipGraphExec_t gexec = nullptr;        // one step
    hipGraphExec_t gexec_multi = nullptr;  // kGraphSteps steps
    // kernel timing
    std::vector<double> kms_sum;
    int64_t kms_count = 0;
    // block tuning (block_tuner.hip); the layer fields above that describe
    // one weight are unused then
    ar::rt::BlockPart* blk = nullptr;
    ar::rt::DecoderPart* dec = nullptr;
};

namespace ar {
namespace rt {

void destroy_tuner(ar_tuner* t);
// Shared by the layer and block tuners: the schedule / step-size tables, the
// resume point of the options, and the caller's loss trace.
ar_status upload_tables(ar_tuner* t, const ar_tune_opts* o, const int32_t* ids_override);
void set_resume(ar_tuner* t, const ar_tune_opts* o);
void write_host_trace(const ar_tuner* t, const StepState& hs, const std::vector<double>& tr);
ar_status join_user(ar_tuner* t);
ar_status run_impl(ar_tuner* t, int32_t nsteps, int32_t flags);
// Kernel `k` of a step of a block tuner, its name, and release of the block part.
ar_status block_enqueue_kernel(ar_tuner* t, int k);
const char* block_kernel_name(int k);
void block_release(ar_tuner* t);
ar_status decoder_enqueue_kernel(ar_tuner* t, int k);
const char* decoder_kernel_name(int k);
void decoder_release(ar_tuner* t);
// Decoder-block tuner (decoder_tuner.hip): create, finish and one-step gradients.
ar_status decoder_create_impl(ar_tuner** out, const ar_block_desc* d, const void* X, ar_dtype xt, int64_t S, int64_t T,
                              const ar_qconfig* qcfg, const ar_tune_opts* o, const float* const V0[],
                              const float* const al0[], const float* const be0[], void* stream,
                              const int32_t* ids_override);
// Host-side argument checks of a block descriptor (no HIP call): the ones
// ar_block_tuner_create runs for the MLP block and for the decoder block.
ar_status block_validate(const ar_block_desc* d, const void* X, ar_dtype xt, int64_t S, int64_t T,
                         const ar_qconfig* qcfg, ar_gemm_mode mode, int32_t* g);
ar_status decoder_validate(const ar_block_desc* d, const void* X, ar_dtype xt, int64_t S, int64_t T,
                           const ar_qconfig* qcfg, ar_gemm_mode mode, int32_t* g);
ar_status decoder_finish_impl(ar_tuner* t, float* const V[], float* const al[], float* const be[], void* Yq,
                              float* best_loss, int32_t* best_step);
ar_status decoder_grads_impl(const ar_block_desc* desc, const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                             const int32_t* ids, int32_t B, const ar_qconfig* qcfg, ar_gemm_mode mode,
                             const float* const V[], const float* const alpha[], const float* const beta[],
                             double* loss, float* const G[], float* const dV[], float* const dalpha[],
                             float* const dbeta[], void* stream);

}  // namespace rt
}  // namespace ar
