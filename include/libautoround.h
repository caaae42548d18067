/*
 * libautoround -- AutoRound-style post-training weight quantization on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (AutoRound blog "Low-Bit Quantization in Practice with vLLM:
 * Core Mechanisms and Architectural Optimizations of AutoRound", sec. 2-4):
 * each weight of a linear layer W[N, K] (nn.Linear layout, output rows n,
 * input columns k) gets a learnable rounding offset V in [-0.5, 0.5]; each
 * group of g consecutive weights along K gets clip factors alpha, beta in
 * [0.5, 1] that scale the group's max and min.  The fake quantizer is
 *     mx = max(0, max W_g), mn = min(0, min W_g)
 *     s  = (alpha*mx - beta*mn) / Q,   Q = 2^bits - 1   (s = 1 if the range is 0)
 *     z  = rint(-beta*mn / s)
 *     q  = clamp(rint(W/s + V) + z, 0, Q)          (integer code)
 *     w^ = s * (q - z)                             (dequantized weight)
 * in fp32 with that operation order, IEEE division and round-half-to-even.
 * Tuning minimises the mean squared error between X W^T and X w^T over
 * calibration activations X with SignSGD (p <- clamp(p - lr_t*sign(dL/dp)))
 * through a straight-through estimator, keeping the best-loss state; the
 * result is packed to INT4 codes with per-group fp32 scale and uint8 zero.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are caller-owned; "DEVICE" pointers are HIP device
 *    memory on the current device, "HOST" pointers are host memory.  The
 *    library never frees or retains them after the call returns.
 *  - All argument checks happen on the host before any HIP call; on an
 *    error no output is modified.  Unsupported combinations are errors,
 *    never a silent fallback to another path.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls that return
 *    host results synchronize that stream; the others are stream-ordered.
 *  - Row-major layouts throughout; groups run along K; requires
 *    K % group_size == 0 and group_size % 8 == 0.
 *  - ar_last_error() describes the last failure on the calling thread.
 */
#ifndef LIBAUTOROUND_H
#define LIBAUTOROUND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define AR_API __attribute__((visibility("default")))
#else
#define AR_API
#endif

typedef enum {
    AR_OK = 0,
    AR_ERR_INVALID_ARG = 1,   /* bad shape, NULL required pointer, bad option  */
    AR_ERR_UNSUPPORTED = 2,   /* valid request this library does not implement */
    AR_ERR_NONFINITE = 3,     /* NaN/Inf in W or X, or a non-finite loss        */
    AR_ERR_OUT_OF_MEMORY = 4, /* device allocation failed or exceeds the cap    */
    AR_ERR_HIP = 5            /* HIP runtime error; text in ar_last_error()     */
} ar_status;

typedef enum { AR_F32 = 0, AR_BF16 = 1 } ar_dtype;

/* GEMM arithmetic of the tuning loop.  BF16: the dequantized weight, the
 * activations and the output gradient enter bf16 MFMA with fp32
 * accumulation (the blog's QDQ-then-BF16-GEMM, sec. 3-4).  F32: fp32 MFMA
 * throughout, used to validate against the fp64 oracle. */
typedef enum { AR_GEMM_BF16 = 0, AR_GEMM_F32 = 1 } ar_gemm_mode;

typedef struct {
    int32_t bits;       /* 2..8                                               */
    int32_t group_size; /* > 0 and dividing K, or -1 for one group per row    */
    int32_t sym;        /* 0: asymmetric, s = (alpha*max - beta*min)/Q with
                           zero-point z = rint(-beta*min/s); 1: symmetric,
                           s = alpha*max|W_g|/(2^(bits-1) - 1), z = 2^(bits-1)
                           (coordinates page sec. 1.2), beta unused          */
    int32_t format;     /* ar_format.  AR_FMT_INT: the integer grid above, the
                           one the tuning entry points run on.  The float
                           formats are tensor-level QDQ only (blog sec. 4,
                           data-type decoupling: a registered QDQ function
                           evaluates a new type's accuracy), through
                           ar_qdq_rtn with V = beta = NULL (alpha clips the
                           group maximum); every other entry point returns
                           AR_ERR_UNSUPPORTED for them:
                           AR_FMT_FP8_E4M3: bits 8, s = alpha*max|W_g|/448,
                             codes are E4M3 bytes, zero written as 0;
                           AR_FMT_MXFP4: bits 4, group_size 32, s = 2^e with
                             e = floor(log2(alpha*max|W_b|)) - 2, codes are
                             E2M1 nibbles, zero receives e + 127 (E8M0).
                           Float rounding: nearest value, ties to the even
                           code, saturating at 448 / 6.                      */
} ar_qconfig;

typedef enum { AR_FMT_INT = 0, AR_FMT_FP8_E4M3 = 1, AR_FMT_MXFP4 = 2 } ar_format;

/* Presets of the blog's sec. 8 table (batch, iterations, seq len, samples;
 * lr 5e-3 for all).  The sequence length and sample count describe the
 * caller's calibration pool; the options carry batch and iterations. */
typedef enum { AR_PRESET_DEFAULT = 0, AR_PRESET_BEST = 1, AR_PRESET_LIGHT = 2, AR_PRESET_FAST = 3 } ar_preset;

typedef struct {
    int32_t iters;           /* SignSGD steps T (>= 0)                               */
    float lr;                /* step size of V (>= 0)                                */
    float lr_clip;           /* step size of alpha/beta (>= 0; 0 freezes them)       */
    int32_t lr_decay;        /* 1: lr_t = lr*(1 - t/T) (linear to 0), 0: constant    */
    float clip_lo, clip_hi;  /* box of alpha and beta, 0 <= clip_lo <= clip_hi        */
    int32_t batch_samples;   /* B: samples per step, 1..S                            */
    const int32_t* schedule; /* HOST [iters * B] sample ids in [0, S); NULL: every
                                step uses samples 0..B-1                             */
    ar_gemm_mode gemm_mode;
    int32_t return_last;     /* 1: return the state after the last update instead
                                of the best-loss snapshot                            */
    float* loss_trace;       /* HOST [iters] per-step loss, nullable                 */
    size_t max_workspace_bytes; /* 0 = unlimited                                     */
    int32_t unfused;         /* 0: run the straight-through backward, update and next
                                fake quantization inside the weight-gradient GEMM when
                                the group size divides its tile width (bf16 GEMMs);
                                1: separate kernels (same results bit for bit)       */
    int32_t start_step;      /* resume point in [0, iters]: the call evaluates steps
                                start_step..iters-1 of the iters-step run, reading
                                schedule rows and lr_t at those indices (blog sec. 3
                                algorithm flow; the linear decay keeps its T = iters).
                                V/alpha/beta in are the state before step start_step.
                                loss_trace entries before start_step are untouched.  */
    float best_loss_in;      /* best loss of the steps before start_step (+inf from
                                ar_tune_opts_init: no earlier snapshot).  A step is
                                kept only if its loss is strictly below it; if none
                                is, best_step is -1, final_best_loss is best_loss_in
                                and V/alpha/beta receive the state after the last
                                update (the caller's earlier snapshot stays the best).
                                Must be >= 0 (AR_ERR_INVALID_ARG otherwise).        */
} ar_tune_opts;

/* Fill `opts` with a preset: lr = lr_clip = 5e-3, linear decay, clip box
 * [0.5, 1], bf16 GEMMs, batch and iterations from the preset table, a fresh
 * run (start_step 0, best_loss_in +inf).
 * Errors: AR_ERR_INVALID_ARG for NULL or an unknown preset. */
AR_API ar_status ar_tune_opts_init(ar_tune_opts* opts, int32_t preset);

/* Fake-quantize W (blog sec. 2 RTN and sec. 4 QDQ).
 *  W      DEVICE [N, K] of dtype wt (AR_F32 or AR_BF16)
 *  V      DEVICE fp32 [N, K] or NULL (= 0)
 *  alpha, beta  DEVICE fp32 [N, G] or NULL (= 1); G = K / group_size
 *  W_qdq  DEVICE [N, K] of dtype out_dt (bf16 is the RNE rounding of w^), nullable
 *  codes  DEVICE uint8 [N, K] integer codes q, nullable
 *  scale  DEVICE fp32 [N, G], zero DEVICE uint8 [N, G], nullable
 * With V = NULL and alpha = beta = NULL this is round-to-nearest group
 * quantization.  Stream-ordered, no synchronization. */
AR_API ar_status ar_qdq_rtn(const void* W, ar_dtype wt, int64_t N, int64_t K, const ar_qconfig* qcfg,
                     const float* V, const float* alpha, const float* beta,
                     void* W_qdq, ar_dtype out_dt,
                     uint8_t* codes, float* scale, uint8_t* zero, void* stream);

/* ar_qdq_rtn for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, checks and results (bit for bit) as ar_qdq_rtn, which takes its
 * per-group range buffer (2 * N * G floats) from hipMallocAsync; this entry
 * point uses instead a static device buffer of 64 MiB that the library holds
 * on every GPU it runs on until the process ends, so it calls no hipMalloc,
 * hipFree or allocating library routine.  Limit: N * G <= 8,388,608 groups
 * (G = K / group_size), else AR_ERR_OUT_OF_MEMORY before any HIP call.  The
 * first call on a device looks up that device's buffer (hipGetSymbolAddress).
 * Every call on one GPU shares the buffer: calls that overlap on one GPU
 * (other streams, or other host threads, without ordering between them)
 * race and may produce wrong results; calls ordered on one stream are safe.
 * Stream-ordered, no synchronization. */
AR_API ar_status ar_qdq_rtn_noalloc(const void* W, ar_dtype wt, int64_t N, int64_t K, const ar_qconfig* qcfg,
                             const float* V, const float* alpha, const float* beta,
                             void* W_qdq, ar_dtype out_dt,
                             uint8_t* codes, float* scale, uint8_t* zero, void* stream);

/* Quantize with the given (tuned) parameters and pack to INT4 (coordinates
 * page sec. 2-3: codes, scale, zero-point, packing).  bits must be 4 and K
 * even.  packed DEVICE uint8 [N, K/2]: byte j of a row holds code 2j in its
 * low nibble and code 2j+1 in its high nibble.  scale DEVICE fp32 [N, G],
 * zero DEVICE uint8 [N, G].  V, alpha, beta as in ar_qdq_rtn.
 * Stream-ordered. */
AR_API ar_status ar_pack_int4(const void* W, ar_dtype wt, int64_t N, int64_t K, const ar_qconfig* qcfg,
                       const float* V, const float* alpha, const float* beta,
                       uint8_t* packed, float* scale, uint8_t* zero, void* stream);

/* INT4-weight GEMM on the output of ar_pack_int4 (the deployment form of a
 * tuned layer: AutoRound blog sec. 4, QDQ versus real INT4 kernels;
 * coordinates page sec. 2-3, packed weight + per-group scale and zero-point):
 *   Y[m, n] = sum_k X[m, k] * bf16(scale[n, k/g] * (q[n, k] - zero[n, k/g]))
 * with q the 4-bit codes of `packed` and fp32 accumulation.  The weight
 * operand is bit for bit the bf16 rounding of the quantizer's w^, so Y is
 * X times the bf16 fake-quantized weight.
 *  X       DEVICE bf16 [M, K], row-major, contiguous
 *  packed  DEVICE uint8 [N, K/2] (layout of ar_pack_int4), scale DEVICE fp32
 *          [N, G], zero DEVICE uint8 [N, G]; G = K / g, g = group_size (-1 = K)
 *  Y       DEVICE [M, N] row-major of dtype yt (AR_F32, or AR_BF16 = the RNE
 *          rounding of the fp32 sum)
 * M = 0 is an empty product and returns AR_OK (X and Y may then be NULL).
 * Errors: AR_ERR_INVALID_ARG for NULL pointers, M < 0, N or K <= 0 or a group
 * size that does not divide K; AR_ERR_UNSUPPORTED for a non-bf16 X, K not a multiple of 64 (or not
 * below 2^30), a group size not a multiple of 8, or X not 16-byte / packed
 * not 4-byte aligned.  The caller keeps ownership of every buffer;
 * nothing is allocated.  Stream-ordered, no synchronization. */
AR_API ar_status ar_w4a16_gemm(const void* X, ar_dtype xt, int64_t M, int64_t K,
                        const uint8_t* packed, const float* scale, const uint8_t* zero, int64_t N,
                        int32_t group_size, void* Y, ar_dtype yt, void* stream);

/* One evaluation of the tuning objective and its straight-through gradients
 * (blog sec. 3 algorithm flow, steps 2-4) on the samples ids[0..B-1] of the
 * pool X_pool DEVICE [S, T, K] (dtype xt; M = B*T rows):
 *   L = sum((X_b w^T - X_b W^T)^2) / (M*N)
 *   G = dL/dw^ (fp32 [N, K]), dV = G*s*m, dalpha, dbeta (fp32 [N, G]),
 * m = [0 <= rint(W/s+V)+z <= Q].  ids is HOST int32 [B].  loss is HOST
 * (double), the gradient outputs are DEVICE and nullable.  Synchronizes.
 * T must be a multiple of 64.  Same dtype rules as ar_tune_layer. */
AR_API ar_status ar_layer_grads(const void* W, ar_dtype wt, int64_t N, int64_t K,
                         const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                         const int32_t* ids, int32_t B,
                         const ar_qconfig* qcfg, ar_gemm_mode mode,
                         const float* V, const float* alpha, const float* beta,
                         double* loss, float* G, float* dV, float* dalpha, float* dbeta,
                         void* stream);

/* Tune one linear layer (blog sec. 3 algorithm flow, steps 1-6): reference
 * output once, then opts->iters SignSGD steps on minibatches of
 * opts->batch_samples samples, keeping the best-loss state.
 *  W       DEVICE [N, K] (wt), X_pool DEVICE [S, T, K] (xt).  AR_GEMM_BF16
 *          needs bf16 W and X; AR_GEMM_F32 takes either (bf16 widens exactly)
 *  V       DEVICE fp32 [N, K]       in: initial offsets, out: tuned
 *  alpha, beta DEVICE fp32 [N, G]   in: initial factors, out: tuned
 *  final_best_loss HOST, best_step HOST, nullable.
 * Synchronizes once at the end.  A non-finite loss stops the updates and
 * returns AR_ERR_NONFINITE with the best state so far written back. */
AR_API ar_status ar_tune_layer(const void* W, ar_dtype wt, int64_t N, int64_t K,
                        const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                        const ar_qconfig* qcfg, const ar_tune_opts* opts,
                        float* V, float* alpha, float* beta,
                        float* final_best_loss, int32_t* best_step, void* stream);

/* Stepwise form of ar_tune_layer for callers that time or interleave the
 * loop.  create() validates, allocates the workspace (hipMallocAsync on
 * `stream`), scans for non-finite inputs and computes the reference output
 * (synchronizes); run() enqueues `nsteps` further steps (stream-ordered;
 * flags below); finish() writes the best (or last) state to the caller's
 * V/alpha/beta and the loss results (synchronizes); destroy() waits for the
 * tuner's own work and frees the workspace on `stream` (hipFreeAsync), so
 * that stream must stay valid until destroy().  The one-call entry points
 * (ar_tune_layer, ar_tune_block, ar_tune_blocks, ar_layer_grads,
 * ar_block_grads) free their workspace the same way before returning.  The
 * caller's W and X_pool must stay valid until destroy(). */
typedef struct ar_tuner ar_tuner;

enum {
    AR_RUN_GRAPH = 1,  /* replay captured HIP graphs: one per step, or (layer
                          tuner, iters >= 8) one per 8 steps while 8 remain;
                          captured on the first such run                          */
    AR_RUN_EVENTS = 2, /* bracket each kernel of each step with HIP events; read
                          the per-kernel mean durations with ar_tuner_kernel_ms   */
    AR_RUN_KERNEL_GRAPHS = 4  /* timing only: for each kernel of a step in turn, a
                          graph of nsteps launches of that kernel alone, replayed
                          between two HIP events (durations as inside a captured
                          step, without an event between kernels; read them with
                          ar_tuner_kernel_ms).  Uses nsteps of the iteration
                          budget; the weight-gradient launches reuse the last
                          forward's outputs, so the state they leave is not a
                          tuning trajectory                                       */
};

AR_API ar_status ar_tuner_create(ar_tuner** out, const void* W, ar_dtype wt, int64_t N, int64_t K,
                          const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                          const ar_qconfig* qcfg, const ar_tune_opts* opts,
                          const float* V0, const float* alpha0, const float* beta0, void* stream);
AR_API ar_status ar_tuner_run(ar_tuner* t, int32_t nsteps, int32_t flags);
AR_API ar_status ar_tuner_finish(ar_tuner* t, float* V, float* alpha, float* beta,
                          float* final_best_loss, int32_t* best_step);
AR_API ar_status ar_tuner_destroy(ar_tuner* t);
/* Number and names of the kernels one step launches, and (after a run with
 * AR_RUN_EVENTS, which synchronizes) their mean durations in ms, HOST
 * float [ar_tuner_num_kernels()]. */
AR_API int32_t ar_tuner_num_kernels(const ar_tuner* t);
AR_API const char* ar_tuner_kernel_name(const ar_tuner* t, int32_t i);
AR_API ar_status ar_tuner_kernel_ms(const ar_tuner* t, float* mean_ms);

/* Block-wise tuning (AutoRound blog sec. 3, "Why Block-Wise Optimization"
 * and steps 1-7 of the algorithm flow): the rounding offsets and clip factors
 * of every linear of a block are tuned jointly on the MSE of the block's
 * output against its reference output with the original weights, with one
 * best-loss snapshot for the block, and the quantized block's output is what
 * the next block takes as input.
 *
 * Built: the gated MLP of Llama-style decoders (kind AR_BLOCK_MLP_SWIGLU) on
 * the normalized block input X [S, T, H]:
 *     Y = (silu(X Wg^T) * (X Wu^T)) Wd^T,  silu(a) = a / (1 + exp(-a)),
 * weights[0] = gate Wg [F, H], weights[1] = up Wu [F, H], weights[2] = down
 * Wd [H, F] (H = hidden, F = ffn), all of dtype weight_dtype.  A residual
 * added to both outputs cancels in the loss.  L = sum((Y_q - Y_ref)^2) /
 * (M H) over the M = B T rows of a step.  Parameter arrays are indexed
 * 0 = gate, 1 = up, 2 = down: V[i] fp32 [N_i, K_i], alpha[i] / beta[i] fp32
 * [N_i, K_i / g] (g divides both H and F).  In AR_GEMM_BF16 mode every GEMM
 * operand is bf16 (fake-quantized weights, the activation entering the down
 * projection, dY and the gradients entering the gate/up weight gradients)
 * with fp32 accumulation; the reference forward rounds at the same places;
 * AR_GEMM_F32 rounds nothing.
 *
 * Also built: a whole Llama-style decoder block (kind AR_BLOCK_LLAMA_DECODER;
 * pre-normalization, rotary positions, causal grouped-query attention and
 * the gated MLP) on the block input x [S, T, H] (the residual stream):
 *     h1 = rmsnorm(x) w1,  q = h1 Wq^T, k = h1 Wk^T, v = h1 Wv^T
 *     q, k rotated per head (pairs i and i + d/2 of a head of size d, angle
 *         t theta^(-2i/d) at token t of its sample)
 *     o = causal softmax(q k^T / sqrt(d)) v per sample and head (query head
 *         j reads KV head j / (heads / kv_heads))
 *     h = x + o Wo^T,  h2 = rmsnorm(h) w2,  y = h + (silu(h2 Wg^T) * (h2 Wu^T)) Wd^T
 * with rmsnorm(z) = z / sqrt(mean(z^2) + norm_eps) per token.  weights[0..6]
 * = q [heads d, H], k [kv_heads d, H], v [kv_heads d, H], o [H, heads d],
 * gate [F, H], up [F, H], down [H, F] (d = head_dim), parameter arrays
 * indexed the same way; norm_weights[0] = w1, [1] = w2, DEVICE fp32 [H],
 * nullable (all ones).  Requirements (AR_ERR_UNSUPPORTED otherwise): bf16
 * weights and x, AR_GEMM_BF16, head_dim 64 or 128, T a multiple of 64 and
 * at most 256, H, F and heads d multiples of 64, a group size g dividing H,
 * F and heads d; heads a multiple of kv_heads (AR_ERR_INVALID_ARG).  GEMM
 * and attention operands are bf16 (h1, h2, the fake-quantized weights, the
 * rotated q and k, v, the softmax probabilities, the attention output, the
 * MLP activation, dY, the gradients entering each GEMM) with fp32
 * accumulation and fp32 normalization, softmax and rotation; the reference
 * forward rounds at the same places.  Y_q_out is bf16. */
typedef enum { AR_BLOCK_MLP_SWIGLU = 0, AR_BLOCK_LLAMA_DECODER = 1 } ar_block_kind;

typedef struct {
    int32_t kind;                /* ar_block_kind */
    ar_dtype weight_dtype;       /* dtype of every weight */
    int64_t hidden, ffn, heads, kv_heads, head_dim;
    float norm_eps, rope_theta;  /* decoder block only */
    const void* weights[7];      /* DEVICE; MLP: gate, up, down */
    const void* norm_weights[2]; /* decoder block only */
} ar_block_desc;

/* Tune the block in one call: ar_block_tuner_create, run all opts->iters
 * steps (captured graph), ar_block_tuner_finish.  V/alpha/beta are DEVICE
 * in/out (initial state in, tuned state out).  Y_q_out DEVICE [S, T, H] of
 * dtype xt, nullable: the block's output on every pool sample with the tuned
 * fake-quantized weights (blog sec. 3 step 7), the next block's input.
 * Errors as ar_tune_layer; AR_ERR_UNSUPPORTED for an unsupported kind. */
AR_API ar_status ar_tune_block(const ar_block_desc* desc, const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                        const ar_qconfig* qcfg, const ar_tune_opts* opts,
                        float* const V[], float* const alpha[], float* const beta[],
                        void* Y_q_out, float* final_best_loss, int32_t* best_step, void* stream);

/* Stepwise form: ar_tuner_run, ar_tuner_destroy and the kernel-timing calls
 * of the layer tuner apply; finish with ar_block_tuner_finish (writes the
 * best state, or the last with opts->return_last, and optionally Y_q_out). */
AR_API ar_status ar_block_tuner_create(ar_tuner** out, const ar_block_desc* desc, const void* X_pool, ar_dtype xt,
                                int64_t S, int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* opts,
                                const float* const V0[], const float* const alpha0[],
                                const float* const beta0[], void* stream);
AR_API ar_status ar_block_tuner_finish(ar_tuner* t, float* const V[], float* const alpha[], float* const beta[],
                                void* Y_q_out, float* final_best_loss, int32_t* best_step);

/* One evaluation of the block objective and its straight-through gradients
 * on the pool samples ids[0..B-1] (HOST int32): loss (HOST double), and per
 * linear i the DEVICE fp32 outputs G[i] = dL/dw^ [N_i, K_i], dV[i], dalpha[i],
 * dbeta[i] (arrays and entries nullable).  Synchronizes. */
AR_API ar_status ar_block_grads(const ar_block_desc* desc, const void* X_pool, ar_dtype xt, int64_t S, int64_t T,
                         const int32_t* ids, int32_t B, const ar_qconfig* qcfg, ar_gemm_mode mode,
                         const float* const V[], const float* const alpha[], const float* const beta[],
                         double* loss, float* const G[], float* const dV[], float* const dalpha[],
                         float* const dbeta[], void* stream);

/* Block-by-block quantization of a stack of blocks whose weights stay in host
 * memory (blog sec. 3 "Algorithm Flow" step 7: each block is tuned on the
 * quantized output of the block before it, then frozen; blog sec. 4
 * "Compatibility with Block-by-Block Loading": only the block being tuned is
 * on the device).  Blocks 0..n_blocks-1 are tuned in order, each as
 * ar_tune_block tunes it (same kernels, same results), block b on the
 * output of block b-1 computed with its tuned fake-quantized weights (block
 * 0 on X_pool).  The device holds two blocks at a time: while block b tunes
 * on `stream`, a copy stream of the library moves block b+1's weights and
 * initial state host -> device, and block b's tuned state goes back to the
 * caller's arrays after it finishes.
 *  blocks   HOST [n_blocks] descriptors (n_blocks >= 1, else
 *           AR_ERR_INVALID_ARG) whose weights[] and norm_weights[]
 *           are HOST pointers.  Page-locked memory (hipHostMalloc) lets the
 *           copies overlap the tuning; pageable memory gives the same results
 *           with copies that do not overlap.  Every block has the hidden size
 *           of block 0; kinds may differ.
 *  X_pool   DEVICE [S, T, hidden] of dtype xt: block 0's input.
 *  qcfg, opts  shared by every block.  opts->start_step must be 0 and
 *           opts->best_loss_in is ignored (every block starts fresh);
 *           opts->loss_trace, when set, is HOST [n_blocks * iters] with block
 *           b's trace at offset b * iters.
 *  V, alpha, beta  HOST arrays of 7 * n_blocks pointers: entry 7 b + i is
 *           linear i of block b (index as ar_block_desc.weights; entries past
 *           a block's linears are ignored), each HOST fp32 of the shape
 *           ar_tune_block takes; in/out: initial state in, tuned state out.
 *  Y_out    DEVICE [S, T, hidden] of dtype xt, nullable: the last block's
 *           quantized output; must not overlap X_pool.
 *  best_losses, best_steps  HOST [n_blocks], nullable.
 * Every argument of every block is checked before the first HIP call
 * (AR_ERR_INVALID_ARG / AR_ERR_UNSUPPORTED as ar_tune_block, message prefixed
 * with the block index; AR_ERR_INVALID_ARG for a differing hidden size or a
 * non-zero start_step).  A block that fails stops the stack: earlier blocks'
 * states are written; a block that halts on a non-finite loss gets its best
 * state written and AR_ERR_NONFINITE is returned; later blocks are untouched.
 * Device memory (stream-ordered allocations on `stream`, freed before
 * return): two slots of the largest block's weights and parameters, two
 * activation buffers, and each block tuner's workspace in turn
 * (AR_ERR_OUT_OF_MEMORY if an allocation fails).  Synchronizes `stream`
 * and the copy stream before returning, on every path. */
AR_API ar_status ar_tune_blocks(const ar_block_desc* blocks, int32_t n_blocks, const void* X_pool, ar_dtype xt,
                         int64_t S, int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* opts,
                         float* const V[], float* const alpha[], float* const beta[], void* Y_out,
                         float* best_losses, int32_t* best_steps, void* stream);

/* Text of the last error on the calling thread (valid until its next call). */
AR_API const char* ar_last_error(void);
AR_API const char* ar_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBAUTOROUND_H */
