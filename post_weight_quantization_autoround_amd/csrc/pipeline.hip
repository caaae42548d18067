// Block-sequential quantization of a stack of blocks whose weights stay in
// host memory (AutoRound blog, sec. 3 "Algorithm Flow" step 7: a tuned block
// is frozen and its quantized output is the next block's input; sec. 4
// "Compatibility with Block-by-Block Loading": only the block being tuned
// needs to be on the device).
//
// Two device slots hold the weights and tuning state of two blocks.  While
// block b tunes on the caller's stream, a copy stream moves block b-1's tuned
// state back to the caller's host arrays and then block b+1's weights and
// initial state into the slot block b-1 held.  The quantized outputs
// alternate between two activation buffers.  Each block is tuned by the
// block tuner (ar_block_tuner_create / ar_tuner_run / ar_block_tuner_finish),
// so a staged block computes exactly what ar_tune_block computes on the same
// device-resident inputs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "tuner.h"

namespace ar {
namespace rt {
namespace {

constexpr int kStride = 7;  // parameter-array entries per block (the decoder's seven linears)

struct BlockShapes {
    int n = 0;                 // linears
    int64_t N[kStride] = {}, K[kStride] = {}, G[kStride] = {};
    size_t wbytes = 0;         // weights (+ the decoder's two norm vectors)
    size_t pbytes = 0;         // V, alpha, beta
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Linear shapes [N, K] of a block, in the order of ar_block_desc.weights.
void block_shapes(const ar_block_desc& d, int32_t g, BlockShapes& s) {
    const int64_t H = d.hidden, F = d.ffn;
    if (d.kind == AR_BLOCK_MLP_SWIGLU) {
        const int64_t dims[3][2] = {{F, H}, {F, H}, {H, F}};
        s.n = 3;
        for (int i = 0; i < 3; ++i) { s.N[i] = dims[i][0]; s.K[i] = dims[i][1]; }
    } else {
        const int64_t NQ = d.heads * d.head_dim, NKV = d.kv_heads * d.head_dim;
        const int64_t dims[7][2] = {{NQ, H}, {NKV, H}, {NKV, H}, {H, NQ}, {F, H}, {F, H}, {H, F}};
        s.n = 7;
        for (int i = 0; i < 7; ++i) { s.N[i] = dims[i][0]; s.K[i] = dims[i][1]; }
    }
    s.wbytes = s.pbytes = 0;
    for (int i = 0; i < s.n; ++i) {
        s.G[i] = s.K[i] / g;
        s.wbytes += align256((size_t)(s.N[i] * s.K[i]) * esize(d.weight_dtype));
        s.pbytes += align256((size_t)(s.N[i] * s.K[i]) * sizeof(float)) +
                    2 * align256((size_t)(s.N[i] * s.G[i]) * sizeof(float));
    }
    if (d.kind == AR_BLOCK_LLAMA_DECODER) s.wbytes += 2 * align256((size_t)H * sizeof(float));
}

// Device copy of one block: weights, norm vectors, parameter arrays.
struct Slot {
    char* base = nullptr;
    const void* w[kStride] = {};
    const void* norm[2] = {};
    float *V[kStride] = {}, *al[kStride] = {}, *be[kStride] = {};
};

void carve_slot(Slot& sl, const ar_block_desc& d, const BlockShapes& s) {
    char* p = sl.base;
    for (int i = 0; i < s.n; ++i) {
        sl.w[i] = p;
        p += align256((size_t)(s.N[i] * s.K[i]) * esize(d.weight_dtype));
    }
    for (int j = 0; j < 2; ++j) {
        sl.norm[j] = nullptr;
        if (d.kind == AR_BLOCK_LLAMA_DECODER && d.norm_weights[j]) sl.norm[j] = p;
        if (d.kind == AR_BLOCK_LLAMA_DECODER) p += align256((size_t)d.hidden * sizeof(float));
    }
    for (int i = 0; i < s.n; ++i) {
        sl.V[i] = reinterpret_cast<float*>(p);
        p += align256((size_t)(s.N[i] * s.K[i]) * sizeof(float));
        sl.al[i] = reinterpret_cast<float*>(p);
        p += align256((size_t)(s.N[i] * s.G[i]) * sizeof(float));
        sl.be[i] = reinterpret_cast<float*>(p);
        p += align256((size_t)(s.N[i] * s.G[i]) * sizeof(float));
    }
}

// Owns the device memory, the copy stream and the events; the destructor
// waits for the copy stream, so no copy into the caller's host arrays is
// still in flight when the call returns, on any path.
// The buffers are stream-ordered allocations on the caller's stream, freed
// on it after the copy stream has drained.
struct Staging {
    hipStream_t user = nullptr;
    char* wmem = nullptr;      // two slots of weights + parameters
    char* act = nullptr;       // two activation buffers
    hipStream_t cs = nullptr;
    hipEvent_t ev_in[2] = {nullptr, nullptr};
    ~Staging() {
        if (cs) (void)hipStreamSynchronize(cs);
        for (hipEvent_t e : ev_in)
            if (e) (void)hipEventDestroy(e);
        if (cs) (void)hipStreamDestroy(cs);
        if (wmem) (void)hipFreeAsync(wmem, user);
        if (act) (void)hipFreeAsync(act, user);
    }
};

// Host -> device copies of block d's weights and initial state into slot sl,
// on the copy stream; ev marks their completion.
ar_status stage_in(const ar_block_desc& d, const BlockShapes& s, const Slot& sl, float* const V[],
                   float* const al[], float* const be[], hipStream_t cs, hipEvent_t ev) {
    for (int i = 0; i < s.n; ++i) {
        const size_t nk = (size_t)(s.N[i] * s.K[i]), ng = (size_t)(s.N[i] * s.G[i]);
        HIPCHK(hipMemcpyAsync(const_cast<void*>(sl.w[i]), d.weights[i], nk * esize(d.weight_dtype),
                              hipMemcpyHostToDevice, cs));
        HIPCHK(hipMemcpyAsync(sl.V[i], V[i], nk * sizeof(float), hipMemcpyHostToDevice, cs));
        HIPCHK(hipMemcpyAsync(sl.al[i], al[i], ng * sizeof(float), hipMemcpyHostToDevice, cs));
        HIPCHK(hipMemcpyAsync(sl.be[i], be[i], ng * sizeof(float), hipMemcpyHostToDevice, cs));
    }
    for (int j = 0; j < 2; ++j)
        if (sl.norm[j])
            HIPCHK(hipMemcpyAsync(const_cast<void*>(sl.norm[j]), d.norm_weights[j], (size_t)d.hidden * sizeof(float),
                                  hipMemcpyHostToDevice, cs));
    HIPCHK(hipEventRecord(ev, cs));
    return AR_OK;
}

ar_status stage_out(const BlockShapes& s, const Slot& sl, float* const V[], float* const al[], float* const be[],
                    hipStream_t cs) {
    for (int i = 0; i < s.n; ++i) {
        const size_t nk = (size_t)(s.N[i] * s.K[i]), ng = (size_t)(s.N[i] * s.G[i]);
        HIPCHK(hipMemcpyAsync(V[i], sl.V[i], nk * sizeof(float), hipMemcpyDeviceToHost, cs));
        HIPCHK(hipMemcpyAsync(al[i], sl.al[i], ng * sizeof(float), hipMemcpyDeviceToHost, cs));
        HIPCHK(hipMemcpyAsync(be[i], sl.be[i], ng * sizeof(float), hipMemcpyDeviceToHost, cs));
    }
    return AR_OK;
}

ar_status tune_blocks_impl(const ar_block_desc* blocks, int32_t nb, const void* X_pool, ar_dtype xt, int64_t S,
                           int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* opts, float* const V[],
                           float* const alpha[], float* const beta[], void* Y_out, float* best_losses,
                           int32_t* best_steps, void* stream) {
    // ---- every check of every block before the first HIP call
    if (!blocks) return fail(AR_ERR_INVALID_ARG, "blocks is NULL");
    if (nb < 1) return fail(AR_ERR_INVALID_ARG, "n_blocks must be >= 1, got %d", nb);
    if (!X_pool) return fail(AR_ERR_INVALID_ARG, "X_pool is NULL");
    if (!opts) return fail(AR_ERR_INVALID_ARG, "opts is NULL");
    if (!V || !alpha || !beta) return fail(AR_ERR_INVALID_ARG, "V, alpha and beta arrays must be non-NULL");
    if (opts->start_step != 0)
        return fail(AR_ERR_INVALID_ARG, "start_step must be 0 for a stack of blocks (resume one block with ar_tune_block)");
    ar_status st = validate_opts(opts, S);
    if (st != AR_OK) return st;
    std::vector<BlockShapes> shapes((size_t)nb);
    size_t slot_bytes = 0;
    for (int32_t b = 0; b < nb; ++b) {
        const ar_block_desc& d = blocks[b];
        if (d.hidden != blocks[0].hidden)
            return fail(AR_ERR_INVALID_ARG, "block %d has hidden %lld, block 0 %lld: a block's output is the next "
                        "block's input", b, (long long)d.hidden, (long long)blocks[0].hidden);
        int32_t g = 0;
        if (d.kind == AR_BLOCK_LLAMA_DECODER)
            st = decoder_validate(&d, X_pool, xt, S, T, qcfg, opts->gemm_mode, &g);
        else
            st = block_validate(&d, X_pool, xt, S, T, qcfg, opts->gemm_mode, &g);
        if (st != AR_OK) return fail(st, "block %d: %s", b, ar_last_error());
        block_shapes(d, g, shapes[(size_t)b]);
        for (int i = 0; i < shapes[(size_t)b].n; ++i) {
            const size_t e = (size_t)b * kStride + (size_t)i;
            if (!V[e] || !alpha[e] || !beta[e])
                return fail(AR_ERR_INVALID_ARG, "V/alpha/beta entry %zu (block %d, linear %d) is NULL", e, b, i);
        }
        const size_t sb = shapes[(size_t)b].wbytes + shapes[(size_t)b].pbytes;
        if (sb > slot_bytes) slot_bytes = sb;
    }

    // ---- device slots, activation buffers, copy stream
    hipStream_t user = static_cast<hipStream_t>(stream);
    const size_t act_bytes = align256((size_t)(S * T * blocks[0].hidden) * esize(xt));
    const int n_act = nb > 2 ? 2 : nb - 1;   // outputs of blocks 0..nb-2 (the last one goes to Y_out)
    Staging sg;
    sg.user = user;
    if (hipMallocAsync(reinterpret_cast<void**>(&sg.wmem), 2 * slot_bytes, user) != hipSuccess) {
        sg.wmem = nullptr;
        (void)hipGetLastError();
        return fail(AR_ERR_OUT_OF_MEMORY, "two block slots of %zu bytes", slot_bytes);
    }
    if (n_act > 0 && hipMallocAsync(reinterpret_cast<void**>(&sg.act), (size_t)n_act * act_bytes, user) != hipSuccess) {
        sg.act = nullptr;
        (void)hipGetLastError();
        return fail(AR_ERR_OUT_OF_MEMORY, "activation buffers of %zu bytes", (size_t)n_act * act_bytes);
    }
    HIPCHK(hipStreamCreateWithFlags(&sg.cs, hipStreamNonBlocking));
    for (hipEvent_t& e : sg.ev_in) HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    // the copy stream's first use of the slots follows their allocation
    HIPCHK(hipEventRecord(sg.ev_in[1], user));
    HIPCHK(hipStreamWaitEvent(sg.cs, sg.ev_in[1], 0));
    Slot slot[2];
    slot[0].base = sg.wmem;
    slot[1].base = sg.wmem + slot_bytes;
    auto act = [&](int32_t b) -> void* { return sg.act + (size_t)(b & 1) * act_bytes; };
    auto prm = [&](float* const* a, int32_t b) { return a + (size_t)b * kStride; };

    carve_slot(slot[0], blocks[0], shapes[0]);
    if ((st = stage_in(blocks[0], shapes[0], slot[0], prm(V, 0), prm(alpha, 0), prm(beta, 0), sg.cs, sg.ev_in[0])) != AR_OK)
        return st;
    // The copy-out of a finished block waits until the next block's tuner
    // exists: its workspace allocation may synchronize the device, so copies
    // enqueued after it overlap that block's steps instead of the allocation.
    // A finished block's state is complete on the host's side (its finish
    // synchronized the tuner's stream), so the copy stream needs no event.
    int32_t pending = -1;
    auto flush = [&]() -> ar_status {
        if (pending < 0) return AR_OK;
        const int32_t p = pending;
        pending = -1;
        return stage_out(shapes[(size_t)p], slot[p & 1], prm(V, p), prm(alpha, p), prm(beta, p), sg.cs);
    };
    for (int32_t b = 0; b < nb; ++b) {
        Slot& sl = slot[b & 1];
        HIPCHK(hipStreamWaitEvent(user, sg.ev_in[b & 1], 0));
        ar_block_desc d = blocks[b];
        for (int i = 0; i < kStride; ++i) d.weights[i] = i < shapes[(size_t)b].n ? sl.w[i] : nullptr;
        d.norm_weights[0] = sl.norm[0];
        d.norm_weights[1] = sl.norm[1];
        ar_tune_opts o = *opts;
        o.loss_trace = opts->loss_trace ? opts->loss_trace + (size_t)b * (size_t)opts->iters : nullptr;
        o.start_step = 0;
        o.best_loss_in = INFINITY;
        const void* in = b == 0 ? X_pool : act(b - 1);
        void* out = b + 1 < nb ? act(b) : Y_out;
        const float* V0[kStride] = {};
        const float* a0[kStride] = {};
        const float* b0[kStride] = {};
        for (int i = 0; i < shapes[(size_t)b].n; ++i) {
            V0[i] = sl.V[i];
            a0[i] = sl.al[i];
            b0[i] = sl.be[i];
        }
        ar_tuner* t = nullptr;
        if ((st = ar_block_tuner_create(&t, &d, in, xt, S, T, qcfg, &o, V0, a0, b0, stream)) != AR_OK) {
            const std::string err(ar_last_error());
            (void)flush();   // the blocks before this one keep their tuned states
            return fail(st, "block %d: %s", b, err.c_str());
        }
        // block b-1's state out, then block b+1's inputs into the slot it held
        st = flush();
        if (st == AR_OK && b + 1 < nb) {
            Slot& nx = slot[(b + 1) & 1];
            carve_slot(nx, blocks[b + 1], shapes[(size_t)b + 1]);
            st = stage_in(blocks[b + 1], shapes[(size_t)b + 1], nx, prm(V, b + 1), prm(alpha, b + 1), prm(beta, b + 1),
                          sg.cs, sg.ev_in[(b + 1) & 1]);
        }
        if (st != AR_OK) {
            ar_tuner_destroy(t);
            return st;
        }
        st = run_impl(t, o.iters, AR_RUN_GRAPH);
        float bl = 0.0f;
        int32_t bs = -1;
        if (st == AR_OK || st == AR_ERR_NONFINITE) {
            // the best state goes back into the slot's parameter arrays
            const ar_status st2 = ar_block_tuner_finish(t, sl.V, sl.al, sl.be, out, &bl, &bs);
            if (st == AR_OK) st = st2;
        }
        const std::string err = st == AR_OK ? std::string() : std::string(ar_last_error());
        ar_tuner_destroy(t);
        if (st != AR_OK && st != AR_ERR_NONFINITE) return fail(st, "block %d: %s", b, err.c_str());
        if (best_losses) best_losses[b] = bl;
        if (best_steps) best_steps[b] = bs;
        pending = b;
        if (st == AR_ERR_NONFINITE) {
            const ar_status so = flush();
            if (so != AR_OK) return so;
            HIPCHK(hipStreamSynchronize(sg.cs));
            return fail(st, "block %d: %s", b, err.c_str());
        }
    }
    if ((st = flush()) != AR_OK) return st;
    HIPCHK(hipStreamSynchronize(sg.cs));
    HIPCHK(hipStreamSynchronize(user));
    return AR_OK;
}

}  // namespace
}  // namespace rt
}  // namespace ar

extern "C" {

ar_status ar_tune_blocks(const ar_block_desc* blocks, int32_t n_blocks, const void* X_pool, ar_dtype xt, int64_t S,
                         int64_t T, const ar_qconfig* qcfg, const ar_tune_opts* opts, float* const V[],
                         float* const alpha[], float* const beta[], void* Y_out, float* best_losses,
                         int32_t* best_steps, void* stream) {
    return ar::rt::tune_blocks_impl(blocks, n_blocks, X_pool, xt, S, T, qcfg, opts, V, alpha, beta, Y_out,
                                    best_losses, best_steps, stream);
}

}  // extern "C"
