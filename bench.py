"""Benchmark: SignSGD tuning steps/s of one 4096 x 4096 bf16 linear layer
(int4 asymmetric, group 128, 2048 calibration tokens per step: 8 samples of
256 tokens from a 128-sample pool), on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 10]

One step is the whole hot path: forward GEMM on the fake-quantized weight
with the MSE epilogue, loss decision, weight-gradient GEMM whose epilogue
runs the straight-through backward, the SignSGD update and the fake
quantization of the updated state for the next step.  Inputs are synthetic (seeded), resident in HBM
before timing; the reference output, transposed pool and group ranges are
prepared by the untimed tuner setup.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(n, k, m, g, bf16=True):
    """Per-launch algorithmic work of each kernel: flops for the GEMMs,
    bytes (minimum HBM traffic of the operation) for the streaming kernels."""
    e = n * k
    G = n * (k // g)
    wb = 2 if bf16 else 4
    return {
        "qdq_fwd": ("GB/s", e * (wb + 4 + wb) + G * 16),                  # W, V in; w^ out; alpha, beta, mx, mn
        "gemm_fwd_loss": ("TFLOP/s", 2.0 * m * n * k),
        "loss_decide": ("GB/s", 0),
        "gemm_wgrad": ("TFLOP/s", 2.0 * m * n * k),
        "ste_bwd": ("GB/s", e * (4 + wb + 4 + 4) + G * 24),               # G, W, V in; dV out; group terms
        "signsgd_update": ("GB/s", e * 12 + G * 24),                      # V, dV in; V out; alpha, beta
        # weight-gradient GEMM with the backward, update and next fake
        # quantization in its epilogue: priced by its MFMA work; its streamed
        # bytes are W, V in and V, w^ out (12 B per weight) plus the operands
        "gemm_wgrad_ste_update": ("TFLOP/s", 2.0 * m * n * k),
    }


def streamed_bytes(n, k, m, g):
    """Algorithmic HBM bytes of the fused weight-gradient kernel: dY^T and
    X_b^T operands (bf16), W and V in, V and w^ out, group parameters."""
    e = n * k
    G = n * (k // g)
    return 2 * n * m + 2 * k * m + e * (2 + 4 + 4 + 2) + G * 24


def blas_info():
    """BLAS library, version and thread count numpy runs the oracle's GEMMs on."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"blas": f"{i.get('internal_api')} {i.get('version')}", "blas_threads": i.get("num_threads"),
                        "blas_arch": i.get("architecture")}
    except Exception:
        pass
    return {"blas": "unknown", "blas_threads": None, "blas_arch": None}


def cpu_baseline(wl, budget_s=15.0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    as many full tuning steps (loss, STE gradients, SignSGD update) of the
    4096 x 4096 layer as fit in about `budget_s` seconds, at least one."""
    import oracle

    info = blas_info()
    affinity = len(os.sched_getaffinity(0))
    threads = info["blas_threads"] or affinity
    V = np.zeros((wl.n, wl.k), np.float32)
    G = wl.k // wl.group
    al = np.ones((wl.n, G), np.float32)
    be = np.ones((wl.n, G), np.float32)
    lrs = oracle.lr_table(wl.lr, wl.iters)
    t0 = time.perf_counter()
    steps = 0
    while True:
        Xb = oracle.gather_batch(wl.X, wl.schedule[steps])
        r = oracle.loss_and_grads(wl.W, Xb, V, al, be, wl.bits, wl.group, mode="bf16")
        V = oracle.signsgd_step(V, r["dV"], lrs[steps], -0.5, 0.5)
        al = oracle.signsgd_step(al, r["dalpha"], lrs[steps], 0.5, 1.0)
        be = oracle.signsgd_step(be, r["dbeta"], lrs[steps], 0.5, 1.0)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 50:
            break
    return {"value": steps / el, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} full tuning steps (bf16-mode oracle: fp32 QDQ, fp64 GEMMs and gradients, "
                      f"fp32 update) of the 4096x4096 g128 layer, 2048 tokens each, {el:.1f} s",
            "blas": info["blas"], "blas_threads": info["blas_threads"], "blas_arch": info["blas_arch"],
            "affinity_cpus": affinity, "os_cpu_count": os.cpu_count()}


def _time_w4a16(ar, torch, Xm, packed, scale, zero, group, reps, repeats):
    """(graph ms, host-loop ms) per launch of ar_w4a16_gemm: `reps` launches
    captured in one graph, replayed between HIP events on torch's current
    stream (median of `repeats`), its output checked against an eager call."""
    m, n = Xm.shape[0], packed.shape[0]
    Y = torch.empty((m, n), dtype=torch.float32, device=Xm.device)
    for _ in range(3):
        ar.w4a16_gemm(Xm, packed, scale, zero, group_size=group, out=Y)
    ref = Y.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ar.w4a16_gemm(Xm, packed, scale, zero, group_size=group, out=Y)
    e1.record()
    torch.cuda.synchronize()
    loop_ms = e0.elapsed_time(e1) / reps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(reps):
            ar.w4a16_gemm(Xm, packed, scale, zero, group_size=group, out=Y)
    torch.cuda.synchronize()
    Y.zero_()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(Y, ref):
        raise RuntimeError(f"INT4-weight GEMM {m}x{n}: graph replay differs from the eager call")
    times = []
    for _ in range(repeats):
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    del graph
    return sorted(times)[len(times) // 2], loop_ms


def w4a16_measurement(ar, torch, W, X_pool, res, wl, reps=50, repeats=5):
    """Time the INT4-weight GEMM on the tuned, packed layer: the 2048-token
    batch (MFMA-bound) and a 16-token decode batch (bound by streaming the
    packed weight); then, as context, the decode batch on a packed weight of
    the 70B block's gate shape (28672 x 8192, random bf16 weight), where one
    launch streams 14x the bytes.  Graph-replayed launches (_time_w4a16); the
    same launches from a Python loop are timed too (`us_host_loop`): for the
    decode batch that loop, not the GPU, sets the pace."""
    packed, scale, zero = ar.pack_int4(W, group_size=wl.group, V=res["V"], alpha=res["alpha"], beta=res["beta"])
    n, k = W.shape
    out = {}
    cases = [("batch", X_pool.reshape(-1, k)[:wl.b * wl.t].contiguous(), packed, scale, zero),
             ("decode", X_pool.reshape(-1, k)[:16].contiguous(), packed, scale, zero)]
    for label, Xm, pk, sc, zp in cases:
        ms, loop_ms = _time_w4a16(ar, torch, Xm, pk, sc, zp, wl.group, reps, repeats)
        out[label] = _w4_entry(Xm.shape[0], pk.shape[0], Xm.shape[1], wl.group, ms, loop_ms, reps, repeats)
    del packed, scale, zero
    gen = torch.Generator(device=W.device).manual_seed(5)
    nl, kl = 28672, 8192
    Wl = (torch.randn((nl, kl), generator=gen, device=W.device) * 0.02).to(torch.bfloat16)
    pl, sl, zl = ar.pack_int4(Wl, group_size=wl.group)
    del Wl
    Xl = (torch.randn((16, kl), generator=gen, device=W.device)).to(torch.bfloat16)
    ms, loop_ms = _time_w4a16(ar, torch, Xl, pl, sl, zl, wl.group, reps, repeats)
    out["decode_28672x8192"] = _w4_entry(16, nl, kl, wl.group, ms, loop_ms, reps, repeats)
    out["decode_28672x8192"]["weight"] = "random N(0, 0.02^2) bf16, round-to-nearest codes (context, not the tuned layer)"
    del pl, sl, zl, Xl
    return out


def _w4_entry(m, n, k, group, ms, loop_ms, reps, repeats):
    G = k // group
    flops = 2.0 * m * n * k
    nbytes = n * k // 2 + 5 * n * G + 2 * m * k + 4 * m * n
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"M": m, "N": n, "K": k, "group": group, "us": round(ms * 1e3, 2), "us_host_loop": round(loop_ms * 1e3, 2),
            "timing": f"graph of {reps} launches, median of {repeats}", "TFLOP/s": round(tf, 1),
            "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


def timed_run(torch, tuner, steps):
    """Seconds for `steps` graph-replayed steps: HIP events on the caller's
    stream, which the tuner's stream follows and joins back."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    tuner.run(steps, graph=True)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def block_measurement(ar, torch, steps=20, warmup=3, event_steps=5):
    """Block-wise tuning of the Llama-7B-shaped SwiGLU MLP block (hidden
    4096, intermediate 11008, int4 g128, 2048-token steps): steps/s of the
    captured step and per-kernel durations (HIP events on the tuner's
    stream).  Seven GEMMs of 2*M*H*F flops each per step (gate and up in one launch)."""
    from synthetic_inputs import make_block_workload

    iters = warmup + steps + event_steps
    t0 = time.perf_counter()
    wl = make_block_workload("mlp4096_11008_g128", iters=iters)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    ws = [torch.from_numpy(a).to(dev).to(torch.bfloat16) for a in (wl.Wg, wl.Wu, wl.Wd, wl.X)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tuner = ar.BlockTuner(*ws, bits=wl.bits, group_size=wl.group, iters=iters, lr=wl.lr, batch_samples=wl.b,
                          schedule=wl.schedule.tolist())
    setup_s = time.perf_counter() - t0
    tuner.run(warmup, graph=True)
    el = timed_run(torch, tuner, steps)
    tuner.run(event_steps, graph=False, kernel_graphs=True)
    kms = tuner.kernel_ms()
    res = tuner.finish()
    tuner.close()
    M, H, F = wl.b * wl.t, wl.h, wl.f
    gemm_flops = 2.0 * M * H * F
    byte_work = {"swiglu_fwd": 12.0 * F * M, "swiglu_bwd": 16.0 * F * M, "transpose_dy": 4.0 * H * M}
    kernels = {}
    for name, ms in kms.items():
        entry = {"ms": round(ms, 5)}
        if name.startswith("gemm_"):
            tf = (2 if name == "gemm_gate_up_fwd" else 1) * gemm_flops / (ms * 1e-3) / 1e12
            entry.update({"TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        elif name in byte_work:
            gbs = byte_work[name] / (ms * 1e-3) / 1e9
            entry.update({"GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)})
        kernels[name] = entry
    sps = steps / el
    return {"workload": wl.name, "H": H, "F": F, "group": wl.group, "tokens_per_step": M,
            "pool": f"{wl.s}x{wl.t}", "steps": steps, "steps_per_s": round(sps, 2),
            "ms_per_step": round(el * 1e3 / steps, 4),
            "mfma_util": round(sps * 7 * gemm_flops / 1e12 / PEAK_BF16_TFLOPS, 4),
            "setup_s": round(setup_s, 3), "input_generation_s": round(gen_s, 1),
            "loss_step0": res["losses"][0], "best_loss": res["best_loss"], "kernels": kernels}


def decoder_measurement(ar, torch, name, steps=20, warmup=3, event_steps=5):
    """Block-wise tuning of a Llama-style decoder block (all seven linears,
    attention and the MLP): steps/s of the captured step and per-kernel
    durations (HIP events on the tuner's stream).  Linear GEMM flops per step:
    forward and weight gradient of all seven linears, input gradient of o,
    gate, up and down (h1 is not a function of the tuned parameters).
    Attention flops count the causal half of each T x T product: two products
    forward, three in the dQ kernel and four in the dK/dV kernel."""
    from synthetic_inputs import make_decoder_workload

    iters = warmup + steps + event_steps
    t0 = time.perf_counter()
    wl = make_decoder_workload(name, iters=iters)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    weights = {n: torch.from_numpy(wl.W[n]).to(dev).to(torch.bfloat16) for n in ar.DECODER_LINEARS}
    X = torch.from_numpy(wl.X).to(dev).to(torch.bfloat16)
    norms = (torch.from_numpy(wl.w1).to(dev), torch.from_numpy(wl.w2).to(dev))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tuner = ar.DecoderTuner(weights, X, wl.heads, wl.kv_heads, wl.head_dim, norm_weights=norms, eps=wl.norm_eps,
                            theta=wl.rope_theta, bits=wl.bits, group_size=wl.group, iters=iters, lr=wl.lr,
                            batch_samples=wl.b, schedule=wl.schedule.tolist())
    setup_s = time.perf_counter() - t0
    tuner.run(warmup, graph=True)
    el = timed_run(torch, tuner, steps)
    tuner.run(event_steps, graph=False, kernel_graphs=True)
    kms = tuner.kernel_ms()
    res = tuner.finish()
    tuner.close()
    M, H, F, T = wl.b * wl.t, wl.h, wl.f, wl.t
    NQ, NKV = wl.heads * wl.head_dim, wl.kv_heads * wl.head_dim
    lin = {"q": 2.0 * M * H * NQ, "k": 2.0 * M * H * NKV, "v": 2.0 * M * H * NKV, "o": 2.0 * M * NQ * H,
           "gate": 2.0 * M * H * F, "up": 2.0 * M * H * F, "down": 2.0 * M * F * H}
    att = 2.0 * wl.b * wl.heads * (T * (T + 1) / 2) * wl.head_dim      # one causal T x T x d product
    flops = {"gemm_qkv": lin["q"] + lin["k"] + lin["v"], "gemm_oproj": lin["o"],
             "gemm_gate_up_fwd": lin["gate"] + lin["up"], "gemm_down_fwd_loss": lin["down"], "gemm_dh": lin["down"],
             "gemm_dh2": lin["gate"] + lin["up"], "gemm_do": lin["o"],
             "attn_fwd": 2 * att, "attn_bwd_dq": 3 * att, "attn_bwd_dkdv": 4 * att}
    for n in ar.DECODER_LINEARS:
        flops[f"gemm_wgrad_{n}_ste_update"] = lin[n]
    # Algorithmic HBM bytes of the streaming kernels (each tensor read or
    # written once): at T <= 256 attention moves more bytes per flop than the
    # MFMA roofline allows for, so HBM bounds it.
    NQKV = NQ + 2 * NKV
    rows = float(M) * wl.heads * 4                                        # lse or Di
    byte_work = {
        "rope_fwd": 8.0 * M * NQKV,                                       # qkv fp32 in; q, k, v and transposes out
        "attn_fwd": 2.0 * M * (NQ + 2 * NKV) + 4.0 * M * NQ + rows,        # q, k, v^T in; o, o^T, lse out
        "attn_bwd_prep": 6.0 * M * NQ + 4.0 * M * NQ + rows,              # dO fp32, o in; dO bf16 + transpose, Di out
        "attn_bwd_dq": 4.0 * M * NQ + 6.0 * M * NKV + 2 * rows + 4.0 * M * NQ,
        "attn_bwd_dkdv": 8.0 * M * NQ + 4.0 * M * NKV + 2 * rows + 8.0 * M * NQ,
        "rope_bwd": 12.0 * M * NQ + 2.0 * M * NQKV,                      # dq, dk, dv partials fp32 in; [dq dk dv]^T out
        "swiglu_fwd": 12.0 * F * M,                                       # A, B fp32 in; h, h^T bf16 out
        "swiglu_bwd": 20.0 * F * M,                                       # dH, A, B fp32 in; dA^T, dB^T, [dA dB] out
    }
    kernels = {}
    for kname, ms in kms.items():
        entry = {"ms": round(ms, 5)}
        if kname in flops and ms > 0:
            tf = flops[kname] / (ms * 1e-3) / 1e12
            entry.update({"TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        if kname in byte_work and ms > 0:
            gbs = byte_work[kname] / (ms * 1e-3) / 1e9
            entry.update({"GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        kernels[kname] = entry
    step_flops = 2 * sum(lin.values()) + lin["o"] + lin["gate"] + lin["up"] + lin["down"] + 9 * att
    sps = steps / el
    return {"workload": wl.name, "H": H, "F": F, "heads": wl.heads, "kv_heads": wl.kv_heads,
            "head_dim": wl.head_dim, "group": wl.group, "tokens_per_step": M, "pool": f"{wl.s}x{wl.t}",
            "steps": steps, "steps_per_s": round(sps, 2), "ms_per_step": round(el * 1e3 / steps, 4),
            "step_TFLOP": round(step_flops / 1e12, 4),
            "mfma_util": round(sps * step_flops / 1e12 / PEAK_BF16_TFLOPS, 4),
            "setup_s": round(setup_s, 3), "input_generation_s": round(gen_s, 1),
            "loss_step0": res["losses"][0], "best_loss": res["best_loss"], "kernels": kernels}


def stack_measurement(ar, torch, n_blocks=3, iters=200):
    """Block-by-block quantization of a stack of Llama-7B-shaped decoder
    blocks whose weights and parameters stay in page-locked host memory
    (ar_tune_blocks), against the same chain with every block already on the
    device (ar_tune_block per block, host-timed, synchronized).  The stack
    reuses one synthetic block's weights, in its own host copy per block.  A
    plain host-to-device copy of one block's weights and initial state gives
    the link rate the staging overlaps with the tuning."""
    from synthetic_inputs import make_decoder_workload

    wl = make_decoder_workload("llama7b_decoder_g128", iters=iters)
    dev = torch.device("cuda:0")
    kw = dict(heads=wl.heads, kv_heads=wl.kv_heads, head_dim=wl.head_dim, eps=wl.norm_eps, theta=wl.rope_theta,
              bits=wl.bits, group_size=wl.group, iters=iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist())
    X = torch.from_numpy(wl.X).to(dev).to(torch.bfloat16)
    host0 = {n: torch.from_numpy(wl.W[n]).to(torch.bfloat16) for n in ar.DECODER_LINEARS}
    host0["norm1"], host0["norm2"] = torch.from_numpy(wl.w1), torch.from_numpy(wl.w2)
    stack = [{k: v.pin_memory() for k, v in host0.items()} for _ in range(n_blocks)]
    dw = {n: stack[0][n].to(dev) for n in ar.DECODER_LINEARS}
    norms = (stack[0]["norm1"].to(dev), stack[0]["norm2"].to(dev))
    wbytes = sum(int(stack[0][n].numel()) * 2 for n in ar.DECODER_LINEARS)
    pbytes = sum(int(stack[0][n].numel()) * 4 * (1 + 2 / wl.group) for n in ar.DECODER_LINEARS)
    # link rate: one block's weights + initial state, pinned host -> device
    src = torch.empty(int(wbytes + pbytes) // 4, dtype=torch.float32, pin_memory=True)
    dst = torch.empty_like(src, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    h2d_s = time.perf_counter() - t0
    del src, dst
    # warm-up of both paths (code objects, allocator), then one timed run each
    ar.tune_decoder(dw, X, norm_weights=norms, output=True, **dict(kw, iters=2, schedule=kw["schedule"][:2]))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    x = X
    for _ in range(n_blocks):
        x = ar.tune_decoder(dw, x, norm_weights=norms, output=True, **kw)["output"]
    torch.cuda.synchronize()
    resident_s = time.perf_counter() - t0
    params = [{n: (torch.zeros(stack[0][n].shape, pin_memory=True),
                   torch.ones((stack[0][n].shape[0], stack[0][n].shape[1] // wl.group), pin_memory=True),
                   torch.ones((stack[0][n].shape[0], stack[0][n].shape[1] // wl.group), pin_memory=True))
               for n in ar.DECODER_LINEARS} for _ in range(n_blocks)]
    t0 = time.perf_counter()
    st = ar.tune_blocks(stack, X, params=params, inplace=True, **kw)
    torch.cuda.synchronize()
    staged_s = time.perf_counter() - t0
    same = bool(torch.equal(st["output"], x))
    return {"workload": f"{n_blocks} x {wl.name}, weights in page-locked host memory", "iters_per_block": iters,
            "tokens_per_step": wl.b * wl.t, "pool": f"{wl.s}x{wl.t}",
            "block_weight_bytes": wbytes, "block_param_bytes": int(pbytes),
            "h2d_GBps": round((wbytes + pbytes) / h2d_s / 1e9, 1),
            "staged_s": round(staged_s, 3), "resident_s": round(resident_s, 3),
            "staging_overhead": round(staged_s / resident_s - 1.0, 4), "same_output_as_resident": same}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--event-steps", type=int, default=50)
    ap.add_argument("--repeats", type=int, default=5, help="timed runs of --steps steps; the median is reported")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-block", action="store_true", help="skip the SwiGLU MLP block measurement")
    ap.add_argument("--no-decoder", action="store_true", help="skip the decoder block measurements")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the block-by-block stack with host-resident weights")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library tunes on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import post_weight_quantization_autoround_amd as ar
    from synthetic_inputs import make_layer_workload

    K_steps, W_steps, E_steps, R = args.steps, args.warmup, args.event_steps, args.repeats
    iters = W_steps + R * K_steps + E_steps
    t0 = time.perf_counter()
    wl = make_layer_workload("linear4096_g128", iters=iters)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    W = torch.from_numpy(wl.W).to(dev).to(torch.bfloat16)
    X = torch.from_numpy(wl.X).to(dev).to(torch.bfloat16)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    tuner = ar.Tuner(W, X, bits=wl.bits, group_size=wl.group, iters=iters, lr=wl.lr, batch_samples=wl.b,
                     schedule=wl.schedule.tolist(), gemm_mode=ar.AR_GEMM_BF16)
    log(f"tuner setup (reference output, transposed pool, ranges) {time.perf_counter() - t0:.2f} s")

    # R repeats of K graph-replayed steps, each bracketed by HIP events on
    # the caller's stream (the tuner orders its own stream after it and joins
    # back before returning) and by a host clock; the reported time is the
    # median over the repeats.
    tuner.run(W_steps, graph=True)
    torch.cuda.synchronize()
    ev_ms, host_ms = [], []
    for _ in range(R):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        tuner.run(K_steps, graph=True)
        e1.record()
        torch.cuda.synchronize()
        host_ms.append((time.perf_counter() - t0) * 1e3)
        ev_ms.append(e0.elapsed_time(e1))
    el = float(np.median(ev_ms)) * 1e-3
    log(f"timed {R} x {K_steps} steps: events {['%.2f' % x for x in ev_ms]} ms, host {['%.2f' % x for x in host_ms]} ms")

    # Per-kernel durations with HIP events on the library's stream: each
    # kernel of the step replayed in a graph of E launches of it alone.
    tuner.run(E_steps, graph=False, kernel_graphs=True)
    kms = tuner.kernel_ms()
    res = tuner.finish()
    tuner.close()
    log("kernel ms:", json.dumps(kms))
    w4 = w4a16_measurement(ar, torch, W, X, res, wl)
    log("int4-weight GEMM:", json.dumps(w4))
    log(f"loss step0 {res['losses'][0]:.6e}  best {res['best_loss']:.6e} at {res['best_step']}")

    M = wl.b * wl.t
    kernel_sum = float(sum(kms.values()))    # eager event-timed kernels of one step
    work = algorithmic_work(wl.n, wl.k, M, wl.group)
    kernels = {}
    for name, ms in kms.items():
        unit, amount = work[name]
        if amount <= 0 or ms <= 0:
            kernels[name] = {"ms": ms}
            continue
        if unit == "TFLOP/s":
            ach = amount / (ms * 1e-3) / 1e12
            peak = PEAK_BF16_TFLOPS
        else:
            ach = amount / (ms * 1e-3) / 1e9
            peak = PEAK_HBM_GBS
        kernels[name] = {"ms": round(ms, 5), "achieved": round(ach, 1), "unit": unit, "frac": round(ach / peak, 4)}
        if name == "gemm_wgrad_ste_update":
            kernels[name]["streamed_GB/s"] = round(streamed_bytes(wl.n, wl.k, M, wl.group) / (ms * 1e-3) / 1e9, 1)
    dominant = max(kms, key=lambda n: kms[n])
    dunit, damount = work[dominant]
    dms = kms[dominant]
    if dunit == "TFLOP/s":
        roof = {"bound": "mfma", "achieved": round(damount / (dms * 1e-3) / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(damount / (dms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dominant
    # HBM bytes per launch of that kernel from the committed rocprofv3 --pmc
    # summary (FETCH_SIZE + WRITE_SIZE, calibrated against a 256 MiB copy);
    # None when the kernel sources changed after the counters were taken.
    from post_weight_quantization_autoround_amd.profiling import read_traffic
    roof["traffic"] = read_traffic(os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                                "hbm_traffic_linear4096_g128.txt"), dominant)

    # on-box peaks (streaming copy, register-only MFMA loop) beside the spec figures
    try:
        from post_weight_quantization_autoround_amd import peaks
        measured = peaks.measure()
    except Exception as exc:          # the probe library is a measurement aid
        measured = {"error": str(exc)}
    if roof["unit"] == "TFLOP/s" and "mfma_bf16_TFLOP/s" in measured:
        roof["measured_peak"] = measured["mfma_bf16_TFLOP/s"]
        roof["frac_of_measured_peak"] = round(roof["achieved"] / measured["mfma_bf16_TFLOP/s"], 4)

    steps_per_s = K_steps / el
    step_flops = 4.0 * M * wl.n * wl.k
    out = {
        "metric": "SignSGD tuning steps/sec (4096² linear, g128, 2048 tok); MFMA util %",
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": round(el * 1e3 / K_steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "linear4096_g128", "N": wl.n, "K": wl.k, "group": wl.group, "bits": wl.bits,
                   "tokens_per_step": M, "pool": f"{wl.s}x{wl.t}", "batch_samples": wl.b,
                   "lr": wl.lr, "parallelism": "none"},
        "mfma_util": round(steps_per_s * step_flops / 1e12 / PEAK_BF16_TFLOPS, 4),
        "timing": {"method": f"HIP events on the caller's stream around {K_steps} graph-replayed steps; "
                             f"median of {R} repeats", "repeats_ms_per_step": [round(x / K_steps, 5) for x in ev_ms],
                   "host_clock_ms_per_step": [round(x / K_steps, 5) for x in host_ms],
                   "kernel_sum_ms": round(kernel_sum, 5),
                   "gap_ms_per_step": round(el * 1e3 / K_steps - kernel_sum, 5)},
        "roofline": roof,
        "measured_peaks": measured,
        "kernels": kernels,
        "w4a16_gemm": w4,
    }
    if not args.no_block:
        del W, X
        torch.cuda.empty_cache()
        out["block_mlp"] = block_measurement(ar, torch)
        log("block:", json.dumps(out["block_mlp"]))
    if not args.no_decoder:
        for key, name in (("block_decoder_7b", "llama7b_decoder_g128"), ("block_decoder_70b", "llama70b_decoder_g32")):
            torch.cuda.empty_cache()
            out[key] = decoder_measurement(ar, torch, name)
            log(f"{key}:", json.dumps(out[key]))
    if not args.no_stack:
        torch.cuda.empty_cache()
        out["block_stack_staged"] = stack_measurement(ar, torch)
        log("block_stack_staged:", json.dumps(out["block_stack_staged"]))
    # A plain 256 MiB device copy, the last device copy of the run: its HBM
    # counters (FETCH_SIZE / WRITE_SIZE under rocprofv3 --pmc) calibrate the
    # per-kernel traffic figures against a transfer of known size.
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if not args.no_cpu_baseline:
        wl_cpu = make_layer_workload("linear4096_g128", iters=50)
        out["cpu_baseline"] = cpu_baseline(wl_cpu, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
