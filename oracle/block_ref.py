"""Oracle of block-wise tuning for a SwiGLU MLP block -- test infrastructure.

The AutoRound blog (sec. 3, "Why Block-Wise Optimization" and the algorithm
flow) tunes the rounding offsets and clip factors of every linear of a block
jointly, on the MSE of the block's output: wrap each linear with the fake
quantizer, take the reference output of the block with the original weights
(a BF16 forward), then repeat {QDQ forward of the block, MSE and backward,
SignSGD on all parameters}, keep the best state, and hand the quantized
block's output to the next block.

Block: the gated MLP of Llama-style decoders on the (already normalized)
block input X [M, H]:
    A = X Wg^T, B = X Wu^T          (gate, up: [F, H] weights)
    Hh = silu(A) * B,  silu(a) = a * sigmoid(a)
    Y = Hh Wd^T                     (down: [H, F] weight)
A residual added to both the reference and the quantized output cancels in
their difference, so the loss is that of the MLP alone.

Precision: the quantizer is the layer oracle's (fp32, fixed order); GEMMs,
activations, loss and gradients are fp64.  In mode "bf16" every GEMM operand
is rounded to bf16 where the GPU path rounds it -- the fake-quantized weights,
the activation Hh entering the down projection, dY, and the gradients dA, dB
entering the gate/up weight gradients -- and the reference forward rounds the
same places (the blog's BF16 reference forward).  Mode "f32" rounds nothing.
"""
from __future__ import annotations

import numpy as np

from .autoround_ref import (F32, _smooth_qdq, bf16_round, gather_batch, lr_table, qdq, signsgd_step,
                            ste_grads)

LINEARS = ("gate", "up", "down")


def silu(a):
    """a * sigmoid(a), fp64."""
    a = np.asarray(a, np.float64)
    return a / (1.0 + np.exp(-a))


def _rounder(mode: str):
    if mode == "bf16":
        return lambda x: bf16_round(np.asarray(x, np.float64).astype(F32)).astype(np.float64)
    if mode in ("f32", "smooth"):
        return lambda x: np.asarray(x, np.float64)
    raise ValueError(mode)


def swiglu_forward(X, Wg, Wu, Wd, mode: str = "f32"):
    """Block output Y = (silu(X Wg^T) * (X Wu^T)) Wd^T with the operand
    rounding of ``mode``; returns (Y, A, B, Hh) in fp64."""
    r = _rounder(mode)
    X = np.asarray(X, np.float64)
    A = X @ r(Wg).T
    B = X @ r(Wu).T
    Hh = silu(A) * B
    Y = r(Hh) @ r(Wd).T
    return Y, A, B, Hh


def block_reference(X_pool, Ws, mode: str = "f32"):
    """Reference output of every pool sample with the original weights
    (blog sec. 3 step 2): [S, T, H]."""
    S, T, H = X_pool.shape
    Y, _, _, _ = swiglu_forward(X_pool.reshape(S * T, H), Ws["gate"], Ws["up"], Ws["down"], mode)
    return Y.reshape(S, T, -1)


def block_loss_and_grads(X_b, Y_ref_b, Ws, Vs, alphas, betas, bits: int, g: int, mode: str = "f32",
                         smooth: bool = False, sym: bool = False):
    """MSE of the fake-quantized block against the reference and the STE
    gradients of every linear's (V, alpha, beta).

    Forward as ``swiglu_forward`` with w_hat in place of each weight;
    D = Y - Y_ref, L = sum(D^2) / (M H).  Backward (chain rule, rounded
    operands as in the forward):
        dY  = 2 D / (M H)
        G_d = dY^T Hh                      dL/dw_hat of down  [H, F]
        dHh = dY w_hat_d                   [M, F]
        dA  = dHh * B * sigmoid(A) * (1 + A (1 - sigmoid(A)))
        dB  = dHh * silu(A)
        G_g = dA^T X,  G_u = dB^T X        [F, H]
    and each G goes through the layer oracle's straight-through estimator.
    ``smooth`` replaces every rounding by the identity (finite-difference
    tests).  Returns dict(L, D, G={name: G}, grads={name: (dV, dalpha, dbeta)},
    qd={name: quantizer state})."""
    r = _rounder("smooth" if smooth else mode)
    qfun = _smooth_qdq if smooth else qdq
    qd = {nm: qfun(np.asarray(Ws[nm], F32), Vs[nm], alphas[nm], betas[nm], bits, g, sym) for nm in LINEARS}
    w = {nm: r(qd[nm]["w_hat"]) for nm in LINEARS}
    X = np.asarray(X_b, np.float64)
    M = X.shape[0]
    A = X @ w["gate"].T
    B = X @ w["up"].T
    sg = 1.0 / (1.0 + np.exp(-A))
    Hh = A * sg * B
    Hop = r(Hh)
    Y = Hop @ w["down"].T
    D = Y - np.asarray(Y_ref_b, np.float64)
    Hdim = Y.shape[1]
    L = float(np.sum(D * D) / (M * Hdim))
    dY = r((2.0 / (M * Hdim)) * D)
    G = {"down": dY.T @ Hop}
    dHh = dY @ w["down"]
    dA = r(dHh * B * sg * (1.0 + A * (1.0 - sg)))
    dB = r(dHh * A * sg)
    G["gate"] = dA.T @ X
    G["up"] = dB.T @ X
    grads = {nm: ste_grads(np.asarray(Ws[nm], F32), G[nm], qd[nm], bits, g, sym) for nm in LINEARS}
    return dict(L=L, D=D, G=G, grads=grads, qd=qd)


def tune_block(X_pool, Ws, schedule, bits: int, g: int, iters: int, lr: float, decay: bool = True,
               mode: str = "f32", clip_lo: float = 0.5, clip_hi: float = 1.0, lr_clip: float | None = None,
               return_last: bool = False, sym: bool = False, init=None):
    """Joint SignSGD tuning of the block's three linears (blog sec. 3 steps
    3-6): one loss and one best-loss snapshot (strict <) for the whole block,
    every parameter moved by lr_t * sign(grad) with the layer oracle's clamps.
    ``init`` optionally gives {name: (V, alpha, beta)}.  Returns dict(params=
    {name: (V, alpha, beta)}, best_loss, best_step, losses)."""
    Y_ref = block_reference(X_pool, Ws, mode)
    p = {}
    for nm in LINEARS:
        n, k = np.asarray(Ws[nm]).shape
        if init is not None:
            p[nm] = tuple(np.array(a, dtype=F32) for a in init[nm])
        else:
            p[nm] = (np.zeros((n, k), F32), np.ones((n, k // g), F32), np.ones((n, k // g), F32))
    lrs = lr_table(lr, iters, decay)
    lrs_c = lrs if lr_clip is None else lr_table(lr_clip, iters, decay)
    best, best_step = np.inf, -1
    snap = {nm: tuple(a.copy() for a in p[nm]) for nm in LINEARS}
    losses = np.zeros(iters, np.float64)
    for t in range(iters):
        X_b = gather_batch(X_pool, schedule[t])
        Yr = gather_batch(Y_ref, schedule[t])
        res = block_loss_and_grads(X_b, Yr, Ws, {nm: p[nm][0] for nm in LINEARS},
                                   {nm: p[nm][1] for nm in LINEARS}, {nm: p[nm][2] for nm in LINEARS},
                                   bits, g, mode=mode, sym=sym)
        losses[t] = res["L"]
        if res["L"] < best:
            best, best_step = res["L"], t
            snap = {nm: tuple(a.copy() for a in p[nm]) for nm in LINEARS}
        for nm in LINEARS:
            V, al, be = p[nm]
            dV, da, db = res["grads"][nm]
            p[nm] = (signsgd_step(V, dV, lrs[t], -0.5, 0.5), signsgd_step(al, da, lrs_c[t], clip_lo, clip_hi),
                     signsgd_step(be, db, lrs_c[t], clip_lo, clip_hi))
    if return_last:
        snap = p
    return dict(params=snap, best_loss=best, best_step=best_step, losses=losses)


def quantized_block_output(X_pool, Ws, params, bits: int, g: int, mode: str = "f32", sym: bool = False):
    """Output of the block with its tuned fake-quantized weights for every
    pool sample: what the next block takes as input (blog sec. 3 step 7)."""
    wq = {nm: qdq(np.asarray(Ws[nm], F32), *params[nm], bits, g, sym)["w_hat"] for nm in LINEARS}
    return block_reference(X_pool, wq, mode)
