"""Oracle of block-wise tuning for a Llama-style decoder block -- test
infrastructure.

The AutoRound blog (sec. 3, "Why Block-Wise Optimization") tunes every
linear of a Transformer decoder block jointly on the MSE of the block's
output, because quantization errors of the attention and MLP sub-layers
propagate into each other.  Block (pre-normalization, as in Llama):

    h1 = rmsnorm(x) * w1
    q = h1 Wq^T, k = h1 Wk^T, v = h1 Wv^T        (nq, nkv heads of size d)
    q, k <- rope(q), rope(k)                      (rotate-half pairing, base theta)
    o_h = softmax(q_h k_g^T / sqrt(d) + causal) v_g,  g = h // (nq / nkv)
    h = x + o Wo^T
    h2 = rmsnorm(h) * w2
    y = h + (silu(h2 Wg^T) * (h2 Wu^T)) Wd^T
    rmsnorm(z) = z / sqrt(mean(z^2) + eps) per token; attention within a sample.

L = sum((y_q - y_ref)^2) / (M H).  The reference forward uses the original
weights.  Mode "f32": fp64 throughout; mode "bf16": every GEMM and attention
operand is rounded to bf16 where the GPU path rounds it (weights, h1, h2,
the rotated q, k and v, P, the attention output, Hh, dY, dA/dB, dh, dO and
dq/dk/dv); accumulation and the elementwise steps in fp64.  The quantizer
and the straight-through estimator are the layer oracle's.
"""
from __future__ import annotations

import numpy as np

from .autoround_ref import F32, _smooth_qdq, bf16_round, gather_batch, lr_table, qdq, signsgd_step, ste_grads

LINEARS = ("q", "k", "v", "o", "gate", "up", "down")


def _rounder(mode: str):
    if mode == "bf16":
        return lambda x: bf16_round(np.asarray(x, np.float64).astype(F32)).astype(np.float64)
    if mode in ("f32", "smooth"):
        return lambda x: np.asarray(x, np.float64)
    raise ValueError(mode)


def rms_norm(z, w, eps):
    z = np.asarray(z, np.float64)
    r = 1.0 / np.sqrt(np.mean(z * z, axis=1, keepdims=True) + eps)
    return z * r * np.asarray(w, np.float64)[None, :], r


def rope_tables(T: int, d: int, theta: float):
    """cos, sin [T, d/2]: angle t * theta^(-2i/d)."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / d)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, cos, sin, nheads: int, d: int, inverse: bool = False):
    """Rotate-half RoPE on [M, nheads*d] with positions from the cos/sin rows
    (one row per token).  ``inverse`` applies the transpose (the backward)."""
    M = x.shape[0]
    xh = np.asarray(x, np.float64).reshape(M, nheads, d)
    a, b = xh[..., : d // 2], xh[..., d // 2:]
    c, s = cos[:, None, :], sin[:, None, :]
    if inverse:
        out = np.concatenate([a * c + b * s, -a * s + b * c], axis=2)
    else:
        out = np.concatenate([a * c - b * s, b * c + a * s], axis=2)
    return out.reshape(M, nheads * d)


def _attention(qr, kr, vv, T, nq, nkv, d, r):
    """Causal softmax attention per sample of T tokens; returns (o, P) with
    P [n_samples, nq, T, T]."""
    M = qr.shape[0]
    nb = M // T
    rep = nq // nkv
    q = qr.reshape(nb, T, nq, d).transpose(0, 2, 1, 3)
    k = kr.reshape(nb, T, nkv, d).transpose(0, 2, 1, 3)
    v = vv.reshape(nb, T, nkv, d).transpose(0, 2, 1, 3)
    kx = np.repeat(k, rep, axis=1)
    vx = np.repeat(v, rep, axis=1)
    S = q @ kx.transpose(0, 1, 3, 2) / np.sqrt(d)
    mask = np.triu(np.ones((T, T), bool), 1)
    S = np.where(mask, -np.inf, S)
    S = S - S.max(axis=3, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=3, keepdims=True)
    o = r(P) @ vx
    return o.transpose(0, 2, 1, 3).reshape(M, nq * d), P


def decoder_forward(X, Ws, cfg, mode: str = "f32"):
    """Block output and the intermediates the backward needs.  ``Ws`` maps the
    linear names to weights (fake-quantized or original); cfg has H, nq, nkv,
    d, F, T, eps, theta, w1, w2."""
    r = _rounder(mode)
    H, nq, nkv, d, T = cfg["H"], cfg["nq"], cfg["nkv"], cfg["d"], cfg["T"]
    X = np.asarray(X, np.float64)
    M = X.shape[0]
    cos, sin = rope_tables(T, d, cfg["theta"])
    cosM, sinM = np.tile(cos, (M // T, 1)), np.tile(sin, (M // T, 1))
    h1, r1 = rms_norm(X, cfg["w1"], cfg["eps"])
    h1o = r(h1)
    q = h1o @ r(Ws["q"]).T
    k = h1o @ r(Ws["k"]).T
    v = h1o @ r(Ws["v"]).T
    qr = r(rope(q, cosM, sinM, nq, d))
    kr = r(rope(k, cosM, sinM, nkv, d))
    vv = r(v)
    o, P = _attention(qr, kr, vv, T, nq, nkv, d, r)
    oo = r(o)
    h = X + oo @ r(Ws["o"]).T
    h2, r2 = rms_norm(h, cfg["w2"], cfg["eps"])
    h2o = r(h2)
    A = h2o @ r(Ws["gate"]).T
    B = h2o @ r(Ws["up"]).T
    sg = 1.0 / (1.0 + np.exp(-A))
    Hh = A * sg * B
    Hop = r(Hh)
    y = h + Hop @ r(Ws["down"]).T
    return dict(y=y, h1o=h1o, qr=qr, kr=kr, vv=vv, P=P, oo=oo, h=h, r2=r2, h2o=h2o, A=A, B=B, sg=sg, Hop=Hop,
                cosM=cosM, sinM=sinM)


def decoder_reference(X_pool, Ws, cfg, mode: str = "f32"):
    S, T, H = X_pool.shape
    return decoder_forward(X_pool.reshape(S * T, H), Ws, cfg, mode)["y"].reshape(S, T, H)


def decoder_loss_and_grads(X_b, Y_ref_b, Ws, Vs, alphas, betas, bits: int, g: int, cfg, mode: str = "f32",
                           smooth: bool = False, sym: bool = False, ste_rows=None):
    """MSE of the fake-quantized decoder block and the STE gradients of all
    seven linears.  Returns dict(L, D, G={name: G}, grads={name: (dV, dalpha,
    dbeta)}).  ``ste_rows`` ({name: row indices}, optional) evaluates the
    straight-through step only on those weight rows of each linear (a row of
    dV, dalpha, dbeta depends only on the same row of G and of the weight),
    so a test of a very large block can sample rows; G stays whole."""
    r = _rounder("smooth" if smooth else mode)
    qfun = _smooth_qdq if smooth else qdq
    qd = {nm: qfun(np.asarray(Ws[nm], F32), Vs[nm], alphas[nm], betas[nm], bits, g, sym) for nm in LINEARS}
    wq = {nm: qd[nm]["w_hat"] for nm in LINEARS}
    f = decoder_forward(X_b, wq, cfg, "smooth" if smooth else mode)
    H, nq, nkv, d, T = cfg["H"], cfg["nq"], cfg["nkv"], cfg["d"], cfg["T"]
    w = {nm: r(wq[nm]) for nm in LINEARS}
    M = f["y"].shape[0]
    D = f["y"] - np.asarray(Y_ref_b, np.float64)
    L = float(np.sum(D * D) / (M * H))
    dY = r((2.0 / (M * H)) * D)
    G = {}
    # MLP
    G["down"] = dY.T @ f["Hop"]
    dHh = dY @ w["down"]
    A, B, sg = f["A"], f["B"], f["sg"]
    dA = r(dHh * B * sg * (1.0 + A * (1.0 - sg)))
    dB = r(dHh * A * sg)
    G["gate"] = dA.T @ f["h2o"]
    G["up"] = dB.T @ f["h2o"]
    dh2 = dA @ w["gate"] + dB @ w["up"]
    # second norm and the residual
    h, r2 = f["h"], f["r2"]
    w2 = np.asarray(cfg["w2"], np.float64)[None, :]
    u = dh2 * w2
    dh = dY + u * r2 - h * r2 ** 3 * np.sum(h * u, axis=1, keepdims=True) / H
    dho = r(dh)
    # attention output projection
    G["o"] = dho.T @ f["oo"]
    dO = r(dho @ w["o"])
    # attention core
    nb = M // T
    rep = nq // nkv
    q = f["qr"].reshape(nb, T, nq, d).transpose(0, 2, 1, 3)
    k = np.repeat(f["kr"].reshape(nb, T, nkv, d).transpose(0, 2, 1, 3), rep, axis=1)
    v = np.repeat(f["vv"].reshape(nb, T, nkv, d).transpose(0, 2, 1, 3), rep, axis=1)
    dOh = dO.reshape(nb, T, nq, d).transpose(0, 2, 1, 3)
    P = f["P"]
    Pr = r(P)
    dV = Pr.transpose(0, 1, 3, 2) @ dOh
    dP = dOh @ v.transpose(0, 1, 3, 2)
    dS = r(P * (dP - np.sum(dP * P, axis=3, keepdims=True)) / np.sqrt(d))
    dQ = dS @ k
    dK = dS.transpose(0, 1, 3, 2) @ q
    dK = dK.reshape(nb, nkv, rep, T, d).sum(axis=2)
    dV = dV.reshape(nb, nkv, rep, T, d).sum(axis=2)
    dq = dQ.transpose(0, 2, 1, 3).reshape(M, nq * d)
    dk = dK.transpose(0, 2, 1, 3).reshape(M, nkv * d)
    dv = dV.transpose(0, 2, 1, 3).reshape(M, nkv * d)
    dq_pre = r(rope(dq, f["cosM"], f["sinM"], nq, d, inverse=True))
    dk_pre = r(rope(dk, f["cosM"], f["sinM"], nkv, d, inverse=True))
    G["q"] = dq_pre.T @ f["h1o"]
    G["k"] = dk_pre.T @ f["h1o"]
    G["v"] = r(dv).T @ f["h1o"]
    if ste_rows is None:
        grads = {nm: ste_grads(np.asarray(Ws[nm], F32), G[nm], qd[nm], bits, g, sym) for nm in LINEARS}
    else:
        grads = {}
        for nm in LINEARS:
            rows = np.asarray(ste_rows[nm])
            sub = {key: np.asarray(val)[rows] for key, val in qd[nm].items()}
            grads[nm] = ste_grads(np.asarray(Ws[nm], F32)[rows], G[nm][rows], sub, bits, g, sym)
    return dict(L=L, D=D, G=G, grads=grads)


def tune_decoder(X_pool, Ws, cfg, schedule, bits: int, g: int, iters: int, lr: float, decay: bool = True,
                 mode: str = "f32", clip_lo: float = 0.5, clip_hi: float = 1.0, lr_clip: float | None = None,
                 return_last: bool = False, sym: bool = False):
    """Joint SignSGD tuning of the seven linears: one loss, one snapshot."""
    Y_ref = decoder_reference(X_pool, Ws, cfg, mode)
    p = {}
    for nm in LINEARS:
        n, k = np.asarray(Ws[nm]).shape
        p[nm] = (np.zeros((n, k), F32), np.ones((n, k // g), F32), np.ones((n, k // g), F32))
    lrs = lr_table(lr, iters, decay)
    lrs_c = lrs if lr_clip is None else lr_table(lr_clip, iters, decay)
    best, best_step = np.inf, -1
    snap = {nm: tuple(a.copy() for a in p[nm]) for nm in LINEARS}
    losses = np.zeros(iters, np.float64)
    for t in range(iters):
        X_b = gather_batch(X_pool, schedule[t])
        Yr = gather_batch(Y_ref, schedule[t])
        res = decoder_loss_and_grads(X_b, Yr, Ws, {nm: p[nm][0] for nm in LINEARS},
                                     {nm: p[nm][1] for nm in LINEARS}, {nm: p[nm][2] for nm in LINEARS},
                                     bits, g, cfg, mode=mode, sym=sym)
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


def quantized_decoder_output(X_pool, Ws, cfg, params, bits: int, g: int, mode: str = "f32", sym: bool = False):
    wq = {nm: qdq(np.asarray(Ws[nm], F32), *params[nm], bits, g, sym)["w_hat"] for nm in LINEARS}
    return decoder_reference(X_pool, wq, cfg, mode)
