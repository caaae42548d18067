"""Reference (oracle) implementation of AutoRound-style weight-only tuning.

Test infrastructure only -- see the package docstring.  Citations name the
page ("AutoRound blog" = "Low-Bit Quantization in Practice with vLLM: Core
Mechanisms and Architectural Optimizations of AutoRound", English version;
"coordinates page" = the Chinese quantization-coordinates article) and the
section, equation or table.

Notation (nn.Linear layout):
  W [N, K]   frozen weight, output rows n, input columns k
  g          group size along K; G = K / g groups per row
  b, Q       bit width and top code Q = 2^b - 1
  V [N, K]   rounding offset, in [-0.5, 0.5]      (blog sec. 3, variable table)
  alpha, beta [N, G]  factors on the group max / min (the blog's learnable
             "max" and "min", re-parameterised as alpha*max and beta*min)
  X_b [M, K] calibration rows of one step; Y = X_b W^T is [M, N]
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 precision, ties to even, returned as fp32.

    bf16 keeps the top 16 bits of the fp32 pattern; rounding adds
    0x7FFF + (bit 16) before truncation.  NaN/Inf are not expected here."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(F32)


def _as_groups(a: np.ndarray, g: int) -> np.ndarray:
    n, k = a.shape
    return a.reshape(n, k // g, g)


# --------------------------------------------------------------------------
# quantize / dequantize  (blog sec. 2 "Essence", sec. 3 variables, sec. 4 table)
# --------------------------------------------------------------------------
def group_range(W: np.ndarray, g: int):
    """Per-group range of the frozen weight, including zero.

    The blog's learnable min/max start at the group minimum/maximum (sec. 3,
    variable table).  The range is widened to contain 0: the sec. 2 worked
    example gives scale = 8.0/15 for [0.1, 0.2, 0.15, 8.0], which is
    (max - min(0, min))/15, and only then dequantizes back to [0, 0, 0, 8.0].
    Returns mx = max(0, max W_g), mn = min(0, min W_g), fp32 [N, G]."""
    Wg = _as_groups(np.asarray(W, dtype=F32), g)
    mx = np.maximum(Wg.max(axis=2), F32(0.0))
    mn = np.minimum(Wg.min(axis=2), F32(0.0))
    return mx.astype(F32), mn.astype(F32)


def group_scale_zero(mx, mn, alpha, beta, bits: int, sym: bool = False):
    """Clip bounds, scale and zero-point of each group (fp32, fixed order).

    Asymmetric (default): wmax = alpha*mx, wmin = beta*mn (the clipped range,
    blog sec. 2 strategy B and sec. 3 "min"/"max"); s = (wmax - wmin)/Q (scale
    from the range, blog sec. 2 "Scaling"); an all-zero range uses s = 1.  The
    zero-point is the integer that wmin maps to: z = rint(-wmin/s) (asymmetric
    mapping with a zero-point, coordinates page sec. 1.2 and the blog's
    w = 0.37 example).

    Symmetric (coordinates page sec. 1.2: q = clip(round(x/s), qmin, qmax),
    x^ = s q): the scale is the clipped maximum magnitude over the largest
    positive level, s = alpha*max(mx, -mn) / (2^(b-1) - 1) (blog sec. 2
    "Scaling": max absolute value over the largest representable value);
    beta is unused.  Codes are stored unsigned with the fixed zero-point
    z = 2^(b-1), so q - z spans [-2^(b-1), 2^(b-1) - 1].  Returns wmin = -wmax."""
    Q = F32(2 ** bits - 1)
    if sym:
        qp = F32(2 ** (bits - 1) - 1)
        amax = np.maximum(np.asarray(mx, dtype=F32), (-np.asarray(mn, dtype=F32)).astype(F32))
        wmax = (np.asarray(alpha, dtype=F32) * amax).astype(F32)
        wmin = (-wmax).astype(F32)
        s = np.where(wmax == F32(0.0), F32(1.0), (wmax / qp).astype(F32)).astype(F32)
        z = np.full(np.shape(s), F32(2 ** (bits - 1)), dtype=F32)
        return wmax, wmin, s, z
    wmax = (np.asarray(alpha, dtype=F32) * np.asarray(mx, dtype=F32)).astype(F32)
    wmin = (np.asarray(beta, dtype=F32) * np.asarray(mn, dtype=F32)).astype(F32)
    d = (wmax - wmin).astype(F32)
    s = np.where(d == F32(0.0), F32(1.0), (d / Q).astype(F32)).astype(F32)
    z = np.rint((-wmin / s).astype(F32)).astype(F32)
    z = np.minimum(np.maximum(z, F32(0.0)), Q)  # identity whenever alpha, beta >= 0
    z = z + F32(0.0)                             # -0.0 -> +0.0
    return wmax, wmin, s, z


def quantize_codes(W, V, s, z, bits: int, g: int):
    """Integer codes: q = clamp(rint(W/s + V) + z, 0, Q).

    The offset V is added before rounding (blog sec. 3: v in [-0.5, 0.5]
    decides round-up vs round-down; the 3.3 example) and the zero-point after
    it (blog sec. 4: q = round(0.37/0.05) + 8, clamped to 15).
    Returns (t, q): t is the unclamped integer, q the code, both fp32 values."""
    Q = F32(2 ** bits - 1)
    Wg = _as_groups(np.asarray(W, dtype=F32), g)
    Vg = _as_groups(np.asarray(V, dtype=F32), g)
    s3 = np.asarray(s, dtype=F32)[:, :, None]
    z3 = np.asarray(z, dtype=F32)[:, :, None]
    u = ((Wg / s3).astype(F32) + Vg).astype(F32)
    t = (np.rint(u).astype(F32) + z3).astype(F32)
    q = np.minimum(np.maximum(t, F32(0.0)), Q).astype(F32)
    n, k = np.asarray(W).shape
    return t.reshape(n, k), q.reshape(n, k)


def dequantize(q, s, z, g: int):
    """w_hat = s * (q - z), fp32 (blog sec. 4 table, step 2)."""
    qg = _as_groups(np.asarray(q, dtype=F32), g)
    s3 = np.asarray(s, dtype=F32)[:, :, None]
    z3 = np.asarray(z, dtype=F32)[:, :, None]
    w = (s3 * (qg - z3).astype(F32)).astype(F32)
    n, k = np.asarray(q).shape
    return w.reshape(n, k)


def qdq(W, V, alpha, beta, bits: int, g: int, sym: bool = False):
    """Full fake-quantizer: returns dict with mx, mn, wmax, wmin, s, z, t, q, w_hat."""
    mx, mn = group_range(W, g)
    wmax, wmin, s, z = group_scale_zero(mx, mn, alpha, beta, bits, sym)
    t, q = quantize_codes(W, V, s, z, bits, g)
    w_hat = dequantize(q, s, z, g)
    return dict(mx=mx, mn=mn, wmax=wmax, wmin=wmin, s=s, z=z, t=t, q=q, w_hat=w_hat)


def rtn(W, bits: int, g: int, sym: bool = False):
    """Round-to-nearest group quantization: V = 0, alpha = beta = 1."""
    n, k = np.asarray(W).shape
    G = k // g
    return qdq(W, np.zeros((n, k), F32), np.ones((n, G), F32), np.ones((n, G), F32), bits, g, sym)


# --------------------------------------------------------------------------
# loss and straight-through gradients (blog sec. 3 algorithm flow, steps 2-4)
# --------------------------------------------------------------------------
def gather_batch(X_pool: np.ndarray, ids) -> np.ndarray:
    """Rows of the samples ``ids`` of a [S, T, K] pool, as [len(ids)*T, K]."""
    S, T, K = X_pool.shape
    return np.concatenate([X_pool[int(i)] for i in ids], axis=0).reshape(-1, K)


def _smooth_qdq(W, V, alpha, beta, bits: int, g: int, sym: bool = False):
    """fp64 fake-quantizer with both roundings replaced by the identity: the
    smooth surrogate whose exact derivative the straight-through estimator
    uses.  Only tests call it (finite-difference checks)."""
    Q = float(2 ** bits - 1)
    n, k = np.asarray(W).shape
    mx, mn = group_range(W, g)
    if sym:
        wmax = np.asarray(alpha, np.float64) * np.maximum(mx, -mn).astype(np.float64)
        wmin = -wmax
        s = wmax / float(2 ** (bits - 1) - 1)
        z = np.full(s.shape, float(2 ** (bits - 1)))
    else:
        wmax = np.asarray(alpha, np.float64) * mx.astype(np.float64)
        wmin = np.asarray(beta, np.float64) * mn.astype(np.float64)
        s = (wmax - wmin) / Q
        z = -wmin / s
    Wg = _as_groups(np.asarray(W, np.float64), g)
    Vg = _as_groups(np.asarray(V, np.float64), g)
    t = Wg / s[:, :, None] + Vg + z[:, :, None]
    q = np.clip(t, 0.0, Q)
    w_hat = s[:, :, None] * (q - z[:, :, None])
    return dict(mx=mx, mn=mn, wmax=wmax, wmin=wmin, s=s, z=z,
                t=t.reshape(n, k), q=q.reshape(n, k), w_hat=w_hat.reshape(n, k))


def loss_and_grads(W, X_b, V, alpha, beta, bits: int, g: int, mode: str = "f32",
                   smooth: bool = False, sym: bool = False):
    """Block-output MSE of the fake-quantized layer and its STE gradients.

    Forward (blog sec. 3, steps 2-4): Y_ref = X_b W^T with the original
    weight; Y = X_b W_op^T with W_op = w_hat (mode "f32") or the bf16 rounding
    of w_hat (mode "bf16", the QDQ-then-FP-GEMM of blog sec. 4);
    D = Y - Y_ref, L = sum(D^2)/(M*N).  All GEMMs in fp64.

    Backward: G = dL/dW_op = (2/(M*N)) D^T X_b.  The straight-through
    estimator treats both roundings (code and zero-point) as the identity
    (blog sec. 3 "SignSGD": rounding is a step function, its gradient is
    approximated; the Intel AutoRound article: rounding taken as identity).
    With m = [0 <= t <= Q] (clamp passes gradient on the closed range) and
    c = dw_hat/ds = (q - z) - m*W/s + (m - 1)*wmin/s:
        dV     = G * s * m
        dalpha = (mx/Q)   * sum_g G*c
        dbeta  = mn       * sum_g G*((1 - m) - c/Q)
    Symmetric (``sym``): the zero-point is a constant and s = alpha*amax/qp
    (qp = 2^(b-1) - 1), so c = (q - z) - m*W/s, dalpha = (amax/qp) sum_g G*c
    and dbeta = 0.
    ``smooth`` evaluates everything on the fp64 surrogate without rounding
    (tests only).  Returns dict(L, D, G, dV, dalpha, dbeta, qd), fp64 arrays."""
    W = np.asarray(W, dtype=F32)
    Q = 2 ** bits - 1
    n, k = W.shape
    qd = (_smooth_qdq(W, V, alpha, beta, bits, g, sym) if smooth
          else qdq(W, V, alpha, beta, bits, g, sym))
    if mode == "bf16":
        W_op = bf16_round(np.asarray(qd["w_hat"], F32)).astype(np.float64)
    elif mode == "f32":
        W_op = np.asarray(qd["w_hat"], dtype=np.float64)
    else:
        raise ValueError(mode)

    X = np.asarray(X_b, dtype=np.float64)
    M = X.shape[0]
    Y_ref = X @ W.astype(np.float64).T
    Y = X @ W_op.T
    D = Y - Y_ref
    L = float(np.sum(D * D) / (M * n))
    G = (2.0 / (M * n)) * (D.T @ X)                       # [N, K]
    dV, dalpha, dbeta = ste_grads(W, G, qd, bits, g, sym)
    return dict(L=L, D=D, G=G, dV=dV, dalpha=dalpha, dbeta=dbeta, qd=qd)


def ste_grads(W, G, qd, bits: int, g: int, sym: bool = False):
    """Straight-through gradients of (V, alpha, beta) from G = dL/dw_hat and
    the quantizer state ``qd`` (the formulas of ``loss_and_grads``)."""
    W = np.asarray(W, dtype=F32)
    Q = 2 ** bits - 1
    n, k = W.shape
    s64 = np.asarray(qd["s"], np.float64)[:, :, None]
    z64 = np.asarray(qd["z"], np.float64)[:, :, None]
    wmin64 = np.asarray(qd["wmin"], np.float64)[:, :, None]
    Wg = _as_groups(W.astype(np.float64), g)
    tg = _as_groups(np.asarray(qd["t"], np.float64), g)
    qg = _as_groups(np.asarray(qd["q"], np.float64), g)
    Gg = _as_groups(G, g)
    m = ((tg >= 0.0) & (tg <= Q)).astype(np.float64)
    dV = (Gg * s64 * m).reshape(n, k)
    if sym:
        qp = 2 ** (bits - 1) - 1
        amax = np.maximum(np.asarray(qd["mx"], np.float64), -np.asarray(qd["mn"], np.float64))
        c = (qg - z64) - m * Wg / s64
        dalpha = (amax / qp) * np.sum(Gg * c, axis=2)
        dbeta = np.zeros_like(dalpha)
    else:
        c = (qg - z64) - m * Wg / s64 + (m - 1.0) * wmin64 / s64
        dalpha = (np.asarray(qd["mx"], np.float64) / Q) * np.sum(Gg * c, axis=2)
        dbeta = np.asarray(qd["mn"], np.float64) * np.sum(Gg * ((1.0 - m) - c / Q), axis=2)
    return dV, dalpha, dbeta


# --------------------------------------------------------------------------
# SignSGD (blog sec. 3, update rule) with linear decay, clamps and snapshot
# --------------------------------------------------------------------------
def lr_table(lr: float, iters: int, decay: bool = True) -> np.ndarray:
    """lr_t = lr * (1 - t/iters) in fp64, stored fp32; constant when not decaying.

    The step size is a single-precision number (the blog's sec. 8 preset
    table gives 5e-3 without a precision; the tuner's options carry it as
    fp32), so the table starts from fp32(lr), widened exactly to fp64, and
    not from the decimal literal: with lr = 0.005 the two tables differ by an
    ulp on 62 of 200 steps."""
    lr64 = float(np.float32(lr))
    t = np.arange(iters, dtype=np.float64)
    if decay:
        return (lr64 * (1.0 - t / iters)).astype(F32)
    return np.full(iters, lr64, dtype=F32)


def signsgd_step(p, grad, lr_t, lo: float, hi: float):
    """p <- clamp(p - lr_t * sign(grad), lo, hi) in fp32; sign(0) = 0.

    The blog writes the step as lr * sign(grad) with equal-size moves; descent
    subtracts it.  Bounds: V in [-0.5, 0.5] (blog sec. 3), alpha, beta in the
    clip box."""
    p = np.asarray(p, dtype=F32)
    step = (F32(lr_t) * np.sign(grad).astype(F32)).astype(F32)
    out = (p - step).astype(F32)
    return np.minimum(np.maximum(out, F32(lo)), F32(hi)).astype(F32)


def tune_layer(W, X_pool, schedule, bits: int, g: int, iters: int, lr: float,
               decay: bool = True, mode: str = "f32", V0=None, alpha0=None, beta0=None,
               clip_lo: float = 0.5, clip_hi: float = 1.0, lr_clip: float | None = None,
               return_last: bool = False, sym: bool = False):
    """SignSGD tuning of one linear layer (blog sec. 3 algorithm flow, steps 3-6).

    For t = 0..iters-1: evaluate L_t and the STE gradients at p_t on the
    minibatch schedule[t]; if L_t < best (strict) the pre-update state p_t
    becomes the snapshot; then p_{t+1} = SignSGD(p_t).  ``lr_clip`` (default
    lr) is the step size for alpha/beta; 0 freezes them.
    Returns dict(V, alpha, beta, best_loss, best_step, losses)."""
    W = np.asarray(W, dtype=F32)
    n, k = W.shape
    G = k // g
    V = np.zeros((n, k), F32) if V0 is None else np.array(V0, dtype=F32)
    al = np.ones((n, G), F32) if alpha0 is None else np.array(alpha0, dtype=F32)
    be = np.ones((n, G), F32) if beta0 is None else np.array(beta0, dtype=F32)
    lrs = lr_table(lr, iters, decay)
    lrs_c = lrs if lr_clip is None else lr_table(lr_clip, iters, decay)
    best = np.inf
    best_step = -1
    snap = (V.copy(), al.copy(), be.copy())
    losses = np.zeros(iters, np.float64)
    for t in range(iters):
        X_b = gather_batch(X_pool, schedule[t])
        r = loss_and_grads(W, X_b, V, al, be, bits, g, mode=mode, sym=sym)
        losses[t] = r["L"]
        if r["L"] < best:
            best = r["L"]
            best_step = t
            snap = (V.copy(), al.copy(), be.copy())
        V = signsgd_step(V, r["dV"], lrs[t], -0.5, 0.5)
        al = signsgd_step(al, r["dalpha"], lrs_c[t], clip_lo, clip_hi)
        be = signsgd_step(be, r["dbeta"], lrs_c[t], clip_lo, clip_hi)
    if return_last:
        snap = (V, al, be)
    return dict(V=snap[0], alpha=snap[1], beta=snap[2], best_loss=best,
                best_step=best_step, losses=losses)


# --------------------------------------------------------------------------
# INT4 packing (coordinates page sec. 2/3: packing/layout, bytes formula)
# --------------------------------------------------------------------------
def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, row-major [N, K/2]: byte j of a row holds
    code 2j in its low nibble and code 2j+1 in its high nibble."""
    qi = np.asarray(q).astype(np.uint8)
    n, k = qi.shape
    out = np.zeros((n, k // 2), np.uint8)
    for j in range(k // 2):
        out[:, j] = (qi[:, 2 * j] & 0xF) | ((qi[:, 2 * j + 1] & 0xF) << 4)
    return out


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    n, h = p.shape
    q = np.zeros((n, 2 * h), np.uint8)
    q[:, 0::2] = p & 0xF
    q[:, 1::2] = p >> 4
    return q


def packed_bytes(n: int, k: int, g: int, bits: int = 4) -> int:
    """Bytes of the packed layer: P*b/8 for the codes plus fp32 scale and
    uint8 zero-point per group (coordinates page sec. 3 bytes estimate; this
    layout needs no padding when K is even)."""
    return n * k * bits // 8 + 4 * n * (k // g) + n * (k // g)


def w4a16_matmul(X, packed, scale, zero, g: int) -> np.ndarray:
    """Y = X * W_op^T for the packed INT4 layer, in fp64.

    W_op is the bf16 rounding of the dequantized weight s * (q - z) (fp32,
    the quantizer's own w_hat), i.e. the operand the fake-quantized bf16 GEMM
    uses; a real INT4 kernel consumes the packed codes, scale and zero
    instead of that weight (AutoRound blog sec. 4, QDQ versus real INT4;
    coordinates page sec. 2-3, packed weight with per-group scale and
    zero-point)."""
    q = unpack_int4(packed).astype(F32)
    w_op = bf16_round(dequantize(q, np.asarray(scale, F32), np.asarray(zero, F32), g))
    return np.asarray(X, np.float64) @ w_op.astype(np.float64).T
