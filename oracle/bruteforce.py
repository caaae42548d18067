"""Exhaustive search over rounding choices -- TEST INFRASTRUCTURE.

The AutoRound blog (sec. 2, trade-off discussion) notes that the space of
per-element round-up / round-down decisions grows as 2^N, which is why RTN
cannot search it and AutoRound tunes a continuous offset instead.  For tiny
layers the space can be enumerated, giving the exact optimum that any tuned
offset is bounded below by.  Written independently of autoround_ref (plain
loops; the loss is the quadratic form of the weight error with X^T X).
"""
from __future__ import annotations

import itertools

import numpy as np


def _f32(x):
    return np.float32(x)


def bruteforce_min_loss(W, X, bits: int, g: int):
    """Minimum over every reachable code assignment of the layer MSE.

    Clip factors stay at 1 (the range is the zero-inclusive group min/max).
    An element's reachable codes are the integers rint(fl(W/s) + v) + z for
    v in [-0.5, 0.5], i.e. every integer between the roundings at v = -0.5
    and v = +0.5, clamped to [0, Q].  Rows are independent at fixed scales,
    so each row is searched separately.  Returns (min_loss, rtn_loss), fp64,
    both as mean over the M x N outputs."""
    W = np.asarray(W, dtype=np.float32)
    X = np.asarray(X, dtype=np.float64)
    n, k = W.shape
    M = X.shape[0]
    Q = 2 ** bits - 1
    H = X.T @ X                                   # [K, K]
    total_min = 0.0
    total_rtn = 0.0
    for r in range(n):
        choices = []
        w_rtn = []
        for j0 in range(0, k, g):
            grp = [float(v) for v in W[r, j0:j0 + g]]
            hi = _f32(max(0.0, max(grp)))
            lo = _f32(min(0.0, min(grp)))
            d = _f32(hi - lo)
            s = _f32(1.0) if d == 0 else _f32(d / _f32(Q))
            z = float(np.rint(_f32(-lo / s)))
            for j in range(j0, j0 + g):
                u = _f32(W[r, j] / s)
                a = int(np.rint(_f32(u - _f32(0.5))))
                b = int(np.rint(_f32(u + _f32(0.5))))
                opts = sorted({min(max(c + z, 0.0), float(Q)) for c in range(a, b + 1)})
                choices.append([float(_f32(s * _f32(c - z))) for c in opts])
                c0 = min(max(float(np.rint(u)) + z, 0.0), float(Q))
                w_rtn.append(float(_f32(s * _f32(c0 - z))))
        w_row = W[r].astype(np.float64)
        best = np.inf
        for combo in itertools.product(*choices):
            e = np.asarray(combo, np.float64) - w_row
            val = float(e @ H @ e)
            if val < best:
                best = val
        e0 = np.asarray(w_rtn, np.float64) - w_row
        total_min += best
        total_rtn += float(e0 @ H @ e0)
    return total_min / (M * n), total_rtn / (M * n)


def _reachable(W, bits: int, g: int):
    """Per element of W: the dequantized values reachable with v in
    [-0.5, 0.5] at clip factors 1, and the RTN value (plain loops)."""
    W = np.asarray(W, dtype=np.float32)
    n, k = W.shape
    Q = 2 ** bits - 1
    choices, rtn = [], []
    for r in range(n):
        for j0 in range(0, k, g):
            grp = [float(v) for v in W[r, j0:j0 + g]]
            hi = _f32(max(0.0, max(grp)))
            lo = _f32(min(0.0, min(grp)))
            d = _f32(hi - lo)
            s = _f32(1.0) if d == 0 else _f32(d / _f32(Q))
            z = float(np.rint(_f32(-lo / s)))
            for j in range(j0, j0 + g):
                u = _f32(W[r, j] / s)
                a = int(np.rint(_f32(u - _f32(0.5))))
                b = int(np.rint(_f32(u + _f32(0.5))))
                opts = sorted({min(max(c + z, 0.0), float(Q)) for c in range(a, b + 1)})
                choices.append([float(_f32(s * _f32(c - z))) for c in opts])
                c0 = min(max(float(np.rint(u)) + z, 0.0), float(Q))
                rtn.append(float(_f32(s * _f32(c0 - z))))
    return choices, rtn


def bruteforce_block_min_loss(X, Wg, Wu, Wd, bits: int, g: int):
    """Minimum block MSE over every reachable joint code assignment of the
    three linears of a gated MLP (Y = (silu(X Wg^T) * X Wu^T) Wd^T), and the
    RTN loss.  The block loss couples all weights, so the search is joint;
    only for tiny blocks.  fp64, mean over the M x H outputs."""
    X = np.asarray(X, dtype=np.float64)
    shapes = [np.asarray(w).shape for w in (Wg, Wu, Wd)]
    parts = [_reachable(w, bits, g) for w in (Wg, Wu, Wd)]
    sizes = [a * b for a, b in shapes]

    def block_out(flat):
        ws, o = [], 0
        for (a, b), sz in zip(shapes, sizes):
            ws.append(np.asarray(flat[o:o + sz], np.float64).reshape(a, b))
            o += sz
        A = X @ ws[0].T
        B = X @ ws[1].T
        return (A / (1.0 + np.exp(-A)) * B) @ ws[2].T

    flat_orig = np.concatenate([np.asarray(w, np.float32).astype(np.float64).ravel() for w in (Wg, Wu, Wd)])
    Y_ref = block_out(flat_orig)
    denom = Y_ref.size
    all_choices = parts[0][0] + parts[1][0] + parts[2][0]
    best = np.inf
    for combo in itertools.product(*all_choices):
        D = block_out(combo) - Y_ref
        val = float(np.sum(D * D)) / denom
        if val < best:
            best = val
    D0 = block_out(parts[0][1] + parts[1][1] + parts[2][1]) - Y_ref
    return best, float(np.sum(D0 * D0)) / denom
