"""Oracle of the tensor-level QDQ for low-bit float formats -- test
infrastructure.

The AutoRound blog (sec. 4, "data-type decoupling") notes that a new data
type such as FP8 or MXFP4 is supported by registering a tensor-level QDQ
function, which lets its effect on accuracy be evaluated before any kernel
for it exists.  Two formats are modelled, each by its table of values:

* FP8 E4M3 (1 sign, 4 exponent, 3 mantissa bits; exponent bias 7; no
  infinities, the all-ones exponent with all-ones mantissa is NaN, so the
  largest finite magnitude is 448; subnormals 2^-9 * m).  Per-group scale
  s = alpha * max|W_g| / 448 (1 for an all-zero group); codes are E4M3
  values of W/s, ŵ = s * code.
* MXFP4: E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in blocks of
  32 along K sharing a power-of-two scale 2^e with e = floor(log2(alpha *
  max|W_b|)) - 2 (2 = the largest E2M1 exponent), i.e. the block maximum
  maps into [4, 8); the scale is stored as its biased 8-bit exponent e + 127.

Rounding is to the nearest representable value, ties to the value whose code
is even; magnitudes above the largest finite value saturate to it.  Written
from the value tables (no bit tricks), so it shares nothing with the GPU
path's grid-spacing arithmetic.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def e4m3_table():
    """(codes, values) of the non-negative finite E4M3 values, by code."""
    codes, vals = [], []
    for c in range(0x80):
        e, m = c >> 3, c & 7
        if e == 15 and m == 7:
            continue                      # NaN
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(v)
    return np.array(codes), np.array(vals)


def e2m1_table():
    """(codes, values) of the non-negative E2M1 values, by code."""
    codes, vals = [], []
    for c in range(8):
        e, m = c >> 1, c & 1
        v = (m / 2.0) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        codes.append(c)
        vals.append(v)
    return np.array(codes), np.array(vals)


def _round_table(x, table):
    """Nearest table value to |x| (ties: even code), saturating; sign kept.
    Returns (value fp64, code with the sign in the bit above the magnitude)."""
    codes, vals = table
    x = np.asarray(x, np.float64)
    mag = np.minimum(np.abs(x), vals.max())
    d = np.abs(mag[..., None] - vals)
    best = d.min(axis=-1, keepdims=True)
    cand = (d == best)
    # among the tied candidates prefer the even code
    even = cand & (codes % 2 == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, cand)
    idx = np.argmax(pick, axis=-1)
    v = vals[idx]
    sign = np.signbit(x) & (v != 0)
    return np.where(sign, -v, v), codes[idx], sign


def e4m3_round(x):
    v, c, s = _round_table(x, e4m3_table())
    return v, (c | (s.astype(np.int64) << 7)).astype(np.uint8)


def e2m1_round(x):
    v, c, s = _round_table(x, e2m1_table())
    return v, (c | (s.astype(np.int64) << 3)).astype(np.uint8)


def qdq_fp8_e4m3(W, g: int, alpha=None):
    """Per-group FP8 E4M3 fake quantization: dict(s, codes, w_hat), fp32."""
    W = np.asarray(W, F32)
    n, k = W.shape
    G = k // g
    al = np.ones((n, G), F32) if alpha is None else np.asarray(alpha, F32)
    Wg = W.reshape(n, G, g)
    amax = np.abs(Wg).max(axis=2).astype(F32)
    wmax = (al * amax).astype(F32)
    s = np.where(wmax == 0, F32(1.0), (wmax / F32(448.0)).astype(F32)).astype(F32)
    x = (Wg / s[:, :, None]).astype(F32)
    v, codes = e4m3_round(x)
    w_hat = (s[:, :, None] * v.astype(F32)).astype(F32)
    return dict(s=s, codes=codes.reshape(n, k), w_hat=w_hat.reshape(n, k))


def qdq_mxfp4(W, alpha=None, block: int = 32):
    """MXFP4 fake quantization (E2M1 elements, shared power-of-two scale per
    block of 32 along K): dict(s, scale_bits, codes, w_hat), fp32."""
    W = np.asarray(W, F32)
    n, k = W.shape
    G = k // block
    al = np.ones((n, G), F32) if alpha is None else np.asarray(alpha, F32)
    Wb = W.reshape(n, G, block)
    amax = (al * np.abs(Wb).max(axis=2).astype(F32)).astype(F32)
    e = np.zeros((n, G), np.int64)
    nz = amax > 0
    e[nz] = np.floor(np.log2(amax[nz].astype(np.float64))).astype(np.int64) - 2
    s = np.where(nz, np.ldexp(1.0, e), 1.0).astype(F32)
    x = (Wb / s[:, :, None]).astype(F32)
    v, codes = e2m1_round(x)
    w_hat = (s[:, :, None] * v.astype(F32)).astype(F32)
    scale_bits = np.where(nz, e + 127, 127).astype(np.uint8)
    return dict(s=s, scale_bits=scale_bits, codes=codes.reshape(n, k), w_hat=w_hat.reshape(n, k))
