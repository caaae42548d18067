"""Oracle QDQ pinned to invariants, closed forms and a library routine.

* error bounds of the AutoRound blog's error taxonomy (sec. 2 figure panels
  2 and 3): inside the clipped range RTN error is at most half a step; outside
  it the error is the clipping error;
* zero maps to zero; grid-exact weights are reproduced bit for bit;
* the reachable codes of a rounding offset v in [-0.5, 0.5] (blog sec. 3)
  are the floor/ceil neighbours of RTN;
* RTN at alpha = beta = 1 agrees with torch's per-channel affine fake
  quantizer (a library routine) away from rounding ties.
"""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle

F32 = np.float32


def _weights(n, k, seed, outliers=True):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    if outliers:
        idx = rng.choice(n * k, size=max(1, n * k // 200), replace=False)
        W.reshape(-1)[idx] *= F32(20)
    return W


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2 ** 31 - 1), bits=st.integers(2, 8),
       g=st.sampled_from([4, 8, 32]), clip=st.floats(0.5, 1.0))
def test_error_bounds(seed, bits, g, clip):
    n, k = 6, 64
    W = _weights(n, k, seed)
    G = k // g
    al = np.full((n, G), clip, F32)
    be = np.full((n, G), clip, F32)
    r = oracle.qdq(W, np.zeros_like(W), al, be, bits, g)
    s = np.repeat(r["s"], g, axis=1)
    wmax = np.repeat(r["wmax"], g, axis=1)
    wmin = np.repeat(r["wmin"], g, axis=1)
    err = W.astype(np.float64) - r["w_hat"].astype(np.float64)
    slack = 4e-6 * (np.abs(W) + s)                 # a few fp32 ulps
    inside = (W >= wmin) & (W <= wmax)
    # rounding error (panel 2): half a grid step, plus the shift of the grid
    # that rounding the zero-point causes (|z*s + wmin| <= s/2)
    off = np.repeat(np.abs(r["z"].astype(np.float64) * r["s"] + r["wmin"]), g, axis=1)
    assert np.all(off <= r["s"].max() / 2 + 1e-6)
    assert np.all(np.abs(err[inside]) <= s[inside] / 2 + off[inside] + slack[inside])
    # above the range: error is the clipping error w - (top of grid)
    above = W > wmax
    top = np.repeat(r["s"] * (F32(2 ** bits - 1) - r["z"]), g, axis=1)
    np.testing.assert_allclose(err[above], (W - top)[above], rtol=0, atol=1e-6)
    below = W < wmin
    bot = np.repeat(r["s"] * (0 - r["z"]), g, axis=1)
    np.testing.assert_allclose(err[below], (W - bot)[below], rtol=0, atol=1e-6)
    # codes and zero-points are valid integers
    assert np.all(r["q"] == np.round(r["q"])) and r["q"].min() >= 0 and r["q"].max() <= 2 ** bits - 1
    assert np.all(r["z"] >= 0) and np.all(r["z"] <= 2 ** bits - 1)


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2 ** 31 - 1), bits=st.integers(2, 8), g=st.sampled_from([4, 16, 64]))
def test_rtn_error_half_step_when_zero_on_grid(seed, bits, g):
    # At alpha = beta = 1 the zero-inclusive range puts 0 on the grid when
    # -mn/s is an integer; in general the grid is offset by < s/2 and the
    # in-range RTN error is at most s/2 + |z*s - (-mn)|.
    W = _weights(4, 64, seed)
    r = oracle.rtn(W, bits, g)
    s = np.repeat(r["s"], g, axis=1).astype(np.float64)
    off = np.repeat(np.abs(r["z"].astype(np.float64) * r["s"] + r["mn"]), g, axis=1)
    err = np.abs(W.astype(np.float64) - r["w_hat"])
    assert np.all(err <= s / 2 + off + 4e-6 * (np.abs(W) + s))


def test_zero_maps_to_zero_and_sign_of_zero():
    W = _weights(8, 64, 3)
    W[:, ::7] = 0.0
    r = oracle.rtn(W, 4, 32)
    assert np.all(r["w_hat"][W == 0] == 0)
    assert not np.any(np.signbit(r["w_hat"][W == 0]))
    # an all-zero group: scale 1, zero 0, codes 0
    W2 = np.zeros((2, 32), F32)
    r2 = oracle.rtn(W2, 4, 32)
    assert np.all(r2["s"] == 1) and np.all(r2["z"] == 0) and np.all(r2["q"] == 0)


def test_grid_exact_identity():
    # W = 2^-7 (k - 8), k in 0..15, both ends present in every group:
    # s = 1/128, z = 8 exactly and QDQ is the identity bit for bit.
    rng = np.random.default_rng(0)
    ks = rng.integers(0, 16, size=(8, 128))
    ks[:, 0] = 0
    ks[:, 127] = 15
    ks[:, 64] = 0
    ks[:, 63] = 15
    W = (np.ldexp(1.0, -7) * (ks - 8)).astype(F32)
    r = oracle.rtn(W, 4, 64)
    assert np.all(r["s"] == F32(2.0 ** -7)) and np.all(r["z"] == 8)
    np.testing.assert_array_equal(r["w_hat"], W)
    np.testing.assert_array_equal(r["q"], ks)


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2 ** 31 - 1), vscale=st.floats(0.0, 0.5))
def test_offset_moves_code_at_most_one(seed, vscale):
    W = _weights(4, 64, seed)
    rng = np.random.default_rng(seed + 1)
    V = (rng.uniform(-1, 1, W.shape) * vscale).astype(F32)
    al = np.full((4, 2), 0.8, F32)
    be = np.full((4, 2), 0.9, F32)
    q0 = oracle.qdq(W, np.zeros_like(W), al, be, 4, 32)["q"]
    q1 = oracle.qdq(W, V, al, be, 4, 32)["q"]
    assert np.max(np.abs(q1 - q0)) <= 1
    # positive offsets never round down, negative never up
    assert np.all(q1[V > 0] >= q0[V > 0]) and np.all(q1[V < 0] <= q0[V < 0])


def test_rtn_matches_torch_per_channel_fake_quant_away_from_ties():
    # Per-group RTN == torch's per-channel affine fake quantizer applied to
    # each group as a channel (quant range [0, Q], integer zero-point).
    # torch multiplies by 1/scale and adds the zero-point before rounding,
    # so elements within 1e-4 of a rounding tie may differ by one code.
    n, k, g, bits = 64, 256, 32, 4
    W = _weights(n, k, 11)
    r = oracle.rtn(W, bits, g)
    Wt = torch.from_numpy(W).reshape(n * k // g, g)
    scale = torch.from_numpy(r["s"].reshape(-1).astype(np.float32))
    zp = torch.from_numpy(r["z"].reshape(-1).astype(np.int32))
    ref = torch.fake_quantize_per_channel_affine(Wt, scale, zp, 0, 0, 2 ** bits - 1)
    ref = ref.reshape(n, k).numpy()
    u = W / np.repeat(r["s"], g, axis=1)
    near_tie = np.abs(np.abs(u - np.floor(u)) - 0.5) < 1e-4
    ok = ~near_tie
    assert ok.mean() > 0.99
    np.testing.assert_allclose(r["w_hat"][ok], ref[ok], rtol=0, atol=1e-7)


def test_per_channel_is_group_equal_k():
    W = _weights(16, 64, 5)
    a = oracle.rtn(W, 4, 64)
    b = oracle.rtn(W, 4, 32)
    assert a["s"].shape == (16, 1) and b["s"].shape == (16, 2)
    # the per-channel scale covers both half-row scales
    assert np.all(a["s"][:, 0] >= b["s"].max(axis=1) - 1e-9)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(F32)
    # include exact ties
    x[:100] = (np.arange(100, dtype=np.uint32) << 16 | 0x8000).view(F32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), ref)
