"""Decoder-block oracle pinned to library routines (torch's scaled dot-product
attention with causal masking, rms_norm, a complex-number form of the rotary
embedding), to finite differences of the smooth surrogate and torch autograd
for the straight-through gradients of all seven linears, and to the MLP-block
oracle when the attention output is exactly zero."""
import numpy as np
import pytest
import torch

import oracle
from oracle import decoder_ref as dr

F32 = np.float32


def _cfg(H, nq, nkv, d, F, T):
    return dict(H=H, nq=nq, nkv=nkv, d=d, F=F, T=T, eps=1e-5, theta=10000.0, w1=np.ones(H), w2=np.ones(H))


def _weights(cfg, seed, scale=0.3):
    rng = np.random.default_rng(seed)
    H, nq, nkv, d, F = cfg["H"], cfg["nq"], cfg["nkv"], cfg["d"], cfg["F"]
    shapes = {"q": (nq * d, H), "k": (nkv * d, H), "v": (nkv * d, H), "o": (H, nq * d), "gate": (F, H),
              "up": (F, H), "down": (H, F)}
    return {nm: (rng.standard_normal(sh) * scale).astype(F32) for nm, sh in shapes.items()}


def _params(Ws, g, seed, clip=(0.6, 0.95)):
    rng = np.random.default_rng(seed)
    out = {}
    for nm, W in Ws.items():
        n, k = W.shape
        out[nm] = (rng.uniform(-0.5, 0.5, (n, k)).astype(F32), rng.uniform(*clip, (n, k // g)).astype(F32),
                   rng.uniform(*clip, (n, k // g)).astype(F32))
    return out


def test_rope_is_the_complex_rotation_and_its_inverse_the_transpose():
    T, d, nh = 7, 8, 3
    cos, sin = dr.rope_tables(T, d, 10000.0)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((T, nh * d))
    y = dr.rope(x, cos, sin, nh, d)
    xh = x.reshape(T, nh, d)
    z = xh[..., : d // 2] + 1j * xh[..., d // 2:]
    ang = np.arange(T)[:, None, None] * 10000.0 ** (-2.0 * np.arange(d // 2) / d)[None, None, :]
    zr = z * np.exp(1j * ang)
    np.testing.assert_allclose(y.reshape(T, nh, d), np.concatenate([zr.real, zr.imag], axis=2), atol=1e-12)
    np.testing.assert_allclose(dr.rope(y, cos, sin, nh, d, inverse=True), x, atol=1e-12)


def test_attention_and_norm_match_torch():
    T, nq, nkv, d, nb = 6, 4, 2, 8, 2
    rng = np.random.default_rng(1)
    q = rng.standard_normal((nb * T, nq * d))
    k = rng.standard_normal((nb * T, nkv * d))
    v = rng.standard_normal((nb * T, nkv * d))
    o, _ = dr._attention(q, k, v, T, nq, nkv, d, lambda x: x)
    t = lambda a, n: torch.tensor(a).reshape(nb, T, n, d).transpose(1, 2)
    kk = t(k, nkv).repeat_interleave(nq // nkv, dim=1)
    vv = t(v, nkv).repeat_interleave(nq // nkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q, nq), kk, vv, is_causal=True)
    np.testing.assert_allclose(o, ref.transpose(1, 2).reshape(nb * T, nq * d).numpy(), atol=1e-12)
    z = rng.standard_normal((5, 16))
    w = rng.uniform(0.5, 1.5, 16)
    got, _ = dr.rms_norm(z, w, 1e-5)
    ref = torch.nn.functional.rms_norm(torch.tensor(z), (16,), torch.tensor(w), eps=1e-5)
    np.testing.assert_allclose(got, ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("nkv", [2, 1])
def test_decoder_smooth_gradients_match_finite_differences(nkv):
    cfg = _cfg(H=8, nq=2, nkv=nkv, d=4, F=12, T=4)
    g = 4
    Ws = _weights(cfg, 2)
    rng = np.random.default_rng(3)
    X = rng.standard_normal((8, 8))
    Y_ref = dr.decoder_forward(X, Ws, cfg)["y"]
    p = _params(Ws, g, 4)
    Vs = {nm: p[nm][0] for nm in dr.LINEARS}
    als = {nm: p[nm][1] for nm in dr.LINEARS}
    bes = {nm: p[nm][2] for nm in dr.LINEARS}
    res = dr.decoder_loss_and_grads(X, Y_ref, Ws, Vs, als, bes, 4, g, cfg, smooth=True)

    def loss(V_, a_, b_):
        return dr.decoder_loss_and_grads(X, Y_ref, Ws, V_, a_, b_, 4, g, cfg, smooth=True)["L"]

    eps = 1e-6
    for nm in dr.LINEARS:
        for which, arr, grad in (("V", Vs, res["grads"][nm][0]), ("alpha", als, res["grads"][nm][1]),
                                 ("beta", bes, res["grads"][nm][2])):
            fd = np.zeros_like(grad)
            for idx in np.ndindex(arr[nm].shape):
                hi = {k: v.astype(np.float64).copy() for k, v in arr.items()}
                lo = {k: v.astype(np.float64).copy() for k, v in arr.items()}
                hi[nm][idx] += eps
                lo[nm][idx] -= eps
                a_hi = [hi if a is arr else a for a in (Vs, als, bes)]
                a_lo = [lo if a is arr else a for a in (Vs, als, bes)]
                fd[idx] = (loss(*a_hi) - loss(*a_lo)) / (2 * eps)
            scale = np.max(np.abs(fd)) + 1e-30
            assert np.max(np.abs(fd - grad)) / scale < 1e-5, (nm, which)


def test_decoder_ste_gradients_match_torch_autograd():
    cfg = _cfg(H=16, nq=4, nkv=2, d=4, F=24, T=5)
    g, bits = 8, 4
    Ws = _weights(cfg, 5)
    rng = np.random.default_rng(6)
    X = rng.standard_normal((10, 16))
    Y_ref = dr.decoder_forward(X, Ws, cfg)["y"]
    p = _params(Ws, g, 7)
    res = dr.decoder_loss_and_grads(X, Y_ref, Ws, {n: p[n][0] for n in dr.LINEARS},
                                    {n: p[n][1] for n in dr.LINEARS}, {n: p[n][2] for n in dr.LINEARS},
                                    bits, g, cfg)
    Q = 2 ** bits - 1
    tv = {}

    def fq(nm):
        W = torch.tensor(Ws[nm], dtype=torch.float64)
        n, k = W.shape
        Wg = W.reshape(n, k // g, g)
        mx = Wg.max(dim=2).values.clamp(min=0)
        mn = Wg.min(dim=2).values.clamp(max=0)
        V, al, be = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in p[nm])
        tv[nm] = (V, al, be)
        s = (al * mx - be * mn) / Q
        z0 = -be * mn / s
        z = z0 + (torch.round(z0) - z0).detach()
        u = Wg / s[:, :, None] + V.reshape(n, k // g, g)
        t = u + (torch.round(u) - u).detach() + z[:, :, None]
        q = torch.clamp(t, 0.0, float(Q))
        return (s[:, :, None] * (q - z[:, :, None])).reshape(n, k)

    w = {nm: fq(nm) for nm in dr.LINEARS}
    H, nq, nkv, d, T = 16, 4, 2, 4, 5
    Xt = torch.tensor(X)
    nrm = lambda z: z / torch.sqrt((z * z).mean(dim=1, keepdim=True) + 1e-5)
    h1 = nrm(Xt)
    cos, sin = (torch.tensor(np.tile(a, (2, 1))) for a in dr.rope_tables(T, d, 1e4))

    def rot(x, nh):
        xh = x.reshape(-1, nh, d)
        a, b = xh[..., : d // 2], xh[..., d // 2:]
        c, s = cos[:, None, :], sin[:, None, :]
        return torch.cat([a * c - b * s, b * c + a * s], dim=2).reshape(-1, nh * d)

    q = rot(h1 @ w["q"].T, nq).reshape(2, T, nq, d).transpose(1, 2)
    k = rot(h1 @ w["k"].T, nkv).reshape(2, T, nkv, d).transpose(1, 2).repeat_interleave(2, dim=1)
    v = (h1 @ w["v"].T).reshape(2, T, nkv, d).transpose(1, 2).repeat_interleave(2, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    h = Xt + o.transpose(1, 2).reshape(10, nq * d) @ w["o"].T
    h2 = nrm(h)
    y = h + (torch.nn.functional.silu(h2 @ w["gate"].T) * (h2 @ w["up"].T)) @ w["down"].T
    L = ((y - torch.tensor(Y_ref)) ** 2).sum() / y.numel()
    L.backward()
    assert res["L"] == pytest.approx(L.item(), rel=1e-6)
    for nm in dr.LINEARS:
        for got, ref in zip(res["grads"][nm], tv[nm]):
            rr = ref.grad.numpy()
            np.testing.assert_allclose(got, rr, rtol=1e-4, atol=1e-6 * (np.abs(rr).max() + 1e-30))


def test_mlp_part_reduces_to_the_mlp_block_when_attention_output_is_zero():
    cfg = _cfg(H=16, nq=2, nkv=2, d=8, F=32, T=4)
    g = 8
    Ws = _weights(cfg, 8)
    Ws["o"] = np.zeros_like(Ws["o"])           # an all-zero group quantizes to exactly zero
    rng = np.random.default_rng(9)
    X = rng.standard_normal((8, 16))
    Y_ref = dr.decoder_forward(X, Ws, cfg)["y"]
    p = _params(Ws, g, 10)
    dec = dr.decoder_loss_and_grads(X, Y_ref, Ws, {n: p[n][0] for n in dr.LINEARS},
                                    {n: p[n][1] for n in dr.LINEARS}, {n: p[n][2] for n in dr.LINEARS}, 4, g, cfg)
    h2, _ = dr.rms_norm(X, cfg["w2"], cfg["eps"])
    mlp_W = {nm: Ws[nm] for nm in ("gate", "up", "down")}
    Yb, *_ = oracle.swiglu_forward(h2, Ws["gate"], Ws["up"], Ws["down"])
    blk = oracle.block_loss_and_grads(h2, Yb, mlp_W, {n: p[n][0] for n in mlp_W}, {n: p[n][1] for n in mlp_W},
                                      {n: p[n][2] for n in mlp_W}, 4, g)
    assert dec["L"] == pytest.approx(blk["L"], rel=1e-12)
    for nm in ("gate", "up", "down"):
        for a, b in zip(dec["grads"][nm], blk["grads"][nm]):
            np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-14)


def test_row_sampled_straight_through_step_equals_rows_of_the_full_one():
    # ste_rows restricts the straight-through step to sampled weight rows
    # (used for blocks too large to evaluate whole): each row equals the
    # corresponding row of the full evaluation, bit for bit
    cfg = _cfg(H=16, nq=4, nkv=2, d=4, F=24, T=5)
    g, bits = 8, 4
    Ws = _weights(cfg, 8)
    X = np.random.default_rng(9).standard_normal((10, 16))
    Y_ref = dr.decoder_forward(X, Ws, cfg, "bf16")["y"]
    p = _params(Ws, g, 10)
    args = (X, Y_ref, Ws, {n: p[n][0] for n in dr.LINEARS}, {n: p[n][1] for n in dr.LINEARS},
            {n: p[n][2] for n in dr.LINEARS}, bits, g, cfg)
    full = dr.decoder_loss_and_grads(*args, mode="bf16")
    rows = {nm: np.array([0, Ws[nm].shape[0] - 1, 3]) for nm in dr.LINEARS}
    part = dr.decoder_loss_and_grads(*args, mode="bf16", ste_rows=rows)
    assert part["L"] == full["L"]
    for nm in dr.LINEARS:
        np.testing.assert_array_equal(part["G"][nm], full["G"][nm])
        for a, b in zip(part["grads"][nm], full["grads"][nm]):
            np.testing.assert_array_equal(a, b[rows[nm]])
