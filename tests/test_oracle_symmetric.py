"""Oracle symmetric variant pinned to the coordinates page's symmetric
mapping (sec. 1.2: q = clip(round(x/s), qmin, qmax), x^ = s q), to torch's
per-channel fake quantizer, to error bounds, and to finite differences and
torch autograd for its straight-through gradients."""
import numpy as np
import pytest
import torch

import oracle

F32 = np.float32


def _w(n, k, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    W.reshape(-1)[rng.choice(n * k, max(1, n * k // 200), replace=False)] *= F32(20)
    return W


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_symmetric_rtn_matches_torch_per_channel_signed(bits):
    n, k, g = 32, 256, 64
    W = _w(n, k, bits)
    r = oracle.rtn(W, bits, g, sym=True)
    assert np.all(r["z"] == 2 ** (bits - 1))
    Wt = torch.from_numpy(W).reshape(n * k // g, g)
    scale = torch.from_numpy(r["s"].reshape(-1).astype(np.float32))
    zp = torch.zeros(n * k // g, dtype=torch.int32)
    ref = torch.fake_quantize_per_channel_affine(Wt, scale, zp, 0, -2 ** (bits - 1), 2 ** (bits - 1) - 1)
    ref = ref.reshape(n, k).numpy()
    u = W / np.repeat(r["s"], g, axis=1)
    ok = np.abs(np.abs(u - np.floor(u)) - 0.5) >= 1e-4
    assert ok.mean() > 0.99
    np.testing.assert_allclose(r["w_hat"][ok], ref[ok], rtol=0, atol=1e-7)


def test_symmetric_scale_error_bounds_and_zero():
    n, k, g, bits = 16, 128, 32, 4
    W = _w(n, k, 5)
    W[:, ::9] = 0.0
    rng = np.random.default_rng(0)
    al = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    r = oracle.qdq(W, np.zeros_like(W), al, np.ones_like(al), bits, g, sym=True)
    amax = np.maximum(r["mx"], -r["mn"])
    np.testing.assert_array_equal(r["s"], (al * amax / F32(7)).astype(F32))
    assert np.all(r["w_hat"][W == 0] == 0)
    qz = r["q"] - np.repeat(r["z"], g, axis=1)
    assert qz.min() >= -8 and qz.max() <= 7
    s = np.repeat(r["s"], g, axis=1)
    wmax = np.repeat(r["wmax"], g, axis=1)
    inside = np.abs(W) <= wmax
    err = np.abs(W.astype(np.float64) - r["w_hat"])
    assert np.all(err[inside] <= s[inside] / 2 + 4e-6 * (np.abs(W[inside]) + s[inside]))
    above = W > wmax
    np.testing.assert_allclose(r["w_hat"][above], (7 * s)[above], rtol=1e-6)


def test_symmetric_smooth_gradients_match_finite_differences():
    n, k, m, g, bits = 3, 16, 12, 8, 4
    rng = np.random.default_rng(3)
    W = _w(n, k, 3)
    X = rng.standard_normal((m, k))
    V = rng.uniform(-0.5, 0.5, (n, k))
    al = rng.uniform(0.5, 0.9, (n, k // g))
    be = np.ones_like(al)
    r = oracle.loss_and_grads(W, X, V, al, be, bits, g, smooth=True, sym=True)
    assert np.all(r["dbeta"] == 0)
    h = 1e-6
    for name, arr, grad in [("V", V, r["dV"]), ("alpha", al, r["dalpha"])]:
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += h
            q = arr.copy(); q[idx] -= h
            if name == "V":
                lp = oracle.loss_and_grads(W, X, p, al, be, bits, g, smooth=True, sym=True)["L"]
                lm = oracle.loss_and_grads(W, X, q, al, be, bits, g, smooth=True, sym=True)["L"]
            else:
                lp = oracle.loss_and_grads(W, X, V, p, be, bits, g, smooth=True, sym=True)["L"]
                lm = oracle.loss_and_grads(W, X, V, q, be, bits, g, smooth=True, sym=True)["L"]
            fd[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(fd - grad)) / (np.max(np.abs(fd)) + 1e-30) < 1e-5, name


def test_symmetric_ste_gradients_match_torch_autograd():
    n, k, m, g, bits = 4, 32, 20, 16, 4
    rng = np.random.default_rng(9)
    W = _w(n, k, 9)
    X = rng.standard_normal((m, k))
    V = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
    al = rng.uniform(0.6, 1.0, (n, k // g)).astype(F32)
    r = oracle.loss_and_grads(W, X, V, al, np.ones_like(al), bits, g, sym=True)

    Wt = torch.tensor(W, dtype=torch.float64)
    Wg = Wt.reshape(n, k // g, g)
    amax = torch.maximum(Wg.max(dim=2).values.clamp(min=0), -Wg.min(dim=2).values.clamp(max=0))
    Vt = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    at = torch.tensor(al, dtype=torch.float64, requires_grad=True)
    s = at * amax / (2 ** (bits - 1) - 1)
    u = Wg / s[:, :, None] + Vt.reshape(n, k // g, g)
    q = torch.clamp(u + (torch.round(u) - u).detach(), -2.0 ** (bits - 1), 2.0 ** (bits - 1) - 1)
    w_hat = (s[:, :, None] * q).reshape(n, k)
    Xt = torch.tensor(X, dtype=torch.float64)
    D = Xt @ w_hat.T - Xt @ Wt.T
    L = (D * D).sum() / (m * n)
    L.backward()
    assert r["L"] == pytest.approx(L.item(), rel=1e-5)
    np.testing.assert_allclose(r["dV"], Vt.grad.numpy(), rtol=1e-4, atol=1e-9 * np.abs(Vt.grad.numpy()).max())
    np.testing.assert_allclose(r["dalpha"], at.grad.numpy(), rtol=1e-4, atol=1e-6 * np.abs(at.grad.numpy()).max())
