"""Oracle loss and STE gradients pinned to finite differences, to torch
autograd, and to closed forms.

The gradient formula in the oracle is the chain rule through the fake
quantizer with the roundings taken as the identity (the AutoRound blog,
sec. 3 "SignSGD": straight-through estimator).  Two independent checks:
(i) on the smooth surrogate (no rounding at all, fp64) the formula must equal
central finite differences of the loss; (ii) with real rounding it must equal
torch CPU autograd of the same forward written with the detach trick.
"""
import numpy as np
import pytest
import torch

import oracle

F32 = np.float32


def _layer(n, k, m, g, seed, clip=0.8):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    W.reshape(-1)[rng.choice(n * k, 3, replace=False)] *= 20
    X = rng.standard_normal((m, k))
    X[:, 1] *= 50
    V = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
    G = k // g
    al = rng.uniform(0.5, 1.0, (n, G)).astype(F32) * clip / 0.8
    be = rng.uniform(0.5, 1.0, (n, G)).astype(F32) * clip / 0.8
    return W, X, V, al.astype(F32), be.astype(F32)


def _smooth_loss(W, X, V, al, be, bits, g):
    return oracle.loss_and_grads(W, X, V, al, be, bits, g, mode="f32", smooth=True)["L"]


def test_smooth_gradients_match_finite_differences():
    n, k, m, g, bits = 3, 16, 12, 8, 4
    W, X, V, al, be = _layer(n, k, m, g, 7)
    V = V.astype(np.float64)
    al = al.astype(np.float64)
    be = be.astype(np.float64)
    r = oracle.loss_and_grads(W, X, V, al, be, bits, g, smooth=True)
    # some elements must be clipped for the (1 - m) terms to be exercised
    t = r["qd"]["t"]
    clipped = np.mean((t < 0) | (t > 2 ** bits - 1))
    assert 0.05 < clipped < 0.9
    h = 1e-6
    for name, arr, grad in [("V", V, r["dV"]), ("alpha", al, r["dalpha"]), ("beta", be, r["dbeta"])]:
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += h
            mm = arr.copy(); mm[idx] -= h
            args = dict(V=V, al=al, be=be)
            key = {"V": "V", "alpha": "al", "beta": "be"}[name]
            args[key] = p
            lp = _smooth_loss(W, X, args["V"], args["al"], args["be"], bits, g)
            args[key] = mm
            lm = _smooth_loss(W, X, args["V"], args["al"], args["be"], bits, g)
            fd[idx] = (lp - lm) / (2 * h)
        scale = np.max(np.abs(fd)) + 1e-30
        assert np.max(np.abs(fd - grad)) / scale < 1e-5, name


def _torch_ste_loss(W, X, V, al, be, bits, g):
    Q = 2 ** bits - 1
    Wt = torch.tensor(W, dtype=torch.float64)
    n, k = Wt.shape
    Wg = Wt.reshape(n, k // g, g)
    mx = torch.clamp(Wg.max(dim=2).values, min=0.0)
    mn = torch.clamp(Wg.min(dim=2).values, max=0.0)
    Vt = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    at = torch.tensor(al, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(be, dtype=torch.float64, requires_grad=True)

    def ste_round(x):
        return x + (torch.round(x) - x).detach()

    wmax = at * mx
    wmin = bt * mn
    s = (wmax - wmin) / Q
    z = ste_round(-wmin / s)
    u = Wg / s[:, :, None] + Vt.reshape(n, k // g, g)
    q = torch.clamp(ste_round(u) + z[:, :, None], 0.0, float(Q))
    w_hat = (s[:, :, None] * (q - z[:, :, None])).reshape(n, k)
    Xt = torch.tensor(X, dtype=torch.float64)
    D = Xt @ w_hat.T - Xt @ Wt.T
    L = (D * D).sum() / (X.shape[0] * n)
    L.backward()
    return L.item(), Vt.grad.numpy(), at.grad.numpy(), bt.grad.numpy()


@pytest.mark.parametrize("seed,clip", [(1, 0.8), (2, 0.6), (3, 1.0)])
def test_ste_gradients_match_torch_autograd(seed, clip):
    # fp64 copies of the fp32 parameters; the oracle's fp32 QDQ and torch's
    # fp64 forward agree on codes except at fp32-vs-fp64 rounding ties,
    # which random data almost never hits (checked below).
    n, k, m, g, bits = 4, 32, 20, 16, 4
    W, X, V, al, be = _layer(n, k, m, g, seed, clip)
    r = oracle.loss_and_grads(W, X, V, al, be, bits, g)
    L, gV, ga, gb = _torch_ste_loss(W, X, V.astype(np.float64), al.astype(np.float64),
                                    be.astype(np.float64), bits, g)
    assert r["L"] == pytest.approx(L, rel=1e-5)
    np.testing.assert_allclose(r["dV"], gV, rtol=1e-4, atol=1e-9 * np.abs(gV).max())
    np.testing.assert_allclose(r["dalpha"], ga, rtol=1e-4, atol=1e-6 * np.abs(ga).max())
    np.testing.assert_allclose(r["dbeta"], gb, rtol=1e-4, atol=1e-6 * np.abs(gb).max())


def test_loss_is_mean_square_of_output_error():
    # L = mean((X W_hat^T - X W^T)^2) written out with explicit loops
    n, k, m, g, bits = 3, 8, 5, 4, 4
    W, X, V, al, be = _layer(n, k, m, g, 4)
    r = oracle.loss_and_grads(W, X, V, al, be, bits, g)
    wh = r["qd"]["w_hat"].astype(np.float64)
    tot = 0.0
    for i in range(m):
        for j in range(n):
            y = sum(X[i, kk] * wh[j, kk] for kk in range(k))
            yr = sum(X[i, kk] * float(W[j, kk]) for kk in range(k))
            tot += (y - yr) ** 2
    assert r["L"] == pytest.approx(tot / (m * n), rel=1e-12)
    # G[j, kk] = dL/dw_hat[j, kk] by explicit loops
    j, kk = 1, 5
    gj = sum(2 * (sum(X[i, a] * (wh[j, a] - W[j, a]) for a in range(k))) * X[i, kk] for i in range(m)) / (m * n)
    assert r["G"][j, kk] == pytest.approx(gj, rel=1e-10)


def test_grid_exact_layer_has_zero_loss_and_gradients():
    rng = np.random.default_rng(0)
    ks = rng.integers(0, 16, size=(4, 64))
    ks[:, 0] = 0
    ks[:, 1] = 15
    ks[:, 32] = 0
    ks[:, 33] = 15
    W = (np.ldexp(1.0, -7) * (ks - 8)).astype(F32)
    X = rng.standard_normal((16, 64))
    r = oracle.loss_and_grads(W, X, np.zeros_like(W), np.ones((4, 2), F32), np.ones((4, 2), F32), 4, 32)
    assert r["L"] == 0.0
    assert np.all(r["dV"] == 0) and np.all(r["dalpha"] == 0) and np.all(r["dbeta"] == 0)
    res = oracle.tune_layer(W, X.reshape(1, 16, 64).astype(F32), np.zeros((5, 1), np.int32), 4, 32, 5, 0.005)
    assert np.all(res["V"] == 0) and np.all(res["alpha"] == 1) and np.all(res["beta"] == 1)


def test_bf16_mode_rounds_the_gemm_operand_only():
    n, k, m, g, bits = 8, 64, 16, 32, 4
    W, X, V, al, be = _layer(n, k, m, g, 9)
    r32 = oracle.loss_and_grads(W, X, V, al, be, bits, g, mode="f32")
    r16 = oracle.loss_and_grads(W, X, V, al, be, bits, g, mode="bf16")
    np.testing.assert_array_equal(r32["qd"]["q"], r16["qd"]["q"])
    Xd = X.astype(np.float64)
    D = Xd @ oracle.bf16_round(r32["qd"]["w_hat"]).astype(np.float64).T - Xd @ W.astype(np.float64).T
    assert r16["L"] == pytest.approx(np.mean(D * D), rel=1e-12)
    assert r16["L"] != r32["L"]
