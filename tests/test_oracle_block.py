"""Block-wise oracle (SwiGLU MLP) pinned to library routines (scipy's
sigmoid, torch's silu and autograd), to finite differences of the smooth
surrogate for the chain rule through the gated MLP, to the layer oracle when
gate and up are exactly representable, and to exhaustive search over the
joint rounding choices of a tiny block."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle

F32 = np.float32


def _block(h, f, m, g, seed, clip=(0.6, 0.95)):
    rng = np.random.default_rng(seed)
    Ws = {"gate": (rng.standard_normal((f, h)) * 0.5).astype(F32),
          "up": (rng.standard_normal((f, h)) * 0.5).astype(F32),
          "down": (rng.standard_normal((h, f)) * 0.5).astype(F32)}
    X = rng.standard_normal((m, h))
    Vs, als, bes = {}, {}, {}
    for nm, W in Ws.items():
        n, k = W.shape
        Vs[nm] = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
        als[nm] = rng.uniform(*clip, (n, k // g)).astype(F32)
        bes[nm] = rng.uniform(*clip, (n, k // g)).astype(F32)
    return Ws, X, Vs, als, bes


def test_silu_and_block_forward_match_library_routines():
    a = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(a), a * scipy.special.expit(a), rtol=1e-14, atol=1e-300)
    Ws, X, *_ = _block(8, 12, 5, 4, 0)
    Y, A, B, Hh = oracle.swiglu_forward(X, Ws["gate"], Ws["up"], Ws["down"])
    t = lambda x: torch.tensor(np.asarray(x, np.float64))
    ref = (torch.nn.functional.silu(t(X) @ t(Ws["gate"]).T) * (t(X) @ t(Ws["up"]).T)) @ t(Ws["down"]).T
    np.testing.assert_allclose(Y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_bf16_mode_rounds_the_gemm_operands():
    Ws, X, *_ = _block(8, 12, 5, 4, 1)
    Y, A, B, Hh = oracle.swiglu_forward(X, Ws["gate"], Ws["up"], Ws["down"], mode="bf16")
    r = lambda x: oracle.bf16_round(np.asarray(x, np.float64).astype(F32)).astype(np.float64)
    np.testing.assert_array_equal(Y, r(Hh) @ r(Ws["down"]).T)
    np.testing.assert_array_equal(A, X @ r(Ws["gate"]).T)


@pytest.mark.parametrize("sym", [False, True])
def test_block_smooth_gradients_match_finite_differences(sym):
    h, f, m, g = 4, 6, 10, 2
    Ws, X, Vs, als, bes = _block(h, f, m, g, 3)
    Y_ref, *_ = oracle.swiglu_forward(X, Ws["gate"], Ws["up"], Ws["down"])
    res = oracle.block_loss_and_grads(X, Y_ref, Ws, Vs, als, bes, 4, g, smooth=True, sym=sym)

    def loss(Vs_, als_, bes_):
        return oracle.block_loss_and_grads(X, Y_ref, Ws, Vs_, als_, bes_, 4, g, smooth=True, sym=sym)["L"]

    eps = 1e-6
    for nm in oracle.LINEARS:
        dV, da, db = res["grads"][nm]
        for which, arr, grad in (("V", Vs, dV), ("alpha", als, da), ("beta", bes, db)):
            fd = np.zeros_like(grad)
            for idx in np.ndindex(arr[nm].shape):
                hi = {k: v.astype(np.float64).copy() for k, v in arr.items()}
                lo = {k: v.astype(np.float64).copy() for k, v in arr.items()}
                hi[nm][idx] += eps
                lo[nm][idx] -= eps
                args_hi = [hi if a is arr else a for a in (Vs, als, bes)]
                args_lo = [lo if a is arr else a for a in (Vs, als, bes)]
                fd[idx] = (loss(*args_hi) - loss(*args_lo)) / (2 * eps)
            scale = np.max(np.abs(fd)) + 1e-30
            assert np.max(np.abs(fd - grad)) / scale < 1e-5, (nm, which)
    if sym:
        for nm in oracle.LINEARS:
            assert np.all(res["grads"][nm][2] == 0)


def test_block_ste_gradients_match_torch_autograd():
    h, f, m, g, bits = 8, 16, 12, 4, 4
    Ws, X, Vs, als, bes = _block(h, f, m, g, 5)
    Y_ref, *_ = oracle.swiglu_forward(X, Ws["gate"], Ws["up"], Ws["down"])
    res = oracle.block_loss_and_grads(X, Y_ref, Ws, Vs, als, bes, bits, g)
    Q = 2 ** bits - 1
    tv = {}

    def fake_quant(nm):
        W = torch.tensor(Ws[nm], dtype=torch.float64)
        n, k = W.shape
        Wg = W.reshape(n, k // g, g)
        mx = Wg.max(dim=2).values.clamp(min=0)
        mn = Wg.min(dim=2).values.clamp(max=0)
        V = torch.tensor(Vs[nm], dtype=torch.float64, requires_grad=True)
        al = torch.tensor(als[nm], dtype=torch.float64, requires_grad=True)
        be = torch.tensor(bes[nm], dtype=torch.float64, requires_grad=True)
        tv[nm] = (V, al, be)
        s = (al * mx - be * mn) / Q
        z0 = -be * mn / s
        z = z0 + (torch.round(z0) - z0).detach()
        u = Wg / s[:, :, None] + V.reshape(n, k // g, g)
        t = u + (torch.round(u) - u).detach() + z[:, :, None]
        q = torch.clamp(t, 0.0, float(Q))
        return (s[:, :, None] * (q - z[:, :, None])).reshape(n, k)

    wq = {nm: fake_quant(nm) for nm in oracle.LINEARS}
    Xt = torch.tensor(X, dtype=torch.float64)
    Y = (torch.nn.functional.silu(Xt @ wq["gate"].T) * (Xt @ wq["up"].T)) @ wq["down"].T
    L = ((Y - torch.tensor(Y_ref)) ** 2).sum() / Y.numel()
    L.backward()
    # the oracle's quantizer is fp32, torch's here fp64: agreement to fp32 level
    assert res["L"] == pytest.approx(L.item(), rel=1e-6)
    for nm in oracle.LINEARS:
        for got, ref in zip(res["grads"][nm], tv[nm]):
            r = ref.grad.numpy()
            np.testing.assert_allclose(got, r, rtol=1e-4, atol=1e-6 * np.abs(r).max())


def test_down_projection_reduces_to_the_layer_when_gate_and_up_are_exact():
    # grid-exact gate/up weights (both ends of the grid in every group): the
    # fake quantizer is the identity on them, so the block is the down
    # projection applied to a fixed activation and its gradients are the
    # layer oracle's
    h, f, m, g = 16, 32, 20, 16
    rng = np.random.default_rng(7)
    Ws = {}
    for nm in ("gate", "up"):
        k = rng.integers(0, 16, (f, h))
        k[:, ::g] = 0
        k[:, 1::g] = 15
        Ws[nm] = (2.0 ** -4 * (k - 8)).astype(F32)
    Ws["down"] = (rng.standard_normal((h, f)) * 0.05).astype(F32)
    X = rng.standard_normal((m, h))
    Vs = {nm: np.zeros_like(W) for nm, W in Ws.items()}
    Vs["down"] = rng.uniform(-0.5, 0.5, Ws["down"].shape).astype(F32)
    als = {nm: np.ones((W.shape[0], W.shape[1] // g), F32) for nm, W in Ws.items()}
    bes = {nm: a.copy() for nm, a in als.items()}
    als["down"] = rng.uniform(0.6, 1.0, als["down"].shape).astype(F32)
    for nm in ("gate", "up"):
        np.testing.assert_array_equal(oracle.qdq(Ws[nm], Vs[nm], als[nm], bes[nm], 4, g)["w_hat"], Ws[nm])
    Y_ref, _, _, Hh = oracle.swiglu_forward(X, Ws["gate"], Ws["up"], Ws["down"])
    blk = oracle.block_loss_and_grads(X, Y_ref, Ws, Vs, als, bes, 4, g)
    lay = oracle.loss_and_grads(Ws["down"], Hh, Vs["down"], als["down"], bes["down"], 4, g)
    assert blk["L"] == pytest.approx(lay["L"], rel=1e-12)
    np.testing.assert_allclose(blk["G"]["down"], lay["G"], rtol=1e-10, atol=1e-15)
    for got, ref in zip(blk["grads"]["down"], (lay["dV"], lay["dalpha"], lay["dbeta"])):
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-15)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_tuning_between_bruteforce_optimum_and_rtn(seed):
    h, f, m, g, bits, iters = 2, 2, 8, 2, 3, 60
    rng = np.random.default_rng(100 + seed)
    Ws = {"gate": rng.standard_normal((f, h)).astype(F32), "up": rng.standard_normal((f, h)).astype(F32),
          "down": rng.standard_normal((h, f)).astype(F32)}
    X = rng.standard_normal((1, m, h))
    lo, rtn = oracle.bruteforce_block_min_loss(X[0], Ws["gate"], Ws["up"], Ws["down"], bits, g)
    res = oracle.tune_block(X, Ws, [[0]] * iters, bits, g, iters, 0.02, lr_clip=0.0)
    assert res["losses"][0] == pytest.approx(rtn, rel=1e-9)
    assert lo - 1e-12 <= res["best_loss"] <= rtn * (1 + 1e-12)
    for nm in oracle.LINEARS:
        assert np.all(res["params"][nm][1] == 1) and np.all(res["params"][nm][2] == 1)


def test_quantized_output_is_the_forward_of_the_best_state():
    h, f, m, g = 8, 16, 6, 4
    rng = np.random.default_rng(9)
    Ws = {"gate": rng.standard_normal((f, h)).astype(F32), "up": rng.standard_normal((f, h)).astype(F32),
          "down": rng.standard_normal((h, f)).astype(F32)}
    X = rng.standard_normal((2, m, h))
    res = oracle.tune_block(X, Ws, [[0], [1]] * 3, 4, g, 6, 0.01)
    Yq = oracle.quantized_block_output(X, Ws, res["params"], 4, g)
    wq = {nm: oracle.qdq(Ws[nm], *res["params"][nm], 4, g)["w_hat"] for nm in oracle.LINEARS}
    Y, *_ = oracle.swiglu_forward(X.reshape(-1, h), wq["gate"], wq["up"], wq["down"])
    np.testing.assert_array_equal(Yq.reshape(-1, h), Y)
    # the snapshot's loss is recomputed from the returned state
    bs = res["best_step"]
    ids = [[0], [1]][bs % 2]
    Y_ref = oracle.block_reference(X, Ws)
    again = oracle.block_loss_and_grads(oracle.gather_batch(X, ids), oracle.gather_batch(Y_ref, ids), Ws,
                                        {nm: res["params"][nm][0] for nm in oracle.LINEARS},
                                        {nm: res["params"][nm][1] for nm in oracle.LINEARS},
                                        {nm: res["params"][nm][2] for nm in oracle.LINEARS}, 4, g)
    assert again["L"] == res["best_loss"]
