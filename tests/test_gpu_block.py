"""GPU parity of block-wise tuning of a SwiGLU MLP block against the block
oracle: loss and straight-through gradients of all three linears (fp32 and
bf16 GEMM modes), the fp32 validation trajectory, fused against separate
kernels, the quantized block output handed to the next block, and the
Llama-7B-shaped block (hidden 4096, intermediate 11008) at full size."""
import numpy as np
import pytest
import torch

import oracle
from synthetic_inputs import make_block_workload

pytestmark = pytest.mark.gpu
F32 = np.float32
NAMES = oracle.LINEARS


@pytest.fixture(scope="module")
def ar():
    import post_weight_quantization_autoround_amd as mod
    assert torch.cuda.is_available()
    return mod


def _dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if bf16 else t


def _weights(wl):
    return {"gate": wl.Wg, "up": wl.Wu, "down": wl.Wd}


def _random_params(wl, seed):
    rng = np.random.default_rng(seed)
    out = {}
    for nm, W in _weights(wl).items():
        n, k = W.shape
        out[nm] = (rng.uniform(-0.5, 0.5, (n, k)).astype(F32), rng.uniform(0.5, 1.0, (n, k // wl.group)).astype(F32),
                   rng.uniform(0.5, 1.0, (n, k // wl.group)).astype(F32))
    return out


def _relf(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / (np.linalg.norm(b) + 1e-300))


def _small(dtype, **kw):
    cfg = dict(h=256, f=384, s=4, t=64, b=2, group=64, iters=10, dtype=dtype)
    cfg.update(kw)
    return make_block_workload("mlp4096_11008_g128", **cfg)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_block_gradients_match_oracle(ar, mode):
    wl = _small(mode)
    bf = mode == "bf16"
    params = _random_params(wl, 3)
    ids = [3, 1]
    Ws = _weights(wl)
    Y_ref = oracle.block_reference(wl.X, Ws, mode)
    ref = oracle.block_loss_and_grads(oracle.gather_batch(wl.X, ids), oracle.gather_batch(Y_ref, ids), Ws,
                                      {n: params[n][0] for n in NAMES}, {n: params[n][1] for n in NAMES},
                                      {n: params[n][2] for n in NAMES}, wl.bits, wl.group, mode=mode)
    out = ar.block_grads(_dev(wl.Wg, bf), _dev(wl.Wu, bf), _dev(wl.Wd, bf), _dev(wl.X, bf), ids,
                         params={n: tuple(_dev(a) for a in params[n]) for n in NAMES}, bits=wl.bits,
                         group_size=wl.group, gemm_mode=ar.AR_GEMM_BF16 if bf else ar.AR_GEMM_F32)
    assert out["loss"] == pytest.approx(ref["L"], rel=1e-3 if bf else 2e-5)
    tol = 1e-2 if bf else 2e-4
    for n in NAMES:
        assert _relf(out["G"][n].cpu().numpy(), ref["G"][n]) <= tol, n
        for key, r in zip(("dV", "dalpha", "dbeta"), ref["grads"][n]):
            assert _relf(out[key][n].cpu().numpy(), r) <= tol, (n, key)


def test_block_validation_trajectory(ar):
    wl = _small("f32", iters=12)
    Ws = _weights(wl)
    ref = oracle.tune_block(wl.X, Ws, wl.schedule, wl.bits, wl.group, wl.iters, wl.lr, mode="f32")
    res = ar.tune_block(_dev(wl.Wg), _dev(wl.Wu), _dev(wl.Wd), _dev(wl.X), bits=wl.bits, group_size=wl.group,
                        iters=wl.iters, lr=wl.lr, batch_samples=wl.b, schedule=wl.schedule.tolist(),
                        gemm_mode=ar.AR_GEMM_F32)
    losses = np.asarray(res["losses"], np.float64)
    rel = np.abs(losses[:10] - ref["losses"][:10]) / ref["losses"][:10]
    assert np.all(rel <= 1e-4), rel
    for n in NAMES:
        got = [a.cpu().numpy() for a in res["params"][n]]
        q_gpu = oracle.qdq(Ws[n], *got, wl.bits, wl.group)["q"]
        q_ref = oracle.qdq(Ws[n], *ref["params"][n], wl.bits, wl.group)["q"]
        assert float(np.mean(q_gpu == q_ref)) >= 0.995, n


def test_block_fused_matches_separate_kernels(ar):
    wl = _small("bf16", group=128, h=256, f=512, iters=8)
    args = [_dev(a, True) for a in (wl.Wg, wl.Wu, wl.Wd, wl.X)]
    kw = dict(bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist(), return_last=True, output=False)
    fused = ar.tune_block(*args, **kw)
    sep = ar.tune_block(*args, unfused=True, **kw)
    assert fused["losses"] == sep["losses"]
    for n in NAMES:
        for a, b in zip(fused["params"][n], sep["params"][n]):
            assert torch.equal(a, b), n


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_block_output_for_the_next_block(ar, mode):
    bf = mode == "bf16"
    wl = _small(mode, iters=6)
    Ws = _weights(wl)
    res = ar.tune_block(_dev(wl.Wg, bf), _dev(wl.Wu, bf), _dev(wl.Wd, bf), _dev(wl.X, bf), bits=wl.bits,
                        group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
                        schedule=wl.schedule.tolist(), gemm_mode=ar.AR_GEMM_BF16 if bf else ar.AR_GEMM_F32)
    params = {n: tuple(a.cpu().numpy() for a in res["params"][n]) for n in NAMES}
    ref = oracle.quantized_block_output(wl.X, Ws, params, wl.bits, wl.group, mode=mode)
    got = res["output"].float().cpu().numpy()
    assert got.shape == wl.X.shape
    assert _relf(got, ref) <= (1e-2 if bf else 1e-5)
    # the returned state is the best one: its loss on the best step's batch
    bs = res["best_step"]
    ids = wl.schedule[bs]
    Y_ref = oracle.block_reference(wl.X, Ws, mode)
    again = oracle.block_loss_and_grads(oracle.gather_batch(wl.X, ids), oracle.gather_batch(Y_ref, ids), Ws,
                                        {n: params[n][0] for n in NAMES}, {n: params[n][1] for n in NAMES},
                                        {n: params[n][2] for n in NAMES}, wl.bits, wl.group, mode=mode)
    assert res["best_loss"] == pytest.approx(again["L"], rel=1e-3 if bf else 1e-5)


def test_block_snapshot_and_determinism(ar):
    wl = _small("bf16", iters=10, group=128, f=512)
    args = [_dev(a, True) for a in (wl.Wg, wl.Wu, wl.Wd, wl.X)]
    kw = dict(bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist(), output=False)
    a = ar.tune_block(*args, **kw)
    b = ar.tune_block(*args, **kw)
    assert a["losses"] == b["losses"] and a["best_step"] == b["best_step"]
    assert a["best_loss"] == pytest.approx(min(a["losses"]), rel=1e-6)
    assert a["best_step"] == int(np.argmin(a["losses"]))
    for n in NAMES:
        for x, y in zip(a["params"][n], b["params"][n]):
            assert torch.equal(x, y)


def test_full_size_block_gradients(ar):
    # hidden 4096, intermediate 11008, g128, one 256-token sample
    wl = make_block_workload("mlp4096_11008_g128", s=2, b=1, iters=1)
    params = _random_params(wl, 5)
    ids = [1]
    Ws = _weights(wl)
    X_b = oracle.gather_batch(wl.X, ids)
    Y_ref, *_ = oracle.swiglu_forward(X_b, wl.Wg, wl.Wu, wl.Wd, mode="bf16")
    ref = oracle.block_loss_and_grads(X_b, Y_ref, Ws, {n: params[n][0] for n in NAMES},
                                      {n: params[n][1] for n in NAMES}, {n: params[n][2] for n in NAMES},
                                      wl.bits, wl.group, mode="bf16")
    out = ar.block_grads(_dev(wl.Wg, True), _dev(wl.Wu, True), _dev(wl.Wd, True), _dev(wl.X, True), ids,
                         params={n: tuple(_dev(a) for a in params[n]) for n in NAMES}, bits=wl.bits,
                         group_size=wl.group)
    assert out["loss"] == pytest.approx(ref["L"], rel=1e-3)
    for n in NAMES:
        assert _relf(out["G"][n].cpu().numpy(), ref["G"][n]) <= 1e-2, n
        for key, r in zip(("dV", "dalpha", "dbeta"), ref["grads"][n]):
            assert _relf(out[key][n].cpu().numpy(), r) <= 1e-2, (n, key)


def test_full_size_block_gradients_2048_tokens(ar):
    # hidden 4096, intermediate 11008, g128, 8 samples x 256 tokens: the dH
    # GEMM's 344 tiles of 256 x 256 run as one whole round plus a launch of
    # 256 x 128 tiles for the remaining rows
    wl = make_block_workload("mlp4096_11008_g128", s=9, b=8, iters=1)
    params = _random_params(wl, 7)
    ids = [8, 0, 1, 2, 3, 4, 5, 6]
    Ws = _weights(wl)
    X_b = oracle.gather_batch(wl.X, ids)
    Y_ref, *_ = oracle.swiglu_forward(X_b, wl.Wg, wl.Wu, wl.Wd, mode="bf16")
    ref = oracle.block_loss_and_grads(X_b, Y_ref, Ws, {n: params[n][0] for n in NAMES},
                                      {n: params[n][1] for n in NAMES}, {n: params[n][2] for n in NAMES},
                                      wl.bits, wl.group, mode="bf16")
    out = ar.block_grads(_dev(wl.Wg, True), _dev(wl.Wu, True), _dev(wl.Wd, True), _dev(wl.X, True), ids,
                         params={n: tuple(_dev(a) for a in params[n]) for n in NAMES}, bits=wl.bits,
                         group_size=wl.group)
    assert out["loss"] == pytest.approx(ref["L"], rel=1e-3)
    for n in NAMES:
        assert _relf(out["G"][n].cpu().numpy(), ref["G"][n]) <= 1e-2, n
        for key, r in zip(("dV", "dalpha", "dbeta"), ref["grads"][n]):
            assert _relf(out[key][n].cpu().numpy(), r) <= 1e-2, (n, key)
