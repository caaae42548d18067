"""GPU parity of the tuning path against the oracle.

* loss and straight-through gradients at given states (ar_layer_grads):
  fp32-MFMA mode near-exact, bf16 mode within 1e-2 relative Frobenius error;
* the free-running SignSGD loop in fp32-MFMA mode on the 256 x 256 g32
  layer: per-step loss within 1e-4 relative for the first 10 steps and
  >= 99.5% of final codes equal;
* bf16 loop on a minibatch schedule: gradients at the GPU's own states
  match the oracle, the snapshot is the best evaluated loss, runs repeat
  bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic_inputs import make_layer_workload

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.fixture(scope="module")
def ar():
    import post_weight_quantization_autoround_amd as mod
    assert torch.cuda.is_available()
    return mod


def _dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if bf16 else t


def _relf(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def _random_state(n, k, g, seed, scale=0.3):
    rng = np.random.default_rng(seed)
    V = rng.uniform(-scale, scale, (n, k)).astype(F32)
    al = rng.uniform(0.6, 1.0, (n, k // g)).astype(F32)
    be = rng.uniform(0.6, 1.0, (n, k // g)).astype(F32)
    return V, al, be


@pytest.mark.parametrize("name,over,mode,ids", [
    ("linear256_g32", {}, "f32", [0]),
    ("linear4096_g128", dict(n=320, k=384, s=5, b=3, t=64, iters=1), "f32", [4, 0, 2]),
    ("linear4096_g128", dict(n=320, k=384, s=5, b=3, t=64, iters=1), "bf16", [4, 0, 2]),
    ("linear4096_g128", dict(n=512, k=1024, s=4, b=2, t=128, iters=1), "bf16", [1, 3]),
    ("linear4096_g128", dict(n=96, k=200, group=40, s=3, b=2, t=64, iters=1), "f32", [2, 1]),
])
def test_layer_grads_match_oracle(ar, name, over, mode, ids):
    wl = make_layer_workload(name, **over)
    n, k, g = wl.n, wl.k, wl.group
    V, al, be = _random_state(n, k, g, 5)
    Xb = oracle.gather_batch(wl.X, ids)
    ref = oracle.loss_and_grads(wl.W, Xb, V, al, be, wl.bits, g, mode=mode)
    bf16 = wl.dtype == "bf16"
    gm = ar.AR_GEMM_F32 if mode == "f32" else ar.AR_GEMM_BF16
    out = ar.layer_grads(_dev(wl.W, bf16), _dev(wl.X, bf16), ids, _dev(V), _dev(al), _dev(be),
                         bits=wl.bits, group_size=g, gemm_mode=gm)
    G = out["G"].cpu().numpy()
    dV = out["dV"].cpu().numpy()
    da = out["dalpha"].cpu().numpy()
    db = out["dbeta"].cpu().numpy()
    if mode == "f32":
        assert out["loss"] == pytest.approx(ref["L"], rel=2e-5)
        tol = 2e-4
    else:
        assert out["loss"] == pytest.approx(ref["L"], rel=1e-3)
        tol = 1e-2
    for name_, got, exp in [("G", G, ref["G"]), ("dV", dV, ref["dV"]), ("dalpha", da, ref["dalpha"]),
                            ("dbeta", db, ref["dbeta"])]:
        assert _relf(got, exp) <= tol, (name_, _relf(got, exp))
    # clamped weights get exactly zero offset gradient
    t = ref["qd"]["t"]
    outside = (t < 0) | (t > 2 ** wl.bits - 1)
    assert np.all(dV[outside] == 0)


def test_validation_mode_trajectory_linear256(ar):
    wl = make_layer_workload("linear256_g32")
    ref = oracle.tune_layer(wl.W, wl.X, wl.schedule, wl.bits, wl.group, wl.iters, wl.lr, mode="f32")
    res = ar.tune_layer(_dev(wl.W), _dev(wl.X), bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr,
                        batch_samples=wl.b, schedule=wl.schedule.tolist(), gemm_mode=ar.AR_GEMM_F32)
    losses = np.asarray(res["losses"], np.float64)
    rel = np.abs(losses[:10] - ref["losses"][:10]) / ref["losses"][:10]
    assert np.all(rel <= 1e-4), rel
    assert ref["losses"][-1] < ref["losses"][0]        # tuning helps on this layer
    q_gpu = oracle.qdq(wl.W, res["V"].cpu().numpy(), res["alpha"].cpu().numpy(), res["beta"].cpu().numpy(),
                       wl.bits, wl.group)["q"]
    q_ref = oracle.qdq(wl.W, ref["V"], ref["alpha"], ref["beta"], wl.bits, wl.group)["q"]
    agree = float(np.mean(q_gpu == q_ref))
    assert agree >= 0.995, agree
    assert res["best_loss"] == pytest.approx(float(np.min(losses)), rel=1e-6)


def test_bf16_loop_gradients_at_gpu_states(ar):
    # Trajectories part ways after any sign flip, so the oracle is fed the
    # GPU's own states: run t steps (return_last), then compare gradients.
    wl = make_layer_workload("linear4096_g128", n=256, k=512, s=6, b=2, t=64, iters=12)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    for t_stop in [1, 5, 11]:
        # state after the last update of a t_stop-step run of the same schedule
        part = ar.tune_layer(W, X, bits=4, group_size=128, iters=t_stop, lr=wl.lr, batch_samples=wl.b,
                             schedule=wl.schedule[:t_stop].tolist(), return_last=True)
        V, al, be = (part[x].cpu().numpy() for x in ("V", "alpha", "beta"))
        ids = wl.schedule[t_stop].tolist() if t_stop < wl.iters else wl.schedule[0].tolist()
        ref = oracle.loss_and_grads(wl.W, oracle.gather_batch(wl.X, ids), V, al, be, 4, 128, mode="bf16")
        out = ar.layer_grads(W, X, ids, part["V"], part["alpha"], part["beta"], bits=4, group_size=128)
        for key in ["G", "dV", "dalpha", "dbeta"]:
            assert _relf(out[key].cpu().numpy(), ref[key]) <= 1e-2, (t_stop, key)
        assert out["loss"] == pytest.approx(ref["L"], rel=1e-3)


def test_snapshot_and_determinism(ar):
    wl = make_layer_workload("linear4096_g128", n=256, k=512, s=6, b=2, t=64, iters=15)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    a = ar.tune_layer(W, X, bits=4, group_size=128, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
                      schedule=wl.schedule.tolist())
    b = ar.tune_layer(W, X, bits=4, group_size=128, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
                      schedule=wl.schedule.tolist())
    for key in ["V", "alpha", "beta"]:
        assert torch.equal(a[key], b[key])
    assert a["losses"] == b["losses"]
    losses = np.asarray(a["losses"])
    assert a["best_step"] == int(np.argmin(losses))
    # the returned state evaluates to the best loss on its own minibatch
    ids = wl.schedule[a["best_step"]].tolist()
    chk = ar.layer_grads(W, X, ids, a["V"], a["alpha"], a["beta"], bits=4, group_size=128)
    assert chk["loss"] == pytest.approx(float(losses[a["best_step"]]), rel=1e-6)
    # parameters stay in their boxes
    assert float(a["V"].abs().max()) <= 0.5
    assert float(a["alpha"].min()) >= 0.5 and float(a["alpha"].max()) <= 1.0


def test_update_bit_exact_given_signs(ar):
    # One step from a random state: given the gradients the GPU computed,
    # the GPU's updated parameters equal the oracle's fp32 SignSGD update of
    # the same signs, bit for bit.
    wl = make_layer_workload("linear4096_g128", n=128, k=256, s=2, b=1, t=64, iters=1)
    V, al, be = _random_state(wl.n, wl.k, 128, 8)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    ids = wl.schedule[0].tolist()
    res = ar.tune_layer(W, X, bits=4, group_size=128, iters=1, lr=0.01, batch_samples=1,
                        schedule=[ids], return_last=True, V0=_dev(V), alpha0=_dev(al), beta0=_dev(be))
    g = ar.layer_grads(W, X, ids, _dev(V), _dev(al), _dev(be), bits=4, group_size=128)
    lr0 = oracle.lr_table(0.01, 1)[0]
    expV = oracle.signsgd_step(V, g["dV"].cpu().numpy(), lr0, -0.5, 0.5)
    expA = oracle.signsgd_step(al, g["dalpha"].cpu().numpy(), lr0, 0.5, 1.0)
    expB = oracle.signsgd_step(be, g["dbeta"].cpu().numpy(), lr0, 0.5, 1.0)
    np.testing.assert_array_equal(res["V"].cpu().numpy(), expV)
    np.testing.assert_array_equal(res["alpha"].cpu().numpy(), expA)
    np.testing.assert_array_equal(res["beta"].cpu().numpy(), expB)


@pytest.mark.parametrize("over", [
    dict(n=256, k=512, s=6, b=2, t=64, iters=12),                 # 128-wide tiles, g128
    dict(n=320, k=320, group=64, s=5, b=3, t=64, iters=8),        # ragged rows and columns
    dict(n=192, k=256, group=32, s=4, b=2, t=128, iters=8),       # g32, 8 groups per tile row
])
def test_fused_update_matches_separate_kernels(ar, over):
    # The weight-gradient GEMM with the backward, update and next fake
    # quantization in its epilogue must reproduce the six-kernel step bit for bit.
    wl = make_layer_workload("linear4096_g128", **over)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    kw = dict(bits=4, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist(), return_last=True)
    fused = ar.tune_layer(W, X, **kw)
    sep = ar.tune_layer(W, X, unfused=True, **kw)
    assert fused["losses"] == sep["losses"]
    for key in ["V", "alpha", "beta"]:
        assert torch.equal(fused[key], sep[key]), key
    t = ar.Tuner(W, X, bits=4, group_size=wl.group, iters=1, batch_samples=wl.b, schedule=wl.schedule[:1].tolist())
    n_k = ar.lib.ar_tuner_num_kernels(t._h)
    t.close()
    assert n_k == 2      # forward GEMM with the loss; weight-gradient GEMM taking the decision and the update


@pytest.mark.parametrize("unfused", [False, True])
def test_nonfinite_loss_halts_the_loop(ar, unfused):
    # Finite bf16 weights and activations whose products overflow fp32: the
    # reference output and the first loss are not finite.  The loop stops at
    # step 0 (the fused weight-gradient launch takes this decision itself,
    # the six-kernel step in its own kernel) and reports AR_ERR_NONFINITE;
    # every kernel runs to its end.
    wl = make_layer_workload("linear4096_g128", n=256, k=512, s=4, b=2, t=64, iters=4)
    # every |w x| >= 1e39 > fp32 max; both stay far below the bf16 maximum
    W = _dev(np.where(wl.W < 0, -1.0, 1.0) * (1.0 + np.abs(wl.W) / np.abs(wl.W).max()) * 1e19, True)
    X = _dev(np.where(wl.X < 0, -1.0, 1.0) * (1.0 + np.abs(wl.X) / np.abs(wl.X).max()) * 1e20, True)
    assert torch.isfinite(W.float()).all() and torch.isfinite(X.float()).all()
    with pytest.raises(ar.ARError) as e:
        ar.tune_layer(W, X, bits=4, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
                      schedule=wl.schedule.tolist(), unfused=unfused)
    assert e.value.status == ar.AR_ERR_NONFINITE
    assert "step 0" in str(e.value)


def test_fused_full_size_layer_matches_separate_kernels(ar):
    # 4096 x 4096 bf16, g128, 2048 tokens per step: the 256 x 256 tile path
    wl = make_layer_workload("linear4096_g128", iters=4)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    kw = dict(bits=4, group_size=128, iters=4, lr=wl.lr, batch_samples=8, schedule=wl.schedule.tolist(),
              return_last=True)
    fused = ar.tune_layer(W, X, **kw)
    sep = ar.tune_layer(W, X, unfused=True, **kw)
    assert fused["losses"] == sep["losses"]
    for key in ["V", "alpha", "beta"]:
        assert torch.equal(fused[key], sep[key]), key
    # sampled oracle check at full size: a row of G (and of dV, dalpha, dbeta)
    # depends only on that row of the weight, so the oracle evaluates 48 rows
    # exactly; its 2/(M*N) normalisation uses the sampled row count.
    rng = np.random.default_rng(0)
    V = rng.uniform(-0.3, 0.3, (4096, 4096)).astype(F32)
    al = rng.uniform(0.6, 1.0, (4096, 32)).astype(F32)
    be = rng.uniform(0.6, 1.0, (4096, 32)).astype(F32)
    ids = wl.schedule[1].tolist()
    out = ar.layer_grads(W, X, ids, _dev(V), _dev(al), _dev(be), bits=4, group_size=128)
    rows = np.sort(rng.choice(4096, 48, replace=False))
    ref = oracle.loss_and_grads(wl.W[rows], oracle.gather_batch(wl.X, ids), V[rows], al[rows], be[rows], 4, 128,
                                mode="bf16")
    scale = len(rows) / 4096.0
    for key in ["G", "dV", "dalpha", "dbeta"]:
        got = out[key].cpu().numpy()[rows]
        assert _relf(got, ref[key] * scale) <= 1e-2, key


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_symmetric_layer_grads_match_oracle(ar, mode):
    wl = make_layer_workload("linear4096_g128", n=320, k=384, s=5, b=3, t=64, iters=1)
    V, al, be = _random_state(wl.n, wl.k, 128, 12)
    ids = [4, 0, 2]
    ref = oracle.loss_and_grads(wl.W, oracle.gather_batch(wl.X, ids), V, al, be, 4, 128, mode=mode, sym=True)
    gm = ar.AR_GEMM_F32 if mode == "f32" else ar.AR_GEMM_BF16
    out = ar.layer_grads(_dev(wl.W, True), _dev(wl.X, True), ids, _dev(V), _dev(al), _dev(be), bits=4,
                         group_size=128, gemm_mode=gm, sym=True)
    tol = 2e-4 if mode == "f32" else 1e-2
    assert out["loss"] == pytest.approx(ref["L"], rel=2e-5 if mode == "f32" else 1e-3)
    for key in ["G", "dV", "dalpha"]:
        assert _relf(out[key].cpu().numpy(), ref[key]) <= tol, key
    assert float(out["dbeta"].abs().max()) == 0.0


def test_symmetric_validation_trajectory(ar):
    wl = make_layer_workload("linear256_g32")
    ref = oracle.tune_layer(wl.W, wl.X, wl.schedule, wl.bits, wl.group, wl.iters, wl.lr, mode="f32", sym=True)
    res = ar.tune_layer(_dev(wl.W), _dev(wl.X), bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr,
                        batch_samples=wl.b, schedule=wl.schedule.tolist(), gemm_mode=ar.AR_GEMM_F32, sym=True)
    losses = np.asarray(res["losses"], np.float64)
    rel = np.abs(losses[:10] - ref["losses"][:10]) / ref["losses"][:10]
    assert np.all(rel <= 1e-4), rel
    q_gpu = oracle.qdq(wl.W, res["V"].cpu().numpy(), res["alpha"].cpu().numpy(), res["beta"].cpu().numpy(),
                       wl.bits, wl.group, sym=True)["q"]
    q_ref = oracle.qdq(wl.W, ref["V"], ref["alpha"], ref["beta"], wl.bits, wl.group, sym=True)["q"]
    assert float(np.mean(q_gpu == q_ref)) >= 0.995
    assert torch.equal(res["beta"], torch.ones_like(res["beta"]))


def test_symmetric_fused_matches_separate_kernels(ar):
    wl = make_layer_workload("linear4096_g128", n=256, k=512, s=6, b=2, t=64, iters=10)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    kw = dict(bits=4, group_size=128, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist(), return_last=True, sym=True)
    fused = ar.tune_layer(W, X, **kw)
    sep = ar.tune_layer(W, X, unfused=True, **kw)
    assert fused["losses"] == sep["losses"]
    for key in ["V", "alpha", "beta"]:
        assert torch.equal(fused[key], sep[key]), key


def test_graph_replays_match_eager_steps(ar):
    # 19 steps through captured graphs (two 8-step graphs, then three
    # single-step ones) against 19 eagerly enqueued steps, and a run split
    # over several calls: the same losses and parameters bit for bit.
    wl = make_layer_workload("linear4096_g128", n=256, k=512, s=6, b=2, t=64, iters=19)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    kw = dict(bits=4, group_size=128, iters=wl.iters, lr=wl.lr, batch_samples=wl.b, schedule=wl.schedule.tolist())
    outs = []
    for plan in ([(19, True)], [(19, False)], [(3, True), (9, True), (7, False)]):
        t = ar.Tuner(W, X, **kw)
        for n, graph in plan:
            t.run(n, graph=graph)
        outs.append(t.finish())
        t.close()
    for o in outs[1:]:
        assert o["losses"] == outs[0]["losses"]
        for key in ["V", "alpha", "beta"]:
            assert torch.equal(o[key], outs[0][key]), key
    assert all(np.isfinite(outs[0]["losses"]))


def test_full_size_tuning_improves_on_rtn(ar):
    # 200 SignSGD steps on the 4096 x 4096 bf16 g128 layer (2048 tokens per
    # step): the returned state beats round-to-nearest on held-in minibatches,
    # by the GPU's loss and by the oracle's on 64 sampled rows (the loss is a
    # sum over rows, each depending only on its own weight row)
    wl = make_layer_workload("linear4096_g128")
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    res = ar.tune_layer(W, X, bits=4, group_size=128, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
                        schedule=wl.schedule.tolist())
    assert all(np.isfinite(res["losses"]))
    V0 = torch.zeros_like(res["V"])
    A0 = torch.ones_like(res["alpha"])
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(wl.n, 64, replace=False))
    Vt, at, bt = (res[x].cpu().numpy() for x in ("V", "alpha", "beta"))
    for ids in (wl.schedule[0].tolist(), wl.schedule[wl.iters // 2].tolist()):
        tuned = ar.layer_grads(W, X, ids, res["V"], res["alpha"], res["beta"], bits=4, group_size=128)["loss"]
        rtn = ar.layer_grads(W, X, ids, V0, A0, A0.clone(), bits=4, group_size=128)["loss"]
        assert tuned < rtn, (tuned, rtn)
        Xb = oracle.gather_batch(wl.X, ids)
        o_t = oracle.loss_and_grads(wl.W[rows], Xb, Vt[rows], at[rows], bt[rows], 4, 128, mode="bf16")["L"]
        o_r = oracle.loss_and_grads(wl.W[rows], Xb, np.zeros_like(Vt[rows]), np.ones_like(at[rows]),
                                    np.ones_like(bt[rows]), 4, 128, mode="bf16")["L"]
        assert o_t < o_r, (o_t, o_r)


def test_full_run_on_a_row_slice_tracks_the_oracle(ar):
    # A row's sign updates depend only on that row, so a 256-row slice of the
    # 4096 x 4096 layer replays the full layer's trajectory for those rows.
    # 200 bf16 steps (state after the last update) against the oracle: the
    # first 20 losses agree to 1e-3, and after sign flips part the two ways
    # they still follow one curve (median gap, lowest loss).
    wl = make_layer_workload("linear4096_g128")
    Ws = np.ascontiguousarray(wl.W[:256])
    gpu = ar.tune_layer(_dev(Ws, True), _dev(wl.X, True), bits=4, group_size=128, iters=wl.iters, lr=wl.lr,
                        batch_samples=wl.b, schedule=wl.schedule.tolist(), return_last=True)
    ref = oracle.tune_layer(Ws, wl.X, wl.schedule, 4, 128, wl.iters, wl.lr, mode="bf16", return_last=True)
    g, r = np.asarray(gpu["losses"], np.float64), np.asarray(ref["losses"], np.float64)
    rel = np.abs(g - r) / r
    assert np.all(rel[:20] <= 1e-3), rel[:20]
    assert float(np.median(rel)) <= 0.05, float(np.median(rel))
    assert abs(g.min() - r.min()) / r.min() <= 0.05, (g.min(), r.min())


def test_tail_split_gradient_gemm_rows_match_oracle(ar):
    # 4352 x 4096 layer, 512 tokens: the stored weight-gradient GEMM has
    # 17 x 16 tiles of 256 x 256, so rows 0..4095 run as one round and rows
    # 4096..4351 as a second launch of 256 x 128 tiles.  Rows on both sides of
    # the seam against the oracle (each row of G depends only on its own row).
    wl = make_layer_workload("linear4096_g128", n=4352, s=4, b=2, iters=1)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    rng = np.random.default_rng(4)
    V = rng.uniform(-0.3, 0.3, (wl.n, wl.k)).astype(F32)
    al = rng.uniform(0.6, 1.0, (wl.n, wl.k // 128)).astype(F32)
    be = rng.uniform(0.6, 1.0, (wl.n, wl.k // 128)).astype(F32)
    ids = [3, 1]
    out = ar.layer_grads(W, X, ids, _dev(V), _dev(al), _dev(be), bits=4, group_size=128)
    rows = np.array([0, 1, 255, 2048, 4094, 4095, 4096, 4097, 4200, 4351])
    ref = oracle.loss_and_grads(wl.W[rows], oracle.gather_batch(wl.X, ids), V[rows], al[rows], be[rows], 4, 128,
                                mode="bf16")
    scale = len(rows) / wl.n
    for key in ["G", "dV", "dalpha", "dbeta"]:
        got = out[key].cpu().numpy()[rows]
        assert _relf(got, ref[key] * scale) <= 1e-2, key
        for j, r in enumerate(rows):   # each row on its own, so a misplaced tail row cannot hide
            assert _relf(got[j], ref[key][j] * scale) <= 2e-2, (key, int(r))


@pytest.mark.parametrize("iters,t_idx,lr", [(200, 6, 0.005), (20, 3, 0.005), (200, 137, 0.005)])
def test_update_bit_exact_given_signs_on_later_steps(ar, iters, t_idx, lr):
    # One step at index t_idx of an iters-step run (resumed there with
    # start_step): the update uses lr_t of that index.  At t = 6 of 200 and
    # t = 3 of 20, fp32(0.005) and the decimal 0.005 give step sizes one ulp
    # apart; the GPU must equal the oracle's table bit for bit.
    wl = make_layer_workload("linear4096_g128", n=128, k=256, s=2, b=1, t=64, iters=1)
    V, al, be = _random_state(wl.n, wl.k, 128, 9)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    ids = [1]
    sched = [[0]] * iters
    sched[t_idx] = ids
    tu = ar.Tuner(W, X, bits=4, group_size=128, iters=iters, lr=lr, batch_samples=1, schedule=sched,
                  return_last=True, V0=_dev(V), alpha0=_dev(al), beta0=_dev(be), start_step=t_idx)
    tu.run(1)
    res = tu.finish()
    tu.close()
    assert res["best_step"] == t_idx and np.isnan(res["losses"][t_idx - 1]) and np.isnan(res["losses"][t_idx + 1])
    g = ar.layer_grads(W, X, ids, _dev(V), _dev(al), _dev(be), bits=4, group_size=128)
    assert res["losses"][t_idx] == pytest.approx(g["loss"], rel=1e-6)
    lr_t = oracle.lr_table(lr, iters)[t_idx]
    expV = oracle.signsgd_step(V, g["dV"].cpu().numpy(), lr_t, -0.5, 0.5)
    expA = oracle.signsgd_step(al, g["dalpha"].cpu().numpy(), lr_t, 0.5, 1.0)
    expB = oracle.signsgd_step(be, g["dbeta"].cpu().numpy(), lr_t, 0.5, 1.0)
    np.testing.assert_array_equal(res["V"].cpu().numpy(), expV)
    np.testing.assert_array_equal(res["alpha"].cpu().numpy(), expA)
    np.testing.assert_array_equal(res["beta"].cpu().numpy(), expB)


@pytest.mark.parametrize("mode,over,k_split", [
    ("f32", dict(n=256, k=512, s=6, b=2, t=64, iters=20), 7),
    ("bf16", dict(n=256, k=512, s=6, b=2, t=64, iters=20), 9),    # fused weight-gradient epilogue
    ("bf16", dict(n=256, k=512, s=6, b=2, t=64, iters=20), 16),   # resumes inside the 8-step graphs' range
])
def test_split_run_equals_full_run(ar, mode, over, k_split):
    # Steps 0..k-1 in one call and k..T-1 in a second call resumed with
    # start_step = k, best_loss_in = the first call's best loss, from the state
    # after step k-1: the same losses, snapshot and state as one T-step run.
    wl = make_layer_workload("linear4096_g128", **over)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    gm = ar.AR_GEMM_F32 if mode == "f32" else ar.AR_GEMM_BF16
    kw = dict(bits=4, group_size=128, iters=wl.iters, lr=wl.lr, batch_samples=wl.b, schedule=wl.schedule.tolist(),
              gemm_mode=gm)
    full = ar.tune_layer(W, X, **kw)
    parts = []
    for last in (True, False):
        tu = ar.Tuner(W, X, return_last=last, **kw)
        tu.run(k_split)
        parts.append(tu.finish())
        tu.close()
    cur, best1 = parts
    assert cur["best_loss"] == best1["best_loss"] and cur["best_step"] == best1["best_step"]
    second = ar.tune_layer(W, X, V0=cur["V"], alpha0=cur["alpha"], beta0=cur["beta"], start_step=k_split,
                           best_loss_in=best1["best_loss"], **kw)
    assert np.all(np.isnan(second["losses"][:k_split]))
    assert second["losses"][k_split:] == full["losses"][k_split:]
    assert best1["losses"][:k_split] == full["losses"][:k_split]
    if full["best_step"] >= k_split:
        assert second["best_step"] == full["best_step"]
        chosen = second
    else:
        assert second["best_step"] == -1 and second["best_loss"] == best1["best_loss"]
        assert best1["best_step"] == full["best_step"]
        chosen = best1
    assert chosen["best_loss"] == full["best_loss"]
    for key in ["V", "alpha", "beta"]:
        assert torch.equal(chosen[key], full[key]), key


def _config2():
    return make_layer_workload("linear4096_g128")


def test_validation_mode_trajectory_config2_slice(ar):
    # fp32-MFMA validation run of the 4096 x 4096 g128 layer (2048 tokens per
    # step, 200 steps, lr 0.005) on its first 256 rows.  A row's gradients
    # and sign updates depend only on that row, so the slice follows the full
    # layer's rows; the loss is the slice's own mean.  First 10 losses within
    # 1e-4 relative of the oracle, >= 99.5% of the final codes equal.
    wl = _config2()
    Ws = np.ascontiguousarray(wl.W[:256])
    gpu = ar.tune_layer(_dev(Ws, True), _dev(wl.X, True), bits=4, group_size=128, iters=wl.iters, lr=wl.lr,
                        batch_samples=wl.b, schedule=wl.schedule.tolist(), gemm_mode=ar.AR_GEMM_F32)
    ref = oracle.tune_layer(Ws, wl.X, wl.schedule, 4, 128, wl.iters, wl.lr, mode="f32")
    g, r = np.asarray(gpu["losses"], np.float64), ref["losses"]
    rel = np.abs(g[:10] - r[:10]) / r[:10]
    assert np.all(rel <= 1e-4), rel
    q_gpu = oracle.qdq(Ws, gpu["V"].cpu().numpy(), gpu["alpha"].cpu().numpy(), gpu["beta"].cpu().numpy(),
                       4, 128)["q"]
    q_ref = oracle.qdq(Ws, ref["V"], ref["alpha"], ref["beta"], 4, 128)["q"]
    agree = float(np.mean(q_gpu == q_ref))
    first_diff = int(np.argmax(np.abs(g - r) / r > 1e-4)) if np.any(np.abs(g - r) / r > 1e-4) else -1
    print(f"config-2 slice fp32: code agreement {agree:.5f}, best steps {gpu['best_step']}/{ref['best_step']}, "
          f"first step with loss gap > 1e-4: {first_diff}", flush=True)
    assert agree >= 0.995, agree


def test_bf16_gradients_at_gpu_states_config2(ar):
    # The 4096 x 4096 bf16 g128 layer run with its 200-step schedule; at
    # t in {0, 1, 10, 100, 199} the GPU's own state (after t updates, lr
    # decaying over the full 200 steps) is fed to the oracle on 48 sampled
    # rows, with that step's minibatch: G, dV, dalpha and dbeta within 1e-2
    # relative Frobenius error (a row of each depends only on its own row;
    # the oracle's 2/(M*N) uses the sampled row count, hence the scale).
    wl = _config2()
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    tu = ar.Tuner(W, X, bits=4, group_size=128, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
                  schedule=wl.schedule.tolist(), return_last=True)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(wl.n, 48, replace=False))
    done = 0
    for t_stop in [0, 1, 10, 100, 199]:
        tu.run(t_stop - done)
        done = t_stop
        st = tu.finish()
        ids = wl.schedule[t_stop].tolist()
        out = ar.layer_grads(W, X, ids, st["V"], st["alpha"], st["beta"], bits=4, group_size=128)
        V, al, be = (st[x].cpu().numpy()[rows] for x in ("V", "alpha", "beta"))
        ref = oracle.loss_and_grads(wl.W[rows], oracle.gather_batch(wl.X, ids), V, al, be, 4, 128, mode="bf16")
        scale = len(rows) / wl.n
        errs = {}
        for key in ["G", "dV", "dalpha", "dbeta"]:
            errs[key] = _relf(out[key].cpu().numpy()[rows], ref[key] * scale)
        print(f"t={t_stop}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
        for key, e in errs.items():
            assert e <= 1e-2, (t_stop, key, e)
    tu.close()


def test_fused_g32_full_size_layer_matches_oracle(ar):
    # 4096 x 4096 bf16 with g32: the fused 256 x 256 weight-gradient tile
    # runs the straight-through backward, the update and the next fake
    # quantization for 8 groups per tile row.  One step from a random state:
    # on 48 sampled rows the updated V, alpha, beta equal the oracle's update
    # with the oracle's own gradient signs wherever that gradient is not
    # within the bf16 error of zero; a second call checks fused = separate
    # kernels bit for bit over 3 steps.
    wl = make_layer_workload("linear4096_g128", group=32, iters=3)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    V, al, be = _random_state(wl.n, wl.k, 32, 21)
    ids = wl.schedule[0].tolist()
    one = ar.tune_layer(W, X, bits=4, group_size=32, iters=1, lr=wl.lr, batch_samples=wl.b, schedule=[ids],
                        return_last=True, V0=_dev(V), alpha0=_dev(al), beta0=_dev(be))
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(wl.n, 48, replace=False))
    ref = oracle.loss_and_grads(wl.W[rows], oracle.gather_batch(wl.X, ids), V[rows], al[rows], be[rows], 4, 32,
                                mode="bf16")
    lr0 = oracle.lr_table(wl.lr, 1)[0]
    for key, p0, grad, lo, hi in [("V", V, ref["dV"], -0.5, 0.5), ("alpha", al, ref["dalpha"], 0.5, 1.0),
                                  ("beta", be, ref["dbeta"], 0.5, 1.0)]:
        exp = oracle.signsgd_step(p0[rows], grad, lr0, lo, hi)
        got = one[key].cpu().numpy()[rows]
        # an element whose oracle gradient is below 2% of its row's rms may take either sign
        rms = np.sqrt(np.mean(grad * grad, axis=1, keepdims=True))
        sure = np.abs(grad) > 0.02 * rms
        assert np.array_equal(got[sure], exp[sure]), (key, int(np.sum(got[sure] != exp[sure])))
        assert float(np.mean(got == exp)) >= 0.99, key
    kw = dict(bits=4, group_size=32, iters=3, lr=wl.lr, batch_samples=wl.b, schedule=wl.schedule.tolist(),
              return_last=True)
    fused = ar.tune_layer(W, X, **kw)
    sep = ar.tune_layer(W, X, unfused=True, **kw)
    assert fused["losses"] == sep["losses"]
    for key in ["V", "alpha", "beta"]:
        assert torch.equal(fused[key], sep[key]), key


def test_timing_modes(ar):
    # AR_RUN_EVENTS: eager steps with a HIP event between kernels give the
    # same trajectory as graph steps and a positive mean duration per kernel.
    # AR_RUN_KERNEL_GRAPHS: per-kernel graphs for timing only; they still
    # advance the step counter within iters and the tuner finishes.
    wl = make_layer_workload("linear4096_g128", n=256, k=512, s=6, b=2, t=64, iters=12)
    W, X = _dev(wl.W, True), _dev(wl.X, True)
    kw = dict(bits=4, group_size=128, iters=wl.iters, lr=wl.lr, batch_samples=wl.b, schedule=wl.schedule.tolist())
    full = ar.tune_layer(W, X, **kw)
    tu = ar.Tuner(W, X, **kw)
    tu.run(4, events=True)
    ev = tu.kernel_ms()
    tu.run(wl.iters - 4)
    res = tu.finish()
    tu.close()
    assert ev and all(v > 0 for v in ev.values()), ev
    assert res["losses"] == full["losses"] and res["best_step"] == full["best_step"]
    for key in ["V", "alpha", "beta"]:
        assert torch.equal(res[key], full[key]), key
    tu = ar.Tuner(W, X, **kw)
    tu.run(6, kernel_graphs=True)
    kg = tu.kernel_ms()
    with pytest.raises(ar.ARError):
        tu.run(wl.iters - 5)      # past iters: refused on the host
    tu.run(wl.iters - 6)
    tu.finish()
    tu.close()
    assert set(kg) == set(ev) and all(v > 0 for v in kg.values()), kg
