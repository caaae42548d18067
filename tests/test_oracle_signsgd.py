"""Oracle SignSGD, snapshot, brute-force optimum and INT4 packing, pinned to
closed forms, exhaustive search and round trips.

* SignSGD (AutoRound blog sec. 3 update rule): equal-size moves of lr_t per
  step against the gradient sign, no move for a zero gradient, parameters
  kept in their boxes (v in [-0.5, 0.5], blog sec. 3 variable table);
* tuning can only improve on RTN (step 0 is the RTN state and the best
  snapshot is kept) and can never beat the exhaustive optimum over the 2^N
  rounding choices (blog sec. 2 trade-off discussion);
* packing: two codes per byte and the coordinates page's byte formula.
"""
import numpy as np
import pytest

import oracle

F32 = np.float32


def test_signsgd_closed_form_constant_sign():
    T = 50
    lrs = oracle.lr_table(0.005, T)
    p = np.asarray([0.0, 0.1, -0.3, 0.49], F32)
    grad = np.asarray([1.0, -2.0, 0.0, -1e-30])
    q = p.copy()
    for t in range(T):
        q = oracle.signsgd_step(q, grad, lrs[t], -0.5, 0.5)
        assert np.all(q >= -0.5) and np.all(q <= 0.5)
    total = float(np.sum(lrs.astype(np.float64)))        # 0.005 * (T+1)/2
    assert total == pytest.approx(0.005 * (T + 1) / 2, rel=1e-6)
    assert q[0] == pytest.approx(-total, abs=1e-6)
    assert q[1] == pytest.approx(min(0.1 + total, 0.5), abs=1e-6)
    assert q[2] == F32(-0.3)                               # sign(0) = 0: no move
    assert q[3] == F32(0.5)                                # clamped at the top


def test_signsgd_step_is_exact_fp32_subtract():
    rng = np.random.default_rng(0)
    p = rng.uniform(-0.5, 0.5, 1000).astype(F32)
    g = rng.standard_normal(1000)
    lr = F32(0.0031)
    out = oracle.signsgd_step(p, g, lr, -0.5, 0.5)
    exp = np.where(g > 0, p - lr, p + lr).astype(F32)
    np.testing.assert_array_equal(out, np.clip(exp, F32(-0.5), F32(0.5)))


def test_lr_table_linear_decay():
    lrs = oracle.lr_table(0.005, 200)
    assert lrs.dtype == np.float32 and lrs.shape == (200,)
    assert np.all(np.diff(lrs.astype(np.float64)) < 0)
    np.testing.assert_allclose(lrs, 0.005 * (1 - np.arange(200) / 200), rtol=1e-7)
    np.testing.assert_array_equal(oracle.lr_table(0.005, 7, decay=False), np.full(7, F32(0.005)))


def test_lr_table_starts_from_the_single_precision_lr():
    # The step size reaches the tuner as fp32, so fp32(0.005) = 0.004999999888...
    # is the value decayed.  The decimal 0.005 would give a table that differs
    # in the last place at these steps (counted by hand from the two exact
    # products: 0.97 * 0.004999999888 = 0.0048499998917 rounds down to
    # 0.0048499997, where 0.97 * 0.005 = 0.00485 rounds to 0.00485).
    lrs = oracle.lr_table(0.005, 200)
    assert lrs[0] == F32(0.005)
    assert lrs[6] == F32(0.0048499997)
    assert lrs[6] != F32(0.00485)
    assert float(lrs[6]) < 0.97 * 0.005
    short = oracle.lr_table(0.005, 20)
    assert short[3] == np.nextafter(F32(0.85 * 0.005), F32(0))   # one ulp below the decimal table


def _tiny(seed, n=2, k=12):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    W[0, 3] *= 20
    X = rng.standard_normal((1, 24, k)).astype(F32)
    return W, X


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4, 5])
def test_tuning_between_bruteforce_optimum_and_rtn(seed):
    W, X = _tiny(seed)
    k = W.shape[1]
    bits, g, iters = 3, k, 60
    lo, rtn_loss = oracle.bruteforce_min_loss(W, X[0], bits, g)
    sched = np.zeros((iters, 1), np.int32)
    res = oracle.tune_layer(W, X, sched, bits, g, iters, lr=0.02, lr_clip=0.0)
    assert np.all(res["alpha"] == 1) and np.all(res["beta"] == 1)
    assert res["losses"][0] == pytest.approx(rtn_loss, rel=1e-9)   # step 0 is RTN
    assert lo <= res["best_loss"] + 1e-15
    assert res["best_loss"] <= rtn_loss * (1 + 1e-9)
    if seed in (0, 1, 5):                                           # these improve
        assert res["best_loss"] < rtn_loss
    if seed in (1, 5):                                              # and reach the optimum
        assert res["best_loss"] == pytest.approx(lo, rel=1e-9)
    # the snapshot's loss is the best loss
    r = oracle.loss_and_grads(W, X[0], res["V"], res["alpha"], res["beta"], bits, g)
    assert r["L"] == pytest.approx(res["best_loss"], rel=1e-12)
    assert res["best_loss"] == pytest.approx(res["losses"].min(), rel=0)
    assert res["best_step"] == int(np.argmin(res["losses"]))


def test_bruteforce_is_exhaustive_on_one_row():
    # k = 16: 2^16 rounding choices; compare with an independent enumeration
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((1, 16)) * 0.02).astype(F32)
    X = rng.standard_normal((32, 16)).astype(F32)
    lo, rtn_loss = oracle.bruteforce_min_loss(W, X, 4, 16)
    assert lo <= rtn_loss
    # random offsets never beat the exhaustive minimum
    for s in range(20):
        V = np.random.default_rng(s).uniform(-0.5, 0.5, (1, 16)).astype(F32)
        L = oracle.loss_and_grads(W, X, V, np.ones((1, 1), F32), np.ones((1, 1), F32), 4, 16)["L"]
        assert lo <= L + 1e-15


def test_snapshot_strict_less_keeps_first_minimum():
    # with lr 0 the state never changes: every loss ties, the first wins
    W, X = _tiny(3)
    res = oracle.tune_layer(W, X, np.zeros((5, 1), np.int32), 4, 12, 5, lr=0.0)
    assert res["best_step"] == 0
    assert np.all(res["losses"] == res["losses"][0])


def test_pack_roundtrip_and_bytes():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 16, size=(7, 64)).astype(F32)
    p = oracle.pack_int4(q)
    assert p.shape == (7, 32) and p.dtype == np.uint8
    np.testing.assert_array_equal(oracle.unpack_int4(p), q.astype(np.uint8))
    # low nibble = even column
    assert p[0, 0] == (int(q[0, 0]) | (int(q[0, 1]) << 4))
    # coordinates page bytes formula: P*b/8 + scale + zero-point metadata
    assert oracle.packed_bytes(4096, 4096, 128) == 4096 * 4096 // 2 + 4096 * 32 * 5
    assert oracle.packed_bytes(256, 256, 32) == 32768 + 8192 + 2048
