"""Oracle pinned to the worked examples the AutoRound blog prints
(fixtures in tests/golden/blog_worked_examples.json, each with its citation)."""
import json
import os

import numpy as np
import pytest

import oracle

F32 = np.float32
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "blog_worked_examples.json")))


def test_strategy_a_outlier_collapses_small_values():
    ex = GOLD["strategy_a"]
    W = np.asarray([ex["W"]], F32)
    r = oracle.rtn(W, ex["bits"], g=4)
    assert abs(float(r["s"][0, 0]) - ex["scale_approx"]) < 1e-3
    # the page's dequantized result, exactly
    np.testing.assert_array_equal(r["w_hat"][0], np.asarray(ex["w_hat"], F32))
    np.testing.assert_array_equal(r["q"][0], [0, 0, 0, 15])


def test_strategy_a_needs_zero_inclusive_range():
    # Plain min/max (no zero) would give scale (8.0-0.1)/15 and dequantize 8.0
    # to something other than 8.0 -- contradicting the page; the zero-inclusive
    # range reproduces it.  This pins the reading, not just the arithmetic.
    ex = GOLD["strategy_a"]
    W = np.asarray(ex["W"], F32)
    s_plain = F32((W.max() - W.min()) / F32(15))
    z_plain = np.rint(F32(-W.min() / s_plain))
    q_plain = np.clip(np.rint(W / s_plain) + z_plain, 0, 15)
    w_plain = s_plain * (q_plain - z_plain)
    assert w_plain[3] != F32(8.0)


def test_strategy_b_clipping():
    ex = GOLD["strategy_b"]
    W = np.asarray([ex["W"]], F32)
    mx, mn = oracle.group_range(W, 4)
    alpha = np.asarray([[ex["clip_max"] / 8.0]], F32)      # 0.075: wmax = 0.6
    beta = np.ones((1, 1), F32)
    wmax, wmin, s, z = oracle.group_scale_zero(mx, mn, alpha, beta, ex["bits"])
    assert float(wmax[0, 0]) == pytest.approx(0.6, abs=1e-7)
    assert float(s[0, 0]) == pytest.approx(ex["scale_approx"], abs=1e-7)
    r = oracle.qdq(W, np.zeros_like(W), alpha, beta, ex["bits"], 4)
    wh = r["w_hat"][0]
    assert any(abs(float(wh[0]) - a) < 1e-6 for a in ex["element0_accepted"])
    np.testing.assert_allclose(wh[1:], ex["w_hat_approx"][1:], atol=1e-6)
    assert float(W[0, 3] - wh[3]) == pytest.approx(ex["outlier_clip_error"], abs=1e-6)


def test_clipping_panel():
    ex = GOLD["clipping_panel"]
    # a group whose range is [0, 0.95] clipped at 0.6
    W = np.asarray([[0.0, 0.3, 0.5, ex["value"]]], F32)
    alpha = np.asarray([[F32(ex["clip_max"]) / F32(ex["value"])]], F32)
    r = oracle.qdq(W, np.zeros_like(W), alpha, np.ones((1, 1), F32), ex["bits"], 4)
    assert float(r["w_hat"][0, 3]) == pytest.approx(ex["w_hat"], abs=1e-6)
    assert float(W[0, 3] - r["w_hat"][0, 3]) == pytest.approx(ex["error"], abs=1e-6)
    assert float(r["q"][0, 3]) == 15


def test_zero_point_example():
    ex = GOLD["zero_point"]
    W = np.asarray([[ex["w"]]], F32)
    s = np.asarray([[ex["scale"]]], F32)
    z = np.asarray([[ex["zero"]]], F32)
    t, q = oracle.quantize_codes(W, np.zeros_like(W), s, z, ex["bits"], 1)
    assert float(t[0, 0]) == 15.0   # round(7.4) + 8, not yet clamped
    assert float(q[0, 0]) == ex["q"]
    wh = oracle.dequantize(q, s, z, 1)
    assert float(wh[0, 0]) == pytest.approx(ex["w_hat"], abs=1e-6)
    assert float(W[0, 0] - wh[0, 0]) == pytest.approx(ex["delta"], abs=1e-6)


def test_zero_point_added_after_rounding():
    # round(W/s) + z and round(W/s + z) differ in fp32 near ties: the page's
    # order (zero added to the rounded value) is the one implemented.
    # W = 0.07499999, s = 0.05: W/s = 1.4999998 -> 1, + 4 = 5; adding the
    # zero first gives fl(5.4999998) = 5.5 -> 6.
    W = np.asarray([[0.07499999]], F32)
    s = np.asarray([[0.05]], F32)
    z = np.asarray([[4.0]], F32)
    _, q = oracle.quantize_codes(W, np.zeros_like(W), s, z, 4, 1)
    assert float(q[0, 0]) == 5.0


def test_offset_3_3_example():
    ex = GOLD["offset_3_3"]
    W = np.asarray([[ex["u"]]], F32)
    s = np.ones((1, 1), F32)
    z = np.zeros((1, 1), F32)
    for v, code in [(0.0, ex["code_v0"]), (0.19, ex["code_v0"]), (0.2, ex["code_up"]),
                    (0.5, ex["code_up"]), (-0.5, 3)]:
        _, q = oracle.quantize_codes(W, np.full_like(W, v), s, z, 8, 1)
        assert float(q[0, 0]) == code, v
    wh0 = oracle.dequantize(np.asarray([[3.0]], F32), s, z, 1)
    wh1 = oracle.dequantize(np.asarray([[4.0]], F32), s, z, 1)
    assert abs(float(W[0, 0] - wh0[0, 0])) == pytest.approx(ex["error_v0"], abs=1e-6)
    assert abs(float(W[0, 0] - wh1[0, 0])) == pytest.approx(ex["error_up"], abs=1e-6)


def test_presets_table_lr():
    ex = GOLD["presets"]
    assert ex["lr"] == 0.005
    # linear decay starts at the preset lr and ends one step above zero
    lrs = oracle.lr_table(ex["lr"], ex["default"][1])
    assert lrs[0] == F32(0.005)
    assert lrs[-1] == F32(0.005 / 200)
