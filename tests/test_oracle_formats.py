"""Float-format QDQ oracle (FP8 E4M3, MXFP4) pinned to the formats'
definitions: value tables (largest finite value, smallest subnormal, count),
torch's float8_e4m3fn cast on in-range values, hand-worked E2M1 ties,
saturation, and the error and scale properties of the group / block QDQ."""
import numpy as np
import pytest
import torch

from oracle import float_formats as ff

F32 = np.float32


def test_e4m3_table_matches_the_format():
    codes, vals = ff.e4m3_table()
    assert len(vals) == 127 and vals[0] == 0.0
    assert vals.max() == 448.0 and vals[1] == 2.0 ** -9
    assert np.all(np.diff(vals) > 0)                  # monotone in the code
    # every value is what torch's float8_e4m3fn encodes for that bit pattern
    t = torch.tensor(codes.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(t, vals.astype(F32))


def test_e4m3_rounding_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 40.0)]).astype(F32)
    x = x[np.abs(x) <= 448]
    # exact midpoints between neighbouring values: ties go to the even code
    _, vals = ff.e4m3_table()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(F32)
    x = np.concatenate([x, mids, -mids])
    v, _ = ff.e4m3_round(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(v.astype(F32), ref)


def test_e4m3_saturates_and_codes_carry_the_sign():
    v, c = ff.e4m3_round(np.array([1000.0, -500.0, 448.0, 464.0, -0.0], F32))
    np.testing.assert_array_equal(v, [448.0, -448.0, 448.0, 448.0, 0.0])
    assert list(c[:2]) == [0x7E, 0xFE]


def test_e2m1_values_and_hand_worked_ties():
    _, vals = ff.e2m1_table()
    np.testing.assert_array_equal(vals, [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.3, -2.6], F32)
    v, c = ff.e2m1_round(x)
    np.testing.assert_array_equal(v, [0, 1, 1, 2, 2, 4, 4, 6, 6, -0.5, -3])
    assert c[-1] == (0x8 | 5)


def test_fp8_group_qdq_error_bound_and_extremes():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(F32)
    W[3, 5] = 0.9
    r = ff.qdq_fp8_e4m3(W, 64)
    s = np.repeat(r["s"], 64, axis=1)
    x = np.abs(W / s)
    # relative error of E4M3 rounding: at most half a step, 2^-4 of the binade
    # for normal values, half of 2^-9 below them
    step = np.where(x >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(x, 1e-30))) - 3), 2.0 ** -9)
    assert np.all(np.abs(W - r["w_hat"]) <= (0.5 * step) * s * (1 + 1e-6) + 1e-12)
    # the group maximum maps to 448 and dequantizes back to (nearly) itself
    amax = np.abs(W).reshape(16, 4, 64).max(axis=2)
    np.testing.assert_allclose(np.abs(r["w_hat"]).reshape(16, 4, 64).max(axis=2), amax, rtol=2e-7)


def test_mxfp4_block_scale_is_a_power_of_two_placing_the_maximum_in_4_to_8():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((8, 128)) * 0.05).astype(F32)
    W[0, :32] = 0.0
    r = ff.qdq_mxfp4(W)
    s = r["s"]
    assert np.all(np.log2(s) == np.round(np.log2(s)))
    np.testing.assert_array_equal(r["scale_bits"].astype(np.int64) - 127, np.log2(s).astype(np.int64))
    amax = np.abs(W).reshape(8, 4, 32).max(axis=2)
    ratio = amax[amax > 0] / s[amax > 0]
    assert np.all((ratio >= 4) & (ratio < 8))
    codes_mag = np.abs(r["w_hat"]).reshape(8, 4, 32) / s[:, :, None]
    assert codes_mag.max() <= 6
    assert np.all(r["w_hat"][0, :32] == 0)


def test_clip_factor_shrinks_the_scale():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((4, 64)) * 0.02).astype(F32)
    a = ff.qdq_fp8_e4m3(W, 32, alpha=np.full((4, 2), 0.5, F32))
    b = ff.qdq_fp8_e4m3(W, 32)
    np.testing.assert_array_equal(a["s"], (np.float32(0.5) * np.abs(W).reshape(4, 2, 32).max(axis=2)
                                          / np.float32(448)).astype(F32))
    assert np.all(a["s"] < b["s"])
