"""Oracle of the INT4-weight GEMM pinned to closed forms (identity and
scaled-identity weights, an all-zero-point layer) and to the fake-quantized
product it must equal (the QDQ-versus-real-INT4 comparison of the AutoRound
blog, sec. 4)."""
import numpy as np

import oracle
from synthetic_inputs import make_weight, to_bf16_values

F32 = np.float32


def _x(m, k, seed):
    return to_bf16_values(np.random.default_rng(seed).standard_normal((m, k)).astype(F32))


def test_identity_codes_reproduce_the_activations():
    # one group per row, z = 8, s = 1, code 9 on the diagonal: w = I
    n = k = 16
    q = np.full((n, k), 8, np.uint8)
    np.fill_diagonal(q, 9)
    scale = np.ones((n, 1), F32)
    zero = np.full((n, 1), 8, np.uint8)
    X = _x(5, k, 0)
    Y = oracle.w4a16_matmul(X, oracle.pack_int4(q), scale, zero, k)
    np.testing.assert_array_equal(Y, X.astype(np.float64))


def test_scaled_permutation_and_negative_codes():
    # code 8 - 4 = -4 times s = 0.25 on a permutation: Y = -X[:, perm]
    n = k = 32
    perm = np.random.default_rng(1).permutation(k)
    q = np.full((n, k), 8, np.uint8)
    q[np.arange(n), perm] = 4
    X = _x(7, k, 2)
    Y = oracle.w4a16_matmul(X, oracle.pack_int4(q), np.full((n, 2), 0.25, F32), np.full((n, 2), 8, np.uint8), 16)
    np.testing.assert_array_equal(Y, -X[:, perm].astype(np.float64))


def test_codes_at_the_zero_point_give_zero():
    n, k, g = 8, 64, 32
    rng = np.random.default_rng(3)
    z = rng.integers(0, 16, (n, k // g)).astype(np.uint8)
    q = np.repeat(z, g, axis=1)
    s = rng.uniform(0.01, 1.0, (n, k // g)).astype(F32)
    Y = oracle.w4a16_matmul(_x(4, k, 4), oracle.pack_int4(q), s, z, g)
    assert np.all(Y == 0.0)


def test_equals_x_times_the_bf16_fake_quantized_weight():
    # the packed layer and the quantizer's w_hat describe the same weight
    n, k, g = 48, 256, 64
    rng = np.random.default_rng(5)
    W = to_bf16_values(make_weight(rng, n, k))
    V = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
    al = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    be = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    r = oracle.qdq(W, V, al, be, 4, g)
    X = _x(9, k, 6)
    Y = oracle.w4a16_matmul(X, oracle.pack_int4(r["q"]), r["s"], r["z"].astype(np.uint8), g)
    ref = X.astype(np.float64) @ oracle.bf16_round(r["w_hat"]).astype(np.float64).T
    np.testing.assert_array_equal(Y, ref)
    # and differs from the unquantized product by the quantization error only
    err = np.abs(Y - X.astype(np.float64) @ W.astype(np.float64).T)
    bound = np.abs(X).astype(np.float64) @ np.repeat(r["s"], g, axis=1).astype(np.float64).T
    assert np.all(err <= bound)
