"""GPU parity of the INT4-weight GEMM (ar_w4a16_gemm) against the oracle:
bit-exact where every partial sum is exact in fp32, within the fp32
accumulation bound otherwise, on ragged tiles, every group size class, the
decode-sized and the full 2048 x 4096 x 4096 problem, and on the packed output
of ar_pack_int4."""
import numpy as np
import pytest
import torch

import oracle
from synthetic_inputs import make_weight, to_bf16_values

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.fixture(scope="module")
def ar():
    import post_weight_quantization_autoround_amd as mod
    assert torch.cuda.is_available()
    return mod


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(dtype) if dtype is not None else t


def _exact_case(m, n, k, g, seed):
    """Integer activations and power-of-two scales: every product and partial
    sum is a multiple of 1/8 below 2^17, so fp32 sums are exact in any order."""
    rng = np.random.default_rng(seed)
    g = k if g == -1 else g
    X = rng.integers(-8, 9, (m, k)).astype(F32)
    q = rng.integers(0, 16, (n, k)).astype(np.uint8)
    G = k // g
    scale = np.full((n, G), 0.125, F32)
    zero = rng.integers(0, 16, (n, G)).astype(np.uint8)
    return X, oracle.pack_int4(q), scale, zero


@pytest.mark.parametrize("m,n,k,g", [
    (300, 200, 512, 128),     # ragged in M and N, two tiles each way
    (256, 128, 256, 64),      # exactly one tile
    (64, 384, 640, 32),       # two groups per k-step
    (17, 130, 1024, 1024),    # one group per row (g = K)
    (1, 64, 128, 8),          # decode row, smallest group
    (33, 96, 192, 24),        # group not a power of two
    # at most 16 rows, K a multiple of 128: the decode kernel, X straight into registers
    (1, 4096, 4096, 128),
    (16, 200, 1024, 128),     # ragged N
    (7, 48, 768, 32),         # four groups per 128-wide super-step
    (3, 32, 256, 128),        # fewer super-steps than wavefronts
    (16, 48, 2048, 32),       # four groups per super-step
    (5, 40, 1536, 24),        # group not a power of two, ragged N
    (12, 64, 4096, 256),      # one round of super-steps
    (16, 32, 4608, 128),      # 36 super-steps: a second, partial round
    (2, 24, 10240, -1),       # one group per row, three rounds
    (9, 8200, 512, 64),       # two 16-row tiles per workgroup, the last one past N
    (16, 16400, 256, 128),    # four tiles per workgroup (8 wavefronts), ragged last workgroup
    (3, 16448, 128, 32),      # the same with one group per lane and super-step (g32)
    (4, 16448, 2304, 128),    # four tiles per workgroup, 18 super-steps: rounds of 8, 8 and 2
    # 17..64 rows, K a multiple of 128: the streaming kernel
    (29, 64, 2048, 256),      # two 16-row blocks of X
    (64, 80, 384, 24),        # four 16-row blocks, non-power-of-two group
    (50, 16, 8192, -1),       # one group per row, K spread over all wavefronts
    (17, 24, 2048, 128),      # one row past 16
])
def test_exact_sums_bit_exact(ar, m, n, k, g):
    X, packed, scale, zero = _exact_case(m, n, k, g, m + n + k)
    ref = oracle.w4a16_matmul(X, packed, scale, zero, k if g == -1 else g)
    Xd = _dev(X, torch.bfloat16)
    y = ar.w4a16_gemm(Xd, _dev(packed), _dev(scale), _dev(zero), group_size=g)
    y16 = ar.w4a16_gemm(Xd, _dev(packed), _dev(scale), _dev(zero), group_size=g, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref.astype(F32))
    np.testing.assert_array_equal(y16.float().cpu().numpy().view(np.uint32),
                                  oracle.bf16_round(ref.astype(F32)).view(np.uint32))


@pytest.mark.parametrize("m", [1, 16])
def test_codes_not_16_byte_aligned(ar, m):
    # packed rows 4-byte but not 16-byte aligned: the tiled kernel, which
    # loads codes 4 bytes at a time, takes batches of up to 16 rows too
    n, k, g = 40, 1024, 128
    X, packed, scale, zero = _exact_case(m, n, k, g, 5 + m)
    ref = oracle.w4a16_matmul(X, packed, scale, zero, g)
    buf = torch.zeros(n * k // 2 + 4, dtype=torch.uint8, device="cuda")
    view = buf[4:].view(n, k // 2)
    view.copy_(_dev(packed))
    assert view.data_ptr() % 16 == 4
    y = ar.w4a16_gemm(_dev(X, torch.bfloat16), view, _dev(scale), _dev(zero), group_size=g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref.astype(F32))


def _tuned_layer(n, k, g, seed):
    rng = np.random.default_rng(seed)
    W = to_bf16_values(make_weight(rng, n, k))
    V = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
    al = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    be = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    return W, V, al, be


def _within_accumulation_bound(y, ref, X, packed, scale, zero, g):
    k = X.shape[1]
    w_op = oracle.bf16_round(oracle.dequantize(oracle.unpack_int4(packed).astype(F32), scale,
                                               zero.astype(F32), g)).astype(np.float64)
    mag = np.abs(X.astype(np.float64)) @ np.abs(w_op).T
    bound = k * 2.0 ** -24 * mag + 1e-30
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= bound), float(np.max(err / bound))


def test_packed_output_of_the_quantizer(ar):
    m, n, k, g = 320, 256, 768, 128
    W, V, al, be = _tuned_layer(n, k, g, 11)
    packed, scale, zero = ar.pack_int4(_dev(W, torch.bfloat16), group_size=g, V=_dev(V), alpha=_dev(al),
                                       beta=_dev(be))
    rng = np.random.default_rng(12)
    X = rng.standard_normal((m, k)).astype(F32)
    X[:, rng.choice(k, 4, replace=False)] *= 50
    X = to_bf16_values(X)        # round after scaling: the GPU sees bf16 values
    y = ar.w4a16_gemm(_dev(X, torch.bfloat16), packed, scale, zero, group_size=g)
    torch.cuda.synchronize()
    p, s, z = packed.cpu().numpy(), scale.cpu().numpy(), zero.cpu().numpy()
    ref = oracle.w4a16_matmul(X, p, s, z, g)
    _within_accumulation_bound(y.cpu().numpy(), ref, X, p, s, z, g)
    # the same layer through the fake quantizer: X times bf16(w_hat)
    wq = oracle.qdq(W, V, al, be, 4, g)["w_hat"]
    np.testing.assert_array_equal(ref, X.astype(np.float64) @ oracle.bf16_round(wq).astype(np.float64).T)


@pytest.mark.parametrize("m", [16, 48])
def test_decode_batches_of_the_quantized_layer(ar, m):
    n, k, g = 1024, 4096, 128
    W, V, al, be = _tuned_layer(n, k, g, 21 + m)
    packed, scale, zero = ar.pack_int4(_dev(W, torch.bfloat16), group_size=g, V=_dev(V), alpha=_dev(al),
                                       beta=_dev(be))
    rng = np.random.default_rng(22)
    X = rng.standard_normal((m, k)).astype(F32)
    X[:, rng.choice(k, 8, replace=False)] *= 50
    X = to_bf16_values(X)
    y = ar.w4a16_gemm(_dev(X, torch.bfloat16), packed, scale, zero, group_size=g)
    torch.cuda.synchronize()
    p, s, z = packed.cpu().numpy(), scale.cpu().numpy(), zero.cpu().numpy()
    _within_accumulation_bound(y.cpu().numpy(), oracle.w4a16_matmul(X, p, s, z, g), X, p, s, z, g)


def test_full_size_sampled_rows(ar):
    # the 4096 x 4096 g128 layer on a 2048-token batch, as benchmarked; rows
    # of Y are independent, so sampled rows are checked against the oracle
    m, n, k, g = 2048, 4096, 4096, 128
    rng = np.random.default_rng(13)
    W = to_bf16_values(make_weight(rng, n, k))
    packed, scale, zero = ar.pack_int4(_dev(W, torch.bfloat16), group_size=g)
    X = to_bf16_values(rng.standard_normal((m, k)).astype(F32))
    y = ar.w4a16_gemm(_dev(X, torch.bfloat16), packed, scale, zero, group_size=g)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(m, 24, replace=False))
    p, s, z = packed.cpu().numpy(), scale.cpu().numpy(), zero.cpu().numpy()
    ref = oracle.w4a16_matmul(X[rows], p, s, z, g)
    _within_accumulation_bound(y.cpu().numpy()[rows], ref, X[rows], p, s, z, g)


def test_empty_batch_and_rejections(ar):
    k, n, g = 256, 64, 128
    packed = torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda")
    scale = torch.ones((n, k // g), dtype=torch.float32, device="cuda")
    zero = torch.zeros((n, k // g), dtype=torch.uint8, device="cuda")
    y = ar.w4a16_gemm(torch.zeros((0, k), dtype=torch.bfloat16, device="cuda"), packed, scale, zero, group_size=g)
    assert y.shape == (0, n)
    Xf = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ar.ARError) as e:
        ar.w4a16_gemm(Xf, torch.zeros((n, 48), dtype=torch.uint8, device="cuda"),
                      torch.ones((n, 3), device="cuda"), torch.zeros((n, 3), dtype=torch.uint8, device="cuda"),
                      group_size=32)
    assert e.value.status == ar.AR_ERR_UNSUPPORTED      # K = 96 is not a multiple of 64
