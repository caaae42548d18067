"""GPU parity of the float-format tensor-level QDQ (FP8 E4M3 per group,
MXFP4 blocks of 32) against the oracle: codes, scales, block exponents and
dequantized weights bit for bit, with and without a clip factor."""
import numpy as np
import pytest
import torch

from oracle import bf16_round
from oracle import float_formats as ff
from synthetic_inputs import make_weight, to_bf16_values

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


def _check(ar, W, bf16, g, fmt, bits, alpha, ref, zero_ref):
    kw = dict(bits=bits, group_size=g, fmt=fmt, alpha=None if alpha is None else _dev(alpha))
    out = ar.qdq_rtn(_dev(W, bf16), out_dtype=torch.float32, **kw)
    out16 = ar.qdq_rtn(_dev(W, bf16), out_dtype=torch.bfloat16, codes=False, scale_zero=False, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["codes"].cpu().numpy(), ref["codes"])
    np.testing.assert_array_equal(out["scale"].cpu().numpy().view(np.uint32), ref["s"].view(np.uint32))
    np.testing.assert_array_equal(out["zero"].cpu().numpy(), zero_ref)
    np.testing.assert_array_equal(out["w_hat"].cpu().numpy().view(np.uint32), ref["w_hat"].view(np.uint32))
    np.testing.assert_array_equal(out16["w_hat"].float().cpu().numpy().view(np.uint32),
                                  bf16_round(ref["w_hat"]).view(np.uint32))


@pytest.mark.parametrize("n,k,g,bf16,clip", [
    (64, 256, 32, False, False),
    (128, 1024, 128, True, True),
    (37, 384, -1, True, False),
])
def test_fp8_e4m3_bit_exact(ar, n, k, g, bf16, clip):
    rng = np.random.default_rng(n + k)
    W = make_weight(rng, n, k)
    W[0, :8] = [0.0, -0.0, 1e-9, -3e-6, 0.5, -0.5, 0.25, 7.0]
    W = to_bf16_values(W) if bf16 else W
    gg = k if g == -1 else g
    alpha = rng.uniform(0.5, 1.0, (n, k // gg)).astype(F32) if clip else None
    ref = ff.qdq_fp8_e4m3(W, gg, alpha)
    _check(ar, W, bf16, g, ar.AR_FMT_FP8_E4M3, 8, alpha, ref, np.zeros((n, k // gg), np.uint8))


@pytest.mark.parametrize("n,k,bf16,clip", [(64, 256, False, False), (96, 2048, True, True)])
def test_mxfp4_bit_exact(ar, n, k, bf16, clip):
    rng = np.random.default_rng(k)
    W = make_weight(rng, n, k)
    W[1, :32] = 0.0                      # an all-zero block
    W = to_bf16_values(W) if bf16 else W
    alpha = rng.uniform(0.5, 1.0, (n, k // 32)).astype(F32) if clip else None
    ref = ff.qdq_mxfp4(W, alpha)
    _check(ar, W, bf16, 32, ar.AR_FMT_MXFP4, 4, alpha, ref, ref["scale_bits"])
