"""GPU parity of the fake quantizer and the INT4 pack against the oracle:
bit-exact codes, scales, zero-points and dequantized weights (fp32 and the
bf16 rounding), for RTN and for arbitrary (V, alpha, beta) states."""
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


def _w(n, k, seed, bf16):
    w = make_weight(np.random.default_rng(seed), n, k)
    return to_bf16_values(w) if bf16 else w


def _to_dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if bf16 else t


def _compare(ar, W, bits, g, V=None, al=None, be=None, bf16_in=False, sym=False):
    n, k = W.shape
    G = k // (k if g == -1 else g)
    gg = k if g == -1 else g
    Vn = np.zeros_like(W) if V is None else V
    aln = np.ones((n, G), F32) if al is None else al
    ben = np.ones((n, G), F32) if be is None else be
    ref = oracle.qdq(W, Vn, aln, ben, bits, gg, sym=sym)
    Wd = _to_dev(W, bf16_in)
    kw = dict(V=None if V is None else _to_dev(V), alpha=None if al is None else _to_dev(al),
              beta=None if be is None else _to_dev(be))
    out = ar.qdq_rtn(Wd, bits=bits, group_size=g, out_dtype=torch.float32, sym=sym, **kw)
    out16 = ar.qdq_rtn(Wd, bits=bits, group_size=g, out_dtype=torch.bfloat16, codes=False, scale_zero=False,
                       sym=sym, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["codes"].cpu().numpy(), ref["q"].astype(np.uint8))
    np.testing.assert_array_equal(out["scale"].cpu().numpy().view(np.uint32), ref["s"].view(np.uint32))
    np.testing.assert_array_equal(out["zero"].cpu().numpy(), ref["z"].astype(np.uint8))
    np.testing.assert_array_equal(out["w_hat"].cpu().numpy().view(np.uint32), ref["w_hat"].view(np.uint32))
    got16 = out16["w_hat"].float().cpu().numpy()
    np.testing.assert_array_equal(got16.view(np.uint32), oracle.bf16_round(ref["w_hat"]).view(np.uint32))
    return ref


@pytest.mark.parametrize("n,k,g,bits,bf16", [
    (256, 256, 32, 4, False),      # the 256 x 256 fp32 g32 validation layer
    (512, 1024, 128, 4, True),     # bf16 g128
    (37, 384, 128, 4, True),       # ragged row count
    (64, 256, -1, 4, False),       # one group per row
    (64, 200, 40, 3, False),       # group not a power of two
    (32, 128, 8, 2, True),
    (32, 128, 64, 8, False),
])
def test_rtn_bit_exact(ar, n, k, g, bits, bf16):
    W = _w(n, k, n * 1000 + k, bf16)
    _compare(ar, W, bits, g, bf16_in=bf16)


def test_rtn_bit_exact_full_4096_bf16_g128(ar):
    W = _w(4096, 4096, 1, True)
    _compare(ar, W, 4, 128, bf16_in=True)


@pytest.mark.parametrize("seed", [0, 1])
def test_random_states_bit_exact(ar, seed):
    n, k, g = 128, 512, 128
    rng = np.random.default_rng(seed)
    W = _w(n, k, seed + 7, True)
    V = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
    al = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    be = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    ref = _compare(ar, W, 4, g, V, al, be, bf16_in=True)
    # the states exercise clipping at both ends
    assert np.any(ref["t"] < 0) and np.any(ref["t"] > 15)


def test_edge_groups(ar):
    # all-zero groups, single-sign groups, exact zeros, blog sec. 2 example row
    W = np.zeros((4, 64), F32)
    W[1, :32] = np.abs(_w(1, 32, 3, False))       # only positive
    W[2, 32:] = -np.abs(_w(1, 32, 4, False))      # only negative
    W[3, :4] = [0.1, 0.2, 0.15, 8.0]
    ref = _compare(ar, W, 4, 32)
    assert np.all(ref["w_hat"][0] == 0)
    assert ref["w_hat"][3, 3] == F32(8.0)


def test_pack_bit_exact_and_roundtrip(ar):
    n, k, g = 256, 512, 128
    rng = np.random.default_rng(3)
    W = _w(n, k, 9, True)
    V = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
    al = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    be = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    ref = oracle.qdq(W, V, al, be, 4, g)
    packed, scale, zero = ar.pack_int4(_to_dev(W, True), group_size=g, V=_to_dev(V), alpha=_to_dev(al),
                                       beta=_to_dev(be))
    torch.cuda.synchronize()
    p = packed.cpu().numpy()
    np.testing.assert_array_equal(p, oracle.pack_int4(ref["q"]))
    np.testing.assert_array_equal(scale.cpu().numpy().view(np.uint32), ref["s"].view(np.uint32))
    np.testing.assert_array_equal(zero.cpu().numpy(), ref["z"].astype(np.uint8))
    # dequantizing the packed form reproduces the fake-quantized weight bit for bit
    q = oracle.unpack_int4(p).astype(F32)
    wh = oracle.dequantize(q, scale.cpu().numpy(), zero.cpu().numpy().astype(F32), g)
    np.testing.assert_array_equal(wh.view(np.uint32), ref["w_hat"].view(np.uint32))
    assert p.nbytes + scale.numel() * 4 + zero.numel() == oracle.packed_bytes(n, k, g)


@pytest.mark.parametrize("n,k,g,bits,bf16", [
    (256, 256, 32, 4, False),
    (512, 1024, 128, 4, True),
    (37, 384, 128, 3, True),
    (64, 256, -1, 8, False),
])
def test_symmetric_rtn_bit_exact(ar, n, k, g, bits, bf16):
    W = _w(n, k, n + k + 17, bf16)
    ref = _compare(ar, W, bits, g, bf16_in=bf16, sym=True)
    assert np.all(ref["z"] == 2 ** (bits - 1))


def test_symmetric_random_states_bit_exact(ar):
    n, k, g = 128, 512, 64
    rng = np.random.default_rng(21)
    W = _w(n, k, 23, True)
    V = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
    al = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    be = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)   # unused by the symmetric scale
    ref = _compare(ar, W, 4, g, V, al, be, bf16_in=True, sym=True)
    assert np.any(ref["t"] > 15) or np.any(ref["t"] < 0)


def test_symmetric_pack_bit_exact(ar):
    n, k, g = 64, 256, 32
    W = _w(n, k, 31, True)
    ref = oracle.rtn(W, 4, g, sym=True)
    packed, scale, zero = ar.pack_int4(_to_dev(W, True), group_size=g, sym=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(packed.cpu().numpy(), oracle.pack_int4(ref["q"]))
    np.testing.assert_array_equal(scale.cpu().numpy().view(np.uint32), ref["s"].view(np.uint32))
    assert np.all(zero.cpu().numpy() == 8)
