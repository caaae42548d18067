"""ar_qdq_rtn_noalloc (the fake quantizer for callers that cannot allocate:
its group-range buffer is the library's static per-GPU array) against
ar_qdq_rtn, through the C ABI: codes, scale, zero and w^ equal bit for bit
on two calls in a row, the second on a smaller input (the buffer keeps the
first call's contents), and again after an ordinary call in between; and
inside a captured graph, replayed several times."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ar():
    import post_weight_quantization_autoround_amd as mod
    assert torch.cuda.is_available()
    return mod


def _call(ar, fn, W, bits, g, V, al, be, sym, out_dt):
    N, K = W.shape
    G = K // (K if g == -1 else g)
    dev = W.device
    w_hat = torch.empty((N, K), dtype=out_dt, device=dev)
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    scale = torch.empty((N, G), dtype=torch.float32, device=dev)
    zero = torch.empty((N, G), dtype=torch.uint8, device=dev)
    q = ar.QConfig(bits, g, int(sym), ar.AR_FMT_INT)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = fn(W.data_ptr(), ar.AR_BF16 if W.dtype == torch.bfloat16 else ar.AR_F32, N, K, ctypes.byref(q),
            ptr(V), ptr(al), ptr(be), w_hat.data_ptr(), ar.AR_BF16 if out_dt == torch.bfloat16 else ar.AR_F32,
            codes.data_ptr(), scale.data_ptr(), zero.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == ar.AR_OK, ar.lib.ar_last_error().decode()
    return w_hat, codes, scale, zero


def _case(n, k, g, dtype, seed, params=True):
    rng = np.random.default_rng(seed)
    W = torch.from_numpy((rng.standard_normal((n, k)) * 0.02).astype(np.float32)).cuda().to(dtype)
    if not params:
        return W, None, None, None
    G = k // g
    V = torch.from_numpy(rng.uniform(-0.5, 0.5, (n, k)).astype(np.float32)).cuda()
    al = torch.from_numpy(rng.uniform(0.5, 1.0, (n, G)).astype(np.float32)).cuda()
    be = torch.from_numpy(rng.uniform(0.5, 1.0, (n, G)).astype(np.float32)).cuda()
    return W, V, al, be


def _same(a, b):
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and x.shape == y.shape
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y)


def test_noalloc_equals_allocating_entry_point_on_successive_calls(ar):
    cases = [
        # (N, K, group, dtype, bits, sym, output dtype, with V/alpha/beta)
        (4096, 4096, 128, torch.bfloat16, 4, False, torch.bfloat16, True),   # the 4096 x 4096 g128 layer
        (300, 640, 64, torch.float32, 3, True, torch.float32, True),         # smaller, ragged, symmetric
        (520, 256, 32, torch.bfloat16, 4, False, torch.float32, False),      # RTN, smaller still
    ]
    for i, (n, k, g, dt, bits, sym, odt, params) in enumerate(cases):
        print(f"noalloc case {i}: N={n} K={k} g={g} bits={bits} sym={sym}", flush=True)
        W, V, al, be = _case(n, k, g, dt, 30 + i, params)
        got = _call(ar, ar.lib.ar_qdq_rtn_noalloc, W, bits, g, V, al, be, sym, odt)
        ref = _call(ar, ar.lib.ar_qdq_rtn, W, bits, g, V, al, be, sym, odt)
        torch.cuda.synchronize()
        _same(got, ref)
    # the largest input the static buffer takes: 8 Mi groups (2 * N * G floats = 64 MiB)
    W, V, al, be = _case(8192, 8192, 8, torch.bfloat16, 40, params=False)
    got = _call(ar, ar.lib.ar_qdq_rtn_noalloc, W, 4, 8, None, None, None, False, torch.bfloat16)
    ref = _call(ar, ar.lib.ar_qdq_rtn, W, 4, 8, None, None, None, False, torch.bfloat16)
    torch.cuda.synchronize()
    _same(got, ref)


def test_noalloc_rejects_inputs_beyond_its_buffer(ar):
    W = torch.zeros((8192, 8200), dtype=torch.bfloat16, device="cuda")   # 8,396,800 groups of 8
    q = ar.QConfig(4, 8, 0, ar.AR_FMT_INT)
    out = torch.empty((8192, 8200), dtype=torch.uint8, device="cuda")
    st = ar.lib.ar_qdq_rtn_noalloc(W.data_ptr(), ar.AR_BF16, 8192, 8200, ctypes.byref(q), None, None, None, None,
                                   ar.AR_F32, out.data_ptr(), None, None, torch.cuda.current_stream().cuda_stream)
    assert st == ar.AR_ERR_OUT_OF_MEMORY
    assert "groups" in ar.lib.ar_last_error().decode()


def test_noalloc_inside_a_captured_graph(ar):
    # The callers it is for: captured once (its set-up done by an earlier
    # call), then replayed three times with eager work in between that
    # changes V and alpha in place; every replay equals ar_qdq_rtn on the
    # current inputs.
    W, V, al, be = _case(1024, 2048, 128, torch.bfloat16, 50)
    _call(ar, ar.lib.ar_qdq_rtn_noalloc, W, 4, 128, V, al, be, False, torch.bfloat16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        got = _call(ar, ar.lib.ar_qdq_rtn_noalloc, W, 4, 128, V, al, be, False, torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(51)
    for r in range(3):
        print(f"noalloc graph replay {r}", flush=True)
        V.copy_(torch.from_numpy(rng.uniform(-0.5, 0.5, tuple(V.shape)).astype(np.float32)))
        al.mul_(0.99).clamp_(0.5, 1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = _call(ar, ar.lib.ar_qdq_rtn, W, 4, 128, V, al, be, False, torch.bfloat16)
        torch.cuda.synchronize()
        _same(got, ref)
    del graph
