"""C-ABI contract on the CPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call
(so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libautoround.h")
LIB = os.path.join(ROOT, "post_weight_quantization_autoround_amd", "libautoround.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libautoround.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"AR_API\s+[\w\s\*]+?\b(ar_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ["ar_qdq_rtn", "ar_tune_layer", "ar_tune_block", "ar_pack_int4", "ar_layer_grads", "ar_w4a16_gemm",
                     "ar_tuner_create", "ar_tuner_run", "ar_tuner_finish", "ar_tuner_destroy",
                     "ar_last_error", "ar_version", "ar_tune_opts_init"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for name in _declared():
        assert hasattr(lib, name), name


def _ar():
    import post_weight_quantization_autoround_amd as ar
    return ar


def test_version_and_presets():
    ar = _ar()
    assert "gfx950" in ar.version()
    d = ar.default_opts(ar.AR_PRESET_DEFAULT)
    assert (d.batch_samples, d.iters) == (8, 200) and abs(d.lr - 0.005) < 1e-9
    assert (ar.default_opts(ar.AR_PRESET_BEST).iters, ar.default_opts(ar.AR_PRESET_LIGHT).iters) == (1000, 50)
    assert ar.default_opts(ar.AR_PRESET_FAST).batch_samples == 4
    with pytest.raises(ar.ARError) as e:
        ar.default_opts(7)
    assert e.value.status == ar.AR_ERR_INVALID_ARG


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: checks fail first


def _q(bits=4, g=128, sym=0):
    ar = _ar()
    return ar.QConfig(bits, g, sym)


@pytest.mark.parametrize("N,K,bits,g,sym,expect", [
    (0, 128, 4, 128, 0, 1),        # empty
    (16, 128, 1, 128, 0, 1),       # bits out of range
    (16, 128, 9, 128, 0, 1),
    (16, 130, 4, 128, 0, 1),       # group does not divide K
    (16, 120, 4, 12, 0, 2),        # group not a multiple of 8
    (16, 128, 4, 0, 0, 1),
    (16, 128, 4, 128, 2, 1),       # sym must be 0 or 1
])
def test_qdq_rejects_bad_arguments(N, K, bits, g, sym, expect):
    ar = _ar()
    q = _q(bits, g, sym)
    st = ar.lib.ar_qdq_rtn(FAKE, ar.AR_BF16, N, K, ctypes.byref(q), None, None, None, FAKE, ar.AR_F32,
                           None, None, None, None)
    assert st == expect
    assert ar.lib.ar_last_error().decode()


def test_noalloc_qdq_checks_arguments_and_its_limit_on_the_host():
    ar = _ar()
    q = _q(4, 8)
    # 8192 x 8200 with g8: 8,396,800 groups > the static buffer's 8,388,608
    st = ar.lib.ar_qdq_rtn_noalloc(FAKE, ar.AR_BF16, 8192, 8200, ctypes.byref(q), None, None, None, FAKE, ar.AR_F32,
                                   None, None, None, None)
    assert st == ar.AR_ERR_OUT_OF_MEMORY
    assert "groups" in ar.lib.ar_last_error().decode()
    q = _q(9, 128)
    assert ar.lib.ar_qdq_rtn_noalloc(FAKE, ar.AR_BF16, 16, 128, ctypes.byref(q), None, None, None, FAKE, ar.AR_F32,
                                     None, None, None, None) == ar.AR_ERR_INVALID_ARG


def test_qdq_rejects_null_weight():
    ar = _ar()
    q = _q()
    assert ar.lib.ar_qdq_rtn(None, ar.AR_BF16, 4, 128, ctypes.byref(q), None, None, None, FAKE, ar.AR_F32,
                             None, None, None, None) == ar.AR_ERR_INVALID_ARG
    assert ar.lib.ar_qdq_rtn(FAKE, ar.AR_BF16, 4, 128, None, None, None, None, FAKE, ar.AR_F32,
                             None, None, None, None) == ar.AR_ERR_INVALID_ARG


def test_pack_needs_four_bits_and_outputs():
    ar = _ar()
    q = _q(bits=3)
    assert ar.lib.ar_pack_int4(FAKE, ar.AR_BF16, 4, 128, ctypes.byref(q), None, None, None, FAKE, FAKE, FAKE,
                               None) == ar.AR_ERR_INVALID_ARG
    q = _q()
    assert ar.lib.ar_pack_int4(FAKE, ar.AR_BF16, 4, 128, ctypes.byref(q), None, None, None, None, FAKE, FAKE,
                               None) == ar.AR_ERR_INVALID_ARG


def _tune(ar, **kw):
    args = dict(W=FAKE, wt=ar.AR_BF16, N=64, K=128, X=FAKE, xt=ar.AR_BF16, S=4, T=64)
    args.update(kw)
    o = kw.pop("opts", None) or ar.default_opts()
    q = kw.pop("q", None) or _q()
    bl = ctypes.c_float()
    bs = ctypes.c_int32()
    return ar.lib.ar_tune_layer(args["W"], args["wt"], args["N"], args["K"], args["X"], args["xt"], args["S"],
                                args["T"], ctypes.byref(q), ctypes.byref(o), FAKE, FAKE, FAKE,
                                ctypes.byref(bl), ctypes.byref(bs), None)


def test_tune_rejects_bad_problems():
    ar = _ar()
    o = ar.default_opts()
    o.batch_samples = 2
    assert _tune(ar, T=48, opts=o) == ar.AR_ERR_UNSUPPORTED          # T not a multiple of 64
    assert _tune(ar, S=0, opts=o) == ar.AR_ERR_INVALID_ARG
    assert _tune(ar, X=None, opts=o) == ar.AR_ERR_INVALID_ARG
    assert _tune(ar, wt=ar.AR_F32, opts=o) == ar.AR_ERR_UNSUPPORTED  # bf16 GEMMs need bf16 inputs
    o2 = ar.default_opts()
    o2.batch_samples = 5                                             # > S
    assert _tune(ar, opts=o2) == ar.AR_ERR_INVALID_ARG
    o3 = ar.default_opts()
    o3.batch_samples = 2
    o3.clip_lo, o3.clip_hi = 1.0, 0.5
    assert _tune(ar, opts=o3) == ar.AR_ERR_INVALID_ARG
    o4 = ar.default_opts()
    o4.batch_samples = 2
    o4.lr = -1.0
    assert _tune(ar, opts=o4) == ar.AR_ERR_INVALID_ARG


def test_resume_options_default_and_checks():
    # start_step / best_loss_in (the resume point of an iters-step run)
    ar = _ar()
    d = ar.default_opts()
    assert d.start_step == 0 and d.best_loss_in == float("inf")
    for start, best, expect in [(-1, float("inf"), ar.AR_ERR_INVALID_ARG),
                                (201, float("inf"), ar.AR_ERR_INVALID_ARG),     # beyond iters = 200
                                (10, -1.0, ar.AR_ERR_INVALID_ARG),              # a loss is >= 0
                                (10, float("nan"), ar.AR_ERR_INVALID_ARG)]:
        o = ar.default_opts()
        o.batch_samples = 2
        o.start_step, o.best_loss_in = start, best
        assert _tune(ar, opts=o) == expect, (start, best)
        assert "start_step" in ar.lib.ar_last_error().decode() or "best_loss_in" in ar.lib.ar_last_error().decode()


def test_tune_rejects_schedule_out_of_range():
    ar = _ar()
    o = ar.default_opts()
    o.iters = 2
    o.batch_samples = 2
    sched = (ctypes.c_int32 * 4)(0, 1, 2, 4)     # 4 is outside [0, S=4)
    o.schedule = ctypes.cast(sched, ctypes.POINTER(ctypes.c_int32))
    assert _tune(ar, opts=o) == ar.AR_ERR_INVALID_ARG
    assert "schedule" in ar.lib.ar_last_error().decode()


def _block_call(ar, kind=0, wdt=1, H=128, F=256, T=64, g=64, mode=0, weights=True, sym=0):
    d = ar.BlockDesc()
    d.kind = kind
    d.weight_dtype = wdt
    d.hidden, d.ffn = H, F
    if weights:
        for i in range(3):
            d.weights[i] = FAKE.value
    q = ar.QConfig(4, g, sym)
    o = ar.default_opts()
    o.batch_samples = 2
    o.gemm_mode = mode
    arr = (ctypes.c_void_p * 3)(FAKE.value, FAKE.value, FAKE.value)
    bl = ctypes.c_float()
    bs = ctypes.c_int32()
    return ar.lib.ar_tune_block(ctypes.byref(d), FAKE, 1, 4, T, ctypes.byref(q), ctypes.byref(o), arr, arr, arr,
                                None, ctypes.byref(bl), ctypes.byref(bs), None)


def test_tune_block_checks_arguments_on_the_host():
    ar = _ar()
    assert _block_call(ar, kind=1) == ar.AR_ERR_INVALID_ARG          # a decoder needs all seven weights
    assert "NULL" in ar.lib.ar_last_error().decode()
    assert _block_call(ar, kind=5) == ar.AR_ERR_INVALID_ARG
    assert _block_call(ar, weights=False) == ar.AR_ERR_INVALID_ARG
    assert _block_call(ar, F=200) == ar.AR_ERR_INVALID_ARG           # group 64 does not divide ffn
    assert _block_call(ar, g=-1) == ar.AR_ERR_UNSUPPORTED            # per-channel differs between linears
    assert _block_call(ar, wdt=0) == ar.AR_ERR_UNSUPPORTED           # bf16 GEMMs need bf16 weights
    assert _block_call(ar, T=48) == ar.AR_ERR_UNSUPPORTED
    assert _block_call(ar, sym=3) == ar.AR_ERR_INVALID_ARG


def _decoder_call(ar, H=256, F=512, nq=4, nkv=2, d=64, T=128, g=64, mode=0, wdt=1, eps=1e-5, theta=1e4,
                  nweights=7, grads_ids=None):
    desc = ar.BlockDesc()
    desc.kind = ar.AR_BLOCK_LLAMA_DECODER
    desc.weight_dtype = wdt
    desc.hidden, desc.ffn, desc.heads, desc.kv_heads, desc.head_dim = H, F, nq, nkv, d
    desc.norm_eps, desc.rope_theta = eps, theta
    for i in range(nweights):
        desc.weights[i] = FAKE.value
    q = ar.QConfig(4, g, 0)
    arr = (ctypes.c_void_p * 7)(*([FAKE.value] * 7))
    if grads_ids is not None:
        ids = (ctypes.c_int32 * len(grads_ids))(*grads_ids)
        loss = ctypes.c_double()
        return ar.lib.ar_block_grads(ctypes.byref(desc), FAKE, 1, 4, T, ids, len(grads_ids), ctypes.byref(q), mode,
                                     arr, arr, arr, ctypes.byref(loss), None, None, None, None, None)
    o = ar.default_opts()
    o.batch_samples = 2
    o.gemm_mode = mode
    bl = ctypes.c_float()
    bs = ctypes.c_int32()
    return ar.lib.ar_tune_block(ctypes.byref(desc), FAKE, 1, 4, T, ctypes.byref(q), ctypes.byref(o), arr, arr, arr,
                                None, ctypes.byref(bl), ctypes.byref(bs), None)


def test_decoder_block_checks_arguments_on_the_host():
    ar = _ar()
    assert _decoder_call(ar, nweights=6) == ar.AR_ERR_INVALID_ARG     # w_down missing
    assert _decoder_call(ar, nq=3, nkv=2) == ar.AR_ERR_INVALID_ARG    # query heads not a multiple of KV heads
    assert _decoder_call(ar, eps=0.0) == ar.AR_ERR_INVALID_ARG
    assert _decoder_call(ar, theta=-1.0) == ar.AR_ERR_INVALID_ARG
    assert _decoder_call(ar, mode=1) == ar.AR_ERR_UNSUPPORTED         # bf16 GEMMs and attention only
    assert _decoder_call(ar, wdt=0) == ar.AR_ERR_UNSUPPORTED
    assert _decoder_call(ar, d=96) == ar.AR_ERR_UNSUPPORTED           # head size 64 or 128
    assert _decoder_call(ar, T=320) == ar.AR_ERR_UNSUPPORTED          # at most 256 tokens per sample
    assert _decoder_call(ar, T=96) == ar.AR_ERR_UNSUPPORTED           # whole 64-token query tiles
    assert _decoder_call(ar, F=200) == ar.AR_ERR_UNSUPPORTED
    assert _decoder_call(ar, g=-1) == ar.AR_ERR_UNSUPPORTED
    assert _decoder_call(ar, g=48) == ar.AR_ERR_INVALID_ARG           # group does not divide hidden
    assert _decoder_call(ar, grads_ids=[0, 4]) == ar.AR_ERR_INVALID_ARG   # sample id outside the pool
    assert _decoder_call(ar, grads_ids=[0], mode=1) == ar.AR_ERR_UNSUPPORTED


def _stack_call(ar, n=2, hidden=(128, 128), kinds=(0, 0), T=64, start_step=0, null_entry=None, nblocks=None):
    descs = (ar.BlockDesc * n)()
    for b in range(n):
        d = descs[b]
        d.kind = kinds[b]
        d.weight_dtype = 1
        d.hidden, d.ffn = hidden[b], 256
        d.heads, d.kv_heads, d.head_dim = 2, 1, 64
        d.norm_eps, d.rope_theta = 1e-5, 1e4
        for i in range(7 if kinds[b] == 1 else 3):
            d.weights[i] = FAKE.value
    q = ar.QConfig(4, 64, 0)
    o = ar.default_opts()
    o.batch_samples = 2
    o.start_step = start_step
    arr = (ctypes.c_void_p * (7 * n))(*([FAKE.value] * (7 * n)))
    if null_entry is not None:
        arr[null_entry] = None
    return ar.lib.ar_tune_blocks(descs, n if nblocks is None else nblocks, FAKE, 1, 4, T, ctypes.byref(q),
                                 ctypes.byref(o), arr, arr, arr, None, None, None, None)


def test_block_stack_checks_every_block_on_the_host():
    # ar_tune_blocks checks all blocks before its first HIP call, so these
    # calls return on a machine without a GPU
    ar = _ar()
    assert _stack_call(ar, nblocks=0) == ar.AR_ERR_INVALID_ARG
    assert _stack_call(ar, hidden=(128, 192)) == ar.AR_ERR_INVALID_ARG        # outputs feed the next block
    assert "hidden" in ar.lib.ar_last_error().decode()
    assert _stack_call(ar, start_step=3) == ar.AR_ERR_INVALID_ARG
    assert _stack_call(ar, T=48) == ar.AR_ERR_UNSUPPORTED                      # block 0 refuses it
    assert _stack_call(ar, kinds=(0, 1), T=320) == ar.AR_ERR_UNSUPPORTED       # only block 1 refuses it
    assert ar.lib.ar_last_error().decode().startswith("block 1:")
    assert _stack_call(ar, kinds=(0, 4)) == ar.AR_ERR_INVALID_ARG              # unknown kind
    assert _stack_call(ar, null_entry=7 + 2) == ar.AR_ERR_INVALID_ARG          # block 1, linear 2


def test_binding_refuses_host_tensors():
    ar = _ar()
    import torch
    W = torch.zeros(16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ar.qdq_rtn(W)


@pytest.mark.parametrize("M,K,g,xt,yt,expect", [
    (-1, 128, 128, 1, 0, 1),       # negative M
    (4, 128, 96, 1, 0, 1),         # group does not divide K
    (4, 128, 12, 1, 0, 1),         # ... nor a multiple of 8 (12 does not divide 128 either)
    (4, 320, 20, 1, 0, 2),         # group not a multiple of 8
    (4, 96, 32, 1, 0, 2),          # K not a multiple of 64
    (4, 128, 128, 0, 0, 2),        # fp32 activations
    (4, 128, 128, 1, 7, 1),        # unknown output dtype
    (0, 128, 128, 1, 0, 0),        # empty product: nothing to do
])
def test_w4a16_checks_arguments_on_the_host(M, K, g, xt, yt, expect):
    ar = _ar()
    st = ar.lib.ar_w4a16_gemm(FAKE, xt, M, K, FAKE, FAKE, FAKE, 64, g, FAKE, yt, None)
    assert st == expect
    if expect:
        assert ar.lib.ar_last_error().decode()


def test_w4a16_rejects_null_pointers():
    ar = _ar()
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        X, P, S, Z, Y = ptrs
        assert ar.lib.ar_w4a16_gemm(X, 1, 4, 128, P, S, Z, 64, 128, Y, 0, None) == ar.AR_ERR_INVALID_ARG
    # an empty product needs no activations or output
    assert ar.lib.ar_w4a16_gemm(None, 1, 0, 128, FAKE, FAKE, FAKE, 64, 128, None, 0, None) == ar.AR_OK


def test_float_formats_are_qdq_only():
    ar = _ar()
    fp8 = ar.QConfig(8, 128, 0, ar.AR_FMT_FP8_E4M3)
    # a rounding offset has no meaning on a float grid
    assert ar.lib.ar_qdq_rtn(FAKE, ar.AR_BF16, 4, 128, ctypes.byref(fp8), FAKE, None, None, FAKE, ar.AR_F32,
                             None, None, None, None) == ar.AR_ERR_UNSUPPORTED
    bad = ar.QConfig(4, 128, 0, ar.AR_FMT_FP8_E4M3)
    assert ar.lib.ar_qdq_rtn(FAKE, ar.AR_BF16, 4, 128, ctypes.byref(bad), None, None, None, FAKE, ar.AR_F32,
                             None, None, None, None) == ar.AR_ERR_INVALID_ARG
    mx = ar.QConfig(4, 64, 0, ar.AR_FMT_MXFP4)                     # blocks are 32 wide
    assert ar.lib.ar_qdq_rtn(FAKE, ar.AR_BF16, 4, 128, ctypes.byref(mx), None, None, None, FAKE, ar.AR_F32,
                             None, None, None, None) == ar.AR_ERR_INVALID_ARG
    unknown = ar.QConfig(4, 128, 0, 9)
    assert ar.lib.ar_qdq_rtn(FAKE, ar.AR_BF16, 4, 128, ctypes.byref(unknown), None, None, None, FAKE, ar.AR_F32,
                             None, None, None, None) == ar.AR_ERR_INVALID_ARG
    o = ar.default_opts()
    o.batch_samples = 2
    assert _tune(ar, q=fp8, opts=o) == ar.AR_ERR_UNSUPPORTED
    assert ar.lib.ar_pack_int4(FAKE, ar.AR_BF16, 4, 128, ctypes.byref(ar.QConfig(4, 32, 0, ar.AR_FMT_MXFP4)),
                               None, None, None, FAKE, FAKE, FAKE, None) == ar.AR_ERR_UNSUPPORTED


PROBE_LIB = os.path.join(ROOT, "post_weight_quantization_autoround_amd", "libarpeaks.so")
PROBE_HEADER = os.path.join(ROOT, "include", "ar_peaks.h")


@pytest.mark.skipif(not os.path.exists(PROBE_LIB), reason="libarpeaks.so not built")
def test_peak_probe_exports_and_checks_arguments():
    names = sorted(set(re.findall(r"ARP_API\s+[\w\s\*]+?\b(ar_\w+)\s*\(", open(PROBE_HEADER).read())))
    assert names == ["ar_peak_copy_gbs", "ar_peak_mfma_tflops", "ar_peak_read_gbs"]
    from post_weight_quantization_autoround_amd import peaks
    lib = peaks._lib()
    out = ctypes.c_double()
    # argument errors come back (hipErrorInvalidValue = 1) before any HIP call
    assert lib.ar_peak_copy_gbs(1000, 1, ctypes.byref(out)) == 1        # not a multiple of 4096
    assert lib.ar_peak_copy_gbs(4096, 0, ctypes.byref(out)) == 1
    assert lib.ar_peak_copy_gbs(4096, 1, None) == 1
    assert lib.ar_peak_read_gbs(1000, 1, ctypes.byref(out)) == 1
    assert lib.ar_peak_read_gbs(4096, 1, ctypes.byref(out)) == 1        # not a multiple of 65536
    assert lib.ar_peak_read_gbs(4096, 0, ctypes.byref(out)) == 1
    assert lib.ar_peak_read_gbs(4096, 1, None) == 1
    assert lib.ar_peak_mfma_tflops(0, ctypes.byref(out)) == 1
