"""The tuning entry points' contract at its edges, through the C ABI.

* every argument check of ar_tune_layer returns its documented status
  before any device work, leaves the caller's V, alpha and beta untouched,
  and the library stays usable afterwards;
* non-finite W or X_pool is reported as AR_ERR_NONFINITE;
* zero iterations return the initial state;
* degenerate weight groups (all zero, constant, a single non-zero,
  subnormal magnitudes whose scale has no usable reciprocal) give the
  oracle's gradients and codes, and the fused and six-kernel steps agree bit
  for bit on them.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from synthetic_inputs import make_layer_workload, to_bf16_values

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


N, K, S, T, GS = 64, 256, 3, 64, 128


@pytest.fixture(scope="module")
def small(ar):
    wl = make_layer_workload("linear4096_g128", n=N, k=K, s=S, b=2, t=T, iters=2)
    return dict(W=_dev(wl.W, True), X=_dev(wl.X, True), Wf=_dev(wl.W), wl=wl)


def _call(ar, small, q=None, o=None, W="W", wt=None, n=N, k=K, s=S, t=T, V=True):
    """ar_tune_layer on the small layer with one thing changed; returns
    (status, V, alpha, beta) with the caller's buffers after the call."""
    qc = ar.QConfig(4, GS, 0) if q is None else q
    opts = ar.default_opts()
    opts.iters, opts.batch_samples, opts.lr, opts.lr_clip = 2, 2, 0.005, 0.005
    if o is not None:
        o(opts)
    Wt = small[W] if W is not None else None
    if wt is None:
        wt = ar.AR_BF16 if W == "W" else ar.AR_F32
    G = max(K // GS, 1)
    Vb = torch.full((N, K), 0.25, dtype=torch.float32, device="cuda")
    al = torch.full((N, G), 0.75, dtype=torch.float32, device="cuda")
    be = torch.full((N, G), 0.875, dtype=torch.float32, device="cuda")
    bl, bs = ctypes.c_float(0.0), ctypes.c_int32(-7)
    st = ar.lib.ar_tune_layer(
        None if Wt is None else Wt.data_ptr(), wt, n, k, small["X"].data_ptr(), ar.AR_BF16, s, t,
        ctypes.byref(qc), ctypes.byref(opts), Vb.data_ptr() if V else None, al.data_ptr(), be.data_ptr(),
        ctypes.byref(bl), ctypes.byref(bs), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, Vb, al, be


def _set(**kv):
    def f(o):
        for key, val in kv.items():
            setattr(o, key, val)
    return f


BAD_SCHEDULE = (ctypes.c_int32 * 4)(0, 1, 2, S)    # the last id is outside [0, S)

CASES = {
    "bits=1": (dict(q=lambda ar: ar.QConfig(1, GS, 0)), "AR_ERR_INVALID_ARG"),
    "bits=9": (dict(q=lambda ar: ar.QConfig(9, GS, 0)), "AR_ERR_INVALID_ARG"),
    "group=0": (dict(q=lambda ar: ar.QConfig(4, 0, 0)), "AR_ERR_INVALID_ARG"),
    "group=96 does not divide K": (dict(q=lambda ar: ar.QConfig(4, 96, 0)), "AR_ERR_INVALID_ARG"),
    "group=4 not a multiple of 8": (dict(q=lambda ar: ar.QConfig(4, 4, 0)), "AR_ERR_UNSUPPORTED"),
    "sym=2": (dict(q=lambda ar: ar.QConfig(4, GS, 2)), "AR_ERR_INVALID_ARG"),
    "fp8 format": (dict(q=lambda ar: _fmt(ar.QConfig(8, GS, 0), 1)), "AR_ERR_UNSUPPORTED"),
    "N=0": (dict(n=0), "AR_ERR_INVALID_ARG"),
    "K=0": (dict(k=0), "AR_ERR_INVALID_ARG"),
    "S=0": (dict(s=0), "AR_ERR_INVALID_ARG"),
    "T=48": (dict(t=48), "AR_ERR_UNSUPPORTED"),
    "W NULL": (dict(W=None), "AR_ERR_INVALID_ARG"),
    "V NULL": (dict(V=False), "AR_ERR_INVALID_ARG"),
    "fp32 W with bf16 GEMMs": (dict(W="Wf"), "AR_ERR_UNSUPPORTED"),
    "gemm_mode=7": (dict(o=_set(gemm_mode=7)), "AR_ERR_INVALID_ARG"),
    "iters=-1": (dict(o=_set(iters=-1)), "AR_ERR_INVALID_ARG"),
    "lr<0": (dict(o=_set(lr=-0.005)), "AR_ERR_INVALID_ARG"),
    "lr NaN": (dict(o=_set(lr=float("nan"))), "AR_ERR_INVALID_ARG"),
    "clip box inverted": (dict(o=_set(clip_lo=1.0, clip_hi=0.5)), "AR_ERR_INVALID_ARG"),
    "lr_decay=2": (dict(o=_set(lr_decay=2)), "AR_ERR_INVALID_ARG"),
    "batch 0": (dict(o=_set(batch_samples=0)), "AR_ERR_INVALID_ARG"),
    "batch > S": (dict(o=_set(batch_samples=S + 1)), "AR_ERR_INVALID_ARG"),
    "schedule id out of range": (dict(o=_set(schedule=ctypes.cast(BAD_SCHEDULE, ctypes.POINTER(ctypes.c_int32)))),
                                 "AR_ERR_INVALID_ARG"),
    "workspace cap": (dict(o=_set(max_workspace_bytes=4096)), "AR_ERR_OUT_OF_MEMORY"),
}


def _fmt(q, f):
    q.format = f
    return q


@pytest.mark.parametrize("case", list(CASES))
def test_tune_layer_rejects_bad_arguments(ar, small, case):
    kw, status = CASES[case]
    kw = dict(kw)
    if "q" in kw:
        kw["q"] = kw["q"](ar)
    st, Vb, al, be = _call(ar, small, **kw)
    assert st == getattr(ar, status), (case, st, ar.lib.ar_last_error())
    assert ar.lib.ar_last_error()            # the message names the problem
    assert bool((Vb == 0.25).all()) and bool((al == 0.75).all()) and bool((be == 0.875).all())


def test_library_usable_after_rejections(ar, small):
    assert _call(ar, small, q=ar.QConfig(9, GS, 0))[0] == ar.AR_ERR_INVALID_ARG
    st, Vb, al, be = _call(ar, small)
    assert st == ar.AR_OK
    assert float(Vb.abs().max()) <= 0.5 and float(al.min()) >= 0.5 and float(be.max()) <= 1.0


@pytest.mark.parametrize("where", ["W", "X"])
def test_nonfinite_inputs_are_reported(ar, small, where):
    W, X = small["W"].clone(), small["X"].clone()
    if where == "W":
        W[5, 17] = float("nan")
    else:
        X[1, 3, 40] = float("inf")
    with pytest.raises(ar.ARError) as e:
        ar.tune_layer(W, X, bits=4, group_size=GS, iters=2, batch_samples=2)
    assert e.value.status == ar.AR_ERR_NONFINITE
    with pytest.raises(ar.ARError) as e:
        ar.Tuner(W, X, bits=4, group_size=GS, iters=2, batch_samples=2)
    assert e.value.status == ar.AR_ERR_NONFINITE


def test_zero_iterations_return_the_initial_state(ar, small):
    rng = np.random.default_rng(3)
    V0 = _dev(rng.uniform(-0.5, 0.5, (N, K)).astype(F32))
    a0 = _dev(rng.uniform(0.5, 1.0, (N, K // GS)).astype(F32))
    b0 = _dev(rng.uniform(0.5, 1.0, (N, K // GS)).astype(F32))
    res = ar.tune_layer(small["W"], small["X"], bits=4, group_size=GS, iters=0, batch_samples=2,
                        V0=V0, alpha0=a0, beta0=b0)
    assert torch.equal(res["V"], V0) and torch.equal(res["alpha"], a0) and torch.equal(res["beta"], b0)
    assert res["best_step"] == -1 and res["losses"] == []
    t = ar.Tuner(small["W"], small["X"], bits=4, group_size=GS, iters=3, batch_samples=2)
    with pytest.raises(ar.ARError) as e:
        t.run(4)                                  # more steps than iters
    assert e.value.status == ar.AR_ERR_INVALID_ARG
    t.run(0)
    out = t.finish()
    t.close()
    assert out["best_step"] == -1 and bool((out["V"] == 0).all())
    assert all(np.isnan(out["losses"]))          # no step evaluated


def _degenerate_weight(n, k, g, seed):
    """Rows cycling through the degenerate group shapes, bf16 values."""
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, 0.02, (n, k)).astype(F32)
    for r in range(n):
        kind = r % 8
        if kind == 0:
            W[r] = 0.0                                        # all-zero groups: s = 1, z = 0
        elif kind == 1:
            W[r] = 0.03                                       # constant positive (min clipped to 0)
        elif kind == 2:
            W[r] = -0.05                                      # constant negative (max clipped to 0)
        elif kind == 3:
            W[r] = 0.0
            W[r, ::g] = rng.normal(0.0, 0.05, k // g)         # one non-zero per group
        elif kind == 4:
            W[r] *= 1e-38                                     # subnormal scale: division fallback
        elif kind == 5:
            W[r, : k // 2] = 0.0                              # half the groups zero
    return to_bf16_values(W)


def test_degenerate_groups_match_the_oracle(ar):
    n, k, g, s, t = 128, 512, 128, 3, 64
    wl = make_layer_workload("linear4096_g128", n=n, k=k, s=s, b=2, t=t, iters=6)
    Wn = _degenerate_weight(n, k, g, 11)
    # cast on the host, where subnormals are kept, then move the bf16 bits
    W = torch.from_numpy(Wn).to(torch.bfloat16).cuda()
    X = _dev(wl.X, True)
    assert np.array_equal(W.cpu().float().numpy(), Wn)
    assert np.count_nonzero((Wn != 0) & (np.abs(Wn) < np.finfo(F32).tiny)) > 0
    rng = np.random.default_rng(12)
    V = rng.uniform(-0.5, 0.5, (n, k)).astype(F32)
    al = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    be = rng.uniform(0.5, 1.0, (n, k // g)).astype(F32)
    ids = [2, 0]
    ref = oracle.loss_and_grads(Wn, oracle.gather_batch(wl.X, ids), V, al, be, 4, g, mode="f32")
    out = ar.layer_grads(W, X, ids, _dev(V), _dev(al), _dev(be), bits=4, group_size=g, gemm_mode=ar.AR_GEMM_F32)
    assert out["loss"] == pytest.approx(ref["L"], rel=2e-5)
    got = {key: out[key].cpu().numpy() for key in ["G", "dV", "dalpha", "dbeta"]}
    for key in got:
        assert np.all(np.isfinite(got[key])), key
        assert _relf(got[key], ref[key]) <= 2e-4, (key, _relf(got[key], ref[key]))
    zero_rows = np.arange(0, n, 8)
    # all-zero groups: s = 1 and nothing is clipped, so dV = G exactly, and
    # the clip factors scale a zero range, so their gradients are zero
    np.testing.assert_array_equal(got["dV"][zero_rows], got["G"][zero_rows])
    assert np.all(got["dalpha"][zero_rows] == 0) and np.all(got["dbeta"][zero_rows] == 0)

    # codes at the GPU's tuned state are the oracle's, and the fused step is
    # the six-kernel step bit for bit on these groups
    kw = dict(bits=4, group_size=g, iters=wl.iters, lr=0.05, batch_samples=2, schedule=wl.schedule.tolist(),
              return_last=True)
    fused = ar.tune_layer(W, X, **kw)
    sep = ar.tune_layer(W, X, unfused=True, **kw)
    assert fused["losses"] == sep["losses"] and all(np.isfinite(fused["losses"]))
    for key in ["V", "alpha", "beta"]:
        assert torch.equal(fused[key], sep[key]), key
    Vt, at, bt = (fused[x].cpu().numpy() for x in ("V", "alpha", "beta"))
    qd = ar.qdq_rtn(W, bits=4, group_size=g, V=fused["V"], alpha=fused["alpha"], beta=fused["beta"])
    exp = oracle.qdq(Wn, Vt, at, bt, 4, g)
    np.testing.assert_array_equal(qd["codes"].cpu().numpy(), exp["q"].astype(np.uint8))
    np.testing.assert_array_equal(qd["scale"].cpu().numpy(), exp["s"])


# ---- block-wise entry points (ar_tune_block) --------------------------------

H, F, HEADS, KV, HD = 128, 192, 2, 1, 64


def _bf16_randn(shape, seed, scale=0.02):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).cuda()


def _decoder_weights(heads=HEADS, kv=KV, hd=HD, dtype=torch.bfloat16):
    import post_weight_quantization_autoround_amd as mod
    shapes = mod.decoder_weight_shapes(H, F, heads, kv, hd)
    return {nm: _bf16_randn(sh, 20 + i).to(dtype) for i, (nm, sh) in enumerate(zip(mod.DECODER_LINEARS, shapes))}


def _pool(t=64, s=2, dtype=torch.bfloat16):
    return _bf16_randn((s, t, H), 30, scale=1.0).to(dtype)


DECODER_CASES = {
    "heads not a multiple of kv_heads": (dict(heads=3, kv=2), {}, "AR_ERR_INVALID_ARG"),
    "head_dim 32": (dict(heads=4, hd=32), {}, "AR_ERR_UNSUPPORTED"),
    "T = 320": (dict(t=320), {}, "AR_ERR_UNSUPPORTED"),
    "per-row groups": ({}, dict(group_size=-1), "AR_ERR_UNSUPPORTED"),
    "group 48 does not divide H": ({}, dict(group_size=48), "AR_ERR_INVALID_ARG"),
    "fp32 weights": (dict(dtype=torch.float32), {}, "AR_ERR_UNSUPPORTED"),
    "norm eps 0": ({}, dict(eps=0.0), "AR_ERR_INVALID_ARG"),
    "NaN in the o weight": (dict(nan="o"), {}, "AR_ERR_NONFINITE"),
}


@pytest.mark.parametrize("case", list(DECODER_CASES))
def test_decoder_block_rejections(ar, case):
    shape, kw, status = DECODER_CASES[case]
    shape = dict(shape)
    t = shape.pop("t", 64)
    nan = shape.pop("nan", None)
    dtype = shape.get("dtype", torch.bfloat16)
    w = _decoder_weights(**shape)
    if nan:
        w[nan][3, 5] = float("nan")
    heads, kv, hd = shape.get("heads", HEADS), shape.get("kv", KV), shape.get("hd", HD)
    args = dict(bits=4, group_size=64, iters=1, batch_samples=1, output=False)
    args.update(kw)
    with pytest.raises(ar.ARError) as e:
        ar.tune_decoder(w, _pool(t, dtype=dtype), heads, kv, hd, **args)
    assert e.value.status == getattr(ar, status), (case, str(e.value))


def test_decoder_block_valid_baseline(ar):
    # the unmodified configuration of the rejection cases runs
    res = ar.tune_decoder(_decoder_weights(), _pool(), HEADS, KV, HD, bits=4, group_size=64, iters=2,
                          batch_samples=1, output=True)
    assert all(np.isfinite(res["losses"])) and res["output"].shape == (2, 64, H)


@pytest.mark.parametrize("case", ["T = 48", "per-row groups", "NaN in down", "fp32 weights with bf16 GEMMs"])
def test_mlp_block_rejections(ar, case):
    gate, up, down = _bf16_randn((F, H), 40), _bf16_randn((F, H), 41), _bf16_randn((H, F), 42)
    X = _pool()
    args = dict(bits=4, group_size=64, iters=1, batch_samples=1, output=False)
    expected = ar.AR_ERR_UNSUPPORTED
    if case == "T = 48":
        X = _pool(48)
    elif case == "per-row groups":
        args["group_size"] = -1
    elif case == "NaN in down":
        down[7, 9] = float("nan")
        expected = ar.AR_ERR_NONFINITE
    else:
        gate, up, down = gate.float(), up.float(), down.float()
        X = X.float()
    with pytest.raises(ar.ARError) as e:
        ar.tune_block(gate, up, down, X, **args)
    assert e.value.status == expected, (case, str(e.value))
    # the same block with valid arguments runs
    ok = ar.tune_block(_bf16_randn((F, H), 40), _bf16_randn((F, H), 41), _bf16_randn((H, F), 42), _pool(),
                       bits=4, group_size=64, iters=2, batch_samples=1, output=False)
    assert all(np.isfinite(ok["losses"]))


def test_peak_probe_within_published_peaks():
    # the on-box denominators of the benchmark's roofline fractions: a device
    # copy and a read-only stream below HBM3E's 8 TB/s and a bf16 MFMA loop below the dense 2.5
    # PFLOP/s, both well above what a broken probe would show; argument
    # errors return 1 before any HIP call
    from post_weight_quantization_autoround_amd import peaks
    lib = peaks._lib()
    out = ctypes.c_double(-1.0)
    assert lib.ar_peak_copy_gbs(0, 5, ctypes.byref(out)) == 1 and out.value == -1.0
    assert lib.ar_peak_mfma_tflops(0, ctypes.byref(out)) == 1 and out.value == -1.0
    assert lib.ar_peak_copy_gbs(1 << 20, 5, None) == 1
    assert lib.ar_peak_read_gbs(1 << 20, 5, None) == 1
    copy = peaks.copy_gbs(256 << 20, 5)
    read = peaks.read_gbs(1 << 30, 5)
    mfma = peaks.mfma_tflops(4000)
    assert 1000.0 < copy <= 8000.0, copy
    assert 1000.0 < read <= 8000.0, read
    assert 300.0 < mfma <= 2500.0, mfma
