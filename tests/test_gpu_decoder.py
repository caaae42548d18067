"""GPU parity of block-wise tuning of a Llama decoder block against the
decoder oracle (bf16 mode): loss and straight-through gradients of all seven
linears (MHA and GQA, head size 64 and 128, ragged query tiles), fused
against separate kernels, the snapshot and determinism, the quantized block
output handed to the next block, and the Llama-7B-shaped block (hidden 4096,
32 heads x 128, FFN 11008, 256 tokens) at full size."""
import numpy as np
import pytest
import torch

import oracle
from oracle import decoder_ref as dr
from synthetic_inputs import make_decoder_workload

pytestmark = pytest.mark.gpu
F32 = np.float32
NAMES = dr.LINEARS


@pytest.fixture(scope="module")
def ar():
    import post_weight_quantization_autoround_amd as mod
    assert torch.cuda.is_available()
    return mod


def _dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if bf16 else t


def _relf(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / (np.linalg.norm(b) + 1e-300))


def _small(**kw):
    cfg = dict(h=256, f=512, heads=4, kv_heads=2, head_dim=64, s=4, t=128, b=2, group=64, iters=8)
    cfg.update(kw)
    return make_decoder_workload("llama7b_decoder_g128", **cfg)


def _gpu_args(wl):
    return dict(weights={n: _dev(wl.W[n], True) for n in NAMES}, X_pool=_dev(wl.X, True), heads=wl.heads,
                kv_heads=wl.kv_heads, head_dim=wl.head_dim, norm_weights=(_dev(wl.w1), _dev(wl.w2)),
                eps=wl.norm_eps, theta=wl.rope_theta)


def _random_params(wl, seed):
    rng = np.random.default_rng(seed)
    out = {}
    for nm, (n, k) in wl.shapes().items():
        out[nm] = (rng.uniform(-0.5, 0.5, (n, k)).astype(F32), rng.uniform(0.5, 1.0, (n, k // wl.group)).astype(F32),
                   rng.uniform(0.5, 1.0, (n, k // wl.group)).astype(F32))
    return out


def _oracle_grads(wl, params, ids, Y_ref=None):
    cfg = wl.cfg()
    if Y_ref is None:
        Y_ref = dr.decoder_reference(wl.X[ids], wl.W, cfg, "bf16")
        Yb = Y_ref.reshape(-1, wl.h)
    else:
        Yb = oracle.gather_batch(Y_ref, ids)
    return dr.decoder_loss_and_grads(oracle.gather_batch(wl.X, ids), Yb, wl.W,
                                     {n: params[n][0] for n in NAMES}, {n: params[n][1] for n in NAMES},
                                     {n: params[n][2] for n in NAMES}, wl.bits, wl.group, cfg, mode="bf16")


def _check_grads(out, ref):
    assert out["loss"] == pytest.approx(ref["L"], rel=1e-3)
    for n in NAMES:
        assert _relf(out["G"][n].cpu().numpy(), ref["G"][n]) <= 1e-2, n
        for key, r in zip(("dV", "dalpha", "dbeta"), ref["grads"][n]):
            assert _relf(out[key][n].cpu().numpy(), r) <= 1e-2, (n, key)


CASES = {
    # grouped-query attention, head size 64, two query tiles per sample
    "gqa_d64": dict(h=256, f=512, heads=4, kv_heads=2, head_dim=64, t=128, s=4, group=64),
    # one KV head for two query heads, head size 128, three query tiles (ragged causal chunks)
    "d128_t192": dict(h=256, f=384, heads=2, kv_heads=1, head_dim=128, t=192, s=3, group=128),
    # multi-head attention at the longest sample, 8 KV groups of one head
    "mha_t256": dict(h=512, f=768, heads=8, kv_heads=8, head_dim=64, t=256, s=2, group=128),
    # 8 query heads per KV head, g32 (the 70B block's grouping at a small width)
    "gqa8_g32": dict(h=512, f=1024, heads=8, kv_heads=1, head_dim=64, t=64, s=3, group=32),
    # hidden 320 and FFN 576: the GEMMs that read a weight in place (transposed
    # operand) end in a partial 128-wide tile along that operand
    "ragged_h320_f576": dict(h=320, f=576, heads=4, kv_heads=2, head_dim=64, t=128, s=3, group=64),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_decoder_gradients_match_oracle(ar, case):
    wl = _small(b=2, **CASES[case])
    params = _random_params(wl, 3)
    ids = [wl.s - 1, 0]
    ref = _oracle_grads(wl, params, ids)
    out = ar.decoder_grads(ids=ids, params={n: tuple(_dev(a) for a in params[n]) for n in NAMES}, bits=wl.bits,
                           group_size=wl.group, **_gpu_args(wl))
    _check_grads(out, ref)


def test_decoder_rtn_gradients_single_sample(ar):
    # default parameters (V = 0, alpha = beta = 1), one sample per step
    wl = _small(s=2, b=1)
    ids = [1]
    params = {n: (np.zeros((N, K), F32), np.ones((N, K // wl.group), F32), np.ones((N, K // wl.group), F32))
              for n, (N, K) in wl.shapes().items()}
    ref = _oracle_grads(wl, params, ids)
    out = ar.decoder_grads(ids=ids, bits=wl.bits, group_size=wl.group, **_gpu_args(wl))
    _check_grads(out, ref)


def test_decoder_fused_matches_separate_kernels(ar):
    wl = _small(group=128, iters=6)
    kw = dict(bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist(), return_last=True, output=False)
    fused = ar.tune_decoder(**_gpu_args(wl), **kw)
    sep = ar.tune_decoder(**_gpu_args(wl), unfused=True, **kw)
    assert fused["losses"] == sep["losses"]
    for n in NAMES:
        for a, b in zip(fused["params"][n], sep["params"][n]):
            assert torch.equal(a, b), n


def test_decoder_snapshot_and_determinism(ar):
    wl = _small(iters=8)
    kw = dict(bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist(), output=False)
    a = ar.tune_decoder(**_gpu_args(wl), **kw)
    b = ar.tune_decoder(**_gpu_args(wl), **kw)
    assert a["losses"] == b["losses"] and a["best_step"] == b["best_step"]
    assert a["best_loss"] == pytest.approx(min(a["losses"]), rel=1e-6)
    assert a["best_step"] == int(np.argmin(a["losses"]))
    for n in NAMES:
        for x, y in zip(a["params"][n], b["params"][n]):
            assert torch.equal(x, y)


def test_decoder_first_step_loss_and_stepwise_api(ar):
    # the first step's loss is the oracle's at RTN on the first minibatch; the
    # stepwise API gives the same trajectory as the one-call API
    wl = _small(iters=5)
    kw = dict(bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist())
    one = ar.tune_decoder(**_gpu_args(wl), output=False, **kw)
    ids = [int(i) for i in wl.schedule[0]]
    params = {n: (np.zeros((N, K), F32), np.ones((N, K // wl.group), F32), np.ones((N, K // wl.group), F32))
              for n, (N, K) in wl.shapes().items()}
    ref = _oracle_grads(wl, params, ids)
    assert one["losses"][0] == pytest.approx(ref["L"], rel=1e-3)
    t = ar.DecoderTuner(**_gpu_args(wl), **kw)
    t.run(2)
    t.run(wl.iters - 2, graph=False)
    res = t.finish()
    t.close()
    assert res["losses"] == one["losses"]
    for n in NAMES:
        for x, y in zip(res["params"][n], one["params"][n]):
            assert torch.equal(x, y)


def test_decoder_output_for_the_next_block(ar):
    wl = _small(iters=6)
    res = ar.tune_decoder(**_gpu_args(wl), bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr,
                          batch_samples=wl.b, schedule=wl.schedule.tolist())
    params = {n: tuple(a.cpu().numpy() for a in res["params"][n]) for n in NAMES}
    cfg = wl.cfg()
    ref = dr.quantized_decoder_output(wl.X, wl.W, cfg, params, wl.bits, wl.group, mode="bf16")
    got = res["output"].float().cpu().numpy()
    assert got.shape == wl.X.shape
    # the output is stored in bf16 (the pool's dtype): each element is within
    # one bf16 ulp of the oracle's fp64 value, up to a small absolute error
    # where the residual and the block's update nearly cancel, and nearly all
    # elements are that value's nearest bf16
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    excess = np.abs(got - ref) - ulp
    atol = 2e-2 * float(np.sqrt(np.mean((ref - wl.X) ** 2)))
    assert np.all(excess <= atol), (float(excess.max()), atol, int(np.sum(excess > 0)))
    nearest = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    frac = float(np.mean(got == nearest))
    assert frac >= 0.95, frac
    # the returned state is the best one: its loss on the best step's batch
    ids = [int(i) for i in wl.schedule[res["best_step"]]]
    again = _oracle_grads(wl, params, ids)
    assert res["best_loss"] == pytest.approx(again["L"], rel=1e-3)


def test_full_size_decoder_gradients(ar):
    # Llama-7B-shaped block: hidden 4096, 32 heads x 128, FFN 11008, g128, one 256-token sample
    wl = make_decoder_workload("llama7b_decoder_g128", s=2, b=1, iters=1)
    params = _random_params(wl, 5)
    ids = [1]
    ref = _oracle_grads(wl, params, ids)
    out = ar.decoder_grads(ids=ids, params={n: tuple(_dev(a) for a in params[n]) for n in NAMES}, bits=wl.bits,
                           group_size=wl.group, **_gpu_args(wl))
    _check_grads(out, ref)


def test_full_size_70b_decoder_fused_matches_separate_kernels(ar):
    # 70B-shaped block (hidden 8192, 64 / 8 heads x 128, FFN 28672, g32, 4
    # samples per step) in the launch configuration the benchmark times: the
    # fused steps equal the separate-kernel steps bit for bit, and a rerun is
    # identical.  (Oracle parity for 8:1 GQA with g32 is checked at a small
    # width above; the oracle at this size needs minutes and ~50 GB.)
    wl = make_decoder_workload("llama70b_decoder_g32", s=8, iters=2)
    args = _gpu_args(wl)
    kw = dict(bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist(), return_last=True, output=False)
    fused = ar.tune_decoder(**args, **kw)
    again = ar.tune_decoder(**args, **kw)
    sep = ar.tune_decoder(**args, unfused=True, **kw)
    assert all(np.isfinite(fused["losses"]))
    assert fused["losses"] == sep["losses"] == again["losses"]
    for n in NAMES:
        for a, b, c in zip(fused["params"][n], sep["params"][n], again["params"][n]):
            assert torch.equal(a, b) and torch.equal(a, c), n


def test_split_reduction_gemm_gradients_match_oracle(ar):
    # 8 samples x 256 tokens at hidden 4096 with FFN 2048: the dh2 GEMM (a
    # 2048 x 4096 output whose 256 x 256 tiles fill half the CUs, reduction
    # 2F = 4096) runs as two reduction halves summed by the RMSNorm backward
    wl = make_decoder_workload("llama7b_decoder_g128", h=4096, f=2048, heads=4, kv_heads=2, head_dim=128, s=9, t=256,
                               b=8, group=128, iters=1)
    params = _random_params(wl, 5)
    ids = [8, 0, 1, 2, 3, 4, 5, 6]
    ref = _oracle_grads(wl, params, ids)
    out = ar.decoder_grads(ids=ids, params={n: tuple(_dev(a) for a in params[n]) for n in NAMES}, bits=wl.bits,
                           group_size=wl.group, **_gpu_args(wl))
    _check_grads(out, ref)


def test_tail_split_qkv_gemm_gradients_match_oracle(ar):
    # 8 samples x 256 tokens, 32 + 32 + 32 heads of 128 at hidden 4096: the
    # QKV GEMM has 8 x 48 tiles of 256 x 256, so its first 8192 output columns
    # run as one round and the last 4096 as a second launch of 256 x 128 tiles
    wl = make_decoder_workload("llama7b_decoder_g128", h=4096, f=1024, heads=32, kv_heads=32, head_dim=128, s=9,
                               t=256, b=8, group=128, iters=1)
    params = _random_params(wl, 6)
    ids = [8, 0, 1, 2, 3, 4, 5, 6]
    ref = _oracle_grads(wl, params, ids)
    out = ar.decoder_grads(ids=ids, params={n: tuple(_dev(a) for a in params[n]) for n in NAMES}, bits=wl.bits,
                           group_size=wl.group, **_gpu_args(wl))
    _check_grads(out, ref)


@pytest.mark.timeout(1200)
def test_full_size_70b_decoder_gradients_on_sampled_rows(ar):
    # 70B-shaped block at its own shape: hidden 8192, 64 query / 8 KV heads
    # x 128, FFN 28672, g32, one 256-token sample, from a random state.  The
    # decoder oracle runs the whole forward and backward (G of every linear
    # whole) and the straight-through step on 24 sampled rows per linear; the
    # GPU's loss, G and dV / dalpha / dbeta on those rows must agree within
    # the bf16 tolerances.  The fused 256 x 256 g32 epilogue is covered by the
    # layer test at 4096 x 4096 g32 and by fused = separate kernels here.
    print("70B-shaped decoder: building the workload", flush=True)
    wl = make_decoder_workload("llama70b_decoder_g32", s=2, b=1, iters=1)
    params = _random_params(wl, 11)
    ids = [1]
    rng = np.random.default_rng(12)
    rows = {n: np.sort(rng.choice(wl.shapes()[n][0], 24, replace=False)) for n in NAMES}
    out = ar.decoder_grads(ids=ids, params={n: tuple(_dev(a) for a in params[n]) for n in NAMES}, bits=wl.bits,
                           group_size=wl.group, **_gpu_args(wl))
    got = {k: {n: out[k][n].cpu().numpy() for n in NAMES} for k in ("G", "dV", "dalpha", "dbeta")}
    loss = out["loss"]
    del out
    torch.cuda.empty_cache()
    print("70B-shaped decoder: GPU done, running the oracle", flush=True)
    cfg = wl.cfg()
    Y_ref = dr.decoder_reference(wl.X[ids], wl.W, cfg, "bf16").reshape(-1, wl.h)
    ref = dr.decoder_loss_and_grads(oracle.gather_batch(wl.X, ids), Y_ref, wl.W, {n: params[n][0] for n in NAMES},
                                    {n: params[n][1] for n in NAMES}, {n: params[n][2] for n in NAMES}, wl.bits,
                                    wl.group, cfg, mode="bf16", ste_rows=rows)
    assert loss == pytest.approx(ref["L"], rel=1e-3)
    for n in NAMES:
        e = _relf(got["G"][n], ref["G"][n])
        print(f"  {n}: G {e:.2e}", flush=True)
        assert e <= 1e-2, n
        for key, r in zip(("dV", "dalpha", "dbeta"), ref["grads"][n]):
            assert _relf(got[key][n][rows[n]], r) <= 1e-2, (n, key)


def test_two_decoder_blocks_in_sequence(ar):
    # Block-sequential quantization (blog sec. 3, algorithm flow step 7):
    # block 1 is tuned on the pool, its quantized output (residual stream,
    # bf16) becomes block 2's pool, and block 2 is tuned on it.  Against the
    # oracle chained the same way: block 1's output at the GPU's chosen state
    # is the oracle's (within bf16 rounding); block 2's losses and gradients
    # at its states, fed the GPU's block-1 output, match; and the oracle's
    # own chain (its block-1 snapshot, its output, block 2 tuned on that)
    # gives block-2 losses within 1e-2 of the GPU's.
    wl1 = _small(b=2, iters=4, **CASES["gqa_d64"])
    wl2 = make_decoder_workload("llama70b_decoder_g32", h=wl1.h, f=wl1.f, heads=wl1.heads, kv_heads=wl1.kv_heads,
                                head_dim=wl1.head_dim, s=wl1.s, t=wl1.t, b=wl1.b, group=wl1.group, iters=wl1.iters)
    kw = dict(bits=wl1.bits, group_size=wl1.group, iters=wl1.iters, lr=wl1.lr, batch_samples=wl1.b,
              schedule=wl1.schedule.tolist())
    a1 = _gpu_args(wl1)
    r1 = ar.tune_decoder(**a1, **kw)
    Y1 = r1["output"]
    a2 = _gpu_args(wl2)
    a2["X_pool"] = Y1
    r2 = ar.tune_decoder(**a2, **kw)
    cfg1, cfg2 = wl1.cfg(), wl2.cfg()
    p1 = {n: tuple(a.cpu().numpy() for a in r1["params"][n]) for n in NAMES}
    y1_ref = dr.quantized_decoder_output(wl1.X, wl1.W, cfg1, p1, wl1.bits, wl1.group, mode="bf16")
    y1 = Y1.float().cpu().numpy()
    assert _relf(y1, y1_ref) <= 4e-3
    # block 2 on the GPU's block-1 output: loss of each evaluated step and the
    # gradients at the state it returned
    x2 = y1
    Yr2 = dr.decoder_reference(x2, wl2.W, cfg2, "bf16")
    p2 = {n: tuple(a.cpu().numpy() for a in r2["params"][n]) for n in NAMES}
    ids = [int(i) for i in wl1.schedule[r2["best_step"]]]
    chk = dr.decoder_loss_and_grads(oracle.gather_batch(x2, ids), oracle.gather_batch(Yr2, ids), wl2.W,
                                    {n: p2[n][0] for n in NAMES}, {n: p2[n][1] for n in NAMES},
                                    {n: p2[n][2] for n in NAMES}, wl2.bits, wl2.group, cfg2, mode="bf16")
    assert r2["best_loss"] == pytest.approx(chk["L"], rel=1e-3)
    out = ar.decoder_grads(**a2, ids=ids, params={n: tuple(_dev(a) for a in p2[n]) for n in NAMES},
                           bits=wl2.bits, group_size=wl2.group)
    _check_grads(out, chk)
    # the oracle's own chain
    o1 = dr.tune_decoder(wl1.X, wl1.W, cfg1, wl1.schedule, wl1.bits, wl1.group, wl1.iters, wl1.lr, mode="bf16")
    x2_o = dr.quantized_decoder_output(wl1.X, wl1.W, cfg1, o1["params"], wl1.bits, wl1.group, mode="bf16")
    x2_o = oracle.bf16_round(x2_o.astype(F32)).astype(F32)          # the pool dtype the next block reads
    o2 = dr.tune_decoder(x2_o, wl2.W, cfg2, wl1.schedule, wl2.bits, wl2.group, wl1.iters, wl1.lr, mode="bf16")
    rel1 = np.abs(np.asarray(r1["losses"]) - o1["losses"]) / o1["losses"]
    rel2 = np.abs(np.asarray(r2["losses"]) - o2["losses"]) / o2["losses"]
    assert np.all(rel1[:2] <= 1e-3), rel1
    assert np.all(rel2 <= 1e-2), rel2


@pytest.mark.parametrize("k_split", [3, 8])
def test_decoder_split_run_equals_full_run(ar, k_split):
    # steps 0..k-1 through the stepwise API, then k..T-1 in a resumed one-call
    # run (start_step = k, best_loss_in = the first part's best loss): the same
    # losses, snapshot and state as one T-step run
    wl = _small(iters=12)
    kw = dict(bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist())
    full = ar.tune_decoder(**_gpu_args(wl), output=False, **kw)
    parts = []
    for last in (True, False):
        tu = ar.DecoderTuner(**_gpu_args(wl), return_last=last, **kw)
        tu.run(k_split)
        parts.append(tu.finish())
        tu.close()
    cur, best1 = parts
    second = ar.tune_decoder(**_gpu_args(wl), params=cur["params"], start_step=k_split,
                             best_loss_in=best1["best_loss"], output=False, **kw)
    assert np.all(np.isnan(second["losses"][:k_split]))
    assert second["losses"][k_split:] == full["losses"][k_split:]
    assert best1["losses"][:k_split] == full["losses"][:k_split]
    if full["best_step"] >= k_split:
        assert second["best_step"] == full["best_step"]
        chosen = second
    else:
        assert second["best_step"] == -1 and second["best_loss"] == best1["best_loss"]
        chosen = best1
    assert chosen["best_loss"] == full["best_loss"]
    for n in NAMES:
        for a, b in zip(chosen["params"][n], full["params"][n]):
            assert torch.equal(a, b), n


def test_decoder_stack_with_host_weights_matches_resident_chain(ar):
    # ar_tune_blocks on two decoder blocks (GQA, head size 64) whose weights
    # and norm vectors stay in page-locked host memory: bit for bit what
    # ar_tune_block gives on device copies chained by hand.
    wl1 = _small(b=2, iters=6, **CASES["gqa_d64"])
    wl2 = make_decoder_workload("llama70b_decoder_g32", h=wl1.h, f=wl1.f, heads=wl1.heads, kv_heads=wl1.kv_heads,
                                head_dim=wl1.head_dim, s=wl1.s, t=wl1.t, b=wl1.b, group=wl1.group, iters=wl1.iters)
    kw = dict(bits=wl1.bits, group_size=wl1.group, iters=wl1.iters, lr=wl1.lr, batch_samples=wl1.b,
              schedule=wl1.schedule.tolist())
    a1 = _gpu_args(wl1)
    r1 = ar.tune_decoder(**a1, **kw)
    a2 = _gpu_args(wl2)
    a2["X_pool"] = r1["output"]
    r2 = ar.tune_decoder(**a2, **kw)

    def host(wl):
        d = {n: torch.from_numpy(np.ascontiguousarray(wl.W[n])).to(torch.bfloat16).pin_memory() for n in NAMES}
        d["norm1"] = torch.from_numpy(np.ascontiguousarray(wl.w1, dtype=F32)).pin_memory()
        d["norm2"] = torch.from_numpy(np.ascontiguousarray(wl.w2, dtype=F32)).pin_memory()
        return d

    st = ar.tune_blocks([host(wl1), host(wl2)], a1["X_pool"], heads=wl1.heads, kv_heads=wl1.kv_heads,
                        head_dim=wl1.head_dim, eps=wl1.norm_eps, theta=wl1.rope_theta, **kw)
    for b, r in enumerate((r1, r2)):
        assert st["losses"][b] == r["losses"], b
        assert st["best_losses"][b] == r["best_loss"] and st["best_steps"][b] == r["best_step"], b
        for n in NAMES:
            for a, ref in zip(st["params"][b][n], r["params"][n]):
                assert torch.equal(a, ref.cpu()), (b, n)
    assert torch.equal(st["output"], r2["output"])


@pytest.mark.gpu
def test_full_size_decoder_stack_matches_resident_chain(ar):
    # ar_tune_blocks at the Llama-7B block shape (hidden 4096, FFN 11008,
    # 32 heads of 128, g128, 8 samples of 256 tokens per step), two blocks
    # with weights and norm vectors in page-locked host memory, 3 steps
    # each: the staged stack gives bit for bit what ar_tune_block gives on
    # device copies chained by hand.  Both blocks take the same weights; the
    # second one sees the first one's quantized output.
    wl = make_decoder_workload("llama7b_decoder_g128", iters=3)
    kw = dict(bits=wl.bits, group_size=wl.group, iters=wl.iters, lr=wl.lr, batch_samples=wl.b,
              schedule=wl.schedule.tolist())
    a = _gpu_args(wl)
    r1 = ar.tune_decoder(**a, output=True, **kw)
    a2 = dict(a, X_pool=r1["output"])
    r2 = ar.tune_decoder(**a2, output=True, **kw)
    host = {n: torch.from_numpy(np.ascontiguousarray(wl.W[n])).to(torch.bfloat16).pin_memory() for n in NAMES}
    host["norm1"] = torch.from_numpy(np.ascontiguousarray(wl.w1, dtype=F32)).pin_memory()
    host["norm2"] = torch.from_numpy(np.ascontiguousarray(wl.w2, dtype=F32)).pin_memory()
    st = ar.tune_blocks([host, dict(host)], a["X_pool"], heads=wl.heads, kv_heads=wl.kv_heads,
                        head_dim=wl.head_dim, eps=wl.norm_eps, theta=wl.rope_theta, **kw)
    for b, r in enumerate((r1, r2)):
        assert st["losses"][b] == r["losses"], b
        assert st["best_losses"][b] == r["best_loss"] and st["best_steps"][b] == r["best_step"], b
        for n in NAMES:
            for x, ref in zip(st["params"][b][n], r["params"][n]):
                assert torch.equal(x, ref.cpu()), (b, n)
    assert torch.equal(st["output"], r2["output"])
