"""AutoRound-style post-training weight quantization for AMD MI355X (gfx950).

Thin ctypes binding over libautoround (include/libautoround.h): every step of
the quantize / tune / pack path runs in the library's HIP kernels; this module
only checks tensors and passes pointers and the current HIP stream.  Importing
it fails loudly when the library has not been built
(python post_weight_quantization_autoround_amd/build.py).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libautoround.so")

AR_OK, AR_ERR_INVALID_ARG, AR_ERR_UNSUPPORTED, AR_ERR_NONFINITE, AR_ERR_OUT_OF_MEMORY, AR_ERR_HIP = range(6)
AR_F32, AR_BF16 = 0, 1
AR_GEMM_BF16, AR_GEMM_F32 = 0, 1
AR_PRESET_DEFAULT, AR_PRESET_BEST, AR_PRESET_LIGHT, AR_PRESET_FAST = range(4)
AR_RUN_GRAPH, AR_RUN_EVENTS, AR_RUN_KERNEL_GRAPHS = 1, 2, 4
AR_BLOCK_MLP_SWIGLU, AR_BLOCK_LLAMA_DECODER = 0, 1
LINEARS = ("gate", "up", "down")
DECODER_LINEARS = ("q", "k", "v", "o", "gate", "up", "down")

_STATUS_NAMES = {
    AR_ERR_INVALID_ARG: "AR_ERR_INVALID_ARG",
    AR_ERR_UNSUPPORTED: "AR_ERR_UNSUPPORTED",
    AR_ERR_NONFINITE: "AR_ERR_NONFINITE",
    AR_ERR_OUT_OF_MEMORY: "AR_ERR_OUT_OF_MEMORY",
    AR_ERR_HIP: "AR_ERR_HIP",
}


class ARError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


AR_FMT_INT, AR_FMT_FP8_E4M3, AR_FMT_MXFP4 = 0, 1, 2


class QConfig(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("sym", ctypes.c_int32),
                ("format", ctypes.c_int32)]


class TuneOpts(ctypes.Structure):
    _fields_ = [
        ("iters", ctypes.c_int32),
        ("lr", ctypes.c_float),
        ("lr_clip", ctypes.c_float),
        ("lr_decay", ctypes.c_int32),
        ("clip_lo", ctypes.c_float),
        ("clip_hi", ctypes.c_float),
        ("batch_samples", ctypes.c_int32),
        ("schedule", ctypes.POINTER(ctypes.c_int32)),
        ("gemm_mode", ctypes.c_int),
        ("return_last", ctypes.c_int32),
        ("loss_trace", ctypes.POINTER(ctypes.c_float)),
        ("max_workspace_bytes", ctypes.c_size_t),
        ("unfused", ctypes.c_int32),
        ("start_step", ctypes.c_int32),
        ("best_loss_in", ctypes.c_float),
    ]


class BlockDesc(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int),
        ("hidden", ctypes.c_int64), ("ffn", ctypes.c_int64), ("heads", ctypes.c_int64),
        ("kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("weights", ctypes.c_void_p * 7),
        ("norm_weights", ctypes.c_void_p * 2),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python post_weight_quantization_autoround_amd/build.py`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
    st = ctypes.c_int
    qc = ctypes.POINTER(QConfig)
    op = ctypes.POINTER(TuneOpts)
    sig = {
        "ar_tune_opts_init": (st, [op, I32]),
        "ar_qdq_rtn": (st, [P, st, I64, I64, qc, P, P, P, P, st, P, P, P, P]),
        "ar_qdq_rtn_noalloc": (st, [P, st, I64, I64, qc, P, P, P, P, st, P, P, P, P]),
        "ar_pack_int4": (st, [P, st, I64, I64, qc, P, P, P, P, P, P, P]),
        "ar_w4a16_gemm": (st, [P, st, I64, I64, P, P, P, I64, I32, P, st, P]),
        "ar_layer_grads": (st, [P, st, I64, I64, P, st, I64, I64, ctypes.POINTER(ctypes.c_int32), I32, qc, st,
                                P, P, P, ctypes.POINTER(D), P, P, P, P, P]),
        "ar_tune_layer": (st, [P, st, I64, I64, P, st, I64, I64, qc, op, P, P, P,
                               ctypes.POINTER(F), ctypes.POINTER(I32), P]),
        "ar_tuner_create": (st, [ctypes.POINTER(P), P, st, I64, I64, P, st, I64, I64, qc, op, P, P, P, P]),
        "ar_tuner_run": (st, [P, I32, I32]),
        "ar_tuner_finish": (st, [P, P, P, P, ctypes.POINTER(F), ctypes.POINTER(I32)]),
        "ar_tuner_destroy": (st, [P]),
        "ar_tuner_num_kernels": (I32, [P]),
        "ar_tuner_kernel_name": (ctypes.c_char_p, [P, I32]),
        "ar_tuner_kernel_ms": (st, [P, ctypes.POINTER(F)]),
        "ar_tune_block": (st, [ctypes.POINTER(BlockDesc), P, st, I64, I64, qc, op, P, P, P, P,
                               ctypes.POINTER(F), ctypes.POINTER(I32), P]),
        "ar_block_tuner_create": (st, [ctypes.POINTER(P), ctypes.POINTER(BlockDesc), P, st, I64, I64, qc, op,
                                       P, P, P, P]),
        "ar_block_tuner_finish": (st, [P, P, P, P, P, ctypes.POINTER(F), ctypes.POINTER(I32)]),
        "ar_block_grads": (st, [ctypes.POINTER(BlockDesc), P, st, I64, I64, ctypes.POINTER(ctypes.c_int32), I32, qc,
                                st, P, P, P, ctypes.POINTER(D), P, P, P, P, P]),
        "ar_tune_blocks": (st, [ctypes.POINTER(BlockDesc), I32, P, st, I64, I64, qc, op, P, P, P, P,
                                ctypes.POINTER(F), ctypes.POINTER(I32), P]),
        "ar_last_error": (ctypes.c_char_p, []),
        "ar_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != AR_OK:
        raise ARError(status, lib.ar_last_error().decode())


def version() -> str:
    return lib.ar_version().decode()


# ------------------------------------------------------------------ helpers
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return AR_F32
    if t.dtype == torch.bfloat16:
        return AR_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _opt(t, name, dtype, shape):
    return None if t is None else _dev(t, name, dtype, shape)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _group(K: int, group_size: int) -> int:
    return K if group_size == -1 else group_size


@dataclass
class QuantConfig:
    bits: int = 4
    group_size: int = 128
    sym: bool = False

    def c(self) -> QConfig:
        return QConfig(self.bits, self.group_size, int(self.sym))


# ------------------------------------------------------------------ API
def qdq_rtn(W: torch.Tensor, bits: int = 4, group_size: int = 128, V=None, alpha=None, beta=None,
            out_dtype: torch.dtype | None = torch.float32, codes: bool = True, scale_zero: bool = True,
            sym: bool = False, fmt: int = AR_FMT_INT, noalloc: bool = False):
    """Fake-quantize W [N, K]; returns dict(w_hat, codes, scale, zero) (entries
    not requested are None).  V/alpha/beta default to 0/1/1 (RTN).  `fmt`
    selects the integer grid or a float format (AR_FMT_FP8_E4M3 with bits 8,
    AR_FMT_MXFP4 with bits 4 and group_size 32).  `noalloc` calls
    ar_qdq_rtn_noalloc (the library's static device buffer instead of an
    allocation; the outputs here are still torch tensors)."""
    N, K = W.shape
    G = K // _group(K, group_size)
    pw = _dev(W, "W")
    dev = W.device
    out = {"w_hat": None, "codes": None, "scale": None, "zero": None}
    if out_dtype is not None:
        out["w_hat"] = torch.empty((N, K), dtype=out_dtype, device=dev)
    if codes:
        out["codes"] = torch.empty((N, K), dtype=torch.uint8, device=dev)
    if scale_zero:
        out["scale"] = torch.empty((N, G), dtype=torch.float32, device=dev)
        out["zero"] = torch.empty((N, G), dtype=torch.uint8, device=dev)
    q = QConfig(bits, group_size, int(sym), fmt)
    fn = lib.ar_qdq_rtn_noalloc if noalloc else lib.ar_qdq_rtn
    _check(fn(
        pw, _dtype_code(W), N, K, ctypes.byref(q),
        _opt(V, "V", torch.float32, (N, K)), _opt(alpha, "alpha", torch.float32, (N, G)),
        _opt(beta, "beta", torch.float32, (N, G)),
        None if out["w_hat"] is None else out["w_hat"].data_ptr(),
        AR_F32 if out_dtype in (None, torch.float32) else _dtype_code(out["w_hat"]),
        None if out["codes"] is None else out["codes"].data_ptr(),
        None if out["scale"] is None else out["scale"].data_ptr(),
        None if out["zero"] is None else out["zero"].data_ptr(),
        _stream()))
    return out


def pack_int4(W: torch.Tensor, group_size: int = 128, V=None, alpha=None, beta=None, sym: bool = False):
    """INT4 codes of W with the given parameters, packed two per byte (low
    nibble = even column); returns (packed uint8 [N, K/2], scale fp32 [N, G],
    zero uint8 [N, G])."""
    N, K = W.shape
    G = K // _group(K, group_size)
    pw = _dev(W, "W")
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scale = torch.empty((N, G), dtype=torch.float32, device=W.device)
    zero = torch.empty((N, G), dtype=torch.uint8, device=W.device)
    q = QConfig(4, group_size, int(sym))
    _check(lib.ar_pack_int4(
        pw, _dtype_code(W), N, K, ctypes.byref(q),
        _opt(V, "V", torch.float32, (N, K)), _opt(alpha, "alpha", torch.float32, (N, G)),
        _opt(beta, "beta", torch.float32, (N, G)),
        packed.data_ptr(), scale.data_ptr(), zero.data_ptr(), _stream()))
    return packed, scale, zero


def w4a16_gemm(X: torch.Tensor, packed: torch.Tensor, scale: torch.Tensor, zero: torch.Tensor,
               group_size: int = 128, out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None):
    """Y = X * bf16(scale * (q - zero))^T on the packed INT4 weight of
    pack_int4; X bf16 [M, K], packed uint8 [N, K/2] -> Y [M, N] (fp32 sums,
    or their bf16 rounding)."""
    M, K = X.shape
    N = packed.shape[0]
    G = K // _group(K, group_size)
    px = _dev(X, "X", torch.bfloat16)
    pp = _dev(packed, "packed", torch.uint8, (N, K // 2))
    ps = _dev(scale, "scale", torch.float32, (N, G))
    pz = _dev(zero, "zero", torch.uint8, (N, G))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    py = _dev(out, "out", out_dtype, (M, N))
    _check(lib.ar_w4a16_gemm(px, AR_BF16, M, K, pp, ps, pz, N, group_size, py, _dtype_code(out), _stream()))
    return out


def layer_grads(W: torch.Tensor, X_pool: torch.Tensor, ids, V, alpha, beta, bits: int = 4,
                group_size: int = 128, gemm_mode: int = AR_GEMM_BF16, sym: bool = False):
    """Loss and STE gradients at (V, alpha, beta) on the samples `ids` of the
    pool X_pool [S, T, K]; returns dict(loss, G, dV, dalpha, dbeta)."""
    N, K = W.shape
    S, T, K2 = X_pool.shape
    if K2 != K:
        raise ValueError("X_pool and W disagree on K")
    G = K // _group(K, group_size)
    ids_arr = (ctypes.c_int32 * len(ids))(*[int(i) for i in ids])
    dev = W.device
    res = {
        "G": torch.empty((N, K), dtype=torch.float32, device=dev),
        "dV": torch.empty((N, K), dtype=torch.float32, device=dev),
        "dalpha": torch.empty((N, G), dtype=torch.float32, device=dev),
        "dbeta": torch.empty((N, G), dtype=torch.float32, device=dev),
    }
    loss = ctypes.c_double(0.0)
    q = QConfig(bits, group_size, int(sym))
    _check(lib.ar_layer_grads(
        _dev(W, "W"), _dtype_code(W), N, K, _dev(X_pool, "X_pool"), _dtype_code(X_pool), S, T,
        ids_arr, len(ids), ctypes.byref(q), gemm_mode,
        _dev(V, "V", torch.float32, (N, K)), _dev(alpha, "alpha", torch.float32, (N, G)),
        _dev(beta, "beta", torch.float32, (N, G)), ctypes.byref(loss),
        res["G"].data_ptr(), res["dV"].data_ptr(), res["dalpha"].data_ptr(), res["dbeta"].data_ptr(),
        _stream()))
    res["loss"] = loss.value
    return res


def default_opts(preset: int = AR_PRESET_DEFAULT) -> TuneOpts:
    o = TuneOpts()
    _check(lib.ar_tune_opts_init(ctypes.byref(o), preset))
    return o


def _make_opts(iters, lr, lr_clip, lr_decay, clip, batch_samples, schedule, gemm_mode, return_last, unfused=False,
               start_step=0, best_loss_in=float("inf")):
    o = default_opts()
    o.unfused = int(unfused)
    o.start_step = int(start_step)
    o.best_loss_in = float(best_loss_in)
    o.iters = iters
    o.lr = lr
    o.lr_clip = lr if lr_clip is None else lr_clip
    o.lr_decay = int(lr_decay)
    o.clip_lo, o.clip_hi = clip
    o.batch_samples = batch_samples
    o.gemm_mode = gemm_mode
    o.return_last = int(return_last)
    keep = []
    if schedule is not None:
        flat = [int(v) for row in schedule for v in row]
        if len(flat) != iters * batch_samples:
            raise ValueError("schedule must have iters x batch_samples entries")
        arr = (ctypes.c_int32 * len(flat))(*flat)
        keep.append(arr)
        o.schedule = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return o, keep


def _trace(iters):
    """Host loss trace for the C ABI, NaN where no step of the call wrote."""
    tr = (ctypes.c_float * max(iters, 1))()
    for i in range(max(iters, 1)):
        tr[i] = float("nan")
    return tr


class Tuner:
    """Stepwise SignSGD tuning of one linear layer (ar_tuner_*).  With
    start_step > 0 the tuner resumes an iters-step run at that step (the
    state passed in is the one before it); best_loss_in is the best loss of
    the earlier steps."""

    def __init__(self, W, X_pool, bits=4, group_size=128, iters=200, lr=0.005, lr_clip=None,
                 lr_decay=True, clip=(0.5, 1.0), batch_samples=8, schedule=None,
                 gemm_mode=AR_GEMM_BF16, return_last=False, V0=None, alpha0=None, beta0=None, unfused=False,
                 sym=False, start_step=0, best_loss_in=float("inf")):
        N, K = W.shape
        S, T, K2 = X_pool.shape
        if K2 != K:
            raise ValueError("X_pool and W disagree on K")
        self.N, self.K, self.G = N, K, K // _group(K, group_size)
        self.iters = iters
        dev = W.device
        self.V0 = torch.zeros((N, K), dtype=torch.float32, device=dev) if V0 is None else V0
        self.alpha0 = torch.ones((N, self.G), dtype=torch.float32, device=dev) if alpha0 is None else alpha0
        self.beta0 = torch.ones((N, self.G), dtype=torch.float32, device=dev) if beta0 is None else beta0
        self._opts, self._keep = _make_opts(iters, lr, lr_clip, lr_decay, clip, batch_samples, schedule,
                                            gemm_mode, return_last, unfused, start_step, best_loss_in)
        self._trace = _trace(iters)
        self._opts.loss_trace = ctypes.cast(self._trace, ctypes.POINTER(ctypes.c_float))
        self._q = QConfig(bits, group_size, int(sym))
        self._W, self._X = W, X_pool      # keep the caller's tensors alive
        h = ctypes.c_void_p()
        _check(lib.ar_tuner_create(
            ctypes.byref(h), _dev(W, "W"), _dtype_code(W), N, K, _dev(X_pool, "X_pool"), _dtype_code(X_pool), S, T,
            ctypes.byref(self._q), ctypes.byref(self._opts),
            _dev(self.V0, "V0", torch.float32, (N, K)), _dev(self.alpha0, "alpha0", torch.float32, (N, self.G)),
            _dev(self.beta0, "beta0", torch.float32, (N, self.G)), _stream()))
        self._h = h

    def run(self, nsteps: int, graph: bool = True, events: bool = False, kernel_graphs: bool = False) -> None:
        """Enqueue nsteps steps (captured graphs or eager launches); `events`
        times every kernel of eager steps, `kernel_graphs` times each kernel
        in a graph of nsteps launches of it alone (timing only)."""
        flags = ((AR_RUN_GRAPH if graph else 0) | (AR_RUN_EVENTS if events else 0)
                 | (AR_RUN_KERNEL_GRAPHS if kernel_graphs else 0))
        _check(lib.ar_tuner_run(self._h, nsteps, flags))

    def kernel_ms(self) -> dict:
        n = lib.ar_tuner_num_kernels(self._h)
        arr = (ctypes.c_float * n)()
        _check(lib.ar_tuner_kernel_ms(self._h, arr))
        return {lib.ar_tuner_kernel_name(self._h, i).decode(): float(arr[i]) for i in range(n)}

    def finish(self):
        dev = self._W.device
        V = torch.empty((self.N, self.K), dtype=torch.float32, device=dev)
        al = torch.empty((self.N, self.G), dtype=torch.float32, device=dev)
        be = torch.empty((self.N, self.G), dtype=torch.float32, device=dev)
        bl = ctypes.c_float(0.0)
        bs = ctypes.c_int32(-1)
        status = lib.ar_tuner_finish(self._h, V.data_ptr(), al.data_ptr(), be.data_ptr(), ctypes.byref(bl),
                                     ctypes.byref(bs))
        out = dict(V=V, alpha=al, beta=be, best_loss=bl.value, best_step=bs.value,
                   losses=[float(self._trace[i]) for i in range(self.iters)])
        _check(status)
        return out

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib.ar_tuner_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tune_layer(W, X_pool, bits=4, group_size=128, iters=200, lr=0.005, lr_clip=None, lr_decay=True,
               clip=(0.5, 1.0), batch_samples=8, schedule=None, gemm_mode=AR_GEMM_BF16, return_last=False,
               V0=None, alpha0=None, beta0=None, unfused=False, sym=False, start_step=0,
               best_loss_in=float("inf")):
    """ar_tune_layer: returns dict(V, alpha, beta, best_loss, best_step, losses).  start_step > 0
    resumes an iters-step run at that step from the state (V0, alpha0, beta0), with best_loss_in the best
    loss of the earlier steps; losses before start_step are NaN, and best_step is -1 when no step of this
    call improved on best_loss_in (V, alpha, beta are then the state after the last update)."""
    N, K = W.shape
    S, T, K2 = X_pool.shape
    if K2 != K:
        raise ValueError("X_pool and W disagree on K")
    G = K // _group(K, group_size)
    dev = W.device
    V = (torch.zeros((N, K), dtype=torch.float32, device=dev) if V0 is None else V0.clone())
    al = (torch.ones((N, G), dtype=torch.float32, device=dev) if alpha0 is None else alpha0.clone())
    be = (torch.ones((N, G), dtype=torch.float32, device=dev) if beta0 is None else beta0.clone())
    opts, keep = _make_opts(iters, lr, lr_clip, lr_decay, clip, batch_samples, schedule, gemm_mode, return_last,
                            unfused, start_step, best_loss_in)
    trace = _trace(iters)
    opts.loss_trace = ctypes.cast(trace, ctypes.POINTER(ctypes.c_float))
    q = QConfig(bits, group_size, int(sym))
    bl = ctypes.c_float(0.0)
    bs = ctypes.c_int32(-1)
    _check(lib.ar_tune_layer(
        _dev(W, "W"), _dtype_code(W), N, K, _dev(X_pool, "X_pool"), _dtype_code(X_pool), S, T,
        ctypes.byref(q), ctypes.byref(opts),
        _dev(V, "V", torch.float32, (N, K)), _dev(al, "alpha", torch.float32, (N, G)),
        _dev(be, "beta", torch.float32, (N, G)), ctypes.byref(bl), ctypes.byref(bs), _stream()))
    del keep
    return dict(V=V, alpha=al, beta=be, best_loss=bl.value, best_step=bs.value,
                losses=[float(trace[i]) for i in range(iters)])


def _block_desc(gate, up, down) -> BlockDesc:
    F, H = gate.shape
    if tuple(up.shape) != (F, H) or tuple(down.shape) != (H, F):
        raise ValueError("expected gate, up [F, H] and down [H, F]")
    if not (gate.dtype == up.dtype == down.dtype):
        raise TypeError("the three weights must share a dtype")
    d = BlockDesc()
    d.kind = AR_BLOCK_MLP_SWIGLU
    d.weight_dtype = _dtype_code(gate)
    d.hidden, d.ffn = H, F
    for i, (w, nm) in enumerate(zip((gate, up, down), LINEARS)):
        d.weights[i] = _dev(w, nm)
    return d


def _ptrs(ts, names, shapes):
    return (ctypes.c_void_p * len(ts))(*[_dev(t, n, torch.float32, sh) for t, n, sh in zip(ts, names, shapes)])


def _param_shapes(wshapes, group_size):
    """V shapes and alpha/beta shapes of linears with weight shapes [N, K]."""
    vs = [tuple(sh) for sh in wshapes]
    gs = [(n, k // _group(k, group_size)) for n, k in wshapes]
    return vs, gs


def _block_shapes(gate, group_size):
    F, H = gate.shape
    return _param_shapes([(F, H), (F, H), (H, F)], group_size)


def _init_params(names, vs, gs, dev, params):
    out = {}
    for i, nm in enumerate(names):
        if params is not None and nm in params:
            V, al, be = params[nm]
            out[nm] = (V.clone(), al.clone(), be.clone())
        else:
            out[nm] = (torch.zeros(vs[i], dtype=torch.float32, device=dev),
                       torch.ones(gs[i], dtype=torch.float32, device=dev),
                       torch.ones(gs[i], dtype=torch.float32, device=dev))
    return out


def _block_init(gate, group_size, params):
    vs, gs = _block_shapes(gate, group_size)
    return _init_params(LINEARS, vs, gs, gate.device, params)


def _tune_desc(d, names, vs, gs, X_pool, p, bits, group_size, iters, lr, lr_clip, lr_decay, clip,
               batch_samples, schedule, gemm_mode, return_last, unfused, sym, output, start_step=0,
               best_loss_in=float("inf")):
    S, T, H = X_pool.shape
    if H != d.hidden:
        raise ValueError("X_pool and the weights disagree on the hidden size")
    n = len(names)
    opts, keep = _make_opts(iters, lr, lr_clip, lr_decay, clip, batch_samples, schedule, gemm_mode, return_last,
                            unfused, start_step, best_loss_in)
    trace = _trace(iters)
    opts.loss_trace = ctypes.cast(trace, ctypes.POINTER(ctypes.c_float))
    q = QConfig(bits, group_size, int(sym))
    Y = torch.empty((S, T, H), dtype=X_pool.dtype, device=X_pool.device) if output else None
    bl = ctypes.c_float(0.0)
    bs = ctypes.c_int32(-1)
    _check(lib.ar_tune_block(
        ctypes.byref(d), _dev(X_pool, "X_pool"), _dtype_code(X_pool), S, T, ctypes.byref(q), ctypes.byref(opts),
        _ptrs([p[m][0] for m in names], ["V"] * n, vs), _ptrs([p[m][1] for m in names], ["alpha"] * n, gs),
        _ptrs([p[m][2] for m in names], ["beta"] * n, gs), None if Y is None else Y.data_ptr(),
        ctypes.byref(bl), ctypes.byref(bs), _stream()))
    del keep
    return dict(params=p, best_loss=bl.value, best_step=bs.value, losses=[float(trace[i]) for i in range(iters)],
                output=Y)


def tune_block(gate, up, down, X_pool, bits=4, group_size=128, iters=200, lr=0.005, lr_clip=None, lr_decay=True,
               clip=(0.5, 1.0), batch_samples=8, schedule=None, gemm_mode=AR_GEMM_BF16, return_last=False,
               params=None, unfused=False, sym=False, output=True, start_step=0, best_loss_in=float("inf")):
    """ar_tune_block on a SwiGLU MLP block (gate/up [F, H], down [H, F]) with
    block input X_pool [S, T, H].  Returns dict(params={name: (V, alpha,
    beta)}, best_loss, best_step, losses, output) where output is the quantized
    block's output [S, T, H] (the next block's input) or None."""
    d = _block_desc(gate, up, down)
    vs, gs = _block_shapes(gate, group_size)
    p = _block_init(gate, group_size, params)
    return _tune_desc(d, LINEARS, vs, gs, X_pool, p, bits, group_size, iters, lr, lr_clip, lr_decay, clip,
                      batch_samples, schedule, gemm_mode, return_last, unfused, sym, output, start_step,
                      best_loss_in)


class _DescTuner:
    """Stepwise block-wise tuning through ar_block_tuner_* (one loss and one
    snapshot for all linears named in `names`)."""

    def _create(self, d, names, shapes, keepalive, X_pool, params, bits, group_size, iters, lr, lr_clip, lr_decay,
                clip, batch_samples, schedule, gemm_mode, return_last, unfused, sym):
        S, T, H = X_pool.shape
        self._d, self._names, self._shapes = d, names, shapes
        self.iters = iters
        vs, gs = shapes
        self._init = _init_params(names, vs, gs, X_pool.device, params)
        self._opts, self._keep = _make_opts(iters, lr, lr_clip, lr_decay, clip, batch_samples, schedule,
                                            gemm_mode, return_last, unfused)
        self._trace = _trace(iters)
        self._opts.loss_trace = ctypes.cast(self._trace, ctypes.POINTER(ctypes.c_float))
        self._q = QConfig(bits, group_size, int(sym))
        self._keepalive = keepalive
        self._X = X_pool
        n = len(names)
        h = ctypes.c_void_p()
        _check(lib.ar_block_tuner_create(
            ctypes.byref(h), ctypes.byref(self._d), _dev(X_pool, "X_pool"), _dtype_code(X_pool), S, T,
            ctypes.byref(self._q), ctypes.byref(self._opts),
            _ptrs([self._init[m][0] for m in names], ["V0"] * n, vs),
            _ptrs([self._init[m][1] for m in names], ["alpha0"] * n, gs),
            _ptrs([self._init[m][2] for m in names], ["beta0"] * n, gs), _stream()))
        self._h = h

    run = Tuner.run
    kernel_ms = Tuner.kernel_ms
    close = Tuner.close
    __del__ = Tuner.__del__

    def finish(self, output: bool = False):
        vs, gs = self._shapes
        names, dev, n = self._names, self._X.device, len(self._names)
        p = {m: (torch.empty(vs[i], dtype=torch.float32, device=dev),
                 torch.empty(gs[i], dtype=torch.float32, device=dev),
                 torch.empty(gs[i], dtype=torch.float32, device=dev)) for i, m in enumerate(names)}
        Y = torch.empty(self._X.shape, dtype=self._X.dtype, device=dev) if output else None
        bl = ctypes.c_float(0.0)
        bs = ctypes.c_int32(-1)
        status = lib.ar_block_tuner_finish(
            self._h, _ptrs([p[m][0] for m in names], ["V"] * n, vs),
            _ptrs([p[m][1] for m in names], ["alpha"] * n, gs), _ptrs([p[m][2] for m in names], ["beta"] * n, gs),
            None if Y is None else Y.data_ptr(), ctypes.byref(bl), ctypes.byref(bs))
        out = dict(params=p, best_loss=bl.value, best_step=bs.value, output=Y,
                   losses=[float(self._trace[i]) for i in range(self.iters)])
        _check(status)
        return out


class BlockTuner(_DescTuner):
    """Stepwise block-wise tuning of a SwiGLU MLP block (ar_block_tuner_*)."""

    def __init__(self, gate, up, down, X_pool, bits=4, group_size=128, iters=200, lr=0.005, lr_clip=None,
                 lr_decay=True, clip=(0.5, 1.0), batch_samples=8, schedule=None, gemm_mode=AR_GEMM_BF16,
                 return_last=False, params=None, unfused=False, sym=False):
        self._create(_block_desc(gate, up, down), LINEARS, _block_shapes(gate, group_size), (gate, up, down),
                     X_pool, params, bits, group_size, iters, lr, lr_clip, lr_decay, clip, batch_samples, schedule,
                     gemm_mode, return_last, unfused, sym)


def _grads_desc(d, names, vs, gs, X_pool, ids, p, bits, group_size, gemm_mode, sym):
    S, T, H = X_pool.shape
    dev = X_pool.device
    n = len(names)
    res = {k: {m: torch.empty(sh[i], dtype=torch.float32, device=dev) for i, m in enumerate(names)}
           for k, sh in (("G", vs), ("dV", vs), ("dalpha", gs), ("dbeta", gs))}
    ids_arr = (ctypes.c_int32 * len(ids))(*[int(i) for i in ids])
    loss = ctypes.c_double(0.0)
    q = QConfig(bits, group_size, int(sym))
    out_ptrs = {k: (ctypes.c_void_p * n)(*[res[k][m].data_ptr() for m in names]) for k in res}
    _check(lib.ar_block_grads(
        ctypes.byref(d), _dev(X_pool, "X_pool"), _dtype_code(X_pool), S, T, ids_arr, len(ids), ctypes.byref(q),
        gemm_mode, _ptrs([p[m][0] for m in names], ["V"] * n, vs), _ptrs([p[m][1] for m in names], ["alpha"] * n, gs),
        _ptrs([p[m][2] for m in names], ["beta"] * n, gs), ctypes.byref(loss),
        out_ptrs["G"], out_ptrs["dV"], out_ptrs["dalpha"], out_ptrs["dbeta"], _stream()))
    res["loss"] = loss.value
    return res


def block_grads(gate, up, down, X_pool, ids, params=None, bits=4, group_size=128, gemm_mode=AR_GEMM_BF16,
                sym=False):
    """Block loss and STE gradients at `params` ({name: (V, alpha, beta)},
    default RTN) on the samples `ids`; returns dict(loss, G, dV, dalpha, dbeta)
    with one tensor per linear name."""
    d = _block_desc(gate, up, down)
    vs, gs = _block_shapes(gate, group_size)
    p = _block_init(gate, group_size, params)
    return _grads_desc(d, LINEARS, vs, gs, X_pool, ids, p, bits, group_size, gemm_mode, sym)


# ------------------------------------------------------ Llama decoder block
def decoder_weight_shapes(hidden, ffn, heads, kv_heads, head_dim):
    """[N, K] of q, k, v, o, gate, up, down."""
    nq, nkv = heads * head_dim, kv_heads * head_dim
    return [(nq, hidden), (nkv, hidden), (nkv, hidden), (hidden, nq), (ffn, hidden), (ffn, hidden), (hidden, ffn)]


def _decoder_desc(weights, heads, kv_heads, head_dim, norm_weights, eps, theta):
    H = weights["q"].shape[1]
    F = weights["gate"].shape[0]
    shapes = decoder_weight_shapes(H, F, heads, kv_heads, head_dim)
    dt = weights["q"].dtype
    d = BlockDesc()
    d.kind = AR_BLOCK_LLAMA_DECODER
    d.weight_dtype = _dtype_code(weights["q"])
    d.hidden, d.ffn, d.heads, d.kv_heads, d.head_dim = H, F, heads, kv_heads, head_dim
    d.norm_eps, d.rope_theta = eps, theta
    for i, (nm, sh) in enumerate(zip(DECODER_LINEARS, shapes)):
        d.weights[i] = _dev(weights[nm], nm, dt, sh)
    nw = norm_weights if norm_weights is not None else (None, None)
    for i in range(2):
        d.norm_weights[i] = _opt(nw[i], f"norm_weights[{i}]", torch.float32, (H,))
    return d, shapes


def tune_decoder(weights, X_pool, heads, kv_heads, head_dim, norm_weights=None, eps=1e-5, theta=10000.0, bits=4,
                 group_size=128, iters=200, lr=0.005, lr_clip=None, lr_decay=True, clip=(0.5, 1.0),
                 batch_samples=8, schedule=None, return_last=False, params=None, unfused=False, sym=False,
                 output=True, start_step=0, best_loss_in=float("inf")):
    """ar_tune_block on a Llama decoder block: `weights` maps q, k, v, o, gate,
    up, down to bf16 tensors of decoder_weight_shapes; norm_weights = (w1, w2)
    fp32 [H] or None (= 1).  Returns what tune_block returns, with the seven
    linears in params."""
    d, shapes = _decoder_desc(weights, heads, kv_heads, head_dim, norm_weights, eps, theta)
    vs, gs = _param_shapes(shapes, group_size)
    p = _init_params(DECODER_LINEARS, vs, gs, X_pool.device, params)
    return _tune_desc(d, DECODER_LINEARS, vs, gs, X_pool, p, bits, group_size, iters, lr, lr_clip, lr_decay, clip,
                      batch_samples, schedule, AR_GEMM_BF16, return_last, unfused, sym, output, start_step,
                      best_loss_in)


class DecoderTuner(_DescTuner):
    """Stepwise block-wise tuning of a Llama decoder block (ar_block_tuner_*)."""

    def __init__(self, weights, X_pool, heads, kv_heads, head_dim, norm_weights=None, eps=1e-5, theta=10000.0,
                 bits=4, group_size=128, iters=200, lr=0.005, lr_clip=None, lr_decay=True, clip=(0.5, 1.0),
                 batch_samples=8, schedule=None, return_last=False, params=None, unfused=False, sym=False):
        d, shapes = _decoder_desc(weights, heads, kv_heads, head_dim, norm_weights, eps, theta)
        self._create(d, DECODER_LINEARS, _param_shapes(shapes, group_size), (weights, norm_weights), X_pool,
                     params, bits, group_size, iters, lr, lr_clip, lr_decay, clip, batch_samples, schedule,
                     AR_GEMM_BF16, return_last, unfused, sym)


def decoder_grads(weights, X_pool, ids, heads, kv_heads, head_dim, norm_weights=None, eps=1e-5, theta=10000.0,
                  params=None, bits=4, group_size=128, sym=False):
    """Decoder-block loss and STE gradients of the seven linears at `params`
    (default RTN) on the samples `ids`; returns dict(loss, G, dV, dalpha,
    dbeta), one tensor per linear name."""
    d, shapes = _decoder_desc(weights, heads, kv_heads, head_dim, norm_weights, eps, theta)
    vs, gs = _param_shapes(shapes, group_size)
    p = _init_params(DECODER_LINEARS, vs, gs, X_pool.device, params)
    return _grads_desc(d, DECODER_LINEARS, vs, gs, X_pool, ids, p, bits, group_size, AR_GEMM_BF16, sym)


# --------------------------------------- block-by-block stack, host weights
def _host(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cpu":
        raise ValueError(f"{name} must be in host memory (a CPU tensor), got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def tune_blocks(blocks, X_pool, heads=None, kv_heads=None, head_dim=None, eps=1e-5, theta=10000.0, bits=4,
                group_size=128, iters=200, lr=0.005, lr_clip=None, lr_decay=True, clip=(0.5, 1.0), batch_samples=8,
                schedule=None, gemm_mode=AR_GEMM_BF16, return_last=False, unfused=False, sym=False, output=True,
                params=None, pin=True, inplace=False):
    """ar_tune_blocks: block-by-block quantization of a stack of blocks whose
    weights stay in host memory.  `blocks` is a list of dicts of CPU tensors:
    SwiGLU MLP blocks {gate, up, down}, or (with heads, kv_heads, head_dim)
    Llama decoder blocks {q, k, v, o, gate, up, down} plus optional fp32 [H]
    norm1 / norm2.  Block b is tuned on block b-1's quantized output, block 0
    on X_pool (device).  The parameters live in host memory (page-locked when
    `pin`), initialised to V = 0, alpha = beta = 1 unless `params` (a list of
    {name: (V, alpha, beta)} CPU tensors per block) is given; with `inplace`
    the given tensors (contiguous fp32, host) are passed as they are and
    receive the tuned state.  Returns
    dict(params=[{name: (V, alpha, beta)}], best_losses, best_steps,
    losses=[[per-step loss] per block], output) with output the last block's
    quantized output [S, T, H] on the device, or None."""
    S, T, H = X_pool.shape
    nb = len(blocks)
    descs = (BlockDesc * max(nb, 1))()
    names_of, shapes_of = [], []
    for b, w in enumerate(blocks):
        d = descs[b]
        dec = "q" in w
        names = DECODER_LINEARS if dec else LINEARS
        if dec:
            if heads is None or kv_heads is None or head_dim is None:
                raise ValueError("decoder blocks need heads, kv_heads and head_dim")
            Hb, F = w["q"].shape[1], w["gate"].shape[0]
            shapes = decoder_weight_shapes(Hb, F, heads, kv_heads, head_dim)
            d.kind = AR_BLOCK_LLAMA_DECODER
            d.heads, d.kv_heads, d.head_dim = heads, kv_heads, head_dim
            d.norm_eps, d.rope_theta = eps, theta
            for j, key in enumerate(("norm1", "norm2")):
                nw = w.get(key)
                d.norm_weights[j] = None if nw is None else _host(nw, f"blocks[{b}].{key}", torch.float32, (Hb,))
        else:
            F, Hb = w["gate"].shape
            shapes = [(F, Hb), (F, Hb), (Hb, F)]
            d.kind = AR_BLOCK_MLP_SWIGLU
        d.hidden, d.ffn = Hb, F
        dt = w[names[0]].dtype
        d.weight_dtype = _dtype_code(w[names[0]])
        for i, (nm, sh) in enumerate(zip(names, shapes)):
            d.weights[i] = _host(w[nm], f"blocks[{b}].{nm}", dt, sh)
        names_of.append(names)
        shapes_of.append(_param_shapes(shapes, group_size))
    pinned = pin and torch.cuda.is_available()
    p = []
    for b in range(nb):
        vs, gs = shapes_of[b]
        given = params[b] if params is not None else {}
        if inplace:
            if set(given) != set(names_of[b]):
                raise ValueError(f"inplace needs params for every linear of block {b}")
            p.append({nm: tuple(given[nm]) for nm in names_of[b]})
            continue
        pb = {}
        for i, nm in enumerate(names_of[b]):
            fill = [torch.zeros(vs[i]), torch.ones(gs[i]), torch.ones(gs[i])]
            if nm in given:
                fill = [a.detach().to("cpu", torch.float32) for a in given[nm]]
            pb[nm] = tuple(torch.empty(a.shape, dtype=torch.float32, pin_memory=pinned).copy_(a) for a in fill)
        p.append(pb)
    ptr = {k: (ctypes.c_void_p * (7 * max(nb, 1)))() for k in range(3)}
    for b in range(nb):
        vs, gs = shapes_of[b]
        for i, nm in enumerate(names_of[b]):
            for k in range(3):
                ptr[k][7 * b + i] = _host(p[b][nm][k], ("V", "alpha", "beta")[k], torch.float32,
                                          vs[i] if k == 0 else gs[i])
    opts, keep = _make_opts(iters, lr, lr_clip, lr_decay, clip, batch_samples, schedule, gemm_mode, return_last,
                            unfused)
    trace = _trace(iters * max(nb, 1))
    opts.loss_trace = ctypes.cast(trace, ctypes.POINTER(ctypes.c_float))
    q = QConfig(bits, group_size, int(sym))
    Y = torch.empty((S, T, H), dtype=X_pool.dtype, device=X_pool.device) if output else None
    bl = (ctypes.c_float * max(nb, 1))()
    bs = (ctypes.c_int32 * max(nb, 1))()
    _check(lib.ar_tune_blocks(
        descs, nb, _dev(X_pool, "X_pool"), _dtype_code(X_pool), S, T, ctypes.byref(q), ctypes.byref(opts),
        ptr[0], ptr[1], ptr[2], None if Y is None else Y.data_ptr(), bl, bs, _stream()))
    del keep
    return dict(params=p, best_losses=[bl[b] for b in range(nb)], best_steps=[bs[b] for b in range(nb)],
                losses=[[float(trace[b * iters + i]) for i in range(iters)] for b in range(nb)], output=Y)
