"""Thin ctypes binding over libqlora.so (include/qlora.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every arithmetic step runs in the library's HIP kernels.  If the
library is missing this module raises; there is no CPU fallback.
"""

import contextlib
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqlora.so")

QL_OK = 0
QL_EINVAL, QL_EUNSUPPORTED, QL_EWORKSPACE, QL_EHIP, QL_ENONFINITE, QL_ESTATE, QL_EOVERFLOW = (
    -1, -2, -3, -4, -5, -6, -7)
FMT_Q4_0, FMT_NF4, FMT_FP8, FMT_MXFP4, FMT_Q8_0, FMT_NVFP4 = 1, 2, 3, 4, 5, 6
OP_PACK, OP_FWD, OP_BWD = 0, 1, 2
BLOCK = {FMT_Q4_0: 32, FMT_NF4: 64, FMT_FP8: 32, FMT_MXFP4: 32, FMT_Q8_0: 32, FMT_NVFP4: 32}

EXPORTS = (
    "ql_last_error", "ql_version", "ql_nf4_levels", "qlora_workspace_bytes", "quant_pack",
    "qlora_dequant", "ql_act_quant_e4m3", "qlora_linear_fwd", "qlora_linear_bwd",
    "ql_pool_create", "layer_stream_prefetch", "ql_pool_acquire", "ql_pool_release",
    "ql_pool_stats", "ql_pool_debug", "ql_pool_destroy", "ql_adamw_step",
    "ql_plan_create", "ql_plan_add_fwd", "ql_plan_add_bwd", "ql_plan_add_event", "ql_plan_size",
    "ql_plan_run", "ql_plan_destroy", "qlora_linear_fwd_group", "qlora_linear_bwd_group",
    "ql_plan_add_fwd_group", "ql_plan_add_bwd_group", "ql_stack_adapters", "qlora_linear_bwd_noalloc",
    "ql_adamw8_step", "ql_dyn8_levels", "ql_stream_read",
)
ADAMW8_BLOCK = 2048
STREAM_READ_THREADS = 65536
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
STACK_MAX = 8
GROUP_MAX = 8
ADAMW_MAX_TENSORS = 32


class QLError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libqlora error {code}: {msg}")
        self.code = code


class QWeightC(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_out", ctypes.c_int64), ("k_in", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class FwdCallC(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("lora_a", ctypes.c_void_p),
                ("lora_b", ctypes.c_void_p), ("alpha", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("y", ctypes.c_void_p), ("u_save", ctypes.c_void_p), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t)]


class BwdCallC(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("dy", ctypes.c_void_p),
                ("u_save", ctypes.c_void_p), ("lora_a", ctypes.c_void_p), ("lora_b", ctypes.c_void_p),
                ("alpha", ctypes.c_float), ("accumulate", ctypes.c_int32), ("dx", ctypes.c_void_p),
                ("d_a", ctypes.c_void_p), ("d_b", ctypes.c_void_p), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t)]


class AdapterC(ctypes.Structure):
    _fields_ = [("lora_a", ctypes.c_void_p), ("lora_b", ctypes.c_void_p), ("r", ctypes.c_int32),
                ("alpha", ctypes.c_float)]


class AdamwTensorC(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("param_bf16", ctypes.c_void_p), ("n", ctypes.c_int64)]


class Adamw8TensorC(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_absmax", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("exp_avg_sq_absmax", ctypes.c_void_p), ("param_bf16", ctypes.c_void_p), ("n", ctypes.c_int64)]


class AdamwHparamsC(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("grad_scale", ctypes.c_double),
                ("step", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def load(path=LIB_PATH):
    """Load libqlora.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with python -m quantized_base_lora_amd.build")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    QW = ctypes.POINTER(QWeightC)
    sig = {
        "ql_last_error": (ctypes.c_char_p, []),
        "ql_version": (I32, []),
        "ql_nf4_levels": (ctypes.c_int, [P]),
        "qlora_workspace_bytes": (SZ, [I32, I32, I64, I64, I64, I32]),
        "quant_pack": (ctypes.c_int, [I32, P, I64, I64, P, P, P, SZ, P]),
        "qlora_dequant": (ctypes.c_int, [QW, P, P, P]),
        "ql_act_quant_e4m3": (ctypes.c_int, [P, I64, I64, P, P, P, P]),
        "qlora_linear_fwd": (ctypes.c_int, [QW, P, I64, P, P, I32, F, P, P, P, SZ, P]),
        "qlora_linear_bwd": (ctypes.c_int, [QW, P, P, P, I64, P, P, I32, F, P, P, P, I32, P, SZ, P]),
        "qlora_linear_bwd_noalloc": (ctypes.c_int, [QW, P, P, P, I64, P, P, I32, F, P, P, P, I32, P]),
        "ql_pool_create": (ctypes.c_int, [ctypes.POINTER(P), I32, ctypes.POINTER(P), SZ, I32,
                                          ctypes.POINTER(P), ctypes.POINTER(SZ)]),
        "layer_stream_prefetch": (ctypes.c_int, [P, I32, P]),
        "ql_pool_acquire": (ctypes.c_int, [P, I32, P, ctypes.POINTER(P)]),
        "ql_pool_release": (ctypes.c_int, [P, I32, P]),
        "ql_pool_stats": (ctypes.c_int, [P, ctypes.POINTER(I64)]),
        "ql_pool_debug": (ctypes.c_int, [P, I32, I32, I32]),
        "ql_pool_destroy": (ctypes.c_int, [P]),
        "ql_adamw_step": (ctypes.c_int, [ctypes.POINTER(AdamwTensorC), I32,
                                         ctypes.POINTER(AdamwHparamsC), P]),
        "ql_plan_create": (ctypes.c_int, [ctypes.POINTER(P)]),
        "ql_plan_add_fwd": (ctypes.c_int, [P, QW, P, I64, P, P, I32, F, P, P, P, SZ]),
        "ql_plan_add_bwd": (ctypes.c_int, [P, QW, P, P, P, I64, P, P, I32, F, P, P, P, I32, P, SZ]),
        "ql_plan_add_event": (ctypes.c_int, [P, P]),
        "ql_plan_size": (ctypes.c_int, [P]),
        "ql_plan_run": (ctypes.c_int, [P, P]),
        "ql_plan_destroy": (ctypes.c_int, [P]),
        "qlora_linear_fwd_group": (ctypes.c_int, [ctypes.POINTER(FwdCallC), I32, I64, I32, P]),
        "qlora_linear_bwd_group": (ctypes.c_int, [ctypes.POINTER(BwdCallC), I32, I64, I32, P]),
        "ql_plan_add_fwd_group": (ctypes.c_int, [P, ctypes.POINTER(FwdCallC), I32, I64, I32]),
        "ql_plan_add_bwd_group": (ctypes.c_int, [P, ctypes.POINTER(BwdCallC), I32, I64, I32]),
        "ql_adamw8_step": (ctypes.c_int, [ctypes.POINTER(Adamw8TensorC), I32,
                                          ctypes.POINTER(AdamwHparamsC), P]),
        "ql_dyn8_levels": (ctypes.c_int, [I32, P]),
        "ql_stream_read": (ctypes.c_int, [P, I64, P, P]),
        "ql_stack_adapters": (ctypes.c_int, [ctypes.POINTER(AdapterC), I32, I64, I64, P, P,
                                             ctypes.POINTER(ctypes.c_float), P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _check(rc):
    if rc != QL_OK:
        raise QLError(rc, load().ql_last_error().decode())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context for a call's temporaries: the caching allocator then
    ties them to the stream the library enqueues on, so a temporary freed on
    return is not reused by other work until that stream has passed the call."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


# ----------------------------------------------------------------------------- plain queries

def version():
    return load().ql_version()


def nf4_levels():
    """The library's NF4 levels (host call, needs no GPU)."""
    buf = (ctypes.c_float * 16)()
    _check(load().ql_nf4_levels(buf))
    return [float(v) for v in buf]


def workspace_bytes(op, fmt, n, k, m=0, r=16):
    return int(load().qlora_workspace_bytes(op, fmt, n, k, m, r))


# ----------------------------------------------------------------------------- packed weight

class QWeight:
    """A packed frozen base weight: codes and scales tensors plus shape and format."""

    def __init__(self, fmt, n, k, codes, scales):
        self.fmt, self.n, self.k = int(fmt), int(n), int(k)
        self.codes, self.scales = codes, scales
        self._c = QWeightC(self.fmt, 0, self.n, self.k, codes.data_ptr(), scales.data_ptr())

    @property
    def cstruct(self):
        return ctypes.byref(self._c)

    @staticmethod
    def alloc(fmt, n, k, device="cuda"):
        if fmt == FMT_FP8:
            codes = torch.empty((n, k), dtype=torch.uint8, device=device)
            scales = torch.empty(1, dtype=torch.float32, device=device)
        elif fmt == FMT_Q4_0:
            codes = torch.empty((n, k // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((n, k // 32), dtype=torch.int16, device=device)
        elif fmt == FMT_NF4:
            codes = torch.empty((n, k // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((n, k // 64), dtype=torch.float32, device=device)
        elif fmt == FMT_MXFP4:
            codes = torch.empty((n, k // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((n, k // 32), dtype=torch.uint8, device=device)
        elif fmt == FMT_Q8_0:
            codes = torch.empty((n, k), dtype=torch.uint8, device=device)
            scales = torch.empty((n, k // 32), dtype=torch.int16, device=device)
        elif fmt == FMT_NVFP4:
            # the tensor scale and 12 zero bytes, then one E4M3 byte per 16 elements
            codes = torch.empty((n, k // 2), dtype=torch.uint8, device=device)
            scales = torch.empty(16 + n * (k // 16), dtype=torch.uint8, device=device)
        else:
            raise ValueError(f"unknown format {fmt}")
        return QWeight(fmt, n, k, codes, scales)

    @staticmethod
    def view(fmt, n, k, codes_ptr, scales_ptr, keepalive=None):
        """A weight whose codes/scales live at raw device addresses (e.g. a pool slot)."""
        qw = QWeight.__new__(QWeight)
        qw.fmt, qw.n, qw.k = int(fmt), int(n), int(k)
        qw.codes = qw.scales = keepalive
        qw._c = QWeightC(qw.fmt, 0, qw.n, qw.k, int(codes_ptr), int(scales_ptr))
        return qw

    def nbytes(self):
        return self.codes.numel() * self.codes.element_size() + self.scales.numel() * self.scales.element_size()


def quant_pack(fmt, w, out=None, ws=None, stream=None):
    """Pack fp32 W [N, K] (device) into a QWeight (blocks until done)."""
    _need(w, "w", torch.float32)
    n, k = w.shape
    with _on(stream):
        qw = out if out is not None else QWeight.alloc(fmt, n, k, device=w.device)
        if ws is None:
            ws = torch.empty(workspace_bytes(OP_PACK, fmt, n, k), dtype=torch.uint8, device=w.device)
    _check(load().quant_pack(fmt, _ptr(w), n, k, _ptr(qw.codes), _ptr(qw.scales), _ptr(ws),
                             ws.numel(), _stream(stream)))
    return qw


def dequant(qw, want_f32=True, want_bf16=True, stream=None):
    dev = qw.codes.device
    with _on(stream):
        f = torch.empty((qw.n, qw.k), dtype=torch.float32, device=dev) if want_f32 else None
        b = torch.empty((qw.n, qw.k), dtype=torch.bfloat16, device=dev) if want_bf16 else None
    _check(load().qlora_dequant(qw.cstruct, _ptr(f), _ptr(b), _stream(stream)))
    return f, b


def act_quant_e4m3(x, stream=None):
    _need(x, "x", torch.bfloat16)
    m, k = x.shape
    with _on(stream):
        hi = torch.empty((m, k), dtype=torch.uint8, device=x.device)
        lo = torch.empty((m, k), dtype=torch.uint8, device=x.device)
        s = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(load().ql_act_quant_e4m3(_ptr(x), m, k, _ptr(hi), _ptr(lo), _ptr(s), _stream(stream)))
    return hi, lo, s


def stream_read(buf, sink, stream=None):
    """One streaming read of the device tensor buf (the HBM ceiling kernel);
    sink: int32 device tensor of STREAM_READ_THREADS entries, whose XOR is the
    XOR of every 32-bit word of buf."""
    if not buf.is_cuda or not sink.is_cuda or sink.dtype != torch.int32 or sink.numel() != STREAM_READ_THREADS:
        raise ValueError("buf and sink must be device tensors, sink int32 of STREAM_READ_THREADS entries")
    if not buf.is_contiguous() or not sink.is_contiguous():
        raise ValueError("buf and sink must be contiguous")
    _check(load().ql_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


# ----------------------------------------------------------------------------- layer

def linear_fwd(qw, x, a, b, alpha, y=None, u=None, ws=None, stream=None):
    """y = x.deq(W)^T + (alpha/r).(x.A^T).B^T ; returns (y, U)."""
    m = x.shape[0]
    r = a.shape[0]
    _need(x, "x", torch.bfloat16, (m, qw.k))
    _need(a, "A", torch.bfloat16, (r, qw.k))
    _need(b, "B", torch.bfloat16, (qw.n, r))
    need = workspace_bytes(OP_FWD, qw.fmt, qw.n, qw.k, m, r)
    with _on(stream):
        if y is None:
            y = torch.empty((m, qw.n), dtype=torch.bfloat16, device=x.device)
        if u is None:
            u = torch.empty((m, r), dtype=torch.float32, device=x.device)
        if ws is None and need:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(load().qlora_linear_fwd(qw.cstruct, _ptr(x), m, _ptr(a), _ptr(b), r, float(alpha),
                                   _ptr(y), _ptr(u), _ptr(ws), ws.numel() if ws is not None else 0,
                                   _stream(stream)))
    return y, u


def linear_bwd(qw, x, dy, u, a, b, alpha, need_dx=True, accumulate=False, dx=None, da=None,
               db=None, ws=None, stream=None):
    """Returns (dX or None, dA fp32 [r, K], dB fp32 [N, r])."""
    m = x.shape[0]
    r = a.shape[0]
    _need(x, "x", torch.bfloat16, (m, qw.k))
    _need(dy, "dY", torch.bfloat16, (m, qw.n))
    _need(u, "U", torch.float32, (m, r))
    dev = x.device
    need = workspace_bytes(OP_BWD, qw.fmt, qw.n, qw.k, m, r)
    with _on(stream):
        if need_dx and dx is None:
            dx = torch.empty((m, qw.k), dtype=torch.bfloat16, device=dev)
        if da is None:
            da = torch.zeros((r, qw.k), dtype=torch.float32, device=dev)
        if db is None:
            db = torch.zeros((qw.n, r), dtype=torch.float32, device=dev)
        if ws is None:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(load().qlora_linear_bwd(qw.cstruct, _ptr(x), _ptr(dy), _ptr(u), m, _ptr(a), _ptr(b), r,
                                   float(alpha), _ptr(dx) if need_dx else None, _ptr(da), _ptr(db),
                                   1 if accumulate else 0, _ptr(ws), ws.numel(), _stream(stream)))
    return (dx if need_dx else None), da, db


def linear_bwd_noalloc(qw, x, dy, u, a, b, alpha, dx, da, db, accumulate=False, stream=None):
    """The backward without a workspace: the library's own fixed scratch
    array is used (shared by every such call on the GPU), and this wrapper
    allocates nothing either, so every output is the caller's."""
    m = x.shape[0]
    r = a.shape[0]
    _need(x, "x", torch.bfloat16, (m, qw.k))
    _need(dy, "dY", torch.bfloat16, (m, qw.n))
    _need(u, "U", torch.float32, (m, r))
    _need(da, "dA", torch.float32, (r, qw.k))
    _need(db, "dB", torch.float32, (qw.n, r))
    if dx is not None:
        _need(dx, "dX", torch.bfloat16, (m, qw.k))
    _check(load().qlora_linear_bwd_noalloc(qw.cstruct, _ptr(x), _ptr(dy), _ptr(u), m, _ptr(a), _ptr(b), r,
                                           float(alpha), _ptr(dx), _ptr(da), _ptr(db), 1 if accumulate else 0,
                                           _stream(stream)))
    return dx, da, db


def _fwd_calls(items):
    """items: (qw, x, a, b, alpha, y, u, ws) tuples -> (ctypes array, m, r)."""
    arr = (FwdCallC * len(items))()
    m, r = items[0][1].shape[0], items[0][2].shape[0]
    for i, (qw, x, a, b, alpha, y, u, ws) in enumerate(items):
        _need(x, "x", torch.bfloat16, (m, qw.k))
        _need(a, "A", torch.bfloat16, (r, qw.k))
        _need(b, "B", torch.bfloat16, (qw.n, r))
        _need(y, "y", torch.bfloat16, (m, qw.n))
        _need(u, "U", torch.float32, (m, r))
        arr[i] = FwdCallC(ctypes.addressof(qw._c), x.data_ptr(), a.data_ptr(), b.data_ptr(), float(alpha), 0,
                          y.data_ptr(), u.data_ptr(), ws.data_ptr() if ws is not None else None,
                          ws.numel() if ws is not None else 0)
    return arr, m, r


def _bwd_calls(items):
    """items: (qw, x, dy, u, a, b, alpha, dx, da, db, ws, accumulate) tuples."""
    arr = (BwdCallC * len(items))()
    m, r = items[0][1].shape[0], items[0][4].shape[0]
    for i, (qw, x, dy, u, a, b, alpha, dx, da, db, ws, acc) in enumerate(items):
        _need(x, "x", torch.bfloat16, (m, qw.k))
        _need(dy, "dY", torch.bfloat16, (m, qw.n))
        _need(u, "U", torch.float32, (m, r))
        _need(da, "dA", torch.float32, (r, qw.k))
        _need(db, "dB", torch.float32, (qw.n, r))
        if dx is not None:
            _need(dx, "dX", torch.bfloat16, (m, qw.k))
        arr[i] = BwdCallC(ctypes.addressof(qw._c), x.data_ptr(), dy.data_ptr(), u.data_ptr(), a.data_ptr(),
                          b.data_ptr(), float(alpha), 1 if acc else 0, dx.data_ptr() if dx is not None else None,
                          da.data_ptr(), db.data_ptr(), ws.data_ptr(), ws.numel())
    return arr, m, r


def linear_fwd_group(items, stream=None):
    """Independent forward calls of one format, token count and rank in one
    library call (one launch for all on the tile path above 64 tokens; one
    split launch and one reduction at <= 64 tokens)."""
    arr, m, r = _fwd_calls(items)
    _check(load().qlora_linear_fwd_group(arr, len(items), m, r, _stream(stream)))


def linear_bwd_group(items, stream=None):
    arr, m, r = _bwd_calls(items)
    _check(load().qlora_linear_bwd_group(arr, len(items), m, r, _stream(stream)))


class Plan:
    """A recorded sequence of forward / backward calls (and event markers),
    enqueued by run() in one library call.  Outputs and workspaces must be
    given (they are referenced, not allocated); the plan keeps the tensors
    alive."""

    def __init__(self):
        self._h = ctypes.c_void_p()
        _check(load().ql_plan_create(ctypes.byref(self._h)))
        self._keep = []

    def add_fwd(self, qw, x, a, b, alpha, y, u, ws):
        m, r = x.shape[0], a.shape[0]
        _need(x, "x", torch.bfloat16, (m, qw.k))
        _need(a, "A", torch.bfloat16, (r, qw.k))
        _need(b, "B", torch.bfloat16, (qw.n, r))
        _need(y, "y", torch.bfloat16, (m, qw.n))
        _need(u, "U", torch.float32, (m, r))
        _check(load().ql_plan_add_fwd(self._h, qw.cstruct, _ptr(x), m, _ptr(a), _ptr(b), r, float(alpha),
                                      _ptr(y), _ptr(u), _ptr(ws), ws.numel() if ws is not None else 0))
        self._keep += [qw, x, a, b, y, u, ws]

    def add_bwd(self, qw, x, dy, u, a, b, alpha, dx, da, db, ws, accumulate=False):
        m, r = x.shape[0], a.shape[0]
        _need(x, "x", torch.bfloat16, (m, qw.k))
        _need(dy, "dY", torch.bfloat16, (m, qw.n))
        _need(u, "U", torch.float32, (m, r))
        _need(da, "dA", torch.float32, (r, qw.k))
        _need(db, "dB", torch.float32, (qw.n, r))
        if dx is not None:
            _need(dx, "dX", torch.bfloat16, (m, qw.k))
        _check(load().ql_plan_add_bwd(self._h, qw.cstruct, _ptr(x), _ptr(dy), _ptr(u), m, _ptr(a), _ptr(b), r,
                                      float(alpha), _ptr(dx), _ptr(da), _ptr(db), 1 if accumulate else 0,
                                      _ptr(ws), ws.numel()))
        self._keep += [qw, x, dy, u, a, b, dx, da, db, ws]

    def add_fwd_group(self, items):
        arr, m, r = _fwd_calls(items)
        _check(load().ql_plan_add_fwd_group(self._h, arr, len(items), m, r))
        self._keep += [t for it in items for t in it if isinstance(t, (torch.Tensor, QWeight))]

    def add_bwd_group(self, items):
        arr, m, r = _bwd_calls(items)
        _check(load().ql_plan_add_bwd_group(self._h, arr, len(items), m, r))
        self._keep += [t for it in items for t in it if isinstance(t, (torch.Tensor, QWeight))]

    def add_event(self, event, stream=None):
        """Record `event` (a torch.cuda.Event) at this point of every run; the
        event is recorded once here so that its handle exists."""
        event.record(stream if stream is not None else torch.cuda.current_stream())
        _check(load().ql_plan_add_event(self._h, ctypes.c_void_p(event.cuda_event)))
        self._keep.append(event)

    def __len__(self):
        return int(load().ql_plan_size(self._h))

    def run(self, stream=None):
        _check(load().ql_plan_run(self._h, _stream(stream)))

    def close(self):
        if self._h:
            load().ql_plan_destroy(self._h)
            self._h = ctypes.c_void_p()
            self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------- layer stream pool

class Pool:
    """Pool of device slots fed from pinned host layer images, one layer ahead."""

    def __init__(self, slots, host_layers):
        lib = load()
        self.slots = list(slots)
        self.host = list(host_layers)
        n_s, n_l = len(self.slots), len(self.host)
        sp = (ctypes.c_void_p * n_s)(*[t.data_ptr() for t in self.slots])
        hp = (ctypes.c_void_p * n_l)(*[t.data_ptr() for t in self.host])
        hb = (ctypes.c_size_t * n_l)(*[t.numel() * t.element_size() for t in self.host])
        slot_bytes = min(t.numel() * t.element_size() for t in self.slots)
        self._h = ctypes.c_void_p()
        _check(lib.ql_pool_create(ctypes.byref(self._h), n_s, sp, slot_bytes, n_l, hp, hb))

    def prefetch(self, layer, copy_stream):
        _check(load().layer_stream_prefetch(self._h, layer, ctypes.c_void_p(copy_stream.cuda_stream)))

    def acquire(self, layer, compute_stream=None):
        out = ctypes.c_void_p()
        _check(load().ql_pool_acquire(self._h, layer, _stream(compute_stream), ctypes.byref(out)))
        return out.value

    def release(self, layer, compute_stream=None):
        _check(load().ql_pool_release(self._h, layer, _stream(compute_stream)))

    def stats(self):
        out = (ctypes.c_int64 * 3)()
        _check(load().ql_pool_stats(self._h, out))
        return {"hits": out[0], "copies": out[1], "bytes": out[2]}

    def debug(self, delay_us=0, poison=False, skip_wait=False):
        _check(load().ql_pool_debug(self._h, int(delay_us), int(bool(poison)), int(bool(skip_wait))))

    def close(self):
        if self._h:
            load().ql_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------- adapter optimizer

class AdamwPlan:
    """The descriptor array of a fixed set of adapter tensors, checked once, so
    that each step is a single library call (the tensors must stay alive)."""

    def __init__(self, tensors):
        self.tensors = list(tensors)
        self.arr = _adamw_array(self.tensors)

    def step(self, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, grad_scale=1.0,
             stream=None):
        hp = AdamwHparamsC(lr, beta1, beta2, eps, weight_decay, grad_scale, int(step), 0)
        _check(load().ql_adamw_step(self.arr, len(self.tensors), ctypes.byref(hp), _stream(stream)))


def adamw_step(tensors, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
               grad_scale=1.0, stream=None):
    """One AdamW step, in place, on every (param, grad, exp_avg, exp_avg_sq,
    param_bf16 or None) tuple of `tensors` (fp32 device tensors of equal
    sizes; param_bf16 a bf16 tensor of the same size), in one launch."""
    AdamwPlan(tensors).step(step, lr, beta1, beta2, eps, weight_decay, grad_scale, stream)


def _adamw_array(tensors):
    arr = (AdamwTensorC * max(1, len(tensors)))()
    for i, (p, g, m, v, pb) in enumerate(tensors):
        for name, t in (("param", p), ("grad", g), ("exp_avg", m), ("exp_avg_sq", v)):
            _need(t, name, torch.float32)
            if t.numel() != p.numel():
                raise ValueError(f"{name}: size {t.numel()} differs from param's {p.numel()}")
        if pb is not None:
            _need(pb, "param_bf16", torch.bfloat16)
            if pb.numel() != p.numel():
                raise ValueError("param_bf16 size differs from param's")
        arr[i] = AdamwTensorC(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(),
                              pb.data_ptr() if pb is not None else None, p.numel())
    return arr


class Adamw8State:
    """8-bit block-wise AdamW state of one tensor of n elements: first- and
    second-moment codes (u8 [n]) and their per-block scales (fp32
    [ceil(n / 2048)]); zero codes and scales are the zero state."""

    def __init__(self, n, device="cuda"):
        nb = -(-int(n) // ADAMW8_BLOCK)
        self.n = int(n)
        self.m = torch.zeros(n, dtype=torch.uint8, device=device)
        self.m_absmax = torch.zeros(nb, dtype=torch.float32, device=device)
        self.v = torch.zeros(n, dtype=torch.uint8, device=device)
        self.v_absmax = torch.zeros(nb, dtype=torch.float32, device=device)


class Adamw8Plan:
    """The descriptor array of a fixed set of (param, grad, Adamw8State,
    param_bf16 or None) tensors, checked once, so that each step is a single
    library call (the tensors must stay alive)."""

    def __init__(self, tensors):
        self.tensors = list(tensors)
        arr = (Adamw8TensorC * max(1, len(self.tensors)))()
        for i, (p, g, st, pb) in enumerate(self.tensors):
            for name, t in (("param", p), ("grad", g)):
                _need(t, name, torch.float32)
                if t.numel() != p.numel():
                    raise ValueError(f"{name}: size {t.numel()} differs from param's {p.numel()}")
            if st.n != p.numel():
                raise ValueError("state size differs from param's")
            if pb is not None:
                _need(pb, "param_bf16", torch.bfloat16)
            arr[i] = Adamw8TensorC(p.data_ptr(), g.data_ptr(), st.m.data_ptr(), st.m_absmax.data_ptr(),
                                   st.v.data_ptr(), st.v_absmax.data_ptr(),
                                   pb.data_ptr() if pb is not None else None, p.numel())
        self.arr = arr

    def step(self, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, grad_scale=1.0,
             stream=None):
        hp = AdamwHparamsC(lr, beta1, beta2, eps, weight_decay, grad_scale, int(step), 0)
        _check(load().ql_adamw8_step(self.arr, len(self.tensors), ctypes.byref(hp), _stream(stream)))


def dyn8_levels(signed):
    """The library's levels of the 8-bit state type (host call, needs no GPU)."""
    n = 128 if signed else 256
    buf = (ctypes.c_float * n)()
    _check(load().ql_dyn8_levels(1 if signed else 0, buf))
    return [float(v) for v in buf]


# ----------------------------------------------------------------------------- stacked adapters

def stack_adapters(adapters, stream=None):
    """Frozen lower adapters under a trainable top one (the last of
    `adapters`, a list of (A bf16 [r, K], B bf16 [N, r], alpha)) as one
    adapter: returns (A_cat bf16 [R, K], B_cat bf16 [N, R], alpha_cat) for the
    layer calls; the top adapter's gradients are the last r_top rows of dA and
    columns of dB (see top_grads)."""
    n = len(adapters)
    k, nout = adapters[0][0].shape[1], adapters[0][1].shape[0]
    arr = (AdapterC * n)()
    for i, (a, b, alpha) in enumerate(adapters):
        r = a.shape[0]
        _need(a, "A", torch.bfloat16, (r, k))
        _need(b, "B", torch.bfloat16, (nout, r))
        arr[i] = AdapterC(a.data_ptr(), b.data_ptr(), r, float(alpha))
    R = sum(a.shape[0] for a, _, _ in adapters)
    dev = adapters[0][0].device
    a_cat = torch.empty((R, k), dtype=torch.bfloat16, device=dev)
    b_cat = torch.empty((nout, R), dtype=torch.bfloat16, device=dev)
    alpha_cat = ctypes.c_float()
    _check(load().ql_stack_adapters(arr, n, nout, k, _ptr(a_cat), _ptr(b_cat), ctypes.byref(alpha_cat),
                                    _stream(stream)))
    return a_cat, b_cat, alpha_cat.value


def top_grads(da, db, r_top):
    """The top adapter's (dA, dB) inside the stacked call's gradients (views)."""
    return da[-r_top:], db[:, -r_top:]
