"""Thin ctypes binding of liblora (include/lora.h).

Argument marshalling only: every function here checks tensor placement and
dtype, turns tensors into device pointers and calls the C entry point of the
same name.  All computation happens in the HIP kernels behind the C ABI.
There is no fallback: if liblora.so is missing or the device is not a GPU,
the call raises.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "LoraError", "lib", "LoraLinear", "LoraDropout", "LoraSegment", "LoraAdamwHparams",
    "F32", "BF16", "KIND_A", "KIND_B", "KIND_MAG",
    "lora_workspace_bytes", "lora_forward", "lora_backward",
    "lora_grad_prepare_workspace_bytes", "lora_grad_prepare", "lora_adamw_step",
    "lora_dropout_mask", "lora_dora_row_norms_workspace_bytes", "lora_dora_row_norms",
    "lora_merge_workspace_bytes", "lora_merge", "lora_scaling", "lora_lr_at",
    "lora_status_string", "lora_profile_begin", "lora_profile_end", "lora_set_bf16_config",
    "lora_group_workspace_bytes", "lora_forward_group", "lora_backward_group",
    "lora_slots_workspace_bytes", "lora_forward_slots", "lora_backward_slots",
    "lora_qweight_layout", "lora_grad_prepare_noalloc",
    "lora_dora_row_norms_batch_workspace_bytes", "lora_dora_row_norms_batch", "QWeight", "qweight_pack", "Q_FORMATS", "EXPORTS", "GroupCall",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblora.so")

F32, BF16 = 0, 1
# Block-quantized W formats (lora_dtype): code and plane names in layout order.
Q_FORMATS = {"q8_0": (2, ("qs", "d")), "q4_0": (3, ("qs", "d")),
             "q4_k": (4, ("qs", "sm", "dm")), "q6_k": (5, ("ql", "qh", "sc", "d"))}
KIND_A, KIND_B, KIND_MAG = 0, 1, 2
LORA_E_NONFINITE = -6

# Every symbol include/lora.h declares.
EXPORTS = (
    "lora_workspace_bytes", "lora_forward", "lora_backward",
    "lora_grad_prepare_workspace_bytes", "lora_grad_prepare", "lora_adamw_step",
    "lora_dropout_mask", "lora_dora_row_norms_workspace_bytes", "lora_dora_row_norms",
    "lora_merge_workspace_bytes", "lora_merge", "lora_scaling", "lora_lr_at",
    "lora_status_string", "lora_profile_begin", "lora_profile_end", "lora_set_bf16_config",
    "lora_group_workspace_bytes", "lora_forward_group", "lora_backward_group",
    "lora_slots_workspace_bytes", "lora_forward_slots", "lora_backward_slots",
    "lora_qweight_layout", "lora_grad_prepare_noalloc",
    "lora_dora_row_norms_batch_workspace_bytes", "lora_dora_row_norms_batch",
)


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lora_status_string(status)} (status {status})")


class LoraDropout(C.Structure):
    _fields_ = [("seed", C.c_uint64), ("step", C.c_int64), ("ordinal", C.c_int32),
                ("layer", C.c_int32), ("proj", C.c_int32), ("p", C.c_float)]


class LoraLinear(C.Structure):
    _fields_ = [("tokens", C.c_int64), ("in_dim", C.c_int64), ("out_dim", C.c_int64),
                ("rank", C.c_int64), ("w_dtype", C.c_int32), ("scale", C.c_float),
                ("W", C.c_void_p), ("A", C.c_void_p), ("B", C.c_void_p),
                ("dora_mag", C.c_void_p), ("dora_norm", C.c_void_p), ("dora_from_y", C.c_int32)]


class LoraProfileEntry(C.Structure):
    _fields_ = [("kernel", C.c_char_p), ("M", C.c_int64), ("N", C.c_int64), ("K", C.c_int64),
                ("launches", C.c_int64), ("total_ms", C.c_double), ("flops", C.c_double),
                ("bytes", C.c_double)]


class LoraSegment(C.Structure):
    _fields_ = [("offset", C.c_int64), ("count", C.c_int64), ("kind", C.c_int32)]


class LoraAdamwHparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("plus_ratio", C.c_double),
                ("t", C.c_int64)]


_LIB = None


def lib() -> C.CDLL:
    """Load liblora.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bwd_adamw_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I64, I32, F, SZ = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
        sig = {
            "lora_workspace_bytes": (SZ, [P]),
            "lora_forward": (I32, [P, P, P, P, P, P, P, SZ, P]),
            "lora_backward": (I32, [P, P, P, P, P, P, P, P, P, I32, P, P, SZ, P]),
            "lora_grad_prepare_workspace_bytes": (SZ, [I64]),
            "lora_grad_prepare": (I32, [P, I64, I64, F, P, P, P, P, SZ, P]),
            "lora_grad_prepare_noalloc": (I32, [P, I64, I64, F, P, P, P, P]),
            "lora_adamw_step": (I32, [P, P, P, P, P, I32, P, P, P]),
            "lora_dropout_mask": (I32, [P, I64, I64, P, P]),
            "lora_dora_row_norms_workspace_bytes": (SZ, [P]),
            "lora_dora_row_norms": (I32, [P, P, P, SZ, P]),
            "lora_merge_workspace_bytes": (SZ, [P]),
            "lora_merge": (I32, [P, P, I32, P, P, SZ, P]),
            "lora_scaling": (C.c_double, [C.c_double, I64, I32]),
            "lora_lr_at": (C.c_double, [I64, C.c_double, I32, I64, I64, C.c_double]),
            "lora_status_string": (C.c_char_p, [I32]),
            "lora_profile_begin": (I32, [I32]),
            "lora_profile_end": (I32, [P, I32]),
            "lora_set_bf16_config": (I32, [I32]),
            "lora_group_workspace_bytes": (SZ, [I32, P]),
            "lora_forward_group": (I32, [I32, P, P, P, P, P, P, P, SZ, P]),
            "lora_backward_group": (I32, [I32, P, P, P, P, P, P, P, P, P, I32, P, P, SZ, P]),
            "lora_slots_workspace_bytes": (SZ, [I32, P]),
            "lora_forward_slots": (I32, [I32, P, P, P, P, P, P, P, SZ, P]),
            "lora_backward_slots": (I32, [I32, P, P, P, P, P, P, P, P, P, I32, P, P, SZ, P]),
            "lora_qweight_layout": (SZ, [I32, I64, I64, P]),
            "lora_dora_row_norms_batch_workspace_bytes": (SZ, [I32, P]),
            "lora_dora_row_norms_batch": (I32, [I32, P, P, P, SZ, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


# ------------------------------------------------------------------ helpers
def _ptr(t, name, dtype=torch.float32):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _sized(t, name, need, dtype=torch.float32):
    """_ptr that also refuses a tensor with fewer than `need` elements: the
    kernels address every buffer from the linear's sizes alone."""
    p = _ptr(t, name, dtype)
    if p is not None and t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} elements, the call reads or writes {need}")
    return p


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(fn, rc):
    if rc != 0:
        raise LoraError(fn, rc)


def lora_qweight_layout(fmt: str, out_dim: int, in_dim: int):
    """(total bytes, [offset of each plane]) of a block-quantized W."""
    code, names = Q_FORMATS[fmt]
    off = (C.c_size_t * 4)()
    total = int(lib().lora_qweight_layout(code, int(out_dim), int(in_dim), off))
    if total == 0:
        raise ValueError(f"{fmt} cannot hold a [{out_dim}, {in_dim}] weight")
    return total, [int(o) for o in off[: len(names)]]


class QWeight:
    """A block-quantized W [out_dim, in_dim] in the library's layout: one
    uint8 device buffer holding the format's planes (include/lora.h)."""

    def __init__(self, fmt: str, out_dim: int, in_dim: int, buf: torch.Tensor):
        self.fmt, self.out_dim, self.in_dim, self.buf = fmt, int(out_dim), int(in_dim), buf
        self.code = Q_FORMATS[fmt][0]

    @property
    def shape(self):
        return (self.out_dim, self.in_dim)


def _plane_row_bytes(fmt, K):
    return {"q8_0": (K, K // 16), "q4_0": (K // 2, K // 16),
            "q4_k": (K // 2, K // 16, K // 64),
            "q6_k": (K // 2, K // 4, K // 16, K // 128)}[fmt]


def qweight_pack(fmt: str, out_dim: int, in_dim: int, planes: dict, device="cuda") -> QWeight:
    """Copy the planes (tensors of any dtype, by their bytes, row-major) into
    one device buffer laid out by lora_qweight_layout."""
    total, offs = lora_qweight_layout(fmt, out_dim, in_dim)
    names = Q_FORMATS[fmt][1]
    buf = torch.zeros(total, dtype=torch.uint8, device=device)
    for name, off, rb in zip(names, offs, _plane_row_bytes(fmt, int(in_dim))):
        raw = planes[name].contiguous().view(torch.uint8).reshape(-1)
        if raw.numel() != rb * out_dim:
            raise ValueError(f"{fmt} plane {name} holds {raw.numel()} bytes, the layout "
                             f"needs {rb * out_dim}")
        buf[off:off + raw.numel()].copy_(raw)
    return QWeight(fmt, out_dim, in_dim, buf)


def make_linear(W, A, B, scale, tokens, dora_mag=None, dora_norm=None,
                dora_from_y=False) -> LoraLinear:
    """Descriptor of one adapted linear: W [N,K] (float32 or bfloat16, or a
    QWeight), A [r,K], B [N,r] float32, optional DoRA magnitude and norm [N].
    dora_from_y (DoRA only): the backward takes the forward's Y where it
    would take Z, so the forward need not write Z."""
    if isinstance(W, QWeight):
        wd = W.code
    elif W.dtype in (torch.float32, torch.bfloat16):
        wd = F32 if W.dtype == torch.float32 else BF16
    else:
        raise TypeError(f"W must be float32, bfloat16 or a QWeight, got {W.dtype}")
    N, K = W.shape
    r = A.shape[0] if A is not None else 0
    if A is not None and tuple(A.shape) != (r, K):
        raise ValueError(f"A must be [{r}, {K}], got {list(A.shape)}")
    if B is not None and tuple(B.shape) != (N, r):
        raise ValueError(f"B must be [{N}, {r}], got {list(B.shape)}")
    for t, nm in ((dora_mag, "dora_mag"), (dora_norm, "dora_norm")):
        if t is not None and t.numel() != N:
            raise ValueError(f"{nm} must hold {N} elements, got {t.numel()}")
    wptr = _ptr(W.buf, "W", torch.uint8) if isinstance(W, QWeight) else _ptr(W, "W", None)
    return LoraLinear(int(tokens), int(K), int(N), int(r), wd, float(scale), wptr,
                      _ptr(A, "A"), _ptr(B, "B"), _ptr(dora_mag, "dora_mag"),
                      _ptr(dora_norm, "dora_norm"), 1 if dora_from_y else 0)


def make_dropout(seed, step, ordinal, layer, proj, p) -> LoraDropout:
    return LoraDropout(int(seed), int(step), int(ordinal), int(layer), int(proj), float(p))


def _ref(s):
    return None if s is None else C.byref(s)


# ------------------------------------------------------------ entry points
def lora_status_string(status: int) -> str:
    return lib().lora_status_string(int(status)).decode()


def lora_scaling(alpha: float, rank: int, rslora: bool = False) -> float:
    return lib().lora_scaling(float(alpha), int(rank), 1 if rslora else 0)


def lora_lr_at(k: int, lr: float, schedule: int = 0, warmup: int = 0, total: int = 100,
               lr_min: float = 0.0) -> float:
    return lib().lora_lr_at(int(k), float(lr), int(schedule), int(warmup), int(total), float(lr_min))


def lora_workspace_bytes(lin: LoraLinear) -> int:
    return int(lib().lora_workspace_bytes(C.byref(lin)))


def lora_forward(lin, X, Y, U, Z=None, drop=None, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    T, K, N, r = lin.tokens, lin.in_dim, lin.out_dim, lin.rank
    rc = lib().lora_forward(C.byref(lin), _sized(X, "X", T * K), _sized(Y, "Y", T * N),
                            _sized(U, "U", T * r), _sized(Z, "Z", T * N), _ref(drop),
                            _ptr(ws, "ws", None), ws_bytes, _stream(stream))
    _check("lora_forward", rc)


def lora_backward(lin, X, dY, U, Z, dX, dA, dB, dMag=None, accumulate=False, drop=None,
                  ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    T, K, N, r = lin.tokens, lin.in_dim, lin.out_dim, lin.rank
    rc = lib().lora_backward(C.byref(lin), _sized(X, "X", T * K), _sized(dY, "dY", T * N),
                             _sized(U, "U", T * r), _sized(Z, "Z", T * N), _sized(dX, "dX", T * K),
                             _sized(dA, "dA", r * K), _sized(dB, "dB", N * r),
                             _sized(dMag, "dMag", N), 1 if accumulate else 0, _ref(drop),
                             _ptr(ws, "ws", None), ws_bytes, _stream(stream))
    _check("lora_backward", rc)


MAX_GROUP = 4
MAX_SLOTS = 4


def _linears(lins):
    arr = (LoraLinear * len(lins))(*lins)
    return arr


# Elements of each per-linear tensor argument, from a linear's sizes.
_NEED = {
    "X": lambda l: l.tokens * l.in_dim, "dX": lambda l: l.tokens * l.in_dim,
    "Y": lambda l: l.tokens * l.out_dim, "Z": lambda l: l.tokens * l.out_dim,
    "dY": lambda l: l.tokens * l.out_dim, "U": lambda l: l.tokens * l.rank,
    "dA": lambda l: l.rank * l.in_dim, "dB": lambda l: l.out_dim * l.rank,
    "dMag": lambda l: l.out_dim, "out_norm": lambda l: l.out_dim,
}


def _ptrs(ts, name, lins, optional=False):
    """Array of device pointers, one per linear of `lins`, each checked
    against that linear's sizes; None when every entry is None and the
    argument is optional."""
    if ts is None or (optional and all(t is None for t in ts)):
        if not optional:
            raise ValueError(f"{name} is required")
        return None
    if len(ts) != len(lins):
        raise ValueError(f"{name} has {len(ts)} entries for {len(lins)} linears")
    return (C.c_void_p * len(ts))(*[_sized(t, f"{name}[{i}]", _NEED[name](l))
                                    for i, (t, l) in enumerate(zip(ts, lins))])


def _drops(drops, n):
    if drops is None or all(d is None for d in drops):
        return None
    zero = LoraDropout(0, 0, 0, 0, 0, 0.0)
    return (LoraDropout * n)(*[zero if d is None else d for d in drops])


def lora_group_workspace_bytes(lins) -> int:
    return int(lib().lora_group_workspace_bytes(len(lins), _linears(lins)))


def lora_forward_group(lins, X, Y, U, Z=None, drops=None, ws=None, stream=None):
    """Forward of the linears `lins` that read one X; Y, U (and Z) are lists
    with one tensor per linear."""
    n = len(lins)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().lora_forward_group(n, _linears(lins), _sized(X, "X", _NEED["X"](lins[0])),
                                  _ptrs(Y, "Y", lins), _ptrs(U, "U", lins),
                                  _ptrs(Z, "Z", lins, True), _drops(drops, n), _ptr(ws, "ws", None),
                                  ws_bytes, _stream(stream))
    _check("lora_forward_group", rc)


def lora_backward_group(lins, X, dY, U, Z, dX, dA, dB, dMag=None, accumulate=False, drops=None,
                        ws=None, stream=None):
    """Backward of the linears `lins` that read one X; every other tensor
    argument is a list with one entry per linear."""
    n = len(lins)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().lora_backward_group(n, _linears(lins), _sized(X, "X", _NEED["X"](lins[0])),
                                   _ptrs(dY, "dY", lins), _ptrs(U, "U", lins),
                                   _ptrs(Z, "Z", lins, True), _ptrs(dX, "dX", lins, True),
                                   _ptrs(dA, "dA", lins), _ptrs(dB, "dB", lins),
                                   _ptrs(dMag, "dMag", lins, True),
                                   1 if accumulate else 0, _drops(drops, n), _ptr(ws, "ws", None),
                                   ws_bytes, _stream(stream))
    _check("lora_backward_group", rc)


class GroupCall:
    """Marshalled arguments of lora_forward_group / lora_backward_group for
    one group of linears whose descriptors and trainer-owned buffers stay
    put across calls (Y, U, Z, dX, the gradients, the workspace, the
    stream): they are checked and marshalled once, here.  Each call checks
    and marshals only its own inputs (X, dY, dropout keys); an X or dY list
    whose tensors are the ones of the previous call reuses their pointers."""

    def __init__(self, lins, Y, U, Z=None, dX=None, dA=None, dB=None, dMag=None, ws=None,
                 stream=None):
        self.n = len(lins)
        self.lins = list(lins)
        self.arr = _linears(self.lins)
        self.Y, self.U = _ptrs(Y, "Y", lins), _ptrs(U, "U", lins)
        self.Z = _ptrs(Z, "Z", lins, True)
        # DoRA linears with dora_from_y: the forward writes no Z and the
        # backward reads Y in its place.
        self.from_y = any(l.dora_from_y for l in lins)
        if self.from_y and not all(l.dora_from_y for l in lins):
            raise ValueError("dora_from_y must be set for all linears of a group call or none")
        self.Zf = None if self.from_y else self.Z
        self.Zb = self.Y if self.from_y else self.Z
        self.dX = _ptrs(dX, "dX", lins, True)
        self.dA = None if dA is None else _ptrs(dA, "dA", lins)
        self.dB = None if dB is None else _ptrs(dB, "dB", lins)
        self.dMag = _ptrs(dMag, "dMag", lins, True)
        self.ws = _ptr(ws, "ws", None)
        self.ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
        self.stream = _stream(stream)
        self._held = (Y, U, Z, dX, dA, dB, dMag, ws, stream)   # the marshalled buffers stay alive
        self._x = self._xp = None
        self._dy = self._dyp = None

    def _x_ptr(self, X):
        if X is not self._x:
            self._xp = _sized(X, "X", _NEED["X"](self.lins[0]))
            self._x = X
        return self._xp

    def _dy_ptrs(self, dY):
        if self._dy is None or len(dY) != len(self._dy) or any(a is not b for a, b in zip(dY, self._dy)):
            self._dyp = _ptrs(dY, "dY", self.lins)
            self._dy = list(dY)
        return self._dyp

    def dropouts(self, drops):
        """The marshalled dropout keys (one LoraDropout or None per linear),
        to pass to forward and backward of the same chunk."""
        return _drops(drops, self.n)

    def _d(self, drops):
        return drops if drops is None or isinstance(drops, C.Array) else _drops(drops, self.n)

    def forward(self, X, drops=None):
        rc = lib().lora_forward_group(self.n, self.arr, self._x_ptr(X), self.Y, self.U, self.Zf,
                                      self._d(drops), self.ws, self.ws_bytes, self.stream)
        _check("lora_forward_group", rc)

    def backward(self, X, dY, accumulate=False, drops=None):
        if self.dA is None or self.dB is None:
            raise ValueError("this GroupCall was prepared without gradients")
        rc = lib().lora_backward_group(self.n, self.arr, self._x_ptr(X), self._dy_ptrs(dY),
                                       self.U, self.Zb, self.dX, self.dA, self.dB, self.dMag,
                                       1 if accumulate else 0, self._d(drops), self.ws,
                                       self.ws_bytes, self.stream)
        _check("lora_backward_group", rc)


def lora_slots_workspace_bytes(lins) -> int:
    return int(lib().lora_slots_workspace_bytes(len(lins), _linears(lins)))


def lora_forward_slots(lins, X, Y, U, Z=None, drops=None, ws=None, stream=None):
    """Forward of adapter slots over one W: every tensor argument is a list
    with one entry per slot."""
    n = len(lins)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().lora_forward_slots(n, _linears(lins), _ptrs(X, "X", lins), _ptrs(Y, "Y", lins),
                                  _ptrs(U, "U", lins), _ptrs(Z, "Z", lins, True),
                                  _drops(drops, n), _ptr(ws, "ws", None),
                                  ws_bytes, _stream(stream))
    _check("lora_forward_slots", rc)


def lora_backward_slots(lins, X, dY, U, Z, dX, dA, dB, dMag=None, accumulate=False, drops=None,
                        ws=None, stream=None):
    """Backward of adapter slots over one W: every tensor argument is a list
    with one entry per slot."""
    n = len(lins)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().lora_backward_slots(n, _linears(lins), _ptrs(X, "X", lins), _ptrs(dY, "dY", lins),
                                   _ptrs(U, "U", lins), _ptrs(Z, "Z", lins, True),
                                   _ptrs(dX, "dX", lins, True), _ptrs(dA, "dA", lins),
                                   _ptrs(dB, "dB", lins), _ptrs(dMag, "dMag", lins, True),
                                   1 if accumulate else 0, _drops(drops, n), _ptr(ws, "ws", None),
                                   ws_bytes, _stream(stream))
    _check("lora_backward_slots", rc)


def lora_grad_prepare_workspace_bytes(n: int) -> int:
    return int(lib().lora_grad_prepare_workspace_bytes(int(n)))


def lora_grad_prepare(grads, n_pred_tokens, max_norm, d_scale, d_stats=None, sync=True,
                      ws=None, stream=None):
    """Returns the norm (host float) when sync is True, else None.  A vetoed
    (non-finite) update raises LoraError with status LORA_E_NONFINITE when
    sync is True; otherwise the veto travels in d_scale (NaN)."""
    n = grads.numel()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    h = C.c_double(0.0)
    rc = lib().lora_grad_prepare(_ptr(grads, "grads"), n, int(n_pred_tokens), float(max_norm),
                                 _ptr(d_scale, "d_scale"), _ptr(d_stats, "d_stats", torch.float64),
                                 C.byref(h) if sync else None, _ptr(ws, "ws", None), ws_bytes,
                                 _stream(stream))
    _check("lora_grad_prepare", rc)
    return h.value if sync else None


def lora_grad_prepare_noalloc(grads, n_pred_tokens, max_norm, d_scale, d_stats=None, sync=True,
                              stream=None):
    """lora_grad_prepare with the library's static device scratch in place of
    a workspace (nothing is allocated); same returns and errors."""
    h = C.c_double(0.0)
    rc = lib().lora_grad_prepare_noalloc(_ptr(grads, "grads"), grads.numel(), int(n_pred_tokens),
                                         float(max_norm), _ptr(d_scale, "d_scale"),
                                         _ptr(d_stats, "d_stats", torch.float64),
                                         C.byref(h) if sync else None, _stream(stream))
    _check("lora_grad_prepare_noalloc", rc)
    return h.value if sync else None


def lora_adamw_step(params, grads, m, v, segments, hp: LoraAdamwHparams, d_scale, stream=None):
    segs = (LoraSegment * len(segments))(*[LoraSegment(int(o), int(c), int(k)) for o, c, k in segments])
    end = max((int(o) + int(c) for o, c, _ in segments), default=0)
    rc = lib().lora_adamw_step(_sized(params, "params", end), _sized(grads, "grads", end),
                               _sized(m, "m", end), _sized(v, "v", end), segs, len(segments),
                               C.byref(hp), _sized(d_scale, "d_scale", 1), _stream(stream))
    _check("lora_adamw_step", rc)


def lora_dropout_mask(drop: LoraDropout, tokens, in_dim, mask, stream=None):
    rc = lib().lora_dropout_mask(C.byref(drop), int(tokens), int(in_dim),
                                 _sized(mask, "mask", int(tokens) * int(in_dim), torch.uint8),
                                 _stream(stream))
    _check("lora_dropout_mask", rc)


def lora_dora_row_norms_workspace_bytes(lin: LoraLinear) -> int:
    return int(lib().lora_dora_row_norms_workspace_bytes(C.byref(lin)))


def lora_dora_row_norms(lin: LoraLinear, out_norm, ws=None, stream=None, split=True):
    """Row norms of W + s B A into out_norm.  `ws` is a device uint8 tensor of
    at least lora_dora_row_norms_workspace_bytes(lin) bytes; when it is None
    one is taken from torch's allocator (split=False passes none at all)."""
    if ws is None and split:
        need = lora_dora_row_norms_workspace_bytes(lin)
        if need:
            ws = torch.empty(need, device=out_norm.device, dtype=torch.uint8)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().lora_dora_row_norms(C.byref(lin), _sized(out_norm, "out_norm", lin.out_dim),
                                   _ptr(ws, "ws", None), ws_bytes, _stream(stream))
    _check("lora_dora_row_norms", rc)


def lora_dora_row_norms_batch_workspace_bytes(lins) -> int:
    return int(lib().lora_dora_row_norms_batch_workspace_bytes(len(lins), _linears(lins)))


def lora_dora_row_norms_batch(lins, out_norms, ws=None, stream=None):
    """Row norms of W + s B A for every linear of `lins` into the matching
    entry of `out_norms`; `ws` as lora_dora_row_norms_batch_workspace_bytes
    asks (taken from torch's allocator when None)."""
    if len(lins) == 0:
        return
    if ws is None:
        need = lora_dora_row_norms_batch_workspace_bytes(lins)
        if need:
            ws = torch.empty(need, device=out_norms[0].device, dtype=torch.uint8)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().lora_dora_row_norms_batch(len(lins), _linears(lins),
                                         _ptrs(out_norms, "out_norm", lins), _ptr(ws, "ws", None),
                                         ws_bytes, _stream(stream))
    _check("lora_dora_row_norms_batch", rc)


def lora_merge_workspace_bytes(lin: LoraLinear) -> int:
    return int(lib().lora_merge_workspace_bytes(C.byref(lin)))


def lora_merge(lin: LoraLinear, W_out, rmse=None, ws=None, stream=None):
    """W_out = c (W + s B A) (c = mag/norm for DoRA) as float32 or bfloat16
    (W_out's dtype).  `rmse` is a device float64 tensor of one element or
    None; bf16 output needs `ws` (taken from torch's allocator when None)."""
    if W_out.dtype == torch.float32:
        od = F32
    elif W_out.dtype == torch.bfloat16:
        od = BF16
    else:
        raise TypeError(f"W_out must be float32 or bfloat16, got {W_out.dtype}")
    if rmse is not None and ws is None and od == BF16:
        ws = torch.empty(max(8, lora_merge_workspace_bytes(lin)), device=W_out.device,
                         dtype=torch.uint8)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().lora_merge(C.byref(lin), _sized(W_out, "W_out", lin.out_dim * lin.in_dim, None), od,
                          _sized(rmse, "rmse", 1, torch.float64), _ptr(ws, "ws", None), ws_bytes,
                          _stream(stream))
    _check("lora_merge", rc)


def lora_set_bf16_config(cfg: int):
    """Pin the tile configuration of the bf16-W products (-1: the planner
    chooses per product).  Process-wide; size workspaces after setting it."""
    _check("lora_set_bf16_config", lib().lora_set_bf16_config(int(cfg)))


def lora_profile_begin(max_launches: int = 100000):
    _check("lora_profile_begin", lib().lora_profile_begin(int(max_launches)))


def lora_profile_end(max_entries: int = 512) -> list:
    """Close the profile; returns dicts with kernel, M, N, K, launches,
    total_ms, avg_ms, flops and bytes (per launch)."""
    buf = (LoraProfileEntry * max_entries)()
    n = lib().lora_profile_end(buf, max_entries)
    if n < 0:
        raise LoraError("lora_profile_end", n)
    out = []
    for e in buf[:n]:
        out.append(dict(kernel=e.kernel.decode(), M=e.M, N=e.N, K=e.K, launches=e.launches,
                        total_ms=e.total_ms, avg_ms=e.total_ms / max(1, e.launches),
                        flops=e.flops, bytes=e.bytes))
    return out
