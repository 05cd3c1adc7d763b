"""ctypes binding of libmlora (include/mlora.h): argument marshalling only.

Every function here has the name of the C entry point it calls, turns torch tensors into raw
device pointers and passes torch's current HIP stream.  No step of the layer is computed in
Python: if ``libmlora.so`` is missing, importing this module raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmlora.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -m lora_serving_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

MLORA_OK = 0
MLORA_ERR_ARG = 1
MLORA_ERR_SHAPE = 2
MLORA_ERR_RANK = 3
MLORA_ERR_INDEX = 4
MLORA_ERR_WORKSPACE = 5
MLORA_ERR_HIP = 6
MLORA_ERR_UNSUPPORTED = 7
MLORA_MAX_SLICES = 4
MLORA_MAX_RANK = 512
MLORA_MAX_SLOTS = 16384
MLORA_MAX_K = 8
MLORA_NO_ADAPTERS = 1
MLORA_PATH_DECODE = 2
MLORA_PATH_TILED = 4
MLORA_W_PACKED = 8
MLORA_PATH_GROUPED = 16
MLORA_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("mlora_status_string", "mlora_last_error", "mlora_factor", "mlora_slot_bytes",
           "mlora_workspace_size", "mlora_slot_load", "mlora_packed_weight_bytes",
           "mlora_pack_weight",
           "mlora_validate", "mlora_plan", "mlora_shrink", "mlora_expand", "mlora_linear",
           "mlora_linear_path", "mlora_linear_noalloc", "mlora_trace_start", "mlora_trace_stop")

_P = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class mlora_slots(ctypes.Structure):
    _fields_ = [("A", _P), ("B", _P), ("factor", _P), ("S", _i32), ("R", _i32),
                ("n_slices", _i32), ("slice_start", _i32 * (MLORA_MAX_SLICES + 1)),
                ("rank", _P)]


_SLOTS_P = ctypes.POINTER(mlora_slots)

_lib.mlora_status_string.restype = ctypes.c_char_p
_lib.mlora_status_string.argtypes = [ctypes.c_int]
_lib.mlora_last_error.restype = ctypes.c_char_p
_lib.mlora_last_error.argtypes = []
_lib.mlora_factor.restype = ctypes.c_float
_lib.mlora_factor.argtypes = [ctypes.c_float, _i32, _i32]
_lib.mlora_slot_bytes.restype = _i64
_lib.mlora_slot_bytes.argtypes = [_i32, _i32, _i64, _i64, _i32]
_lib.mlora_workspace_size.restype = ctypes.c_size_t
_lib.mlora_workspace_size.argtypes = [_i64, _i32, _i64, _i64, _SLOTS_P]
_lib.mlora_packed_weight_bytes.restype = _i64
_lib.mlora_packed_weight_bytes.argtypes = [_i64, _i64]
_lib.mlora_pack_weight.restype = ctypes.c_int
_lib.mlora_pack_weight.argtypes = [_P, _i64, _i64, _P, _P]
_lib.mlora_slot_load.restype = ctypes.c_int
_lib.mlora_slot_load.argtypes = [_P, _P, _P, _i32, _i32, _i32, _i64, _i64, _i32, _P, _P, _i32,
                                 ctypes.c_float, _P]
_lib.mlora_validate.restype = ctypes.c_int
_lib.mlora_validate.argtypes = [_P, _i64, _i32, _SLOTS_P, _P, ctypes.POINTER(_i64), _P]
_lib.mlora_plan.restype = ctypes.c_int
_lib.mlora_plan.argtypes = [_P, _i64, _i32, _i32, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.mlora_shrink.restype = ctypes.c_int
_lib.mlora_shrink.argtypes = [_P, _i64, _i64, _SLOTS_P, _P, _i32, _P, _P, _P, ctypes.c_size_t,
                              _P]
_lib.mlora_expand.restype = ctypes.c_int
_lib.mlora_expand.argtypes = [_P, _i64, _i64, _SLOTS_P, _P, _i32, _P, _P]
_lib.mlora_linear.restype = ctypes.c_int
_lib.mlora_linear.argtypes = [_P, _P, _i64, _i64, _i64, _SLOTS_P, _P, _i32, _P, _P, ctypes.c_uint32,
                              _P, ctypes.c_size_t, _P]
_lib.mlora_linear_path.restype = ctypes.c_uint32
_lib.mlora_linear_path.argtypes = [_i64, _i64, _i64, _SLOTS_P, _i32, ctypes.c_uint32]
_lib.mlora_linear_noalloc.restype = ctypes.c_int
_lib.mlora_linear_noalloc.argtypes = [_P, _P, _i64, _i64, _i64, _SLOTS_P, _P, _i32, _P, _P,
                                      ctypes.c_uint32, _P]
_lib.mlora_trace_start.restype = ctypes.c_int
_lib.mlora_trace_start.argtypes = [_i32]
_lib.mlora_trace_stop.restype = _i32
_lib.mlora_trace_stop.argtypes = [ctypes.POINTER(ctypes.c_float), _i32]


class MloraError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        extra = f" [{mlora_last_error()}]" if code == MLORA_ERR_HIP else ""
        super().__init__(f"{where}: {mlora_status_string(code)} (status {code}){extra}")


def _check(code: int, where: str):
    if code != MLORA_OK:
        raise MloraError(code, where)


def mlora_status_string(code: int) -> str:
    return _lib.mlora_status_string(int(code)).decode()


def mlora_last_error() -> str:
    return _lib.mlora_last_error().decode()


def mlora_factor(alpha: float, r: int, use_rslora: bool) -> float:
    return float(_lib.mlora_factor(float(alpha), int(r), int(bool(use_rslora))))


def mlora_slot_bytes(S: int, R: int, n_in: int, n_out: int, n_slices: int = 1) -> int:
    return int(_lib.mlora_slot_bytes(S, R, n_in, n_out, n_slices))


# ---------------------------------------------------------------------------------------------
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtypes, name):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def _bf16(t, name):
    import torch
    return _need(t, (torch.bfloat16, torch.uint16, torch.int16), name)


class Slots:
    """One layer's adapter slots: A [S][n_slices][R][n_in] bf16, B [S][n_out][R] bf16,
    factor [S] fp32 (device tensors), plus the host slice table and optionally the slots' true
    ranks (int32 [S] device tensor; None = every slot R wide)."""

    def __init__(self, A, B, factor, slice_start=None, rank=None):
        import torch
        self.A = _bf16(A, "A")
        self.B = _bf16(B, "B")
        self.factor = _need(factor, (torch.float32,), "factor")
        self.rank = None if rank is None else _need(rank, (torch.int32,), "rank")
        S, n_slices, R, _ = A.shape
        self.S, self.n_slices, self.R = int(S), int(n_slices), int(R)
        self.n_out = int(B.shape[1])
        st = [0] * (MLORA_MAX_SLICES + 1)
        if slice_start is not None:
            for i, v in enumerate(slice_start):
                st[i] = int(v)
        self.struct = mlora_slots(_ptr(self.A), _ptr(self.B), _ptr(self.factor), self.S, self.R,
                                  self.n_slices, (_i32 * (MLORA_MAX_SLICES + 1))(*st),
                                  _ptr(self.rank))

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def mlora_workspace_size(T: int, K: int, n_in: int, n_out: int, slots: Slots) -> int:
    return int(_lib.mlora_workspace_size(T, K, n_in, n_out, slots.ref))


def workspace(T: int, K: int, n_in: int, n_out: int, slots: Slots, device="cuda"):
    """A workspace of mlora_workspace_size() bytes."""
    import torch
    n = mlora_workspace_size(T, K, n_in, n_out, slots)
    if n == 0:
        raise MloraError(MLORA_ERR_ARG, "mlora_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mlora_packed_weight_bytes(n_out: int, n_in: int) -> int:
    return int(_lib.mlora_packed_weight_bytes(int(n_out), int(n_in)))


def mlora_pack_weight(W, stream=None):
    """The packed copy of a bf16 [n_out][n_in] device weight (a new device tensor), for
    mlora_linear(..., flags=MLORA_W_PACKED)."""
    import torch
    _bf16(W, "W")
    n_out, n_in = int(W.shape[0]), int(W.shape[1])
    nbytes = mlora_packed_weight_bytes(n_out, n_in)
    if nbytes <= 0:
        raise MloraError(MLORA_ERR_ARG, "mlora_packed_weight_bytes")
    Wp = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=W.device)
    _check(_lib.mlora_pack_weight(_ptr(W), n_out, n_in, _ptr(Wp), _stream(stream)),
           "mlora_pack_weight")
    return Wp


def mlora_slot_load(slots: Slots, n_in: int, slot: int, A_src, B_src, r: int, f: float,
                    stream=None):
    """Loads one adapter (A_src bf16 [n_slices][r][n_in], B_src bf16 [n_out][r]; host tensors
    pinned for an asynchronous copy, or device tensors) into slot `slot` of `slots`, zero
    padded to the slot width; writes f to the slot's factor."""
    import torch
    for t, name in ((A_src, "A_src"), (B_src, "B_src")):
        if not t.is_contiguous() or t.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
            raise ValueError(f"{name} must be a contiguous bf16 tensor")
    _check(_lib.mlora_slot_load(_ptr(slots.A), _ptr(slots.B), _ptr(slots.factor), slots.S,
                                slots.R, slots.n_slices, int(n_in), slots.n_out, int(slot),
                                _ptr(A_src), _ptr(B_src), int(r), float(f), _stream(stream)),
           "mlora_slot_load")


def mlora_validate(idx, slots: Slots, rank=None, stream=None):
    """Synchronous check; returns (status, offending value)."""
    import torch
    _need(idx, (torch.int32,), "idx")
    T, K = idx.shape
    bad = _i64(0)
    rk = None
    if rank is not None:
        import numpy as np
        rk = np.ascontiguousarray(rank, dtype=np.int32)
    code = _lib.mlora_validate(_ptr(idx), T, K, slots.ref,
                               None if rk is None else rk.ctypes.data_as(_P), ctypes.byref(bad),
                               _stream(stream))
    return code, int(bad.value)


def mlora_plan(idx, S: int, perm, seg_slot, seg_start, seg_len, counts, ws, stream=None):
    import torch
    _need(idx, (torch.int32,), "idx")
    for name, t in (("perm", perm), ("seg_slot", seg_slot), ("seg_start", seg_start),
                    ("seg_len", seg_len), ("counts", counts)):
        _need(t, (torch.int32,), name)
    T, K = idx.shape
    _check(_lib.mlora_plan(_ptr(idx), T, K, S, _ptr(perm), _ptr(seg_slot), _ptr(seg_start),
                           _ptr(seg_len), _ptr(counts), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "mlora_plan")


def mlora_shrink(x, slots: Slots, idx, scale, v, ws=None, stream=None):
    import torch
    _bf16(x, "x")
    _need(idx, (torch.int32,), "idx")
    _need(v, (torch.float32,), "v")
    if scale is not None:
        _need(scale, (torch.float32,), "scale")
    T, n_in = x.shape
    K = idx.shape[1]
    _check(_lib.mlora_shrink(_ptr(x), T, n_in, slots.ref, _ptr(idx), K, _ptr(scale), _ptr(v),
                             _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                             _stream(stream)), "mlora_shrink")


def mlora_expand(v, slots: Slots, idx, y, stream=None):
    import torch
    _need(v, (torch.float32,), "v")
    _need(idx, (torch.int32,), "idx")
    _bf16(y, "y")
    T, n_out = y.shape
    K = idx.shape[1]
    _check(_lib.mlora_expand(_ptr(v), T, n_out, slots.ref, _ptr(idx), K, _ptr(y),
                             _stream(stream)), "mlora_expand")


def mlora_linear(x, W, slots: Slots | None, idx, scale, y, flags: int = 0, ws=None, stream=None):
    import torch
    _bf16(x, "x")
    _bf16(W, "W")
    _bf16(y, "y")
    T, n_in = x.shape
    n_out = y.shape[1]          # W may be the packed (1-D) layout under MLORA_W_PACKED
    K = 1
    if idx is not None:
        _need(idx, (torch.int32,), "idx")
        K = idx.shape[1]
    if scale is not None:
        _need(scale, (torch.float32,), "scale")
    _check(_lib.mlora_linear(_ptr(x), _ptr(W), T, n_in, n_out,
                             None if slots is None else slots.ref, _ptr(idx), K, _ptr(scale),
                             _ptr(y), flags, _ptr(ws),
                             0 if ws is None else ws.numel() * ws.element_size(),
                             _stream(stream)), "mlora_linear")


def mlora_linear_path(T: int, n_in: int, n_out: int, slots: Slots | None, K: int = 1,
                      flags: int = 0) -> int:
    """The path mlora_linear takes for these sizes and flags (MLORA_PATH_DECODE, _TILED or
    _GROUPED), or 0 where its checks would fail."""
    return int(_lib.mlora_linear_path(T, n_in, n_out, None if slots is None else slots.ref, K,
                                      flags))


def mlora_linear_noalloc(x, W, slots: Slots | None, idx, scale, y, flags: int = 0,
                         stream=None):
    """mlora_linear with the library's fixed per-device scratch instead of a workspace."""
    import torch
    _bf16(x, "x")
    _bf16(W, "W")
    _bf16(y, "y")
    T, n_in = x.shape
    n_out = y.shape[1]
    K = 1
    if idx is not None:
        _need(idx, (torch.int32,), "idx")
        K = idx.shape[1]
    if scale is not None:
        _need(scale, (torch.float32,), "scale")
    _check(_lib.mlora_linear_noalloc(_ptr(x), _ptr(W), T, n_in, n_out,
                                     None if slots is None else slots.ref, _ptr(idx), K,
                                     _ptr(scale), _ptr(y), flags, _stream(stream)),
           "mlora_linear_noalloc")


def mlora_trace_start(capacity: int):
    _check(_lib.mlora_trace_start(capacity), "mlora_trace_start")


def mlora_trace_stop(capacity: int) -> list:
    """Durations (ms) of the main product kernel launches recorded since mlora_trace_start."""
    buf = (ctypes.c_float * max(capacity, 1))()
    n = _lib.mlora_trace_stop(buf, capacity)
    if n < 0:
        raise MloraError(MLORA_ERR_HIP, "mlora_trace_stop")
    return [float(buf[i]) for i in range(n)]
