"""CPU oracle for the multi-LoRA adapted linear layer (TEST INFRASTRUCTURE ONLY).

Loads ``oracle.c`` compiled with gcc (fp64 sums, -ffp-contract=off, OpenMP over tokens) and
marshals numpy arrays into it.  The same source is also built with fp32 sums (-DORACLE_ACC=float,
``liboracle_f32.so``): the plain fp32 CPU loop timed as the benchmark's CPU baseline.  Parity
and every pin use the fp64 build.  Only tests, the smoke check and the benchmark's CPU-baseline leg
may import this package; the GPU library never does.  The two sides share nothing but the seeded
inputs, which callers draw from the synthetic-input module and hand to each side.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB = os.path.join(_BUILD, "liboracle.so")
_LIB_F32 = os.path.join(_BUILD, "liboracle_f32.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle.c into oracle/_build/liboracle.so (fp64 sums) and liboracle_f32.so (fp32
    sums) with gcc."""
    os.makedirs(_BUILD, exist_ok=True)
    for lib, extra in ((_LIB, []), (_LIB_F32, ["-DORACLE_ACC=float"])):
        if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
            tmp = lib + f".tmp{os.getpid()}"
            subprocess.run(["gcc", *CFLAGS, *extra, _SRC, "-o", tmp, "-lm"], check=True)
            os.replace(tmp, lib)
    return _LIB


_libs = {}


def _load(acc: str = "f64"):
    """The fp64 build (acc="f64", every pin and parity check) or the fp32 one (acc="f32")."""
    if acc not in _libs:
        path = {"f64": _LIB, "f32": _LIB_F32}[acc]
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        lib.oracle_lora_factor.restype = ctypes.c_double
        lib.oracle_lora_factor.argtypes = [ctypes.c_double, i32, i32]
        lib.oracle_plan.restype = i32
        lib.oracle_plan.argtypes = [P, i64, i32, i32, P, P, P, P, P]
        lib.oracle_shrink.restype = None
        lib.oracle_shrink.argtypes = [P, i64, i64, P, i32, i32, i32, P, P, P, P, i32, P, P]
        lib.oracle_expand.restype = None
        lib.oracle_expand.argtypes = [P, i64, i64, P, i32, i32, i32, P, P, i32, P]
        lib.oracle_linear.restype = None
        lib.oracle_linear.argtypes = [P, P, i64, i64, i64, P, P, i32, i32, i32, P, P, P, P, P,
                                      i32, P, i32, P, i64, P]
        lib.oracle_slot_bytes.restype = i64
        lib.oracle_slot_bytes.argtypes = [i32, i32, i64, i64, i32]
        _libs[acc] = lib
    return _libs[acc]


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def lora_factor(alpha: float, r: int, use_rslora: bool) -> float:
    return _load().oracle_lora_factor(float(alpha), int(r), int(bool(use_rslora)))


def plan(idx: np.ndarray, S: int):
    """Stable sort of the flat (token, position) pairs by slot, -1 dropped.
    Returns (perm, seg_slot, seg_start, seg_len) as int32 arrays."""
    idx = _c(idx, np.int32)
    T = idx.shape[0]
    K = idx.shape[1] if idx.ndim == 2 else 1
    P = T * K
    perm = np.zeros(max(P, 1), np.int32)
    ss = np.zeros(max(S, 1), np.int32)
    st = np.zeros(max(S, 1), np.int32)
    sl = np.zeros(max(S, 1), np.int32)
    npairs = np.zeros(1, np.int64)
    g = _load().oracle_plan(_ptr(idx), T, K, S, _ptr(perm), _ptr(ss), _ptr(st), _ptr(sl),
                            _ptr(npairs))
    if g < 0:
        raise ValueError("index outside [-1, S)")
    n = int(npairs[0])
    return perm[:n].copy(), ss[:g].copy(), st[:g].copy(), sl[:g].copy()


def _slot_args(L):
    return (_c(L.alpha, np.float64), _c(L.rank, np.int32), _c(L.rslora, np.uint8))


def shrink(L) -> np.ndarray:
    """v[K][T][n_slices*R] in fp64 (zeros for -1 pairs)."""
    alpha, rank, rs = _slot_args(L)
    v = np.zeros((L.K, L.T, L.n_slices * L.R), np.float64)
    scale = _c(L.scale, np.float32)
    _load().oracle_shrink(_ptr(_c(L.x, np.uint16)), L.T, L.n_in, _ptr(_c(L.A, np.uint16)), L.S,
                          L.R, L.n_slices, _ptr(alpha), _ptr(rank), _ptr(rs),
                          _ptr(_c(L.idx, np.int32)), L.K, _ptr(scale), _ptr(v))
    return v


def expand(L, v: np.ndarray, y: np.ndarray | None = None) -> np.ndarray:
    """y[T][n_out] (fp64) += expand of v[K][T][n_slices*R]."""
    v = _c(v, np.float64)
    if y is None:
        y = np.zeros((L.T, L.n_out), np.float64)
    else:
        y = _c(y, np.float64).copy()
    _load().oracle_expand(_ptr(v), L.T, L.n_out, _ptr(_c(L.B, np.uint16)), L.S, L.R, L.n_slices,
                          _ptr(_c(L.slice_start, np.int32)), _ptr(_c(L.idx, np.int32)), L.K,
                          _ptr(y))
    return y


def linear(L, tokens=None, with_base: bool = True, acc: str = "f64") -> np.ndarray:
    """y rows for the listed tokens (all when None): base + every slot's delta, summed in fp64
    (acc="f64") or in fp32 (acc="f32", the timed CPU baseline); returned as float64."""
    alpha, rank, rs = _slot_args(L)
    if tokens is None:
        tok = None
        nt = L.T
    else:
        tok = _c(tokens, np.int64)
        nt = tok.shape[0]
        if nt and (tok.min() < 0 or tok.max() >= L.T):
            raise IndexError(f"token indices must lie in [0, {L.T})")
    y = np.zeros((nt, L.n_out), np.float64)
    scale = _c(L.scale, np.float32)
    _load(acc).oracle_linear(_ptr(_c(L.x, np.uint16)), _ptr(_c(L.W, np.uint16)), L.T, L.n_in,
                          L.n_out, _ptr(_c(L.A, np.uint16)), _ptr(_c(L.B, np.uint16)), L.S, L.R,
                          L.n_slices, _ptr(_c(L.slice_start, np.int32)), _ptr(alpha), _ptr(rank),
                          _ptr(rs), _ptr(_c(L.idx, np.int32)), L.K, _ptr(scale),
                          int(bool(with_base)), _ptr(tok), nt, _ptr(y))
    return y


def slot_bytes(S: int, R: int, n_in: int, n_out: int, n_slices: int = 1) -> int:
    return int(_load().oracle_slot_bytes(S, R, n_in, n_out, n_slices))
