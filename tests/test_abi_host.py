"""The C-ABI library on the host: it loads, exports every function include/mlora.h declares,
its host helpers agree with the pages' numbers, and argument checks return their status codes
before any HIP call (nothing here touches a GPU)."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def m():
    from lora_serving_amd import mlora
    return mlora


def header_functions():
    text = open(os.path.join(ROOT, "include", "mlora.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlora_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(m):
    names = header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(m._lib, name), name
    assert set(names) == set(m.EXPORTS)


def test_factor_matches_page_values(m):
    with open(os.path.join(ROOT, "tests", "golden", "rslora.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        assert m.mlora_factor(c["alpha"], c["r"], c["rslora"]) == c["factor"]
    assert m.mlora_factor(16, 0, 0) != m.mlora_factor(16, 0, 0)  # NaN for r < 1


def test_slot_bytes_matches_page_sizing(m):
    with open(os.path.join(ROOT, "tests", "golden", "sizing.json")) as fh:
        g = json.load(fh)
    mods = g["model"]["modules"]

    def adapter(rank, slots=1):
        return g["model"]["layers"] * sum(m.mlora_slot_bytes(slots, rank, i, o, 1)
                                          for i, o in mods.values())

    for r, mib in g["printed"]["adapter_MiB_0dp"].items():
        assert round(adapter(int(r)) / 2 ** 20) == mib
    for slots, rank, gib in g["printed"]["slots_GiB_2dp"]:
        assert round(adapter(rank, slots) / 2 ** 30, 2) == gib
    assert m.mlora_slot_bytes(-1, 16, 1, 1, 1) == -1


def slots_struct(m, S=4, R=16, n_slices=1, starts=None, A=0x1000, B=0x2000, f=0x3000):
    st = (ctypes.c_int32 * 5)(*(starts or [0, 0, 0, 0, 0]))
    return m.mlora_slots(A, B, f, S, R, n_slices, st)


def test_workspace_size(m):
    s = slots_struct(m)
    assert m._lib.mlora_workspace_size(64, 1, 4096, 4096, ctypes.byref(s)) > 0
    assert m._lib.mlora_workspace_size(-1, 1, 4096, 4096, ctypes.byref(s)) == 0
    assert m._lib.mlora_workspace_size(64, 0, 4096, 4096, ctypes.byref(s)) == 0
    bad = slots_struct(m, R=24)
    assert m._lib.mlora_workspace_size(64, 1, 4096, 4096, ctypes.byref(bad)) == 0


def call_linear(m, slots, T=8, n_in=64, n_out=32, K=1, x=0x10000, W=0x20000, y=0x30000,
                idx=0x40000, ws=None, ws_bytes=0, flags=0):
    sp = None if slots is None else ctypes.byref(slots)
    return m._lib.mlora_linear(x, W, T, n_in, n_out, sp, idx, K, None, y, flags, ws, ws_bytes,
                               None)


def test_linear_argument_checks(m):
    s = slots_struct(m)
    assert call_linear(m, s, T=-1) == m.MLORA_ERR_ARG
    assert call_linear(m, s, K=0) == m.MLORA_ERR_ARG
    assert call_linear(m, s, K=9) == m.MLORA_ERR_ARG
    assert call_linear(m, s, n_in=60) == m.MLORA_ERR_SHAPE
    assert call_linear(m, None) == m.MLORA_ERR_ARG
    assert call_linear(m, slots_struct(m, R=24)) == m.MLORA_ERR_UNSUPPORTED
    assert call_linear(m, slots_struct(m, R=1024)) == m.MLORA_ERR_UNSUPPORTED
    assert call_linear(m, slots_struct(m, S=0)) == m.MLORA_ERR_UNSUPPORTED
    assert call_linear(m, slots_struct(m, n_slices=5)) == m.MLORA_ERR_UNSUPPORTED
    assert call_linear(m, slots_struct(m, n_slices=2, starts=[0, 40, 32, 0, 0])) == \
        m.MLORA_ERR_SHAPE
    assert call_linear(m, slots_struct(m, n_slices=2, starts=[0, 16, 31, 0, 0])) == \
        m.MLORA_ERR_SHAPE
    assert call_linear(m, slots_struct(m, A=0)) == m.MLORA_ERR_ARG
    assert call_linear(m, slots_struct(m, A=0x1008)) == m.MLORA_ERR_ARG   # misaligned
    assert call_linear(m, s, x=0) == m.MLORA_ERR_ARG
    assert call_linear(m, s, y=0x30002) == m.MLORA_ERR_ARG
    assert call_linear(m, s, idx=0) == m.MLORA_ERR_ARG
    assert call_linear(m, s) == m.MLORA_ERR_WORKSPACE          # no workspace
    assert call_linear(m, s, ws=0x50000, ws_bytes=16) == m.MLORA_ERR_WORKSPACE
    assert call_linear(m, s, T=0) == m.MLORA_OK                # T = 0 is a no-op
    assert call_linear(m, s, flags=m.MLORA_PATH_DECODE | m.MLORA_PATH_TILED) == m.MLORA_ERR_ARG
    assert call_linear(m, s, flags=m.MLORA_PATH_GROUPED | m.MLORA_PATH_TILED) == m.MLORA_ERR_ARG
    assert call_linear(m, s, flags=m.MLORA_PATH_GROUPED | m.MLORA_PATH_DECODE) == m.MLORA_ERR_ARG
    # base-only hint needs no slots and no index map, but still a workspace
    assert call_linear(m, None, idx=0, flags=m.MLORA_NO_ADAPTERS) == m.MLORA_ERR_WORKSPACE


def test_linear_path_choice(m):
    """The host-side choice of mlora_linear's kernels for the workloads' shapes and the
    forcing flags (no GPU call)."""
    L = m._lib
    dec, til, grp = m.MLORA_PATH_DECODE, m.MLORA_PATH_TILED, m.MLORA_PATH_GROUPED
    s16 = slots_struct(m, S=100, R=16)
    qkv = slots_struct(m, S=64, R=64, n_slices=3, starts=[0, 4096, 5120, 6144, 0])
    path = lambda T, n_in, n_out, s, K=1, flags=0: L.mlora_linear_path(T, n_in, n_out,
                                                                        ctypes.byref(s), K, flags)
    assert path(64, 4096, 4096, s16) == dec            # decode batch
    assert path(256, 4096, 4096, s16) == dec           # 256 tokens at rank 16: gather ~2x W
    assert path(64, 4096, 100_000, s16) == dec         # LM head
    assert path(16384, 4096, 11008, slots_struct(m, S=100, R=64)) == til   # prefill
    assert path(2304, 4096, 6144, qkv) == til          # the mixed batch
    assert path(256, 4096, 6144, qkv) == grp           # its 256 one-token requests: ~12x W
    # the per-pair gather must also be large in itself (200 MB) for the group kernels to pay
    s64, s32 = slots_struct(m, S=64, R=64), slots_struct(m, S=64, R=32)
    assert path(256, 4096, 4096, s64) == grp           # 268 MB of gather
    assert path(128, 4096, 4096, s64) == dec           # 134 MB
    assert path(256, 4096, 4096, s32) == dec           # 134 MB
    assert path(256, 4096, 512, s16) == dec            # narrow layer: 38 MB, 9x W
    assert path(1024, 512, 4096, s16) == dec           # narrow input
    assert path(2048, 512, 4096, s16) == til
    assert path(2048, 4096, 512, s16) == dec           # 8 output tiles of 256 rows
    assert path(4096, 4096, 512, s16) == til
    assert path(1024, 11008, 4096, s16) == til         # wide input: a round of 64 tiles
    assert path(512, 11008, 4096, s16) == dec
    assert path(256, 4096, 6144, qkv, flags=dec) == dec
    assert path(256, 4096, 6144, qkv, flags=til) == til
    assert path(64, 4096, 4096, s16, flags=grp) == grp
    assert path(256, 4096, 6144, qkv, flags=m.MLORA_NO_ADAPTERS) == dec   # base only
    assert path(512, 4096, 100_000, s16, flags=grp) == 0   # 2 tiles of fp32 sums: too wide
    assert path(64, 4096, 4096, s16, flags=dec | grp) == 0
    assert path(64, 4096, 4096, slots_struct(m, R=24)) == 0
    assert path(-1, 4096, 4096, s16) == 0


def test_other_entry_points_argument_checks(m):
    s = slots_struct(m)
    L = m._lib
    assert L.mlora_shrink(0x1000, -1, 64, ctypes.byref(s), 0x2000, 1, None, 0x3000, None, 0,
                          None) == m.MLORA_ERR_ARG
    assert L.mlora_shrink(0x1000, 4, 60, ctypes.byref(s), 0x2000, 1, None, 0x3000, None, 0,
                          None) == m.MLORA_ERR_SHAPE
    assert L.mlora_shrink(0x1000, 4, 64, None, 0x2000, 1, None, 0x3000, None, 0, None) == \
        m.MLORA_ERR_ARG
    assert L.mlora_shrink(0, 4, 64, ctypes.byref(s), 0x2000, 1, None, 0x3000, None, 0, None) == \
        m.MLORA_ERR_ARG
    assert L.mlora_expand(0x1000, 4, 32, ctypes.byref(s), 0x2000, 0, 0x3000, None) == \
        m.MLORA_ERR_ARG
    assert L.mlora_expand(0, 4, 32, ctypes.byref(s), 0x2000, 1, 0x3000, None) == m.MLORA_ERR_ARG
    assert L.mlora_plan(0x1000, 4, 1, 0, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 1 << 20,
                        None) == m.MLORA_ERR_UNSUPPORTED
    assert L.mlora_plan(0x1000, 4, 1, 4, 0x2000, 0x3000, 0x4000, 0x5000, None, 0x7000, 1 << 20,
                        None) == m.MLORA_ERR_ARG
    assert L.mlora_plan(0x1000, 4, 1, 4, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, 0,
                        None) == m.MLORA_ERR_WORKSPACE
    bad = ctypes.c_int64(0)
    rk = (ctypes.c_int32 * 4)(8, 16, 17, 4)
    assert L.mlora_validate(0x1000, 0, 1, ctypes.byref(s), rk, ctypes.byref(bad), None) == \
        m.MLORA_ERR_RANK
    assert bad.value == 17
    rk0 = (ctypes.c_int32 * 4)(8, 0, 16, 4)
    assert L.mlora_validate(0x1000, 0, 1, ctypes.byref(s), rk0, ctypes.byref(bad), None) == \
        m.MLORA_ERR_RANK
    ok = (ctypes.c_int32 * 4)(8, 16, 16, 4)
    assert L.mlora_validate(0x1000, 0, 1, ctypes.byref(s), ok, None, None) == m.MLORA_OK


def test_slot_load_argument_checks(m):
    """Rank above the slot width (the pages' rejection of ranks over max_lora_rank), rank 0,
    slot outside [0, S), NULL buffers, unsupported slot widths: all refused before any copy."""
    L = m._lib
    args = dict(A=0x1000, B=0x2000, f=0x3000, S=4, R=16, ns=1, n_in=64, n_out=32, slot=1,
                As=0x4000, Bs=0x5000, r=8)

    def call(**kw):
        a = dict(args, **kw)
        return L.mlora_slot_load(a["A"], a["B"], a["f"], a["S"], a["R"], a["ns"], a["n_in"],
                                 a["n_out"], a["slot"], a["As"], a["Bs"], a["r"], 2.0, None)
    assert call(r=17) == m.MLORA_ERR_RANK
    assert call(r=0) == m.MLORA_ERR_RANK
    assert call(slot=4) == m.MLORA_ERR_ARG
    assert call(slot=-1) == m.MLORA_ERR_ARG
    assert call(A=None) == m.MLORA_ERR_ARG
    assert call(Bs=None) == m.MLORA_ERR_ARG
    assert call(n_in=0) == m.MLORA_ERR_ARG
    assert call(R=12) == m.MLORA_ERR_UNSUPPORTED
    assert call(ns=5) == m.MLORA_ERR_UNSUPPORTED


def test_packed_weight_size_and_argument_checks(m):
    L = m._lib
    # padded to 16 rows and 32 columns, 2 bytes each
    assert m.mlora_packed_weight_bytes(4096, 4096) == 4096 * 4096 * 2
    assert m.mlora_packed_weight_bytes(100000, 4096) == 100000 * 4096 * 2
    assert m.mlora_packed_weight_bytes(520, 392) == 528 * 416 * 2
    assert m.mlora_packed_weight_bytes(0, 64) == 0
    assert L.mlora_pack_weight(None, 16, 64, 0x2000, None) == m.MLORA_ERR_ARG
    assert L.mlora_pack_weight(0x1000, 16, 64, None, None) == m.MLORA_ERR_ARG
    assert L.mlora_pack_weight(0x1008, 16, 64, 0x2000, None) == m.MLORA_ERR_ARG   # misaligned
    assert L.mlora_pack_weight(0x1000, 16, 60, 0x2000, None) == m.MLORA_ERR_SHAPE


def test_trace_hook_argument_checks(m):
    assert m._lib.mlora_trace_start(0) == m.MLORA_ERR_ARG
    assert m._lib.mlora_trace_start((1 << 20) + 1) == m.MLORA_ERR_ARG
    assert m._lib.mlora_trace_stop(None, 0) == 0    # nothing recorded, nothing to release


def test_status_strings(m):
    for code in range(8):
        assert m.mlora_status_string(code)
    assert m.mlora_status_string(99) == "unknown status"
