"""The benchmark's algorithmic byte and flop counts (the numerators of its roofline fractions)
against their closed forms: W, x and y once, each distinct used adapter's A and B rows once at
its true rank, the index map, scales and factors; flops 2 T n_in n_out plus 2 r (n_slices n_in
+ n_out) per used (token, slot).  No GPU needed."""
import types

import numpy as np

import bench
from lora_serving_amd import synth


def test_decode_counts_closed_form():
    L = synth.workload_decode()
    a = bench.algorithmic(L)
    D = len(np.unique(L.idx[L.idx >= 0]))
    used = int(np.count_nonzero(L.idx >= 0))
    assert a["distinct_adapters"] == D
    # rank 16, 4096 -> 4096: an adapter's A and B rows are 2 x 16 x 4096 x 2 bytes
    per_adapter = 2 * 16 * 4096 * 2
    meta = L.T * 4 + L.T * 4 + L.S * 4                 # idx, scale, factor
    w, xy = 4096 * 4096 * 2, 64 * 4096 * 2
    assert a["bytes"] == w + 2 * xy + D * per_adapter + meta
    assert a["decode_kernel_bytes"] == w + xy + D * per_adapter // 2 + meta
    assert a["flops"] == 2.0 * 64 * 4096 * 4096 + used * 2.0 * 16 * (4096 + 4096)
    # the pair: shrink reads x and the A rows and writes v; expand reads v, B, y, writes y
    v = L.K * L.T * L.n_slices * L.R * 4
    assert a["shrink_bytes"] == xy + D * per_adapter // 2 + v + meta
    assert a["expand_bytes"] == 2 * xy + D * per_adapter // 2 + v + meta


def test_prefill_flops_match_the_survey_figures():
    # every token has an adapter (K = 1, rank 64): 1,477.5 G of base product + 31.7 G of LoRA
    L = types.SimpleNamespace(T=16384, K=1, S=100, R=64, n_in=4096, n_out=11008, n_slices=1,
                              idx=np.zeros((16384, 1), np.int32),
                              rank=np.full(100, 64, np.int32),
                              scale=np.ones((16384, 1), np.float32))
    a = bench.algorithmic(L)
    base = 2.0 * 16384 * 4096 * 11008
    lora = 16384 * 2.0 * 64 * (4096 + 11008)
    assert a["flops"] == base + lora
    assert abs(base / 1e9 - 1477.5) < 0.1 and abs(lora / 1e9 - 31.7) < 0.1
    assert a["tiled_kernel_flops"] == base + 16384 * 2.0 * 64 * 11008


def test_decode_shrink_route_label_matches_the_library_cases():
    """The benchmark's copy of the decode path's shrink route (label and byte count of the GEMM)
    gives the routes the GPU test checks from the kernels the library launches."""
    from tests.gpu_util import DECODE_ROUTE_CASES
    for T, n_out, R, K, slices, apart in DECODE_ROUTE_CASES:
        wd = (len(slices) if slices else 1) * R
        assert bench.decode_shrink_apart(T, K, n_out, wd) == apart
