"""mlora_linear_noalloc, the layer for callers that cannot allocate (its scratch is a fixed
array inside the library, one per GPU), against mlora_linear with a caller workspace on the same
inputs: the same kernels, so the same output bits, and the oracle's values within the layer's
acceptance bound.  Consecutive calls share the fixed array: the second call of each pair is
smaller than the first, so anything the first call left behind in the array would show."""
import numpy as np
import pytest

import oracle
from lora_serving_amd import synth
from tests.gpu_util import DevLayer, from_dev_bf16, tol_ok


def _pair(D, flags=0):
    import torch
    from lora_serving_amd import mlora
    T, n_out = D.L.T, D.L.n_out
    slots = mlora.Slots(D.A, D.B, D.factor, slice_start=[int(v) for v in D.L.slice_start],
                        rank=D.rank)
    y_ws = torch.full((T, n_out), 7.0, dtype=torch.bfloat16, device=D.device)
    y_na = torch.full((T, n_out), -3.0, dtype=torch.bfloat16, device=D.device)
    mlora.mlora_linear(D.x, D.W, slots, D.idx, D.scale, y_ws, flags=flags, ws=D.ws)
    mlora.mlora_linear_noalloc(D.x, D.W, slots, D.idx, D.scale, y_na, flags=flags)
    torch.cuda.synchronize()
    return y_ws, y_na


def _check(L, flags=0):
    import torch
    D = DevLayer(L)
    y_ws, y_na = _pair(D, flags)
    print(f"noalloc: T={L.T} K={L.K} n_in={L.n_in} n_out={L.n_out} flags={flags}", flush=True)
    assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16))
    y_ref = oracle.linear(L)
    assert tol_ok(from_dev_bf16(y_na), y_ref).all()


@pytest.mark.gpu
def test_noalloc_decode_two_calls_second_smaller():
    _check(synth.random_layer(7101, T=64, n_in=1024, n_out=2048, S=12, R=16, K=2,
                              p_sentinel=0.2))
    _check(synth.random_layer(7102, T=21, n_in=512, n_out=392, S=5, R=32, K=1,
                              slice_sizes=[256, 136], p_sentinel=0.3))


@pytest.mark.gpu
def test_noalloc_fused_shrink_decode_then_smaller():
    """The decode path with its shrink in the GEMM pass (the calls above take the shrink
    apart: few row tiles for their pairs), then a smaller call of the same kind."""
    _check(synth.random_layer(7108, T=64, n_in=1024, n_out=4096, S=12, R=16, K=1,
                              p_sentinel=0.2))
    _check(synth.random_layer(7109, T=48, n_in=512, n_out=3072, S=6, R=16, K=1,
                              p_sentinel=0.3))


@pytest.mark.gpu
def test_noalloc_tiled_then_smaller_decode():
    from lora_serving_amd import mlora
    _check(synth.random_layer(7103, T=600, n_in=256, n_out=512, S=6, R=16, K=2,
                              p_sentinel=0.2, contiguous=True), flags=mlora.MLORA_PATH_TILED)
    _check(synth.random_layer(7104, T=40, n_in=256, n_out=320, S=6, R=16, K=3, p_sentinel=0.4))


@pytest.mark.gpu
def test_noalloc_grouped_decode_then_smaller():
    from lora_serving_amd import mlora
    _check(synth.random_layer(7106, T=300, n_in=512, n_out=768, S=20, R=32, K=2,
                              slice_sizes=[512, 128, 128], p_sentinel=0.2),
           flags=mlora.MLORA_PATH_GROUPED)
    _check(synth.random_layer(7107, T=33, n_in=256, n_out=264, S=5, R=16, K=3, p_sentinel=0.3),
           flags=mlora.MLORA_PATH_GROUPED)


@pytest.mark.gpu
def test_noalloc_rejects_calls_beyond_the_fixed_scratch():
    """A 4096 -> 100,000 decode call needs about 100 MB of split partials: refused before any
    launch, y untouched, the needed size named; the next call that fits still works."""
    import torch
    from lora_serving_amd import mlora
    T, n_in, n_out, S, R = 64, 4096, 100_000, 4, 16
    x = torch.zeros((T, n_in), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((n_out, n_in), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((S, 1, R, n_in), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((S, n_out, R), dtype=torch.bfloat16, device="cuda")
    f = torch.ones(S, dtype=torch.float32, device="cuda")
    idx = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
    y = torch.full((T, n_out), 5.0, dtype=torch.bfloat16, device="cuda")
    slots = mlora.Slots(A, B, f)
    with pytest.raises(mlora.MloraError) as e:
        mlora.mlora_linear_noalloc(x, W, slots, idx, None, y)
    assert e.value.code == mlora.MLORA_ERR_WORKSPACE
    assert "scratch" in mlora.mlora_last_error()
    torch.cuda.synchronize()
    assert bool((y == 5.0).all())
    del x, W, A, B, y
    _check(synth.random_layer(7105, T=16, n_in=256, n_out=256, S=4, R=8, K=1))
