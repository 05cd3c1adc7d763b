"""HIP graph capture of the library's calls.

A serving loop captures its decode steps in a graph so that the host's cost per call is paid
once per replay.  mlora_linear (decode path, also on its persistent grid; grouped decode, with
its side stream and on the caller's stream alone; tiled path with stacked and with scattered
tiles), the mlora_shrink / mlora_expand pair and mlora_plan are captured together on torch's
capture stream, then the graph is replayed several times with the program's own eager work
and synchronizations between the replays; every replay must reproduce the eager results bit
for bit (the kernels are deterministic, and no call allocates memory or records a memset).
"""
import sys

import numpy as np
import pytest

from lora_serving_amd import synth
from tests.gpu_util import DevLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lora_serving_amd import mlora  # noqa: F401  (fails loudly if the library is missing)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_graph_replays_match_eager():
    import torch
    from lora_serving_amd import mlora
    # 32 row tiles for 128 (token, slot) pairs: the decode path's shrink runs apart, ahead of a
    # GEMM of the base alone (the 150-token layer below keeps it in the GEMM pass)
    Ld = synth.random_layer(81, T=64, n_in=1024, n_out=2048, S=8, R=16, K=2, p_sentinel=0.2)
    Lt = synth.random_layer(82, T=700, n_in=512, n_out=1024, S=9, R=16, K=2, p_sentinel=0.2,
                            contiguous=True)
    # tokens spread over 40 adapters: scattered tiles (per-adapter shrink items, one expand
    # launch per slot after the GEMM)
    Ls = synth.random_layer(83, T=300, n_in=256, n_out=512, S=40, R=16, K=3, p_sentinel=0.2)
    # three 64-token chunks over 64 row tiles: the decode GEMM's persistent grid, and the
    # grouped decode with all its kernels on the caller's stream
    Lp = synth.random_layer(84, T=150, n_in=1024, n_out=4096, S=8, R=16, K=2, p_sentinel=0.2)
    say(f"[graph] decode T={Ld.T} {Ld.n_in}->{Ld.n_out}, tiled T={Lt.T} {Lt.n_in}->{Lt.n_out}, "
        f"persistent T={Lp.T} {Lp.n_in}->{Lp.n_out}")
    Dd, Dt, Ds, Dp = DevLayer(Ld), DevLayer(Lt), DevLayer(Ls), DevLayer(Lp)
    dev = Dd.device
    bf = torch.bfloat16
    yd = torch.empty((Ld.T, Ld.n_out), dtype=bf, device=dev)
    yt = torch.empty((Lt.T, Lt.n_out), dtype=bf, device=dev)
    ys = torch.empty((Ls.T, Ls.n_out), dtype=bf, device=dev)
    yg = torch.empty((Ld.T, Ld.n_out), dtype=bf, device=dev)
    yp = torch.empty((Lp.T, Lp.n_out), dtype=bf, device=dev)
    ypg = torch.empty((Lp.T, Lp.n_out), dtype=bf, device=dev)
    v = torch.empty((Ld.K, Ld.T, Ld.n_slices * Ld.R), dtype=torch.float32, device=dev)
    y_base = torch.randn((Ld.T, Ld.n_out), device=dev).to(bf)      # expand accumulates onto it
    ye = torch.empty_like(y_base)
    i32 = lambda n: torch.empty((n,), dtype=torch.int32, device=dev)
    perm, ss, st, sl, cnt = i32(Ld.T * Ld.K), i32(Ld.S), i32(Ld.S), i32(Ld.S), i32(2)
    outs = [yd, yt, ys, yg, yp, ypg, v, ye, perm, ss, st, sl, cnt]
    names = ["yd", "yt", "ys", "yg", "yp", "ypg", "v", "ye", "perm", "ss", "st", "sl", "cnt"]

    def work():
        mlora.mlora_linear(Dd.x, Dd.W, Dd.slots, Dd.idx, Dd.scale, yd,
                           flags=mlora.MLORA_PATH_DECODE, ws=Dd.ws)
        mlora.mlora_linear(Dt.x, Dt.W, Dt.slots, Dt.idx, Dt.scale, yt,
                           flags=mlora.MLORA_PATH_TILED, ws=Dt.ws)
        mlora.mlora_linear(Ds.x, Ds.W, Ds.slots, Ds.idx, Ds.scale, ys,
                           flags=mlora.MLORA_PATH_TILED, ws=Ds.ws)
        mlora.mlora_linear(Dd.x, Dd.W, Dd.slots, Dd.idx, Dd.scale, yg,
                           flags=mlora.MLORA_PATH_GROUPED, ws=Dd.ws)
        mlora.mlora_linear(Dp.x, Dp.W, Dp.slots, Dp.idx, Dp.scale, yp,
                           flags=mlora.MLORA_PATH_DECODE, ws=Dp.ws)
        mlora.mlora_linear(Dp.x, Dp.W, Dp.slots, Dp.idx, Dp.scale, ypg,
                           flags=mlora.MLORA_PATH_GROUPED, ws=Dp.ws)
        mlora.mlora_shrink(Dd.x, Dd.slots, Dd.idx, Dd.scale, v, ws=Dd.ws)
        torch.mul(y_base, 1.0, out=ye)         # a kernel, not a copy or memset node
        mlora.mlora_expand(v, Dd.slots, Dd.idx, ye)
        mlora.mlora_plan(Dd.idx, Ld.S, perm, ss, st, sl, cnt, Dd.ws)

    def bits(t):
        return t.view(torch.int16) if t.dtype == bf else t.view(torch.int32)

    # the plan writes only the first n_pairs / n_seg entries: start every run from -1 bits
    for t in outs:
        bits(t).fill_(-1)
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()

    y_other = torch.empty_like(yt)
    for rep in range(4):
        # the program's own eager work between replays: clobber the outputs and run the
        # library on the other layer's inputs
        for t in outs:
            bits(t).fill_(-1)
        mlora.mlora_linear(Dt.x, Dt.W, Dt.slots, Dt.idx, None, y_other,
                           flags=mlora.MLORA_PATH_TILED, ws=Dt.ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"[graph] replay {rep}")
        assert len(names) == len(outs) == len(ref)
        for name, t, r in zip(names, outs, ref):
            assert torch.equal(bits(t), bits(r)), f"replay {rep}: {name} differs from eager"
    assert int(cnt[1].item()) == int(np.count_nonzero(Ld.idx >= 0))
