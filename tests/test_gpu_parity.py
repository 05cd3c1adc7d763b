"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Acceptance (floating point): |y - y_ref| <= 2e-2 (1 + |y_ref|) elementwise, on the whole layer
and on the LoRA delta alone (shrink, then expand into a zero y), so a wrong delta cannot hide
under a large W x.  The mapping plan must match bit-exactly.
"""
import dataclasses
import sys

import numpy as np
import pytest

from lora_serving_amd import synth
from tests.gpu_util import DECODE_ROUTE_CASES, DevLayer, from_dev_bf16, tol_ok, worst

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


def check_linear(oracle_mod, L, tokens=None, label=""):
    say(f"[linear] {label} T={L.T} n_in={L.n_in} n_out={L.n_out} K={L.K} S={L.S} R={L.R} "
        f"slices={L.n_slices}")
    D = DevLayer(L)
    y = from_dev_bf16(D.linear())
    if tokens is None:
        y_ref = oracle_mod.linear(L)
        yy = y
    else:
        y_ref = oracle_mod.linear(L, tokens=tokens)
        yy = y[tokens]
    ok = tol_ok(yy, y_ref)
    assert ok.all(), f"{label}: worst {worst(yy, y_ref):.3e}, {np.sum(~ok)} elements out"
    return D, y


def check_delta(oracle_mod, L, D=None, tokens=None, label=""):
    say(f"[delta] {label} T={L.T} K={L.K}")
    D = D or DevLayer(L)
    d = from_dev_bf16(D.delta())
    d_ref = oracle_mod.linear(L, tokens=tokens, with_base=False)
    dd = d if tokens is None else d[tokens]
    ok = tol_ok(dd, d_ref)
    assert ok.all(), f"{label}: delta worst {worst(dd, d_ref):.3e}"
    assert np.any(d_ref != 0) == np.any(dd != 0)
    return d


# ------------------------------------------------------------------------------------------
SMALL = [
    # seed, T, n_in, n_out, S, R, K, slices
    (1, 1, 64, 48, 3, 8, 1, None),
    (2, 17, 256, 200, 5, 16, 2, None),
    (3, 64, 512, 520, 7, 16, 3, [260, 130, 130]),
    (4, 100, 392, 136, 4, 64, 1, [64, 72]),
    (5, 128, 1024, 1000, 9, 32, 2, None),
    (6, 129, 320, 264, 6, 16, 3, [200, 32, 32]),
    (7, 300, 2056, 136, 11, 8, 1, None),
    (8, 20, 512, 4096, 5, 16, 3, [2048, 1024, 1024]),   # 60 pairs over 5 slots: grouped shrink
    (9, 64, 256, 4096, 40, 32, 1, None),                # 64 pairs, wd > 16: grouped + per pair
    (10, 45, 256, 203, 5, 16, 2, [101, 102]),           # n_out not a multiple of 4
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}" for c in SMALL])
def test_linear_and_delta_small(oracle_mod, case):
    seed, T, n_in, n_out, S, R, K, slices = case
    L = synth.random_layer(seed, T=T, n_in=n_in, n_out=n_out, S=S, R=R, K=K, slice_sizes=slices,
                           p_sentinel=0.25)
    D, _ = check_linear(oracle_mod, L, label=f"small{seed}")
    check_delta(oracle_mod, L, D, label=f"small{seed}")


TILED = [
    # seed, T, n_in, n_out, S, R, K, slices   (tiled prefill kernels forced)
    (41, 300, 392, 520, 7, 16, 3, [260, 130, 130]),
    (42, 257, 256, 256, 5, 64, 1, None),
    (43, 700, 1032, 600, 9, 8, 2, [300, 300]),
    (44, 64, 128, 136, 3, 32, 1, None),
    (45, 520, 512, 1024, 40, 16, 3, [512, 256, 256]),
    (46, 300, 256, 301, 6, 16, 2, [150, 151]),          # n_out not a multiple of 4
]


@pytest.mark.parametrize("case", TILED, ids=[f"t{c[0]}" for c in TILED])
def test_tiled_path_small(oracle_mod, case):
    from lora_serving_amd import mlora
    seed, T, n_in, n_out, S, R, K, slices = case
    for contiguous in (True, False):
        L = synth.random_layer(seed, T=T, n_in=n_in, n_out=n_out, S=S, R=R, K=K,
                               slice_sizes=slices, p_sentinel=0.25, contiguous=contiguous)
        say(f"[tiled] seed={seed} T={T} n_in={n_in} n_out={n_out} K={K} R={R} "
            f"contiguous={contiguous}")
        D = DevLayer(L)
        y = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_TILED))
        y_ref = oracle_mod.linear(L)
        ok = tol_ok(y, y_ref)
        assert ok.all(), f"tiled {seed}: worst {worst(y, y_ref):.3e}, {np.sum(~ok)} out"
        # the tiled and the decode kernels agree within the same bound
        y2 = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_DECODE))
        assert tol_ok(y2, y_ref).all()


GROUPED = [
    # seed, T, n_in, n_out, S, R, K, slices   (grouped decode forced)
    (60, 1, 64, 48, 3, 8, 1, None),
    (61, 37, 256, 200, 5, 16, 2, None),
    (62, 300, 512, 520, 30, 32, 3, [260, 130, 130]),   # two tiles, the second ragged
    (63, 600, 392, 136, 9, 64, 1, [64, 72]),           # two launches: 512 + 88 tokens
    (64, 256, 1024, 1000, 40, 16, 2, None),
    (66, 140, 256, 202, 6, 16, 2, [101, 101]),          # n_out not a multiple of 4
]


@pytest.mark.parametrize("case", GROUPED, ids=[f"g{c[0]}" for c in GROUPED])
def test_grouped_decode_small(oracle_mod, case):
    """The grouped decode (decode kernels' base product, LoRA terms per adapter group with
    every 256-token tile on the scattered route) against the oracle, on maps with runs of one
    adapter and on scattered ones; and the plain decode path within the same bound."""
    from lora_serving_amd import mlora
    seed, T, n_in, n_out, S, R, K, slices = case
    for contiguous in (False, True):
        L = synth.random_layer(seed, T=T, n_in=n_in, n_out=n_out, S=S, R=R, K=K,
                               slice_sizes=slices, p_sentinel=0.25, contiguous=contiguous)
        say(f"[grouped] seed={seed} T={T} n_in={n_in} n_out={n_out} K={K} R={R} "
            f"contiguous={contiguous}")
        D = DevLayer(L)
        y = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_GROUPED))
        y_ref = oracle_mod.linear(L)
        ok = tol_ok(y, y_ref)
        assert ok.all(), f"grouped {seed}: worst {worst(y, y_ref):.3e}, {np.sum(~ok)} out"
        y2 = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_DECODE))
        assert tol_ok(y2, y_ref).all()


def test_grouped_decode_rank_table_and_sentinels(oracle_mod):
    """Grouped decode with the slots' true ranks (V blocks and expand walks sized by the
    tile's largest rank), and an all-sentinel map (y = W x exactly as with MLORA_NO_ADAPTERS)."""
    import torch
    from lora_serving_amd import mlora
    ranks = [8, 16, 64, 24, 8, 40, 16, 5, 12]
    L = synth.random_layer(65, T=400, n_in=512, n_out=384, S=9, R=64, K=2,
                           slice_sizes=[256, 64, 64], ranks=ranks, p_sentinel=0.2)
    say(f"[grouped ranked] T={L.T} ranks={ranks}")
    D = DevLayer(L)
    D.slots = mlora.Slots(D.A, D.B, D.factor, slice_start=[int(v) for v in L.slice_start],
                          rank=torch.tensor(ranks, dtype=torch.int32, device="cuda"))
    y = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_GROUPED))
    y_ref = oracle_mod.linear(L)
    assert tol_ok(y, y_ref).all(), f"worst {worst(y, y_ref):.3e}"
    D.idx.fill_(-1)
    y_all = D.linear(flags=mlora.MLORA_PATH_GROUPED).clone()
    y_base = D.linear(flags=mlora.MLORA_PATH_DECODE | mlora.MLORA_NO_ADAPTERS)
    assert torch.equal(y_all.view(torch.int16), y_base.view(torch.int16))


def test_grouped_decode_chosen_for_heavy_gather(oracle_mod):
    """The mixed batch's 256 one-token requests alone (merged QKV, ranks up to 64 padded to
    64): their per-pair A and B reads are about 12 times W, so the library takes the grouped
    decode by itself (the group shrink and the grouped expand around the decode GEMM and
    finish); the result matches the oracle on every third token and the last."""
    L = synth.workload_mixed_qkv_decode()
    say(f"[grouped auto] T={L.T} {L.n_in}->{L.n_out} R={L.R}")
    from lora_serving_amd import mlora
    D = DevLayer(L)
    assert mlora.mlora_linear_path(L.T, L.n_in, L.n_out, D.slots, L.K) == mlora.MLORA_PATH_GROUPED
    D.linear()
    # the group kernels, which the per-pair decode path never launches (they run on a second
    # stream beside the decode GEMM)
    names = _mlora_kernels_launched(lambda: D.linear())
    assert {"tile_plan_kernel", "sgmv_shrink_kernel", "sc_expand_kernel"} <= names, sorted(names)
    y = from_dev_bf16(D.linear())
    toks = np.unique(np.r_[np.arange(0, L.T, 3), L.T - 1]).astype(np.int64)
    y_ref = oracle_mod.linear(L, tokens=toks)
    assert tol_ok(y[toks], y_ref).all(), f"worst {worst(y[toks], y_ref):.3e}"
    # the decode batch of the headline workload keeps the per-pair path
    Dd = DevLayer(synth.workload_decode())
    Dd.linear()
    names_d = _mlora_kernels_launched(lambda: Dd.linear())
    assert names_d == {"decode_gemm_kernel", "decode_finish_kernel"}, sorted(names_d)


def test_tiled_scattered_tiles_beyond_capacity(oracle_mod):
    """Wide n_out keeps the fp32 sums of only one scattered tile: the first takes the per-adapter
    shrink/expand route, the other two the extra-k-step route; both against the oracle."""
    from lora_serving_amd import mlora
    L = synth.random_layer(48, T=768, n_in=64, n_out=70000, S=8, R=16, K=2, p_sentinel=0.2,
                           contiguous=False)
    say(f"[tiled-cap] T={L.T} n_in={L.n_in} n_out={L.n_out} K={L.K}")
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_TILED))
    toks = np.arange(0, L.T, 11, dtype=np.int64)
    y_ref = oracle_mod.linear(L, tokens=toks)
    ok = tol_ok(y[toks], y_ref)
    assert ok.all(), f"worst {worst(y[toks], y_ref):.3e}, {np.sum(~ok)} out"


def test_scattered_shrink_in_gemm_helpers_same_bits(oracle_mod):
    """The scattered tiles' shrink group items run in helper workgroups of the GEMM launch when
    its output tiles leave CUs idle, else in the shrink kernel.  The same layer at n_out = 32768
    (256 output tiles: no helper) and cut to its first 32512 outputs (254 tiles: helpers) gives
    the same bits on the shared outputs, and the cut one matches the oracle."""
    import dataclasses
    import torch
    from lora_serving_amd import mlora
    L = synth.random_layer(47, T=300, n_in=256, n_out=32768, S=40, R=16, K=2, p_sentinel=0.2)
    n_cut = 32512
    Lc = dataclasses.replace(L, n_out=n_cut, W=np.ascontiguousarray(L.W[:n_cut]),
                             B=np.ascontiguousarray(L.B[:, :n_cut]),
                             slice_start=np.array([0, n_cut], np.int32))
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"[helpers] T={L.T} n_out {L.n_out} vs {n_cut}, {n_cus} CUs")
    if n_cus != 256:
        pytest.skip("tile counts chosen for 256 CUs")
    y_full = from_dev_bf16(DevLayer(L).linear(flags=mlora.MLORA_PATH_TILED))
    y_cut = from_dev_bf16(DevLayer(Lc).linear(flags=mlora.MLORA_PATH_TILED))
    assert np.array_equal(y_cut, y_full[:, :n_cut])
    toks = np.arange(0, L.T, 7, dtype=np.int64)
    y_ref = oracle_mod.linear(Lc, tokens=toks)
    assert tol_ok(y_cut[toks], y_ref).all()


def test_slot_load_rebuilds_padded_slots():
    """Slot activation: every adapter loaded at its true rank (host pinned sources and device
    sources) over slots filled with NaN bits gives back the zero-padded slots bit for bit, and
    the layer's output is unchanged; one adapter has the full slot width (no padding)."""
    import torch
    from lora_serving_amd import mlora
    ranks = [8, 32, 16, 24, 5]
    L = synth.random_layer(49, T=40, n_in=384, n_out=200, S=5, R=32, K=2,
                           slice_sizes=[120, 80], ranks=ranks, p_sentinel=0.2)
    say(f"[slot-load] S={L.S} R={L.R} ranks={ranks}")
    D = DevLayer(L)
    y0 = D.linear().clone()
    A0, B0, f0 = D.A.clone(), D.B.clone(), D.factor.clone()
    D.A.view(torch.int16).fill_(0x7FC0)        # bf16 NaN everywhere
    D.B.view(torch.int16).fill_(0x7FC0)
    D.factor.fill_(float("nan"))
    keep = []                                   # sources stay alive until the copies are done
    for a, r in enumerate(ranks):
        A_src = np.ascontiguousarray(L.A[a, :, :r, :]).view(np.int16)
        B_src = np.ascontiguousarray(L.B[a, :, :r]).view(np.int16)
        if a % 2 == 0:                          # pinned host sources
            As = torch.from_numpy(A_src).pin_memory()
            Bs = torch.from_numpy(B_src).pin_memory()
        else:                                   # device sources
            As = torch.from_numpy(A_src).cuda()
            Bs = torch.from_numpy(B_src).cuda()
        keep.append((As, Bs))
        mlora.mlora_slot_load(D.slots, L.n_in, a, As, Bs, r, float(f0[a].item()))
    torch.cuda.synchronize()
    del keep
    assert torch.equal(D.A.view(torch.int16), A0.view(torch.int16))
    assert torch.equal(D.B.view(torch.int16), B0.view(torch.int16))
    assert torch.equal(D.factor, f0)
    y1 = D.linear()
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))


RANKED = [
    # seed, T, contiguous, path, ranks
    (50, 300, False, "decode", [8, 16, 64, 24, 8, 40, 16, 5, 64]),
    (51, 300, False, "tiled", [8, 16, 64, 24, 8, 40, 16, 5, 64]),   # the scattered route
    (52, 600, True, "tiled", [8, 16, 64, 24, 8, 40, 16, 5, 64]),    # prefill-like runs
    (53, 600, True, "tiled", [8, 16, 8, 24, 8, 5, 16, 5, 12]),      # narrower V blocks
    (54, 90, False, "decode", [8, 16, 8, 24, 8, 5, 16, 5, 12]),
]


@pytest.mark.parametrize("case", RANKED, ids=[f"r{c[0]}-{c[3]}" for c in RANKED])
def test_rank_table_skips_padding_exactly(oracle_mod, case):
    """With the slots' true ranks the kernels skip the zero padding.  The decode kernels skip
    products that are exact zeros without changing the order of the sums that remain, so the
    output is bit-identical to the rank-blind run.  The tiled path also sizes each tile's V block
    (and the GEMM's extra k-steps) by the largest rank in the tile, which regroups the remaining
    products among the MFMAs: there the output is checked within the tolerance of the oracle,
    as is the rank-blind run."""
    import torch
    from lora_serving_amd import mlora
    seed, T, contiguous, path, ranks = case
    L = synth.random_layer(seed, T=T, n_in=512, n_out=384, S=9, R=64, K=2,
                           slice_sizes=[256, 64, 64], ranks=ranks, p_sentinel=0.2,
                           contiguous=contiguous)
    say(f"[ranked] seed={seed} T={T} contiguous={contiguous} path={path}")
    flags = mlora.MLORA_PATH_DECODE if path == "decode" else mlora.MLORA_PATH_TILED
    D = DevLayer(L)
    y0 = D.linear(flags=flags).clone()
    rank_dev = torch.tensor(ranks, dtype=torch.int32, device="cuda")
    D.slots = mlora.Slots(D.A, D.B, D.factor, slice_start=[int(v) for v in L.slice_start],
                          rank=rank_dev)
    y1 = D.linear(flags=flags)
    y_ref = oracle_mod.linear(L)
    if path == "decode":
        assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))
    else:
        assert tol_ok(from_dev_bf16(y0), y_ref).all()
    yy = from_dev_bf16(y1)
    assert tol_ok(yy, y_ref).all(), f"worst {worst(yy, y_ref):.3e}"


DENSE_RANKED = [
    # seed, n_in, R, K, ranks: every 256-token tile dense (2 D R <= n_in / 2), ranks below R
    (58, 2048, 64, 2, [8, 16, 24, 8, 5, 16, 5, 12, 8]),   # n_in in parts: partials + reduce
    (59, 448, 16, 1, [8, 5, 8]),                          # n_in whole: the items write V
]


@pytest.mark.parametrize("seed,n_in,R,K,ranks", DENSE_RANKED,
                         ids=[f"d{c[0]}" for c in DENSE_RANKED])
def test_rank_table_dense_tiles(oracle_mod, seed, n_in, R, K, ranks):
    """Dense tiles with the rank table: A_cat stacks only the first VW rows of each slice of each
    adapter (VW from the tile's largest rank, here below R), on both routes of the dense shrink
    (n_in split in parts with a reduce after, or whole); against the oracle, as is the
    rank-blind run."""
    import torch
    from lora_serving_amd import mlora
    L = synth.random_layer(seed, T=768, n_in=n_in, n_out=384, S=len(ranks), R=R, K=K,
                           slice_sizes=[256, 64, 64], ranks=ranks, p_sentinel=0.2,
                           contiguous=True)
    for m in range(L.T // 256):                 # the case really takes the dense route
        ids = L.idx[m * 256:(m + 1) * 256]
        assert 2 * len(np.unique(ids[ids >= 0])) * R <= n_in // 2
    say(f"[dense ranked] seed={seed} n_in={n_in} R={R} K={K} ranks={ranks}")
    D = DevLayer(L)
    y_ref = oracle_mod.linear(L)
    y0 = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_TILED))
    assert tol_ok(y0, y_ref).all(), f"rank-blind: worst {worst(y0, y_ref):.3e}"
    rank_dev = torch.tensor(ranks, dtype=torch.int32, device="cuda")
    D.slots = mlora.Slots(D.A, D.B, D.factor, slice_start=[int(v) for v in L.slice_start],
                          rank=rank_dev)
    y1 = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_TILED))
    assert tol_ok(y1, y_ref).all(), f"worst {worst(y1, y_ref):.3e}"


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_decode_more_splits_than_loads_in_flight(oracle_mod, path):
    """n_in = 9224 gives the decode GEMM 10 splits of n_in (the last one ragged), more than the
    finish keeps in flight at once (8): splits 8 and 9 are added in a second round, for the
    partials and the shrink pieces alike.  Decode path with LoRA, the grouped decode (its
    finish keeps only the base), and the base alone."""
    from lora_serving_amd import mlora
    L = synth.random_layer(81, T=40, n_in=9224, n_out=136, S=6, R=16, K=2,
                           slice_sizes=[72, 64], p_sentinel=0.25)
    say(f"[splits] path={path} T={L.T} n_in={L.n_in} n_out={L.n_out}")
    flags = mlora.MLORA_PATH_DECODE if path == "decode" else mlora.MLORA_PATH_GROUPED
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=flags))
    y_ref = oracle_mod.linear(L)
    assert tol_ok(y, y_ref).all(), f"worst {worst(y, y_ref):.3e}"
    if path == "decode":
        import dataclasses
        y0 = from_dev_bf16(D.linear(flags=flags | mlora.MLORA_NO_ADAPTERS))
        y0_ref = oracle_mod.linear(dataclasses.replace(L, idx=np.full_like(L.idx, -1)))
        assert tol_ok(y0, y0_ref).all(), f"base: worst {worst(y0, y0_ref):.3e}"


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_decode_persistent_grid_three_chunks(oracle_mod, path):
    """150 tokens in one decode launch (chunks of 64, 64 and 22), 4096 rows (64 row tiles) over
    n_in = 1024 in 4 splits: 768 (chunk, tile, split) items on a persistent grid of 240
    workgroups (each XCD holding all three chunks of 10 (split, tile-lane) pairs), each walking
    3 or 4 row tiles.  Decode path with LoRA and the grouped decode (base only in the GEMM)
    against the oracle."""
    from lora_serving_amd import mlora
    L = synth.random_layer(83, T=150, n_in=1024, n_out=4096, S=8, R=16, K=2, p_sentinel=0.2)
    say(f"[persistent] path={path} T={L.T} n_in={L.n_in} n_out={L.n_out}")
    flags = mlora.MLORA_PATH_DECODE if path == "decode" else mlora.MLORA_PATH_GROUPED
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=flags))
    y_ref = oracle_mod.linear(L)
    assert tol_ok(y, y_ref).all(), f"worst {worst(y, y_ref):.3e}"
    if path == "decode":
        # the base alone on the same grid (no shrink pieces)
        import dataclasses
        y0 = from_dev_bf16(D.linear(flags=flags | mlora.MLORA_NO_ADAPTERS))
        y0_ref = oracle_mod.linear(dataclasses.replace(L, idx=np.full_like(L.idx, -1)))
        assert tol_ok(y0, y0_ref).all(), f"base: worst {worst(y0, y0_ref):.3e}"


def test_narrow_slots_at_the_limits(oracle_mod):
    """Slot width 32 with the most slots per token (8) and slices (4): the decode finish's v
    block (8 tokens x 4 slices x 32 entries, one quad a thread) and its slot loop, and the
    standalone expand's v staging of slots 4..7 (the second row of each wave).  Decode path
    and the standalone pair against the oracle."""
    L = synth.random_layer(82, T=37, n_in=512, n_out=520, S=9, R=32, K=8,
                           slice_sizes=[136, 128, 128, 128], p_sentinel=0.3)
    say(f"[narrow limits] T={L.T} R={L.R} K={L.K} slices={L.n_slices}")
    from lora_serving_amd import mlora
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_DECODE))
    y_ref = oracle_mod.linear(L)
    assert tol_ok(y, y_ref).all(), f"worst {worst(y, y_ref):.3e}"
    check_delta(oracle_mod, L, D=D, label="narrow limits")


@pytest.mark.parametrize("seed,T,K", [(55, 64, 1), (56, 37, 3)])
def test_rank_table_standalone_pair(oracle_mod, seed, T, K):
    """mlora_shrink / mlora_expand with the slots' true ranks: the rows of A and the columns of B
    past each adapter's rank are not read; v and the delta are bit-identical to the rank-blind
    calls and within the tolerance of the oracle's delta."""
    import torch
    from lora_serving_amd import mlora
    ranks = [8, 16, 64, 24, 8, 40, 16, 5, 12]
    L = synth.random_layer(seed, T=T, n_in=512, n_out=384, S=9, R=64, K=K,
                           slice_sizes=[256, 64, 64], ranks=ranks, p_sentinel=0.2)
    say(f"[ranked pair] seed={seed} T={T} K={K}")
    D = DevLayer(L)
    v0 = D.shrink().clone()
    d0 = D.delta().clone()
    rank_dev = torch.tensor(ranks, dtype=torch.int32, device="cuda")
    D.slots = mlora.Slots(D.A, D.B, D.factor, slice_start=[int(v) for v in L.slice_start],
                          rank=rank_dev)
    v1 = D.shrink()
    d1 = D.delta()
    assert torch.equal(v1, v0)
    assert torch.equal(d1.view(torch.int16), d0.view(torch.int16))
    y_ref = oracle_mod.linear(L, with_base=False)
    dd = from_dev_bf16(d1)
    assert tol_ok(dd, y_ref).all(), f"worst {worst(dd, y_ref):.3e}"


def pack_reference(Wbits, n_out, n_in):
    """The packed layout written out directly: Wp[rg][kb][l][e] = W[16 rg + l % 16]
    [32 kb + 8 (l // 16) + e], zero padded."""
    n_rg, n_kb = -(-n_out // 16), -(-n_in // 32)
    Wpad = np.zeros((n_rg * 16, n_kb * 32), np.uint16)
    Wpad[:n_out, :n_in] = Wbits
    out = np.zeros((n_rg, n_kb, 64, 8), np.uint16)
    for l in range(64):
        out[:, :, l, :] = Wpad.reshape(n_rg, 16, n_kb, 32)[:, l % 16, :, 8 * (l // 16):
                                                             8 * (l // 16) + 8]
    return out.reshape(-1)


PACKED = [
    # seed, T, n_in, n_out, K, path
    (60, 64, 4096, 4096, 1, "decode"),
    (61, 37, 392, 520, 3, "decode"),
    (62, 300, 392, 520, 3, "tiled"),
    (63, 520, 1032, 1000, 1, "tiled"),
]


@pytest.mark.parametrize("case", PACKED, ids=[f"w{c[0]}-{c[5]}" for c in PACKED])
def test_packed_weight_same_bits(oracle_mod, case):
    """mlora_pack_weight writes the documented layout, and mlora_linear on the packed weight
    gives the same output bits as on the row-major one (decode and tiled kernels)."""
    import torch
    from lora_serving_amd import mlora
    seed, T, n_in, n_out, K, path = case
    L = synth.random_layer(seed, T=T, n_in=n_in, n_out=n_out, S=6, R=16, K=K, p_sentinel=0.2,
                           contiguous=(path == "tiled"))
    say(f"[packed] seed={seed} T={T} n_in={n_in} n_out={n_out} path={path}")
    D = DevLayer(L)
    Wp = mlora.mlora_pack_weight(D.W)
    torch.cuda.synchronize()
    got = Wp.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, pack_reference(L.W, n_out, n_in))
    flags = mlora.MLORA_PATH_DECODE if path == "decode" else mlora.MLORA_PATH_TILED
    y0 = D.linear(flags=flags).clone()
    y1 = torch.empty_like(y0)
    mlora.mlora_linear(D.x, Wp, D.slots, D.idx, D.scale, y1, flags=flags | mlora.MLORA_W_PACKED,
                       ws=D.ws)
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))


@pytest.mark.parametrize("T", [9, 40])
def test_decode_wide_output(oracle_mod, T):
    """A vocabulary-wide decode product: n_out = 65600 (1025 row tiles of 64) with n_in = 2056
    split in 3 (the last split 8 columns wide); two slices of rank 32 and K = 3 make every
    pair need shrink pieces beyond the first.  Row-major and packed W against the oracle, and
    bit-identical to each other."""
    import torch
    from lora_serving_amd import mlora
    L = synth.random_layer(64 + T, T=T, n_in=2056, n_out=65600, S=6, R=32, K=3,
                           slice_sizes=[40000, 25600], p_sentinel=0.2)
    say(f"[wide-decode] T={T} n_in={L.n_in} n_out={L.n_out} K={L.K}")
    D = DevLayer(L)
    y0 = D.linear(flags=mlora.MLORA_PATH_DECODE).clone()
    toks = (np.arange(L.T, dtype=np.int64) if L.T <= 12
            else np.array(sorted({0, L.T - 1, *range(1, L.T - 1, 4)}), np.int64))
    y_ref = oracle_mod.linear(L, tokens=toks)
    yy = from_dev_bf16(y0)[toks]
    ok = tol_ok(yy, y_ref)
    assert ok.all(), f"worst {worst(yy, y_ref):.3e}, {np.sum(~ok)} out"
    Wp = mlora.mlora_pack_weight(D.W)
    y1 = torch.empty_like(y0)
    mlora.mlora_linear(D.x, Wp, D.slots, D.idx, D.scale, y1,
                       flags=mlora.MLORA_PATH_DECODE | mlora.MLORA_W_PACKED, ws=D.ws)
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))


@pytest.mark.parametrize("path", ["decode", "tiled", "grouped"])
def test_limits_rank_slots_slices(oracle_mod, path):
    """The widest slots (R = 512), the most slots per token (K = 8) and the most slices (4)."""
    from lora_serving_amd import mlora
    L = synth.random_layer(70, T=70 if path == "decode" else 300, n_in=512, n_out=640, S=5,
                           R=512, K=8, slice_sizes=[160, 160, 160, 160], p_sentinel=0.3,
                           contiguous=(path == "tiled"))
    say(f"[limits] path={path} T={L.T} R={L.R} K={L.K} slices={L.n_slices}")
    flags = {"decode": mlora.MLORA_PATH_DECODE, "tiled": mlora.MLORA_PATH_TILED,
             "grouped": mlora.MLORA_PATH_GROUPED}[path]
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=flags))
    y_ref = oracle_mod.linear(L)
    assert tol_ok(y, y_ref).all(), f"worst {worst(y, y_ref):.3e}"


@pytest.mark.parametrize("path", ["decode", "tiled", "grouped"])
def test_limits_most_slots(oracle_mod, path):
    """The most resident slots (S = 16384) with K = 8 slots a token: the tile plan then holds a
    16384-bit adapter map, 16384 counts and ranks and a 2048-entry list in LDS (140 KB of its
    160).  Slot ids are drawn over the whole range; the layer, and the delta of the standalone
    shrink/expand pair, are checked against the oracle."""
    from lora_serving_amd import mlora
    S = 16384
    L = synth.random_layer(73, T=64 if path == "decode" else 300, n_in=64, n_out=96, S=S, R=8,
                           K=8, p_sentinel=0.2, contiguous=(path == "tiled"))
    assert L.idx.max() > S - 2000   # ids near the top of the range occur
    say(f"[most slots] path={path} T={L.T} S={S} K={L.K}")
    flags = {"decode": mlora.MLORA_PATH_DECODE, "tiled": mlora.MLORA_PATH_TILED,
             "grouped": mlora.MLORA_PATH_GROUPED}[path]
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=flags))
    y_ref = oracle_mod.linear(L)
    assert tol_ok(y, y_ref).all(), f"worst {worst(y, y_ref):.3e}"
    if path == "decode":
        check_delta(oracle_mod, L, D, label="most slots")


@pytest.mark.parametrize("path", ["decode", "tiled"])
def test_tensor_parallel_shares(oracle_mod, path):
    """One GPU's share of a layer split 8 ways (merged QKV slices): the library on each column
    shard (its rows of W and B) and each row shard (its columns of W, A and x) against the
    oracle of that shard; the row shards' bf16 outputs, added in fp32, against the oracle's
    whole layer within the sum of their tolerances (the base model's all-reduce would add
    them)."""
    from lora_serving_amd import mlora
    G = 8
    L = synth.random_layer(74, T=64 if path == "decode" else 300, n_in=1024, n_out=1536, S=9,
                           R=16, K=2, p_sentinel=0.2, slice_sizes=[1024, 256, 256],
                           contiguous=(path == "tiled"))
    flags = mlora.MLORA_PATH_DECODE if path == "decode" else mlora.MLORA_PATH_TILED
    say(f"[tp shares] path={path} T={L.T} G={G}")
    total = np.zeros((L.T, L.n_out), np.float64)
    bound = np.zeros((L.T, L.n_out), np.float64)
    for g in range(G):
        for kind in ("col", "row"):
            Ls = synth.shard_layer(L, G, g, kind)
            y = from_dev_bf16(DevLayer(Ls).linear(flags=flags))
            y_ref = oracle_mod.linear(Ls)
            assert tol_ok(y, y_ref).all(), f"{kind} {g}: worst {worst(y, y_ref):.3e}"
            if kind == "row":
                total += y.astype(np.float64)
                bound += 2e-2 * (1 + np.abs(y_ref))
    y_full = oracle_mod.linear(L)
    assert np.all(np.abs(total - y_full) <= bound)


def test_tiled_path_chunks_past_a_million_tokens(oracle_mod):
    """More tokens than one tiled launch takes (4096 tiles of 256): the batch is cut in chunks;
    tokens on both sides of the cut and the ragged end are checked against the oracle."""
    from lora_serving_amd import mlora
    T = 4096 * 256 + 300
    L = synth.random_layer(71, T=T, n_in=64, n_out=64, S=4, R=8, K=1, p_sentinel=0.25,
                           contiguous=True)
    say(f"[million] T={T}")
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_TILED))
    cut = 4096 * 256
    toks = np.array([0, 1, 255, 256, cut - 257, cut - 1, cut, cut + 1, cut + 255, cut + 256,
                     T - 2, T - 1] + list(range(1000, T, 65537)), np.int64)
    toks = np.unique(toks)
    y_ref = oracle_mod.linear(L, tokens=toks)
    assert tol_ok(y[toks], y_ref).all(), f"worst {worst(y[toks], y_ref):.3e}"


@pytest.mark.parametrize("n_tiles,extra", [(1816, 0), (1820, 0), (1820, 77)])
def test_tiled_many_tiles_shrink_stages(oracle_mod, n_tiles, extra):
    """The dense shrink items keep three 48 KB stages in LDS while those, the tiles' item tables
    (9 bytes per tile) and the kernel's own __shared__ arrays fit in 160 KB, else two:
    1816 tiles is the last count with three (8 bytes to spare), 1820 tiles (and 1821, with a
    ragged last tile) take two.  Over three 64-column stages of n_in; tokens of the first,
    middle and last tiles and the ragged end are checked against the oracle."""
    from lora_serving_amd import mlora
    T = n_tiles * 256 + extra
    L = synth.random_layer(72 + n_tiles + extra, T=T, n_in=192, n_out=96, S=6, R=16, K=2,
                           p_sentinel=0.25, contiguous=True)
    say(f"[shrink stages] T={T} tiles={-(-T // 256)} n_in={L.n_in}")
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_TILED))
    toks = np.unique(np.array([0, 1, 255, 256, 511, T // 2, T // 2 + 1, T - 257, T - 256,
                               T - 78, T - 77, T - 2, T - 1] + list(range(333, T, 9973)),
                              np.int64))
    y_ref = oracle_mod.linear(L, tokens=toks)
    assert tol_ok(y[toks], y_ref).all(), f"worst {worst(y[toks], y_ref):.3e}"


DENSE_SPLITS = [
    # n_tiles, extra tokens, n_in, R: parts of n_in (ks) the dense shrink takes
    (2, 0, 1024, 16),     # ks 4 (n_in / 256)
    (3, 0, 256, 8),       # ks 1: V written by the items themselves
    (100, 0, 512, 16),    # ks 2 (256 items over 100 row blocks, at most n_in / 256)
    (100, 77, 256, 8),    # ks 1, ragged last tile
    (180, 0, 512, 16),    # ks 2
]


@pytest.mark.parametrize("n_tiles,extra,n_in,R", DENSE_SPLITS,
                         ids=[f"{c[0]}x{c[2]}r{c[3]}+{c[1]}" for c in DENSE_SPLITS])
def test_tiled_dense_shrink_splits(oracle_mod, n_tiles, extra, n_in, R):
    """The dense shrink splits n_in into ks parts (about 256 items over the tiles' 128-row
    blocks, at most n_in / 256 parts) and adds the parts' fp32 blocks in order in the reduce;
    with ks = 1 the items write V themselves.  Every tile here has one row block (at most 6
    adapters of width 8 or 16), so the tile count and n_in pick ks.  Tokens at the 64-token
    boundaries of the first, second, middle and last tiles are checked against the oracle, on
    the layer and on the LoRA delta alone (the same layer with W = 0)."""
    from lora_serving_amd import mlora
    T = n_tiles * 256 + extra
    L = synth.random_layer(1300 + n_tiles + n_in + extra, T=T, n_in=n_in, n_out=96, S=6, R=R,
                           K=1, p_sentinel=0.25, contiguous=True)
    say(f"[dense split] T={T} tiles={-(-T // 256)} n_in={n_in} R={R}")
    D = DevLayer(L)
    y = from_dev_bf16(D.linear(flags=mlora.MLORA_PATH_TILED))
    offs = np.array([0, 1, 63, 64, 65, 127, 128, 191, 192, 254, 255], np.int64)
    tiles = np.array([0, 1, n_tiles // 2, -(-T // 256) - 1], np.int64)
    toks = np.unique(np.clip((tiles[:, None] * 256 + offs[None, :]).ravel(), 0, T - 1))
    y_ref = oracle_mod.linear(L, tokens=toks)
    assert tol_ok(y[toks], y_ref).all(), f"worst {worst(y[toks], y_ref):.3e}"
    # the same layer with W = 0: the tiled kernels' LoRA delta alone, which a large W x could hide
    L0 = dataclasses.replace(L, W=np.zeros_like(L.W))
    d = from_dev_bf16(DevLayer(L0).linear(flags=mlora.MLORA_PATH_TILED))
    d_ref = oracle_mod.linear(L, tokens=toks, with_base=False)
    assert tol_ok(d[toks], d_ref).all(), f"delta worst {worst(d[toks], d_ref):.3e}"
    assert np.any(d_ref != 0)


def test_tiled_sentinel_rows_and_k3_invariance():
    from lora_serving_amd import mlora
    L1 = synth.random_layer(46, T=300, n_in=256, n_out=512, S=6, R=16, K=1, p_sentinel=0.3)
    L1.idx[::4] = -1
    D1 = DevLayer(L1)
    y1 = from_dev_bf16(D1.linear(flags=mlora.MLORA_PATH_TILED))
    y0 = from_dev_bf16(D1.linear(flags=mlora.MLORA_PATH_TILED | mlora.MLORA_NO_ADAPTERS))
    rows = np.where(L1.idx[:, 0] == -1)[0]
    assert np.array_equal(y1[rows], y0[rows])
    L3 = synth.random_layer(46, T=300, n_in=256, n_out=512, S=6, R=16, K=1, p_sentinel=0.3)
    L3.idx[::4] = -1
    idx = np.full((L1.T, 3), -1, np.int32)
    idx[:, 2] = L3.idx[:, 0]
    sc = np.ones((L1.T, 3), np.float32)
    sc[:, 2] = L3.scale[:, 0]
    L3.idx, L3.scale, L3.K = idx, sc, 3
    y3 = from_dev_bf16(DevLayer(L3).linear(flags=mlora.MLORA_PATH_TILED))
    assert np.array_equal(y3, y1)


def test_shrink_matches_oracle(oracle_mod):
    L = synth.random_layer(21, T=33, n_in=1024, n_out=96, S=6, R=16, K=3,
                           slice_sizes=[32, 32, 32], p_sentinel=0.3)
    D = DevLayer(L)
    v = D.shrink().cpu().numpy().astype(np.float64)
    v_ref = oracle_mod.shrink(L)
    scale = np.abs(v_ref).max()
    assert np.all(np.abs(v - v_ref) <= 1e-4 * (scale + np.abs(v_ref)))
    # pairs holding -1 are exactly zero
    for t in range(L.T):
        for j in range(L.K):
            if L.idx[t, j] == -1:
                assert np.all(v[j, t] == 0)


@pytest.mark.parametrize("T,K", [(1100, 1), (800, 1), (400, 1), (150, 2), (100, 1), (1, 3)])
def test_shrink_every_row_block(oracle_mod, T, K):
    """The standalone shrink takes the most rows of v per workgroup (16, 8, 4, 2, 1) that still
    give 2048 workgroups; with 24 rows per pair (3 slices of rank 8) these pair counts reach
    each choice in turn, 16 rows with a ragged last block.  n_in = 2056 leaves one 8-element
    chunk past the lanes' first two passes."""
    L = synth.random_layer(71 + T, T=T, n_in=2056, n_out=48, S=5, R=8, K=K,
                           slice_sizes=[16, 16, 16], p_sentinel=0.2)
    say(f"[shrink-rb] T={T} K={K}")
    v = DevLayer(L).shrink().cpu().numpy().astype(np.float64)
    v_ref = oracle_mod.shrink(L)
    scale = np.abs(v_ref).max()
    assert np.all(np.abs(v - v_ref) <= 1e-4 * (scale + np.abs(v_ref)))
    for j in range(L.K):
        assert np.all(v[j][L.idx[:, j] == -1] == 0)


@pytest.mark.parametrize("T,n_out,K", [(300, 4100, 2), (40, 1030, 3), (1, 4096, 1)])
def test_expand_both_row_blocks(oracle_mod, T, n_out, K):
    """The standalone expand covers 1024 output rows per workgroup when that gives at least
    1024 workgroups (T = 300 here, with a 4-row last block), else 256 (the others; 1030 rows
    is not a multiple of 4, so the last rows go one at a time).  Slots without an adapter sit
    before and between used ones, so the first slot to store is not always slot 0."""
    L = synth.random_layer(90 + T, T=T, n_in=512, n_out=n_out, S=6, R=16, K=K,
                           p_sentinel=0.35)
    check_delta(oracle_mod, L, label=f"expand T={T} n_out={n_out} K={K}")
    # accumulate mode: rows whose slots are all empty keep y's bits
    import torch
    from lora_serving_amd import mlora
    D = DevLayer(L)
    v = D.shrink()
    y0 = torch.randn((L.T, L.n_out), device=D.device).to(torch.bfloat16)
    y = y0.clone()
    mlora.mlora_expand(v, D.slots, D.idx, y)
    empty = torch.as_tensor(np.where((L.idx == -1).all(axis=1))[0], device=D.device)
    assert torch.equal(y[empty].view(torch.int16), y0[empty].view(torch.int16))


def test_tiny_workload(oracle_mod):
    L = synth.workload_tiny()
    D, _ = check_linear(oracle_mod, L, label="tiny")
    check_delta(oracle_mod, L, D, label="tiny")


def test_decode_workload_full(oracle_mod):
    L = synth.workload_decode()
    D, _ = check_linear(oracle_mod, L, label="decode")
    check_delta(oracle_mod, L, D, label="decode")


def _sample_tokens(L, n=1024, seed=0):
    """At least n tokens (all of them when T <= n): the first and last token of every
    segment, plus seeded random ones.  Tokens are independent, so each is checked exactly."""
    rng = np.random.default_rng(seed)
    if L.T <= n:
        return np.arange(L.T, dtype=np.int64)
    edges = set()
    for first, length in L.segments:
        edges.add(first)
        edges.add(first + length - 1)
    extra = rng.choice(L.T, size=n, replace=False)
    toks = sorted(edges | set(int(e) for e in extra) | {0, L.T - 1})
    return np.array(toks, np.int64)


@pytest.mark.parametrize("which", ["prefill", "mixed_qkv", "compose", "lm_head"])
def test_large_workloads_sampled(oracle_mod, which):
    layers = synth.WORKLOADS[which]()
    if not isinstance(layers, list):
        layers = [layers]
    for L in layers:
        toks = _sample_tokens(L)
        check_linear(oracle_mod, L, tokens=toks, label=f"{which}:{L.name}")


@pytest.mark.parametrize("which", ["decode", "decode256", "lm_head", "mixed_qkv",
                                   "mixed_qkv_prefill_first", "mixed_qkv_decode", "prefill",
                                   "compose"])
def test_workloads_in_bench_configuration(oracle_mod, which):
    """Each bench workload called the way bench.py calls it: the slots carry the true-rank
    table, decode-sized batches (T <= 512) take the packed base weight.  Whole output for the
    decode batches, sampled tokens (segment edges and random ones) for the large ones."""
    import torch
    from lora_serving_amd import mlora
    layers = synth.WORKLOADS[which]()
    if not isinstance(layers, list):
        layers = [layers]
    packed = all(L.T <= 512 for L in layers)
    for L in layers:
        say(f"[bench-config] {which}:{L.name} T={L.T} n_in={L.n_in} n_out={L.n_out} "
            f"packed={packed}")
        D = DevLayer(L)
        slots = mlora.Slots(D.A, D.B, D.factor, slice_start=[int(v) for v in L.slice_start],
                            rank=D.rank)
        W = mlora.mlora_pack_weight(D.W) if packed else D.W
        y = torch.empty((L.T, L.n_out), dtype=torch.bfloat16, device="cuda")
        mlora.mlora_linear(D.x, W, slots, D.idx, D.scale, y,
                           flags=mlora.MLORA_W_PACKED if packed else 0, ws=D.ws)
        yy = from_dev_bf16(y)
        toks = None if L.T <= 512 and L.n_out <= 8192 else _sample_tokens(L)
        y_ref = oracle_mod.linear(L, tokens=toks)
        if toks is not None:
            yy = yy[toks]
        ok = tol_ok(yy, y_ref)
        assert ok.all(), f"{which}: worst {worst(yy, y_ref):.3e}, {np.sum(~ok)} elements out"
        del D, slots, W, y


# ------------------------------------------------------------------------------------------
# invariants
# ------------------------------------------------------------------------------------------
def test_sentinel_rows_equal_base_only_run():
    L = synth.random_layer(31, T=90, n_in=512, n_out=384, S=5, R=16, K=2, p_sentinel=0.3)
    L.idx[::3] = -1
    D = DevLayer(L)
    y = D.linear()
    y0 = D.linear(flags=1)
    rows = np.where(np.all(L.idx == -1, axis=1))[0]
    assert len(rows) > 0
    a = from_dev_bf16(y)[rows]
    b = from_dev_bf16(y0)[rows]
    assert np.array_equal(a, b)


def test_all_sentinel_batch_equals_no_adapters_flag():
    L = synth.random_layer(32, T=64, n_in=256, n_out=256, S=3, R=8, K=1)
    L.idx[:] = -1
    D = DevLayer(L)
    assert np.array_equal(from_dev_bf16(D.linear()), from_dev_bf16(D.linear(flags=1)))


def test_k3_with_sentinels_equals_k1():
    L1 = synth.random_layer(33, T=70, n_in=512, n_out=320, S=6, R=16, K=1, p_sentinel=0.2)
    y1 = from_dev_bf16(DevLayer(L1).linear())
    for pos in range(3):
        L3 = synth.random_layer(33, T=70, n_in=512, n_out=320, S=6, R=16, K=1, p_sentinel=0.2)
        idx = np.full((L1.T, 3), -1, np.int32)
        idx[:, pos] = L1.idx[:, 0]
        sc = np.ones((L1.T, 3), np.float32)
        sc[:, pos] = L1.scale[:, 0]
        L3.idx, L3.scale, L3.K = idx, sc, 3
        assert np.array_equal(from_dev_bf16(DevLayer(L3).linear()), y1), pos


def test_run_to_run_bits_identical():
    import torch
    L = synth.workload_decode(seed=77)
    D = DevLayer(L)
    a = D.linear().view(torch.int16).cpu().numpy()
    b = D.linear().view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b)


def test_t_zero_is_noop():
    import torch
    from lora_serving_amd import mlora
    L = synth.random_layer(34, T=4, n_in=64, n_out=32, S=2, R=8, K=1)
    D = DevLayer(L)
    y = torch.full((0, 32), 1.0, dtype=torch.bfloat16, device="cuda")
    mlora.mlora_linear(D.x[:0], D.W, D.slots, D.idx[:0], None, y, ws=D.ws)


# ------------------------------------------------------------------------------------------
# plan
# ------------------------------------------------------------------------------------------
# maps up to 8192 pairs over up to 1000 slots take the one-workgroup sort, larger ones the
# three-kernel sort: cases 9-11 and 13 sit on both sides of both limits
PLAN_CASES = [(0, 1, 1, 1), (1, 6, 1, 4), (2, 64, 1, 100), (3, 1000, 3, 7), (4, 16384, 1, 100),
              (5, 8192, 3, 32), (6, 3000, 2, 16384), (7, 0, 1, 5), (8, 5000, 8, 1),
              (9, 8192, 1, 1000), (10, 8193, 1, 1000), (11, 4096, 1, 1001), (12, 1500, 2, 50),
              (13, 1170, 7, 3), (14, 32768, 1, 1000),
              # the one-wave sort (up to 512 pairs): its last size, one past it, 7 slots per
              # token, a single key, the most keys, and one key too many for it
              (15, 512, 1, 1000), (16, 513, 1, 1000), (17, 73, 7, 40), (18, 512, 1, 1),
              (19, 300, 1, 1001)]


@pytest.mark.parametrize("case", PLAN_CASES, ids=[f"p{c[0]}" for c in PLAN_CASES])
def test_plan_bit_exact(oracle_mod, case):
    import torch
    from lora_serving_amd import mlora
    seed, T, K, S = case
    say(f"[plan] seed={seed} T={T} K={K} S={S}")
    rng = np.random.default_rng(seed)
    if seed == 1:
        idx = np.array([2, 0, -1, 2, 3, 0], np.int32)[:, None]
    elif seed == 4:
        idx = synth.workload_prefill().idx
    else:
        idx = rng.integers(-1, S, size=(T, K)).astype(np.int32)
    perm_r, ss_r, st_r, sl_r = oracle_mod.plan(idx, S)
    dev = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    perm, ss, st, sl, cnt = dev(T * K), dev(S), dev(S), dev(S), dev(2)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    ws = torch.empty(max(1, T * K * S // 256 + 4 * S + 4096) * 4, dtype=torch.uint8, device="cuda")
    mlora.mlora_plan(idx_d, S, perm, ss, st, sl, cnt, ws)
    cnt = cnt.cpu().numpy()
    g, n = int(cnt[0]), int(cnt[1])
    assert n == len(perm_r) and g == len(ss_r)
    assert np.array_equal(perm.cpu().numpy()[:n], perm_r)
    assert np.array_equal(ss.cpu().numpy()[:g], ss_r)
    assert np.array_equal(st.cpu().numpy()[:g], st_r)
    assert np.array_equal(sl.cpu().numpy()[:g], sl_r)


def test_validate_rejects_bad_index_and_rank():
    import torch
    from lora_serving_amd import mlora
    L = synth.random_layer(35, T=10, n_in=64, n_out=32, S=4, R=16, K=2)
    D = DevLayer(L)
    code, _ = mlora.mlora_validate(D.idx, D.slots, rank=L.rank)
    assert code == mlora.MLORA_OK
    bad = D.idx.clone()
    bad[3, 1] = 4
    code, val = mlora.mlora_validate(bad, D.slots)
    assert code == mlora.MLORA_ERR_INDEX and val == 4
    rk = L.rank.copy()
    rk[2] = 32
    code, val = mlora.mlora_validate(D.idx, D.slots, rank=rk)
    assert code == mlora.MLORA_ERR_RANK and val == 32
    del torch


def _mlora_kernels_launched(fn):
    """Names of the library's kernels that fn() launches, from torch's profiler (kernel
    activity of the device, whoever launched it)."""
    import torch
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    names = set()
    for e in prof.events():
        n = e.name
        if "mlora::" in n:
            names.add(n.split("mlora::", 1)[1].split("<", 1)[0].split("(", 1)[0])
    return names


@pytest.mark.parametrize("T,n_in,n_out,slices", [(64, 4096, 6144, [4096, 1024, 1024]),
                                                  (64, 4096, 5120, None),
                                                  (256, 11008, 1024, None)])
def test_decode_persistent_grid_between_rounds(oracle_mod, T, n_in, n_out, slices):
    """The decode GEMM's persistent grid where one workgroup per item would need between one
    and two rounds of the CUs (one chunk: 384 and 320 items), and for several chunks whose split
    count (11 for n_in = 11008) does not divide an XCD's 64 (split, lane) slots (the slots past
    the last whole lane stay idle).  The kernel that ran is read from the launches; sampled
    tokens of every chunk are checked against the oracle."""
    from lora_serving_amd import mlora
    L = synth.random_layer(91 + T + n_in + n_out, T=T, n_in=n_in, n_out=n_out, S=20, R=16, K=1,
                           p_sentinel=0.1, slice_sizes=slices)
    D = DevLayer(L)
    pf = mlora.MLORA_PATH_DECODE
    D.linear(flags=pf)
    names = _mlora_kernels_launched(lambda: D.linear(flags=pf))
    say(f"[persistent] T={T} n_in={n_in} n_out={n_out}: {sorted(names)}")
    assert "decode_gemm_ps_kernel" in names
    y = from_dev_bf16(D.linear(flags=pf))
    toks = np.unique(np.clip(np.r_[np.arange(0, T, 13), 63, 64, T - 1], 0, T - 1))
    y_ref = oracle_mod.linear(L, tokens=toks)
    assert tol_ok(y[toks], y_ref).all(), f"worst {worst(y[toks], y_ref):.3e}"


@pytest.mark.parametrize("T,n_out,R,K,slices,apart", DECODE_ROUTE_CASES)
def test_decode_shrink_route(oracle_mod, T, n_out, R, K, slices, apart):
    """Where a 64-row tile of the decode GEMM would get 2 or more (token, slot) pairs of a
    64-token chunk and 4 or more 16-row shrink pieces of them (8 with several chunks), which
    its workgroups would chain one after another, the shrink runs apart, as the per-pair kernel
    ahead of a GEMM of the base alone; otherwise it rides in the GEMM pass.  The route is
    checked from the kernels launched, the output against the oracle."""
    from lora_serving_amd import mlora
    L = synth.random_layer(78 + T + n_out + R + K, T=T, n_in=256, n_out=n_out, S=12, R=R, K=K,
                           p_sentinel=0.1, slice_sizes=slices)
    D = DevLayer(L)
    pf = mlora.MLORA_PATH_DECODE
    D.linear(flags=pf)
    names = _mlora_kernels_launched(lambda: D.linear(flags=pf))
    say(f"[shrink route] T={T} n_out={n_out} R={R} K={K}: {sorted(names)}")
    assert ("shrink_rows_kernel" in names) == apart
    assert any(n.startswith("decode_gemm") for n in names)
    assert any(n.startswith("decode_finish") for n in names)
    toks = np.unique(np.r_[np.arange(0, T, 7), T - 1])
    y = from_dev_bf16(D.linear(flags=pf))
    assert tol_ok(y[toks], oracle_mod.linear(L, tokens=toks)).all()


@pytest.mark.parametrize("path", ["decode", "tiled"])
def test_no_adapters_flag_launches_base_kernels_only(path):
    """With MLORA_NO_ADAPTERS no LoRA kernel is launched ("Multi-LoRA Serving Explained": the
    LoRA kernels are skipped when no token uses an adapter): the decode path runs its GEMM and
    the split-K finish only, the tiled path its GEMM only.  Without the flag the same call
    launches the shrink / plan kernels as well (so the profiler does see them)."""
    from lora_serving_amd import mlora
    L = synth.random_layer(77, T=300, n_in=512, n_out=768, S=6, R=16, K=2, p_sentinel=0.2,
                           contiguous=(path == "tiled"))
    D = DevLayer(L)
    pf = mlora.MLORA_PATH_DECODE if path == "decode" else mlora.MLORA_PATH_TILED
    D.linear(flags=pf)
    with_lora = _mlora_kernels_launched(lambda: D.linear(flags=pf))
    base_only = _mlora_kernels_launched(lambda: D.linear(flags=pf | mlora.MLORA_NO_ADAPTERS))
    say(f"[no-adapters] {path}: with adapters {sorted(with_lora)}, flag {sorted(base_only)}")
    if path == "decode":
        assert base_only == {"decode_gemm_kernel", "decode_finish_kernel"}
        # 12 row tiles for 128 pairs a chunk: the shrink runs apart, ahead of the GEMM
        assert with_lora == base_only | {"shrink_rows_kernel"}
    else:
        assert base_only == {"prefill_gemm_kernel"}
        assert {"tile_plan_kernel", "sgmv_shrink_kernel"} <= with_lora
