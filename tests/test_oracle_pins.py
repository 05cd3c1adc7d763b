"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU needed).

Each check pins the oracle to something other than itself: values the pages print for their
worked examples (tests/golden/*.json, each naming its source), the merged-weight identity
computed by a different route (tests/closed_forms.py), textbook routines, exact special cases
and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest

from lora_serving_amd import synth
from lora_serving_amd.synth import bf16_bits, make_layer
from tests import closed_forms as cf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def single_layer(x, W, A_slots, B_slots, idx, alpha, rank, R, scale=None, rslora=None):
    """Layer object from explicit float arrays (rounded to bf16)."""
    idx = np.asarray(idx, np.int32).reshape(len(x), -1)
    S = A_slots.shape[0]
    return synth.Layer(
        name="explicit", T=x.shape[0], n_in=x.shape[1], n_out=W.shape[0], S=S, R=R,
        K=idx.shape[1], n_slices=1, slice_start=np.array([0, W.shape[0]], np.int32),
        x=bf16_bits(x), W=bf16_bits(W), A=bf16_bits(A_slots.reshape(S, 1, R, -1)),
        B=bf16_bits(B_slots), idx=idx,
        scale=(np.ones(idx.shape, np.float32) if scale is None
               else np.asarray(scale, np.float32).reshape(idx.shape)),
        alpha=np.asarray(alpha, np.float64).reshape(S), rank=np.asarray(rank, np.int32).reshape(S),
        rslora=(np.zeros(S, np.uint8) if rslora is None else np.asarray(rslora, np.uint8)),
        seed=-1)


# ------------------------------------------------------------------------------------------
# Scale factor (rsLoRA)
# ------------------------------------------------------------------------------------------
def test_factor_values_from_page(oracle_mod):
    for case in golden("rslora.json")["cases"]:
        got = oracle_mod.lora_factor(case["alpha"], case["r"], case["rslora"])
        assert got == case["factor"], case


def test_rslora_delta_is_exactly_four_times(oracle_mod):
    """r=16, alpha=32: alpha/sqrt(r) = 8 is 4x alpha/r = 2, and scaling by 4 is exact."""
    L = synth.random_layer(11, T=7, n_in=96, n_out=80, S=3, R=16, K=2, ranks=16, alpha=32.0,
                           rslora=0, p_sentinel=0.2)
    d_plain = oracle_mod.linear(L, with_base=False)
    L.rslora = np.ones(L.S, np.uint8)
    d_rs = oracle_mod.linear(L, with_base=False)
    assert np.any(d_plain != 0)
    assert np.array_equal(d_rs, 4.0 * d_plain)


# ------------------------------------------------------------------------------------------
# The pages' worked examples
# ------------------------------------------------------------------------------------------
def test_merge_identity_within_page_residual(oracle_mod):
    """The page's merge example (512 x 512 layer, one rank-8 adapter, alpha 16): running the
    adapter beside the base weight gives the merged-weight result, the page printing a float64
    residual of about 4.3e-14.  The inputs here are this repository's own seeded draws at those
    sizes; the oracle (fp64) must agree with the merged-weight route to the same order."""
    g = golden("merge_identity.json")
    e = g["example"]
    rng = np.random.default_rng(3001)
    x, W, A, B = synth.draw_weights(rng, 1, e["d_in"], e["d_out"], 1, e["r"], 1,
                                    np.array([e["r"]]))
    assert e["r"] * (e["d_in"] + e["d_out"]) == g["printed"]["adapter_numbers"]
    assert e["d_in"] * e["d_out"] == g["printed"]["base_numbers"]
    L = make_layer("merge", 3001, rng, np.zeros((1, 1), np.int32), n_in=e["d_in"],
                   n_out=e["d_out"], S=1, R=e["r"], ranks=e["r"], alpha=e["alpha"])
    L.x, L.W, L.A, L.B = x, W, A, B
    y = oracle_mod.linear(L)[0]
    merged, mag = cf.merged_linear(L)
    diff = np.abs(y - merged[0]).max()
    assert diff <= 50 * g["printed"]["max_difference_about"], diff
    assert np.allclose(y, merged[0]) == g["printed"]["same_result"]
    # the adapter's delta is not negligible next to that residual
    assert np.abs(y - cf.f64(L.W) @ cf.f64(L.x)[0]).max() > 1e6 * diff


def _six_token_layer():
    """The page's six-token batch: four slots of width 16 holding ranks 8, 16, 4, 16, token
    slot ids 2, 0, -1, 2, 3, 0, B A applied with no alpha/r factor (alpha = r gives factor 1).
    Inputs are this repository's own seeded draws at those sizes."""
    g = golden("six_token_batch.json")
    e = g["example"]
    ids = np.array(e["ids"], np.int32)
    ranks = np.array(e["slot_ranks"], np.int32)
    rng = np.random.default_rng(3002)
    L = make_layer("six_token", 3002, rng, ids[:, None], n_in=e["d"], n_out=e["d"],
                   S=e["n_slots"], R=e["max_rank"], ranks=ranks,
                   alpha=ranks.astype(np.float64))
    return g, L


def test_six_token_page_example(oracle_mod):
    g, L = _six_token_layer()
    ids = np.array(g["example"]["ids"])
    y = oracle_mod.linear(L)
    merged, _ = cf.merged_linear(L)
    assert np.allclose(y, merged) == g["printed"]["batched_matches_per_request"]
    assert np.abs(y - merged).max() <= 1e-12 * np.abs(merged).max()
    perm, seg_slot, seg_start, seg_len = oracle_mod.plan(ids[:, None], 4)
    counts = {str(int(a)): int(n) for a, n in zip(seg_slot, seg_len)}
    counts["-1"] = int(np.sum(ids == -1))
    assert counts == g["printed"]["segment_counts"]
    expected_with_sentinel = g["derived_by_hand"]["stable_order_with_sentinel"]
    assert list(perm) == [p for p in expected_with_sentinel if ids[p] != -1]
    assert list(seg_start) == [0, 2, 4]


def test_padding_page_example(oracle_mod):
    """The page's padding example (a rank-8 adapter in a width-64 slot, d = 128): the padded
    slot gives exactly the unpadded result, and holds 16384 numbers against 2048."""
    g = golden("padding.json")
    e = g["example"]
    d, r, R = e["d"], e["r"], e["R"]
    assert r * 2 * d == g["printed"]["numbers_rank_r"]
    assert R * 2 * d == g["printed"]["numbers_rank_R_slot"]
    rng = np.random.default_rng(3003)
    Lr = make_layer("pad_r", 3003, rng, np.zeros((1, 1), np.int32), n_in=d, n_out=d, S=1, R=r,
                    ranks=r, alpha=float(r))
    LR = make_layer("pad_R", 3003, rng, np.zeros((1, 1), np.int32), n_in=d, n_out=d, S=1, R=R,
                    ranks=r, alpha=float(r))
    A = np.zeros((1, 1, R, d), np.uint16); A[:, :, :r] = Lr.A
    B = np.zeros((1, d, R), np.uint16); B[:, :, :r] = Lr.B
    LR.x, LR.W, LR.A, LR.B = Lr.x, Lr.W, A, B
    assert int(np.count_nonzero(synth.bf16_to_f32(LR.A)[0, 0, r:])) == 0
    yr = oracle_mod.linear(Lr, with_base=False)
    yR = oracle_mod.linear(LR, with_base=False)
    assert np.any(yr != 0)
    assert np.array_equal(yr, yR) == g["printed"]["padded_equals_unpadded"]


def test_sizing_page_script(oracle_mod):
    g = golden("sizing.json")
    m, p = g["model"], g["printed"]
    GiB, MiB = 2 ** 30, 2 ** 20

    def adapter(rank, slots=1):
        return m["layers"] * sum(oracle_mod.slot_bytes(slots, rank, i, o, 1)
                                 for i, o in m["modules"].values())

    base = (m["layers"] * sum(i * o for i, o in m["modules"].values())
            + 2 * m["vocab"] * m["hidden"]) * m["bytes"]
    assert round(base / GiB, 2) == p["base_GiB_2dp"]
    for r, mib in p["adapter_MiB_0dp"].items():
        assert round(adapter(int(r)) / MiB) == mib
    assert round(100 * adapter(16) / GiB, 2) == p["hundred_rank16_GiB_2dp"]
    assert round(100 * base / GiB) == p["hundred_full_copies_GiB_0dp"]
    for slots, rank, gib in p["slots_GiB_2dp"]:
        assert round(adapter(rank, slots) / GiB, 2) == gib
    assert adapter(16, 8) / GiB == p["eight_rank16_slots_GiB"]
    # merged QKV as three slices equals q + k + v counted separately
    qkv = oracle_mod.slot_bytes(1, 16, 4096, 6144, 3)
    sep = sum(oracle_mod.slot_bytes(1, 16, i, o, 1) for i, o in
              (m["modules"]["q"], m["modules"]["k"], m["modules"]["v"]))
    assert qkv == sep


# ------------------------------------------------------------------------------------------
# Closed forms and exact special cases
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed,K,slices", [(1, 1, None), (2, 3, None), (3, 2, [40, 24, 16]),
                                           (4, 3, [17, 63])])
def test_merged_route_random(oracle_mod, seed, K, slices):
    """Oracle (shrink then expand, slot by slot) equals the merged-weight route in fp64:
    catches a transposed operand, a wrong slice, a wrong slot or a dropped scale."""
    L = synth.random_layer(seed, T=9, n_in=72, n_out=80, S=5, R=16, K=K, slice_sizes=slices,
                           p_sentinel=0.3)
    y = oracle_mod.linear(L)
    merged, mag = cf.merged_linear(L)
    assert np.all(np.abs(y - merged) <= 1e-12 * (mag + 1e-300))
    d = oracle_mod.linear(L, with_base=False)
    dm, dmag = cf.merged_linear(L, with_base=False)
    assert np.any(dm != 0)
    assert np.all(np.abs(d - dm) <= 1e-12 * (dmag + 1e-300))


def test_bruteforce_tiny_workload(oracle_mod):
    L = synth.workload_tiny()
    y = oracle_mod.linear(L)
    merged, mag = cf.merged_linear(L)
    assert np.all(np.abs(y - merged) <= 1e-12 * mag)


def test_sentinel_token_is_base_exactly(oracle_mod):
    L = synth.random_layer(5, T=12, n_in=64, n_out=48, S=3, R=8, K=2, p_sentinel=0.5)
    L.idx[3, :] = -1
    L.idx[7, :] = -1
    y = oracle_mod.linear(L)
    base = oracle_mod.linear(L, tokens=[3, 7], with_base=True)  # same rows, computed alone
    Lb = synth.random_layer(5, T=12, n_in=64, n_out=48, S=3, R=8, K=2)
    Lb.x, Lb.W = L.x, L.W
    Lb.idx = np.full_like(L.idx, -1)
    y_none = oracle_mod.linear(Lb)
    assert np.array_equal(y[[3, 7]], y_none[[3, 7]])
    assert np.array_equal(base, y[[3, 7]])
    ref = cf.f64(L.W) @ cf.f64(L.x)[[3, 7]].T
    assert np.allclose(y[[3, 7]], ref.T, rtol=0, atol=1e-12 * np.abs(ref).max())
    # and the delta of a sentinel token is exactly zero
    d = oracle_mod.linear(L, with_base=False)
    assert np.all(d[[3, 7]] == 0)


def test_additivity_over_slots(oracle_mod):
    """y(K slots) - Wx equals the sum of the single-slot deltas."""
    L = synth.random_layer(6, T=10, n_in=64, n_out=40, S=4, R=16, K=3, p_sentinel=0.2)
    total = oracle_mod.linear(L, with_base=False)
    parts = np.zeros_like(total)
    for j in range(L.K):
        Lj = synth.random_layer(6, T=10, n_in=64, n_out=40, S=4, R=16, K=3, p_sentinel=0.2)
        keep = np.full_like(L.idx, -1)
        keep[:, j] = L.idx[:, j]
        Lj.idx = keep
        parts += oracle_mod.linear(Lj, with_base=False)
    _, mag = cf.merged_linear(L, with_base=False)
    assert np.all(np.abs(total - parts) <= 1e-12 * (mag + 1e-300))


@pytest.mark.parametrize("G", [2, 4])
def test_tensor_parallel_shards(oracle_mod, G):
    """Tensor-parallel shards (the layer split over G GPUs; every term is linear in x and
    separate per output row): a column shard's outputs are the layer's rows of its part of
    every slice, bit for bit; the row shards' outputs add up to the layer's within fp64
    rounding, the LoRA terms included (each shard's shrink covers its columns of A and x).  A
    wrong slice offset fails the first, a shrink over the whole of x the second."""
    L = synth.random_layer(9, T=12, n_in=64, n_out=48, S=5, R=16, K=2, p_sentinel=0.2,
                           slice_sizes=[24, 12, 12])
    full = oracle_mod.linear(L)
    for g in range(G):
        Lc = synth.shard_layer(L, G, g, "col")
        rows = np.concatenate([np.arange(a + g * (b - a) // G, a + (g + 1) * (b - a) // G)
                               for a, b in zip(L.slice_start[:-1], L.slice_start[1:])])
        assert Lc.n_out == rows.size
        assert np.array_equal(oracle_mod.linear(Lc), full[:, rows])
    total = sum(oracle_mod.linear(synth.shard_layer(L, G, g, "row")) for g in range(G))
    _, mag = cf.merged_linear(L)
    assert np.all(np.abs(total - full) <= 1e-12 * (mag + 1e-300))
    # the row shards' deltas alone are each a proper part: none of them is the whole delta
    d_full = oracle_mod.linear(L, with_base=False)
    d0 = oracle_mod.linear(synth.shard_layer(L, G, 0, "row"), with_base=False)
    assert not np.allclose(d0, d_full)


def test_cat_merged_virtual_adapter(oracle_mod):
    """K-slot composition equals one adapter whose A stacks the K adapters' rows and whose B
    concatenates c_j B_j (the RFC's exact oracle).  Scales are powers of two so c_j B_j is
    exactly representable in bf16."""
    rng = np.random.default_rng(7)
    T, n_in, n_out, R = 6, 48, 40, 8
    ranks = np.array([8, 4, 8])
    alpha = np.array([16.0, 8.0, 8.0])           # f = 2, 2, 1
    scales = np.array([1.0, 0.5, 0.25], np.float32)
    x = rng.standard_normal((T, n_in))
    W = rng.standard_normal((n_out, n_in)) / math.sqrt(n_in)
    A = np.zeros((3, R, n_in)); B = np.zeros((3, n_out, R))
    for a in range(3):
        A[a, :ranks[a]] = rng.uniform(-0.1, 0.1, (ranks[a], n_in))
        B[a, :, :ranks[a]] = rng.standard_normal((n_out, ranks[a])) * 0.1
    idx = np.tile(np.array([0, 1, 2]), (T, 1))
    Lk = single_layer(x, W, A, B, idx, alpha=alpha, rank=ranks, R=R,
                      scale=np.tile(scales, (T, 1)))
    # virtual adapter: A_cat rows = [A_0[:r0]; A_1[:r1]; A_2[:r2]], B_cat = [c_0 B_0 | ...]
    Ab, Bb = cf.f64(Lk.A)[:, 0], cf.f64(Lk.B)
    rc = int(ranks.sum())
    A_cat = np.concatenate([Ab[a, :ranks[a]] for a in range(3)])
    c = scales.astype(np.float64) * (alpha / ranks)
    B_cat = np.concatenate([c[a] * Bb[a, :, :ranks[a]] for a in range(3)], axis=1)
    L1 = single_layer(x, W, A_cat[None], B_cat[None], np.zeros((T, 1), int),
                      alpha=[float(rc)], rank=[rc], R=rc)
    assert np.array_equal(synth.bf16_to_f32(L1.A)[0, 0], A_cat.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(L1.B)[0], B_cat.astype(np.float32))
    yk = oracle_mod.linear(Lk)
    y1 = oracle_mod.linear(L1)
    _, mag = cf.merged_linear(Lk)
    assert np.all(np.abs(yk - y1) <= 1e-12 * mag)


def test_padding_is_bitwise_invariant(oracle_mod):
    L = synth.random_layer(8, T=8, n_in=64, n_out=32, S=3, R=8, K=2, ranks=8, p_sentinel=0.1)
    y8 = oracle_mod.linear(L)
    Lp = synth.random_layer(8, T=8, n_in=64, n_out=32, S=3, R=8, K=2, ranks=8, p_sentinel=0.1)
    R2 = 32
    A = np.zeros((L.S, 1, R2, L.n_in), np.uint16); A[:, :, :8] = L.A
    B = np.zeros((L.S, L.n_out, R2), np.uint16); B[:, :, :8] = L.B
    Lp.A, Lp.B, Lp.R = A, B, R2
    assert np.array_equal(oracle_mod.linear(Lp), y8)


def test_k3_with_sentinels_equals_k1(oracle_mod):
    L1 = synth.random_layer(9, T=11, n_in=64, n_out=40, S=4, R=8, K=1, p_sentinel=0.2)
    y1 = oracle_mod.linear(L1)
    for pos in range(3):
        L3 = synth.random_layer(9, T=11, n_in=64, n_out=40, S=4, R=8, K=1, p_sentinel=0.2)
        idx = np.full((L1.T, 3), -1, np.int32)
        idx[:, pos] = L1.idx[:, 0]
        sc = np.ones((L1.T, 3), np.float32)
        sc[:, pos] = L1.scale[:, 0]
        L3.idx, L3.scale, L3.K = idx, sc, 3
        assert np.array_equal(oracle_mod.linear(L3), y1)


def test_duplicate_slot_in_one_token_is_summed(oracle_mod):
    L = synth.random_layer(10, T=4, n_in=48, n_out=32, S=2, R=8, K=2, p_sentinel=0.0)
    L.idx[:] = 1
    d2 = oracle_mod.linear(L, with_base=False)
    dm, mag = cf.merged_linear(L, with_base=False)
    assert np.all(np.abs(d2 - dm) <= 1e-12 * mag)


def test_shrink_expand_pieces_compose_to_linear(oracle_mod):
    L = synth.random_layer(12, T=9, n_in=56, n_out=44, S=4, R=16, K=3, slice_sizes=[20, 24],
                           p_sentinel=0.3)
    v = oracle_mod.shrink(L)
    # rows of -1 pairs are zero; columns beyond each adapter's rank are zero
    for t in range(L.T):
        for j in range(L.K):
            a = L.idx[t, j]
            row = v[j, t].reshape(L.n_slices, L.R)
            if a == -1:
                assert np.all(row == 0)
            else:
                assert np.all(row[:, L.rank[a]:] == 0)
    d = oracle_mod.expand(L, v)
    dm, mag = cf.merged_linear(L, with_base=False)
    assert np.all(np.abs(d - dm) <= 1e-12 * (mag + 1e-300))
    # doubling every scale doubles v exactly
    L.scale = L.scale * np.float32(2)
    assert np.array_equal(oracle_mod.shrink(L), 2 * v)


# ------------------------------------------------------------------------------------------
# Mapping plan
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed,T,K,S", [(0, 1, 1, 1), (1, 37, 1, 5), (2, 100, 3, 7),
                                        (3, 0, 2, 3), (4, 64, 2, 100)])
def test_plan_is_the_stable_sort(oracle_mod, seed, T, K, S):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-1, S, size=(T, K)).astype(np.int32)
    perm, ss, st, sl = oracle_mod.plan(idx, S)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    order = order[flat[order] != -1]
    assert np.array_equal(perm, order)
    keys, counts = np.unique(flat[flat != -1], return_counts=True)
    assert np.array_equal(ss, keys)
    assert np.array_equal(sl, counts)
    assert np.array_equal(st, np.concatenate([[0], np.cumsum(counts)[:-1]]) if len(counts)
                          else np.zeros(0))


def test_plan_rejects_out_of_range(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.plan(np.array([[0], [3]], np.int32), 3)
    with pytest.raises(ValueError):
        oracle_mod.plan(np.array([[-2]], np.int32), 3)


# ------------------------------------------------------------------------------------------
# The fp32 build (timed as the CPU baseline) against the pinned fp64 build
# ------------------------------------------------------------------------------------------
def test_fp32_build_within_fp32_rounding_of_fp64(oracle_mod):
    """The same loops summed in fp32: each output within a few fp32 roundings per term of the
    fp64 result (bound: n terms x 2^-23 x the sum of the absolute products), and exactly the
    fp64 result where every product and partial sum is exact (all-zero deltas of sentinel
    tokens)."""
    L = synth.random_layer(13, T=10, n_in=256, n_out=64, S=4, R=16, K=2, p_sentinel=0.3)
    y64 = oracle_mod.linear(L)
    y32 = oracle_mod.linear(L, acc="f32")
    _, mag = cf.merged_linear(L)
    n_terms = L.n_in + L.K * L.R
    assert np.all(np.abs(y32 - y64) <= n_terms * 2.0 ** -23 * mag)
    assert np.any(y32 != y64)                  # it really sums in fp32
    d32 = oracle_mod.linear(L, with_base=False, acc="f32")
    rows = np.where(np.all(L.idx == -1, axis=1))[0]
    assert np.all(d32[rows] == 0)


def test_linear_rejects_tokens_out_of_range(oracle_mod):
    """A sampled-token request past the layer's tokens is an error, not a read past x."""
    L = synth.random_layer(11, T=8, n_in=16, n_out=8, S=2, R=8, K=1)
    with pytest.raises(IndexError):
        oracle_mod.linear(L, tokens=np.array([0, 8]))
    with pytest.raises(IndexError):
        oracle_mod.linear(L, tokens=np.array([-1]))
    assert oracle_mod.linear(L, tokens=np.array([7])).shape == (1, 8)
