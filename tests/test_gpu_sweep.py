"""GPU parity over a seeded random sweep of layer shapes and slot sets.

Each case draws its sizes from its seed: batch T (1 to 700, across the 16/64-token groups and the
256-token tiles), n_in (multiples of 8 up to 3064), one to three output slices of any width,
slot width R (8 to 256), slots S (up to 2000), slots per token K (1 to 8), sentinel share, contiguous or
random maps, the slots' true-rank table or none, row-major or packed W, and the path (decode,
tiled, grouped decode, or the library's own choice).  mlora_linear is compared with the oracle
on every token (a seeded sample of tokens, with the first and last, for the largest products);
decode-path cases also compare the standalone shrink / expand pair's delta.  The acceptance
bound is the layer's: |y - y_ref| <= 2e-2 (1 + |y_ref|) elementwise.
"""
import sys

import numpy as np
import pytest

from lora_serving_amd import synth
from tests.gpu_util import DevLayer, from_dev_bf16, tol_ok, worst

pytestmark = pytest.mark.gpu

PATHS = ["decode", "tiled", "grouped", "auto"]
N_CASES = 96


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lora_serving_amd import mlora  # noqa: F401  (fails loudly if the library is missing)


def sweep_case(i):
    """The sizes of case i, drawn from its own seed."""
    rng = np.random.default_rng(7000 + i)
    path = PATHS[i % len(PATHS)]
    T = int(rng.choice([1, 2, 15, 16, 17, 31, 63, 64, 65, 100, 200, 257, 300, 511, 513, 700]))
    if path == "grouped":
        T = min(T, 512)
    n_in = 8 * int(rng.integers(1, 384))
    n_slices = int(rng.choice([1, 1, 2, 3]))
    sizes = [int(v) for v in rng.integers(1, 1200, size=n_slices)]
    R = int(rng.choice([8, 16, 32, 64, 128, 256]))
    S = int(rng.integers(1, 121)) if rng.random() < 0.8 else int(rng.integers(121, 2001))
    K = int(rng.choice([1, 1, 2, 3, 4, 8]))
    # at most about 1 GB of slots (the widest slot sets with many slots have tests of their own)
    slot_bytes = 2 * S * R * (n_slices * n_in + sum(sizes))
    if slot_bytes > 1_000_000_000:
        S = max(1, int(S * 1_000_000_000 / slot_bytes))
    p_sent = float(rng.uniform(0.0, 0.6))
    contiguous = bool(rng.random() < (0.7 if path == "tiled" else 0.3))
    use_rank = bool(rng.random() < 0.5)
    packed = bool(path in ("decode", "tiled") and rng.random() < 0.3)
    return dict(seed=7000 + i, path=path, T=T, n_in=n_in, sizes=sizes, R=R, S=S, K=K,
                p_sent=p_sent, contiguous=contiguous, use_rank=use_rank, packed=packed)


def _tokens(L, seed):
    """All tokens, or a seeded sample (with the first and last) when the product is large."""
    if L.T * L.n_in * L.n_out <= 2_000_000_000:
        return None
    rng = np.random.default_rng(seed)
    pick = rng.choice(L.T, size=min(L.T, 48), replace=False)
    return np.unique(np.r_[0, L.T - 1, pick]).astype(np.int64)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer_against_oracle(oracle_mod, i):
    import torch
    from lora_serving_amd import mlora
    c = sweep_case(i)
    print(f"[sweep {i}] {c}", flush=True)
    sys.stdout.flush()
    sizes = c["sizes"] if len(c["sizes"]) > 1 else None
    n_out = int(sum(c["sizes"]))
    L = synth.random_layer(c["seed"], T=c["T"], n_in=c["n_in"], n_out=n_out, S=c["S"], R=c["R"],
                           K=c["K"], p_sentinel=c["p_sent"], slice_sizes=sizes,
                           contiguous=c["contiguous"])
    D = DevLayer(L)
    if c["use_rank"]:
        D.slots = mlora.Slots(D.A, D.B, D.factor, slice_start=[int(v) for v in L.slice_start],
                              rank=D.rank)
    flags = {"decode": mlora.MLORA_PATH_DECODE, "tiled": mlora.MLORA_PATH_TILED,
             "grouped": mlora.MLORA_PATH_GROUPED, "auto": 0}[c["path"]]
    W = D.W
    if c["packed"]:
        W = mlora.mlora_pack_weight(D.W)
        flags |= mlora.MLORA_W_PACKED
    y = torch.empty((L.T, L.n_out), dtype=torch.bfloat16, device="cuda")
    mlora.mlora_linear(D.x, W, D.slots, D.idx, D.scale, y, flags=flags, ws=D.ws)
    toks = _tokens(L, c["seed"])
    y_ref = oracle_mod.linear(L, tokens=toks)
    yy = from_dev_bf16(y)
    yy = yy if toks is None else yy[toks]
    ok = tol_ok(yy, y_ref)
    assert ok.all(), f"case {i}: worst {worst(yy, y_ref):.3e}, {np.sum(~ok)} elements out"
    if c["path"] == "decode":
        # the standalone pair: the LoRA delta alone, into a zero y
        d = from_dev_bf16(D.delta())
        d_ref = oracle_mod.linear(L, tokens=toks, with_base=False)
        dd = d if toks is None else d[toks]
        okd = tol_ok(dd, d_ref)
        assert okd.all(), f"case {i}: delta worst {worst(dd, d_ref):.3e}"
