"""Seeded synthetic inputs for the multi-LoRA adapted linear layer.

This module draws random numbers, rounds them to bfloat16 and lays them out.  It holds none
of the layer's arithmetic (no products, no scale factors, no sorting): the GPU library's
callers and the CPU oracle's callers both take their inputs from here and nothing else is
shared between the two sides.

Layouts (all row-major, contiguous):
  x      bf16 bits  uint16 [T][n_in]
  W      bf16 bits  uint16 [n_out][n_in]
  A      bf16 bits  uint16 [S][n_slices][R][n_in]   rows >= rank[a] are zero
  B      bf16 bits  uint16 [S][n_out][R]            cols >= rank[a] are zero
  idx    int32 [T][K]      slot of (token, position) or -1 (base model only)
  scale  float32 [T][K]    per-(token, position) user scale s (1 where not drawn)
  alpha  float64 [S], rank int32 [S], rslora uint8 [S]: adapter configuration

Adapters sit zero-padded in slots of width R, the way "Multi-LoRA Serving Explained"
(sevydevy.com, section "Why max-lora-rank costs memory even for small adapters") describes
vLLM's slot buffers.  The k-slot token mapping with sentinel -1 follows "[RFC]: Per-request
activation of multiple LoRA adapters with static scales" (vLLM issue 51940, Proposed Change,
staged implementation step 2).

Value distributions ("variance" notation): x ~ N(0, 1); W ~ N(0, 1/n_in); A ~ U(-1/sqrt(n_in),
+1/sqrt(n_in)); B ~ N(0, 0.02).  Draw order inside one layer: token assignments first (done
by the workload builder), then x, W, A, B, then scales.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SENTINEL = -1


# ----------------------------------------------------------------------------------------
# bfloat16 helpers (storage format only)
# ----------------------------------------------------------------------------------------
def bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bits."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    u = a32.view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact float32 value of bfloat16 bits."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------------
# One adapted layer's inputs
# ----------------------------------------------------------------------------------------
@dataclasses.dataclass
class Layer:
    name: str
    T: int
    n_in: int
    n_out: int
    S: int
    R: int
    K: int
    n_slices: int
    slice_start: np.ndarray      # int32 [n_slices+1]
    x: np.ndarray                # uint16 [T][n_in]
    W: np.ndarray                # uint16 [n_out][n_in]
    A: np.ndarray                # uint16 [S][n_slices][R][n_in]
    B: np.ndarray                # uint16 [S][n_out][R]
    idx: np.ndarray              # int32 [T][K]
    scale: np.ndarray            # float32 [T][K]
    alpha: np.ndarray            # float64 [S]
    rank: np.ndarray             # int32 [S]
    rslora: np.ndarray           # uint8 [S]
    seed: int
    segments: list = dataclasses.field(default_factory=list)  # [(first token, n tokens)] per request

    @property
    def has_scale(self) -> bool:
        return not bool(np.all(self.scale == 1.0))


def draw_weights(rng: np.random.Generator, T: int, n_in: int, n_out: int, S: int, R: int,
                 n_slices: int, ranks: np.ndarray):
    """Draw x, W, A, B (in that order) and zero each slot's padding beyond its rank."""
    x = rng.standard_normal((T, n_in), dtype=np.float32)
    W = rng.standard_normal((n_out, n_in), dtype=np.float32)
    W *= np.float32(1.0 / math.sqrt(n_in))
    bound = np.float32(1.0 / math.sqrt(n_in))
    A = rng.random((S, n_slices, R, n_in), dtype=np.float32)
    A *= np.float32(2.0) * bound
    A -= bound
    B = rng.standard_normal((S, n_out, R), dtype=np.float32)
    B *= np.float32(math.sqrt(0.02))
    for a in range(S):
        r = int(ranks[a])
        A[a, :, r:, :] = 0.0
        B[a, :, r:] = 0.0
    return bf16_bits(x), bf16_bits(W), bf16_bits(A), bf16_bits(B)


def make_layer(name: str, seed: int, rng: np.random.Generator, idx: np.ndarray, *, n_in: int,
               n_out: int, S: int, R: int, ranks, alpha, rslora=None, slice_sizes=None,
               scale: np.ndarray | None = None, segments=None) -> Layer:
    """Build a layer from an already drawn token mapping; draws x, W, A, B next."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    if idx.ndim == 1:
        idx = idx[:, None].copy()
    T, K = idx.shape
    if slice_sizes is None:
        slice_sizes = [n_out]
    n_slices = len(slice_sizes)
    slice_start = np.concatenate([[0], np.cumsum(slice_sizes)]).astype(np.int32)
    assert slice_start[-1] == n_out
    ranks = np.broadcast_to(np.asarray(ranks, dtype=np.int32), (S,)).copy()
    alpha = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (S,)).copy()
    if rslora is None:
        rslora = np.zeros(S, dtype=np.uint8)
    rslora = np.broadcast_to(np.asarray(rslora, dtype=np.uint8), (S,)).copy()
    x, W, A, B = draw_weights(rng, T, n_in, n_out, S, R, n_slices, ranks)
    if scale is None:
        scale = np.ones((T, K), dtype=np.float32)
    return Layer(name=name, T=T, n_in=n_in, n_out=n_out, S=S, R=R, K=K, n_slices=n_slices,
                 slice_start=slice_start, x=x, W=W, A=A, B=B, idx=idx,
                 scale=np.ascontiguousarray(scale, dtype=np.float32), alpha=alpha, rank=ranks,
                 rslora=rslora, seed=seed, segments=list(segments or []))


# ----------------------------------------------------------------------------------------
# The workloads
# ----------------------------------------------------------------------------------------
def finite_zipf_cdf(n: int, s: float) -> np.ndarray:
    """Cumulative distribution of P(a) proportional to (a+1)^-s over a = 0..n-1."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def workload_tiny(seed: int = 1000) -> Layer:
    """T=16, 256->256, 4 adapters of rank 8, alpha 16; P(-1)=0.25 else uniform over {0..3}."""
    rng = np.random.default_rng(seed)
    T, S = 16, 4
    use = rng.random(T) >= 0.25
    pick = rng.integers(0, S, size=T)
    idx = np.where(use, pick, SENTINEL).astype(np.int32)
    return make_layer("tiny", seed, rng, idx, n_in=256, n_out=256, S=S, R=8, ranks=8, alpha=16.0,
                      segments=[(t, 1) for t in range(T)])


def workload_decode(seed: int = 1001, T: int = 64, n_in: int = 4096, n_out: int = 4096,
                    S: int = 100, rank: int = 16, alpha: float = 32.0, n_sentinel: int | None = None
                    ) -> Layer:
    """BGMV decode: T one-token requests, adapter uniform over S, round(0.1 T) tokens -1."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, S, size=T).astype(np.int32)
    if n_sentinel is None:
        n_sentinel = int(round(0.1 * T))
    idx[rng.permutation(T)[:n_sentinel]] = SENTINEL
    return make_layer("decode", seed, rng, idx, n_in=n_in, n_out=n_out, S=S, R=rank, ranks=rank,
                      alpha=alpha, segments=[(t, 1) for t in range(T)])


def workload_prefill(seed: int = 1002, n_req: int = 32, seg_len: int = 512, n_in: int = 4096,
                     n_out: int = 11008, S: int = 100, rank: int = 64, alpha: float = 128.0,
                     zipf_s: float = 1.1) -> Layer:
    """SGMV prefill: n_req contiguous segments of seg_len tokens, adapter ~ finite Zipf(s)."""
    rng = np.random.default_rng(seed)
    cdf = finite_zipf_cdf(S, zipf_s)
    req_adapter = np.searchsorted(cdf, rng.random(n_req), side="right").astype(np.int32)
    req_adapter = np.minimum(req_adapter, S - 1)
    idx = np.repeat(req_adapter, seg_len).astype(np.int32)
    segs = [(r * seg_len, seg_len) for r in range(n_req)]
    return make_layer("prefill", seed, rng, idx, n_in=n_in, n_out=n_out, S=S, R=rank, ranks=rank,
                      alpha=alpha, segments=segs)


def workload_mixed_qkv(seed: int = 1003, n_decode: int = 256, prefill_len: int = 2048,
                       n_in: int = 4096, slice_sizes=(4096, 1024, 1024), S: int = 64, R: int = 64,
                       rank_choices=(8, 16, 64), prefill_first: bool = False) -> Layer:
    """Merged QKV: n_decode one-token requests plus one prefill segment; mixed ranks padded to R."""
    rng = np.random.default_rng(seed)
    ranks = rng.choice(np.asarray(rank_choices, dtype=np.int32), size=S)
    req_adapter = rng.integers(0, S, size=n_decode + 1).astype(np.int32)
    dec = req_adapter[:n_decode]
    pre = np.full(prefill_len, req_adapter[n_decode], dtype=np.int32)
    if prefill_first:
        idx = np.concatenate([pre, dec])
        segs = [(0, prefill_len)] + [(prefill_len + t, 1) for t in range(n_decode)]
    else:
        idx = np.concatenate([dec, pre])
        segs = [(t, 1) for t in range(n_decode)] + [(n_decode, prefill_len)]
    return make_layer("mixed_qkv", seed, rng, idx, n_in=n_in, n_out=int(sum(slice_sizes)), S=S,
                      R=R, ranks=ranks, alpha=2.0 * ranks.astype(np.float64),
                      slice_sizes=list(slice_sizes), segments=segs)


def compose_mapping(rng: np.random.Generator, n_req: int, req_len: int, S: int, K: int):
    """Per request: 1..K distinct adapters (count uniform), ids without replacement in draw
    order in positions 0.., remaining positions -1; per-(request, position) s ~ U(0.2, 1.0)."""
    counts = rng.integers(1, K + 1, size=n_req)
    req_idx = np.full((n_req, K), SENTINEL, dtype=np.int32)
    for q in range(n_req):
        req_idx[q, :counts[q]] = rng.choice(S, size=int(counts[q]), replace=False)
    req_scale = rng.uniform(0.2, 1.0, size=(n_req, K)).astype(np.float32)
    idx = np.repeat(req_idx, req_len, axis=0)
    scale = np.repeat(req_scale, req_len, axis=0)
    return idx, scale


def workload_compose(seed: int = 1004, n_req: int = 64, req_len: int = 128, S: int = 32,
                     rank: int = 16, alpha: float = 32.0, K: int = 3,
                     shapes=((4096, 4096), (11008, 4096))) -> list[Layer]:
    """k-slot composition: each request 1..K distinct adapters of S, scales s ~ U(0.2, 1.0);
    adapters S/2.. use rsLoRA.  One mapping, one layer per (n_in, n_out) in shapes."""
    rng = np.random.default_rng(seed)
    idx, scale = compose_mapping(rng, n_req, req_len, S, K)
    rslora = (np.arange(S) >= S // 2).astype(np.uint8)
    segs = [(q * req_len, req_len) for q in range(n_req)]
    layers = []
    for (n_in, n_out) in shapes:
        name = f"compose_{n_in}x{n_out}"
        layers.append(make_layer(name, seed, rng, idx, n_in=n_in, n_out=n_out, S=S, R=rank,
                                 ranks=rank, alpha=alpha, rslora=rslora, scale=scale,
                                 segments=segs))
    return layers


def workload_lm_head(seed: int = 1005) -> Layer:
    """LM-head LoRA at decode: the decode mapping (64 one-token requests, 100 adapters of rank
    16, 6 tokens base-only) on a vocabulary-wide output, 4096 -> 100,000 (not a multiple of the
    64-row tile, so the last tile is ragged)."""
    L = workload_decode(seed=seed, n_out=100_000)
    L.name = "lm_head"
    return L


def workload_decode256(seed: int = 1006) -> Layer:
    """A larger decode step: 256 one-token requests on the decode layer (4096 -> 4096, 100
    adapters of rank 16, 26 tokens base-only)."""
    L = workload_decode(seed=seed, T=256)
    L.name = "decode256"
    return L


def workload_mixed_qkv_prefill_first(seed: int = 1003) -> Layer:
    """The mixed merged-QKV batch with its 2048-token segment ahead of the 256 one-token
    requests (same draws otherwise): the result must not depend on the order of the parts."""
    L = workload_mixed_qkv(seed=seed, prefill_first=True)
    L.name = "mixed_qkv_prefill_first"
    return L


def workload_mixed_qkv_decode(seed: int = 1003) -> Layer:
    """The mixed merged-QKV batch's one-token requests alone (same draws): the decode part of
    that batch as a call of its own."""
    L = workload_mixed_qkv(seed=seed)
    nd = sum(1 for (_s, n) in L.segments if n == 1)
    return dataclasses.replace(L, name="mixed_qkv_decode", T=nd, x=L.x[:nd].copy(),
                               idx=L.idx[:nd].copy(), scale=L.scale[:nd].copy(),
                               segments=L.segments[:nd])


def shard_layer(L: Layer, G: int, g: int, kind: str) -> Layer:
    """Shard g of G of a layer under tensor parallelism (array slicing only).

    kind "col" (column-parallel: q/k/v/gate/up): each slice's output rows split G ways, shard g
    holding the g-th part of every slice (its rows of W and B); A and x are whole.
    kind "row" (row-parallel: o/down): the input columns split G ways, shard g holding columns
    g n_in / G .. of W, A and x, B whole; the shards' outputs add up to the layer's."""
    if kind == "col":
        rows, starts = [], [0]
        for sg in range(L.n_slices):
            a, b = int(L.slice_start[sg]), int(L.slice_start[sg + 1])
            if (b - a) % G:
                raise ValueError("slice sizes must divide by G")
            part = (b - a) // G
            rows.append(np.arange(a + g * part, a + (g + 1) * part))
            starts.append(starts[-1] + part)
        rows = np.concatenate(rows)
        return dataclasses.replace(L, name=f"{L.name}_col{g}of{G}", n_out=int(rows.size),
                                   slice_start=np.asarray(starts, np.int32),
                                   W=np.ascontiguousarray(L.W[rows]),
                                   B=np.ascontiguousarray(L.B[:, rows]))
    if kind == "row":
        if L.n_in % G:
            raise ValueError("n_in must divide by G")
        c = L.n_in // G
        cols = slice(g * c, (g + 1) * c)
        return dataclasses.replace(L, name=f"{L.name}_row{g}of{G}", n_in=c,
                                   x=np.ascontiguousarray(L.x[:, cols]),
                                   W=np.ascontiguousarray(L.W[:, cols]),
                                   A=np.ascontiguousarray(L.A[..., cols]))
    raise ValueError(kind)


def workload_decode_tp8_col(seed: int = 1001) -> Layer:
    """One GPU's share of the decode layer under 8-way column parallelism: 4096 -> 512 (its
    rows of W and B; A and x whole), the decode mapping."""
    return dataclasses.replace(shard_layer(workload_decode(seed=seed), 8, 0, "col"),
                               name="decode_tp8_col")


def workload_decode_tp8_row(seed: int = 1001) -> Layer:
    """One GPU's share of the decode layer under 8-way row parallelism: 512 -> 4096 (its
    columns of W, A and x; B whole); the GPUs' outputs add up to the layer's."""
    return dataclasses.replace(shard_layer(workload_decode(seed=seed), 8, 0, "row"),
                               name="decode_tp8_row")


WORKLOADS = {
    "tiny": workload_tiny,
    "decode256": workload_decode256,
    "lm_head": workload_lm_head,
    "decode": workload_decode,
    "prefill": workload_prefill,
    "mixed_qkv": workload_mixed_qkv,
    "mixed_qkv_prefill_first": workload_mixed_qkv_prefill_first,
    "mixed_qkv_decode": workload_mixed_qkv_decode,
    "compose": workload_compose,
    "decode_tp8_col": workload_decode_tp8_col,
    "decode_tp8_row": workload_decode_tp8_row,
}


def random_layer(seed: int, T: int, n_in: int, n_out: int, S: int, R: int, K: int,
                 p_sentinel: float = 0.25, slice_sizes=None, ranks=None, rslora=None,
                 with_scale: bool = True, alpha=None, contiguous: bool = False) -> Layer:
    """Small layer for parity tests: any K, sentinels at any position, duplicate slots allowed.
    With contiguous=True tokens come in runs that share their mapping (prefill-like)."""
    rng = np.random.default_rng(seed)
    if contiguous:
        n_runs = max(1, T // 37 + 1)
        cuts = np.sort(rng.choice(np.arange(1, max(T, 2)), size=min(n_runs - 1, max(T - 1, 0)),
                                  replace=False)) if T > 1 else np.array([], dtype=np.int64)
        bounds = np.concatenate([[0], cuts, [T]]).astype(np.int64)
        idx = np.empty((T, K), dtype=np.int32)
        for b0, b1 in zip(bounds[:-1], bounds[1:]):
            row = np.where(rng.random(K) < p_sentinel, SENTINEL, rng.integers(0, S, size=K))
            idx[b0:b1] = row
    else:
        idx = np.where(rng.random((T, K)) < p_sentinel, SENTINEL,
                       rng.integers(0, S, size=(T, K))).astype(np.int32)
    if ranks is None:
        ranks = rng.choice(np.array([r for r in (1, 4, 8, 16, 32, 64, 128) if r <= R] or [R]),
                           size=S)
        ranks[0] = R
    ranks = np.broadcast_to(np.asarray(ranks, dtype=np.int32), (S,)).copy()
    if alpha is None:
        alpha = 2.0 * ranks.astype(np.float64)
    if rslora is None:
        rslora = (rng.random(S) < 0.5).astype(np.uint8)
    scale = (rng.uniform(0.2, 1.0, size=(T, K)).astype(np.float32) if with_scale else None)
    return make_layer(f"random_{seed}", seed, rng, idx, n_in=n_in, n_out=n_out, S=S, R=R,
                      ranks=ranks, alpha=alpha, rslora=rslora, slice_sizes=slice_sizes,
                      scale=scale)
