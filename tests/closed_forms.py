"""Independent NumPy fp64 routes to the layer's output, used to pin the oracle.

None of this imports or mirrors the oracle's code: where the oracle computes the low-rank side
path token by token (shrink, then expand), these helpers first merge each token's adapters into
one effective weight, W_eff = W + sum_j c_j B_a A_a, and multiply once -- the identity
W x + B(A x) = (W + B A) x that "Multi-LoRA Serving Explained" (sevydevy.com, merge-equivalence
script) checks, extended to k slots by the vLLM RFC on per-request composition (Semantics).
"""
from __future__ import annotations

import math

import numpy as np

from lora_serving_amd.synth import bf16_to_f32


def f64(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def factor(alpha: float, r: int, rslora: bool) -> float:
    # [vLLM] LoRA, PEFTHelper section
    return alpha / math.sqrt(r) if rslora else alpha / r


def merged_linear(L, tokens=None, with_base: bool = True):
    """y rows via explicit per-token merged weights; also returns sum of |terms| per element."""
    x, W, A, B = f64(L.x), f64(L.W), f64(L.A), f64(L.B)
    toks = range(L.T) if tokens is None else tokens
    ys, mags = [], []
    for t in toks:
        W_eff = W.copy() if with_base else np.zeros_like(W)
        W_abs = np.abs(W) if with_base else np.zeros_like(W)
        for j in range(L.K):
            a = int(L.idx[t, j])
            if a == -1:
                continue
            c = float(L.scale[t, j]) * factor(float(L.alpha[a]), int(L.rank[a]),
                                              bool(L.rslora[a]))
            for sg in range(L.n_slices):
                r0, r1 = int(L.slice_start[sg]), int(L.slice_start[sg + 1])
                W_eff[r0:r1] += c * (B[a, r0:r1, :] @ A[a, sg])
                W_abs[r0:r1] += abs(c) * (np.abs(B[a, r0:r1, :]) @ np.abs(A[a, sg]))
        ys.append(W_eff @ x[t])
        mags.append(W_abs @ np.abs(x[t]))
    return np.array(ys), np.array(mags)
