"""Acceptance bound of the parity tests, and the device helpers they share with the benchmark."""
from __future__ import annotations

import numpy as np

from lora_serving_amd.device import DevLayer, from_dev_bf16, to_dev_bf16  # noqa: F401


def tol_ok(y, y_ref, rel=2e-2):
    """|y - y_ref| <= rel * (1 + |y_ref|) elementwise (the layer's acceptance bound)."""
    return np.abs(y - y_ref) <= rel * (1.0 + np.abs(y_ref))


def worst(y, y_ref):
    return float(np.max(np.abs(y - y_ref) / (1.0 + np.abs(y_ref)))) if y.size else 0.0


# (T, n_out, R, K, slice sizes, whether the decode path's shrink runs apart from its GEMM):
# apart where a 64-row tile gets 2 or more (token, slot) pairs of a 64-token chunk and 4 or
# more 16-row pieces of them (8 when the launch has several chunks)
DECODE_ROUTE_CASES = [(64, 4096, 16, 1, None, False), (64, 2048, 16, 1, None, False),
                      (64, 1024, 16, 1, None, True), (64, 512, 16, 1, None, True),
                      (64, 4096, 64, 1, None, False), (64, 4096, 16, 3, None, False),
                      (64, 4096, 16, 4, None, True), (64, 1024, 32, 2, None, True),
                      (64, 1536, 16, 1, [1024, 256, 256], True), (16, 512, 16, 1, None, False),
                      (512, 1024, 16, 1, None, False), (256, 512, 16, 1, None, True),
                      (100, 6144, 16, 1, [4096, 1024, 1024], False), (70, 4096, 16, 2, None, False)]
