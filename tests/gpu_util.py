"""Acceptance bound of the parity tests, and the device helpers they share with the benchmark."""
from __future__ import annotations

import numpy as np

from lora_serving_amd.device import DevLayer, from_dev_bf16, to_dev_bf16  # noqa: F401


def tol_ok(y, y_ref, rel=2e-2):
    """|y - y_ref| <= rel * (1 + |y_ref|) elementwise (the layer's acceptance bound)."""
    return np.abs(y - y_ref) <= rel * (1.0 + np.abs(y_ref))


def worst(y, y_ref):
    return float(np.max(np.abs(y - y_ref) / (1.0 + np.abs(y_ref)))) if y.size else 0.0
