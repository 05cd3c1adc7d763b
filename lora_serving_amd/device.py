"""Seeded layers (synth.Layer) moved to the GPU, and calls of the library through its C ABI on
them.  Used by the benchmark and the tests; holds no arithmetic of the layer."""
from __future__ import annotations

import numpy as np

from lora_serving_amd.synth import bf16_to_f32


def to_dev_bf16(bits: np.ndarray, device="cuda"):
    """bf16 bits (uint16 array) as a bfloat16 device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def from_dev_bf16(t) -> np.ndarray:
    """A bfloat16 device tensor as exact float64 values on the host."""
    import torch
    return bf16_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)).astype(
        np.float64)


class DevLayer:
    """Device copies of one Layer plus its Slots binding object and a workspace."""

    def __init__(self, L, device="cuda"):
        import torch
        from lora_serving_amd import mlora
        self.L = L
        self.x = to_dev_bf16(L.x, device)
        self.W = to_dev_bf16(L.W, device)
        self.A = to_dev_bf16(L.A, device)
        self.B = to_dev_bf16(L.B, device)
        self.idx = torch.from_numpy(np.ascontiguousarray(L.idx, np.int32)).to(device)
        self.scale = torch.from_numpy(np.ascontiguousarray(L.scale, np.float32)).to(device)
        f = np.array([mlora.mlora_factor(L.alpha[a], int(L.rank[a]), bool(L.rslora[a]))
                      for a in range(L.S)], np.float32)
        self.factor = torch.from_numpy(f).to(device)
        # the slots' true ranks (passed to the library only when a caller asks for them)
        self.rank = torch.from_numpy(np.ascontiguousarray(L.rank, np.int32)).to(device)
        self.slots = mlora.Slots(self.A, self.B, self.factor,
                                 slice_start=[int(v) for v in L.slice_start])
        self.ws = mlora.workspace(L.T, L.K, L.n_in, L.n_out, self.slots, device)
        self.device = device

    def linear(self, flags=0, use_scale=True, y=None):
        import torch
        from lora_serving_amd import mlora
        if y is None:
            y = torch.empty((self.L.T, self.L.n_out), dtype=torch.bfloat16, device=self.device)
        mlora.mlora_linear(self.x, self.W, self.slots, self.idx,
                           self.scale if use_scale else None, y, flags=flags, ws=self.ws)
        return y

    def shrink(self):
        import torch
        from lora_serving_amd import mlora
        v = torch.empty((self.L.K, self.L.T, self.L.n_slices * self.L.R), dtype=torch.float32,
                        device=self.device)
        mlora.mlora_shrink(self.x, self.slots, self.idx, self.scale, v, ws=self.ws)
        return v

    def delta(self):
        """shrink, then expand into a zero y: the LoRA delta alone, rounded to bf16."""
        import torch
        from lora_serving_amd import mlora
        v = self.shrink()
        y = torch.zeros((self.L.T, self.L.n_out), dtype=torch.bfloat16, device=self.device)
        mlora.mlora_expand(v, self.slots, self.idx, y)
        return y
