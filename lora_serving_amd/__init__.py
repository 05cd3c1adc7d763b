"""MI355X-native multi-LoRA adapted linear layer.

The compute path lives in ``libmlora.so`` (hand-written gfx950 HIP kernels behind a C ABI, see
``include/mlora.h``); ``lora_serving_amd.mlora`` is its thin ctypes binding and
``lora_serving_amd.synth`` draws seeded synthetic inputs.  Importing the package loads nothing.
"""
__version__ = "0.1.0"
