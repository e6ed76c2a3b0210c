"""MI355X-native Mixture-of-Experts feed-forward layer (GPT-OSS / GLM4-MoE style).

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI of
``libmoe_ffn.so`` (declared in ``include/moe_ffn.h``).  ``moe_ffn`` is the thin
ctypes binding; ``workloads`` and ``inputs`` describe the seeded synthetic
workloads.  Importing the package loads nothing native.
"""
