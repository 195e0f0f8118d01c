"""MI355X-native forward pass of one Mixture-of-Experts FFN layer.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, declared in ``include/moe.h``); ``binding`` marshals torch
tensors into it.  ``workloads`` and ``synth`` are plain data and seeded input
generation.  Importing the package loads nothing; ``binding`` loads the
library on first use and raises if it is missing.
"""
__all__ = ["binding", "workloads", "synth"]
