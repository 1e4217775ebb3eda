"""MI355X-native forward pass of one mixture-of-experts FFN layer.

The compute path is a C-ABI library of hand-written HIP kernels for gfx950
(``csrc/``, declared in ``include/moe.h``); ``api`` is the thin Python binding
over it.  PyTorch supplies device memory and streams only.
"""
__all__ = ["api", "workloads", "accounting"]
