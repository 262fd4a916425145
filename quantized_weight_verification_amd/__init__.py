"""Quantized speculative-verify kernels for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libqv.so`` built from ``csrc/`` (hand-written HIP);
``ops`` marshals torch device tensors into it.  Importing the package does not load the
library; the first call into ``ops`` does, and raises if it is missing.
"""

__all__ = ["ops", "synth"]
