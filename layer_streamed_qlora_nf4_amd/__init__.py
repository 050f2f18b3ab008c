"""Layer-streamed LoRA fine-tuning over an NF4 (or bf16) frozen base on MI355X.

The compute path is the C-ABI library ``liblsq.so`` (hand-written gfx950 HIP
kernels plus the native store / pool / step runtime), declared in
``include/lsq.h``.  ``lib`` is its thin ctypes binding: argument marshalling
only.  PyTorch supplies device memory and streams.

Importing the package loads nothing native; ``lib.load()`` does, and raises if
the library has not been built.
"""
from .configs import ModelCfg  # noqa: F401

__all__ = ["ModelCfg"]
