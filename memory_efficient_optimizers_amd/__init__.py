"""Fused optimizer steps of memory-efficient optimizers (Adafactor, CAME, LAMB) for
AMD MI355X, behind the C ABI declared in include/meo.h.

``memory_efficient_optimizers_amd._lib`` is the thin ctypes binding (one Python
function per C entry point); ``Adafactor``, ``CAME`` and ``Lamb`` are
torch.optim front ends that own the state tensors.
"""
from . import _lib  # noqa: F401
from ._lib import MeoError  # noqa: F401
from .optim import CAME, Adafactor, Lamb, moment_dtype  # noqa: F401

__all__ = ["Adafactor", "CAME", "Lamb", "MeoError", "moment_dtype"]
