"""Fused optimizer steps of memory-efficient optimizers (Adafactor, CAME, LAMB and
GaLore's low-rank projected AdamW) for AMD MI355X, behind the C ABI declared in
include/meo.h.

``memory_efficient_optimizers_amd._lib`` is the thin ctypes binding (one Python
function per C entry point); ``Adafactor``, ``CAME``, ``Lamb`` and ``GaLoreAdamW``
are torch.optim front ends that own the state tensors; ``get_galore_param_groups``
forms GaLore's parameter groups from a model.
"""
from . import _lib  # noqa: F401
from ._lib import MeoError  # noqa: F401
from .optim import CAME, Adafactor, GaLoreAdamW, Lamb, get_galore_param_groups, moment_dtype  # noqa: F401

__all__ = ["Adafactor", "CAME", "GaLoreAdamW", "Lamb", "MeoError", "get_galore_param_groups", "moment_dtype"]
