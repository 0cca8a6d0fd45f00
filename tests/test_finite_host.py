"""The non-finite check over per-tensor scalars, on a host-built workspace (CPU):
only the slots an optimizer writes are looked at, and tensors with zero elements
(offset -1) are never listed."""
import math

import pytest
import torch

from memory_efficient_optimizers_amd import _lib

SLOT = {name: i for i, name in enumerate(_lib.SCALAR_SLOTS)}


def workspace(n_tensors: int, bad: dict) -> torch.Tensor:
    """float32 slots, all finite (1.0) except bad[(tensor, slot name)] = value."""
    w = torch.ones(8 * n_tensors, dtype=torch.float32)
    for (k, name), v in bad.items():
        w[8 * k + SLOT[name]] = v
    return w.view(torch.uint8)


@pytest.mark.parametrize("opt", ["adafactor", "came", "lamb"])
def test_flags_exactly_the_named_slots(opt):
    named = _lib.FINITE_CHECK_SLOTS[opt]
    other = [s for s in _lib.SCALAR_SLOTS if s not in named]
    bad = {(1, named[0]): math.nan, (3, named[-1]): math.inf, (4, named[1]): -math.inf}
    bad.update({(0, other[0]): math.nan, (2, other[-1]): math.inf})  # unspecified slots: ignored
    ws = workspace(5, bad)
    assert _lib.nonfinite_tensors(opt, ws, [0, 8, 16, 24, 32]) == [1, 3, 4]
    # offsets as the library lays them out: -1 for a tensor with zero elements; the
    # result indexes the list (its tensors 2 and 3 hold the slots at 8 and 24)
    assert _lib.nonfinite_tensors(opt, ws, [0, -1, 8, 24]) == [2, 3]
    assert _lib.nonfinite_tensors(opt, workspace(3, {}), [0, 8, 16]) == []
    assert _lib.nonfinite_tensors(opt, ws, [-1, -1]) == []


def test_rms_u_and_lamb_norms_are_checked():
    """A non-finite gradient reaches RMS(U) (Adafactor, CAME) and LAMB's direction
    norm; LAMB's parameter norm catches a non-finite parameter."""
    assert "rms_u" in _lib.FINITE_CHECK_SLOTS["adafactor"]
    assert "rms_u" in _lib.FINITE_CHECK_SLOTS["came"]
    assert {"norm_d", "rms_x"} <= set(_lib.FINITE_CHECK_SLOTS["lamb"])
