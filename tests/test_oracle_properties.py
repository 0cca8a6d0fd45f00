"""Invariants of the oracle over random shapes and values (CPU; hypothesis, derandomized
so that every run draws the same examples). The fixed pins in test_oracle_pins.py
check each on chosen inputs; here they must hold on whatever shape (1-D, 2-D with unit
sides, 3-D), gradient scale (over 6 decades) and setting is drawn.

* RMS clipping (the note after "Step 5" of the Colossal-AI distributed-optimizers
  page): the applied update U / kappa has RMS exactly clip_threshold when RMS(U)
  exceeds it, and is U itself otherwise.
* Scale invariance of Adafactor's and CAME's update: U = G / sqrt(V) does not change
  when G is scaled by a power of two, over chained steps with a first moment, as long
  as eps1 = 1e-30 is negligible against every G^2 (it is the only term that does not
  scale): gradients of about 1e-2 and up, scaled by 2^-10 .. 2^30. (Scaled further
  down, a gradient of 1e-4 times 2^-21 has G^2 = 2.5e-21, where eps1 moves the update
  by 4e-10 and the invariance is rightly lost.)
* LAMB's layer-wise trust ratio (DistributedLAMB paragraph): ||x_new - x|| = lr ||x||
  for a nonzero parameter and direction, at every step.
"""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

SHAPES = st.one_of(st.tuples(st.integers(1, 40)),
                   st.tuples(st.integers(1, 12), st.integers(1, 12)),
                   st.tuples(st.integers(1, 3), st.integers(1, 7), st.integers(1, 9)))
RUNS = settings(max_examples=300, derandomize=True, deadline=None)


def _grad(rng, shape, log10_scale):
    return rng.normal(size=shape) * 10.0 ** (log10_scale + rng.uniform(-1, 1, shape))


@RUNS
@given(shape=SHAPES, seed=st.integers(0, 2 ** 31 - 1), clip=st.sampled_from([0.05, 0.3, 1.0, 3.0]),
       scale=st.floats(-3, 3))
def test_clip_sets_the_update_rms(shape, seed, clip, scale):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 0.02, shape)
    g = _grad(rng, shape, scale)
    st0 = oracle.adafactor_init_state(shape)
    # relative step at t = 1: lr = 1e-2; no first moment, no decay, no scaling by RMS(x)
    hp = {"scale_parameter": False, "clip_threshold": clip}
    xn, _ = oracle.adafactor_step_tensor(x, g, st0, hp, 1)
    free, _ = oracle.adafactor_step_tensor(x, g, st0, dict(hp, clip_threshold=1e30), 1)
    rms = math.sqrt(np.mean(((xn - x) / 1e-2) ** 2))
    rms_u = math.sqrt(np.mean(((free - x) / 1e-2) ** 2))
    if rms_u > clip:
        assert math.isclose(rms, clip, rel_tol=1e-10)
    else:
        assert np.allclose(xn, free, rtol=1e-14, atol=0)


@RUNS
@given(shape=SHAPES, seed=st.integers(0, 2 ** 31 - 1), opt=st.sampled_from(["adafactor", "came"]),
       power=st.integers(-10, 30), scale=st.floats(-1, 3))
def test_gradient_scale_leaves_the_update(shape, seed, opt, power, scale):
    rng = np.random.default_rng(seed)
    hp = {"beta1": 0.9, "weight_decay": 0.1} if opt == "adafactor" else {"lr": 2e-4, "weight_decay": 0.05}
    x = rng.normal(0, 0.02, shape)
    a, b = x, x
    sa = oracle.INIT_STATE[opt](shape, hp)
    sb = oracle.INIT_STATE[opt](shape, hp)
    for t in range(1, 4):
        g = _grad(rng, shape, scale)
        a, sa = oracle.STEP_TENSOR[opt](a, g, sa, hp, t)
        b, sb = oracle.STEP_TENSOR[opt](b, g * 2.0 ** power, sb, hp, t)
        assert np.allclose(a, b, rtol=1e-11, atol=0), t


@RUNS
@given(shape=SHAPES, seed=st.integers(0, 2 ** 31 - 1), lr=st.sampled_from([1e-4, 1e-3, 2e-2]),
       wd=st.sampled_from([0.0, 0.01, 0.3]), bias_correction=st.booleans(), scale=st.floats(-3, 2))
def test_lamb_moves_x_by_lr_times_its_norm(shape, seed, lr, wd, bias_correction, scale):
    rng = np.random.default_rng(seed)
    hp = {"lr": lr, "weight_decay": wd, "bias_correction": bias_correction}
    x = rng.normal(0, 0.02, shape)
    s = oracle.lamb_init_state(shape)
    for t in range(1, 5):
        g = _grad(rng, shape, scale)
        sc = {}
        xn, s = oracle.lamb_step_tensor(x, g, s, hp, t, scalars=sc)
        assert sc["x_norm"] > 0 and sc["d_norm"] > 0
        assert math.isclose(np.linalg.norm(xn - x), lr * np.linalg.norm(x), rel_tol=1e-10), t
        x = xn
