"""Evidence for the parity bars of tests/harness.py, on the CPU.

A plain float32 implementation of the method (tests/fp32_replica.py: float32
statistics and per-element arithmetic, fp64 per-tensor scalars) stands in for the
library and is judged against the fp64 oracle with exactly the rules the GPU
parity tests apply, over 10 chained steps with the gradient statistics of the
configurations (config 1: Adafactor defaults, per-row gradient scales 10^U(-2, 2);
configs 2 and 4: bf16 gradients N(0, 1e-3) with row and column scales; config 5:
LAMB, N(0, 1e-2), weights, LayerNorm weights and zero-initialised biases). A
correct fp32 implementation must pass every bar with room to spare; the tests
also record where the floors come from:

* the first moment reaches 4e-6 to 5e-6 under its floor (0.1 RMS(b) and the
  average's terms; 7e-6 to 9e-6 with 0.1 RMS(b) alone): the floor cannot be
  lower;
* S23's floor 1e-2 RMS(b) alone is not reachable for the parameter of a
  zero-initialised bias (default Adafactor) or for CAME's parameter, while the
  floor max(1e-2 RMS(b), RMS(b - x0)) is met at ~1e-6.

tests/test_harness_rules.py plants faults in the same replica and checks that the
bars reject them.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import fp32_replica as rep
from tests.harness import (FLOOR_PARAM, TOL_F32, floored_rel_err, judge_arrays)

# 10 chained steps per case; shapes large enough for the statistics (means over
# hundreds of rows) and small enough for seconds on the CPU.
CASES = {
    "adafactor_defaults": workloads.custom(
        "floors_af_def", "adafactor", [(256, 512), (512,)], hparams={}, grad_dtype=torch.float32, grad_std=1.0,
        grad_scaling="row", kinds=["weight", "bias"]),
    "adafactor_beta1": workloads.custom(
        "floors_af_b1", "adafactor", [(384, 512), (512,)], hparams={"beta1": 0.9}, grad_dtype=torch.bfloat16,
        grad_std=1e-3, grad_scaling="rowcol"),
    "adafactor_beta1_wd": workloads.custom(
        "floors_af_wd", "adafactor", [(384, 512), (512,)], hparams={"beta1": 0.9, "weight_decay": 0.1},
        grad_dtype=torch.bfloat16, grad_std=1e-3, grad_scaling="rowcol"),
    "came": workloads.custom(
        "floors_came", "came", [(384, 512), (512,)], hparams={"lr": 2e-4}, grad_dtype=torch.bfloat16,
        grad_std=1e-3, grad_scaling="rowcol"),
    "lamb": workloads.custom(
        "floors_lamb", "lamb", [(512, 512), (512,), (512,), (1024, 512)], hparams={"weight_decay": 0.01},
        grad_std=1e-2, grad_scaling="none", kinds=["weight", "norm", "bias", "weight"]),
}
STEPS = 10


def _slots(opt, sc):
    """The replica's scalars under the library's slot names."""
    if opt == "lamb":
        return {"rms_x": sc["x_norm"], "norm_d": sc["d_norm"], "trust": sc["trust"]}
    return dict(sc)


def replica_run(wl, steps=STEPS, fault=""):
    """Chained replica and oracle steps; yields (t, tensor index, judged checks,
    replica parameter, oracle parameter, initial parameter) after every step."""
    opt, hp = wl.optimizer, dict(wl.hparams)
    x0 = [p.numpy().astype(np.float64) for p in workloads.init_params(wl, "cpu")]
    scales = workloads.grad_scales(wl, "cpu")
    ox = [x.copy() for x in x0]
    ost = [oracle.INIT_STATE[opt](x.shape, hp) for x in x0]
    rx = [x.astype(np.float32) for x in x0]
    rst = [{k: v.astype(np.float32) for k, v in st.items()} for st in ost]
    for t in range(1, steps + 1):
        gs = [g.to(torch.float64).numpy() for g in workloads.grads(wl, t - 1, scales, "cpu")]
        for k in range(len(x0)):
            ref_sc = {}
            xo_ref, xo_lib, m_prev = ox[k], rx[k], ost[k].get("exp_avg")
            ox[k], ost[k] = oracle.STEP_TENSOR[opt](ox[k], gs[k], ost[k], hp, t, scalars=ref_sc)
            rx[k], rst[k], lib_sc = rep.STEP[opt](rx[k], gs[k], rst[k], hp, t, fault=fault)
            out = [("param", rx[k], ox[k])] + [(key, rst[k][key], ost[k][key]) for key in ost[k]]
            res = judge_arrays(opt, hp, {}, out, x0[k], xo_lib, xo_ref, _slots(opt, lib_sc), ref_sc, m_prev)
            yield t, k, res, rx[k], ox[k], x0[k]


@pytest.mark.parametrize("case", sorted(CASES))
def test_fp32_replica_meets_every_bar(case):
    """A correct fp32 implementation passes every bar. The first moment and the
    step dX are the tightest (up to ~5e-6 against 1e-5, from the update's own fp32
    error of a few ulps carried into an average that crosses zero); the step's
    normwise bar and the scalars' bar leave a factor of five or more."""
    wl = CASES[case]
    worst = {}
    for t, k, res, _, _, _ in replica_run(wl):
        bad = {key: v for key, v in res.items() if not v[0]}
        assert not bad, (case, t, k, bad)
        for key, v in res.items():
            worst[key] = max(worst.get(key, 0.0), v[1])
            if key == "dx":
                worst["dx_normwise"] = max(worst.get("dx_normwise", 0.0), v[5])
    print(case, {k: f"{v:.2e}" for k, v in sorted(worst.items())})
    for key, v in worst.items():
        if key.startswith("scalar:") or key == "dx_normwise":
            assert v <= 2e-7, (case, key, v)


@pytest.mark.parametrize("case", ["adafactor_defaults", "came"])
def test_s23_floor_alone_is_out_of_reach_for_the_parameter(case):
    """With the floor 1e-2 RMS(b) alone, the replica's parameter misses 1e-5 (a
    bias that starts at zero is nothing but its accumulated steps, which cancel to
    near zero; CAME's steps are large against its parameter's RMS), while the
    harness's floor, which also includes RMS(b - x0), holds it to ~1e-6."""
    wl = CASES[case]
    s23 = harness = 0.0
    for t, k, res, rx, ox, x0 in replica_run(wl):
        s23 = max(s23, floored_rel_err(rx, ox, FLOOR_PARAM))
        harness = max(harness, res["param"][1])
    assert s23 > TOL_F32
    assert harness < 0.3 * TOL_F32
