"""CPU checks of the parity bars used by the GPU tests (tests/harness.py): the
16-bit rules accept the one-step rounding disagreements that near-tie values may
take, and reject systematic faults planted on the CPU (truncation instead of
rounding to nearest, a skipped rounding, a wrong value in a tail); the step and
scalar checks reject faults planted in a float32 replica of the step (a step size
or clip divisor 0.1% off, LAMB's decay term dropped, its trust ratio 0.1% off)."""
import numpy as np
import pytest

import oracle
from tests.harness import TOL_F32, bar_kind, check_bar


def _bits_down(a):
    """bf16 by truncation (the planted fault): drop the low 16 bits of the float32."""
    f = np.asarray(a, dtype=np.float32)
    return (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def _one_step_up(a):
    """The next bf16 value away from zero (a one-step rounding disagreement)."""
    f = np.asarray(a, dtype=np.float32)
    return (f.view(np.uint32) + np.uint32(0x10000)).view(np.float32).astype(np.float64)


def test_bar_kinds():
    st = dict(param_bf16=False, exp_avg_bf16=True)
    assert bar_kind("adafactor", {}, st, "param") == "f32"                 # no first moment
    assert bar_kind("adafactor", {"beta1": 0.9}, st, "param") == "rounded"    # stepped by a bf16 moment
    assert bar_kind("came", {}, st, "exp_avg_res_row") == "rounded"
    assert bar_kind("came", {}, st, "exp_avg_sq_col") == "f32"             # depends on G only
    assert bar_kind("lamb", {}, st, "exp_avg_sq") == "f32"
    assert bar_kind("lamb", {}, dict(param_bf16=True), "param") == "rounded"
    assert bar_kind("lamb", {}, dict(param_bf16=True), "exp_avg") == "f32"
    i8 = dict(exp_avg_i8=True)
    assert bar_kind("lamb", {}, i8, "exp_avg") == "codes"
    assert bar_kind("lamb", {}, i8, "exp_avg_scale") == "rounded"
    assert bar_kind("adafactor", {"beta1": 0.9}, i8, "param") == "rounded"
    assert bar_kind("came", {}, i8, "exp_avg_res_col") == "rounded"
    assert bar_kind("came", {}, i8, "exp_avg_sq_row") == "f32"


def test_sixteen_bit_rules():
    rng = np.random.default_rng(5)
    exact = rng.normal(0, 1e-3, 20000)
    ref = oracle.round_bf16(exact)
    # one-step disagreements on a few near-tie elements pass
    lib = ref.copy()
    idx = rng.choice(lib.size, 60, replace=False)
    lib[idx] = _one_step_up(lib[idx])
    ok, err, over, n = check_bar("rounded", "exp_avg", lib, ref)
    assert ok and over == 60 and err <= 2.0 ** -7
    # the same disagreements fail the fp32 bar
    assert not check_bar("f32", "exp_avg", lib, ref)[0]
    # truncation instead of round-to-nearest moves about half the elements
    ok, err, over, n = check_bar("rounded", "exp_avg", _bits_down(exact), ref)
    assert not ok and over > 0.3 * n
    # a skipped rounding (fp32 values stored) moves nearly all of them
    assert not check_bar("rounded", "exp_avg", exact.astype(np.float32).astype(np.float64), ref)[0]
    # garbage in a ragged tail of 7 elements breaks the elementwise bound
    lib = ref.copy()
    lib[-7:] = 0.0
    assert not check_bar("rounded", "exp_avg", lib, ref)[0]
    # an exact match passes both bars
    assert check_bar("f32", "param", ref, ref)[:2] == (True, 0.0)
    assert TOL_F32 == 1e-5


def test_code_rules():
    """8-bit first moment, judged on code x scale against its group's largest
    magnitude: scattered one- and two-step disagreements pass; a value off by 3
    steps, a systematic shift of many codes, or a wrong scale fails."""
    rng = np.random.default_rng(6)
    m = rng.normal(size=128 * 400) * 10.0 ** np.repeat(rng.uniform(-3, 1, 400), 128)
    codes, scales = oracle.quantize_i8(m)
    ref = (codes, scales)
    lib = codes.astype(np.int16)
    idx = rng.choice(lib.size, 100, replace=False)
    lib[idx] = np.clip(lib[idx] + 1, -127, 127)
    lib[idx[:3]] = np.clip(lib[idx[:3]] + 1, -127, 127)   # three values two steps off
    ok, err, over, n = check_bar("codes", "exp_avg", (lib.astype(np.int8), scales), ref)
    assert ok and err <= 2.5 / 127 and over <= 100
    lib[idx[0]] = np.clip(codes[idx[0]] + 3, -127, 127)
    assert not check_bar("codes", "exp_avg", (lib.astype(np.int8), scales), ref)[0]
    shifted = np.clip(codes.astype(np.int16) + (rng.random(codes.size) < 0.2), -127, 127).astype(np.int8)
    assert not check_bar("codes", "exp_avg", (shifted, scales), ref)[0]
    assert not check_bar("codes", "exp_avg", (codes, scales * np.float32(1.03)), ref)[0]


# Faults a kernel could make in the step itself, planted in the float32 replica
# (tests/fp32_replica.py) on the CPU. Each must fail the named check on the weight
# matrices. The step check dX catches them on its own, except CAME's clip divisor:
# a factored CAME step M / sqrt(S) does not change when U is scaled (M and sqrt(S)
# scale alike), so that fault shows in the first moment.
@pytest.mark.parametrize("case,fault,check", [
    ("adafactor_defaults", "alpha*1.001", "dx"),
    ("adafactor_beta1", "alpha*1.001", "dx"),
    ("adafactor_beta1", "kappa*1.001", "dx"),
    ("came", "kappa*1.001", "exp_avg"),
    ("lamb", "no_decay", "dx"),
    ("lamb", "trust*1.001", "dx"),
])
def test_planted_step_faults_fail(case, fault, check):
    from tests.test_tolerance_floors import CASES, replica_run
    wl = CASES[case]
    failed = {}
    for t, k, res, _, _, _ in replica_run(wl, steps=3, fault=fault):
        for key, v in res.items():
            if not v[0]:
                failed.setdefault(key, set()).add(wl.specs[k].kind)
    assert "weight" in failed.get(check, ()), (case, fault, failed)


def test_correct_replica_passes_planted_fault_cases():
    """The same three steps without a fault pass every check (the faults above are
    what fails, not the cases)."""
    from tests.test_tolerance_floors import CASES, replica_run
    for case in ("adafactor_defaults", "adafactor_beta1", "came", "lamb"):
        for t, k, res, _, _, _ in replica_run(CASES[case], steps=3):
            assert all(v[0] for v in res.values()), (case, t, k, {key: v for key, v in res.items() if not v[0]})


def test_lamb_stored_moment_step_is_ratio_times_direction():
    """LAMB with an fp32 parameter and a bf16 first moment: a near-tie element of the
    stored moment moves the trust ratio (and so every element's step) by the same
    small factor, 3e-5 here. The step check compares the direction, the ratio keeps
    its own bar. Planted faults still fail: a step applied with a ratio 0.1% off the
    one the library reports, the reported ratio 0.1% off, a wrong direction."""
    from tests.harness import judge_arrays
    rng = np.random.default_rng(11)
    n, lr = 256, 2e-3
    storage = dict(param_bf16=False, exp_avg_bf16=True, exp_avg_i8=False)
    assert bar_kind("lamb", {}, storage, "param") == "rounded"
    xo = rng.normal(0, 0.02, n)
    d = rng.normal(0, 1, n)
    tau = np.linalg.norm(xo) / np.linalg.norm(d)
    x_ref = xo - lr * tau * d
    ref_sc = {"x_norm": np.linalg.norm(xo), "d_norm": np.linalg.norm(d), "trust": tau}

    def judge(applied, reported, direction=d):
        x_lib = (xo - lr * applied * direction).astype(np.float32).astype(np.float64)
        lib_sc = {"rms_x": ref_sc["x_norm"], "norm_d": ref_sc["d_norm"] * tau / reported, "trust": reported}
        return judge_arrays("lamb", {}, storage, [("param", x_lib, x_ref)], xo, xo, xo, lib_sc, ref_sc)

    near_tie = tau * (1 + 3e-5)
    res = judge(near_tie, near_tie)
    assert res["dx"][0] and res["scalar:trust"][0], res
    assert res["dx"][2] == 0
    # compared element by element without the rescale, the same step fails
    from tests.harness import check_dx
    x_lib = (xo - lr * near_tie * d).astype(np.float32).astype(np.float64)
    assert not check_dx("rounded", x_lib, xo, x_ref, xo)[0]
    # faults
    assert not judge(near_tie * 1.001, near_tie)["dx"][0]
    assert not judge(tau * 1.001, tau * 1.001)["scalar:trust"][0]
    assert not judge(tau, tau, d + 0.05 * d.std() * np.sign(xo))["dx"][0]


def test_small_update_rule_forgives_storage_only():
    """The update check (GaLore; the other optimizers' step check alike) forgives one
    fp32 spacing of the parameter per element: a small update (1.7e-3 of the
    parameter) stored in fp32 passes at 1e-4, while the same update with its
    coefficient 0.1% off, or with the decay term dropped, fails."""
    from tests.harness import dx_errs
    rng = np.random.default_rng(12)
    x0 = rng.normal(0, 0.02, 20000)
    decay, coef = 1 - 1e-3, 2.5e-3
    c = rng.normal(0, 0.011, x0.size)
    want = decay * x0 - coef * c

    def worst(got):
        e, _ = dx_errs(got, x0, want, x0, floor=1.0)
        return float(np.max(e))

    f32 = lambda v: np.asarray(v, dtype=np.float32).astype(np.float64)
    stored = f32(f32(decay * f32(x0)) - f32(coef * c))   # the kernel's roundings
    assert worst(stored) <= 1e-4
    from tests.harness import floored_rel_err
    assert floored_rel_err(stored - x0, want - x0) > 1e-4   # the storage rounding alone, unforgiven
    assert worst(f32(decay * x0 - 1.001 * coef * c)) > 1e-4
    assert worst(f32(x0 - coef * c)) > 1e-4
