"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks oracle *behaviour* (whole steps) against a value that does not
come from the oracle: page text (defaults, messages), closed forms of the page's
schedules, closed-form special cases (rank-1 recovery, zero gradient, unit dims),
invariants (clip, sign, scale, list independence, LAMB's norm identity), a
50-digit brute force on tiny inputs, and Hugging Face's Adafactor, which the page
says the defaults are aligned with.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import brute_mp

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    den = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / den


# ----------------------------------------------------------------------------- page text

def test_defaults_match_page():
    g = _gold("page_defaults.json")
    for name, got in (("adafactor", oracle.ADAFACTOR_DEFAULTS), ("came", oracle.CAME_DEFAULTS),
                      ("lamb", oracle.LAMB_DEFAULTS)):
        exp = g[name]
        assert set(exp) == set(got), name
        for k, v in exp.items():
            gv = got[k]
            if isinstance(v, list):
                assert list(gv) == v, (name, k)
            else:
                assert gv == v, (name, k)


def test_adafactor_validation_messages():
    m = _gold("page_defaults.json")["messages"]
    with pytest.raises(ValueError, match=m["lr_with_relative_step"]):
        oracle.adafactor_hparams({"lr": 1e-3})
    with pytest.raises(ValueError, match=m["warmup_needs_relative_step"]):
        oracle.adafactor_hparams({"lr": 1e-3, "relative_step": False, "warmup_init": True})
    with pytest.raises(ValueError):
        oracle.adafactor_hparams({"relative_step": False})
    oracle.adafactor_hparams({"lr": 1e-3, "relative_step": False})


def test_lamb_and_came_validation():
    for bad in ({"lr": -1.0}, {"eps": -1e-6}, {"betas": (1.0, 0.999)}, {"betas": (0.9, -0.1)}):
        with pytest.raises(ValueError):
            oracle.lamb_hparams(bad)
    with pytest.raises(ValueError):
        oracle.came_hparams({})  # no lr
    with pytest.raises(ValueError):
        oracle.came_hparams({"lr": 1e-3, "betas": (0.9, 0.999, 1.0)})


# ----------------------------------------------------------------------------- schedules

def test_beta2t_schedule_through_state():
    """From a 1-D state V0 = 1 and a zero gradient, one step at index t leaves
    V = beta2t(t) + (1 - beta2t(t)) * eps1: the schedule, observed in the state."""
    sched = _gold("schedule.json")["beta2t"]
    for t_str, b in sched.items():
        t = int(t_str)
        st = {"exp_avg_sq": np.ones(4)}
        _, new = oracle.adafactor_step_tensor(np.ones(4), np.zeros(4), st, {}, t)
        assert np.allclose(new["exp_avg_sq"], b + (1 - b) * 1e-30, rtol=1e-14, atol=1e-300), t


@pytest.mark.parametrize("kind", ["rho", "rho_warmup"])
def test_relative_step_size_through_update(kind):
    """1-D tensor, |g| = 1, V0 = 1: V stays 1, u = sign(g), RMS(u) = 1 so no
    clipping, and with scale_parameter off the update is exactly -rho_t * sign(g)."""
    sched = _gold("schedule.json")[kind]
    hp = {"scale_parameter": False, "warmup_init": kind == "rho_warmup"}
    g = np.array([1.0, -1.0, 1.0, 1.0, -1.0, -1.0])
    for t_str, rho in sched.items():
        t = int(t_str)
        x = np.zeros(6)
        st = {"exp_avg_sq": np.ones(6)}
        xn, _ = oracle.adafactor_step_tensor(x, g, st, hp, t)
        assert np.allclose(xn - x, -rho * np.sign(g), rtol=1e-12, atol=0), t


# ----------------------------------------------------------------------------- closed forms

def _rank1_grad(rng, h, w):
    a = rng.uniform(0.1, 10.0, h) * rng.choice([-1.0, 1.0], h)
    b = rng.uniform(0.1, 10.0, w) * rng.choice([-1.0, 1.0], w)
    s = rng.choice([-1.0, 1.0], (h, w))
    return a[:, None] * s * b[None, :]


@pytest.mark.parametrize("shape", [(12, 20), (1, 9), (7, 1), (3, 5, 6)])
def test_adafactor_rank1_exact_recovery(shape):
    """|G| = |a_i| |b_j| makes G^2 rank-1, so the factored estimate equals G^2
    (eps1 aside) and u = sign(G): every step (constant G is a fixed point of the
    statistics) moves X by exactly -1e-2 * max(1e-3, RMS(X)) * sign(G)."""
    rng = np.random.default_rng(1)
    h, w = shape[-2], shape[-1]
    lead = shape[:-2]
    g = np.stack([_rank1_grad(rng, h, w) for _ in range(int(np.prod(lead)) or 1)])
    g = g.reshape(shape)
    x = rng.normal(0, 0.02, shape)
    st = oracle.adafactor_init_state(shape)
    for t in range(1, 6):
        xn, st = oracle.adafactor_step_tensor(x, g, st, {}, t)
        expect = -1e-2 * max(1e-3, math.sqrt(np.mean(x * x))) * np.sign(g)
        assert np.allclose(xn - x, expect, rtol=1e-10, atol=0), t
        x = xn


def test_adafactor_scale_parameter_floor_on_zero_bias():
    """A zero-initialised bias has RMS(X) = 0 < eps2, so scale_parameter uses the
    floor eps2 = 1e-3: with |g| = 1 at step 1 the update is -1e-2 * 1e-3 * sign(g)."""
    g = np.array([1.0, -1.0, -1.0, 1.0, 1.0])
    xn, _ = oracle.adafactor_step_tensor(np.zeros(5), g, oracle.adafactor_init_state((5,)), {}, 1)
    assert np.allclose(xn, -1e-5 * np.sign(g), rtol=1e-12, atol=0)


def test_adafactor_step1_statistics_are_plain_means():
    """beta2t(1) = 0: step 1's row and column statistics are the plain row and
    column means of G^2 + eps1 (checked by explicit loops), whatever the prior state."""
    rng = np.random.default_rng(2)
    g = rng.normal(size=(5, 7))
    g[2, :] = 0.0
    st = {"exp_avg_sq_row": rng.uniform(1, 2, 5), "exp_avg_sq_col": rng.uniform(1, 2, 7)}
    _, new = oracle.adafactor_step_tensor(rng.normal(size=(5, 7)), g, st, {}, 1)
    for i in range(5):
        s = 0.0
        for j in range(7):
            s += g[i, j] * g[i, j] + 1e-30
        assert math.isclose(new["exp_avg_sq_row"][i], s / 7, rel_tol=1e-14)
    for j in range(7):
        s = 0.0
        for i in range(5):
            s += g[i, j] * g[i, j] + 1e-30
        assert math.isclose(new["exp_avg_sq_col"][j], s / 5, rel_tol=1e-14)


@pytest.mark.parametrize("beta1", [None, 0.9])
def test_adafactor_unit_dims_equal_full_path(beta1):
    """A factored [1, W] or [H, 1] matrix reconstructs the full statistic exactly,
    so over several steps it matches the 1-D path on the same numbers."""
    rng = np.random.default_rng(3)
    hp = {"beta1": beta1, "weight_decay": 0.1}
    for shape in ((1, 9), (9, 1)):
        x2 = rng.normal(0, 0.02, shape)
        x1 = x2.reshape(-1).copy()
        s2 = oracle.adafactor_init_state(shape, hp)
        s1 = oracle.adafactor_init_state((9,), hp)
        for t in range(1, 5):
            g = rng.normal(size=shape) * 10.0 ** rng.uniform(-2, 2, shape)
            x2, s2 = oracle.adafactor_step_tensor(x2, g, s2, hp, t)
            x1, s1 = oracle.adafactor_step_tensor(x1, g.reshape(-1), s1, hp, t)
            assert np.allclose(x2.reshape(-1), x1, rtol=1e-13, atol=0), (shape, t)


@pytest.mark.parametrize("clip", [0.1, 0.5])
def test_adafactor_clip_sets_update_rms(clip):
    """When RMS(u) exceeds clip_threshold, the applied update (before lr) has RMS
    exactly clip_threshold; with a huge threshold the update is left alone."""
    rng = np.random.default_rng(4)
    x = rng.normal(0, 0.02, (16, 24))
    g = rng.normal(size=(16, 24)) * 10.0 ** rng.uniform(-2, 2, (16, 24))
    st = oracle.adafactor_init_state((16, 24))
    hp = {"scale_parameter": False, "clip_threshold": clip}
    xn, _ = oracle.adafactor_step_tensor(x, g, st, hp, 1)
    step = (xn - x) / 1e-2
    assert math.isclose(math.sqrt(np.mean(step ** 2)), clip, rel_tol=1e-12)
    a, _ = oracle.adafactor_step_tensor(x, g, st, {"scale_parameter": False, "clip_threshold": 1e3}, 1)
    b, _ = oracle.adafactor_step_tensor(x, g, st, {"scale_parameter": False, "clip_threshold": 1e6}, 1)
    assert np.array_equal(a, b)
    assert math.sqrt(np.mean(((a - x) / 1e-2) ** 2)) > 1.0  # unclipped RMS is above 1 here


def test_adafactor_zero_grad_is_pure_decay():
    rng = np.random.default_rng(5)
    for shape in ((6, 10), (10,)):
        x = rng.normal(0, 0.02, shape)
        st = oracle.adafactor_init_state(shape, {"beta1": 0.9})
        xn, new = oracle.adafactor_step_tensor(x, np.zeros(shape), st, {"beta1": 0.9, "weight_decay": 0.3}, 1)
        alpha = 1e-2 * max(1e-3, math.sqrt(np.mean(x * x)))
        assert np.allclose(xn, x * (1 - 0.3 * alpha), rtol=1e-15, atol=0)
        assert np.all(new["exp_avg"] == 0)


def test_adafactor_update_opposes_gradient():
    rng = np.random.default_rng(6)
    for shape in ((8, 12), (30,), (2, 4, 6)):
        x = rng.normal(0, 0.02, shape)
        g = rng.normal(size=shape)
        g.flat[::7] = 0.0
        xn, _ = oracle.adafactor_step_tensor(x, g, oracle.adafactor_init_state(shape), {}, 1)
        assert np.array_equal(np.sign(xn - x), -np.sign(g))


def test_adafactor_step1_ignores_prior_state():
    rng = np.random.default_rng(7)
    for shape in ((8, 12), (30,)):
        x = rng.normal(0, 0.02, shape)
        g = rng.normal(size=shape)
        z = oracle.adafactor_init_state(shape)
        r = {k: rng.uniform(0.5, 3.0, v.shape) for k, v in z.items()}
        a, _ = oracle.adafactor_step_tensor(x, g, z, {}, 1)
        b, _ = oracle.adafactor_step_tensor(x, g, r, {}, 1)
        assert np.allclose(a, b, rtol=1e-15, atol=0)


@pytest.mark.parametrize("opt", ["adafactor", "came"])
def test_gradient_scale_invariance(opt):
    """Scaling G by a power of two leaves u, hence every update, unchanged (eps1
    is negligible), over several chained steps."""
    rng = np.random.default_rng(8)
    hp = {"beta1": 0.9} if opt == "adafactor" else {"lr": 2e-4}
    shapes = [(10, 14), (14,)]
    xs = [rng.normal(0, 0.02, s) for s in shapes]
    ya = list(xs)
    yb = list(xs)
    sa = [oracle.INIT_STATE[opt](s, hp) for s in shapes]
    sb = [oracle.INIT_STATE[opt](s, hp) for s in shapes]
    for t in range(1, 4):
        gs = [rng.normal(size=s) * 10.0 ** rng.uniform(-2, 2, s) for s in shapes]
        ya, sa = oracle.STEP[opt](ya, gs, sa, hp, t)
        yb, sb = oracle.STEP[opt](yb, [g * 2.0 ** 20 for g in gs], sb, hp, t)
        for p, q in zip(ya, yb):
            assert np.allclose(p, q, rtol=1e-12, atol=0)


@pytest.mark.parametrize("opt", ["adafactor", "came", "lamb"])
def test_list_equals_per_tensor(opt):
    rng = np.random.default_rng(9)
    hp = {"adafactor": {"beta1": 0.9}, "came": {"lr": 2e-4}, "lamb": {"weight_decay": 0.01}}[opt]
    shapes = [(6, 9), (9,), (3, 4, 5)]
    xs = [rng.normal(0, 0.02, s) for s in shapes]
    gs = [rng.normal(size=s) for s in shapes]
    st = [oracle.INIT_STATE[opt](s, hp) for s in shapes]
    lx, _ = oracle.STEP[opt](xs, gs, st, hp, 1)
    for k in range(3):
        px, _ = oracle.STEP_TENSOR[opt](xs[k], gs[k], st[k], hp, 1)
        assert np.array_equal(px, lx[k])


@pytest.mark.parametrize("opt", ["adafactor", "came", "lamb"])
def test_empty_tensors_leave_the_rest_alone(opt):
    """An empty tensor has no element to take a statistic, a norm or a step over:
    a list holding empty tensors steps its other tensors exactly as the list
    without them does, for three chained steps, and hands the empty ones back with
    their shapes and their states unchanged (the per-tensor reading of the pages'
    loop over parameters, which an empty parameter leaves with nothing to update)."""
    rng = np.random.default_rng(11)
    hp = {"adafactor": {"beta1": 0.9}, "came": {"lr": 2e-4}, "lamb": {"weight_decay": 0.01}}[opt]
    full = [(6, 9), (9,), (3, 4, 5)]
    empty = [(0,), (0, 5), (3, 0), (2, 0, 4)]
    order = [full[0], empty[0], empty[1], full[1], empty[2], full[2], empty[3]]
    xs = {s: rng.normal(0, 0.02, s) for s in order}
    gs = [{s: rng.normal(size=s) for s in order} for _ in range(3)]
    st_all = [oracle.INIT_STATE[opt](s, hp) for s in order]
    st_full = [oracle.INIT_STATE[opt](s, hp) for s in full]
    x_all, x_full = [xs[s] for s in order], [xs[s] for s in full]
    for t in (1, 2, 3):
        x_all, st_all = oracle.STEP[opt](x_all, [gs[t - 1][s] for s in order], st_all, hp, t)
        x_full, st_full = oracle.STEP[opt](x_full, [gs[t - 1][s] for s in full], st_full, hp, t)
        got = {s: (x, st) for s, x, st in zip(order, x_all, st_all)}
        for s, x, st in zip(full, x_full, st_full):
            assert np.array_equal(got[s][0], x)
            assert got[s][1].keys() == st.keys()
            for k in st:
                assert np.array_equal(got[s][1][k], st[k])
        for s in empty:
            x, st = got[s]
            assert x.shape == s
            init = oracle.INIT_STATE[opt](s, hp)
            assert st.keys() == init.keys()
            for k in init:
                assert np.shape(st[k]) == np.shape(init[k]) and np.array_equal(st[k], init[k])


def test_came_rank1_closed_form_over_steps():
    """Constant G with rank-1 G^2: the squared-gradient estimate is
    (1 - beta2^t) G^2, so u = sign(G) / sqrt(1 - beta2^t), RMS clipping brings it
    back to sign(G); the first moment is (1 - beta1^t) sign(G); the instability is
    the constant beta1^(2t) + eps2, so the confidence statistic is a plain EMA of it
    and the step is -lr (1 - beta1^t) sign(G) / sqrt(R_t). At step 1 with the page's
    defaults and lr = 2e-4 that is -2.2222...e-3 sign(G)."""
    rng = np.random.default_rng(10)
    b1, b3, e2, lr = 0.9, 0.9999, 1e-16, 2e-4
    g = _rank1_grad(rng, 12, 20)
    x = rng.normal(0, 0.02, (12, 20))
    st = oracle.came_init_state((12, 20))
    r = 0.0
    for t in range(1, 7):
        xn, st = oracle.came_step_tensor(x, g, st, {"lr": lr}, t)
        r = b3 * r + (1 - b3) * (b1 ** (2 * t) + e2)
        expect = -lr * (1 - b1 ** t) / math.sqrt(r) * np.sign(g)
        assert np.allclose(xn - x, expect, rtol=1e-9, atol=0), t
        if t == 1:
            assert np.allclose(xn - x, -(2e-4 * 0.1 / math.sqrt(1e-4 * (0.81 + 1e-16))) * np.sign(g),
                               rtol=1e-9)
            assert math.isclose(float(np.max(np.abs(xn - x))), 2.0 / 900.0, rel_tol=1e-9)
        x = xn


def test_came_1d_step1_closed_form():
    """1-D CAME at step 1 with |g| > 0: u = sign(g), first moment (1 - beta1) sign(g),
    which is the whole step (no confidence factor on a full statistic)."""
    rng = np.random.default_rng(11)
    g = rng.normal(size=17)
    x = rng.normal(0, 0.02, 17)
    xn, _ = oracle.came_step_tensor(x, g, oracle.came_init_state((17,)), {"lr": 1e-3}, 1)
    assert np.allclose(xn - x, -1e-3 * 0.1 * np.sign(g), rtol=1e-12, atol=0)


def test_lamb_update_norm_is_lr_times_param_norm():
    rng = np.random.default_rng(12)
    hp = {"lr": 3e-3, "weight_decay": 0.01}
    for shape in ((20, 30), (30,), (2, 3, 4)):
        x = rng.normal(0, 0.02, shape)
        st = oracle.lamb_init_state(shape)
        for t in range(1, 5):
            g = rng.normal(0, 1e-2, shape)
            xn, st = oracle.lamb_step_tensor(x, g, st, hp, t)
            assert math.isclose(np.linalg.norm(xn - x), 3e-3 * np.linalg.norm(x), rel_tol=1e-12)
            x = xn
    # zero parameter: ratio 1, the step is lr * ||d||
    g = rng.normal(0, 1e-2, 40)
    xn, _ = oracle.lamb_step_tensor(np.zeros(40), g, oracle.lamb_init_state((40,)), hp, 1)
    d = g / (np.abs(g) + 1e-6)
    assert np.allclose(xn, -3e-3 * d, rtol=1e-12, atol=0)


def test_lamb_step1_bias_corrected_direction():
    """Bias correction at step 1 gives m_hat = g and v_hat = g^2, so the direction
    is g / (|g| + eps) + wd * x, scaled to length lr * ||x||."""
    rng = np.random.default_rng(13)
    x = rng.normal(0, 0.02, (9, 11))
    g = rng.normal(0, 1e-2, (9, 11))
    xn, st = oracle.lamb_step_tensor(x, g, oracle.lamb_init_state((9, 11)), {"weight_decay": 0.01}, 1)
    d = g / (np.abs(g) + 1e-6) + 0.01 * x
    expect = x - 1e-3 * np.linalg.norm(x) / np.linalg.norm(d) * d
    assert np.allclose(xn, expect, rtol=1e-13, atol=0)
    assert np.allclose(st["exp_avg"], 0.1 * g, rtol=1e-15)


# ----------------------------------------------------------------------------- brute force

def _tiny_inputs(rng, shape):
    g = rng.normal(size=shape) * 10.0 ** rng.uniform(-2, 2, shape)
    g.flat[::5] = 0.0  # exact zeros
    return rng.normal(0, 0.02, shape), g


@pytest.mark.parametrize("shape", [(4, 8), (8, 4), (1, 8), (4, 1), (8,)])
@pytest.mark.parametrize("variant", [dict(), dict(beta1=0.9, weight_decay=0.1),
                                     dict(scale_parameter=False, clip_threshold=0.3),
                                     dict(relative_step=False, lr=3e-3, beta1=0.5)])
def test_adafactor_vs_brute_force(shape, variant):
    rng = np.random.default_rng(hash((shape, tuple(variant))) % 2**32)
    fac = len(shape) >= 2
    h, w = (shape if fac else (1, shape[0]))
    x, _ = _tiny_inputs(rng, shape)
    st = oracle.adafactor_init_state(shape, variant)
    bx = x.reshape(h, w)
    bst = {"row": [0] * h, "col": [0] * w, "v": [[0] * w], "m": [[0] * w for _ in range(h)]}
    kw = dict(eps=(1e-30, 1e-3), d=variant.get("clip_threshold", 1.0), beta1=variant.get("beta1"),
              wd=variant.get("weight_decay", 0.0), scale=variant.get("scale_parameter", True),
              lr=variant.get("lr"))
    for t in range(1, 4):
        _, g = _tiny_inputs(rng, shape)
        x, st = oracle.adafactor_step_tensor(x, g, st, variant, t)
        bx, bnew = brute_mp.adafactor(bx, g.reshape(h, w), bst, t, factored=fac, **kw)
        bst.update(bnew)
        assert _rel(x.reshape(h, w), [[float(v) for v in r] for r in bx]) < 1e-12, t
        if variant.get("beta1") is not None:
            assert _rel(st["exp_avg"].reshape(h, w), [[float(v) for v in r] for r in bst["m"]]) < 1e-12
        if fac:
            assert _rel(st["exp_avg_sq_row"], [float(v) for v in bst["row"]]) < 1e-12
            assert _rel(st["exp_avg_sq_col"], [float(v) for v in bst["col"]]) < 1e-12


@pytest.mark.parametrize("shape", [(4, 8), (8, 4), (1, 8), (4, 1), (8,)])
def test_came_vs_brute_force(shape):
    rng = np.random.default_rng(sum(shape) * 31 + len(shape))
    fac = len(shape) >= 2
    h, w = (shape if fac else (1, shape[0]))
    hp = {"lr": 2e-4, "weight_decay": 0.05}
    x, _ = _tiny_inputs(rng, shape)
    st = oracle.came_init_state(shape)
    bx = x.reshape(h, w)
    bst = {"row": [0] * h, "col": [0] * w, "rrow": [0] * h, "rcol": [0] * w, "v": [[0] * w],
           "m": [[0] * w for _ in range(h)]}
    for t in range(1, 4):
        _, g = _tiny_inputs(rng, shape)
        x, st = oracle.came_step_tensor(x, g, st, hp, t)
        bx, bnew = brute_mp.came(bx, g.reshape(h, w), bst, t, factored=fac, lr=2e-4, wd=0.05)
        bst.update(bnew)
        assert _rel(x.reshape(h, w), [[float(v) for v in r] for r in bx]) < 1e-12, t
        assert _rel(st["exp_avg"].reshape(h, w), [[float(v) for v in r] for r in bst["m"]]) < 1e-12
        if fac:
            assert _rel(st["exp_avg_res_row"], [float(v) for v in bst["rrow"]]) < 1e-12
            assert _rel(st["exp_avg_res_col"], [float(v) for v in bst["rcol"]]) < 1e-12


@pytest.mark.parametrize("shape", [(4, 8), (8, 4), (1, 8), (8,)])
@pytest.mark.parametrize("bc", [True, False])
def test_lamb_vs_brute_force(shape, bc):
    rng = np.random.default_rng(sum(shape) * 17 + int(bc))
    h, w = (shape if len(shape) == 2 else (1, shape[0]))
    hp = {"lr": 1e-3, "weight_decay": 0.01, "bias_correction": bc}
    x, _ = _tiny_inputs(rng, shape)
    st = oracle.lamb_init_state(shape)
    bx = x.reshape(h, w)
    bst = {"m": [[0] * w for _ in range(h)], "v": [[0] * w for _ in range(h)]}
    for t in range(1, 4):
        _, g = _tiny_inputs(rng, shape)
        x, st = oracle.lamb_step_tensor(x, g, st, hp, t)
        bx, bst = brute_mp.lamb(bx, g.reshape(h, w), bst, t, bc=bc)
        assert _rel(x.reshape(h, w), [[float(v) for v in r] for r in bx]) < 1e-12, t


# ----------------------------------------------------------------------------- library cross-check

def _hf_adafactor():
    try:
        import torch
        from transformers.optimization import Adafactor
    except Exception:  # pragma: no cover - the image ships both
        pytest.skip("transformers Adafactor not importable")
    return torch, Adafactor


@pytest.mark.parametrize("variant", [
    dict(),
    dict(beta1=0.9),
    dict(beta1=0.9, weight_decay=0.05),
    dict(scale_parameter=False, clip_threshold=0.5),
    dict(relative_step=False, lr=1e-3, beta1=0.8, decay_rate=-0.6),
    dict(warmup_init=True, weight_decay=0.1),
])
def test_adafactor_matches_hugging_face(variant):
    """The page says the defaults are aligned with Hugging Face's Adafactor; its
    implementation, run in float64 on the CPU, agrees with the oracle over several
    steps for every option, including the readings on momentum order, weight decay,
    the warmup rate and leading batch dims."""
    torch, Adafactor = _hf_adafactor()
    rng = np.random.default_rng(14)
    shapes = [(12, 20), (20,), (2, 6, 10), (1, 7)]
    xs = [rng.normal(0, 0.02, s) for s in shapes]
    ps = [torch.nn.Parameter(torch.tensor(x, dtype=torch.float64)) for x in xs]
    opt = Adafactor(ps, **variant)
    st = [oracle.adafactor_init_state(s, variant) for s in shapes]
    for t in range(1, 6):
        gs = [rng.normal(size=s) * 10.0 ** rng.uniform(-2, 2, s) for s in shapes]
        for p, g in zip(ps, gs):
            p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        xs, st = oracle.adafactor_step(xs, gs, st, variant, t)
        for p, x in zip(ps, xs):
            assert _rel(p.detach().numpy(), x) < 1e-12, (variant, t)


# ----------------------------------------------------------------------------- 16-bit storage

def _bf16_from_bits(hi):
    """The bf16 value whose 16 bits are ``hi`` (as the upper half of a float32)."""
    return np.array([hi << 16], dtype=np.uint32).view(np.float32).astype(np.float64)[0]


def test_round_bf16_ties_and_limits():
    """Closed forms of round-to-nearest-even at bf16's 7 fraction bits: 1 + 2^-8
    is the midpoint of 1 and 1 + 2^-7 and goes to the even 1; 1 + 3 * 2^-8 goes up
    to 1 + 2^-6; just above a midpoint goes up; the midpoint above the largest
    finite bf16 (0x7f7f, odd) goes to +inf; signs are symmetric."""
    r = oracle.round_bf16
    assert r(1.0 + 2.0 ** -8) == 1.0
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert r(-(1.0 + 2.0 ** -8)) == -1.0
    assert r(1.0 + 2.0 ** -9) == 1.0
    big = _bf16_from_bits(0x7F7F)
    assert r(big) == big
    mid = np.array([0x7F7F8000], dtype=np.uint32).view(np.float32).astype(np.float64)[0]
    assert r(mid) == math.inf and r(-mid) == -math.inf
    assert math.isnan(r(math.nan))
    assert r(0.0) == 0.0 and math.copysign(1.0, r(-0.0)) == -1.0
    # the smallest bf16 subnormal, and half of it (a tie with zero -> 0)
    tiny = _bf16_from_bits(0x0001)
    assert r(tiny) == tiny and r(tiny / 2) == 0.0


def test_round_bf16_matches_torch():
    """Against PyTorch's CPU float32 -> bfloat16 conversion (round to nearest even)
    on random bit patterns, exact ties, subnormals and out-of-range values."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, 20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    f = np.concatenate([bits.view(np.float32), ties.view(np.float32),
                        np.array([3.4e38, -3.4e38, 1e-40, -1e-45, np.inf, -np.inf], np.float32)])
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(f.astype(np.float64))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kind", ["adafactor", "came", "lamb"])
def test_bf16_storage_outputs_are_bf16_values(kind):
    """With 16-bit storage the new parameter and first moment are bf16 values, the
    fp32-kept statistics equal those of fp32 storage (they depend on g only, except
    CAME's confidence, which depends on the first moment), and the result stays
    within bf16 rounding of the fp32-storage result on the first step."""
    rng = np.random.default_rng(22)
    shape = (6, 10)
    x = oracle.round_bf16(rng.normal(0, 0.02, shape))
    g = rng.normal(size=shape)
    hp = {"adafactor": {"beta1": 0.9}, "came": {"lr": 1e-3}, "lamb": {}}[kind]
    st = oracle.INIT_STATE[kind](shape, hp)
    x16, s16 = oracle.STEP_TENSOR[kind](x, g, st, hp, 1, param_bf16=True, exp_avg_bf16=True)
    x32, s32 = oracle.STEP_TENSOR[kind](x, g, st, hp, 1)
    assert np.array_equal(oracle.round_bf16(x16), x16)
    assert np.array_equal(oracle.round_bf16(s16["exp_avg"]), s16["exp_avg"])
    for key in s32:
        if key not in ("exp_avg", "exp_avg_res_row", "exp_avg_res_col"):
            assert np.array_equal(s16[key], s32[key]), key
    assert np.max(np.abs(s16["exp_avg"] - s32["exp_avg"]) / np.abs(s32["exp_avg"])) <= 2.0 ** -8
    assert not np.array_equal(x16, x32)


@pytest.mark.parametrize("kind", ["adafactor", "came"])
def test_bf16_first_moment_is_the_step(kind):
    """Adafactor with beta1 and 1-D CAME take the first moment itself as the step:
    with 16-bit first-moment storage the step must be the *stored* (rounded) value,
    not the unrounded one (fp32 parameter, no weight decay)."""
    rng = np.random.default_rng(23)
    shape = (6, 10) if kind == "adafactor" else (37,)
    hp = {"adafactor": {"beta1": 0.9, "scale_parameter": False}, "came": {"lr": 1e-3}}[kind]
    scale = 1e-2 if kind == "adafactor" else 1e-3   # the lr that multiplies the moment
    x = rng.normal(0, 0.02, shape)
    st = oracle.INIT_STATE[kind](shape, hp)
    st["exp_avg"] = oracle.round_bf16(rng.normal(0, 1e-3, shape))
    for t in (1, 2):
        g = rng.normal(size=shape)
        xn, st = oracle.STEP_TENSOR[kind](x, g, st, hp, t, exp_avg_bf16=True)
        m = st["exp_avg"]
        assert np.array_equal(oracle.round_bf16(m), m)
        step = (x - xn) if kind == "adafactor" else (x - xn) / scale
        assert np.allclose(step, m, rtol=1e-12, atol=1e-20)
        x = xn


def test_bf16_lamb_direction_uses_stored_moment():
    """LAMB at step 1 with bias correction and no weight decay: the update is
    lr * ||x|| times the unit direction of m_hat / (sqrt(v_hat) + eps), with
    v_hat = g^2; with a bf16 first moment m_hat is the stored round(0.1 g) / 0.1,
    which differs from g, so the direction must follow it."""
    rng = np.random.default_rng(24)
    shape = (7, 9)
    x = rng.normal(0, 0.02, shape)
    g = rng.normal(0, 1e-2, shape)
    xn, st = oracle.lamb_step_tensor(x, g, oracle.lamb_init_state(shape), {}, 1, exp_avg_bf16=True)
    m_hat = st["exp_avg"] / 0.1
    d = m_hat / (np.abs(g) + 1e-6)
    upd = (x - xn) / (1e-3 * np.linalg.norm(x))
    assert np.allclose(upd, d / np.linalg.norm(d), rtol=1e-12, atol=0)
    d32 = g / (np.abs(g) + 1e-6)
    assert not np.allclose(upd, d32 / np.linalg.norm(d32), rtol=1e-6, atol=0)


# ----------------------------------------------------------------------------- 8-bit first moment

def test_quantize_i8_closed_forms():
    """The ms-swift page's group quantizer on values whose results are fixed by its
    definition: scale = 127 / 127 = 1, codes are the values rounded half to even
    (torch.round), a zero group has scale 0 and codes 0, the last short group of a
    300-element tensor is a group of its own, and the most negative value maps to
    -127 (the absmax scale never needs -128)."""
    q, s = oracle.quantize_i8(np.array([127.0, -127, 63.5, 62.5, 0.5, -0.5, 1.49, -2.5]))
    assert s.tolist() == [1.0]
    assert q.tolist() == [127, -127, 64, 62, 0, 0, 1, -2]
    q, s = oracle.quantize_i8(np.zeros(130))
    assert s.tolist() == [0.0, 0.0] and not q.any()
    x = np.concatenate([np.full(128, 2.0), np.full(128, -0.5), np.linspace(-254.0, 0.0, 44)])
    q, s = oracle.quantize_i8(x)
    f32 = np.float32
    assert s.tolist() == [f32(2.0) / f32(127), f32(0.5) / f32(127), 2.0]
    assert (q[:128] == 127).all() and (q[128:256] == -127).all()
    assert q[256] == -127 and q[-1] == 0
    assert np.array_equal(oracle.dequantize_i8(q, s)[256:], np.rint(x[256:] / 2.0) * 2.0)
    # a non-finite value makes its group read back NaN; other groups are unaffected
    x = np.concatenate([np.ones(128), [np.nan] + [1.0] * 127, [np.inf] + [1.0] * 127])
    q, s = oracle.quantize_i8(x)
    d = oracle.dequantize_i8(q, s)
    assert np.isnan(s[1:]).all() and not q[128:].any() and np.isnan(d[128:]).all()
    assert np.array_equal(d[:128], np.ones(128))


def test_quantize_i8_invariants():
    """On magnitudes spanning 8 decades: every nonzero group reaches |code| = 127,
    dequantized values lie within half a step of the (float32) inputs, the map is
    odd, and scaling by a power of two scales the scales and keeps the codes."""
    rng = np.random.default_rng(31)
    x = rng.normal(size=128 * 40 + 17) * 10.0 ** rng.uniform(-4, 4, 128 * 40 + 17)
    q, s = oracle.quantize_i8(x)
    groups = np.concatenate([q, np.zeros(-q.size % 128, np.int8)]).reshape(-1, 128)
    assert (np.abs(groups.astype(int)).max(axis=1) == 127).all()
    x32 = x.astype(np.float32).astype(np.float64)
    step = np.repeat(s.astype(np.float64), 128)[:x.size]
    assert (np.abs(oracle.dequantize_i8(q, s) - x32) <= 0.5 * step * (1 + 1e-6) + 1e-45).all()
    deq = oracle.dequantize_i8(q, s)   # code x scale is a float32 product, as on the page
    assert np.array_equal(deq.astype(np.float32).astype(np.float64), deq)
    qn, sn = oracle.quantize_i8(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    q8, s8 = oracle.quantize_i8(x * 8.0)
    assert np.array_equal(q8, q) and np.array_equal(s8, s * np.float32(8.0))


@pytest.mark.parametrize("kind", ["adafactor", "came", "lamb"])
def test_i8_first_moment_state(kind):
    """With an 8-bit first moment the state holds int8 codes and one float32 scale
    per 128 values; every nonzero group reaches |code| 127; the fp32-kept
    statistics that depend on G only equal those of fp32 storage."""
    rng = np.random.default_rng(32)
    shape = (6, 256) if kind != "lamb" else (700,)
    hp = {"adafactor": {"beta1": 0.9}, "came": {"lr": 1e-3}, "lamb": {}}[kind]
    x = rng.normal(0, 0.02, shape)
    g = rng.normal(size=shape)
    s8 = oracle.INIT_STATE[kind](shape, hp, exp_avg_i8=True)
    s32 = oracle.INIT_STATE[kind](shape, hp)
    for t in (1, 2):
        x8, s8 = oracle.STEP_TENSOR[kind](x, g, s8, hp, t, exp_avg_i8=True)
        x32, s32 = oracle.STEP_TENSOR[kind](x, g, s32, hp, t)
    assert s8["exp_avg"].dtype == np.int8 and s8["exp_avg_scale"].dtype == np.float32
    assert s8["exp_avg_scale"].size == -(-int(np.prod(shape)) // 128)
    codes = np.concatenate([s8["exp_avg"].reshape(-1), np.zeros(-s8["exp_avg"].size % 128, np.int8)])
    assert (np.abs(codes.reshape(-1, 128).astype(int)).max(axis=1) == 127).all()
    for key in s32:
        if key not in ("exp_avg", "exp_avg_res_row", "exp_avg_res_col"):
            assert np.array_equal(s8[key], s32[key]), key
    m8 = oracle.dequantize_i8(s8["exp_avg"], s8["exp_avg_scale"])
    assert np.max(np.abs(m8 - s32["exp_avg"])) <= 2.5 * np.max(s8["exp_avg_scale"])


@pytest.mark.parametrize("kind", ["adafactor", "came"])
def test_i8_step_is_the_dequantized_moment(kind):
    """Adafactor with beta1 and 1-D CAME step by the first moment itself: with 8-bit
    storage that is the dequantized stored value (codes x scale), not the
    pre-quantization one."""
    rng = np.random.default_rng(33)
    shape = (4, 384) if kind == "adafactor" else (300,)
    hp = {"adafactor": {"beta1": 0.9, "scale_parameter": False}, "came": {"lr": 1e-3}}[kind]
    scale = 1.0 if kind == "adafactor" else 1e-3
    x = rng.normal(0, 0.02, shape)
    st = oracle.INIT_STATE[kind](shape, hp, exp_avg_i8=True)
    for t in (1, 2, 3):
        g = rng.normal(size=shape)
        xn, st = oracle.STEP_TENSOR[kind](x, g, st, hp, t, exp_avg_i8=True)
        m = oracle.dequantize_i8(st["exp_avg"], st["exp_avg_scale"])
        # x - x_new cancels: the error is relative to x, so the bound is set by max |m|
        assert np.allclose((x - xn) / scale, m, rtol=1e-12, atol=1e-12 * np.max(np.abs(m)))
        x = xn


def test_i8_lamb_direction_uses_dequantized_moment():
    """LAMB step 1, bias correction, no decay: the update direction is that of
    m_hat / (|g| + eps) with m_hat = dequantized stored m / 0.1."""
    rng = np.random.default_rng(34)
    x = rng.normal(0, 0.02, 512)
    g = rng.normal(0, 1e-2, 512) * 10.0 ** rng.uniform(-2, 2, 512)
    xn, st = oracle.lamb_step_tensor(x, g, oracle.lamb_init_state((512,), exp_avg_i8=True), {}, 1,
                                     exp_avg_i8=True)
    m_hat = oracle.dequantize_i8(st["exp_avg"], st["exp_avg_scale"]) / 0.1
    d = m_hat / (np.abs(g) + 1e-6)
    upd = (x - xn) / (1e-3 * np.linalg.norm(x))
    assert np.allclose(upd, d / np.linalg.norm(d), rtol=1e-12, atol=1e-15)
