"""Closed forms of the method checked directly on the HIP path, with no oracle in
between (the oracle is held to the same forms in tests/test_oracle_pins.py):

* Adafactor with a rank-1 G^2 (G = diag(a) S diag(b), S random signs): the factored
  estimate R_i C_j / mean(R) is G^2 itself (up to eps1), so U = sign(G), RMS(U) = 1
  and the step is -rho * max(eps2, RMS(X)) * sign(G); with the same G every step
  it stays so (the statistics' EMA sits at its fixed point). Note after "Step 5" of
  the Colossal-AI page (beta2t, RMS clip, scale_parameter) and "Step 3" (the
  factored rule), the BJ north star's "exact recovery when g^2 is rank-1".
* Adafactor clipping: RMS of the applied update over alpha equals the clip
  threshold d when RMS(U) > d ("update RMS <= clip_threshold after clipping").
* CAME with rank-1 G^2 at step 1: U = sign(G), M = (1 - b1) sign(G), the
  instability (U - M)^2 + eps2 = b1^2 + eps2 everywhere, so S = (1 - b3)(b1^2 +
  eps2) and the step is -lr (1 - b1) / sqrt(S) sign(G) (the DistributedCAME
  paragraph's defaults with lr 2e-4: -2.2222e-3 sign(G)).
* LAMB: ||X_new - X|| = lr ||X|| for every tensor (trust ratio ||X|| / ||d||), the
  "four optimizers" table's layer-wise trust ratio.
* Zero gradients: Adafactor's parameter only decays, X (1 - wd alpha).
"""
import numpy as np
import pytest
import torch

from tests.harness import lib_hp, lib_states, lib_step, lib_workspace, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from memory_efficient_optimizers_amd import _lib
    _lib.load()


def _rank1_grad(shape, seed):
    """fp32 G = a_i s_ij b_j with |a|, |b| powers of two in [2^-3, 2^3] and random signs
    s: G is exact in fp32 and G^2 = a_i^2 b_j^2 exactly rank-1 per matrix."""
    rng = np.random.default_rng(seed)
    *lead, h, w = shape
    a = 2.0 ** rng.integers(-3, 4, size=(*lead, h, 1))
    b = 2.0 ** rng.integers(-3, 4, size=(*lead, 1, w))
    s = rng.choice([-1.0, 1.0], size=shape)
    return torch.tensor(a * s * b, dtype=torch.float32, device="cuda")


def _params(shapes, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return [(torch.randn(s, generator=g) * 0.02).to("cuda") for s in shapes]


# (256, 512): row-complete strips; (37, 1001): tiled first pass (odd width);
# (2, 64, 136): batched matrices; (1, 4096) and (64, 1): unit dims
RANK1_SHAPES = [(256, 512), (37, 1001), (2, 64, 136), (1, 4096), (64, 1)]


@pytest.mark.parametrize("carry", [False, True])
def test_adafactor_rank1_step_is_minus_alpha_sign(carry):
    from memory_efficient_optimizers_amd import _lib
    hp = {}
    ps = _params(RANK1_SHAPES, 1)
    gs = [_rank1_grad(s, 10 + k) for k, s in enumerate(RANK1_SHAPES)]
    sts = lib_states("adafactor", ps, hp)
    if carry:
        for st in sts:
            st["param_sumsq"] = torch.zeros(1, device="cuda")
    hps = lib_hp("adafactor", hp)
    ws = lib_workspace("adafactor", ps, gs)
    for t in range(1, 4):
        x0 = [to64(p) for p in ps]
        if carry:
            _lib.meo_adafactor_step_carry(hps, t, ps, gs, sts, t > 1, ws)
        else:
            lib_step("adafactor", hps, t, ps, gs, sts, ws)
        torch.cuda.synchronize()
        rho = min(1e-2, 1.0 / np.sqrt(t))
        for k, (x, p, g) in enumerate(zip(x0, ps, gs)):
            alpha = rho * max(1e-3, float(np.sqrt(np.mean(x * x))))
            step = (to64(p) - x) / alpha
            err = float(np.max(np.abs(step + np.sign(to64(g)))))
            # fp32: the new X is rounded at |X| ~ 0.02-0.1, a step of 2e-4 to 1e-3
            assert err <= 2e-3, (t, RANK1_SHAPES[k], err)
            # and the update direction itself is exact to fp32 rounding of X
            assert np.array_equal(np.sign(to64(p) - x), -np.sign(to64(g))), (t, RANK1_SHAPES[k])


@pytest.mark.parametrize("clip", [0.1, 0.5])
def test_adafactor_clipped_update_rms_is_the_threshold(clip):
    """Random G: RMS(U) is about 1 (U = G / sqrt(V_hat), V_hat ~ E[G^2]), above the
    threshold, so the applied update has RMS alpha * d exactly (beta1 None, wd 0)."""
    hp = {"clip_threshold": clip}
    shapes = [(256, 512), (37, 1001), (5000,)]
    ps = _params(shapes, 2)
    g = torch.Generator(device="cpu").manual_seed(3)
    gs = [torch.randn(s, generator=g).to("cuda") for s in shapes]
    sts = lib_states("adafactor", ps, hp)
    hps = lib_hp("adafactor", hp)
    x0 = [to64(p) for p in ps]
    lib_step("adafactor", hps, 1, ps, gs, sts, lib_workspace("adafactor", ps, gs))
    torch.cuda.synchronize()
    for k, (x, p) in enumerate(zip(x0, ps)):
        alpha = 1e-2 * max(1e-3, float(np.sqrt(np.mean(x * x))))
        d = to64(p) - x
        rms = float(np.sqrt(np.mean(d * d))) / alpha
        # fp32 rounding of X (|X| ~ 0.02) against steps of alpha * clip ~ 2e-5..1e-4
        assert abs(rms - clip) <= 2e-3 * clip, (shapes[k], rms)


def test_came_rank1_step1_closed_form():
    hp = {"lr": 2e-4}
    b1, b3, eps2 = 0.9, 0.9999, 1e-16
    want = 2e-4 * (1 - b1) / np.sqrt((1 - b3) * (b1 * b1 + eps2))
    assert abs(want - 2.2222e-3) < 1e-7
    shapes = [(256, 512), (37, 1001), (2, 64, 136)]
    ps = _params(shapes, 4)
    gs = [_rank1_grad(s, 20 + k) for k, s in enumerate(shapes)]
    sts = lib_states("came", ps, hp)
    x0 = [to64(p) for p in ps]
    lib_step("came", lib_hp("came", hp), 1, ps, gs, sts, lib_workspace("came", ps, gs))
    torch.cuda.synchronize()
    for k, (x, p, g) in enumerate(zip(x0, ps, gs)):
        step = to64(p) - x
        err = float(np.max(np.abs(step + want * np.sign(to64(g))))) / want
        assert err <= 1e-3, (shapes[k], err)


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_lamb_update_norm_is_lr_times_param_norm(wd):
    hp = {"lr": 1e-3, "weight_decay": wd}
    shapes = [(1024, 1024), (4096,), (300, 77)]
    ps = _params(shapes, 5)
    g = torch.Generator(device="cpu").manual_seed(6)
    sts = lib_states("lamb", ps, hp)
    hps = lib_hp("lamb", hp)
    for t in range(1, 4):
        gs = [(torch.randn(s, generator=g) * 1e-2).to("cuda") for s in shapes]
        x0 = [to64(p) for p in ps]
        lib_step("lamb", hps, t, ps, gs, sts, lib_workspace("lamb", ps, gs))
        torch.cuda.synchronize()
        for k, (x, p) in enumerate(zip(x0, ps)):
            dn = float(np.linalg.norm(to64(p) - x))
            xn = float(np.linalg.norm(x))
            # ||dX|| = 1e-3 ||X||; fp32 rounding of X adds ~6e-8 |X| per element
            assert abs(dn - 1e-3 * xn) <= 1e-4 * 1e-3 * xn, (t, shapes[k], dn / xn)


def test_adafactor_zero_gradient_is_pure_decay():
    hp = {"weight_decay": 0.1, "beta1": 0.9}
    shapes = [(256, 512), (37, 1001), (5000,)]
    ps = _params(shapes, 7)
    gs = [torch.zeros(s, device="cuda") for s in shapes]
    sts = lib_states("adafactor", ps, hp)
    x0 = [to64(p) for p in ps]
    lib_step("adafactor", lib_hp("adafactor", hp), 1, ps, gs, sts, lib_workspace("adafactor", ps, gs))
    torch.cuda.synchronize()
    for k, (x, p) in enumerate(zip(x0, ps)):
        alpha = 1e-2 * max(1e-3, float(np.sqrt(np.mean(x * x))))
        want = x * (1.0 - 0.1 * alpha)
        err = float(np.max(np.abs(to64(p) - want) / np.maximum(np.abs(want), 1e-30)))
        assert err <= 2 ** -23, (shapes[k], err)
        assert np.all(to64(sts[k]["exp_avg"]) == 0.0)
