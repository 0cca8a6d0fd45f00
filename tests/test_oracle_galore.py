"""Pins of the GaLore oracle against facts that do not come from the oracle itself.

* Hand-derived worked examples (tests/golden/galore_worked.json): matrices whose
  singular vectors are read off by eye, both projection sides, the canonical sign
  and the rank clamp.
* Known-SVD construction: G = A diag(s) B^T with orthonormal A, B chosen by the
  test; the projector must be B's (m >= n) or A's (m < n) leading columns.
* Library routine: the non-projected path, and a full-rank projection whose basis
  is the identity, must equal torch.optim.AdamW in float64 over several steps.
* Structural facts of the pages: the rank / min(m, n) state compression, the
  refresh schedule (every update_proj_gap steps), the update lying in the
  projector's span, linearity in scale, and oddness in the gradient.
"""
import json
import os

import numpy as np
import pytest

from oracle import galore as ga
from oracle import round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "galore_worked.json")


def _orthonormal(rng, n, k):
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_worked_examples(case):
    x, g = np.array(case["x"], float), np.array(case["g"], float)
    st = ga.galore_init_state(x.shape, case["hp"])
    x_new, new = ga.galore_step_tensor(x, g, st, case["hp"], case["t"],
                                       projector_bf16=case.get("projector_bf16", True))
    np.testing.assert_allclose(new["projector"], np.array(case["projector"]), atol=1e-15, rtol=0)
    np.testing.assert_allclose(x_new, np.array(case["x_new"]), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("shape", [(40, 24), (24, 40), (32, 32)])
def test_projector_is_known_singular_basis(shape):
    rng = np.random.default_rng(1)
    m, n = shape
    k = min(m, n)
    a, b = _orthonormal(rng, m, k), _orthonormal(rng, n, k)
    s = np.linspace(10.0, 1.0, k)
    g = a @ np.diag(s) @ b.T
    r = 7
    u = ga.galore_projector(g, r, projector_bf16=False)
    want = (b if m >= n else a)[:, :r]
    # Same vectors up to sign; the sign is the canonical one.
    np.testing.assert_allclose(np.abs(np.sum(u * want, axis=0)), np.ones(r), atol=1e-10)
    for c in range(r):
        i = np.argmax(np.abs(u[:, c]))
        assert u[i, c] > 0
    np.testing.assert_allclose(u.T @ u, np.eye(r), atol=1e-12)


def test_projector_rounded_to_bf16():
    rng = np.random.default_rng(2)
    g = round_bf16(rng.standard_normal((48, 32)))
    exact = ga.galore_projector(g, 8, projector_bf16=False)
    stored = ga.galore_projector(g, 8)
    np.testing.assert_array_equal(round_bf16(stored), stored)
    # bf16 keeps 8 significant bits: nearest rounding is within 2^-8 relative.
    assert np.all(np.abs(stored - exact) <= 2.0 ** -8 * np.abs(exact))


@pytest.mark.parametrize("shape,rank", [((64, 16), 4), ((16, 64), 4), ((30, 30), 50)])
def test_state_compression(shape, rank):
    """Optimizer state of a projected matrix is rank / min(m, n) of the full one."""
    st = ga.galore_init_state(shape, dict(rank=rank))
    r = min(rank, min(shape))
    assert st["exp_avg"].shape == (max(shape), r)
    assert st["exp_avg_sq"].shape == (max(shape), r)
    assert st["exp_avg"].size / (shape[0] * shape[1]) == pytest.approx(r / min(shape))


def _torch_adamw(x, gs, lr, betas, eps, wd):
    import torch
    p = torch.nn.Parameter(torch.tensor(x, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lr, betas=betas, eps=eps, weight_decay=wd)
    for g in gs:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    return p.detach().numpy()


def test_unprojected_tensor_is_adamw():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(37)
    gs = [rng.standard_normal(37) for _ in range(4)]
    hp = dict(lr=3e-2, betas=(0.8, 0.95), eps=1e-6, weight_decay=0.1)
    st = ga.galore_init_state(x.shape, hp)
    y = x
    for t, g in enumerate(gs, 1):
        y, st = ga.galore_step_tensor(y, g, st, hp, t)
    np.testing.assert_allclose(y, _torch_adamw(x, gs, 3e-2, (0.8, 0.95), 1e-6, 0.1), rtol=1e-12, atol=1e-14)


def test_identity_basis_full_rank_is_adamw():
    """Orthogonal columns with decreasing norms: the full-rank basis is the identity,
    so the projected step is AdamW with lr * scale (and the decay at lr)."""
    rng = np.random.default_rng(4)
    m, n = 9, 4
    hp = dict(lr=1e-2, rank=8, scale=0.5, weight_decay=0.0, update_proj_gap=1)
    x = rng.standard_normal((m, n))
    gs = []
    for _ in range(3):
        g = np.zeros((m, n))
        for j in range(n):  # column j lives on its own rows; norms 4, 3, 2, 1
            g[2 * j:2 * j + 2, j] = (4 - j) * _orthonormal(rng, 2, 1)[:, 0]
        gs.append(g)
    st = ga.galore_init_state(x.shape, hp)
    y = x
    for t, g in enumerate(gs, 1):
        y, st = ga.galore_step_tensor(y, g, st, hp, t)
        np.testing.assert_array_equal(st["projector"], np.eye(n))
    np.testing.assert_allclose(y, _torch_adamw(x, gs, 1e-2 * 0.5, (0.9, 0.999), 1e-8, 0.0),
                               rtol=1e-12, atol=1e-14)


def test_refresh_schedule():
    """The projector comes from the gradient at t = 1, 1 + gap, ...; between those
    steps it is kept. G1 points along column 0, G2 along column 1."""
    x = np.zeros((3, 2))
    g1 = np.array([[3.0, 0], [0, 1], [0, 0]])
    g2 = np.array([[0.0, 0], [0, 5], [0, 0]])
    for gap, refreshed in ((200, False), (1, True)):
        hp = dict(lr=1.0, rank=1, update_proj_gap=gap)
        st = ga.galore_init_state(x.shape, hp)
        y, st = ga.galore_step_tensor(x, g1, st, hp, 1)
        np.testing.assert_array_equal(st["projector"], [[1.0], [0.0]])
        y2, st2 = ga.galore_step_tensor(y, g2, st, hp, 2)
        d = y2 - y
        if refreshed:
            np.testing.assert_array_equal(st2["projector"], [[0.0], [1.0]])
            assert np.all(d[:, 0] == 0) and np.any(d[:, 1] != 0)
        else:
            np.testing.assert_array_equal(st2["projector"], [[1.0], [0.0]])
            assert np.all(d[:, 1] == 0) and np.any(d[:, 0] != 0)
    # t = gap + 1 refreshes again.
    hp = dict(lr=1.0, rank=1, update_proj_gap=3)
    st = ga.galore_init_state(x.shape, hp)
    y, st = ga.galore_step_tensor(x, g1, st, hp, 1)
    for t in (2, 3):
        y, st = ga.galore_step_tensor(y, g2, st, hp, t)
        np.testing.assert_array_equal(st["projector"], [[1.0], [0.0]])
    y, st = ga.galore_step_tensor(y, g2, st, hp, 4)
    np.testing.assert_array_equal(st["projector"], [[0.0], [1.0]])


@pytest.mark.parametrize("shape", [(20, 12), (12, 20)])
def test_update_in_projector_span_and_linear_in_scale(shape):
    rng = np.random.default_rng(5)
    x = rng.standard_normal(shape)
    g = round_bf16(rng.standard_normal(shape))
    deltas = []
    for scale in (0.25, 0.5):
        hp = dict(lr=1e-2, rank=5, scale=scale)
        y, st = ga.galore_step_tensor(x, g, ga.galore_init_state(shape, hp), hp, 1)
        deltas.append(y - x)
    u = st["projector"]
    d = deltas[0]
    # right: rows of the update lie in span(U); left: columns do.
    v = d if shape[0] >= shape[1] else d.T
    coef, *_ = np.linalg.lstsq(u, v.T, rcond=None)
    np.testing.assert_allclose(u @ coef, v.T, atol=1e-14)
    # Differences of O(1) parameters: absolute rounding of 1e-15.
    np.testing.assert_allclose(deltas[1], 2 * deltas[0], rtol=1e-12, atol=1e-15)


def test_update_odd_in_gradient():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((16, 10))
    g = rng.standard_normal((16, 10))
    hp = dict(lr=1e-2, rank=3)
    a, _ = ga.galore_step_tensor(x, g, ga.galore_init_state(x.shape, hp), hp, 1)
    b, _ = ga.galore_step_tensor(x, -g, ga.galore_init_state(x.shape, hp), hp, 1)
    np.testing.assert_allclose(a - x, -(b - x), rtol=1e-12, atol=1e-18)


def test_hparam_validation():
    with pytest.raises(ValueError):
        ga.galore_hparams(dict(proj_type="right"))
    assert ga.galore_hparams(dict(proj_type="reverse_std"))["proj_type"] == "reverse_std"
    with pytest.raises(ValueError):
        ga.galore_hparams(dict(rank=0))
    with pytest.raises(ValueError):
        ga.galore_hparams(dict(update_proj_gap=0))
    assert ga.GALORE_DEFAULTS["rank"] == 256
    assert ga.GALORE_DEFAULTS["update_proj_gap"] == 200
    assert ga.GALORE_DEFAULTS["scale"] == 0.25


@pytest.mark.parametrize("shape,rank", [((64, 16), 4), ((16, 64), 4)])
def test_reverse_std_shapes_and_basis(shape, rank):
    """reverse_std keeps the projector on the longer side: [max][r] basis, [min][r]
    moments; the basis is the leading singular vectors of that side."""
    rng = np.random.default_rng(7)
    m, n = shape
    k = min(m, n)
    a, b = _orthonormal(rng, m, k), _orthonormal(rng, n, k)
    g = a @ np.diag(np.linspace(5.0, 1.0, k)) @ b.T
    hp = dict(rank=rank, proj_type="reverse_std")
    st = ga.galore_init_state(shape, hp)
    assert st["exp_avg"].shape == (min(shape), rank) and st["projector"].shape == (max(shape), rank)
    u = ga.galore_projector(g, rank, projector_bf16=False, proj_type="reverse_std")
    want = (a if m >= n else b)[:, :rank]
    np.testing.assert_allclose(np.abs(np.sum(u * want, axis=0)), np.ones(rank), atol=1e-10)
