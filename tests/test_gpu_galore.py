"""GPU parity of the GaLore step (meo_galore_step through the C ABI) against the
fp64 oracle (oracle/galore.py), on seeded inputs from workloads.galore_inputs.

Steps here are not refresh steps (t - 1 is not a multiple of update_proj_gap), so
the projector is an input: a seeded random orthonormal basis rounded to bf16,
identical on both sides. Bars:

* exp_avg, exp_avg_sq and an fp32 parameter: the fp32 bar of tests/harness.py
  (1e-5; signed outputs floored at their RMS). The low-rank gradient is a sum of
  d products of bf16 values, exact in fp32, accumulated in fp32 by the matrix
  cores: about sqrt(d / 16) roundings of 2^-24 each, far below the bar.
* The update x_new - x of an fp32 parameter, floored at its RMS: 1e-4. The update
  is about lr * scale / |x| ~ 1e-2 of the parameter here, so the fp32 rounding of
  x_new alone contributes up to 2^-24 / 1e-2 ~ 6e-6; the low-rank direction enters
  the back-projection as two bf16 planes whose sum carries it to 2^-17 relative.
* A bf16 parameter: the 16-bit bar ("rounded").
* The projector and its transpose are not written on such steps (bit-exact).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import galore as ga
from memory_efficient_optimizers_amd import _lib
from tests.harness import floored_rel_err, judge, to64

pytestmark = pytest.mark.gpu

TOL_UPDATE = 1e-4


def run_case(shapes, rank, t=5, hp=None, param_dtype=torch.float32, seed=0, check_update=True):
    dev = "cuda"
    hp = dict(dict(lr=0.05, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, scale=0.25), **(hp or {}))
    hpo = dict(hp, rank=rank)
    params, grads, states = workloads.galore_inputs(shapes, rank, seed, param_dtype=param_dtype, device=dev)
    x0 = [to64(p) for p in params]
    g0 = [to64(g) for g in grads]
    s0 = [{k: to64(v) for k, v in s.items() if k != "projector_t"} for s in states]
    pt0 = [s["projector_t"].clone() if "projector_t" in s else None for s in states]
    h = _lib.galore_hparams(**hpo)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print(f"galore step: shapes={shapes} rank={rank} t={t} param={param_dtype}", flush=True)
    _lib.meo_galore_step(h, t, params, grads, states, ws)
    torch.cuda.synchronize()
    bad = []
    for k, shape in enumerate(shapes):
        if int(np.prod(shape)) == 0:
            continue
        want_x, want_s = ga.galore_step_tensor(x0[k], g0[k], s0[k], hpo, t,
                                               param_bf16=param_dtype == torch.bfloat16)
        got_x = to64(params[k])
        kind = "f32" if param_dtype == torch.float32 else "rounded"
        checks = [(kind, "param", got_x, want_x),
                  ("f32", "exp_avg", to64(states[k]["exp_avg"]), want_s["exp_avg"]),
                  ("f32", "exp_avg_sq", to64(states[k]["exp_avg_sq"]), want_s["exp_avg_sq"])]
        for kd, key, a, b in checks:
            ok, err, over, n = judge(kd, key, a, b)
            if not ok:
                bad.append(f"tensor {k} {shape} {key}: err {err:.3g} ({over}/{n} above 1e-5)")
        if param_dtype == torch.float32 and check_update:
            e = floored_rel_err(got_x - x0[k], want_x - x0[k])
            if e > TOL_UPDATE:
                bad.append(f"tensor {k} {shape} update: err {e:.3g}")
        if "projector" in states[k]:
            assert torch.equal(states[k]["projector"].cpu(), torch.from_numpy(s0[k]["projector"]).to(torch.bfloat16))
            assert torch.equal(states[k]["projector_t"], pt0[k])
    assert not bad, "; ".join(bad)
    return params, states


@pytest.mark.parametrize("shape,rank", [
    ((256, 128), 32),     # m >= n, whole tiles, one active wave
    ((128, 320), 64),     # m < n (transposed gradient tile)
    ((300, 136), 40),     # ragged rows, r not a multiple of 32
    ((72, 333), 24),      # ragged, odd columns: element-wise loads
    ((200, 96), 13),      # r not a multiple of 8
    ((40, 24), 256),      # rank clamped to min(m, n)
    ((512, 384), 256),    # full rank-256 tile, several contraction blocks
    ((300, 600), 256),    # m < n at rank 256
    ((64, 64), 64),       # square: projects the columns' space
    ((1, 48), 8),         # a single row: rank 1
])
def test_step_shapes(shape, rank):
    run_case([shape], rank)


@pytest.mark.parametrize("shape", [(256, 200), (96, 400)])
def test_step_bf16_param(shape):
    run_case([shape], 64, param_dtype=torch.bfloat16)


def test_step_weight_decay_and_late_step():
    run_case([(260, 130), (130, 260)], 48, t=187, hp=dict(weight_decay=0.1, lr=0.02, betas=(0.8, 0.95)))


def test_step_mixed_list():
    """2-D tensors of both sides with 1-D, 3-D (flat AdamW) and empty tensors."""
    run_case([(192, 64), (0, 5), (64, 500), (777,), (3, 5, 7), (1,), (8, 8)], 32, seed=3)


def test_step_llama_sized():
    """One Llama-7B-shaped MLP pair at rank 256 (rows of 4096 and 11008)."""
    run_case([(1024, 4096), (4096, 1024)], 256, seed=4)


def test_list_equals_singles():
    """Every block reads only its own tensor: a list step equals per-tensor steps bitwise."""
    shapes = [(200, 72), (72, 300), (129,)]
    dev = "cuda"
    h = _lib.galore_hparams(lr=0.05, rank=32)
    p1, g1, s1 = workloads.galore_inputs(shapes, 32, 9, device=dev)
    p2, g2, s2 = workloads.galore_inputs(shapes, 32, 9, device=dev)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, p1, g1), dev)
    _lib.meo_galore_step(h, 3, p1, g1, s1, ws)
    for k in range(len(shapes)):
        wk = _lib.workspace(_lib.meo_galore_workspace_size(h, [p2[k]], [g2[k]]), dev)
        _lib.meo_galore_step(h, 3, [p2[k]], [g2[k]], [s2[k]], wk)
    torch.cuda.synchronize()
    for k in range(len(shapes)):
        assert torch.equal(p1[k], p2[k])
        for key in s1[k]:
            assert torch.equal(s1[k][key], s2[k][key])
