"""Shared helpers of the GPU parity tests: run the library and the oracle on the
same seeded inputs and compare.

Tolerance: for every output tensor (parameter and each state),
    err = max_i |a_i - b_i| / max(|b_i|, 1e-2 * RMS(b))
with a = the library's fp32 result and b = the oracle's fp64 result; the bar is
1e-5 for fp32 outputs. The floor 1e-2 * RMS(b) only matters where a value
crosses zero by cancellation (a parameter or first moment near 0), where an
elementwise relative error has no meaning.
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np
import torch

import oracle
import workloads
from memory_efficient_optimizers_amd import _lib

TOL_F32 = 1e-5


def floored_rel_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    if b.size == 0:
        return 0.0
    r = math.sqrt(float(np.mean(b * b)))
    den = np.maximum(np.abs(b), 1e-2 * r)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(a - b) / den))


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_hp(wl: workloads.Workload) -> dict:
    return dict(wl.hparams)


def lib_hp(opt: str, hp: dict):
    return {"adafactor": _lib.adafactor_hparams, "came": _lib.came_hparams,
            "lamb": _lib.lamb_hparams}[opt](**hp)


def lib_states(opt: str, params, hp: dict) -> List[Dict[str, torch.Tensor]]:
    beta1 = hp.get("beta1") is not None
    return [_lib.init_state(opt, p, beta1=beta1) for p in params]


def lib_step(opt, hp_struct, t, params, grads, states, ws, stream=None):
    fn = {"adafactor": _lib.meo_adafactor_step, "came": _lib.meo_came_step,
          "lamb": _lib.meo_lamb_step}[opt]
    fn(hp_struct, t, params, grads, states, ws, stream)


def lib_workspace(opt, params, grads):
    fn = {"adafactor": _lib.meo_adafactor_workspace_size, "came": _lib.meo_came_workspace_size,
          "lamb": _lib.meo_lamb_workspace_size}[opt]
    return _lib.workspace(fn(params, grads), params[0].device)


class Run:
    """The library and the oracle side by side over a workload."""

    def __init__(self, wl: workloads.Workload, device="cuda", hp: dict = None):
        self.wl = wl
        self.opt = wl.optimizer
        self.hp = dict(wl.hparams if hp is None else hp)
        self.device = device
        self.params = workloads.init_params(wl, device)
        self.scales = workloads.grad_scales(wl, device)
        self.states = lib_states(self.opt, self.params, self.hp)
        self.hps = lib_hp(self.opt, self.hp)
        self.ox = [to64(p) for p in self.params]
        self.ost = [oracle.INIT_STATE[self.opt](tuple(p.shape), self.hp) for p in self.params]
        self.ws = None
        self.t = 0

    def grads(self, s: int):
        return workloads.grads(self.wl, s, self.scales, self.device)

    def step(self, grads=None, oracle_too=True):
        self.t += 1
        if grads is None:
            grads = self.grads(self.t - 1)
        if self.ws is None:
            self.ws = lib_workspace(self.opt, self.params, grads)
        lib_step(self.opt, self.hps, self.t, self.params, grads, self.states, self.ws)
        if oracle_too:
            gs = [to64(g) for g in grads]
            self.ox, self.ost = oracle.STEP[self.opt](self.ox, gs, self.ost, self.hp, self.t)
        return grads

    def errors(self) -> Dict[str, float]:
        torch.cuda.synchronize()
        out = {}
        for k, spec in enumerate(self.wl.specs):
            out[f"{spec.name}:param"] = floored_rel_err(to64(self.params[k]), self.ox[k])
            for key, arr in self.ost[k].items():
                out[f"{spec.name}:{key}"] = floored_rel_err(to64(self.states[k][key]), arr)
        return out

    def worst(self):
        errs = self.errors()
        name = max(errs, key=errs.get)
        return errs[name], name
