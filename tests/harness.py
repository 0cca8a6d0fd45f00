"""Shared helpers of the GPU parity tests: run the library and the oracle on the
same seeded inputs and compare.

Tolerance (the bar is a relative error of 1e-5 on every fp32 output tensor):

* positive statistics (``exp_avg_sq*``, ``exp_avg_res*``): plain elementwise
  relative error, max_i |a_i - b_i| / |b_i|. Every term of these averages is
  positive, so nothing cancels and each element must hold 1e-5 on its own.
* signed outputs (the parameter and ``exp_avg``): max_i |a_i - b_i| /
  max(|b_i|, RMS(b)). These are sums of terms of both signs (an EMA of the
  update, a parameter minus its step) and cross zero; fp32 storage and
  arithmetic leave an absolute error of a few ulps of the *terms*, which are of
  the order of the tensor's RMS, so near a zero crossing the error is measured
  against that scale. (A plain fp32 run of the oracle's own arithmetic reaches
  8e-5 if the floor is 1e-2 * RMS instead, and ~1e-6 with this one.)

Here a = the library's fp32 result and b = the oracle's fp64 result.
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


POSITIVE_KEYS = ("exp_avg_sq_row", "exp_avg_sq_col", "exp_avg_sq", "exp_avg_res_row", "exp_avg_res_col")


def floored_rel_err(a, b, floor: float = 1.0) -> float:
    """max_i |a_i - b_i| / max(|b_i|, floor * RMS(b)) (a zero denominator counts as 1)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    if b.size == 0:
        return 0.0
    r = math.sqrt(float(np.mean(b * b))) if floor > 0 else 0.0
    den = np.maximum(np.abs(b), floor * r)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(a - b) / den))


def output_err(key: str, a, b) -> float:
    """The error of one output tensor under the rule above."""
    return floored_rel_err(a, b, 0.0 if key in POSITIVE_KEYS else 1.0)


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
            out[f"{spec.name}:param"] = output_err("param", to64(self.params[k]), self.ox[k])
            for key, arr in self.ost[k].items():
                out[f"{spec.name}:{key}"] = output_err(key, to64(self.states[k][key]), arr)
        return out

    def worst(self):
        errs = self.errors()
        name = max(errs, key=errs.get)
        return errs[name], name
