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

16-bit storage. Both sides round a bf16-stored value (parameter, ``exp_avg``)
to the nearest bf16, but from different pre-rounding values: the library's carries
fp32 arithmetic error (a few fp32 ulps, 2^-24 each, against a bf16 spacing of
2^-8), so where the exact value lies that close to a midpoint between two bf16
values (roughly 1e-4 of the elements per step) the two sides keep neighbouring
bf16 values. Both are correct roundings of the method's value; no oracle can
replay the library's fp32 rounding decisions bit for bit. Such outputs, and every
fp32 output computed from a bf16-stored first moment (CAME's confidence
statistics; a fp32 parameter stepped by a bf16 first moment), are judged by:

* elementwise error (rule above) <= 2e-2, the bar for bf16-cast outputs; and
* at most 1% of the elements (plus 4, for tiny tensors) above the fp32 bar 1e-5.

A systematic fault (truncation instead of rounding to nearest, a wrong dtype, a
mis-rounded tail) moves most elements and fails the second rule.

8-bit first moment. The same near-tie disagreement can move an int8 code by one
step (code = m / scale rounded, decided on each side's own m). Such a step is
1/127 of its group's largest magnitude; it then decays with beta1 in later
steps, but the group's scale may shrink meanwhile, so in codes it can span more
than one step. The first moment is therefore judged on its dequantized values
(code x scale), relative to its group's largest magnitude (127 x scale):
* every value within 2e-2 of it (one code step is 0.79%); and
* at most 1% (+4) of the codes differ.
The scales (max |m| / 127 per group), the parameter and CAME's confidence
statistics follow the 16-bit rules above.
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np
import torch

import oracle
import workloads
from memory_efficient_optimizers_amd import _lib, moment_dtype

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
MAX_SHARE = 1e-2   # share of elements allowed above TOL_F32 where bf16 rounding decides
MAX_EXTRA = 4


POSITIVE_KEYS = ("exp_avg_sq_row", "exp_avg_sq_col", "exp_avg_sq", "exp_avg_res_row", "exp_avg_res_col")


def floored_rel_errs(a, b, floor: float = 1.0) -> np.ndarray:
    """|a_i - b_i| / max(|b_i|, floor * RMS(b)) per element (a zero denominator counts as 1)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    if b.size == 0:
        return np.zeros(0)
    r = math.sqrt(float(np.mean(b * b))) if floor > 0 else 0.0
    den = np.maximum(np.abs(b), floor * r)
    den = np.where(den > 0, den, 1.0)
    return np.abs(a - b) / den


def floored_rel_err(a, b, floor: float = 1.0) -> float:
    """max_i |a_i - b_i| / max(|b_i|, floor * RMS(b))."""
    e = floored_rel_errs(a, b, floor)
    return float(np.max(e)) if e.size else 0.0


def output_errs(key: str, a, b) -> np.ndarray:
    return floored_rel_errs(a, b, 0.0 if key in POSITIVE_KEYS else 1.0)


def output_err(key: str, a, b) -> float:
    """The error of one output tensor under the rule above."""
    return floored_rel_err(a, b, 0.0 if key in POSITIVE_KEYS else 1.0)


def storage_of_tensor(param: torch.Tensor, state: Dict[str, torch.Tensor]) -> dict:
    """The oracle's storage flags for one tensor, read from the library's buffers."""
    m = state.get("exp_avg")
    return dict(param_bf16=param.dtype == torch.bfloat16,
                exp_avg_bf16=m is not None and m.dtype == torch.bfloat16,
                exp_avg_i8=m is not None and m.dtype == torch.int8)


def bar_kind(opt: str, hp: dict, storage: dict, key: str) -> str:
    """"f32": held to 1e-5; "rounded": decided by a storage rounding (stored in
    bf16, or computed from a bf16 or 8-bit first moment), held to the 16-bit rules
    above; "codes": int8 codes of an 8-bit first moment."""
    pb, mb, mi = (storage.get(k, False) for k in ("param_bf16", "exp_avg_bf16", "exp_avg_i8"))
    has_m = opt != "adafactor" or hp.get("beta1") is not None
    if key == "param":
        return "rounded" if pb or ((mb or mi) and has_m) else "f32"
    if key == "exp_avg":
        return "codes" if mi else ("rounded" if mb else "f32")
    if key == "exp_avg_scale":
        return "rounded"
    if key in ("exp_avg_res_row", "exp_avg_res_col"):
        return "rounded" if mb or mi else "f32"
    return "f32"


def check_bar(kind: str, key: str, a, b):
    """(ok, max error, elements off the fp32 bar (or codes that differ), elements)
    of one output under its bar. For "codes", a and b are (codes, scales) pairs."""
    if kind == "codes":
        (ca, sa), (cb, sb) = a, b
        ca, cb = np.asarray(ca).reshape(-1), np.asarray(cb).reshape(-1)
        da = oracle.dequantize_i8(ca, np.asarray(sa, dtype=np.float32))
        db = oracle.dequantize_i8(cb, np.asarray(sb, dtype=np.float32))
        amax = 127.0 * np.repeat(np.asarray(sb, dtype=np.float64), oracle.I8_GROUP)[:cb.size]
        den = np.maximum(np.abs(db), amax)
        den = np.where(den > 0, den, 1.0)
        e = np.abs(da - db) / den
        err = float(np.max(e)) if e.size else 0.0
        over = int(np.count_nonzero(ca.astype(np.int64) != cb.astype(np.int64)))
        return err <= TOL_BF16 and over <= MAX_SHARE * e.size + MAX_EXTRA, err, over, e.size
    e = output_errs(key, a, b)
    err = float(np.max(e)) if e.size else 0.0
    over = int(np.count_nonzero(e > TOL_F32))
    if kind == "f32":
        return err <= TOL_F32, err, over, e.size
    return err <= TOL_BF16 and over <= MAX_SHARE * e.size + MAX_EXTRA, err, over, e.size


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_hp(wl: workloads.Workload) -> dict:
    return dict(wl.hparams)


def lib_hp(opt: str, hp: dict):
    return {"adafactor": _lib.adafactor_hparams, "came": _lib.came_hparams,
            "lamb": _lib.lamb_hparams}[opt](**hp)


def outputs(param: torch.Tensor, state: Dict[str, torch.Tensor], ox, ost) -> list:
    """(key, library value, oracle value) of every output of one tensor; an 8-bit
    first moment is one output made of its codes and scales."""
    out = [("param", to64(param), ox)]
    i8 = "exp_avg_scale" in ost
    for key, ref in ost.items():
        if key == "exp_avg" and i8:
            out.append((key, (state[key].cpu().numpy(), state["exp_avg_scale"].cpu().numpy()),
                        (ref, ost["exp_avg_scale"])))
        else:
            out.append((key, to64(state[key]), ref))
    return out


def lib_states(opt: str, params, hp: dict, state_dtype=torch.float32, min_8bit_size: int = 4096
               ) -> List[Dict[str, torch.Tensor]]:
    """Zero library states; an int8 request applies where moment_dtype allows it."""
    beta1 = hp.get("beta1") is not None
    return [_lib.init_state(opt, p, beta1=beta1,
                            state_dtype=moment_dtype(opt, p.shape, state_dtype, p.dtype, min_8bit_size))
            for p in params]


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

    def __init__(self, wl: workloads.Workload, device="cuda", hp: dict = None, min_8bit_size: int = 4096,
                 carry: bool = False):
        """carry (Adafactor): step through meo_adafactor_step_carry, taking RMS(X)
        from the carried sums from the second step on (``carry_valid``)."""
        self.wl = wl
        self.opt = wl.optimizer
        self.hp = dict(wl.hparams if hp is None else hp)
        self.device = device
        self.params = workloads.init_params(wl, device)
        self.scales = workloads.grad_scales(wl, device)
        self.states = lib_states(self.opt, self.params, self.hp, wl.state_dtype, min_8bit_size)
        self.storage = [storage_of_tensor(p, st) for p, st in zip(self.params, self.states)]
        self.hps = lib_hp(self.opt, self.hp)
        self.ox = [to64(p) for p in self.params]
        self.ost = [oracle.INIT_STATE[self.opt](tuple(p.shape), self.hp, exp_avg_i8=s["exp_avg_i8"])
                    for p, s in zip(self.params, self.storage)]
        self.ws = None
        self.t = 0
        self.carry = carry
        self.carry_valid = False
        if carry:
            assert self.opt == "adafactor"
            for st, p in zip(self.states, self.params):
                st["param_sumsq"] = torch.zeros(1, dtype=torch.float32, device=p.device)

    def grads(self, s: int):
        return workloads.grads(self.wl, s, self.scales, self.device)

    def step(self, grads=None, oracle_too=True):
        self.t += 1
        if grads is None:
            grads = self.grads(self.t - 1)
        if self.ws is None:
            self.ws = lib_workspace(self.opt, self.params, grads)
        if self.carry:
            _lib.meo_adafactor_step_carry(self.hps, self.t, self.params, grads, self.states, self.carry_valid,
                                          self.ws)
            self.carry_valid = True
        else:
            lib_step(self.opt, self.hps, self.t, self.params, grads, self.states, self.ws)
        if oracle_too:
            gs = [to64(g) for g in grads]
            for k in range(len(gs)):
                self.ox[k], self.ost[k] = oracle.STEP_TENSOR[self.opt](self.ox[k], gs[k], self.ost[k], self.hp,
                                                                       self.t, **self.storage[k])
        return grads

    def verdicts(self) -> Dict[str, tuple]:
        """Per output "<tensor>:<key>": (ok, max error, elements above 1e-5, elements, bar kind)."""
        torch.cuda.synchronize()
        out = {}
        for k, spec in enumerate(self.wl.specs):
            for key, lib, ref in outputs(self.params[k], self.states[k], self.ox[k], self.ost[k]):
                kind = bar_kind(self.opt, self.hp, self.storage[k], key)
                out[f"{spec.name}:{key}"] = check_bar(kind, key, lib, ref) + (kind,)
        return out

    def sumsq_errors(self) -> Dict[str, float]:
        """Carry runs: relative error of each tensor's carried sum of squares against
        the sum of squares of the oracle's parameter (by definition, in fp64)."""
        torch.cuda.synchronize()
        out = {}
        for k, spec in enumerate(self.wl.specs):
            if self.params[k].numel() == 0:
                continue
            want = float(np.sum(np.square(self.ox[k])))
            got = float(self.states[k]["param_sumsq"].item())
            out[spec.name] = abs(got - want) / want if want > 0 else abs(got)
        return out

    def errors(self) -> Dict[str, float]:
        return {k: v[1] for k, v in self.verdicts().items()}

    def check(self, label: str = "") -> float:
        """Asserts every output meets its bar; prints and returns the worst fp32-bar error."""
        v = self.verdicts()
        bad = {k: x for k, x in v.items() if not x[0]}
        f32 = {k: x[1] for k, x in v.items() if x[4] == "f32"}
        b16 = {k: x for k, x in v.items() if x[4] != "f32"}
        msg = f"  {self.wl.name} {label}"
        if f32:
            w = max(f32, key=f32.get)
            msg += f" worst fp32 {f32[w]:.3e} at {w}"
        if b16:
            w = max(b16, key=lambda k: b16[k][1])
            share = max(x[2] / max(x[3], 1) for x in b16.values())
            msg += f"; storage-decided worst {b16[w][1]:.3e} at {w}, max share off {share:.2e}"
        print(msg, flush=True)
        assert not bad, f"{label}: " + ", ".join(
            f"{k} ({x[4]} bar): err {x[1]:.3e}, {x[2]}/{x[3]} above 1e-5" for k, x in bad.items())
        return max(f32.values()) if f32 else 0.0
