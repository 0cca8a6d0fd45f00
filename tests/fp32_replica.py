"""A float32 replica of one optimizer step, for tests of the parity bars only.

Why it exists: the bars in tests/harness.py say how far a correct float32
implementation of the method may land from the fp64 oracle. This module is such
an implementation, written plainly with float32 NumPy arrays (float32 statistics,
float32 per-element arithmetic, fp64 only for the per-tensor scalars, as a GPU
implementation would hold them), so that tests can measure on the CPU what fp32
arithmetic and storage cost against the oracle and set each floor from that.
With ``fault`` it also makes the mistakes a faulty kernel could make, so that
tests can check that the bars reject them.

It follows the same pages as the oracle (Colossal-AI distributed-optimizers
page: "Step 3", the note after "Step 5", the "four optimizers" table, the
DistributedCAME and DistributedLAMB paragraphs) but shares no arithmetic with
it: only the hyperparameter defaults and checks are taken from the oracle. Only
fp32 storage is modelled (16-bit and 8-bit storage have bars of their own).

Faults (``fault``):
  "alpha*1.001"   Adafactor: the step size 0.1% too large
  "kappa*1.001"   Adafactor / CAME: the clip divisor 0.1% too large
  "no_decay"      LAMB: the weight-decay term left out of the direction
  "trust*1.001"   LAMB: the trust ratio 0.1% too large
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

import oracle

F = np.float32


def _f32(a) -> np.ndarray:
    return np.asarray(a, dtype=F)


def _sum64(a: np.ndarray) -> float:
    """A float32 array's sum in fp64 (a per-tensor statistic)."""
    return float(np.sum(a, dtype=np.float64))


def _mean(a: np.ndarray, axis: int) -> np.ndarray:
    """Mean of float32 values along an axis, accumulated in fp64 and rounded to
    float32 (a two-stage GPU reduction: short fp32 partial sums, fp64 across them)."""
    return np.mean(a, axis=axis, dtype=np.float64).astype(F)


def _rsqrt(a: np.ndarray) -> np.ndarray:
    return (F(1.0) / np.sqrt(a)).astype(F)


def adafactor_step(x, g, st: Dict[str, np.ndarray], hp: Optional[dict], t: int, fault: str = ""
                   ) -> Tuple[np.ndarray, Dict[str, np.ndarray], Dict[str, float]]:
    """One Adafactor step in float32: (new parameter, new state, scalars)."""
    h = oracle.adafactor_hparams(hp)
    x, g = _f32(x), _f32(g)
    eps1, eps2 = h["eps"]
    sc: Dict[str, float] = {}
    rho = oracle.adafactor_step_size(h, t)
    sc["rho"] = rho
    alpha = rho
    if h["scale_parameter"]:
        sc["rms_x"] = math.sqrt(_sum64(x * x) / x.size)
        alpha = rho * max(eps2, sc["rms_x"])
    if fault == "alpha*1.001":
        alpha *= 1.001
    sc["alpha"] = alpha
    beta = F(1.0 - math.pow(t, h["decay_rate"]))
    omb = F(math.pow(t, h["decay_rate"]))  # 1 - beta2t formed in fp64, then rounded
    q = g * g + F(eps1)
    new: Dict[str, np.ndarray] = {}
    if x.ndim >= 2:
        row = beta * _f32(st["exp_avg_sq_row"]) + omb * _mean(q, -1)
        col = beta * _f32(st["exp_avg_sq_col"]) + omb * _mean(q, -2)
        new["exp_avg_sq_row"], new["exp_avg_sq_col"] = row, col
        mr = row.mean(axis=-1, dtype=np.float64)  # per matrix
        # U = G rsqrt(C_j) rsqrt(R_i) sqrt(mean R), never materialising the estimate
        rf = (_rsqrt(row) * np.sqrt(mr)[..., None].astype(F))[..., :, None]
        u = (g * _rsqrt(col)[..., None, :]) * rf
    else:
        v = beta * _f32(st["exp_avg_sq"]) + omb * q
        new["exp_avg_sq"] = v
        u = g * _rsqrt(v)
    sc["rms_u"] = math.sqrt(_sum64(u * u) / x.size)
    kappa = max(1.0, sc["rms_u"] / h["clip_threshold"])
    if fault == "kappa*1.001":
        kappa *= 1.001
    sc["kappa"] = kappa
    step = u * F(alpha / kappa)
    if h["beta1"] is not None:
        b1 = F(h["beta1"])
        m = b1 * _f32(st["exp_avg"]) + F(1.0 - h["beta1"]) * step
        new["exp_avg"] = m
        step = m
    decay = F(h["weight_decay"] * alpha)
    x_new = (x - decay * x) - step
    return x_new, new, sc


def came_step(x, g, st: Dict[str, np.ndarray], hp: Optional[dict], t: int, fault: str = ""
              ) -> Tuple[np.ndarray, Dict[str, np.ndarray], Dict[str, float]]:
    """One CAME step in float32."""
    h = oracle.came_hparams(hp)
    x, g = _f32(x), _f32(g)
    eps1, eps2 = h["eps"]
    b1, b2, b3 = (F(b) for b in h["betas"])
    omb1, omb2, omb3 = (F(1.0 - b) for b in h["betas"])  # formed in fp64, then rounded
    lr = F(h["lr"])
    sc: Dict[str, float] = {}
    q = g * g + F(eps1)
    new: Dict[str, np.ndarray] = {}
    fac = x.ndim >= 2
    if fac:
        row = b2 * _f32(st["exp_avg_sq_row"]) + omb2 * _mean(q, -1)
        col = b2 * _f32(st["exp_avg_sq_col"]) + omb2 * _mean(q, -2)
        new["exp_avg_sq_row"], new["exp_avg_sq_col"] = row, col
        mr = row.mean(axis=-1, dtype=np.float64)
        u = (g * _rsqrt(col)[..., None, :]) * (_rsqrt(row) * np.sqrt(mr)[..., None].astype(F))[..., :, None]
    else:
        v = b2 * _f32(st["exp_avg_sq"]) + omb2 * q
        new["exp_avg_sq"] = v
        u = g * _rsqrt(v)
    sc["rms_u"] = math.sqrt(_sum64(u * u) / x.size)
    kappa = max(1.0, sc["rms_u"] / h["clip_threshold"])
    if fault == "kappa*1.001":
        kappa *= 1.001
    sc["kappa"] = kappa
    u = u * F(1.0 / kappa)
    m = b1 * _f32(st["exp_avg"]) + omb1 * u
    new["exp_avg"] = m
    if fac:
        e = (u - m) * (u - m) + F(eps2)
        rrow = b3 * _f32(st["exp_avg_res_row"]) + omb3 * _mean(e, -1)
        rcol = b3 * _f32(st["exp_avg_res_col"]) + omb3 * _mean(e, -2)
        new["exp_avg_res_row"], new["exp_avg_res_col"] = rrow, rcol
        ms = rrow.mean(axis=-1, dtype=np.float64)
        step = (m * _rsqrt(rcol)[..., None, :]) * (_rsqrt(rrow) * np.sqrt(ms)[..., None].astype(F))[..., :, None]
    else:
        step = m
    x_new = (x - (lr * F(h["weight_decay"])) * x) - lr * step
    return x_new, new, sc


def lamb_step(x, g, st: Dict[str, np.ndarray], hp: Optional[dict], t: int, fault: str = ""
              ) -> Tuple[np.ndarray, Dict[str, np.ndarray], Dict[str, float]]:
    """One LAMB step in float32 (the whole tensor is one layer)."""
    h = oracle.lamb_hparams(hp)
    x, g = _f32(x), _f32(g)
    b1, b2 = h["betas"]
    m = F(b1) * _f32(st["exp_avg"]) + F(1 - b1) * g
    v = F(b2) * _f32(st["exp_avg_sq"]) + F(1 - b2) * (g * g)
    bc1 = F(1.0 / (1.0 - b1 ** t)) if h["bias_correction"] else F(1)
    bc2 = F(1.0 / (1.0 - b2 ** t)) if h["bias_correction"] else F(1)
    wd = F(0.0) if fault == "no_decay" else F(h["weight_decay"])
    d = (m * bc1) / (np.sqrt(v * bc2) + F(h["eps"])) + wd * x
    sc = {"x_norm": math.sqrt(_sum64(x * x)), "d_norm": math.sqrt(_sum64(d * d))}
    trust = sc["x_norm"] / sc["d_norm"] if (sc["x_norm"] > 0 and sc["d_norm"] > 0) else 1.0
    sc["trust"] = trust
    if fault == "trust*1.001":
        trust *= 1.001
    x_new = x - F(h["lr"] * trust) * d
    return x_new, {"exp_avg": m, "exp_avg_sq": v}, sc


STEP = {"adafactor": adafactor_step, "came": came_step, "lamb": lamb_step}
