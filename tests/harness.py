"""Shared helpers of the GPU parity tests: run the library and the oracle on the
same seeded inputs and compare.

Tolerance (the bar is a relative error of 1e-5 on every fp32 output tensor).
Here a = the library's fp32 result, b = the oracle's fp64 result, x0 = the
tensor's initial parameter.

* positive statistics (``exp_avg_sq*``, ``exp_avg_res*``): plain elementwise
  relative error, max_i |a_i - b_i| / |b_i|. Every term of these averages is
  positive, so nothing cancels and each element must hold 1e-5 on its own.
* the first moment ``exp_avg``: max_i |a_i - b_i| / max(|b_i|, 0.1 RMS(b), t_i),
  t_i = |beta1 m_prev_i| + |b_i - beta1 m_prev_i| the magnitudes of the two terms
  of the average b = beta1 m_prev + (1 - beta1) u (m_prev the oracle's value
  before the step). It is an average of updates of both signs and crosses zero;
  there its error is a few fp32 ulps of its *terms* plus the update's own relative
  error, so it is measured against the terms, and against a tenth of the tensor's
  scale (where gradients span many decades, the terms of one element can lie far
  above the tensor's RMS, so both are needed).
* the parameter: max_i |a_i - b_i| / max(|b_i|, 1e-2 RMS(b), RMS(b - x0)). The
  parameter is its start minus a sum of steps: its error is the storage rounding
  (relative to |b_i|) plus the steps' relative errors, which add up on the scale
  of the accumulated change b - x0. For a weight that change is ~1e-2 of the
  weight; a parameter that starts at zero (a bias) *is* its accumulated change and
  can cancel to near zero, where only that scale applies. GaLore's update has a
  bar of its own, 1e-4 (bf16 matrix cores, N in two bf16 planes), so its
  parameter takes 10 RMS(b - x0) there (``step_tol``).
* the step itself, dX = X_new - X_old on each side (fp32 parameters; the
  library's from its own stored values, the oracle's in fp64):
  max_i max(0, |dXa_i - dXb_i| - s_i) / max(|dXb_i|, 0.1 RMS(dXb)) <= 1e-5, where
  s_i is one fp32 spacing at max(|X_old_i|, |X_new_i|), the library's value: the
  store's rounding and one rounding at the parameter's magnitude inside the
  update (x - decay x) are forgiven, nothing else is. With that slack taken off,
  the normwise error ||dXa - dXb|| / ||dXb|| must be <= 1e-6: a fault that moves
  every element a little (a dropped term, a scalar off by 0.1%) fails here.
* the per-tensor scalars the library leaves in its workspace (step size alpha,
  clip divisor kappa, RMS(U), RMS(X); LAMB's ||X||, ||d|| and trust ratio):
  relative error <= max(1e-6, 1e-5 / sqrt(n)) for a tensor of n elements (a norm
  averages its elements' errors; 1e-6 from n = 100 on), and 1e-4 for those
  computed from a bf16 or 8-bit stored state (TOL_SCALAR_STORAGE).
* beside each bar the unfloored normwise error ||a - b|| / ||b|| is reported.

Evidence for the floors: tests/test_tolerance_floors.py runs a plain float32
replica of the method (tests/fp32_replica.py) against the oracle over 10 chained
steps with the configurations' gradient scales; it lands at about 1e-6 for the
parameter and 2e-6 to 5e-6 for exp_avg and dX under these floors, and shows that
S23's 1e-2 RMS(b) floor alone is not reachable by fp32 arithmetic for a
zero-initialised bias or for CAME's parameter (1e-5 to 3e-5), which is why the
parameter's floor includes RMS(b - x0).

16-bit storage. Both sides round a bf16-stored value (parameter, ``exp_avg``)
to the nearest bf16, but from different pre-rounding values: the library's carries
fp32 arithmetic error (a few fp32 ulps, 2^-24 each, against a bf16 spacing of
2^-8), so where the exact value lies that close to a midpoint between two bf16
values (roughly 1e-4 of the elements per step) the two sides keep neighbouring
bf16 values. Both are correct roundings of the method's value; no oracle can
replay the library's fp32 rounding decisions bit for bit. Such outputs, and every
fp32 output computed from a bf16-stored first moment (CAME's confidence
statistics; a fp32 parameter stepped by a bf16 first moment), are judged by:

* elementwise error, max_i |a_i - b_i| / max(|b_i|, RMS(b)) for signed outputs,
  <= 2e-2, the bar for bf16-cast outputs; and
* at most 1% of the elements (plus 4, for tiny tensors) above the fp32 bar 1e-5.

A systematic fault (truncation instead of rounding to nearest, a wrong dtype, a
mis-rounded tail) moves most elements and fails the second rule. The step dX is
held to the same two rules (floored at RMS(dX)) where the parameter is fp32 and
the first moment bf16 (dX then follows the stored moment); a bf16 parameter's dX
is not separable from its storage rounding and is not checked on its own. LAMB's
step is its per-tensor trust ratio times the direction (the DistributedLAMB
paragraph: a layer-wise ratio), so one near-tie element of the stored moment moves
the ratio, and with it every element's step, by the same factor (3e-5 measured on a
256-element tensor): there the oracle's step is rescaled by the library's ratio over
its own before the two rules, which then judge the direction, and the ratio is held
by its scalar bar (TOL_SCALAR_STORAGE).

8-bit first moment. The same near-tie disagreement can move an int8 code by one
step (code = m / scale rounded, decided on each side's own m). Such a step is
1/127 of its group's largest magnitude; it then decays with beta1 in later
steps, but the group's scale may shrink meanwhile, so in codes it can span more
than one step. The first moment is therefore judged on its dequantized values
(code x scale), relative to its group's largest magnitude (127 x scale):
* every value within 2e-2 of it (one code step is 0.79%); and
* at most 1% (+4) of the codes differ.
The scales (max |m| / 127 per group), the parameter and CAME's confidence
statistics follow the 16-bit rules above; dX is not checked on its own (a code
step moves it by up to 1/127 of the group's magnitude).
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
TOL_DX_NORM = 1e-6   # normwise error of the step, its storage slack taken off
TOL_SCALAR = 1e-6    # per-tensor scalars (alpha, kappa, RMS(U), RMS(X), norms, trust ratio)
# scalars computed from a 16-bit or 8-bit stored state (RMS(X) and alpha of a bf16
# parameter; LAMB's norms and trust ratio with such a parameter or first moment):
# the storage's near-tie disagreements (<= 1% of the elements, one bf16 step or
# one code step of 1/127 of a group's largest value each) move a norm over n
# elements by about 0.024 * 0.1 / sqrt(n) relative, 2e-5 at n = 16384.
TOL_SCALAR_STORAGE = 1e-4
G_ONLY_SCALARS = ("rms_u", "kappa")   # depend on the gradient and its statistics only
# floors (x RMS(b)) of the signed fp32 outputs
FLOOR_PARAM = 1e-2
FLOOR_EXP_AVG = 0.1
FLOOR_DX = 0.1


POSITIVE_KEYS = ("exp_avg_sq_row", "exp_avg_sq_col", "exp_avg_sq", "exp_avg_res_row", "exp_avg_res_col")


def _rms(a: np.ndarray) -> float:
    return math.sqrt(float(np.mean(a * a))) if a.size else 0.0


def floored_rel_errs(a, b, floor: float = 1.0, scale=0.0) -> np.ndarray:
    """|a_i - b_i| / max(|b_i|, floor * RMS(b), scale_i) per element (``scale``: a
    number or an array of b's size; a zero denominator counts as 1)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    if b.size == 0:
        return np.zeros(0)
    r = _rms(b) if floor > 0 else 0.0
    scale = np.asarray(scale, dtype=np.float64).reshape(-1) if np.ndim(scale) else scale
    den = np.maximum(np.maximum(np.abs(b), floor * r), scale)
    den = np.where(den > 0, den, 1.0)
    return np.abs(a - b) / den


def floored_rel_err(a, b, floor: float = 1.0) -> float:
    """max_i |a_i - b_i| / max(|b_i|, floor * RMS(b))."""
    e = floored_rel_errs(a, b, floor)
    return float(np.max(e)) if e.size else 0.0


def normwise_err(a, b) -> float:
    """||a - b|| / ||b|| (unfloored; |a - b| when b is zero)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    if b.size == 0:
        return 0.0
    nb = float(np.linalg.norm(b))
    d = float(np.linalg.norm(a - b))
    return d / nb if nb > 0 else d


def ema_terms(b, prev, beta: float) -> np.ndarray:
    """|beta * prev_i| + |b_i - beta * prev_i|: the magnitudes of the two terms of
    the average b = beta * prev + (1 - beta) * u, whose fp32 rounding error is
    relative to them, not to b where they cancel."""
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    p = beta * np.asarray(prev, dtype=np.float64).reshape(-1)
    return np.abs(p) + np.abs(b - p)


def output_errs(key: str, a, b, x0=None, prev=None, beta1=None, step_tol: float = TOL_F32) -> np.ndarray:
    """Elementwise errors of one fp32 output under its bar (rules above). x0, the
    initial parameter, sets the parameter's accumulated-change floor, scaled by
    step_tol / 1e-5 where the steps carry a bar of their own (GaLore's update,
    1e-4 on bf16 matrix cores); prev and beta1, the first moment's previous value
    and weight, its terms' floor."""
    if key in POSITIVE_KEYS:
        return floored_rel_errs(a, b, 0.0)
    if key == "param":
        scale = 0.0
        if x0 is not None:
            scale = (step_tol / TOL_F32) * _rms(np.asarray(b, dtype=np.float64).reshape(-1)
                                                - np.asarray(x0, dtype=np.float64).reshape(-1))
        return floored_rel_errs(a, b, FLOOR_PARAM, scale)
    if key == "exp_avg":
        scale = ema_terms(b, prev, beta1) if (prev is not None and beta1 is not None) else 0.0
        return floored_rel_errs(a, b, FLOOR_EXP_AVG, scale)
    return floored_rel_errs(a, b, 1.0)


def output_err(key: str, a, b, x0=None, prev=None, beta1=None) -> float:
    """The error of one fp32 output tensor under the rule above."""
    e = output_errs(key, a, b, x0, prev, beta1)
    return float(np.max(e)) if e.size else 0.0


def beta1_of(opt: str, hp: dict):
    """The first moment's weight beta1 of the step (None: no first moment)."""
    if opt == "adafactor":
        return oracle.adafactor_hparams(hp)["beta1"]
    return (oracle.came_hparams(hp) if opt == "came" else oracle.lamb_hparams(hp))["betas"][0]


def scalar_bar(n: int) -> float:
    """Bar of a per-tensor scalar over n elements: each element's value carries a
    few fp32 roundings and the chained states' own error (up to ~1e-5 relative);
    a norm or RMS over n elements averages independent errors by sqrt(n)."""
    return max(TOL_SCALAR, 1e-5 / math.sqrt(max(n, 1)))


def dx_errs(xn_lib, xo_lib, xn_ref, xo_ref, floor: float = FLOOR_DX):
    """(elementwise errors, normwise error) of the step dX = X_new - X_old, with
    one fp32 spacing of the library's parameter forgiven per element; floor x
    RMS(dX) under the fp32 bar, RMS(dX) under the 16-bit rules."""
    xn_lib = np.asarray(xn_lib, dtype=np.float64).reshape(-1)
    xo_lib = np.asarray(xo_lib, dtype=np.float64).reshape(-1)
    da = xn_lib - xo_lib
    db = np.asarray(xn_ref, dtype=np.float64).reshape(-1) - np.asarray(xo_ref, dtype=np.float64).reshape(-1)
    if db.size == 0:
        return np.zeros(0), 0.0
    big = np.maximum(np.abs(xn_lib), np.abs(xo_lib)).astype(np.float32)
    slack = np.spacing(big).astype(np.float64)
    num = np.maximum(np.abs(da - db) - slack, 0.0)
    den = np.maximum(np.abs(db), floor * _rms(db))
    den = np.where(den > 0, den, 1.0)
    nb = float(np.linalg.norm(db))
    nn = float(np.linalg.norm(num))
    return num / den, (nn / nb if nb > 0 else nn)


def check_dx(kind: str, xn_lib, xo_lib, xn_ref, xo_ref):
    """(ok, max error, elements above 1e-5, elements, normwise) of the step under
    its bar: "f32" (fp32 parameter and moment) or "rounded" (fp32 parameter stepped
    by a bf16 first moment)."""
    e, nw = dx_errs(xn_lib, xo_lib, xn_ref, xo_ref, FLOOR_DX if kind == "f32" else 1.0)
    err = float(np.max(e)) if e.size else 0.0
    over = int(np.count_nonzero(e > TOL_F32))
    if kind == "f32":
        return err <= TOL_F32 and nw <= TOL_DX_NORM, err, over, e.size, nw
    return err <= TOL_BF16 and over <= MAX_SHARE * e.size + MAX_EXTRA, err, over, e.size, nw


def dx_kind(opt: str, hp: dict, storage: dict) -> str:
    """How a tensor's step is judged: "f32", "rounded", or "" (not on its own)."""
    if storage.get("param_bf16") or storage.get("exp_avg_i8"):
        return ""
    return bar_kind(opt, hp, storage, "param")


# Library slot -> oracle key of the per-tensor scalars, per optimizer.
SCALAR_KEYS = {
    "adafactor": (("alpha", "alpha"), ("kappa", "kappa"), ("rms_u", "rms_u"), ("rms_x", "rms_x")),
    "came": (("kappa", "kappa"), ("rms_u", "rms_u")),
    "lamb": (("rms_x", "x_norm"), ("norm_d", "d_norm"), ("trust", "trust")),
}


def scalar_errs(opt: str, lib: Dict[str, float], ref: Dict[str, float]) -> Dict[str, float]:
    """Relative error of each per-tensor scalar the oracle reports (RMS(X) only
    with scale_parameter, when the oracle computes it)."""
    out = {}
    for slot, key in SCALAR_KEYS[opt]:
        if key not in ref:
            continue
        b = float(ref[key])
        a = float(lib[slot])
        out[key] = abs(a - b) / abs(b) if b != 0 else abs(a)
    return out


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


def check_bar(kind: str, key: str, a, b, x0=None, prev=None, beta1=None, step_tol: float = TOL_F32):
    """(ok, max error, elements off the fp32 bar (or codes that differ), elements)
    of one output under its bar. For "codes", a and b are (codes, scales) pairs.
    fp32 bar: x0, the initial parameter, for the parameter's floor; prev and beta1
    for the first moment's (see output_errs)."""
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
    if kind == "f32":
        e = output_errs(key, a, b, x0, prev, beta1, step_tol)
    else:
        e = floored_rel_errs(a, b, 0.0 if key in POSITIVE_KEYS else 1.0)
    err = float(np.max(e)) if e.size else 0.0
    over = int(np.count_nonzero(e > TOL_F32))
    if kind == "f32":
        return err <= TOL_F32, err, over, e.size
    return err <= TOL_BF16 and over <= MAX_SHARE * e.size + MAX_EXTRA, err, over, e.size


def judge_arrays(opt: str, hp: dict, storage: dict, out: list, x0, xo_lib=None, xo_ref=None,
                 lib_scalars=None, ref_scalars=None, m_prev=None) -> Dict[str, tuple]:
    """Every check of one tensor after a step, from host arrays: ``out`` is the
    list of (key, library value, oracle value) of its outputs (see ``outputs``; its
    "param" entry's library value is the stored parameter). Returns {name: (ok, max
    error, elements above 1e-5, elements, bar kind, normwise error)} for the
    outputs, the step "dx" (when the previous parameters are given) and the
    scalars "scalar:<name>". ``m_prev``: the oracle's first moment before the
    step (as a value), for its terms' floor."""
    res = {}
    lib_x = ref_x = None
    b1 = beta1_of(opt, hp)
    for key, lib, ref in out:
        kind = bar_kind(opt, hp, storage, key)
        ok, err, over, n = check_bar(kind, key, lib, ref, x0 if key == "param" else None,
                                     m_prev if key == "exp_avg" else None, b1)
        nw = normwise_err(lib, ref) if kind != "codes" else float("nan")
        res[key] = (ok, err, over, n, kind, nw)
        if key == "param":
            lib_x, ref_x = lib, ref
    dk = dx_kind(opt, hp, storage)
    if dk and xo_lib is not None and xo_ref is not None:
        want_x = ref_x
        if (opt == "lamb" and dk == "rounded" and lib_scalars is not None and ref_scalars is not None
                and ref_scalars.get("trust")):
            # the direction, with the ratio judged below (see the module notes)
            xo = np.asarray(xo_ref, dtype=np.float64)
            want_x = xo + (np.asarray(ref_x, dtype=np.float64) - xo) * (lib_scalars["trust"] / ref_scalars["trust"])
        ok, err, over, n, nw = check_dx(dk, lib_x, xo_lib, want_x, xo_ref)
        res["dx"] = (ok, err, over, n, dk, nw)
    if lib_scalars is not None and ref_scalars is not None:
        stored = any(storage.get(k) for k in ("param_bf16", "exp_avg_bf16", "exp_avg_i8"))
        numel = int(np.size(ref_x)) if ref_x is not None else 1
        for name, e in scalar_errs(opt, lib_scalars, ref_scalars).items():
            bar = TOL_SCALAR_STORAGE if stored and name not in G_ONLY_SCALARS else scalar_bar(numel)
            res["scalar:" + name] = (e <= bar, e, int(e > bar), 1, "scalar", e)
    return res


def judge_tensor(opt: str, hp: dict, storage: dict, param: torch.Tensor, state: Dict[str, torch.Tensor],
                 ox, ost, x0, xo_lib=None, xo_ref=None, lib_scalars=None, ref_scalars=None,
                 ost_prev=None) -> Dict[str, tuple]:
    """judge_arrays for a tensor the library stepped (its parameter and states);
    ``ost_prev``: the oracle's state before the step."""
    m_prev = None
    if ost_prev is not None and "exp_avg" in ost_prev and "exp_avg_scale" not in ost_prev:
        m_prev = ost_prev["exp_avg"]
    return judge_arrays(opt, hp, storage, outputs(param, state, ox, ost), x0, xo_lib, xo_ref, lib_scalars,
                        ref_scalars, m_prev)


def summarize(label: str, res: Dict[str, tuple]) -> str:
    """One line: the worst error per bar kind, and the worst normwise error."""
    parts = []
    for kind in ("f32", "rounded", "codes", "scalar"):
        sel = {k: v for k, v in res.items() if v[4] == kind}
        if sel:
            w = max(sel, key=lambda k: sel[k][1])
            parts.append(f"{kind} {sel[w][1]:.2e} ({w})")
    nws = {k: v[5] for k, v in res.items() if v[4] in ("f32", "rounded") and not math.isnan(v[5])}
    if nws:
        w = max(nws, key=nws.get)
        parts.append(f"normwise {nws[w]:.2e} ({w})")
    return f"{label}: " + "; ".join(parts)


def failures(res: Dict[str, tuple]) -> Dict[str, tuple]:
    return {k: v for k, v in res.items() if not v[0]}


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


def lib_scalar_offsets(opt, params, grads):
    return getattr(_lib, f"meo_{opt}_scalar_offsets")(params, grads)


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
        self.x0 = [x.copy() for x in self.ox]
        self.ost = [oracle.INIT_STATE[self.opt](tuple(p.shape), self.hp, exp_avg_i8=s["exp_avg_i8"])
                    for p, s in zip(self.params, self.storage)]
        self.ws = None
        self.offsets = None
        self.t = 0
        self.carry = carry
        self.carry_valid = False
        # the previous parameters of both sides, the scalars of the last step
        self.xo_lib = self.xo_ref = None
        self.lib_scalars = self.ref_scalars = None
        self.ost_prev = None
        self.oracle_stepped = False
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
        if oracle_too:
            self.xo_lib = [to64(p) for p in self.params]
            self.xo_ref = list(self.ox)
            self.ost_prev = list(self.ost)
        if self.carry:
            _lib.meo_adafactor_step_carry(self.hps, self.t, self.params, grads, self.states, self.carry_valid,
                                          self.ws)
            self.carry_valid = True
        else:
            lib_step(self.opt, self.hps, self.t, self.params, grads, self.states, self.ws)
        self.oracle_stepped = oracle_too
        if oracle_too:
            if self.offsets is None:
                self.offsets = lib_scalar_offsets(self.opt, self.params, grads)
            self.lib_scalars = _lib.read_scalars(self.ws, self.offsets) if self.ws is not None else \
                [None] * len(self.params)
            gs = [to64(g) for g in grads]
            self.ref_scalars = []
            for k in range(len(gs)):
                sc = {}
                self.ox[k], self.ost[k] = oracle.STEP_TENSOR[self.opt](self.ox[k], gs[k], self.ost[k], self.hp,
                                                                       self.t, scalars=sc, **self.storage[k])
                self.ref_scalars.append(sc)
        return grads

    def judged(self) -> Dict[str, tuple]:
        """Per check "<tensor>:<name>": (ok, max error, elements above 1e-5, elements,
        bar kind, normwise error); see judge_tensor."""
        torch.cuda.synchronize()
        out = {}
        fresh = self.oracle_stepped
        for k, spec in enumerate(self.wl.specs):
            res = judge_tensor(self.opt, self.hp, self.storage[k], self.params[k], self.states[k], self.ox[k],
                               self.ost[k], self.x0[k],
                               self.xo_lib[k] if fresh and self.xo_lib else None,
                               self.xo_ref[k] if fresh and self.xo_ref else None,
                               self.lib_scalars[k] if fresh and self.lib_scalars else None,
                               self.ref_scalars[k] if fresh and self.ref_scalars else None,
                               self.ost_prev[k] if fresh and self.ost_prev else None)
            for key, v in res.items():
                out[f"{spec.name}:{key}"] = v
        return out

    def verdicts(self) -> Dict[str, tuple]:
        """Per output "<tensor>:<key>": (ok, max error, elements above 1e-5, elements, bar kind)."""
        return {k: v[:5] for k, v in self.judged().items()}

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
        return {k: v[1] for k, v in self.judged().items()}

    def check(self, label: str = "") -> float:
        """Asserts every check meets its bar; prints the worst errors and returns the
        worst fp32-bar error of the outputs."""
        v = self.judged()
        print("  " + summarize(f"{self.wl.name} {label}", v), flush=True)
        bad = failures(v)
        assert not bad, f"{label}: " + ", ".join(
            f"{k} ({x[4]} bar): err {x[1]:.3e}, {x[2]}/{x[3]} above 1e-5, normwise {x[5]:.2e}"
            for k, x in bad.items())
        f32 = [x[1] for k, x in v.items() if x[4] == "f32" and not k.endswith(":dx")]
        return max(f32) if f32 else 0.0


def list_run(wl: workloads.Workload, sample_idx, steps: int, check_steps=None, carry: bool = False,
             workers: int = 1, device="cuda", on_check=None):
    """One library call over the whole list per step (the bench's launch shape),
    with the oracle following only the tensors in ``sample_idx`` (every statistic is
    per tensor, so a tensor's result does not depend on the rest of the list).

    ``check_steps``: the steps after which every check of every sampled tensor is
    judged (default: all). ``carry`` (Adafactor): meo_adafactor_step_carry, reading
    X on the first call and the carried sums after. ``workers``: host threads
    stepping the oracle's tensors side by side (NumPy releases the interpreter lock
    inside its array operations). ``on_check(t, params, states, oracle_params)``, if
    given, runs after the checks of each checked step. Asserts every check; returns
    the worst error per bar kind over all checked steps."""
    import concurrent.futures as cf

    opt, hp = wl.optimizer, dict(wl.hparams)
    ps = workloads.init_params(wl, device)
    sts = lib_states(opt, ps, hp, wl.state_dtype)
    if carry:
        for st in sts:
            st["param_sumsq"] = torch.zeros(1, dtype=torch.float32, device=device)
    hps = lib_hp(opt, hp)
    scales = workloads.grad_scales(wl, device)
    sample_idx = list(sample_idx)
    storage = {k: storage_of_tensor(ps[k], sts[k]) for k in sample_idx}
    ox = {k: to64(ps[k]) for k in sample_idx}
    x0 = {k: ox[k].copy() for k in sample_idx}
    ost = {k: oracle.INIT_STATE[opt](tuple(ps[k].shape), hp, exp_avg_i8=storage[k]["exp_avg_i8"])
           for k in sample_idx}
    check_steps = set(range(1, steps + 1) if check_steps is None else check_steps)
    ws, offs = None, None
    worst: Dict[str, float] = {}
    pool = cf.ThreadPoolExecutor(max_workers=max(1, workers))
    try:
        for t in range(1, steps + 1):
            gs = workloads.grads(wl, t - 1, scales, device)
            if ws is None:
                ws = lib_workspace(opt, ps, gs)
                offs = lib_scalar_offsets(opt, ps, gs)
            judge_now = t in check_steps
            xo_lib = dict(zip(sample_idx, pool.map(lambda k: to64(ps[k]), sample_idx))) if judge_now else {}
            if carry:
                _lib.meo_adafactor_step_carry(hps, t, ps, gs, sts, t > 1, ws)
            else:
                lib_step(opt, hps, t, ps, gs, sts, ws)
            torch.cuda.synchronize()
            lib_sc = _lib.read_scalars(ws, offs) if (judge_now and ws is not None) else None

            def one(k):
                sc = {}
                xo, so = ox[k], ost[k]
                nx, nst = oracle.STEP_TENSOR[opt](xo, to64(gs[k]), so, hp, t, scalars=sc, **storage[k])
                res = None
                if judge_now:
                    res = judge_tensor(opt, hp, storage[k], ps[k], sts[k], nx, nst, x0[k], xo_lib[k], xo,
                                       lib_sc[k] if lib_sc else None, sc, so)
                return k, nx, nst, res

            results = list(pool.map(one, sample_idx))
            del gs
            for k, nx, nst, res in results:
                ox[k], ost[k] = nx, nst
                if res is None:
                    continue
                if len(sample_idx) <= 8:
                    print("  " + summarize(f"{wl.name} step {t} {wl.specs[k].name}", res), flush=True)
                for key, v in res.items():
                    worst[v[4]] = max(worst.get(v[4], 0.0), v[1])
                bad = failures(res)
                assert not bad, (t, wl.specs[k].name, {key: v for key, v in bad.items()})
            if judge_now:
                print(f"  {wl.name} step {t}: {len(sample_idx)} tensors checked, worst per bar "
                      + ", ".join(f"{kd} {e:.2e}" for kd, e in sorted(worst.items())), flush=True)
                if on_check is not None:
                    on_check(t, ps, sts, ox)
            del xo_lib
    finally:
        pool.shutdown(wait=True)
    return worst
