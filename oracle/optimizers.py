"""Plain fp64 NumPy oracle for one optimizer step of Adafactor, CAME and LAMB.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import this module; the library never does, and it
shares no code, constant table or helper with the HIP path.

Everything is done in float64 with whole-array NumPy operations in the order the
method states, and the second-moment estimate of the factored path is
*materialised* as a full array (the HIP path never builds it). States are plain
dicts of float64 arrays named as on the Colossal-AI distributed-optimizers page
("Colossal-AI 分布式优化器全解析", blog.gitcode.com; section "Step 3"):
``exp_avg``, ``exp_avg_sq_row``, ``exp_avg_sq_col``, ``exp_avg_sq``. CAME's
confidence statistics, which the page describes but does not name, are
``exp_avg_res_row`` / ``exp_avg_res_col``; LAMB's moments are ``exp_avg`` /
``exp_avg_sq``.

Functions take and return new arrays; nothing is modified in place. ``t`` is the
1-based index of the step being taken (the counter is incremented before use).

Sources (the pages), by function:

* Adafactor: the page's section "Step 3" (defaults, relative step size and its
  ValueError texts, optional first moment, factored-vs-full rule with the row
  and column statistic shapes), the note after "Step 5" (beta2t = 1 - step **
  decay_rate, RMS clipping by clip_threshold, scale_parameter), and the "four
  optimizers" table (second moment approximated by row * col).
* CAME: the "four optimizers" table (confidence matrix on top of Adafactor's
  factorisation, three betas) and the "DistributedCAME" paragraph of the "other
  optimizers' key parameters" section (defaults). The step order follows the CAME
  paper the page cites (arXiv:2307.02047).
* LAMB: the "four optimizers" table (layer-wise trust ratio) and the
  "DistributedLAMB" paragraph (defaults, validation). The step follows the LAMB
  paper the page cites (arXiv:1904.00962).

* 16-bit storage: the DistributedCAME paragraph says the optimizer supports a
  memory-saving 16-bit path under mixed precision. With ``param_bf16`` /
  ``exp_avg_bf16`` the parameter / first moment is held in bfloat16: the inputs
  are bf16 values (exact in float64), the arithmetic is unchanged, and each new
  value is rounded to bf16 as it is formed (``round_bf16``), so the rest of the
  step uses the stored first moment.
* 8-bit first moment: the GaLore section's 8-bit optimizer base (nbits=8,
  block_wise=True) and the ms-swift page's Q-GaLore ``quantize_tensor`` (groups of
  128 values, one absmax scale per group, int8 codes). With ``exp_avg_i8`` the
  state holds ``exp_avg`` as int8 codes and ``exp_avg_scale`` as one float32 scale
  per group; each step dequantizes, updates and re-quantizes the first moment, and
  the rest of the step uses the dequantized new value (``quantize_i8``).

Readings where the pages are silent are listed, with reasons, in the design notes
of this repository; each is marked "reading" at the line that applies it.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

Array = np.ndarray
State = Dict[str, Array]

# ----------------------------------------------------------------------------- defaults

# Page "Step 3": the distributed Adafactor's defaults, aligned with Hugging Face's.
ADAFACTOR_DEFAULTS = dict(lr=None, eps=(1e-30, 1e-3), clip_threshold=1.0, decay_rate=-0.8,
                          beta1=None, weight_decay=0.0, scale_parameter=True,
                          relative_step=True, warmup_init=False)
# Page "DistributedCAME" paragraph.
CAME_DEFAULTS = dict(lr=None, eps=(1e-30, 1e-16), clip_threshold=1.0,
                     betas=(0.9, 0.999, 0.9999), weight_decay=0.0)
# Page "DistributedLAMB" paragraph.
LAMB_DEFAULTS = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-6, weight_decay=0.0,
                     bias_correction=True)

# Error texts printed on the page ("Step 3").
MSG_LR_WITH_RELATIVE = "Cannot combine manual lr and relative_step=True options"
MSG_WARMUP_NEEDS_RELATIVE = "warmup_init=True requires relative_step=True"


def _hp(defaults: dict, hp: Optional[dict]) -> dict:
    out = dict(defaults)
    if hp:
        unknown = set(hp) - set(defaults)
        if unknown:
            raise TypeError(f"unknown hyperparameters: {sorted(unknown)}")
        out.update(hp)
    return out


def rms(a: Array) -> float:
    """Root mean square over every element of the tensor (population RMS)."""
    a = np.asarray(a, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return math.sqrt(float(np.mean(a * a)))


def round_bf16(a) -> Array:
    """Nearest bfloat16 value of each element, as float64.

    bfloat16 is the upper half of an IEEE float32 (sign, the 8 exponent bits, the
    first 7 of the 23 fraction bits). reading: the value is first rounded to
    float32, the type in which the GPU forms it, then to the nearest bf16 with ties
    to the even last kept bit; values beyond the largest bf16 go to +-inf, NaN
    stays NaN."""
    f = np.atleast_1d(np.asarray(a, dtype=np.float64)).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    # Adding 0x7fff plus the last kept bit carries into the kept half exactly when
    # the dropped half is above the midpoint, or at it with an odd kept half.
    rounded = ((bits + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    out = (rounded & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).astype(np.float64)
    out[np.isnan(f)] = np.nan
    return out.reshape(np.shape(a))


def _stored(a: Array, bf16: bool) -> Array:
    """A new value of a tensor as its storage holds it (reading: 16-bit storage)."""
    return round_bf16(a) if bf16 else a


I8_GROUP = 128  # the group_size of the ms-swift page's quantize_tensor


def quantize_i8(a) -> Tuple[Array, Array]:
    """(codes, scales) of the ms-swift page's group-wise int8 quantization (section
    on Q-GaLore): the values, flattened, are cut into groups of 128 consecutive
    ones; each group's scale is its largest magnitude / 127 and each code is
    value / scale rounded to the nearest integer and clamped to [-128, 127].

    reading: the arithmetic is that of the page's float32 tensors: values are first
    rounded to float32, the scale is the float32 quotient and each code the float32
    quotient rounded half to even (torch.round).
    reading: a group of zeros gets scale 0 and codes 0 (the page would divide by 0).
    reading: a group holding a NaN or an infinity has no finite scale; it keeps
    scale NaN and codes 0, so the whole group reads back NaN (a non-finite moment
    stays visible, as it does in float32 storage).
    reading: when the element count is not a multiple of 128 the last, shorter
    group is a group of its own (the page's reshape needs a multiple)."""
    x = np.asarray(a, dtype=np.float64).reshape(-1).astype(np.float32)
    n = x.size
    ng = -(-n // I8_GROUP)
    padded = np.zeros(ng * I8_GROUP, dtype=np.float32)
    padded[:n] = x
    groups = padded.reshape(ng, I8_GROUP)
    with np.errstate(invalid="ignore", over="ignore"):
        scale = (np.max(np.abs(groups), axis=1) / np.float32(127.0)).astype(np.float32)
        scale[~np.isfinite(scale)] = np.float32(np.nan)
        usable = np.isfinite(scale) & (scale > 0)
        safe = np.where(usable, scale, np.float32(1.0)).astype(np.float32)
        q = np.rint(groups / safe[:, None]).astype(np.float32)
        q = np.where(usable[:, None], q, np.float32(0.0))
    codes = np.clip(q, -128, 127).astype(np.int8).reshape(-1)[:n]
    return codes.reshape(np.shape(a)), scale


def dequantize_i8(codes, scales) -> Array:
    """code * scale of its group, in float32 as on the page, returned as float64."""
    q = np.asarray(codes).reshape(-1).astype(np.float32)
    s = np.repeat(np.asarray(scales, dtype=np.float32), I8_GROUP)[:q.size]
    return (q * s).astype(np.float64).reshape(np.shape(codes))


def _moment_in(state: State, i8: bool) -> Array:
    """The stored first moment as a value (dequantized when it is kept in 8 bits)."""
    if i8:
        return dequantize_i8(state["exp_avg"], state["exp_avg_scale"])
    return state["exp_avg"]


def _moment_out(m: Array, new: State, bf16: bool, i8: bool) -> Array:
    """Stores a new first moment in `new` as its storage keeps it and returns the
    value the rest of the step uses (reading: the stored one)."""
    if i8:
        codes, scales = quantize_i8(m)
        new["exp_avg"], new["exp_avg_scale"] = codes, scales
        return dequantize_i8(codes, scales)
    new["exp_avg"] = _stored(m, bf16)
    return new["exp_avg"]


def is_factored(shape: Tuple[int, ...]) -> bool:
    """Page "Step 3": the statistics are factored for tensors of two or more
    dimensions, full for the others."""
    return len(shape) >= 2


def _untouched(x: Array, state: State) -> Tuple[Array, State]:
    """reading: a tensor with no elements has nothing to update; its statistics
    (means over zero entries) are left as they were."""
    return np.array(x, dtype=np.float64), {k: np.array(v) for k, v in state.items()}


# ----------------------------------------------------------------------------- Adafactor

def adafactor_hparams(hp: Optional[dict] = None) -> dict:
    """Defaults merged with ``hp`` and validated as the page states ("Step 3")."""
    h = _hp(ADAFACTOR_DEFAULTS, hp)
    if h["lr"] is not None and h["relative_step"]:
        raise ValueError(MSG_LR_WITH_RELATIVE)
    if h["warmup_init"] and not h["relative_step"]:
        raise ValueError(MSG_WARMUP_NEEDS_RELATIVE)
    if h["lr"] is None and not h["relative_step"]:
        # reading: without a relative step there is no learning rate at all.
        raise ValueError("lr is required when relative_step=False")
    return h


def adafactor_step_size(h: dict, t: int) -> float:
    """rho_t. Page "Step 3": with relative_step the rate is min(1e-2, 1/sqrt(step)),
    and warmup_init replaces the 1e-2 by 1e-6 * step (reading: the linear ramp sits
    inside the same min). Without relative_step it is the given lr."""
    if h["relative_step"]:
        cap = 1e-6 * t if h["warmup_init"] else 1e-2
        return min(cap, 1.0 / math.sqrt(t))
    return float(h["lr"])


def adafactor_beta2t(h: dict, t: int) -> float:
    """Note after "Step 5": beta2t = 1 - step ** decay_rate."""
    return 1.0 - math.pow(t, h["decay_rate"])


def _i8_state(st: State, shape) -> State:
    """Zero 8-bit first moment: int8 codes and one float32 scale per 128 values."""
    n = int(np.prod(shape)) if len(shape) else 1
    st["exp_avg"] = np.zeros(shape, dtype=np.int8)
    st["exp_avg_scale"] = np.zeros(-(-n // I8_GROUP), dtype=np.float32)
    return st


def adafactor_init_state(shape: Tuple[int, ...], hp: Optional[dict] = None, *, exp_avg_i8: bool = False
                         ) -> State:
    """Zero state with the shapes of page "Step 3": row statistic over shape[:-1],
    column statistic over shape[:-2] + shape[-1:], full statistic for 1-D, and
    ``exp_avg`` only when beta1 is set (as codes and scales with ``exp_avg_i8``)."""
    h = adafactor_hparams(hp)
    shape = tuple(shape)
    st: State = {}
    if h["beta1"] is not None:
        if exp_avg_i8:
            _i8_state(st, shape)
        else:
            st["exp_avg"] = np.zeros(shape)
    if is_factored(shape):
        st["exp_avg_sq_row"] = np.zeros(shape[:-1])
        st["exp_avg_sq_col"] = np.zeros(shape[:-2] + shape[-1:])
    else:
        st["exp_avg_sq"] = np.zeros(shape)
    return st


def adafactor_step_tensor(x: Array, g: Array, state: State, hp: Optional[dict], t: int, *,
                          param_bf16: bool = False, exp_avg_bf16: bool = False, exp_avg_i8: bool = False,
                          scalars: Optional[dict] = None) -> Tuple[Array, State]:
    """One Adafactor step of one tensor; returns (new parameter, new state).

    ``scalars``, if given, receives the step's per-tensor values: ``rho`` (the
    relative or given step size), ``rms_x`` (with scale_parameter), ``alpha``
    (the scaled step size), ``rms_u`` (RMS of the unclipped update) and ``kappa``
    (the clip divisor max(1, RMS(u) / clip_threshold))."""
    h = adafactor_hparams(hp)
    if t < 1:
        raise ValueError("step must be >= 1")
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if x.size == 0:
        return _untouched(x, state)
    eps1, eps2 = h["eps"]

    # Learning rate: relative step, scaled by the parameter's RMS before this
    # step's update (reading: the RMS is taken when the rate is computed).
    alpha = adafactor_step_size(h, t)
    out = {} if scalars is None else scalars
    out["rho"] = alpha
    if h["scale_parameter"]:
        out["rms_x"] = rms(x)
        alpha *= max(eps2, out["rms_x"])
    out["alpha"] = alpha

    b2 = adafactor_beta2t(h, t)
    q = g * g + eps1  # reading: eps1 enters with the squared gradient
    new = {}
    if is_factored(x.shape):
        row = b2 * state["exp_avg_sq_row"] + (1.0 - b2) * q.mean(axis=-1)
        col = b2 * state["exp_avg_sq_col"] + (1.0 - b2) * q.mean(axis=-2)
        new["exp_avg_sq_row"], new["exp_avg_sq_col"] = row, col
        # "row * col" estimate, normalised by the row statistic's mean over each
        # matrix (the leading dims are independent matrices), materialised in full.
        v_hat = row[..., :, None] * col[..., None, :] / row.mean(axis=-1)[..., None, None]
    else:
        v = b2 * state["exp_avg_sq"] + (1.0 - b2) * q
        new["exp_avg_sq"] = v
        v_hat = v
    u = g / np.sqrt(v_hat)
    # RMS clipping (note after "Step 5"): divide by max(1, RMS(u) / clip_threshold).
    out["rms_u"] = rms(u)
    out["kappa"] = max(1.0, out["rms_u"] / h["clip_threshold"])
    u = u / out["kappa"]
    u = alpha * u
    if h["beta1"] is not None:
        # reading: the first moment averages the clipped, lr-scaled update.
        m = h["beta1"] * _moment_in(state, exp_avg_i8) + (1.0 - h["beta1"]) * u
        delta = _moment_out(m, new, exp_avg_bf16, exp_avg_i8)
    else:
        delta = u
    # reading: decoupled weight decay on the pre-update parameter, scaled by alpha.
    x_new = _stored(x - h["weight_decay"] * alpha * x - delta, param_bf16)
    return x_new, new


def adafactor_step(xs: Sequence[Array], gs: Sequence[Array], states: Sequence[State],
                   hp: Optional[dict], t: int, **storage) -> Tuple[List[Array], List[State]]:
    """A step over a list: every statistic is per tensor, so each is independent."""
    out_x, out_s = [], []
    for x, g, st in zip(xs, gs, states):
        a, b = adafactor_step_tensor(x, g, st, hp, t, **storage)
        out_x.append(a)
        out_s.append(b)
    return out_x, out_s


# ----------------------------------------------------------------------------- CAME

def came_hparams(hp: Optional[dict] = None) -> dict:
    h = _hp(CAME_DEFAULTS, hp)
    if h["lr"] is None:
        # reading: CAME has no relative step, so the lr must be supplied.
        raise ValueError("CAME requires an explicit lr")
    if h["lr"] < 0:
        raise ValueError(f"Invalid learning rate: {h['lr']}")
    for i, b in enumerate(h["betas"]):
        if not 0.0 <= b < 1.0:
            raise ValueError(f"Invalid beta parameter at index {i}: {b}")
    return h


def came_init_state(shape: Tuple[int, ...], hp: Optional[dict] = None, *, exp_avg_i8: bool = False
                    ) -> State:
    """Zero state: first moment, factored (or full) squared-gradient statistic and,
    for factored tensors, the factored confidence statistic."""
    shape = tuple(shape)
    st: State = _i8_state({}, shape) if exp_avg_i8 else {"exp_avg": np.zeros(shape)}
    if is_factored(shape):
        st["exp_avg_sq_row"] = np.zeros(shape[:-1])
        st["exp_avg_sq_col"] = np.zeros(shape[:-2] + shape[-1:])
        st["exp_avg_res_row"] = np.zeros(shape[:-1])
        st["exp_avg_res_col"] = np.zeros(shape[:-2] + shape[-1:])
    else:
        st["exp_avg_sq"] = np.zeros(shape)
    return st


def _factored_estimate(row: Array, col: Array) -> Array:
    """row_i * col_j / mean_i(row_i) per matrix, materialised."""
    return row[..., :, None] * col[..., None, :] / row.mean(axis=-1)[..., None, None]


def came_step_tensor(x: Array, g: Array, state: State, hp: Optional[dict], t: int, *,
                     param_bf16: bool = False, exp_avg_bf16: bool = False, exp_avg_i8: bool = False,
                     scalars: Optional[dict] = None) -> Tuple[Array, State]:
    """One CAME step of one tensor; returns (new parameter, new state).

    ``scalars``, if given, receives ``rms_u`` (RMS of the unclipped update) and
    ``kappa`` (the clip divisor)."""
    h = came_hparams(hp)
    if t < 1:
        raise ValueError("step must be >= 1")
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if x.size == 0:
        return _untouched(x, state)
    eps1, eps2 = h["eps"]
    beta1, beta2, beta3 = h["betas"]
    lr = float(h["lr"])
    new = {}

    # Squared-gradient statistic: Adafactor's factorisation with a constant beta2
    # (reading: no decay schedule and no bias correction).
    q = g * g + eps1
    fac = is_factored(x.shape)
    if fac:
        row = beta2 * state["exp_avg_sq_row"] + (1.0 - beta2) * q.mean(axis=-1)
        col = beta2 * state["exp_avg_sq_col"] + (1.0 - beta2) * q.mean(axis=-2)
        new["exp_avg_sq_row"], new["exp_avg_sq_col"] = row, col
        v_hat = _factored_estimate(row, col)
    else:
        v = beta2 * state["exp_avg_sq"] + (1.0 - beta2) * q
        new["exp_avg_sq"] = v
        v_hat = v
    u = g / np.sqrt(v_hat)
    out = {} if scalars is None else scalars
    out["rms_u"] = rms(u)
    out["kappa"] = max(1.0, out["rms_u"] / h["clip_threshold"])
    u = u / out["kappa"]

    m = _moment_out(beta1 * _moment_in(state, exp_avg_i8) + (1.0 - beta1) * u, new, exp_avg_bf16, exp_avg_i8)

    if fac:
        # Instability of the update against its running mean, factored the same
        # way; its reconstruction is the confidence that scales the step.
        e = (u - m) ** 2 + eps2
        rrow = beta3 * state["exp_avg_res_row"] + (1.0 - beta3) * e.mean(axis=-1)
        rcol = beta3 * state["exp_avg_res_col"] + (1.0 - beta3) * e.mean(axis=-2)
        new["exp_avg_res_row"], new["exp_avg_res_col"] = rrow, rcol
        s = _factored_estimate(rrow, rcol)
        delta = m / np.sqrt(s)
    else:
        # reading: a full 1-D statistic carries no factorisation error to correct.
        delta = m
    x_new = _stored(x - lr * h["weight_decay"] * x - lr * delta, param_bf16)
    return x_new, new


def came_step(xs, gs, states, hp, t, **storage):
    out_x, out_s = [], []
    for x, g, st in zip(xs, gs, states):
        a, b = came_step_tensor(x, g, st, hp, t, **storage)
        out_x.append(a)
        out_s.append(b)
    return out_x, out_s


# ----------------------------------------------------------------------------- LAMB

def lamb_hparams(hp: Optional[dict] = None) -> dict:
    """Defaults merged with ``hp``; the page says the constructor validates lr, eps
    and betas (reading: lr >= 0, eps >= 0, 0 <= beta < 1)."""
    h = _hp(LAMB_DEFAULTS, hp)
    if not h["lr"] >= 0.0:
        raise ValueError(f"Invalid learning rate: {h['lr']}")
    if not h["eps"] >= 0.0:
        raise ValueError(f"Invalid epsilon value: {h['eps']}")
    for i, b in enumerate(h["betas"]):
        if not 0.0 <= b < 1.0:
            raise ValueError(f"Invalid beta parameter at index {i}: {b}")
    return h


def lamb_init_state(shape: Tuple[int, ...], hp: Optional[dict] = None, *, exp_avg_i8: bool = False
                    ) -> State:
    shape = tuple(shape)
    st: State = _i8_state({}, shape) if exp_avg_i8 else {"exp_avg": np.zeros(shape)}
    st["exp_avg_sq"] = np.zeros(shape)
    return st


def lamb_step_tensor(x: Array, g: Array, state: State, hp: Optional[dict], t: int, *,
                     param_bf16: bool = False, exp_avg_bf16: bool = False, exp_avg_i8: bool = False,
                     scalars: Optional[dict] = None) -> Tuple[Array, State]:
    """One LAMB step of one tensor (the whole tensor is one layer for the trust ratio).

    ``scalars``, if given, receives ``x_norm`` and ``d_norm`` (the 2-norms of the
    parameter and of the update direction) and ``trust`` (the trust ratio)."""
    h = lamb_hparams(hp)
    if t < 1:
        raise ValueError("step must be >= 1")
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if x.size == 0:
        return _untouched(x, state)
    beta1, beta2 = h["betas"]
    new: State = {}
    m = _moment_out(beta1 * _moment_in(state, exp_avg_i8) + (1.0 - beta1) * g, new, exp_avg_bf16, exp_avg_i8)
    v = beta2 * state["exp_avg_sq"] + (1.0 - beta2) * g * g
    if h["bias_correction"]:
        m_hat = m / (1.0 - beta1 ** t)
        v_hat = v / (1.0 - beta2 ** t)
    else:
        m_hat, v_hat = m, v
    # reading: eps outside the square root; decay added to the Adam direction.
    d = m_hat / (np.sqrt(v_hat) + h["eps"]) + h["weight_decay"] * x
    x_norm = float(np.sqrt(np.sum(x * x)))
    d_norm = float(np.sqrt(np.sum(d * d)))
    # reading: identity scaling of the parameter norm; ratio 1 when either norm is 0.
    trust = x_norm / d_norm if (x_norm > 0.0 and d_norm > 0.0) else 1.0
    if scalars is not None:
        scalars.update(x_norm=x_norm, d_norm=d_norm, trust=trust)
    x_new = _stored(x - h["lr"] * trust * d, param_bf16)
    new["exp_avg_sq"] = v
    return x_new, new


def lamb_step(xs, gs, states, hp, t, **storage):
    out_x, out_s = [], []
    for x, g, st in zip(xs, gs, states):
        a, b = lamb_step_tensor(x, g, st, hp, t, **storage)
        out_x.append(a)
        out_s.append(b)
    return out_x, out_s


# ----------------------------------------------------------------------------- dispatch

STEP = {"adafactor": adafactor_step, "came": came_step, "lamb": lamb_step}
STEP_TENSOR = {"adafactor": adafactor_step_tensor, "came": came_step_tensor,
               "lamb": lamb_step_tensor}
INIT_STATE = {"adafactor": adafactor_init_state, "came": came_init_state,
              "lamb": lamb_init_state}
