"""ctypes binding of libmeo.so: argument marshalling only.

Every function here has the name of the C entry point it calls and does nothing
but turn torch tensors into the C structs (device pointers and sizes), pass the
current HIP stream, and turn a negative return code into ``MeoError``. All
arithmetic of the step runs in the library's HIP kernels. The library must be
built (``python -m memory_efficient_optimizers_amd.build``); without it every call
raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, List, Optional, Sequence

import torch  # loaded first: the library binds to the HIP runtime torch has loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmeo.so")

c_int32, c_int64, c_double, c_void_p, c_size_t = (ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                                  ctypes.c_void_p, ctypes.c_size_t)
c_float_p = ctypes.POINTER(ctypes.c_float)

MEO_OK, MEO_EINVAL, MEO_ESHAPE, MEO_EDTYPE, MEO_ENULL, MEO_EWORKSPACE, MEO_EALIGN, MEO_EHIP, MEO_EMEMORY = (
    0, -1, -2, -3, -4, -5, -6, -7, -8)
MEO_F32, MEO_BF16, MEO_I8 = 0, 1, 2
I8_GROUP = 128  # values per scale of an 8-bit first moment
ERROR_NAMES = {MEO_EINVAL: "MEO_EINVAL", MEO_ESHAPE: "MEO_ESHAPE", MEO_EDTYPE: "MEO_EDTYPE",
               MEO_ENULL: "MEO_ENULL", MEO_EWORKSPACE: "MEO_EWORKSPACE", MEO_EALIGN: "MEO_EALIGN",
               MEO_EHIP: "MEO_EHIP", MEO_EMEMORY: "MEO_EMEMORY"}
EXPORTS = [
    "meo_adafactor_defaults", "meo_adafactor_workspace_size", "meo_adafactor_validate",
    "meo_adafactor_step", "meo_adafactor_step_carry", "meo_came_defaults", "meo_came_workspace_size", "meo_came_validate",
    "meo_came_step", "meo_lamb_defaults", "meo_lamb_workspace_size", "meo_lamb_validate",
    "meo_lamb_step", "meo_last_error", "meo_release_plans", "meo_version", "meo_profile_enable",
    "meo_pass_name", "meo_profile_collect",
    "meo_adafactor_partials_size", "meo_adafactor_shard_stats", "meo_adafactor_shard_apply",
    "meo_adafactor_shard_stats_carry", "meo_adafactor_shard_apply_carry",
    "meo_lamb_partials_size", "meo_lamb_shard_stats", "meo_lamb_shard_apply",
    "meo_came_partials_size", "meo_came_confidence_size", "meo_came_shard_stats", "meo_came_shard_moment",
    "meo_came_shard_apply",
    "meo_galore_defaults", "meo_galore_rank", "meo_galore_workspace_size", "meo_galore_validate",
    "meo_galore_step", "meo_galore_refresh",
    "meo_adafactor_scalar_offsets", "meo_came_scalar_offsets", "meo_lamb_scalar_offsets",
    "meo_adafactor_step_noalloc",
]
MEO_NOALLOC_SCRATCH_BYTES = 64 << 20
MEO_NUM_PASSES = 17


class MeoError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code
        self.message = message


class meo_tensor(ctypes.Structure):
    _fields_ = [("param", c_void_p), ("grad", c_void_p), ("batch", c_int64), ("rows", c_int64),
                ("cols", c_int64), ("ndim", c_int32), ("param_dtype", c_int32),
                ("grad_dtype", c_int32), ("state_dtype", c_int32)]


class meo_shard(ctypes.Structure):
    _fields_ = [("rows_total", c_int64)]


class meo_adafactor_hparams(ctypes.Structure):
    _fields_ = [("lr", c_double), ("eps1", c_double), ("eps2", c_double),
                ("clip_threshold", c_double), ("decay_rate", c_double), ("beta1", c_double),
                ("weight_decay", c_double), ("has_lr", c_int32), ("has_beta1", c_int32),
                ("scale_parameter", c_int32), ("relative_step", c_int32),
                ("warmup_init", c_int32), ("reserved", c_int32)]


class meo_adafactor_state(ctypes.Structure):
    _fields_ = [("exp_avg", c_void_p), ("exp_avg_sq_row", c_void_p), ("exp_avg_sq_col", c_void_p),
                ("exp_avg_sq", c_void_p), ("exp_avg_scale", c_void_p), ("param_sumsq", c_void_p)]


class meo_came_hparams(ctypes.Structure):
    _fields_ = [("lr", c_double), ("eps1", c_double), ("eps2", c_double),
                ("clip_threshold", c_double), ("beta1", c_double), ("beta2", c_double),
                ("beta3", c_double), ("weight_decay", c_double), ("has_lr", c_int32),
                ("reserved", c_int32)]


class meo_came_state(ctypes.Structure):
    _fields_ = [("exp_avg", c_void_p), ("exp_avg_sq_row", c_void_p), ("exp_avg_sq_col", c_void_p),
                ("exp_avg_res_row", c_void_p), ("exp_avg_res_col", c_void_p),
                ("exp_avg_sq", c_void_p), ("exp_avg_scale", c_void_p)]


class meo_lamb_hparams(ctypes.Structure):
    _fields_ = [("lr", c_double), ("beta1", c_double), ("beta2", c_double), ("eps", c_double),
                ("weight_decay", c_double), ("bias_correction", c_int32), ("reserved", c_int32)]


class meo_lamb_state(ctypes.Structure):
    _fields_ = [("exp_avg", c_void_p), ("exp_avg_sq", c_void_p), ("exp_avg_scale", c_void_p)]


MEO_GALORE_STD, MEO_GALORE_REVERSE_STD = 0, 1
_PROJ_TYPE = {"std": MEO_GALORE_STD, "reverse_std": MEO_GALORE_REVERSE_STD}


class meo_galore_hparams(ctypes.Structure):
    _fields_ = [("lr", c_double), ("beta1", c_double), ("beta2", c_double), ("eps", c_double),
                ("weight_decay", c_double), ("rank", c_int32), ("update_proj_gap", c_int32),
                ("scale", c_double), ("proj_type", c_int32), ("reserved", c_int32)]


class meo_galore_state(ctypes.Structure):
    _fields_ = [("exp_avg", c_void_p), ("exp_avg_sq", c_void_p), ("projector", c_void_p),
                ("projector_t", c_void_p)]


_lib: Optional[ctypes.CDLL] = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads libmeo.so once and declares the signatures; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m memory_efficient_optimizers_amd.build`")
    lib = ctypes.CDLL(path)
    T = ctypes.POINTER(meo_tensor)
    for opt, hp, st in (("adafactor", meo_adafactor_hparams, meo_adafactor_state),
                        ("came", meo_came_hparams, meo_came_state),
                        ("lamb", meo_lamb_hparams, meo_lamb_state)):
        getattr(lib, f"meo_{opt}_defaults").argtypes = [ctypes.POINTER(hp)]
        getattr(lib, f"meo_{opt}_defaults").restype = None
        getattr(lib, f"meo_{opt}_workspace_size").argtypes = [c_int32, T]
        getattr(lib, f"meo_{opt}_workspace_size").restype = c_size_t
        getattr(lib, f"meo_{opt}_scalar_offsets").argtypes = [c_int32, T, ctypes.POINTER(c_int64)]
        getattr(lib, f"meo_{opt}_scalar_offsets").restype = ctypes.c_int
        getattr(lib, f"meo_{opt}_validate").argtypes = [ctypes.POINTER(hp), c_int64, c_int32, T,
                                                        ctypes.POINTER(st)]
        getattr(lib, f"meo_{opt}_validate").restype = ctypes.c_int
        getattr(lib, f"meo_{opt}_step").argtypes = [ctypes.POINTER(hp), c_int64, c_int32, T,
                                                    ctypes.POINTER(st), c_void_p, c_size_t, c_void_p]
        getattr(lib, f"meo_{opt}_step").restype = ctypes.c_int
    lib.meo_adafactor_step_carry.argtypes = [ctypes.POINTER(meo_adafactor_hparams), c_int64, c_int32, T,
                                             ctypes.POINTER(meo_adafactor_state), c_int32, c_void_p, c_size_t,
                                             c_void_p]
    lib.meo_adafactor_step_carry.restype = ctypes.c_int
    lib.meo_adafactor_step_noalloc.argtypes = [ctypes.POINTER(meo_adafactor_hparams), c_int64, c_int32, T,
                                               ctypes.POINTER(meo_adafactor_state), c_void_p]
    lib.meo_adafactor_step_noalloc.restype = ctypes.c_int
    S = ctypes.POINTER(meo_shard)
    for opt, hp, st in (("adafactor", meo_adafactor_hparams, meo_adafactor_state),
                        ("lamb", meo_lamb_hparams, meo_lamb_state)):
        getattr(lib, f"meo_{opt}_partials_size").argtypes = [c_int32, T]
        getattr(lib, f"meo_{opt}_partials_size").restype = c_size_t
        for stage in ("stats", "apply"):
            fn = getattr(lib, f"meo_{opt}_shard_{stage}")
            fn.argtypes = [ctypes.POINTER(hp), c_int64, c_int32, T, S, ctypes.POINTER(st), c_void_p, c_void_p,
                           c_size_t, c_void_p]
            fn.restype = ctypes.c_int
    AH, AS = ctypes.POINTER(meo_adafactor_hparams), ctypes.POINTER(meo_adafactor_state)
    lib.meo_adafactor_shard_stats_carry.argtypes = [AH, c_int64, c_int32, T, S, AS, c_int32, c_void_p, c_void_p,
                                                    c_size_t, c_void_p]
    lib.meo_adafactor_shard_stats_carry.restype = ctypes.c_int
    lib.meo_adafactor_shard_apply_carry.argtypes = [AH, c_int64, c_int32, T, S, AS, c_void_p, c_void_p, c_size_t,
                                                    c_void_p]
    lib.meo_adafactor_shard_apply_carry.restype = ctypes.c_int
    CH, CS = ctypes.POINTER(meo_came_hparams), ctypes.POINTER(meo_came_state)
    for name in ("meo_came_partials_size", "meo_came_confidence_size"):
        getattr(lib, name).argtypes = [c_int32, T]
        getattr(lib, name).restype = c_size_t
    for name in ("meo_came_shard_stats", "meo_came_shard_apply"):
        getattr(lib, name).argtypes = [CH, c_int64, c_int32, T, S, CS, c_void_p, c_void_p, c_size_t, c_void_p]
        getattr(lib, name).restype = ctypes.c_int
    lib.meo_came_shard_moment.argtypes = [CH, c_int64, c_int32, T, S, CS, c_void_p, c_void_p, c_void_p, c_size_t,
                                          c_void_p]
    lib.meo_came_shard_moment.restype = ctypes.c_int
    lib.meo_last_error.argtypes = []
    lib.meo_last_error.restype = ctypes.c_char_p
    lib.meo_release_plans.argtypes = []
    lib.meo_release_plans.restype = None
    lib.meo_version.argtypes = []
    lib.meo_version.restype = ctypes.c_int
    lib.meo_profile_enable.argtypes = [ctypes.c_int]
    lib.meo_profile_enable.restype = ctypes.c_int
    lib.meo_pass_name.argtypes = [ctypes.c_int]
    lib.meo_pass_name.restype = ctypes.c_char_p
    lib.meo_profile_collect.argtypes = [ctypes.POINTER(c_double), ctypes.POINTER(c_int64)]
    lib.meo_profile_collect.restype = ctypes.c_int
    GH, GS = ctypes.POINTER(meo_galore_hparams), ctypes.POINTER(meo_galore_state)
    lib.meo_galore_defaults.argtypes = [GH]
    lib.meo_galore_defaults.restype = None
    lib.meo_galore_rank.argtypes = [GH, T]
    lib.meo_galore_rank.restype = c_int32
    lib.meo_galore_workspace_size.argtypes = [GH, c_int32, T]
    lib.meo_galore_workspace_size.restype = c_size_t
    lib.meo_galore_validate.argtypes = [GH, c_int64, c_int32, T, GS]
    lib.meo_galore_validate.restype = ctypes.c_int
    lib.meo_galore_step.argtypes = [GH, c_int64, c_int32, T, GS, c_void_p, c_size_t, c_void_p]
    lib.meo_galore_step.restype = ctypes.c_int
    lib.meo_galore_refresh.argtypes = [GH, c_int32, T, GS, c_void_p, c_size_t, c_void_p]
    lib.meo_galore_refresh.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != MEO_OK:
        msg = load().meo_last_error().decode("utf-8", "replace")
        raise MeoError(rc, msg)


# ----------------------------------------------------------------------------- marshalling

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


_DTYPE = {torch.float32: MEO_F32, torch.bfloat16: MEO_BF16}
_STATE_DTYPE = {torch.float32: MEO_F32, torch.bfloat16: MEO_BF16, torch.int8: MEO_I8}


def tensor_struct(param: torch.Tensor, grad: torch.Tensor,
                  state_dtype: torch.dtype = torch.float32) -> meo_tensor:
    """[batch, rows, cols] view of a parameter and its gradient (see meo.h);
    ``state_dtype`` is the element type of the parameter's first moment."""
    if param.dtype not in _DTYPE:
        raise TypeError("parameters must be float32 or bfloat16")
    if grad.dtype not in _DTYPE:
        raise TypeError("gradients must be float32 or bfloat16")
    if state_dtype not in _STATE_DTYPE:
        raise TypeError("the first moment must be float32, bfloat16 or int8")
    if not (param.is_contiguous() and grad.is_contiguous()):
        raise ValueError("parameter and gradient must be contiguous")
    if grad.shape != param.shape:
        raise ValueError(f"gradient shape {tuple(grad.shape)} != parameter shape {tuple(param.shape)}")
    shape = tuple(param.shape)
    if len(shape) >= 2:
        batch = 1
        for s in shape[:-2]:
            batch *= s
        rows, cols = shape[-2], shape[-1]
    else:
        batch, rows, cols = 1, 1, param.numel()
    return meo_tensor(param.data_ptr(), grad.data_ptr(), batch, rows, cols, len(shape),
                      _DTYPE[param.dtype], _DTYPE[grad.dtype], _STATE_DTYPE[state_dtype])


def _tensors(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor], states=None):
    if len(params) != len(grads):
        raise ValueError("params and grads differ in length")
    if states is not None and len(states) != len(params):
        raise ValueError("params and states differ in length")
    arr = (meo_tensor * max(len(params), 1))()
    for i, (p, g) in enumerate(zip(params, grads)):
        m = None if states is None else states[i].get("exp_avg")
        arr[i] = tensor_struct(p, g, torch.float32 if m is None else m.dtype)
    return arr


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ws(workspace: Optional[torch.Tensor]):
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _states(cls, keys, states: Sequence[Dict[str, torch.Tensor]]):
    arr = (cls * max(len(states), 1))()
    for i, st in enumerate(states):
        for k in keys:
            t = st.get(k)
            if t is not None and t.dtype != torch.float32 and not (k == "exp_avg" and t.dtype in _STATE_DTYPE):
                raise TypeError(f"state {k} must be float32" + (", bfloat16 or int8" if k == "exp_avg" else ""))
            if t is not None and not t.is_contiguous():
                raise ValueError(f"state {k} must be contiguous (row-major)")
        arr[i] = cls(*[_ptr(st.get(k)) for k in keys])
    return arr


ADAFACTOR_KEYS = ["exp_avg", "exp_avg_sq_row", "exp_avg_sq_col", "exp_avg_sq", "exp_avg_scale", "param_sumsq"]
CAME_KEYS = ["exp_avg", "exp_avg_sq_row", "exp_avg_sq_col", "exp_avg_res_row", "exp_avg_res_col",
             "exp_avg_sq", "exp_avg_scale"]
LAMB_KEYS = ["exp_avg", "exp_avg_sq", "exp_avg_scale"]


# ----------------------------------------------------------------------------- hparams

def adafactor_hparams(lr=None, eps=(1e-30, 1e-3), clip_threshold=1.0, decay_rate=-0.8, beta1=None,
                      weight_decay=0.0, scale_parameter=True, relative_step=True,
                      warmup_init=False) -> meo_adafactor_hparams:
    return meo_adafactor_hparams(0.0 if lr is None else float(lr), float(eps[0]), float(eps[1]),
                                 float(clip_threshold), float(decay_rate),
                                 0.0 if beta1 is None else float(beta1), float(weight_decay),
                                 int(lr is not None), int(beta1 is not None), int(bool(scale_parameter)),
                                 int(bool(relative_step)), int(bool(warmup_init)), 0)


def came_hparams(lr=None, eps=(1e-30, 1e-16), clip_threshold=1.0, betas=(0.9, 0.999, 0.9999),
                 weight_decay=0.0) -> meo_came_hparams:
    return meo_came_hparams(0.0 if lr is None else float(lr), float(eps[0]), float(eps[1]),
                            float(clip_threshold), float(betas[0]), float(betas[1]), float(betas[2]),
                            float(weight_decay), int(lr is not None), 0)


def lamb_hparams(lr=1e-3, betas=(0.9, 0.999), eps=1e-6, weight_decay=0.0,
                 bias_correction=True) -> meo_lamb_hparams:
    return meo_lamb_hparams(float(lr), float(betas[0]), float(betas[1]), float(eps),
                            float(weight_decay), int(bool(bias_correction)), 0)


def galore_hparams(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, rank=256, update_proj_gap=200,
                   scale=0.25, proj_type="std") -> meo_galore_hparams:
    if proj_type not in _PROJ_TYPE:
        raise ValueError("proj_type must be 'std' or 'reverse_std'")
    return meo_galore_hparams(float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay),
                              int(rank), int(update_proj_gap), float(scale), _PROJ_TYPE[proj_type], 0)


def meo_adafactor_defaults() -> meo_adafactor_hparams:
    hp = meo_adafactor_hparams()
    load().meo_adafactor_defaults(ctypes.byref(hp))
    return hp


def meo_came_defaults() -> meo_came_hparams:
    hp = meo_came_hparams()
    load().meo_came_defaults(ctypes.byref(hp))
    return hp


def meo_lamb_defaults() -> meo_lamb_hparams:
    hp = meo_lamb_hparams()
    load().meo_lamb_defaults(ctypes.byref(hp))
    return hp


# ----------------------------------------------------------------------------- entry points

def meo_adafactor_workspace_size(params, grads) -> int:
    return int(load().meo_adafactor_workspace_size(len(params), _tensors(params, grads)))


def meo_came_workspace_size(params, grads) -> int:
    return int(load().meo_came_workspace_size(len(params), _tensors(params, grads)))


def meo_lamb_workspace_size(params, grads) -> int:
    return int(load().meo_lamb_workspace_size(len(params), _tensors(params, grads)))


SCALAR_SLOTS = ("alpha", "coef", "decay", "rms_u", "rms_x", "norm_d", "kappa", "trust")


def _scalar_offsets(opt, params, grads):
    out = (c_int64 * max(len(params), 1))()
    _check(getattr(load(), f"meo_{opt}_scalar_offsets")(len(params), _tensors(params, grads), out))
    return [int(out[k]) for k in range(len(params))]


def meo_adafactor_scalar_offsets(params, grads):
    return _scalar_offsets("adafactor", params, grads)


def meo_came_scalar_offsets(params, grads):
    return _scalar_offsets("came", params, grads)


def meo_lamb_scalar_offsets(params, grads):
    return _scalar_offsets("lamb", params, grads)


def read_scalars(workspace: torch.Tensor, offsets) -> List[Optional[Dict[str, float]]]:
    """The per-tensor scalars a completed step left in ``workspace`` (slots named as
    in SCALAR_SLOTS; None for tensors with zero elements). Synchronises the device."""
    live = [off for off in offsets if off >= 0]
    if not live:
        return [None] * len(offsets)
    flat = workspace.view(torch.float32)
    idx = torch.tensor([off + i for off in live for i in range(len(SCALAR_SLOTS))], dtype=torch.int64,
                       device=flat.device)
    vals = flat[idx].cpu().tolist()
    out, j = [], 0
    for off in offsets:
        if off < 0:
            out.append(None)
            continue
        out.append(dict(zip(SCALAR_SLOTS, vals[j:j + len(SCALAR_SLOTS)])))
        j += len(SCALAR_SLOTS)
    return out

# The per-tensor slots each optimizer writes (include/meo.h, meo_*_scalar_offsets)
# through which a non-finite gradient shows: RMS(U) and the clip divisor built on
# it (Adafactor, CAME), the direction's norm and the trust ratio (LAMB, whose
# direction also holds the decayed parameter, so its norm slot catches a
# non-finite parameter as well).
FINITE_CHECK_SLOTS = {"adafactor": ("coef", "rms_u", "kappa"), "came": ("coef", "rms_u", "kappa"),
                      "lamb": ("rms_x", "norm_d", "trust")}


def nonfinite_tensors(optimizer: str, workspace: torch.Tensor, offsets) -> List[int]:
    """Indices of the tensors whose scalars, left in ``workspace`` by a completed
    step call, hold a NaN or an infinity, so that the call's update of that tensor is
    not finite: a NaN or infinite gradient element does that for every optimizer;
    for Adafactor and CAME so does a factored tensor's element whose square
    overflows float32 (LAMB's v then turns infinite and that element's direction is
    0, a finite step). Tensors with zero elements are never listed. Synchronises the
    device."""
    slots = FINITE_CHECK_SLOTS[optimizer]
    out = []
    for k, sc in enumerate(read_scalars(workspace, offsets)):
        if sc is not None and not all(math.isfinite(sc[name]) for name in slots):
            out.append(k)
    return out


def meo_adafactor_validate(hp, step, params, grads, states) -> None:
    _check(load().meo_adafactor_validate(ctypes.byref(hp), step, len(params), _tensors(params, grads, states),
                                         _states(meo_adafactor_state, ADAFACTOR_KEYS, states)))


def meo_came_validate(hp, step, params, grads, states) -> None:
    _check(load().meo_came_validate(ctypes.byref(hp), step, len(params), _tensors(params, grads, states),
                                    _states(meo_came_state, CAME_KEYS, states)))


def meo_lamb_validate(hp, step, params, grads, states) -> None:
    _check(load().meo_lamb_validate(ctypes.byref(hp), step, len(params), _tensors(params, grads, states),
                                    _states(meo_lamb_state, LAMB_KEYS, states)))


def meo_adafactor_step(hp, step, params, grads, states, workspace=None, stream=None) -> None:
    ws, nb = _ws(workspace)
    _check(load().meo_adafactor_step(ctypes.byref(hp), step, len(params), _tensors(params, grads, states),
                                     _states(meo_adafactor_state, ADAFACTOR_KEYS, states), ws, nb,
                                     _stream(stream)))


def meo_adafactor_step_carry(hp, step, params, grads, states, param_sumsq_valid: bool, workspace=None,
                             stream=None) -> None:
    """meo_adafactor_step that leaves each tensor's sum of squares of its updated
    parameter in ``states[k]["param_sumsq"]`` (float32 [1]) and, with
    ``param_sumsq_valid``, takes RMS(X) from the sums the previous call left."""
    ws, nb = _ws(workspace)
    _check(load().meo_adafactor_step_carry(ctypes.byref(hp), step, len(params), _tensors(params, grads, states),
                                           _states(meo_adafactor_state, ADAFACTOR_KEYS, states),
                                           1 if param_sumsq_valid else 0, ws, nb, _stream(stream)))


def meo_adafactor_step_noalloc(hp, step, params, grads, states, stream=None) -> None:
    """meo_adafactor_step without a workspace: the library's per-GPU scratch holds
    the call's launch tables and workspace (at most MEO_NOALLOC_SCRATCH_BYTES)."""
    _check(load().meo_adafactor_step_noalloc(ctypes.byref(hp), step, len(params), _tensors(params, grads, states),
                                             _states(meo_adafactor_state, ADAFACTOR_KEYS, states), _stream(stream)))


def meo_came_step(hp, step, params, grads, states, workspace=None, stream=None) -> None:
    ws, nb = _ws(workspace)
    _check(load().meo_came_step(ctypes.byref(hp), step, len(params), _tensors(params, grads, states),
                                _states(meo_came_state, CAME_KEYS, states), ws, nb, _stream(stream)))


def meo_lamb_step(hp, step, params, grads, states, workspace=None, stream=None) -> None:
    ws, nb = _ws(workspace)
    _check(load().meo_lamb_step(ctypes.byref(hp), step, len(params), _tensors(params, grads, states),
                                _states(meo_lamb_state, LAMB_KEYS, states), ws, nb, _stream(stream)))


# ----------------------------------------------------------------------------- row-sharded steps

def _shards(totals: Sequence[int]):
    arr = (meo_shard * max(len(totals), 1))()
    for i, t in enumerate(totals):
        arr[i] = meo_shard(int(t))
    return arr


def meo_adafactor_partials_size(params, grads) -> int:
    """Floats of the partial-sum record of a row-sharded Adafactor step."""
    return int(load().meo_adafactor_partials_size(len(params), _tensors(params, grads)))


def meo_lamb_partials_size(params, grads) -> int:
    return int(load().meo_lamb_partials_size(len(params), _tensors(params, grads)))


def _shard_call(opt, stage, hp, step, params, grads, totals, states, partials, workspace, stream):
    cls, keys = {"adafactor": (meo_adafactor_state, ADAFACTOR_KEYS), "lamb": (meo_lamb_state, LAMB_KEYS)}[opt]
    ws, nb = _ws(workspace)
    _check(getattr(load(), f"meo_{opt}_shard_{stage}")(
        ctypes.byref(hp), step, len(params), _tensors(params, grads, states), _shards(totals),
        _states(cls, keys, states), _ptr(partials), ws, nb, _stream(stream)))


def meo_adafactor_shard_stats(hp, step, params, grads, totals, states, partials, workspace=None, stream=None):
    """Stage 1 of a row-sharded step: the shard's statistics and its partial sums
    (``totals[k]``: rows of the whole matrix, or elements of a whole 1-D tensor)."""
    _shard_call("adafactor", "stats", hp, step, params, grads, totals, states, partials, workspace, stream)


def meo_adafactor_shard_apply(hp, step, params, grads, totals, states, partials, workspace=None, stream=None):
    """Stage 3: the update of the shard from the partial sums reduced over all ranks."""
    _shard_call("adafactor", "apply", hp, step, params, grads, totals, states, partials, workspace, stream)


def meo_adafactor_shard_stats_carry(hp, step, params, grads, totals, states, param_sumsq_valid: bool, partials,
                                    workspace=None, stream=None):
    """meo_adafactor_shard_stats whose record takes the shard's carried sum of X^2
    (``states[k]["param_sumsq"]``) when ``param_sumsq_valid``."""
    ws, nb = _ws(workspace)
    _check(load().meo_adafactor_shard_stats_carry(
        ctypes.byref(hp), step, len(params), _tensors(params, grads, states), _shards(totals),
        _states(meo_adafactor_state, ADAFACTOR_KEYS, states), 1 if param_sumsq_valid else 0, _ptr(partials), ws, nb,
        _stream(stream)))


def meo_adafactor_shard_apply_carry(hp, step, params, grads, totals, states, partials, workspace=None, stream=None):
    """meo_adafactor_shard_apply that leaves each shard's sum of squares of its
    updated rows in ``states[k]["param_sumsq"]``."""
    _shard_call("adafactor", "apply_carry", hp, step, params, grads, totals, states, partials, workspace, stream)


def meo_lamb_shard_stats(hp, step, params, grads, totals, states, partials, workspace=None, stream=None):
    _shard_call("lamb", "stats", hp, step, params, grads, totals, states, partials, workspace, stream)


def meo_lamb_shard_apply(hp, step, params, grads, totals, states, partials, workspace=None, stream=None):
    _shard_call("lamb", "apply", hp, step, params, grads, totals, states, partials, workspace, stream)


def meo_came_partials_size(params, grads) -> int:
    return int(load().meo_came_partials_size(len(params), _tensors(params, grads)))


def meo_came_confidence_size(params, grads) -> int:
    """Floats of CAME's second record (confidence sums) in a row-sharded step."""
    return int(load().meo_came_confidence_size(len(params), _tensors(params, grads)))


def _came_args(hp, step, params, grads, totals, states):
    return (ctypes.byref(hp), step, len(params), _tensors(params, grads, states), _shards(totals),
            _states(meo_came_state, CAME_KEYS, states))


def meo_came_shard_stats(hp, step, params, grads, totals, states, partials, workspace=None, stream=None):
    ws, nb = _ws(workspace)
    _check(load().meo_came_shard_stats(*_came_args(hp, step, params, grads, totals, states), _ptr(partials), ws, nb,
                                       _stream(stream)))


def meo_came_shard_moment(hp, step, params, grads, totals, states, partials, confidence, workspace=None,
                          stream=None):
    """CAME's second stage: from the reduced ``partials``, the moment update of the
    shard and its confidence sums (``confidence``, to be reduced over the ranks)."""
    ws, nb = _ws(workspace)
    _check(load().meo_came_shard_moment(*_came_args(hp, step, params, grads, totals, states), _ptr(partials),
                                        _ptr(confidence), ws, nb, _stream(stream)))


def meo_came_shard_apply(hp, step, params, grads, totals, states, confidence, workspace=None, stream=None):
    ws, nb = _ws(workspace)
    _check(load().meo_came_shard_apply(*_came_args(hp, step, params, grads, totals, states), _ptr(confidence), ws,
                                       nb, _stream(stream)))


class PreparedShardStep:
    """The calls of a row-sharded step over a fixed list, marshalled once (see
    PreparedStep): ``stats(step)`` fills ``partials`` and, after the caller has
    summed them over the ranks, ``apply(step)`` updates the shard. CAME has a call
    between the two: ``moment(step)`` takes the summed ``partials`` and fills
    ``confidence``, which ``apply(step)`` takes summed over the ranks.
    ``carry`` (Adafactor): the carry calls; the first ``stats`` reads the shard's
    parameter, later ones take its carried sum of X^2 until ``invalidate()``."""

    _KIND = {"adafactor": (meo_adafactor_state, ADAFACTOR_KEYS), "lamb": (meo_lamb_state, LAMB_KEYS),
             "came": (meo_came_state, CAME_KEYS)}

    def __init__(self, optimizer: str, hp, params, grads, totals, states, partials, workspace=None,
                 confidence=None, carry: bool = False):
        cls, keys = self._KIND[optimizer]
        lib = load()
        self.came = optimizer == "came"
        if self.came and confidence is None:
            raise ValueError("CAME's row-sharded step needs the confidence buffer")
        if carry and optimizer != "adafactor":
            raise ValueError("only Adafactor carries sum(X^2)")
        self.carry = carry
        self.valid = False
        sfx = "_carry" if carry else ""
        self._fns = (getattr(lib, f"meo_{optimizer}_shard_stats{sfx}"),
                     getattr(lib, f"meo_{optimizer}_shard_apply{sfx}"),
                     lib.meo_came_shard_moment if self.came else None)
        self.hp = hp
        self.n = len(params)
        self.tensors = _tensors(params, grads, states)
        self.shards = _shards(totals)
        self.states = _states(cls, keys, states)
        self.partials = _ptr(partials)
        self.confidence = _ptr(confidence)
        self.ws, self.ws_bytes = _ws(workspace)
        self._keep = (list(params), list(grads), list(states), partials, confidence, workspace)

    def _call(self, fn, step, stream, *bufs):
        _check(fn(ctypes.byref(self.hp), step, self.n, self.tensors, self.shards, self.states, *bufs,
                  self.ws, self.ws_bytes, _stream(stream)))

    def invalidate(self) -> None:
        self.valid = False

    def stats(self, step: int, stream=None) -> None:
        if self.carry:
            self._call(self._fns[0], step, stream, 1 if self.valid else 0, self.partials)
            return
        self._call(self._fns[0], step, stream, self.partials)

    def moment(self, step: int, stream=None) -> None:
        if not self.came:
            raise ValueError("only CAME's row-sharded step has a moment call")
        self._call(self._fns[2], step, stream, self.partials, self.confidence)

    def apply(self, step: int, stream=None) -> None:
        self._call(self._fns[1], step, stream, self.confidence if self.came else self.partials)
        self.valid = self.carry


def meo_last_error() -> str:
    return load().meo_last_error().decode("utf-8", "replace")


def meo_release_plans() -> None:
    load().meo_release_plans()


def meo_version() -> int:
    return int(load().meo_version())


def meo_profile_enable(on: bool) -> None:
    _check(load().meo_profile_enable(int(bool(on))))


def meo_pass_name(i: int) -> str:
    return load().meo_pass_name(i).decode()


def meo_profile_collect() -> Dict[str, Dict[str, float]]:
    """{pass name: {"ms": total milliseconds, "launches": count}} since the last collect."""
    ms = (c_double * MEO_NUM_PASSES)()
    n = (c_int64 * MEO_NUM_PASSES)()
    _check(load().meo_profile_collect(ms, n))
    return {meo_pass_name(i): {"ms": ms[i], "launches": int(n[i])} for i in range(MEO_NUM_PASSES) if n[i]}


class PreparedStep:
    """The C arguments of one optimizer's step over a fixed list, marshalled once:
    repeated calls (a training loop, a benchmark) then only pass the step index and
    the stream. The tensors must stay alive and in place."""

    _KIND = {"adafactor": (meo_adafactor_state, ADAFACTOR_KEYS),
             "came": (meo_came_state, CAME_KEYS), "lamb": (meo_lamb_state, LAMB_KEYS)}

    def __init__(self, optimizer: str, hp, params, grads, states, workspace=None, carry: bool = False):
        """carry (Adafactor): call meo_adafactor_step_carry; the first call reads
        RMS(X) from the parameters, later ones take it from the carried sums until
        ``invalidate()`` (for callers that write the parameters between steps)."""
        cls, keys = self._KIND[optimizer]
        if carry and optimizer != "adafactor":
            raise ValueError("only Adafactor carries sum(X^2)")
        self.fn = getattr(load(), f"meo_{optimizer}_step_carry" if carry else f"meo_{optimizer}_step")
        self.carry = carry
        self.valid = False
        self.hp = hp
        self.n = len(params)
        self.tensors = _tensors(params, grads, states)
        self.states = _states(cls, keys, states)
        self.ws, self.ws_bytes = _ws(workspace)
        self._keep = (list(params), list(grads), list(states), workspace)

    def invalidate(self) -> None:
        self.valid = False

    def __call__(self, step: int, stream=None) -> None:
        if self.carry:
            _check(self.fn(ctypes.byref(self.hp), step, self.n, self.tensors, self.states, 1 if self.valid else 0,
                           self.ws, self.ws_bytes, _stream(stream)))
            self.valid = True
            return
        _check(self.fn(ctypes.byref(self.hp), step, self.n, self.tensors, self.states, self.ws,
                       self.ws_bytes, _stream(stream)))


# ----------------------------------------------------------------------------- GaLore

GALORE_KEYS = ["exp_avg", "exp_avg_sq", "projector", "projector_t"]


def meo_galore_defaults() -> meo_galore_hparams:
    hp = meo_galore_hparams()
    load().meo_galore_defaults(ctypes.byref(hp))
    return hp


def _galore_states(states):
    arr = (meo_galore_state * max(len(states), 1))()
    for i, st in enumerate(states):
        for k in ("exp_avg", "exp_avg_sq"):
            if st[k].dtype != torch.float32:
                raise TypeError(f"GaLore state {k} must be float32")
        for k in ("projector", "projector_t"):
            if st.get(k) is not None and st[k].dtype != torch.bfloat16:
                raise TypeError(f"GaLore state {k} must be bfloat16")
        for k in GALORE_KEYS:
            t = st.get(k)
            if t is not None and not t.is_contiguous():
                raise ValueError(f"GaLore state {k} must be contiguous (row-major)")
        arr[i] = meo_galore_state(*[_ptr(st.get(k)) for k in GALORE_KEYS])
    return arr


def meo_galore_rank(hp, param) -> int:
    return int(load().meo_galore_rank(ctypes.byref(hp), ctypes.byref(tensor_struct(param, param))))


def meo_galore_workspace_size(hp, params, grads) -> int:
    return int(load().meo_galore_workspace_size(ctypes.byref(hp), len(params), _tensors(params, grads)))


def meo_galore_validate(hp, step, params, grads, states) -> None:
    _check(load().meo_galore_validate(ctypes.byref(hp), step, len(params), _tensors(params, grads),
                                      _galore_states(states)))


def meo_galore_step(hp, step, params, grads, states, workspace=None, stream=None) -> None:
    ws, nb = _ws(workspace)
    _check(load().meo_galore_step(ctypes.byref(hp), step, len(params), _tensors(params, grads),
                                  _galore_states(states), ws, nb, _stream(stream)))


def meo_galore_refresh(hp, params, grads, states, workspace=None, stream=None) -> None:
    ws, nb = _ws(workspace)
    _check(load().meo_galore_refresh(ctypes.byref(hp), len(params), _tensors(params, grads),
                                     _galore_states(states), ws, nb, _stream(stream)))


def galore_state_shapes(shape, rank: int, proj_type: str = "std") -> Dict[str, tuple]:
    """Shapes of one parameter's GaLore states (meo.h): a 2-D parameter keeps
    [D][r] moments and the projector [d][r] with its transpose, where d is the
    projected side (std: the shorter, reverse_std: the longer) and D the other."""
    shape = tuple(shape)
    if len(shape) == 2 and shape[0] > 0 and shape[1] > 0:
        r = min(rank, min(shape))
        d = min(shape) if proj_type == "std" else max(shape)
        D = shape[0] * shape[1] // d
        return {"exp_avg": (D, r), "exp_avg_sq": (D, r), "projector": (d, r), "projector_t": (r, d)}
    return {"exp_avg": shape, "exp_avg_sq": shape}


def galore_init_state(param: torch.Tensor, rank: int, proj_type: str = "std") -> Dict[str, torch.Tensor]:
    """Zero GaLore states for one parameter (projectors in bfloat16)."""
    return {k: torch.zeros(s, dtype=torch.bfloat16 if k.startswith("projector") else torch.float32,
                           device=param.device)
            for k, s in galore_state_shapes(param.shape, rank, proj_type).items()}


# ----------------------------------------------------------------------------- state allocation

def state_shapes(optimizer: str, shape, *, beta1: bool = True, i8: bool = False) -> Dict[str, tuple]:
    """Shapes of the state tensors of one parameter, as meo.h expects them; with
    ``i8`` the first moment also has one scale per 128 values."""
    shape = tuple(shape)
    n = 1
    for d in shape:
        n *= d
    groups = ((n + I8_GROUP - 1) // I8_GROUP,)
    if optimizer == "lamb":
        st = {"exp_avg": shape, "exp_avg_sq": shape}
        if i8:
            st["exp_avg_scale"] = groups
        return st
    st: Dict[str, tuple] = {}
    if optimizer == "came" or beta1:
        st["exp_avg"] = shape
        if i8:
            st["exp_avg_scale"] = groups
    if len(shape) >= 2:
        st["exp_avg_sq_row"] = shape[:-1]
        st["exp_avg_sq_col"] = shape[:-2] + shape[-1:]
        if optimizer == "came":
            st["exp_avg_res_row"] = shape[:-1]
            st["exp_avg_res_col"] = shape[:-2] + shape[-1:]
    else:
        st["exp_avg_sq"] = shape
    return st


def init_state(optimizer: str, param: torch.Tensor, *, beta1: bool = True,
               state_dtype: torch.dtype = torch.float32) -> Dict[str, torch.Tensor]:
    """Zero state tensors for one parameter, with the shapes of meo.h: float32,
    except the first moment ``exp_avg``, which is ``state_dtype`` (float32, bfloat16,
    or int8 codes with float32 ``exp_avg_scale``)."""
    shapes = state_shapes(optimizer, param.shape, beta1=beta1, i8=state_dtype == torch.int8)
    return {k: torch.zeros(s, dtype=state_dtype if k == "exp_avg" else torch.float32, device=param.device)
            for k, s in shapes.items()}


def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A device scratch buffer of at least ``nbytes`` (torch allocations are 256-byte aligned)."""
    if nbytes <= 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)
