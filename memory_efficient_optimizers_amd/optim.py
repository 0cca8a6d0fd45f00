"""torch.optim front ends over the C ABI: Adafactor, CAME, Lamb and GaLoreAdamW.

Each class owns its state tensors (on the parameter's device, named as on the
Colossal-AI distributed-optimizers page: ``step``, ``exp_avg``,
``exp_avg_sq_row``, ``exp_avg_sq_col``, ``exp_avg_sq``; CAME adds
``exp_avg_res_row`` / ``exp_avg_res_col``) and a device workspace, and hands
every parameter with a gradient to one library call per parameter group (and per
step count, should parameters have taken different numbers of steps). The update
itself runs in the HIP kernels; ``state_dict()`` / ``load_state_dict()`` work as
for any torch optimizer.

Parameters may be float32 or bfloat16 (the page's DistributedCAME paragraph
mentions a memory-saving 16-bit path). Statistics are always float32; the first
moment ``exp_avg`` is kept in ``state_dtype``, which by default follows the
parameter (bfloat16 parameters get a bfloat16 first moment, float32 ones a
float32 one). The arithmetic is float32 throughout, and bfloat16 values are
rounded to nearest even when stored. ``state_dtype=torch.int8`` keeps the first
moment 8-bit group-quantized (128 values per float32 scale, the GaLore section's
8-bit base and the ms-swift page's quantizer) for every tensor that
``moment_dtype`` allows; the others keep it in float32.

Failure detection: with ``check_finite=True`` (Adafactor, CAME, Lamb) each call's
per-tensor scalars are read back once it completes, and ``nonfinite_params()``
lists the parameters whose gradient held a NaN or an infinity. The pages speak of
detecting NaNs and falling back to another optimizer; the fallback is left to the
caller.
"""
from __future__ import annotations

from collections import defaultdict
from typing import Dict, List, Optional, Tuple

import torch

from . import _lib


def moment_dtype(optimizer: str, shape, requested: Optional[torch.dtype], param_dtype: torch.dtype,
                 min_8bit_size: int = 4096) -> torch.dtype:
    """The first moment's dtype for one parameter. None follows the parameter
    (bfloat16 -> bfloat16, else float32). int8 applies to tensors of at least
    ``min_8bit_size`` elements (the GaLore section's 8-bit optimizer default: smaller
    ones stay 32-bit) whose rows hold whole groups of 128 when the statistics are
    factored (Adafactor and CAME with ndim >= 2); other tensors get float32."""
    if requested is None:
        return torch.bfloat16 if param_dtype == torch.bfloat16 else torch.float32
    if requested != torch.int8:
        return requested
    shape = tuple(shape)
    n = 1
    for d in shape:
        n *= d
    factored = optimizer != "lamb" and len(shape) >= 2
    if n < min_8bit_size or (factored and shape[-1] % _lib.I8_GROUP != 0):
        return torch.float32
    return torch.int8


class _MeoOptimizer(torch.optim.Optimizer):
    _kind = ""

    def __init__(self, params, defaults, state_dtype: Optional[torch.dtype] = None, min_8bit_size: int = 4096,
                 check_finite: bool = False):
        if state_dtype not in (None, torch.float32, torch.bfloat16, torch.int8):
            raise TypeError("state_dtype must be None, torch.float32, torch.bfloat16 or torch.int8")
        super().__init__(params, defaults)
        self._state_dtype = state_dtype
        self._min_8bit_size = min_8bit_size
        self._workspace: Dict[torch.device, torch.Tensor] = {}
        self._check_finite = bool(check_finite)
        self._nonfinite: List[torch.Tensor] = []

    def nonfinite_params(self) -> List[torch.Tensor]:
        """With ``check_finite=True``: the parameters whose update was not finite in
        the steps since the last call (a NaN or an infinity in the gradient; see
        ``_lib.nonfinite_tensors``), in step order, each once per step; from then on
        their state is not finite either. What to do then (restore a saved state,
        lower the loss scale, change optimizer) is the caller's choice. Clears the
        list."""
        out, self._nonfinite = self._nonfinite, []
        return out

    def _moment_dtype(self, p: torch.Tensor) -> torch.dtype:
        return moment_dtype(self._kind, p.shape, self._state_dtype, p.dtype, self._min_8bit_size)

    def _ws(self, nbytes: int, device) -> Optional[torch.Tensor]:
        if nbytes <= 0:
            return None
        ws = self._workspace.get(device)
        if ws is None or ws.numel() < nbytes:
            ws = _lib.workspace(nbytes, device)
            self._workspace[device] = ws
        return ws

    def load_state_dict(self, state_dict) -> None:
        """As torch's, except that state tensors keep the dtypes they were saved
        with: torch would cast them to the parameter's dtype, rounding the float32
        statistics of a bfloat16 parameter to bfloat16."""
        saved = state_dict["state"]
        super().load_state_dict(state_dict)
        ids = [i for g in state_dict["param_groups"] for i in g["params"]]
        params = [p for g in self.param_groups for p in g["params"]]
        for i, p in zip(ids, params):
            for key, v in saved.get(i, {}).items():
                if torch.is_tensor(v) and key != "step":
                    self.state[p][key] = v.to(device=p.device, copy=True).contiguous()

    def _state_for(self, p: torch.Tensor, group) -> Dict[str, torch.Tensor]:
        raise NotImplementedError

    def _call(self, group, step: int, params, grads, states, ws):
        raise NotImplementedError

    def _wsize(self, params, grads) -> int:
        raise NotImplementedError

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for group in self.param_groups:
            buckets: Dict[Tuple[torch.device, int], List[torch.Tensor]] = defaultdict(list)
            for p in group["params"]:
                if p.grad is None:
                    continue
                if p.grad.is_sparse:
                    raise RuntimeError(f"{type(self).__name__} does not support sparse gradients")
                st = self.state[p]
                if len(st) == 0:
                    st["step"] = 0
                    st.update(self._state_for(p, group))
                st["step"] += 1
                buckets[(p.device, st["step"])].append(p)
            for (device, step), ps in buckets.items():
                grads = [p.grad if p.grad.is_contiguous() else p.grad.contiguous() for p in ps]
                states = [self.state[p] for p in ps]
                ws = self._ws(self._wsize(ps, grads), device)
                with torch.cuda.device(device):
                    self._call(group, step, ps, grads, states, ws)
                    if self._check_finite:
                        # read before the next call reuses the workspace (one
                        # synchronisation per call)
                        offs = getattr(_lib, f"meo_{self._kind}_scalar_offsets")(ps, grads)
                        self._nonfinite.extend(ps[k] for k in _lib.nonfinite_tensors(self._kind, ws, offs))
        return loss


class Adafactor(_MeoOptimizer):
    """Adafactor with the page's defaults ("Step 3"): lr=None, eps=(1e-30, 1e-3),
    clip_threshold=1.0, decay_rate=-0.8, beta1=None, weight_decay=0.0,
    scale_parameter=True, relative_step=True, warmup_init=False. ``state_dtype``:
    element type of ``exp_avg`` (None: that of the parameter; torch.int8: 8-bit where
    ``moment_dtype`` allows, with ``min_8bit_size``).

    ``carry_param_sumsq``: with scale_parameter, keep each parameter's sum of
    squares from the step that stored it (state ``param_sumsq``) and take the next
    step's RMS(X) from it instead of reading the parameter again (4 or 2 bytes per
    parameter less HBM traffic per step). It is used only while every parameter of
    the call is unchanged since the previous step: the optimizer compares the
    parameter's version counter (bumped by every in-place operation on the
    parameter or its views), storage and the state tensor. Writes through
    ``param.data`` bypass the version counter; a caller that writes parameters
    that way must leave this off or call ``invalidate_param_sumsq()``."""

    _kind = "adafactor"
    _HP = ("lr", "eps", "clip_threshold", "decay_rate", "beta1", "weight_decay", "scale_parameter",
           "relative_step", "warmup_init")

    def __init__(self, params, lr=None, eps=(1e-30, 1e-3), clip_threshold=1.0, decay_rate=-0.8,
                 beta1=None, weight_decay=0.0, scale_parameter=True, relative_step=True,
                 warmup_init=False, state_dtype=None,
                 min_8bit_size=4096, carry_param_sumsq=False, check_finite=False):
        if lr is not None and relative_step:
            raise ValueError("Cannot combine manual lr and relative_step=True options")
        if warmup_init and not relative_step:
            raise ValueError("warmup_init=True requires relative_step=True")
        defaults = dict(lr=lr, eps=eps, clip_threshold=clip_threshold, decay_rate=decay_rate,
                        beta1=beta1, weight_decay=weight_decay, scale_parameter=scale_parameter,
                        relative_step=relative_step, warmup_init=warmup_init)
        super().__init__(params, defaults, state_dtype, min_8bit_size, check_finite)
        self._carry = bool(carry_param_sumsq)
        # id(param) -> (version, data_ptr, id of its param_sumsq) after the last carry step
        self._carried: Dict[int, Tuple[int, int, int]] = {}

    def invalidate_param_sumsq(self) -> None:
        """The next step reads every parameter for RMS(X) again."""
        self._carried.clear()

    def load_state_dict(self, state_dict) -> None:
        super().load_state_dict(state_dict)
        self._carried.clear()

    def _state_for(self, p, group):
        st = _lib.init_state("adafactor", p, beta1=group["beta1"] is not None,
                             state_dtype=self._moment_dtype(p))
        if self._carry:
            st["param_sumsq"] = torch.zeros(1, dtype=torch.float32, device=p.device)
        return st

    def _tag(self, p, st):
        return (p._version, p.data_ptr(), id(st["param_sumsq"]))

    def _wsize(self, params, grads):
        return _lib.meo_adafactor_workspace_size(params, grads)

    def _call(self, group, step, params, grads, states, ws):
        hp = _lib.adafactor_hparams(**{k: group[k] for k in self._HP})
        if not (self._carry and group["scale_parameter"]):
            _lib.meo_adafactor_step(hp, step, params, grads, states, ws)
            # the library's writes do not bump the version counter: a plain step
            # leaves any carried sum of these parameters stale
            for p in params:
                self._carried.pop(id(p), None)
            return
        for p, st in zip(params, states):
            if "param_sumsq" not in st:  # e.g. state loaded from a run without the carry
                st["param_sumsq"] = torch.zeros(1, dtype=torch.float32, device=p.device)
        valid = all(self._carried.get(id(p)) == self._tag(p, st) for p, st in zip(params, states))
        _lib.meo_adafactor_step_carry(hp, step, params, grads, states, valid, ws)
        for p, st in zip(params, states):
            self._carried[id(p)] = self._tag(p, st)


class CAME(_MeoOptimizer):
    """CAME with the page's defaults (DistributedCAME paragraph):
    eps=(1e-30, 1e-16), clip_threshold=1.0, betas=(0.9, 0.999, 0.9999),
    weight_decay=0.0; lr must be given. ``state_dtype``: element type of
    ``exp_avg`` (None: that of the parameter)."""

    _kind = "came"
    _HP = ("lr", "eps", "clip_threshold", "betas", "weight_decay")

    def __init__(self, params, lr=None, eps=(1e-30, 1e-16), clip_threshold=1.0,
                 betas=(0.9, 0.999, 0.9999), weight_decay=0.0, state_dtype=None,
                 min_8bit_size=4096, check_finite=False):
        if lr is None:
            raise ValueError("CAME requires an explicit lr")
        defaults = dict(lr=lr, eps=eps, clip_threshold=clip_threshold, betas=betas,
                        weight_decay=weight_decay)
        super().__init__(params, defaults, state_dtype, min_8bit_size, check_finite)

    def _state_for(self, p, group):
        return _lib.init_state("came", p, state_dtype=self._moment_dtype(p))

    def _wsize(self, params, grads):
        return _lib.meo_came_workspace_size(params, grads)

    def _call(self, group, step, params, grads, states, ws):
        hp = _lib.came_hparams(**{k: group[k] for k in self._HP})
        _lib.meo_came_step(hp, step, params, grads, states, ws)


class Lamb(_MeoOptimizer):
    """LAMB with the page's defaults (DistributedLAMB paragraph): lr=1e-3,
    betas=(0.9, 0.999), eps=1e-6, weight_decay=0, bias_correction=True.
    ``state_dtype``: element type of ``exp_avg`` (None: that of the parameter);
    ``exp_avg_sq`` is float32."""

    _kind = "lamb"
    _HP = ("lr", "betas", "eps", "weight_decay", "bias_correction")

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-6, weight_decay=0.0,
                 bias_correction=True, state_dtype=None,
                 min_8bit_size=4096, check_finite=False):
        if not lr >= 0.0:
            raise ValueError(f"Invalid learning rate: {lr}")
        if not eps >= 0.0:
            raise ValueError(f"Invalid epsilon value: {eps}")
        for i, b in enumerate(betas):
            if not 0.0 <= b < 1.0:
                raise ValueError(f"Invalid beta parameter at index {i}: {b}")
        defaults = dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay,
                        bias_correction=bias_correction)
        super().__init__(params, defaults, state_dtype, min_8bit_size, check_finite)

    def _state_for(self, p, group):
        return _lib.init_state("lamb", p, state_dtype=self._moment_dtype(p))

    def _wsize(self, params, grads):
        return _lib.meo_lamb_workspace_size(params, grads)

    def _call(self, group, step, params, grads, states, ws):
        hp = _lib.lamb_hparams(**{k: group[k] for k in self._HP})
        _lib.meo_lamb_step(hp, step, params, grads, states, ws)


_NO_DECAY = ("bias", "LayerNorm.weight")


def get_galore_param_groups(model: torch.nn.Module, weight_decay: float, rank: int = 256,
                            update_proj_gap: int = 200, scale: float = 0.25, proj_type: str = "std"):
    """Parameter groups for ``GaLoreAdamW``, following the grouping rule of the
    Colossal-AI page's GaLore section: 2-D parameters get the projection fields
    (rank, update_proj_gap, scale, proj_type) and ``weight_decay``; the other
    parameters take plain AdamW with ``weight_decay``; parameters whose name holds
    ``bias`` or ``LayerNorm.weight`` take no weight decay (the no-decay rule is
    applied first). Empty groups are left out."""
    galore, other, no_decay = [], [], []
    for name, p in model.named_parameters():
        if not p.requires_grad:
            continue
        if any(nd in name for nd in _NO_DECAY):
            no_decay.append(p)
        elif p.dim() == 2:
            galore.append(p)
        else:
            other.append(p)
    groups = [dict(params=galore, weight_decay=weight_decay, rank=rank, update_proj_gap=update_proj_gap,
                   scale=scale, proj_type=proj_type),
              dict(params=other, weight_decay=weight_decay),
              dict(params=no_decay, weight_decay=0.0)]
    return [g for g in groups if g["params"]]


class GaLoreAdamW(_MeoOptimizer):
    """AdamW under GaLore's low-rank gradient projection (the Colossal-AI page's
    GaLore section, with its group fields; the ms-swift page's low-rank projection).

    A parameter group with a ``rank`` field projects its 2-D parameters: every
    ``update_proj_gap`` steps (default 200) the projector is refreshed from the
    gradient's leading ``rank`` singular vectors (default 256) on the shorter side,
    AdamW runs on the projected gradient, and the update is projected back and
    multiplied by ``scale`` (default 0.25). ``proj_type`` "std" (default) projects
    along the shorter side of each matrix, "reverse_std" along the longer. Groups
    without ``rank``, and the other parameters of a group with one, take plain
    AdamW. Weight decay is decoupled (applied to the parameter before the update).

    The projection runs on bf16 matrix cores: a projected parameter's gradient is
    read in bfloat16 (converted if it is float32), and its projector is kept in
    bfloat16. States: ``exp_avg`` and ``exp_avg_sq`` float32 ([max(m, n)][r] when
    projected), ``projector`` [min(m, n)][r] and ``projector_t`` [r][min(m, n)]."""

    _kind = "galore"

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0):
        if not lr >= 0.0:
            raise ValueError(f"Invalid learning rate: {lr}")
        if not eps >= 0.0:
            raise ValueError(f"Invalid epsilon value: {eps}")
        for i, b in enumerate(betas):
            if not 0.0 <= b < 1.0:
                raise ValueError(f"Invalid beta parameter at index {i}: {b}")
        defaults = dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay)
        super().__init__(params, defaults, None)
        for g in self.param_groups:
            if "rank" in g:
                g.setdefault("update_proj_gap", 200)
                g.setdefault("scale", 0.25)
                g.setdefault("proj_type", "std")
                if g["proj_type"] not in ("std", "reverse_std"):
                    raise ValueError("proj_type must be 'std' or 'reverse_std'")

    @staticmethod
    def _projected(p: torch.Tensor, group) -> bool:
        return "rank" in group and p.dim() == 2 and p.numel() > 0

    def _state_for(self, p, group):
        if self._projected(p, group):
            return _lib.galore_init_state(p, group["rank"], group["proj_type"])
        return {k: torch.zeros(p.shape, dtype=torch.float32, device=p.device) for k in ("exp_avg", "exp_avg_sq")}

    def _lists(self, group, params, grads, states):
        # Tensors that are not projected go to the library as flat views, which it
        # steps with AdamW whatever their shape.
        ps, gs, ss = [], [], []
        for p, g, st in zip(params, grads, states):
            if self._projected(p, group):
                ps.append(p)
                gs.append(g if g.dtype == torch.bfloat16 else g.to(torch.bfloat16))
                ss.append(st)
            else:
                ps.append(p.view(-1))
                gs.append(g.reshape(-1))
                ss.append({k: st[k].view(-1) for k in ("exp_avg", "exp_avg_sq")})
        return ps, gs, ss

    def _hp(self, group):
        return _lib.galore_hparams(lr=group["lr"], betas=group["betas"], eps=group["eps"],
                                   weight_decay=group["weight_decay"], rank=group.get("rank", 256),
                                   update_proj_gap=group.get("update_proj_gap", 200),
                                   scale=group.get("scale", 0.25), proj_type=group.get("proj_type", "std"))

    def _wsize(self, params, grads):
        return 0  # computed in _call, where the group is known

    def _call(self, group, step, params, grads, states, ws):
        ps, gs, ss = self._lists(group, params, grads, states)
        hp = self._hp(group)
        ws = self._ws(_lib.meo_galore_workspace_size(hp, ps, gs), ps[0].device)
        _lib.meo_galore_step(hp, step, ps, gs, ss, ws)
