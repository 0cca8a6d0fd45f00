"""Seeded synthetic workloads for the optimizer step.

This module holds shapes, initial parameter values and gradient draws only: no
optimizer arithmetic. Both the fp64 oracle (through the tests and the bench's CPU
leg) and the HIP library are fed from here, so a parity check always compares the
two on the same bits.

Shapes are model architectures (a Llama-7B decoder stack and BERT-large), not data
items: the optimizer step sees only parameter and gradient tensors, so synthetic
gradients with the statistics described below stand in for real training
gradients.

Random streams. Every tensor k of a workload draws from its own torch generator
seeded with ``seed * 2**20 + k * 2**8 + stream``; stream 0 is the initial value,
stream 1 the fixed per-tensor gradient scales, stream 2 + s the N(0, 1) noise of
step s (0-based). A generator lives on the device the tensors are made on, so the
CPU and a GPU draw different (but each reproducible) values; parity tests copy
the GPU's draws to the host for the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    kind: str  # "weight" (N(0, 0.02) init), "norm" (ones), "bias" (zeros)

    @property
    def numel(self) -> int:
        return math.prod(self.shape)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    optimizer: str  # "adafactor" | "came" | "lamb"
    hparams: Dict[str, object]
    specs: Tuple[TensorSpec, ...]
    grad_dtype: torch.dtype
    grad_std: float
    grad_scaling: str  # "row": per-row scale; "rowcol": row x col scales; "none"
    steps: int
    seed: int = 0
    param_dtype: torch.dtype = torch.float32   # storage of the parameter
    state_dtype: torch.dtype = torch.float32   # storage of the first moment (exp_avg); int8 applies
                                               # where the optimizer's 8-bit rule allows it

    @property
    def numel(self) -> int:
        return sum(s.numel for s in self.specs)


# ----------------------------------------------------------------------------- shapes

def llama_layer_specs(prefix: str = "", hidden: int = 4096, ffn: int = 11008) -> List[TensorSpec]:
    """One Llama decoder layer in parameter order: attention q, k, v, o, MLP gate,
    up, down, then the two RMSNorm weights."""
    h, f = hidden, ffn
    return [
        TensorSpec(prefix + "self_attn.q_proj.weight", (h, h), "weight"),
        TensorSpec(prefix + "self_attn.k_proj.weight", (h, h), "weight"),
        TensorSpec(prefix + "self_attn.v_proj.weight", (h, h), "weight"),
        TensorSpec(prefix + "self_attn.o_proj.weight", (h, h), "weight"),
        TensorSpec(prefix + "mlp.gate_proj.weight", (f, h), "weight"),
        TensorSpec(prefix + "mlp.up_proj.weight", (f, h), "weight"),
        TensorSpec(prefix + "mlp.down_proj.weight", (h, f), "weight"),
        TensorSpec(prefix + "input_layernorm.weight", (h,), "norm"),
        TensorSpec(prefix + "post_attention_layernorm.weight", (h,), "norm"),
    ]


def llama_specs(layers: int = 32, hidden: int = 4096, ffn: int = 11008, vocab: int = 32000) -> List[TensorSpec]:
    """A Llama causal LM in parameter order: embedding, decoder layers, final norm, lm_head."""
    out = [TensorSpec("model.embed_tokens.weight", (vocab, hidden), "weight")]
    for i in range(layers):
        out += llama_layer_specs(f"model.layers.{i}.", hidden, ffn)
    out.append(TensorSpec("model.norm.weight", (hidden,), "norm"))
    out.append(TensorSpec("lm_head.weight", (vocab, hidden), "weight"))
    return out


def bert_specs(layers: int = 24, hidden: int = 1024, ffn: int = 4096, vocab: int = 30522,
               max_pos: int = 512) -> List[TensorSpec]:
    """A BERT encoder in parameter order: word and position embeddings and their
    LayerNorm, then per layer q, k, v, o (+ biases), FFN in/out (+ biases) and two
    LayerNorms (weight and bias each)."""
    h, f = hidden, ffn
    out = [
        TensorSpec("embeddings.word_embeddings.weight", (vocab, h), "weight"),
        TensorSpec("embeddings.position_embeddings.weight", (max_pos, h), "weight"),
        TensorSpec("embeddings.LayerNorm.weight", (h,), "norm"),
        TensorSpec("embeddings.LayerNorm.bias", (h,), "bias"),
    ]
    for i in range(layers):
        p = f"encoder.layer.{i}."
        for n in ("attention.self.query", "attention.self.key", "attention.self.value",
                  "attention.output.dense"):
            out.append(TensorSpec(p + n + ".weight", (h, h), "weight"))
            out.append(TensorSpec(p + n + ".bias", (h,), "bias"))
        out.append(TensorSpec(p + "attention.output.LayerNorm.weight", (h,), "norm"))
        out.append(TensorSpec(p + "attention.output.LayerNorm.bias", (h,), "bias"))
        out.append(TensorSpec(p + "intermediate.dense.weight", (f, h), "weight"))
        out.append(TensorSpec(p + "intermediate.dense.bias", (f,), "bias"))
        out.append(TensorSpec(p + "output.dense.weight", (h, f), "weight"))
        out.append(TensorSpec(p + "output.dense.bias", (h,), "bias"))
        out.append(TensorSpec(p + "output.LayerNorm.weight", (h,), "norm"))
        out.append(TensorSpec(p + "output.LayerNorm.bias", (h,), "bias"))
    return out


# ----------------------------------------------------------------------------- workloads

_AF_DEFAULT: Dict[str, object] = {}
_AF_BETA1 = {"beta1": 0.9}
_CAME = {"lr": 2e-4, "betas": (0.9, 0.999, 0.9999), "eps": (1e-30, 1e-16),
         "clip_threshold": 1.0, "weight_decay": 0.0}
_LAMB = {"lr": 1e-3, "betas": (0.9, 0.999), "eps": 1e-6, "weight_decay": 0.01,
         "bias_correction": True}


def _wl(name, opt, hp, specs, gdt, gstd, scaling, steps):
    return Workload(name, opt, dict(hp), tuple(specs), gdt, gstd, scaling, steps)


WORKLOADS: Dict[str, Workload] = {}


def _register(w: Workload) -> None:
    WORKLOADS[w.name] = w


# The five measured configurations.
_register(_wl("adafactor_small", "adafactor", _AF_DEFAULT,
              [TensorSpec("weight", (256, 512), "weight"), TensorSpec("bias", (512,), "bias")],
              torch.float32, 1.0, "row", 10))
_register(_wl("adafactor_llama_layer", "adafactor", _AF_BETA1, llama_layer_specs(),
              torch.bfloat16, 1e-3, "rowcol", 20))
_register(_wl("adafactor_llama7b", "adafactor", _AF_BETA1, llama_specs(),
              torch.bfloat16, 1e-3, "rowcol", 5))
_register(_wl("came_llama_layer", "came", _CAME, llama_layer_specs(),
              torch.bfloat16, 1e-3, "rowcol", 20))
_register(_wl("lamb_bert_large", "lamb", _LAMB, bert_specs(),
              torch.float32, 1e-2, "none", 20))

# CAME and LAMB over the same Llama-7B-shaped list as the headline (measurement at
# that scale; bf16 gradients as in the Adafactor 7B configuration).
_register(_wl("came_llama7b", "came", _CAME, llama_specs(), torch.bfloat16, 1e-3, "rowcol", 5))
_register(_wl("lamb_llama7b", "lamb", _LAMB, llama_specs(), torch.bfloat16, 1e-3, "rowcol", 5))

# 16-bit storage: the 7B and one-layer Adafactor configurations with bf16
# parameters and bf16 first moments.
_register(dataclasses.replace(WORKLOADS["adafactor_llama7b"], name="adafactor_llama7b_bf16",
                              param_dtype=torch.bfloat16, state_dtype=torch.bfloat16))
_register(dataclasses.replace(WORKLOADS["adafactor_llama_layer"], name="adafactor_llama_layer_bf16",
                              param_dtype=torch.bfloat16, state_dtype=torch.bfloat16))
# 8-bit first moment (fp32 parameters and statistics).
_register(dataclasses.replace(WORKLOADS["adafactor_llama7b"], name="adafactor_llama7b_i8", state_dtype=torch.int8))
_register(dataclasses.replace(WORKLOADS["adafactor_llama_layer"], name="adafactor_llama_layer_i8",
                              state_dtype=torch.int8))
_register(dataclasses.replace(WORKLOADS["came_llama_layer"], name="came_llama_layer_i8", state_dtype=torch.int8))
_register(dataclasses.replace(WORKLOADS["lamb_bert_large"], name="lamb_bert_large_i8", state_dtype=torch.int8))

# Scaled-down versions of the same structure (ragged widths included) that the
# oracle runs element by element in seconds.
_register(_wl("adafactor_llama_mini", "adafactor", _AF_BETA1,
              llama_specs(layers=2, hidden=256, ffn=688, vocab=1000),
              torch.bfloat16, 1e-3, "rowcol", 10))
_register(_wl("came_llama_mini", "came", _CAME,
              llama_specs(layers=2, hidden=256, ffn=688, vocab=1000),
              torch.bfloat16, 1e-3, "rowcol", 10))
_register(_wl("lamb_bert_mini", "lamb", _LAMB,
              bert_specs(layers=2, hidden=128, ffn=512, vocab=3001, max_pos=64),
              torch.float32, 1e-2, "none", 10))

# Scaled-down 16-bit-storage and 8-bit-moment versions.
for _n in ("adafactor_llama_mini", "came_llama_mini", "lamb_bert_mini"):
    _register(dataclasses.replace(WORKLOADS[_n], name=_n + "_bf16", param_dtype=torch.bfloat16,
                                  state_dtype=torch.bfloat16))
    _register(dataclasses.replace(WORKLOADS[_n], name=_n + "_i8", state_dtype=torch.int8))
del _n


def custom(name: str, optimizer: str, shapes: Sequence[Tuple[int, ...]], *, hparams=None,
           grad_dtype=torch.float32, grad_std=1.0, grad_scaling="row", steps=3,
           kinds: Optional[Sequence[str]] = None, seed: int = 0,
           param_dtype=torch.float32, state_dtype=torch.float32) -> Workload:
    """An ad-hoc workload over the given shapes (edge cases in tests)."""
    specs = []
    for i, shp in enumerate(shapes):
        kind = kinds[i] if kinds else ("weight" if len(shp) >= 2 else "norm")
        specs.append(TensorSpec(f"t{i}", tuple(int(s) for s in shp), kind))
    return Workload(name, optimizer, dict(hparams or {}), tuple(specs), grad_dtype, grad_std,
                    grad_scaling, steps, seed, param_dtype, state_dtype)


# ----------------------------------------------------------------------------- draws

def _gen(wl: Workload, k: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * (1 << 20) + k * (1 << 8) + stream)
    return g


def _pick(wl: Workload, indices):
    ks = range(len(wl.specs)) if indices is None else indices
    return [(k, wl.specs[k]) for k in ks]


def init_params(wl: Workload, device="cpu", indices=None, out=None) -> List[torch.Tensor]:
    """Parameters of the workload's param dtype: 2-D+ weights N(0, 0.02) drawn in
    fp32 (then rounded to a 16-bit dtype), norm weights 1, biases 0. ``indices``
    selects tensors (same draws as in the full list); ``out`` gives tensors of the
    param dtype to fill in place (e.g. views into one flat buffer)."""
    res = []
    for j, (k, s) in enumerate(_pick(wl, indices)):
        t = out[j] if out is not None else torch.empty(s.shape, dtype=wl.param_dtype, device=device)
        if s.kind == "weight":
            if t.dtype == torch.float32:
                t.normal_(0.0, 0.02, generator=_gen(wl, k, 0, t.device))
            else:
                w = torch.empty(s.shape, dtype=torch.float32, device=t.device)
                t.copy_(w.normal_(0.0, 0.02, generator=_gen(wl, k, 0, t.device)))
        elif s.kind == "norm":
            t.fill_(1.0)
        else:
            t.zero_()
        res.append(t)
    return res


def _log_uniform(n: int, gen: torch.Generator, device) -> torch.Tensor:
    u = torch.empty(n, dtype=torch.float32, device=device).uniform_(-2.0, 2.0, generator=gen)
    return torch.pow(10.0, u)


def grad_scales(wl: Workload, device="cpu", indices=None
                ) -> List[Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]]:
    """Per-tensor fixed scales, drawn once: 10**U(-2, 2) over rows (dim -2) and,
    for "rowcol", over columns (dim -1). 1-D tensors get one scale per element."""
    out = []
    for k, s in _pick(wl, indices):
        if wl.grad_scaling == "none":
            out.append((None, None))
            continue
        gen = _gen(wl, k, 1, device)
        if len(s.shape) < 2:
            out.append((_log_uniform(max(s.numel, 1), gen, device).reshape(s.shape), None))
            continue
        a = _log_uniform(s.shape[-2], gen, device)
        b = _log_uniform(s.shape[-1], gen, device) if wl.grad_scaling == "rowcol" else None
        out.append((a, b))
    return out


def grads(wl: Workload, step_index: int, scales, device="cpu", indices=None, out=None) -> List[torch.Tensor]:
    """Gradients of 0-based step ``step_index``: std * z * row_scale * col_scale,
    z ~ N(0, 1) redrawn each step, computed in fp32 then cast to the grad dtype.
    ``scales`` must come from grad_scales with the same ``indices``; ``out`` gives
    tensors of the grad dtype to fill in place."""
    res = []
    for j, (k, s) in enumerate(_pick(wl, indices)):
        z = torch.empty(s.shape, dtype=torch.float32, device=device)
        z.normal_(0.0, 1.0, generator=_gen(wl, k, 2 + step_index, device))
        g = z * wl.grad_std
        a, b = scales[j]
        if a is not None:
            if len(s.shape) < 2:
                g = g * a
            else:
                g = g * a.unsqueeze(-1)
                if b is not None:
                    g = g * b
        if out is not None:
            out[j].copy_(g)
            res.append(out[j])
        else:
            res.append(g.to(wl.grad_dtype).contiguous())
    return res


# ----------------------------------------------------------------------------- GaLore

def galore_inputs(shapes: Sequence[Tuple[int, ...]], rank: int, seed: int = 0, *,
                  param_dtype=torch.float32, device="cpu", gstd: float = 1e-3,
                  state: str = "seeded", spectrum: Optional[Tuple[float, float, int]] = None,
                  proj_type: str = "std"):
    """Parameters, bf16 gradients and GaLore states (meo.h layout) for `shapes`.

    Drawn on the CPU from torch.Generator(seed) (the same bits on every device),
    then moved to `device`. Parameters N(0, 0.02); gradients N(0, gstd^2), or, with
    ``spectrum = (decay, noise, k)``, a rank-k signal plus noise, U diag(s) V^T +
    E with s_i = gstd * sqrt(max(m, n)) * decay^i for i < k (random orthonormal U,
    V) and E ~ N(0, (noise * gstd)^2): the low-rank structure the projection relies
    on, with a spectral gap after the k-th singular value. With
    ``state = "seeded"`` the moments of a mid-run step are drawn (exp_avg
    N(0, gstd^2 / 4), exp_avg_sq gstd^2 * U(0.5, 1.5)) and each 2-D tensor gets a
    random orthonormal projector (QR of a Gaussian) rounded to bf16, stored with
    its transpose; with ``state = "zero"`` everything starts at zero. State shapes
    follow ``proj_type`` (the projector on the shorter side for "std", the longer for
    "reverse_std").
    """
    gen = torch.Generator().manual_seed(seed)
    params, grads, states = [], [], []
    for shape in shapes:
        shape = tuple(shape)
        x = (0.02 * torch.randn(shape, generator=gen, dtype=torch.float64)).to(param_dtype)
        if spectrum is not None and len(shape) == 2:
            m, n = shape
            k = min(m, n, spectrum[2])
            qa, _ = torch.linalg.qr(torch.randn(m, k, generator=gen, dtype=torch.float64))
            qb, _ = torch.linalg.qr(torch.randn(n, k, generator=gen, dtype=torch.float64))
            s = gstd * math.sqrt(max(m, n)) * spectrum[0] ** torch.arange(k, dtype=torch.float64)
            g = (qa * s) @ qb.T + spectrum[1] * gstd * torch.randn(m, n, generator=gen, dtype=torch.float64)
        else:
            g = gstd * torch.randn(shape, generator=gen, dtype=torch.float64)
        g = g.to(torch.bfloat16)
        projected = len(shape) == 2 and shape[0] > 0 and shape[1] > 0
        if projected:
            r = min(rank, min(shape))
            d = min(shape) if proj_type == "std" else max(shape)
            mshape = (shape[0] * shape[1] // d, r)
        else:
            mshape = shape
        if state == "seeded":
            st = {"exp_avg": (0.5 * gstd * torch.randn(mshape, generator=gen, dtype=torch.float64)).float(),
                  "exp_avg_sq": (gstd * gstd * (0.5 + torch.rand(mshape, generator=gen, dtype=torch.float64))).float()}
            if projected:
                q, _ = torch.linalg.qr(torch.randn(d, r, generator=gen, dtype=torch.float64))
                st["projector"] = q.to(torch.bfloat16).contiguous()  # QR returns column-major Q
        else:
            st = {"exp_avg": torch.zeros(mshape), "exp_avg_sq": torch.zeros(mshape)}
            if projected:
                st["projector"] = torch.zeros((d, r), dtype=torch.bfloat16)
        if projected:
            st["projector_t"] = st["projector"].T.contiguous()
        params.append(x.to(device))
        grads.append(g.to(device))
        states.append({k: v.to(device) for k, v in st.items()})
    return params, grads, states
