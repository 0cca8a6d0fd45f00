"""Plain fp64 NumPy oracle for one GaLore step (low-rank projected AdamW).

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import this module; the library never does, and it
shares no code, constant table or helper with the HIP path.

Sources (the pages):

* Colossal-AI distributed-optimizers page ("Colossal-AI 分布式优化器全解析",
  blog.gitcode.com), section "GaLore 的特殊配置": the group-level fields rank
  (default 256), update_proj_gap (200: how often the SVD that refreshes the
  orthogonal projection matrix is redone), scale (0.25: the factor applied when
  projecting back to full rank) and proj_type ("std"); the projector keeps a
  periodically refreshed orthogonal matrix, project() maps the full-rank
  gradient to a low-rank one that takes part in the update, project_back()
  multiplies by scale to restore the full shape, and the optimizer state shrinks
  by about rank / min(m, n). Only 2-D parameters are projected; the others take
  a plain AdamW update. The optimizer under the projection is AdamW (the
  DistGaloreAwamW example: lr, betas, eps; weight decay per group).
* ms-swift page ("ms-swift optimizer 扩展实践", section "低秩投影的艺术"): the
  gradient is approximated through its SVD and only the leading r singular
  directions are kept; Adam runs in the low-rank space and its update is
  projected back.

Readings where the pages are silent (each is marked "reading" where applied):

* proj_type "std" projects along the shorter side of the matrix: for m >= n the
  low-rank gradient is G Q with Q (n x r) the leading right singular vectors;
  for m < n it is P^T G with P (m x r) the leading left singular vectors. This
  is the only choice that gives the rank / min(m, n) state compression the page
  states. "reverse_std", which the page names beside it, is the other side: P^T G
  for m >= n, G Q for m < n. The low-rank tensors are kept as [rows][r] arrays:
  G Q is m x r; P^T G is stored transposed, n x r.
* The effective rank is min(rank, min(m, n)).
* The projector is (re)computed from the current gradient at steps t with
  (t - 1) % update_proj_gap == 0, before projecting; the Adam moments are kept
  across refreshes.
* Singular vectors are defined up to sign: each kept vector is signed so that
  its entry of largest magnitude (the first such entry on a tie) is positive.
* The projector is stored in the gradient's 16-bit type (bfloat16, rounded to
  nearest even) when the gradient is bf16, so that both products run on 16-bit
  matrix inputs; the projected Adam direction itself stays float32.
* AdamW in the low-rank space: m <- b1 m + (1 - b1) R, v <- b2 v + (1 - b2) R^2,
  N = (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps); decoupled weight decay on
  the full parameter before the update: x <- x (1 - lr wd) - lr scale back(N).
  Non-projected tensors take the same AdamW update with N in place of back(N)
  and no scale. Defaults where the pages give none: lr 1e-3, betas (0.9, 0.999),
  eps 1e-8, weight_decay 0.
* nbits = 8 (block-wise 8-bit states of the bitsandbytes base, whose format the
  page defers to that library) is not covered: states are float32.

Functions take and return new arrays; nothing is modified in place. ``t`` is the
1-based index of the step being taken.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .optimizers import round_bf16

Array = np.ndarray
State = Dict[str, Array]

# Section "GaLore 的特殊配置": rank, update_proj_gap, scale, proj_type. AdamW
# fields: reading (the pages name them without values).
GALORE_DEFAULTS = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                       rank=256, update_proj_gap=200, scale=0.25, proj_type="std")


def galore_hparams(hp: Optional[dict] = None) -> dict:
    out = dict(GALORE_DEFAULTS)
    if hp:
        unknown = set(hp) - set(out)
        if unknown:
            raise TypeError(f"unknown GaLore hyperparameters: {sorted(unknown)}")
        out.update(hp)
    if out["proj_type"] not in ("std", "reverse_std"):
        raise ValueError("proj_type must be 'std' or 'reverse_std'")
    if not (isinstance(out["rank"], int) and out["rank"] >= 1):
        raise ValueError("rank must be a positive integer")
    if not (isinstance(out["update_proj_gap"], int) and out["update_proj_gap"] >= 1):
        raise ValueError("update_proj_gap must be a positive integer")
    return out


def is_projected(shape: Tuple[int, ...]) -> bool:
    """Page section "GaLore 的特殊配置", grouping rule 1: 2-D parameters only."""
    return len(shape) == 2


def galore_side(shape: Tuple[int, int], proj_type: str = "std") -> str:
    """"right" (R = G Q, Q from the right singular vectors) or "left" (R = P^T G, P
    from the left ones): std takes the shorter side, reverse_std the longer (reading)."""
    m, n = shape
    short_is_cols = m >= n
    return "right" if short_is_cols == (proj_type == "std") else "left"


def galore_rank(shape: Tuple[int, int], rank: int) -> int:
    return min(rank, min(shape))  # reading


def canonical_signs(u: Array) -> Array:
    """Sign each column so that its largest-magnitude entry is positive (reading)."""
    u = np.array(u, dtype=np.float64)
    for k in range(u.shape[1]):
        i = int(np.argmax(np.abs(u[:, k])))
        if u[i, k] < 0:
            u[:, k] = -u[:, k]
    return u


def galore_projector(g: Array, rank: int, *, projector_bf16: bool = True, proj_type: str = "std") -> Array:
    """The orthonormal basis of the leading singular directions on the projected side.

    right: the leading right singular vectors of G (columns of V), n x r;
    left: the leading left singular vectors (columns of U of the SVD), m x r.
    """
    g = np.asarray(g, dtype=np.float64)
    r = galore_rank(g.shape, rank)
    left, _, vt = np.linalg.svd(g, full_matrices=False)  # library SVD as one step
    basis = vt[:r].T if galore_side(g.shape, proj_type) == "right" else left[:, :r]
    basis = canonical_signs(basis)
    return round_bf16(basis) if projector_bf16 else basis


def galore_project(g: Array, u: Array, proj_type: str = "std") -> Array:
    """project(): the low-rank gradient, m x r for the right side, (P^T G)^T (n x r)
    for the left."""
    g = np.asarray(g, dtype=np.float64)
    return g @ u if galore_side(g.shape, proj_type) == "right" else g.T @ u


def galore_project_back(n_low: Array, u: Array, shape: Tuple[int, int], scale: float,
                        proj_type: str = "std") -> Array:
    """project_back(): the full-shape update, scale times the back-projection."""
    full = n_low @ u.T if galore_side(shape, proj_type) == "right" else u @ n_low.T
    return scale * full


def galore_init_state(shape: Tuple[int, ...], hp: Optional[dict] = None) -> State:
    h = galore_hparams(hp)
    if is_projected(shape):
        r = galore_rank(shape, h["rank"])
        m, n = shape
        rows, basis = (m, n) if galore_side(shape, h["proj_type"]) == "right" else (n, m)
        return dict(exp_avg=np.zeros((rows, r)), exp_avg_sq=np.zeros((rows, r)),
                    projector=np.zeros((basis, r)))
    return dict(exp_avg=np.zeros(shape), exp_avg_sq=np.zeros(shape))


def _adam_direction(m: Array, v: Array, h: dict, t: int) -> Array:
    b1, b2 = h["betas"]
    return (m / (1.0 - b1 ** t)) / (np.sqrt(v / (1.0 - b2 ** t)) + h["eps"])


def galore_refresh_due(h: dict, t: int) -> bool:
    return (t - 1) % h["update_proj_gap"] == 0  # reading


def galore_step_tensor(x: Array, g: Array, state: State, hp: Optional[dict], t: int, *,
                       param_bf16: bool = False, projector_bf16: bool = True) -> Tuple[Array, State]:
    """One step for one tensor; returns (new parameter, new state)."""
    h = galore_hparams(hp)
    if t < 1:
        raise ValueError("step must be >= 1")
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    b1, b2 = h["betas"]
    new: State = {}
    if is_projected(x.shape):
        u = np.asarray(state["projector"], dtype=np.float64)
        if galore_refresh_due(h, t):
            u = galore_projector(g, h["rank"], projector_bf16=projector_bf16, proj_type=h["proj_type"])
        new["projector"] = u
        low = galore_project(g, u, h["proj_type"])
    else:
        low = g
    m = b1 * state["exp_avg"] + (1.0 - b1) * low
    v = b2 * state["exp_avg_sq"] + (1.0 - b2) * low * low
    new["exp_avg"], new["exp_avg_sq"] = m, v
    direction = _adam_direction(m, v, h, t)
    if is_projected(x.shape):
        update = galore_project_back(direction, new["projector"], x.shape, h["scale"], h["proj_type"])
    else:
        update = direction
    x_new = x * (1.0 - h["lr"] * h["weight_decay"]) - h["lr"] * update
    if param_bf16:
        x_new = round_bf16(x_new)
    return x_new, new


def galore_step(xs: Sequence[Array], gs: Sequence[Array], states: Sequence[State],
                hp: Optional[dict], t: int, **storage) -> Tuple[list, list]:
    out_x, out_s = [], []
    for x, g, s in zip(xs, gs, states):
        a, b = galore_step_tensor(x, g, s, hp, t, **storage)
        out_x.append(a)
        out_s.append(b)
    return out_x, out_s
