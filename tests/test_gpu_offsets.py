"""Tensors carved from one flat buffer at element offsets that keep their dtype's
alignment but not 16 bytes (fp32 offsets 1, 2, 3; bf16 offsets 1 .. 7), as
flat-parameter frameworks hand them over. The library must take its unaligned
paths for them: the element-wise loads and, for factored tensors, the tiled
first pass, whose workspace layout differs from the row-complete one. Checked:
the workspace size and scalar layout are those of the unaligned path, and three
chained steps match the oracle under the usual bars, for every optimizer and
storage class (fp32; bf16 parameter and first moment; 8-bit first moment)."""
import pytest
import torch

import oracle
import workloads
from memory_efficient_optimizers_amd import _lib
from memory_efficient_optimizers_amd.optim import moment_dtype
from tests.harness import (failures, judge_tensor, lib_hp, lib_scalar_offsets, lib_step, storage_of_tensor,
                           summarize, to64)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


# W % 8 == 0 everywhere (the aligned layout would take the vector paths); widths
# that are multiples of 128 so that an 8-bit first moment applies.
SHAPES = [(65, 512), (33, 1024), (2, 40, 256), (1000,), (8, 128)]


def _carve(shapes, dtype, offset, fill=None):
    """Views of `shapes` in one buffer, the first starting `offset` elements in
    and each next one right after the previous (so none is 16-byte aligned unless
    by chance), and the buffer itself."""
    sizes = [int(torch.Size(s).numel()) for s in shapes]
    buf = torch.zeros(offset + sum(sizes) + 16, dtype=dtype, device="cuda")
    views, o = [], offset
    for n, s in zip(sizes, shapes):
        views.append(buf[o:o + n].view(s))
        o += n
    return views


def _misaligned(t):
    return t.data_ptr() % 16 != 0


CASES = [
    ("adafactor", {"beta1": 0.9, "weight_decay": 0.1}, "f32"),
    ("adafactor", {"beta1": 0.9}, "bf16"),
    ("adafactor", {"beta1": 0.9}, "i8"),
    ("adafactor", {}, "f32"),
    ("came", {"lr": 2e-4, "weight_decay": 0.05}, "f32"),
    ("came", {"lr": 2e-4}, "bf16"),
    ("came", {"lr": 2e-4}, "i8"),
    ("lamb", {"weight_decay": 0.01}, "f32"),
    ("lamb", {"weight_decay": 0.01}, "bf16"),
    ("lamb", {"weight_decay": 0.01}, "i8"),
]


# fp32 parameters: offsets 1-3 cover every 4-byte misalignment; bf16 ones: 1, 2, 3, 5, 7
OFFSET_CASES = [(opt, hp, store, offset) for opt, hp, store in CASES
                for offset in ([1, 2, 3, 5, 7] if store == "bf16" else [1, 2, 3])]


@pytest.mark.parametrize("opt,hp,store,offset", OFFSET_CASES)
def test_offset_views(opt, hp, store, offset):
    pdt = torch.bfloat16 if store == "bf16" else torch.float32
    sdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}[store]
    wl = workloads.custom(f"offs_{opt}", opt, SHAPES, hparams=hp, grad_dtype=torch.bfloat16, grad_std=1e-3,
                          grad_scaling="rowcol", param_dtype=pdt, state_dtype=sdt)
    ps = _carve(SHAPES, pdt, offset)
    workloads.init_params(wl, "cuda", out=ps)
    gs = _carve(SHAPES, torch.bfloat16, offset)
    scales = workloads.grad_scales(wl, "cuda")
    beta1 = hp.get("beta1") is not None or opt != "adafactor"
    mdts = [moment_dtype(opt, s, sdt, pdt, 0) for s in SHAPES]
    # every state as its own allocation except the first moment, carved too
    sts = [_lib.init_state(opt, p, beta1=beta1, state_dtype=m) for p, m in zip(ps, mdts)]
    if beta1 and store != "i8":
        moments = _carve(SHAPES, sdt, offset)
        for st, m in zip(sts, moments):
            st["exp_avg"] = m
    assert all(_misaligned(p) for p in ps) and all(_misaligned(g) for g in gs)
    # the unaligned layout: the factored tensors' workspace is that of the tiled
    # first pass, not of the row-complete one the same shapes take when aligned
    aligned_p = [torch.zeros(s, dtype=pdt, device="cuda") for s in SHAPES]
    aligned_g = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in SHAPES]
    wsize = getattr(_lib, f"meo_{opt}_workspace_size")
    if opt != "lamb":
        assert wsize(ps, gs) != wsize(aligned_p, aligned_g)
    storage = [storage_of_tensor(p, st) for p, st in zip(ps, sts)]
    assert store != "i8" or all(s["exp_avg_i8"] for s in storage)
    hps = lib_hp(opt, hp)
    ox = [to64(p) for p in ps]
    x0 = [x.copy() for x in ox]
    ost = [oracle.INIT_STATE[opt](tuple(p.shape), hp, exp_avg_i8=s["exp_avg_i8"]) for p, s in zip(ps, storage)]
    ws = _lib.workspace(wsize(ps, gs), "cuda")
    offs = lib_scalar_offsets(opt, ps, gs)
    for t in range(1, 4):
        workloads.grads(wl, t - 1, scales, "cuda", out=gs)
        xo_lib = [to64(p) for p in ps]
        lib_step(opt, hps, t, ps, gs, sts, ws)
        torch.cuda.synchronize()
        lib_sc = _lib.read_scalars(ws, offs)
        for k in range(len(ps)):
            sc, xo, so = {}, ox[k], ost[k]
            ox[k], ost[k] = oracle.STEP_TENSOR[opt](xo, to64(gs[k]), so, hp, t, scalars=sc, **storage[k])
            res = judge_tensor(opt, hp, storage[k], ps[k], sts[k], ox[k], ost[k], x0[k], xo_lib[k], xo, lib_sc[k],
                               sc, so)
            if t == 3:
                print("  " + summarize(f"{opt} {store} offset {offset} step {t} {SHAPES[k]}", res), flush=True)
            assert not failures(res), (t, SHAPES[k], failures(res))
