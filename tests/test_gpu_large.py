"""One batched tensor with more than 2^32 elements: [65537, 256, 256], that is
2^32 + 2^16 elements (a stack of expert matrices is the usual source of such a
tensor). Every pass then addresses it with 64-bit offsets, and CAME's apply takes
its 64-bit range path. Two chained steps of Adafactor and of CAME in one call
each, with fp32 storage, bf16 parameter and first moment, and an 8-bit first
moment (whose group scales are indexed by element); the matrices starting at
elements 0, 2^16, 2^31, 2^32 - 2^16 and 2^32 are compared with the oracle under
the usual bars (outputs and the step dX).

The oracle steps each sampled matrix on its own. That is the same step as the
whole tensor's when no per-tensor scalar depends on the rest of the tensor: the
statistics and the per-matrix coefficients are per matrix, the clip threshold is
set out of reach (the clip divisor is 1 on both sides) and Adafactor runs without
scale_parameter (its step size is then rho_t alone)."""
import pytest
import torch

import oracle
from memory_efficient_optimizers_amd import _lib
from tests.harness import failures, judge_tensor, lib_hp, lib_step, storage_of_tensor, summarize, to64

pytestmark = pytest.mark.gpu

SHAPE = (65537, 256, 256)
# matrices whose first elements are 0, 2^16, 2^31, 2^32 - 2^16 and 2^32
SAMPLE = [0, 1, 32768, 65535, 65536]

AF = {"beta1": 0.9, "scale_parameter": False, "clip_threshold": 1e30, "weight_decay": 0.1}
CM = {"lr": 2e-4, "clip_threshold": 1e30, "weight_decay": 0.05}
CASES = [("adafactor", AF, "f32"), ("adafactor", AF, "bf16"), ("adafactor", AF, "i8"),
         ("came", CM, "f32"), ("came", CM, "bf16"), ("came", CM, "i8")]
GROUP = 128  # values per scale of an 8-bit first moment


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("opt,hp,store", CASES)
def test_tensor_beyond_2_32_elements(opt, hp, store):
    numel = SHAPE[0] * SHAPE[1] * SHAPE[2]
    per = SHAPE[1] * SHAPE[2]
    assert numel == (1 << 32) + (1 << 16) and per % GROUP == 0
    pdt = torch.bfloat16 if store == "bf16" else torch.float32
    sdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}[store]
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    # parameter, first moment, gradient, statistics and workspace
    need = numel * (pdt.itemsize + sdt.itemsize + 2) + (4 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")
    gen = torch.Generator(device="cuda").manual_seed(2024)
    x = torch.randn(SHAPE, generator=gen, device="cuda", dtype=pdt).mul_(0.02)
    g = torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda")
    st = _lib.init_state(opt, x, beta1=True, state_dtype=sdt)
    storage = storage_of_tensor(x, st)
    assert storage == {"param_bf16": store == "bf16", "exp_avg_bf16": store == "bf16",
                       "exp_avg_i8": store == "i8"}
    hps = lib_hp(opt, hp)
    ws = _lib.workspace(getattr(_lib, f"meo_{opt}_workspace_size")([x], [g]), "cuda")
    ox = {b: to64(x[b]) for b in SAMPLE}
    x0 = {b: v.copy() for b, v in ox.items()}
    ost = {b: oracle.INIT_STATE[opt](SHAPE[1:], hp, exp_avg_i8=store == "i8") for b in SAMPLE}

    def mat_state(b):
        """The library's state of matrix b (an 8-bit moment's scales: its groups)."""
        out = {}
        for k, v in st.items():
            out[k] = v[b * per // GROUP:(b + 1) * per // GROUP] if k == "exp_avg_scale" else v[b]
        return out

    try:
        for t in (1, 2):
            torch.randn(SHAPE, generator=gen, device="cuda", dtype=torch.bfloat16, out=g)
            g.mul_(1e-3)
            xo_lib = {b: to64(x[b]) for b in SAMPLE}
            print(f"  {opt} {store} step {t}: one call over {numel} elements", flush=True)
            lib_step(opt, hps, t, [x], [g], [st], ws)
            torch.cuda.synchronize()
            for b in SAMPLE:
                xo, so = ox[b], ost[b]
                ox[b], ost[b] = oracle.STEP_TENSOR[opt](xo, to64(g[b]), so, hp, t, **storage)
                res = judge_tensor(opt, hp, storage, x[b], mat_state(b), ox[b], ost[b], x0[b], xo_lib[b], xo,
                                   ost_prev=so)
                print("  " + summarize(f"{opt} {store} step {t} matrix {b} (element {b * per})", res), flush=True)
                assert not failures(res), (t, b, failures(res))
    finally:
        del x, g, st, ws
        torch.cuda.empty_cache()
