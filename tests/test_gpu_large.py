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
import numpy as np
import pytest
import torch

import oracle
from memory_efficient_optimizers_amd import _lib
from tests.harness import (TOL_F32, check_dx, failures, floored_rel_err, judge_tensor, lib_hp, lib_step,
                           output_errs, storage_of_tensor, summarize, to64)

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


# GaLore over one matrix past 2^32 elements, each side: 65600 x 65536 (m >= n, the
# projection along the rows' space) and its transpose shape (m < n). Not a refresh
# step, so the projector is an input: a random orthonormal basis rounded to bf16.
# The step is independent per row of the gradient on the m >= n side (and per
# column on the other), so blocks of 256 rows (columns) at elements 0, 2^31 and
# past 2^32 are stepped by the oracle on their own. A 256 x 65536 block's shorter
# side is no longer the projected one, so the oracle takes those blocks with
# reverse_std, which projects the longer side: the same side, the same basis and
# the same arithmetic as the whole matrix under std.
#
# Bars: the contraction runs over d = 65536 here, 16 times the 4096 of the Llama-7B
# rows the GaLore bars were set on. The matrix cores accumulate the d products in
# fp32, about sqrt(d / 16) roundings of 2^-24 of the running sum, so the low-rank
# gradient's error grows as sqrt(d): 1e-5 becomes 4e-5 for the moments and the
# parameter (x sqrt(65536 / 4096)), 4e-4 for the step dX.
GA_SCALE = 4.0
GA_SHAPES = [(65600, 65536), (65536, 65600)]
GA_BLOCK = 256


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", GA_SHAPES)
def test_galore_matrix_beyond_2_32_elements(shape):
    from oracle import galore as ga
    m, n = shape
    numel = m * n
    assert numel > (1 << 32)
    r = 256
    right = m >= n
    d, D = (n, m) if right else (m, n)  # projected side, rows of the low-rank arrays
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    need = numel * (4 + 2) + (4 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")
    gen = torch.Generator(device="cuda").manual_seed(2025)
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).mul_(0.02)
    g = torch.randn(shape, generator=gen, device="cuda", dtype=torch.bfloat16).mul_(1e-3)
    q, _ = torch.linalg.qr(torch.randn(d, r, generator=gen, device="cuda", dtype=torch.float32))
    proj = q.to(torch.bfloat16).contiguous()
    st = {"exp_avg": torch.randn(D, r, generator=gen, device="cuda", dtype=torch.float32).mul_(5e-4),
          "exp_avg_sq": torch.rand(D, r, generator=gen, device="cuda", dtype=torch.float32).add_(0.5).mul_(1e-6),
          "projector": proj, "projector_t": proj.t().contiguous()}
    hp = dict(lr=0.05, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, scale=0.25, rank=r)
    t = 5  # not a refresh step (update_proj_gap 200)
    h = _lib.galore_hparams(**hp)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, [x], [g]), "cuda")
    # blocks of rows (m >= n) or columns (m < n): the first, the one at element 2^31 and the last
    starts = [0, (1 << 31) // n if right else 32768, (m if right else n) - GA_BLOCK]
    blk = lambda a, s: a[s:s + GA_BLOCK] if right else a[:, s:s + GA_BLOCK]
    u64 = to64(proj)
    before = {s: (to64(blk(x, s)), to64(blk(g, s)), to64(st["exp_avg"][s:s + GA_BLOCK]),
                  to64(st["exp_avg_sq"][s:s + GA_BLOCK])) for s in starts}
    pt0 = st["projector_t"].clone()
    try:
        print(f"  galore {shape}: one call over {numel} elements", flush=True)
        _lib.meo_galore_step(h, t, [x], [g], [st], ws)
        torch.cuda.synchronize()
        assert torch.equal(st["projector"], proj) and torch.equal(st["projector_t"], pt0)
        hpo = dict(hp, proj_type="reverse_std")
        b1 = hp["betas"][0]
        for s in starts:
            x0, g0, m0, v0 = before[s]
            assert ga.galore_side(x0.shape, "reverse_std") == ("right" if right else "left")
            want_x, want_s = ga.galore_step_tensor(x0, g0, {"exp_avg": m0, "exp_avg_sq": v0, "projector": u64},
                                                   hpo, t)
            got_x = to64(blk(x, s))
            bad = []
            errs = {}
            for key, a, b in (("param", got_x, want_x),
                              ("exp_avg", to64(st["exp_avg"][s:s + GA_BLOCK]), want_s["exp_avg"]),
                              ("exp_avg_sq", to64(st["exp_avg_sq"][s:s + GA_BLOCK]), want_s["exp_avg_sq"])):
                errs[key] = float(np.max(output_errs(key, a, b, x0=x0, prev=m0, beta1=b1, step_tol=1e-4)))
                if errs[key] > GA_SCALE * TOL_F32:
                    bad.append(f"{key}: err {errs[key]:.3g}")
            e = floored_rel_err(got_x - x0, want_x - x0)
            print(f"  galore {shape} block at {s}: update err {e:.2e}; "
                  + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
            if e > GA_SCALE * 1e-4:
                bad.append(f"update: err {e:.3g}")
            assert not bad, (s, bad)
    finally:
        del x, g, st, ws
        torch.cuda.empty_cache()


def _norm64(a: torch.Tensor, b: torch.Tensor = None) -> float:
    """2-norm of a (or of a - b) in fp64, in chunks of 2^27 elements."""
    s = 0.0
    fa = a.reshape(-1)
    fb = None if b is None else b.reshape(-1)
    for i in range(0, fa.numel(), 1 << 27):
        c = fa[i:i + (1 << 27)].double()
        if fb is not None:
            c -= fb[i:i + (1 << 27)].double()
        s += float(torch.dot(c, c))
    return s ** 0.5


@pytest.mark.timeout(600)
def test_lamb_tensor_beyond_2_32_elements():
    """LAMB over the same [65537, 256, 256] tensor (one layer for the trust ratio), a
    mid-run step (t = 3, seeded moments). The trust ratio spans the whole tensor, so
    a matrix cannot be stepped on its own; two facts pin the step instead.
    * Every element's direction is local: on each sampled matrix the library's step
      is its trust ratio times the oracle's direction for that matrix, which the
      oracle's step on the matrix alone gives as (x - x_new) / (lr * its own ratio).
      Moments are local and compared directly.
    * The ratio: the library's ||X|| matches an fp64 reduction of the parameter, and
      the step's norm is lr ||X|| over the whole tensor (LAMB's update has the norm
      lr * trust * ||d|| = lr ||X||), from fp64 reductions on the device."""
    numel = SHAPE[0] * SHAPE[1] * SHAPE[2]
    per = SHAPE[1] * SHAPE[2]
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    need = numel * (4 + 4 + 2 + 4 + 4) + (4 << 30)  # parameter and its copy, gradient, moments
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")
    hp = {"lr": 1e-3, "weight_decay": 0.01}
    t = 3
    gen = torch.Generator(device="cuda").manual_seed(2026)
    x = torch.randn(SHAPE, generator=gen, device="cuda", dtype=torch.float32).mul_(0.02)
    g = torch.randn(SHAPE, generator=gen, device="cuda", dtype=torch.bfloat16).mul_(1e-3)
    st = _lib.init_state("lamb", x, state_dtype=torch.float32)
    torch.randn(SHAPE, generator=gen, device="cuda", dtype=torch.float32, out=st["exp_avg"]).mul_(5e-4)
    torch.rand(SHAPE, generator=gen, device="cuda", dtype=torch.float32, out=st["exp_avg_sq"]).add_(0.5).mul_(1e-6)
    x0 = x.clone()
    xn_ref = _norm64(x0)
    before = {b: (to64(x[b]).reshape(-1), to64(g[b]).reshape(-1), to64(st["exp_avg"][b]).reshape(-1),
                  to64(st["exp_avg_sq"][b]).reshape(-1)) for b in SAMPLE}
    hps = lib_hp("lamb", hp)
    ws = _lib.workspace(_lib.meo_lamb_workspace_size([x], [g]), "cuda")
    offs = _lib._scalar_offsets("lamb", [x], [g])
    try:
        print(f"  lamb step {t}: one call over {numel} elements", flush=True)
        lib_step("lamb", hps, t, [x], [g], [st], ws)
        torch.cuda.synchronize()
        sc = _lib.read_scalars(ws, offs)[0]
        xn, dn, tau = sc["rms_x"], sc["norm_d"], sc["trust"]
        dx_norm = _norm64(x, x0)
        e_xn = abs(xn - xn_ref) / xn_ref
        e_tau = abs(tau - xn / dn) / tau
        e_dx = abs(dx_norm - hp["lr"] * xn_ref) / (hp["lr"] * xn_ref)
        print(f"  lamb: ||X|| {xn:.6e} (fp64 {xn_ref:.6e}, err {e_xn:.1e}); trust {tau:.6e} (err {e_tau:.1e}); "
              f"||dX|| / (lr ||X||) - 1 = {e_dx:.1e}", flush=True)
        assert e_xn <= 1e-6 and e_tau <= 1e-6 and e_dx <= 1e-5, (e_xn, e_tau, e_dx)
        for b in SAMPLE:
            x0b, gb, mb, vb = before[b]
            so = {}
            xo, sto = oracle.STEP_TENSOR["lamb"](x0b, gb, {"exp_avg": mb, "exp_avg_sq": vb}, hp, t, scalars=so)
            d_o = (x0b - xo) / (hp["lr"] * so["trust"])  # the oracle's direction on this matrix
            ok, e, over, _, nw = check_dx("f32", to64(x[b]).reshape(-1), x0b, x0b - hp["lr"] * tau * d_o, x0b)
            em = float(np.max(output_errs("exp_avg", to64(st["exp_avg"][b]).reshape(-1), sto["exp_avg"],
                                          prev=mb, beta1=0.9)))
            ev = float(np.max(output_errs("exp_avg_sq", to64(st["exp_avg_sq"][b]).reshape(-1), sto["exp_avg_sq"])))
            print(f"  lamb matrix {b} (element {b * per}): dX err {e:.2e} (normwise {nw:.1e}), "
                  f"exp_avg {em:.2e}, exp_avg_sq {ev:.2e}", flush=True)
            assert ok and em <= TOL_F32 and ev <= TOL_F32, (b, e, over, nw, em, ev)
    finally:
        del x, x0, g, st, ws
        torch.cuda.empty_cache()
