"""Row-sharded steps on one GPU: N ranks' shares of every tensor, each stepped by
the library's two shard calls, with the ranks' partial-sum records summed in
between (what an all-reduce over the ranks would give; here a sum of the N
buffers on the GPU). After every step the shards, put back together, must match
the oracle's whole-tensor step: the parameter, first moment and row statistic row
by row, and every rank's copy of the column statistic. Bars as in the parity tests
(tests/harness.py): the ranks sum partials in another order than one pass over the
whole tensor, which moves results by fp32 rounding only.

Shapes cover one row per rank (a factored shard of height 1 stays factored, which
the page's DistributedCAME note requires), ranks holding no rows of a small
tensor (their records must read zero), batched matrices, 11008-wide rows (the wide
first-pass class) and 1-D tensors split by elements; LAMB splits every tensor by
elements."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from memory_efficient_optimizers_amd import _lib
from tests.harness import TOL_F32, beta1_of, output_err, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


SHAPES = [(129, 1024), (8, 4096), (4, 8), (2, 3, 72, 136), (40, 11008), (5000,), (300,), (3,)]


def _split(n, parts):
    return [(n * r // parts, n * (r + 1) // parts) for r in range(parts)]


def _shard_of(t, opt, r0, r1):
    """Rows r0:r1 of dim -2 (factored), else elements r0:r1 of the flattened tensor."""
    if opt != "lamb" and t.dim() >= 2:
        return t[..., r0:r1, :].contiguous()
    return t.reshape(-1)[r0:r1].contiguous()


def _ranges(opt, shape, nranks):
    if opt != "lamb" and len(shape) >= 2:
        return _split(shape[-2], nranks), shape[-2]
    n = math.prod(shape)
    return _split(n, nranks), n


@pytest.mark.parametrize("nranks", [1, 3, 8])
@pytest.mark.parametrize("opt,hp", [
    ("adafactor", {"beta1": 0.9, "weight_decay": 0.1}),
    ("adafactor", {}),
    ("adafactor", {"scale_parameter": False, "beta1": 0.5, "clip_threshold": 0.3}),
    ("adafactor-carry", {"beta1": 0.9, "weight_decay": 0.1}),
    ("adafactor-carry", {"warmup_init": True}),
    ("lamb", {"weight_decay": 0.01}),
    ("came", {"lr": 2e-4, "weight_decay": 0.05}),
])
def test_row_sharded_step_matches_whole_tensor(opt, hp, nranks):
    """"adafactor-carry": the carry calls, each rank carrying the sum of X^2 of its
    own shard from the second step on; the ranks' sums add up to the whole
    parameter's."""
    carry = opt == "adafactor-carry"
    check_sharded("adafactor" if carry else opt, hp, SHAPES, nranks, carry)


def check_sharded(opt, hp, shapes, nranks, carry=False, steps=3, seed=0):
    """N ranks' shares of `shapes` stepped `steps` times through the shard calls, the
    records summed in between; after every step the shares put together must match
    the oracle's whole-tensor step."""
    wl = workloads.custom(f"shard_{opt}", opt, shapes, hparams=hp, grad_dtype=torch.bfloat16,
                          grad_scaling="rowcol" if opt != "lamb" else "row", seed=seed)
    full = workloads.init_params(wl, "cuda")
    scales = workloads.grad_scales(wl, "cuda")
    hps = {"adafactor": _lib.adafactor_hparams, "lamb": _lib.lamb_hparams, "came": _lib.came_hparams}[opt](**hp)
    beta1 = hp.get("beta1") is not None or opt == "lamb"
    ranges = [_ranges(opt, tuple(p.shape), nranks) for p in full]
    totals = [tot for _, tot in ranges]
    ranks = []
    for r in range(nranks):
        ps = [_shard_of(p, opt, *ranges[k][0][r]) for k, p in enumerate(full)]
        sts = []
        for k, p in enumerate(ps):
            st = _lib.init_state(opt, p, beta1=beta1)
            for key in ("exp_avg_sq_col", "exp_avg_res_col"):  # column statistics are kept whole on every rank
                if key in st:
                    st[key] = torch.zeros(full[k].shape[:-2] + full[k].shape[-1:], device="cuda")
            if carry:
                st["param_sumsq"] = torch.zeros(1, device="cuda")
            sts.append(st)
        ranks.append({"params": ps, "states": sts})
    size = getattr(_lib, f"meo_{opt}_partials_size")(ranks[0]["params"], ranks[0]["params"])
    csize = _lib.meo_came_confidence_size(ranks[0]["params"], ranks[0]["params"]) if opt == "came" else 0
    stats = getattr(_lib, f"meo_{opt}_shard_stats")
    apply = getattr(_lib, f"meo_{opt}_shard_apply")
    if carry:
        def stats(hps, t, ps, gs, totals, sts, part, ws):
            _lib.meo_adafactor_shard_stats_carry(hps, t, ps, gs, totals, sts, t > 1, part, ws)
        apply = _lib.meo_adafactor_shard_apply_carry
    ox = [to64(p) for p in full]
    x0 = [x.copy() for x in ox]
    ost = [oracle.INIT_STATE[opt](tuple(p.shape), hp) for p in full]
    b1 = beta1_of(opt, hp)
    for t in range(1, steps + 1):
        gfull = workloads.grads(wl, t - 1, scales, "cuda")
        parts = []
        for r, rk in enumerate(ranks):
            gs = [_shard_of(g, opt, *ranges[k][0][r]) for k, g in enumerate(gfull)]
            rk["grads"] = gs
            ws = _lib.workspace(getattr(_lib, f"meo_{opt}_workspace_size")(rk["params"], gs), "cuda")
            rk["ws"] = ws
            part = torch.full((size,), float("nan"), device="cuda")  # every entry must be written
            stats(hps, t, rk["params"], gs, totals, rk["states"], part, ws)
            parts.append(part)
        reduced = torch.stack(parts).sum(0)  # the all-reduce
        assert torch.isfinite(reduced).all()
        if opt == "came":  # the second exchange: the confidence sums
            confs = []
            for rk in ranks:
                conf = torch.full((max(csize, 1),), float("nan"), device="cuda")
                _lib.meo_came_shard_moment(hps, t, rk["params"], rk["grads"], totals, rk["states"], reduced, conf,
                                           rk["ws"])
                confs.append(conf)
            reduced = torch.stack(confs).sum(0)
            assert torch.isfinite(reduced[:csize]).all()
        for rk in ranks:
            apply(hps, t, rk["params"], rk["grads"], totals, rk["states"], reduced, rk["ws"])
        torch.cuda.synchronize()
        ost_prev = ost
        ox, ost = oracle.STEP[opt](ox, [to64(g) for g in gfull], ost, hp, t)
        for k, spec in enumerate(wl.specs):
            fac = opt != "lamb" and len(spec.shape) >= 2
            dim = -2 if fac else 0

            def whole(key):
                pieces = [rk["states"][k][key] if key != "param" else rk["params"][k] for rk in ranks]
                if fac:
                    if key in ("exp_avg_sq_row", "exp_avg_res_row"):
                        return torch.cat(pieces, dim=-1)
                    return torch.cat(pieces, dim=-2)
                return torch.cat([p.reshape(-1) for p in pieces]).reshape(spec.shape)

            errs = {"param": output_err("param", to64(whole("param")), ox[k], x0=x0[k])}
            for key in ost[k]:
                if key in ("exp_avg_sq_col", "exp_avg_res_col"):
                    cols = [rk["states"][k][key] for rk, (r0, r1) in zip(ranks, ranges[k][0]) if r1 > r0]
                    for c in cols[1:]:
                        assert torch.equal(c, cols[0]), "ranks disagree on the column statistic"
                    errs[key] = output_err(key, to64(cols[0]), ost[k][key])
                else:
                    errs[key] = output_err(key, to64(whole(key)), ost[k][key],
                                           prev=ost_prev[k].get(key) if key == "exp_avg" else None, beta1=b1)
            worst = max(errs, key=errs.get)
            print(f"  {opt}{' carry' if carry else ''} N={nranks} step {t} {spec.name} {tuple(spec.shape)}: "
                  f"worst {errs[worst]:.3e} ({worst})", flush=True)
            assert errs[worst] <= TOL_F32, (t, spec.shape, worst, errs[worst])
            if carry:  # the ranks' carried sums add up to the whole parameter's sum of squares
                got = sum(float(rk["states"][k]["param_sumsq"].item())
                          for rk, (r0, r1) in zip(ranks, ranges[k][0]) if r1 > r0)
                want = float(np.sum(np.square(ox[k])))
                assert abs(got - want) <= 1e-5 * want, (t, spec.shape, got, want)


def test_came_confidence_record_layout():
    """CAME's second record: B x (W + 1) floats per factored tensor, none for 1-D."""
    ps = [torch.zeros(s, device="cuda") for s in ((129, 1024), (300,), (2, 3, 72, 136))]
    assert _lib.meo_came_confidence_size(ps, ps) == 1 * 1025 + 0 + 6 * 137


def test_shard_of_the_whole_is_the_whole_step():
    """One rank holding everything: the sharded calls give the whole-tensor step's
    parameters (the same kernels; sums in a different order, so within fp32 bars)."""
    wl = workloads.custom("shard1", "adafactor", [(129, 1024), (300,)], hparams={"beta1": 0.9},
                          grad_dtype=torch.bfloat16)
    a = workloads.init_params(wl, "cuda")
    b = [p.clone() for p in a]
    scales = workloads.grad_scales(wl, "cuda")
    hps = _lib.adafactor_hparams(beta1=0.9)
    sa = [_lib.init_state("adafactor", p, beta1=True) for p in a]
    sb = [_lib.init_state("adafactor", p, beta1=True) for p in b]
    part = torch.zeros(_lib.meo_adafactor_partials_size(a, a), device="cuda")
    for t in range(1, 4):
        gs = workloads.grads(wl, t - 1, scales, "cuda")
        ws = _lib.workspace(_lib.meo_adafactor_workspace_size(a, gs), "cuda")
        _lib.meo_adafactor_step(hps, t, a, gs, sa, ws)
        _lib.meo_adafactor_shard_stats(hps, t, b, gs, [129, 300], sb, part, ws)
        _lib.meo_adafactor_shard_apply(hps, t, b, gs, [129, 300], sb, part, ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert output_err("param", to64(y), to64(x)) <= TOL_F32


def test_prepared_came_shard_of_the_whole_is_the_whole_step():
    """CAME's three prepared calls (stats, moment, apply) on one rank holding
    everything give the whole-tensor step's parameters within the fp32 bar."""
    wl = workloads.custom("shard1c", "came", [(129, 1024), (300,)], hparams={"lr": 2e-4},
                          grad_dtype=torch.bfloat16)
    a = workloads.init_params(wl, "cuda")
    b = [p.clone() for p in a]
    scales = workloads.grad_scales(wl, "cuda")
    hps = _lib.came_hparams(lr=2e-4)
    sa = [_lib.init_state("came", p) for p in a]
    sb = [_lib.init_state("came", p) for p in b]
    part = torch.zeros(_lib.meo_came_partials_size(a, a), device="cuda")
    conf = torch.zeros(max(_lib.meo_came_confidence_size(a, a), 1), device="cuda")
    gs = workloads.grads(wl, 0, scales, "cuda")
    ws = _lib.workspace(max(_lib.meo_came_workspace_size(a, gs), 256), "cuda")
    call = _lib.PreparedShardStep("came", hps, b, gs, [129, 300], sb, part, ws, conf)
    for t in range(1, 4):
        g_new = workloads.grads(wl, t - 1, scales, "cuda")
        for g, n in zip(gs, g_new):
            g.copy_(n)
        _lib.meo_came_step(hps, t, a, gs, sa, ws)
        call.stats(t)
        call.moment(t)
        call.apply(t)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert output_err("param", to64(y), to64(x)) <= TOL_F32


def test_prepared_adafactor_shard_carry_of_the_whole_is_the_whole_step():
    """The prepared carry calls on one rank holding everything give the whole-list
    carry step's parameters and carried sums within the fp32 bar."""
    wl = workloads.custom("shard1a", "adafactor", [(129, 1024), (300,), (2, 3, 72, 136)], hparams={"beta1": 0.9},
                          grad_dtype=torch.bfloat16)
    a = workloads.init_params(wl, "cuda")
    b = [p.clone() for p in a]
    scales = workloads.grad_scales(wl, "cuda")
    hps = _lib.adafactor_hparams(beta1=0.9)
    sa = [_lib.init_state("adafactor", p, beta1=True) for p in a]
    sb = [_lib.init_state("adafactor", p, beta1=True) for p in b]
    for st in sa + sb:
        st["param_sumsq"] = torch.zeros(1, device="cuda")
    totals = [129, 300, 72]
    part = torch.zeros(_lib.meo_adafactor_partials_size(a, a), device="cuda")
    gs = workloads.grads(wl, 0, scales, "cuda")
    ws = _lib.workspace(_lib.meo_adafactor_workspace_size(a, gs), "cuda")
    call = _lib.PreparedShardStep("adafactor", hps, b, gs, totals, sb, part, ws, carry=True)
    for t in range(1, 5):
        for g, n in zip(gs, workloads.grads(wl, t - 1, scales, "cuda")):
            g.copy_(n)
        _lib.meo_adafactor_step_carry(hps, t, a, gs, sa, t > 1, ws)
        call.stats(t)
        call.apply(t)
    torch.cuda.synchronize()
    for x, y, s1, s2 in zip(a, b, sa, sb):
        assert output_err("param", to64(y), to64(x)) <= TOL_F32
        assert abs(s2["param_sumsq"].item() - s1["param_sumsq"].item()) <= 1e-5 * s1["param_sumsq"].item()
