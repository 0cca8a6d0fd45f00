"""Behaviour of the library and its torch.optim front ends beyond single-call
parity: resume from a state_dict, NaN confinement and its detection, mixed gradient
dtypes, several parameter groups, non-default streams, all-or-nothing validation,
and the launch table cache."""
import pytest
import torch

import oracle
import workloads
from memory_efficient_optimizers_amd import CAME, Adafactor, Lamb, _lib
from tests.harness import TOL_F32, Run, lib_states, lib_step, lib_workspace, output_err, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


SHAPES = [(96, 520), (520,), (3, 17, 40), (64, 1024)]


def _params(seed=0, dtype=torch.float32):
    wl = workloads.custom("robust", "adafactor", SHAPES, seed=seed, grad_dtype=dtype, param_dtype=dtype)
    return wl, [torch.nn.Parameter(p) for p in workloads.init_params(wl, "cuda")]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cls,hp", [(Adafactor, {"beta1": 0.9}), (CAME, {"lr": 2e-4}),
                                    (Lamb, {"weight_decay": 0.01})])
def test_state_dict_resume_is_bitwise(cls, hp, dtype):
    """5 steps == 3 steps, state_dict(), a fresh optimizer loading it, 2 more steps;
    with bf16 parameters the statistics stay fp32 through the round trip."""
    wl, ps_a = _params(dtype=dtype)
    _, ps_b = _params(dtype=dtype)
    scales = workloads.grad_scales(wl, "cuda")
    opt_a = cls(ps_a, **hp)
    opt_b = cls(ps_b, **hp)
    for t in range(5):
        gs = workloads.grads(wl, t, scales, "cuda")
        for p, g in zip(ps_a, gs):
            p.grad = g.clone()
        opt_a.step()
        if t < 3:
            for p, g in zip(ps_b, gs):
                p.grad = g.clone()
            opt_b.step()
        if t == 2:
            sd = opt_b.state_dict()
            opt_b = cls(ps_b, **hp)
            opt_b.load_state_dict(sd)
        if t >= 3:
            for p, g in zip(ps_b, gs):
                p.grad = g.clone()
            opt_b.step()
    torch.cuda.synchronize()
    for a, b in zip(ps_a, ps_b):
        assert torch.equal(a.detach(), b.detach())
    for a, b in zip(ps_a, ps_b):
        for k, v in opt_a.state[a].items():
            if torch.is_tensor(v):
                assert v.dtype == (dtype if k == "exp_avg" else torch.float32), k
                assert opt_b.state[b][k].dtype == v.dtype, k
                assert torch.equal(v, opt_b.state[b][k]), k
            else:
                assert v == opt_b.state[b][k]


@pytest.mark.parametrize("opt,hp", [("adafactor", {"beta1": 0.9}), ("came", {"lr": 2e-4}), ("lamb", {})])
def test_nan_gradient_stays_in_its_tensor(opt, hp):
    """A NaN in one tensor's gradient propagates to that tensor's update only; the
    other tensors of the call match the oracle."""
    wl = workloads.custom("nan", opt, SHAPES, hparams=hp)
    run = Run(wl)
    gs = run.grads(0)
    gs[0][5, 7] = float("nan")
    run.t += 1
    ws = lib_workspace(opt, run.params, gs)
    lib_step(opt, run.hps, run.t, run.params, gs, run.states, ws)
    torch.cuda.synchronize()
    assert torch.isnan(run.params[0]).any()
    for k in range(1, len(SHAPES)):
        xk, _ = oracle.STEP_TENSOR[opt](run.ox[k], to64(gs[k]), run.ost[k], run.hp, 1)
        assert torch.isfinite(run.params[k]).all()
        assert output_err("param", to64(run.params[k]), xk, x0=run.x0[k]) <= TOL_F32


@pytest.mark.parametrize("cls,hp", [(Adafactor, {"beta1": 0.9}), (Adafactor, {}), (CAME, {"lr": 2e-4}),
                                    (Lamb, {"weight_decay": 0.01})])
def test_check_finite_names_the_nonfinite_tensors(cls, hp):
    """check_finite=True: after a step whose gradients hold a NaN (the 1-D tensor),
    an infinity (the 3-D one) and a value whose square overflows float32 (the last
    matrix), nonfinite_params() names exactly the parameters whose step is not
    finite, in list order: all three for Adafactor and CAME (the infinite square
    reaches the factored statistics, and V = R C / mean(R) turns NaN), the first two
    for LAMB (there v turns infinite and that element's direction m / sqrt(v) is 0,
    so its step stays finite). The others are stepped to finite values. On the next
    step the named ones hold non-finite states and are named again. A clean run
    names nothing and steps bit for bit as without the option."""
    wl, ps = _params()
    scales = workloads.grad_scales(wl, "cuda")
    opt = cls(ps, check_finite=True, **hp)
    gs = workloads.grads(wl, 0, scales, "cuda")
    gs[1][7] = float("nan")
    gs[2][1, 3, 5] = float("inf")
    gs[3][10, 20] = 3e19
    for p, g in zip(ps, gs):
        p.grad = g
    opt.step()
    named = [1, 2] if cls is Lamb else [1, 2, 3]
    assert [id(p) for p in opt.nonfinite_params()] == [id(ps[k]) for k in named]
    for k in range(len(ps)):
        assert torch.isfinite(ps[k]).all() == (k not in named), k
    assert opt.nonfinite_params() == []  # the list was cleared
    for p, g in zip(ps, workloads.grads(wl, 1, scales, "cuda")):
        p.grad = g
    opt.step()
    assert [id(p) for p in opt.nonfinite_params()] == [id(ps[k]) for k in named]

    wl, ps = _params(seed=1)
    clean = cls(ps, check_finite=True, **hp)
    plain = cls([torch.nn.Parameter(p.detach().clone()) for p in ps], **hp)
    for t in range(2):
        gs = workloads.grads(wl, t, scales, "cuda")
        for p, q, g in zip(ps, plain.param_groups[0]["params"], gs):
            p.grad = g.clone()
            q.grad = g.clone()
        clean.step()
        plain.step()
    assert clean.nonfinite_params() == []
    assert plain.nonfinite_params() == []
    for p, q in zip(ps, plain.param_groups[0]["params"]):
        assert torch.equal(p.detach(), q.detach())  # the check reads, and changes nothing


def test_mixed_gradient_dtypes_in_one_call():
    wl32 = workloads.custom("m32", "adafactor", SHAPES, hparams={"beta1": 0.9}, grad_dtype=torch.float32)
    run = Run(wl32)
    gs = run.grads(0)
    gs = [g.to(torch.bfloat16) if k % 2 == 0 else g for k, g in enumerate(gs)]
    run.step(gs)
    run.check()


def test_param_groups_and_side_stream():
    """Two groups with different hyperparameters, stepped on a non-default stream,
    equal two separate library calls."""
    wl, ps = _params()
    scales = workloads.grad_scales(wl, "cuda")
    gs = workloads.grads(wl, 0, scales, "cuda")
    ref = [p.detach().clone() for p in ps]
    opt = Adafactor([{"params": ps[:2]}, {"params": ps[2:], "beta1": 0.5, "weight_decay": 0.1}])
    for p, g in zip(ps, gs):
        p.grad = g
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        opt.step()
    torch.cuda.current_stream().wait_stream(side)
    st1 = lib_states("adafactor", ref[:2], {})
    st2 = lib_states("adafactor", ref[2:], {"beta1": 0.5})
    lib_step("adafactor", _lib.adafactor_hparams(), 1, ref[:2], gs[:2], st1, lib_workspace("adafactor", ref[:2], gs[:2]))
    lib_step("adafactor", _lib.adafactor_hparams(beta1=0.5, weight_decay=0.1), 1, ref[2:], gs[2:], st2,
             lib_workspace("adafactor", ref[2:], gs[2:]))
    torch.cuda.synchronize()
    for p, q in zip(ps, ref):
        assert torch.equal(p.detach(), q)


def test_rejected_call_changes_nothing():
    """Validation is all-or-nothing: a bad last tensor leaves the whole list as it was."""
    wl = workloads.custom("rej", "adafactor", SHAPES, hparams={"beta1": 0.9})
    run = Run(wl)
    gs = run.grads(0)
    before = [p.clone() for p in run.params] + [v.clone() for st in run.states for v in st.values()]
    bad = [dict(s) for s in run.states]
    del bad[-1]["exp_avg"]
    ws = lib_workspace("adafactor", run.params, gs)
    with pytest.raises(_lib.MeoError) as e:
        lib_step("adafactor", run.hps, 1, run.params, gs, bad, ws)
    assert e.value.code == _lib.MEO_ENULL
    with pytest.raises(_lib.MeoError):
        lib_step("adafactor", _lib.adafactor_hparams(lr=1e-3), 1, run.params, gs, run.states, ws)
    torch.cuda.synchronize()
    after = [p for p in run.params] + [v for st in run.states for v in st.values()]
    for a, b in zip(before, after):
        assert torch.equal(a, b)


def test_launch_table_cache_eviction():
    """More distinct tensor lists than the cache holds (64), revisited: results stay
    exact."""
    outs = {}
    for rep in range(2):
        for i in range(70):
            shape = (8 + i, 64 + 8 * i)
            wl = workloads.custom(f"ev{i}", "adafactor", [shape], hparams={"beta1": 0.9}, seed=i)
            run = Run(wl)
            run.step()
            torch.cuda.synchronize()
            if rep == 0:
                outs[i] = run.params[0].clone()
                run.check()
            else:
                assert torch.equal(outs[i], run.params[0])
    _lib.meo_release_plans()


def test_memory_ranges_are_checked_before_launch():
    """A step checks its pointers with the HIP runtime before enqueueing: a
    workspace described past the end of its allocation and a statistic held in
    (GPU-mapped) pinned host memory are refused, and nothing is modified. The
    cases are chosen so that even a missed refusal would touch only valid memory.
    Views into one shared buffer are accepted."""
    wl = workloads.custom("memchk", "adafactor", [(64, 512), (300,)], hparams={"beta1": 0.9})
    run = Run(wl)
    gs = run.grads(0)
    need = _lib.meo_adafactor_workspace_size(run.params, gs)
    ws = _lib.workspace(need, "cuda")
    hps = _lib.adafactor_hparams(beta1=0.9)
    before = [p.clone() for p in run.params] + [v.clone() for st in run.states for v in st.values()]
    fn = _lib.load().meo_adafactor_step
    args = (_lib.ctypes.byref(hps), 1, 2, _lib._tensors(run.params, gs, run.states),
            _lib._states(_lib.meo_adafactor_state, _lib.ADAFACTOR_KEYS, run.states))
    assert fn(*args, ws.data_ptr(), need + (4 << 30), None) == _lib.MEO_EWORKSPACE
    assert "past the end" in _lib.meo_last_error()
    pinned = torch.zeros(64, dtype=torch.float32, pin_memory=True)
    bad = [dict(st) for st in run.states]
    bad[0]["exp_avg_sq_row"] = pinned
    with pytest.raises(_lib.MeoError) as e:
        lib_step("adafactor", hps, 1, run.params, gs, bad, ws)
    assert e.value.code == _lib.MEO_EMEMORY and "exp_avg_sq_row" in e.value.message
    torch.cuda.synchronize()
    after = [p for p in run.params] + [v for st in run.states for v in st.values()]
    for a, b in zip(before, after):
        assert torch.equal(a, b)
    assert torch.count_nonzero(pinned) == 0
    # tensors as views into one buffer pass the check and step as separate ones
    buf = torch.cat([p.reshape(-1) for p in run.params])
    views = [buf[:64 * 512].view(64, 512), buf[64 * 512:].view(300)]
    sts = lib_states("adafactor", views, {"beta1": 0.9})
    lib_step("adafactor", hps, 1, views, gs, sts, ws)
    lib_step("adafactor", hps, 1, run.params, gs, run.states, ws)
    torch.cuda.synchronize()
    assert torch.equal(views[0], run.params[0]) and torch.equal(views[1], run.params[1])
