"""The Adafactor step that carries sum(X^2) between steps (meo_adafactor_step_carry).

The step size scales with RMS(X) of the parameter before the update
(scale_parameter, the note after "Step 5" of the Colossal-AI page); the carry
call takes it from the sum of squares that the previous call's apply pass formed
from the parameter it stored. Checked here:

* chained steps against the fp64 oracle under the usual bars (the oracle reads
  X afresh every step, so this is the same parity as the plain step's);
* the carried value against its definition: the sum of squares of the stored
  parameter, in fp64, and against the oracle's parameter;
* a first call (param_sumsq_valid = 0) gives the plain step's exact bits;
* without scale_parameter nothing is read or written;
* the torch front end invalidates the carry when a parameter is written between
  steps;
* the 7B list in one call per step (the bench's launch shape).
"""
import numpy as np
import pytest
import torch

import workloads
from tests.harness import Run, lib_hp, lib_states, lib_step, lib_workspace, list_run, to64

pytestmark = pytest.mark.gpu

# Sum of squares of the stored parameter vs the same sum in fp64: per-lane fp32
# sums of 16 rows, an fp32 block sum of 256 lanes, one fp32 rounding of the
# result: at most ~25 roundings of 2^-24 in a chain of positive terms.
SUMSQ_OWN = 2e-6
# against the oracle's parameter, which differs from the stored one within the
# parity bars (bf16 storage: one bf16 step on ~1e-4 of the elements)
SUMSQ_ORACLE = 1e-5


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from memory_efficient_optimizers_amd import _lib
    _lib.load()


def _own_sumsq_err(run):
    worst = 0.0
    for k, p in enumerate(run.params):
        if p.numel() == 0:
            continue
        want = float(np.sum(np.square(to64(p))))
        got = float(run.states[k]["param_sumsq"].item())
        worst = max(worst, abs(got - want) / want if want > 0 else abs(got))
    return worst


def _chain_carry(wl, steps, hp=None):
    run = Run(wl, hp=hp, carry=True)
    for s in range(steps):
        run.step()
        run.check(f"carry step {s + 1}")
        own = _own_sumsq_err(run)
        orc = max(run.sumsq_errors().values())
        print(f"    sum(X^2): vs stored param {own:.2e}, vs oracle param {orc:.2e}", flush=True)
        assert own <= SUMSQ_OWN, (s + 1, own)
        assert orc <= SUMSQ_ORACLE, (s + 1, orc)
    return run


@pytest.mark.parametrize("name", ["adafactor_small", "adafactor_llama_mini", "adafactor_llama_mini_bf16",
                                  "adafactor_llama_mini_i8"])
def test_carry_chained_workloads(name):
    wl = workloads.WORKLOADS[name]
    _chain_carry(wl, min(wl.steps, 6))


EDGE_SHAPES = [(1, 1000), (1000, 1), (37, 1001), (3,), (), (2, 3, 70, 130), (0, 5), (65, 513),
               (129, 1024), (1, 8), (700, 8), (40000,), (2, 3, 72, 136), (70, 5000), (3, 16384)]


@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("hp", [{}, {"beta1": 0.9, "weight_decay": 0.1}, {"warmup_init": True, "beta1": 0.5}])
def test_carry_edge_shapes(hp, gdt):
    """Every first-pass kind (row-complete, tiled, flat), ragged tiles, an empty and
    a 0-d tensor, leading batch dims."""
    wl = workloads.custom("carry_edge", "adafactor", EDGE_SHAPES, hparams=hp, grad_dtype=gdt,
                          grad_std=1.0, grad_scaling="rowcol", steps=4)
    _chain_carry(wl, 4)


@pytest.mark.parametrize("name", ["adafactor_llama_mini", "adafactor_llama_mini_bf16"])
def test_carry_invalid_first_call_is_the_plain_step(name):
    """param_sumsq_valid = 0 reads X exactly as the plain step does: the same bits,
    whatever param_sumsq held before."""
    from memory_efficient_optimizers_amd import _lib
    wl = workloads.WORKLOADS[name]
    opt, hp = wl.optimizer, dict(wl.hparams)
    scales = workloads.grad_scales(wl, "cuda")
    out = []
    for mode in ("plain", "carry"):
        ps = workloads.init_params(wl, "cuda")
        sts = lib_states(opt, ps, hp, wl.state_dtype)
        for st in sts:
            st["param_sumsq"] = torch.full((1,), 12345.0, device="cuda")
        hps = lib_hp(opt, hp)
        for t in range(1, 3):
            gs = workloads.grads(wl, t - 1, scales, "cuda")
            ws = lib_workspace(opt, ps, gs)
            if mode == "plain":
                lib_step(opt, hps, t, ps, gs, sts, ws)
            else:
                _lib.meo_adafactor_step_carry(hps, t, ps, gs, sts, False, ws)
        torch.cuda.synchronize()
        out.append((ps, sts))
    for a, b in zip(out[0][0], out[1][0]):
        assert torch.equal(a, b)
    for sa, sb in zip(out[0][1], out[1][1]):
        for key in sa:
            if key != "param_sumsq":
                assert torch.equal(sa[key], sb[key]), key
    for st in out[0][1]:  # the plain step leaves param_sumsq alone
        assert st["param_sumsq"].item() == 12345.0


def test_carry_without_scale_parameter_touches_nothing():
    from memory_efficient_optimizers_amd import _lib
    wl = workloads.custom("carry_noscale", "adafactor", [(64, 520), (520,)],
                          hparams={"scale_parameter": False, "beta1": 0.9})
    run = Run(wl)
    ps = [p.clone() for p in run.params]
    sts = [{k: v.clone() for k, v in st.items()} for st in run.states]
    for st in sts:
        st["param_sumsq"] = torch.full((1,), -3.0, device="cuda")
    for t in range(1, 3):
        gs = run.step()
        _lib.meo_adafactor_step_carry(run.hps, t, ps, gs, sts, True, run.ws)
    torch.cuda.synchronize()
    for a, b in zip(ps, run.params):
        assert torch.equal(a, b)
    for st in sts:
        assert st["param_sumsq"].item() == -3.0


def test_carry_null_sum_is_refused():
    from memory_efficient_optimizers_amd import _lib
    wl = workloads.custom("carry_null", "adafactor", [(64, 520), (520,)])
    run = Run(wl, carry=True)
    del run.states[1]["param_sumsq"]
    x0 = [p.clone() for p in run.params]
    gs = run.grads(0)
    ws = lib_workspace("adafactor", run.params, gs)
    with pytest.raises(_lib.MeoError) as e:
        _lib.meo_adafactor_step_carry(run.hps, 1, run.params, gs, run.states, False, ws)
    assert e.value.code == _lib.MEO_ENULL and "param_sumsq" in e.value.message
    torch.cuda.synchronize()
    for a, b in zip(x0, run.params):  # all or nothing
        assert torch.equal(a, b)


def test_front_end_carry_and_invalidation():
    """Adafactor(carry_param_sumsq=True) gives the binding's carry results bit for
    bit while nothing touches the parameters; a parameter written in place between
    steps makes the next step read X afresh (the plain step's bits on the
    modified parameter)."""
    from memory_efficient_optimizers_amd import Adafactor
    hp = {"beta1": 0.9, "weight_decay": 0.01}
    wl = workloads.custom("carry_front", "adafactor", [(96, 520), (520,), (3, 17, 40)], hparams=hp)
    scales = workloads.grad_scales(wl, "cuda")
    ref = Run(wl, carry=True)
    ps = [torch.nn.Parameter(p.clone()) for p in workloads.init_params(wl, "cuda")]
    o = Adafactor(ps, carry_param_sumsq=True, **hp)
    for t in range(3):
        gs = workloads.grads(wl, t, scales, "cuda")
        ref.step([g.clone() for g in gs], oracle_too=False)
        for p, g in zip(ps, gs):
            p.grad = g
        o.step()
    torch.cuda.synchronize()
    for p, q in zip(ps, ref.params):
        assert torch.equal(p.detach(), q)
    # write one parameter in place: the carried sums are stale for it
    with torch.no_grad():
        ps[0].mul_(0.5)
    gs = workloads.grads(wl, 3, scales, "cuda")
    # the expected step: the plain step from the same parameters and state
    for p, g in zip(ps, gs):
        p.grad = g
    x_before = [p.detach().clone() for p in ps]
    st_before = [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in o.state[p].items()} for p in ps]
    o.step()
    torch.cuda.synchronize()
    want = [x.clone() for x in x_before]
    sts = [{k: v for k, v in st.items() if k != "step"} for st in st_before]
    lib_step("adafactor", lib_hp("adafactor", hp), 4, want, gs, sts, lib_workspace("adafactor", want, gs))
    torch.cuda.synchronize()
    for p, q in zip(ps, want):
        assert torch.equal(p.detach(), q)


@pytest.mark.timeout(900)
def test_carry_full_llama7b_sampled():
    """The 7B list (291 tensors) in one carry call per step, as the bench runs it:
    three chained steps checked on a q projection, a down projection, the lm_head,
    the embedding and the final norm, and the carried sums of those tensors."""
    wl = workloads.WORKLOADS["adafactor_llama7b"]
    names = [s.name for s in wl.specs]
    sample = [0, names.index("model.layers.17.self_attn.q_proj.weight"),
              names.index("model.layers.30.mlp.down_proj.weight"), names.index("lm_head.weight"),
              names.index("model.norm.weight")]

    def sums(t, ps, sts, ox):
        for k in sample:
            want = float(np.sum(np.square(ox[k])))
            got = float(sts[k]["param_sumsq"].item())
            print(f"  carry 7B step {t} {names[k]}: sum(X^2) rel err {abs(got - want) / want:.2e}", flush=True)
            assert abs(got - want) / want <= SUMSQ_ORACLE

    list_run(wl, sample, 3, carry=True, workers=len(sample), on_check=sums)


def test_front_end_plain_steps_in_between_drop_the_carry():
    """A group switched to scale_parameter=False for a step (the plain step, whose
    writes do not bump version counters) and back: the next carry step reads X
    again, so it equals the plain step on the same parameters and state."""
    from memory_efficient_optimizers_amd import Adafactor
    hp = {"beta1": 0.9}
    wl = workloads.custom("carry_toggle", "adafactor", [(96, 520), (520,)], hparams=hp)
    scales = workloads.grad_scales(wl, "cuda")
    ps = [torch.nn.Parameter(p.clone()) for p in workloads.init_params(wl, "cuda")]
    o = Adafactor(ps, carry_param_sumsq=True, **hp)
    for t in range(4):
        gs = workloads.grads(wl, t, scales, "cuda")
        for p, g in zip(ps, gs):
            p.grad = g
        o.param_groups[0]["scale_parameter"] = t != 2
        if t == 3:
            x_before = [p.detach().clone() for p in ps]
            st_before = [{k: v.clone() for k, v in o.state[p].items() if k != "step"} for p in ps]
        o.step()
    torch.cuda.synchronize()
    want = [x.clone() for x in x_before]
    lib_step("adafactor", lib_hp("adafactor", hp), 4, want, gs, st_before, lib_workspace("adafactor", want, gs))
    torch.cuda.synchronize()
    for p, q in zip(ps, want):
        assert torch.equal(p.detach(), q)
