"""meo_adafactor_step_noalloc, the Adafactor step for callers that cannot allocate
device memory, through the C ABI: it must give exactly the bits of
meo_adafactor_step (same kernels in the same order), with no device allocation,
on two calls in a row (the second over a smaller list, which reuses the scratch
the first left), and refuse a list too large for its scratch before touching
anything."""
import pytest
import torch

import workloads
from memory_efficient_optimizers_amd import _lib
from tests.harness import lib_hp, lib_states, lib_workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


HP = {"beta1": 0.9, "weight_decay": 0.05}
# A Llama-7B decoder layer's shapes at a quarter of the hidden size, plus ragged,
# 1-D, batched and empty tensors (every first-pass kind).
BIG = [(1024, 1024), (2752, 1024), (1024, 2752), (1024,), (37, 1001), (2, 3, 72, 136), (0, 5), (5000,),
       (3, 16384), (700, 8)]
SMALL = [(129, 1024), (300,), (65, 513)]


def _inputs(name, shapes, seed):
    wl = workloads.custom(name, "adafactor", shapes, hparams=HP, grad_dtype=torch.bfloat16, grad_std=1e-3,
                          grad_scaling="rowcol", seed=seed)
    ps = workloads.init_params(wl, "cuda")
    scales = workloads.grad_scales(wl, "cuda")
    return wl, ps, scales


def _clone(ps, sts):
    return [p.clone() for p in ps], [{k: v.clone() for k, v in st.items()} for st in sts]


def _same(a_ps, a_sts, b_ps, b_sts):
    for p, q in zip(a_ps, b_ps):
        assert torch.equal(p, q)
    for sa, sb in zip(a_sts, b_sts):
        for k in sa:
            assert torch.equal(sa[k], sb[k]), k


def test_noalloc_equals_step_on_two_calls_in_a_row():
    hps = lib_hp("adafactor", HP)
    runs = []
    for name, shapes, seed in (("na_big", BIG, 1), ("na_small", SMALL, 2)):
        wl, ps, scales = _inputs(name, shapes, seed)
        sts = lib_states("adafactor", ps, HP)
        runs.append((wl, ps, sts, scales))
    ref = [_clone(ps, sts) for _, ps, sts, _ in runs]
    # the plain entry point, with a workspace of its own
    for (wl, _, _, scales), (ps, sts) in zip(runs, ref):
        for t in (1, 2):
            gs = workloads.grads(wl, t - 1, scales, "cuda")
            _lib.meo_adafactor_step(hps, t, ps, gs, sts, lib_workspace("adafactor", ps, gs))
    torch.cuda.synchronize()
    # the no-allocation entry point: the big list, then the smaller one, twice. The
    # library's code (and with it the scratch array) is loaded on the device by a
    # first call on a throwaway list; the gradients are drawn beforehand, so the
    # device's free memory must not move across the calls.
    wl0, ps0, sc0 = _inputs("na_warm", [(64, 512)], 9)
    _lib.meo_adafactor_step_noalloc(hps, 1, ps0, workloads.grads(wl0, 0, sc0, "cuda"),
                                    lib_states("adafactor", ps0, HP))
    grads = {(i, t): workloads.grads(wl, t - 1, scales, "cuda") for i, (wl, _, _, scales) in enumerate(runs)
             for t in (1, 2)}
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    for t in (1, 2):
        for i, (wl, ps, sts, scales) in enumerate(runs):
            _lib.meo_adafactor_step_noalloc(hps, t, ps, grads[(i, t)], sts)
            torch.cuda.synchronize()
    free_after = torch.cuda.mem_get_info()[0]
    for (_, ps, sts, _), (rps, rsts) in zip(runs, ref):
        _same(ps, sts, rps, rsts)
    assert free_after == free_before, (free_before, free_after)


def test_noalloc_on_a_side_stream():
    hps = lib_hp("adafactor", HP)
    wl, ps, scales = _inputs("na_stream", SMALL, 3)
    sts = lib_states("adafactor", ps, HP)
    rps, rsts = _clone(ps, sts)
    gs = workloads.grads(wl, 0, scales, "cuda")
    _lib.meo_adafactor_step(hps, 1, rps, gs, rsts, lib_workspace("adafactor", rps, gs))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _lib.meo_adafactor_step_noalloc(hps, 1, ps, gs, sts, side)
    torch.cuda.synchronize()
    _same(ps, sts, rps, rsts)


def test_noalloc_refuses_a_list_beyond_its_scratch():
    """70 matrices of 4096 x 4096 need ~75 MB of workspace, more than the scratch's
    64 MiB: refused before anything runs, nothing touched."""
    hps = lib_hp("adafactor", HP)
    shapes = [(4096, 4096)] * 70
    ps = [torch.full(s, 0.5, device="cuda") for s in shapes]
    gs = [torch.full(s, 1e-3, dtype=torch.bfloat16, device="cuda") for s in shapes]
    assert _lib.meo_adafactor_workspace_size(ps, gs) > _lib.MEO_NOALLOC_SCRATCH_BYTES
    sts = lib_states("adafactor", ps, HP)
    with pytest.raises(_lib.MeoError) as e:
        _lib.meo_adafactor_step_noalloc(hps, 1, ps, gs, sts)
    assert e.value.code == _lib.MEO_EWORKSPACE and "at most" in e.value.message
    torch.cuda.synchronize()
    assert all(bool((p == 0.5).all()) for p in ps)
    assert all(not st["exp_avg"].any() and not st["exp_avg_sq_row"].any() for st in sts)


@pytest.mark.parametrize("seed", range(24))
def test_noalloc_equals_step_on_random_lists(seed):
    """Random Adafactor lists (the sweep's draws: edge-sized sides, 1-D to 3-D, every
    storage class, random valid hyperparameters): two steps through the no-allocation
    entry point give the plain step's bits."""
    import random
    from tests.test_gpu_sweep import _hparams, _shape
    rng = random.Random(15000 + seed)
    hp = _hparams(rng, "adafactor")
    shapes = [_shape(rng) for _ in range(rng.randint(1, 5))]
    pdt = rng.choice([torch.float32, torch.bfloat16])
    sdt = rng.choice([torch.float32, torch.bfloat16, torch.int8])
    gdt = rng.choice([torch.float32, torch.bfloat16])
    print(f"noalloc case {seed}: {hp} shapes={shapes} param={pdt} state={sdt} grad={gdt}", flush=True)
    wl = workloads.custom(f"na_rand{seed}", "adafactor", shapes, hparams=hp, grad_dtype=gdt, seed=seed,
                          param_dtype=pdt, state_dtype=sdt)
    scales = workloads.grad_scales(wl, "cuda")
    ps = workloads.init_params(wl, "cuda")
    sts = lib_states("adafactor", ps, hp, sdt, min_8bit_size=1024)
    ref_ps, ref_sts = _clone(ps, sts)
    hps = lib_hp("adafactor", hp)
    for t in (1, 2):
        gs = workloads.grads(wl, t - 1, scales, "cuda")
        _lib.meo_adafactor_step(hps, t, ref_ps, gs, ref_sts, lib_workspace("adafactor", ref_ps, gs))
        _lib.meo_adafactor_step_noalloc(hps, t, ps, gs, sts)
    torch.cuda.synchronize()
    _same(ps, sts, ref_ps, ref_sts)
