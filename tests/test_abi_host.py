"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and validates arguments (codes and page messages) before any
device work. No compute call is made, so these run without a GPU: validation
only inspects pointers, never dereferences them."""
import ctypes
import json
import os
import re

import pytest
import torch

from memory_efficient_optimizers_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "meo.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmeo.so is not built: run `python -m memory_efficient_optimizers_amd.build`")
    return _lib.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(meo_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    declared = int(re.search(r"#define MEO_VERSION (\d+)", open(HEADER).read()).group(1))
    assert _lib.meo_version() == declared


def test_defaults_are_the_pages(lib):
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "page_defaults.json")))
    a = _lib.meo_adafactor_defaults()
    g = gold["adafactor"]
    assert (a.has_lr, a.has_beta1) == (0, 0)
    assert (a.eps1, a.eps2) == tuple(g["eps"])
    assert a.clip_threshold == g["clip_threshold"] and a.decay_rate == g["decay_rate"]
    assert a.weight_decay == g["weight_decay"]
    assert (a.scale_parameter, a.relative_step, a.warmup_init) == (1, 1, 0)
    c = _lib.meo_came_defaults()
    g = gold["came"]
    assert c.has_lr == 0 and (c.eps1, c.eps2) == tuple(g["eps"])
    assert (c.beta1, c.beta2, c.beta3) == tuple(g["betas"])
    assert c.clip_threshold == g["clip_threshold"] and c.weight_decay == g["weight_decay"]
    l = _lib.meo_lamb_defaults()
    g = gold["lamb"]
    assert l.lr == g["lr"] and (l.beta1, l.beta2) == tuple(g["betas"]) and l.eps == g["eps"]
    assert l.weight_decay == g["weight_decay"] and l.bias_correction == 1


def _mk(shapes, gdt=torch.float32):
    ps = [torch.zeros(s, dtype=torch.float32) for s in shapes]
    gs = [torch.zeros(s, dtype=gdt) for s in shapes]
    return ps, gs


def _af_states(ps, beta1=False):
    return [_lib.init_state("adafactor", p, beta1=beta1) for p in ps]


def _code(fn, *a):
    with pytest.raises(_lib.MeoError) as e:
        fn(*a)
    return e.value.code, e.value.message


def test_adafactor_validation(lib):
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "page_defaults.json")))["messages"]
    ps, gs = _mk([(4, 8), (8,)])
    st = _af_states(ps)
    _lib.meo_adafactor_validate(_lib.adafactor_hparams(), 1, ps, gs, st)
    code, msg = _code(_lib.meo_adafactor_validate, _lib.adafactor_hparams(lr=1e-3), 1, ps, gs, st)
    assert code == _lib.MEO_EINVAL and msg == gold["lr_with_relative_step"]
    code, msg = _code(_lib.meo_adafactor_validate,
                      _lib.adafactor_hparams(lr=1e-3, relative_step=False, warmup_init=True), 1, ps, gs, st)
    assert code == _lib.MEO_EINVAL and msg == gold["warmup_needs_relative_step"]
    assert _code(_lib.meo_adafactor_validate, _lib.adafactor_hparams(relative_step=False), 1,
                 ps, gs, st)[0] == _lib.MEO_EINVAL
    assert _code(_lib.meo_adafactor_validate, _lib.adafactor_hparams(clip_threshold=0.0), 1,
                 ps, gs, st)[0] == _lib.MEO_EINVAL
    assert _code(_lib.meo_adafactor_validate, _lib.adafactor_hparams(), 0, ps, gs, st)[0] == _lib.MEO_EINVAL
    # beta1 set but no first moment
    assert _code(_lib.meo_adafactor_validate, _lib.adafactor_hparams(beta1=0.9), 1,
                 ps, gs, st)[0] == _lib.MEO_ENULL
    # factored tensor without its row statistic
    bad = [dict(s) for s in st]
    del bad[0]["exp_avg_sq_row"]
    assert _code(_lib.meo_adafactor_validate, _lib.adafactor_hparams(), 1, ps, gs, bad)[0] == _lib.MEO_ENULL
    # 1-D tensor without its full statistic
    bad = [dict(s) for s in st]
    del bad[1]["exp_avg_sq"]
    assert _code(_lib.meo_adafactor_validate, _lib.adafactor_hparams(), 1, ps, gs, bad)[0] == _lib.MEO_ENULL


def test_tensor_checks(lib):
    ps, gs = _mk([(4, 8)])
    st = _af_states(ps)
    hp = ctypes_hp = _lib.adafactor_hparams()
    t = _lib._tensors(ps, gs)
    sts = _lib._states(_lib.meo_adafactor_state, _lib.ADAFACTOR_KEYS, st)

    def val(tensors):
        return lib.meo_adafactor_validate(_lib.ctypes.byref(ctypes_hp), 1, 1, tensors, sts)

    t[0].grad_dtype = 7
    assert val(t) == _lib.MEO_EDTYPE
    t[0].grad_dtype = _lib.MEO_F32
    t[0].param_dtype = 7
    assert val(t) == _lib.MEO_EDTYPE
    assert "param_dtype" in _lib.meo_last_error()
    t[0].param_dtype = _lib.MEO_F32
    t[0].state_dtype = 7
    assert val(t) == _lib.MEO_EDTYPE
    assert "state_dtype" in _lib.meo_last_error()
    t[0].state_dtype = _lib.MEO_BF16
    assert val(t) == _lib.MEO_OK
    t[0].state_dtype = _lib.MEO_F32
    # a bf16 parameter needs 2-byte alignment only, an fp32 one 4
    t[0].param = t[0].param + 2
    assert val(t) == _lib.MEO_EALIGN
    t[0].param_dtype = _lib.MEO_BF16
    assert val(t) == _lib.MEO_OK
    t[0].param = t[0].param + 1
    assert val(t) == _lib.MEO_EALIGN
    t[0].param = t[0].param - 3
    t[0].param_dtype = _lib.MEO_F32
    t[0].rows = -1
    assert val(t) == _lib.MEO_ESHAPE
    t[0].rows = 4
    t[0].ndim = 1  # 1-D view must have rows == 1
    assert val(t) == _lib.MEO_ESHAPE
    t[0].ndim = 2
    t[0].param = t[0].param + 2
    assert val(t) == _lib.MEO_EALIGN
    t[0].param = None
    assert val(t) == _lib.MEO_ENULL
    assert "param is NULL" in _lib.meo_last_error()
    assert lib.meo_adafactor_validate(_lib.ctypes.byref(hp), 1, 1, None, sts) == _lib.MEO_ENULL
    # a zero-element tensor needs no pointers and is skipped
    t[0].rows = 0
    assert val(t) == _lib.MEO_OK


def test_first_moment_alignment_follows_its_dtype(lib):
    """exp_avg must be 4-byte aligned as fp32 and 2-byte aligned as bf16, for every
    optimizer that keeps it."""
    ps, gs = _mk([(4, 8)])
    for opt, keys, cls, hp in (("adafactor", _lib.ADAFACTOR_KEYS, _lib.meo_adafactor_state,
                                _lib.adafactor_hparams(beta1=0.9)),
                               ("came", _lib.CAME_KEYS, _lib.meo_came_state, _lib.came_hparams(lr=1e-3)),
                               ("lamb", _lib.LAMB_KEYS, _lib.meo_lamb_state, _lib.lamb_hparams())):
        st = [_lib.init_state(opt, ps[0], beta1=True)]
        t = _lib._tensors(ps, gs)
        sts = _lib._states(cls, keys, st)
        fn = getattr(lib, f"meo_{opt}_validate")

        def val():
            return fn(_lib.ctypes.byref(hp), 1, 1, t, sts)

        assert val() == _lib.MEO_OK
        sts[0].exp_avg += 2
        assert val() == _lib.MEO_EALIGN, opt
        t[0].state_dtype = _lib.MEO_BF16
        assert val() == _lib.MEO_OK, opt
        sts[0].exp_avg += 1
        assert val() == _lib.MEO_EALIGN, opt


def test_eight_bit_first_moment_rules(lib):
    """An 8-bit first moment needs its scales, and a factored tensor needs
    cols % 128 == 0 (no quantization group crosses a row); 1-D and LAMB tensors
    take any length. int8 codes need no alignment."""
    for opt, keys, cls, hp in (("adafactor", _lib.ADAFACTOR_KEYS, _lib.meo_adafactor_state,
                                _lib.adafactor_hparams(beta1=0.9)),
                               ("came", _lib.CAME_KEYS, _lib.meo_came_state, _lib.came_hparams(lr=1e-3)),
                               ("lamb", _lib.LAMB_KEYS, _lib.meo_lamb_state, _lib.lamb_hparams())):
        fn = getattr(lib, f"meo_{opt}_validate")
        for shape, ok in (((4, 256), True), ((4, 200), opt == "lamb"), ((300,), True), ((2, 3, 128), True)):
            ps, gs = _mk([shape])
            st = [_lib.init_state(opt, ps[0], beta1=True, state_dtype=torch.int8)]
            assert st[0]["exp_avg"].dtype == torch.int8
            assert st[0]["exp_avg_scale"].numel() == -(-ps[0].numel() // 128)
            t = _lib._tensors(ps, gs, st)
            assert t[0].state_dtype == _lib.MEO_I8
            sts = _lib._states(cls, keys, st)
            code = fn(_lib.ctypes.byref(hp), 1, 1, t, sts)
            assert code == (_lib.MEO_OK if ok else _lib.MEO_ESHAPE), (opt, shape, code)
            if ok:
                sts[0].exp_avg += 1  # codes are bytes
                assert fn(_lib.ctypes.byref(hp), 1, 1, t, sts) == _lib.MEO_OK
                sts[0].exp_avg_scale = None
                assert fn(_lib.ctypes.byref(hp), 1, 1, t, sts) == _lib.MEO_ENULL
                assert "exp_avg_scale" in _lib.meo_last_error()
    # no first moment (Adafactor without beta1): the dtype is not used
    ps, gs = _mk([(4, 200)])
    st = [_lib.init_state("adafactor", ps[0], beta1=False)]
    t = _lib._tensors(ps, gs, st)
    t[0].state_dtype = _lib.MEO_I8
    sts = _lib._states(_lib.meo_adafactor_state, _lib.ADAFACTOR_KEYS, st)
    assert lib.meo_adafactor_validate(_lib.ctypes.byref(_lib.adafactor_hparams()), 1, 1, t, sts) == _lib.MEO_OK


def test_binding_rejects_mismatched_state_dtypes(lib):
    """The binding declares exp_avg's dtype from the tensor itself and refuses
    non-fp32 statistics (the library could not tell)."""
    ps, gs = _mk([(4, 8)])
    st = _lib.init_state("adafactor", ps[0], beta1=True, state_dtype=torch.bfloat16)
    assert st["exp_avg"].dtype == torch.bfloat16 and st["exp_avg_sq_row"].dtype == torch.float32
    assert _lib._tensors(ps, gs, [st])[0].state_dtype == _lib.MEO_BF16
    bad = dict(st)
    bad["exp_avg_sq_row"] = bad["exp_avg_sq_row"].to(torch.bfloat16)
    with pytest.raises(TypeError):
        _lib.meo_adafactor_validate(_lib.adafactor_hparams(beta1=0.9), 1, ps, gs, [bad])
    with pytest.raises(TypeError):
        _lib.tensor_struct(ps[0].to(torch.float16), gs[0])


def test_workspace_checks(lib):
    ps, gs = _mk([(100, 600), (33,)])
    need = _lib.meo_adafactor_workspace_size(ps, gs)
    assert need > 0 and need % 256 == 0
    ps2, gs2 = _mk([(100, 600), (33,), (5000, 7)])
    assert _lib.meo_adafactor_workspace_size(ps2, gs2) > need
    st = _af_states(ps)
    hp = _lib.adafactor_hparams()
    # the workspace is checked before any device work: too small / missing
    small = torch.empty(need - 256, dtype=torch.uint8)
    assert _code(_lib.meo_adafactor_step, hp, 1, ps, gs, st, small, 0)[0] == _lib.MEO_EWORKSPACE
    assert _code(_lib.meo_adafactor_step, hp, 1, ps, gs, st, None, 0)[0] == _lib.MEO_EWORKSPACE
    assert _lib.meo_lamb_workspace_size(ps, gs) > 0
    assert _lib.meo_came_workspace_size(ps, gs) > 0
    # host memory of the right size and alignment is not device memory: refused
    # before anything is enqueued (here, with no device at all, and on a GPU machine)
    host = torch.empty(need + 256, dtype=torch.uint8)
    off = (-host.data_ptr()) % 256
    code, msg = _code(_lib.meo_adafactor_step, hp, 1, ps, gs, st, host[off:off + need], 0)
    assert code in (_lib.MEO_EWORKSPACE, _lib.MEO_EHIP), (code, msg)


def test_came_validation(lib):
    ps, gs = _mk([(4, 8), (8,)], torch.bfloat16)
    st = [_lib.init_state("came", p) for p in ps]
    _lib.meo_came_validate(_lib.came_hparams(lr=2e-4), 1, ps, gs, st)
    assert _code(_lib.meo_came_validate, _lib.came_hparams(), 1, ps, gs, st)[0] == _lib.MEO_EINVAL
    assert _code(_lib.meo_came_validate, _lib.came_hparams(lr=1e-3, betas=(0.9, 0.999, 1.0)), 1,
                 ps, gs, st)[0] == _lib.MEO_EINVAL
    bad = [dict(s) for s in st]
    del bad[0]["exp_avg_res_col"]
    assert _code(_lib.meo_came_validate, _lib.came_hparams(lr=1e-3), 1, ps, gs, bad)[0] == _lib.MEO_ENULL


def test_lamb_validation(lib):
    ps, gs = _mk([(4, 8), (8,)])
    st = [_lib.init_state("lamb", p) for p in ps]
    _lib.meo_lamb_validate(_lib.lamb_hparams(), 1, ps, gs, st)
    for bad in (dict(lr=-1.0), dict(eps=-1.0), dict(betas=(1.0, 0.999)), dict(betas=(0.9, 1.5))):
        assert _code(_lib.meo_lamb_validate, _lib.lamb_hparams(**bad), 1, ps, gs, st)[0] == _lib.MEO_EINVAL
    bad = [dict(s) for s in st]
    del bad[1]["exp_avg"]
    assert _code(_lib.meo_lamb_validate, _lib.lamb_hparams(), 1, ps, gs, bad)[0] == _lib.MEO_ENULL


def test_empty_list_is_a_noop(lib):
    assert lib.meo_adafactor_step(_lib.ctypes.byref(_lib.adafactor_hparams()), 1, 0, None, None, None, 0,
                                  None) == _lib.MEO_OK


def test_shard_checks(lib):
    """Row-sharded entry points validate shards and the partial-sum buffer on the
    host before anything is enqueued."""
    ps, gs = _mk([(4, 8), (8, 20), (30,)])
    st = [_lib.init_state("adafactor", p, beta1=True) for p in ps]
    hp = _lib.adafactor_hparams(beta1=0.9)
    size = _lib.meo_adafactor_partials_size(ps, gs)
    assert size == (2 * 8 + 1) + 1 + (2 * 20 + 1) + 1 + 2
    part = torch.zeros(size)
    # a factored shard needs row-complete rows: cols % 8 == 0
    code, msg = _code(_lib.meo_adafactor_shard_stats, hp, 1, ps, gs, [8, 16, 30], st, part, None, 0)
    assert code == _lib.MEO_ESHAPE and "cols % 8" in msg
    ps, gs = _mk([(4, 8), (8, 24), (30,)])
    st = [_lib.init_state("adafactor", p, beta1=True) for p in ps]
    part = torch.zeros(_lib.meo_adafactor_partials_size(ps, gs))
    code, msg = _code(_lib.meo_adafactor_shard_stats, hp, 1, ps, gs, [8, 4, 30], st, part, None, 0)
    assert code == _lib.MEO_ESHAPE and "rows_total" in msg
    code, msg = _code(_lib.meo_adafactor_shard_stats, hp, 1, ps, gs, [8, 16, 20], st, part, None, 0)
    assert code == _lib.MEO_ESHAPE
    code, msg = _code(_lib.meo_adafactor_shard_apply, hp, 1, ps, gs, [8, 16, 30], st, None, None, 0)
    assert code == _lib.MEO_ENULL and "partials" in msg
    # host memory as partials: refused (no device at all here, or not device memory)
    code, msg = _code(_lib.meo_adafactor_shard_apply, hp, 1, ps, gs, [8, 16, 30], st, part, None, 0)
    assert code in (_lib.MEO_EMEMORY, _lib.MEO_EHIP)
    lst = [_lib.init_state("lamb", p) for p in ps]
    assert _lib.meo_lamb_partials_size(ps, gs) == 6
    code, msg = _code(_lib.meo_lamb_shard_stats, _lib.lamb_hparams(), 1, ps, gs, [31, 191, 30], lst,
                      torch.zeros(6), None, 0)
    assert code == _lib.MEO_ESHAPE   # 4 x 8 = 32 elements > 31


def test_galore_defaults_are_the_pages(lib):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "page_defaults.json")))["galore"]
    h = _lib.meo_galore_defaults()
    assert (h.rank, h.update_proj_gap, h.scale) == (g["rank"], g["update_proj_gap"], g["scale"])
    assert h.proj_type == {"std": _lib.MEO_GALORE_STD}[g["proj_type"]]
    # fields the pages name without values: the readings stated in meo.h
    assert (h.lr, h.beta1, h.beta2, h.eps, h.weight_decay) == (1e-3, 0.9, 0.999, 1e-8, 0.0)


def _ga(shapes, rank=8, gdt=torch.bfloat16):
    ps = [torch.zeros(s, dtype=torch.float32) for s in shapes]
    gs = [torch.zeros(s, dtype=gdt) for s in shapes]
    return ps, gs, [_lib.galore_init_state(p, rank) for p in ps]


def test_galore_validation(lib):
    ps, gs, st = _ga([(16, 40), (40, 16), (9,), (2, 3, 4)])
    h = _lib.galore_hparams(rank=8)
    _lib.meo_galore_validate(h, 1, ps, gs, st)
    assert [_lib.meo_galore_rank(h, p) for p in ps] == [8, 8, 0, 0]
    assert _lib.meo_galore_rank(_lib.galore_hparams(rank=300), torch.zeros(20, 30)) == 20
    # workspace per projected tensor, each array 256-byte aligned: two bf16 planes of
    # [max(m, n)][r] (the step); two fp32 [r][min], one fp32 [r][max] and four fp64
    # [r][r] arrays (the refresh)
    a = lambda b: (b + 255) // 256 * 256
    per = 2 * a(40 * 8 * 2) + 2 * a(8 * 16 * 4) + a(8 * 40 * 4) + 4 * a(8 * 8 * 8)
    assert _lib.meo_galore_workspace_size(h, ps, gs) == 2 * per
    for bad, code in ((dict(lr=-1.0), _lib.MEO_EINVAL), (dict(betas=(1.0, 0.9)), _lib.MEO_EINVAL),
                      (dict(eps=-1e-8), _lib.MEO_EINVAL), (dict(rank=0), _lib.MEO_EINVAL),
                      (dict(update_proj_gap=0), _lib.MEO_EINVAL), (dict(scale=float("nan")), _lib.MEO_EINVAL)):
        assert _code(_lib.meo_galore_validate, _lib.galore_hparams(**dict(dict(rank=8), **bad)), 1, ps, gs, st)[0] == code
    assert _code(_lib.meo_galore_validate, h, 0, ps, gs, st)[0] == _lib.MEO_EINVAL
    # a projected tensor needs a bf16 gradient; the flat ones take fp32 too
    ps2, gs2, st2 = _ga([(16, 40)], gdt=torch.float32)
    code, msg = _code(_lib.meo_galore_validate, h, 1, ps2, gs2, st2)
    assert code == _lib.MEO_EDTYPE and "bf16 gradient" in msg
    ps3, gs3, st3 = _ga([(33,), (2, 3, 4)], gdt=torch.float32)
    _lib.meo_galore_validate(h, 1, ps3, gs3, st3)
    # effective rank above 256
    ps4, gs4, st4 = _ga([(300, 400)], rank=257)
    assert _code(_lib.meo_galore_validate, _lib.galore_hparams(rank=257), 1, ps4, gs4, st4)[0] == _lib.MEO_EINVAL
    # missing projector, float32 state dtype only
    bad = [dict(s) for s in st]
    del bad[0]["projector_t"]
    assert _code(_lib.meo_galore_validate, h, 1, ps, gs, bad)[0] == _lib.MEO_ENULL
    t = _lib._tensors(ps, gs)
    t[0].state_dtype = _lib.MEO_BF16
    assert lib.meo_galore_validate(_lib.ctypes.byref(h), 1, len(ps), t, _lib._galore_states(st)) == _lib.MEO_EDTYPE
    with pytest.raises(TypeError):
        _lib._galore_states([dict(st[0], projector=st[0]["projector"].float())])
    # reverse_std: the projector on the longer side, moments on the shorter
    hr = _lib.galore_hparams(rank=8, proj_type="reverse_std")
    psr, gsr = ps[:2], gs[:2]
    str_ = [_lib.galore_init_state(p, 8, "reverse_std") for p in psr]
    assert str_[0]["projector"].shape == (40, 8) and str_[0]["exp_avg"].shape == (16, 8)
    _lib.meo_galore_validate(hr, 1, psr, gsr, str_)
    per_r = 2 * a(16 * 8 * 2) + 2 * a(8 * 40 * 4) + a(8 * 40 * 4) + 4 * a(8 * 8 * 8)
    assert _lib.meo_galore_workspace_size(hr, psr, gsr) == 2 * per_r
    bad_hp = _lib.galore_hparams(rank=8)
    bad_hp.proj_type = 2
    assert _code(_lib.meo_galore_validate, bad_hp, 1, ps, gs, st)[0] == _lib.MEO_EINVAL
    # an empty list is a no-op
    _lib.meo_galore_step(h, 1, [], [], [], stream=0)


def test_binding_rejects_strided_states(lib):
    """The library reads every state row-major: a transposed view would be read as
    its transpose, so the binding refuses it."""
    ps, gs, st = _ga([(16, 40)])
    bad = [dict(st[0], projector=st[0]["projector_t"].T)]
    with pytest.raises(ValueError):
        _lib._galore_states(bad)
    p = torch.zeros(6, 4)
    s = _lib.init_state("lamb", p)
    s["exp_avg_sq"] = torch.zeros(4, 6).T
    with pytest.raises(ValueError):
        _lib._states(_lib.meo_lamb_state, _lib.LAMB_KEYS, [s])


def test_carry_calls_check_param_sumsq_first(lib):
    """The carry entry points refuse a tensor with elements but no param_sumsq
    (when scale_parameter needs RMS(X)) before touching anything else; an empty
    tensor needs none, and without scale_parameter none is needed at all (the
    call then fails on its missing workspace, the next check)."""
    ps, gs = _mk([(4, 8), (8,), (0, 5)])
    st = _af_states(ps)
    for s in st:
        s["param_sumsq"] = torch.zeros(1)
    hp = _lib.adafactor_hparams()
    miss = [dict(s) for s in st]
    del miss[1]["param_sumsq"]
    code, msg = _code(_lib.meo_adafactor_step_carry, hp, 1, ps, gs, miss, True, None, 0)
    assert code == _lib.MEO_ENULL and msg == "tensor 1: param_sumsq is NULL"
    code, msg = _code(_lib.meo_adafactor_shard_stats_carry, hp, 1, ps, gs, [4, 8, 0], miss, True, None, None, 0)
    assert code == _lib.MEO_ENULL and msg == "tensor 1: param_sumsq is NULL"
    code, msg = _code(_lib.meo_adafactor_shard_apply_carry, hp, 1, ps, gs, [4, 8, 0], miss, None, None, 0)
    assert code == _lib.MEO_ENULL and msg == "tensor 1: param_sumsq is NULL"
    empty_ok = [dict(s) for s in st]
    del empty_ok[2]["param_sumsq"]
    assert _code(_lib.meo_adafactor_step_carry, hp, 1, ps, gs, empty_ok, False, None, 0)[0] == _lib.MEO_EWORKSPACE
    no_scale = _lib.adafactor_hparams(scale_parameter=False)
    assert _code(_lib.meo_adafactor_step_carry, no_scale, 1, ps, gs, miss, True, None, 0)[0] == _lib.MEO_EWORKSPACE
    # the plain step ignores param_sumsq
    assert _code(_lib.meo_adafactor_step, hp, 1, ps, gs, miss, None, 0)[0] == _lib.MEO_EWORKSPACE


@pytest.mark.parametrize("opt", ["adafactor", "came", "lamb"])
def test_scalar_offsets(lib, opt):
    """Each tensor with elements gets its own 8 slots inside the workspace the step
    would use (256-byte aligned, no overlap); empty tensors get -1; bad arguments are
    refused on the host."""
    shapes = [(4, 8), (0, 5), (8,), (3, 70, 130), (), (1000, 1)]
    ps, gs = _mk(shapes)
    offs = getattr(_lib, f"meo_{opt}_scalar_offsets")(ps, gs)
    ws_floats = getattr(_lib, f"meo_{opt}_workspace_size")(ps, gs) // 4
    live = [o for o, s in zip(offs, shapes) if o >= 0]
    assert [o < 0 for o in offs] == [torch.zeros(s).numel() == 0 for s in shapes]
    assert all(o % 64 == 0 and o + len(_lib.SCALAR_SLOTS) <= ws_floats for o in live)
    assert len(set(live)) == len(live)
    spans = sorted((o, o + len(_lib.SCALAR_SLOTS)) for o in live)
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    fn = getattr(lib, f"meo_{opt}_scalar_offsets")
    out = (ctypes.c_int64 * 2)()
    assert fn(-1, None, out) == _lib.MEO_ESHAPE
    assert fn(2, None, out) == _lib.MEO_ENULL
    assert fn(0, None, None) == _lib.MEO_OK
    bad = _lib._tensors(*_mk([(4, 8)]))
    bad[0].rows = -3
    assert fn(1, bad, out) == _lib.MEO_ESHAPE
