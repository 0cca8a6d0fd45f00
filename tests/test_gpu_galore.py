"""GPU parity of the GaLore step (meo_galore_step through the C ABI) against the
fp64 oracle (oracle/galore.py), on seeded inputs from workloads.galore_inputs.

Steps here are not refresh steps (t - 1 is not a multiple of update_proj_gap), so
the projector is an input: a seeded random orthonormal basis rounded to bf16,
identical on both sides. Bars:

* exp_avg, exp_avg_sq and an fp32 parameter: the fp32 bar of tests/harness.py
  (1e-5; signed outputs floored at their RMS). The low-rank gradient is a sum of
  d products of bf16 values, exact in fp32, accumulated in fp32 by the matrix
  cores: about sqrt(d / 16) roundings of 2^-24 each, far below the bar.
* The update x_new - x of an fp32 parameter, floored at its RMS: 1e-4. The update
  is about lr * scale / |x| ~ 1e-2 of the parameter here, so the fp32 rounding of
  x_new alone contributes up to 2^-24 / 1e-2 ~ 6e-6; the low-rank direction enters
  the back-projection as two bf16 planes whose sum carries it to 2^-17 relative.
* A bf16 parameter: the 16-bit bar ("rounded").
* The projector and its transpose are not written on such steps (bit-exact).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import galore as ga
from memory_efficient_optimizers_amd import GaLoreAdamW, _lib
from tests.harness import check_bar, dx_errs, floored_rel_err, to64

pytestmark = pytest.mark.gpu

TOL_UPDATE = 1e-4


def run_case(shapes, rank, t=5, hp=None, param_dtype=torch.float32, seed=0, check_update=True):
    dev = "cuda"
    hp = dict(dict(lr=0.05, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, scale=0.25), **(hp or {}))
    hpo = dict(hp, rank=rank)
    params, grads, states = workloads.galore_inputs(shapes, rank, seed, param_dtype=param_dtype, device=dev,
                                                    proj_type=hp.get("proj_type", "std"))
    x0 = [to64(p) for p in params]
    g0 = [to64(g) for g in grads]
    s0 = [{k: to64(v) for k, v in s.items() if k != "projector_t"} for s in states]
    pt0 = [s["projector_t"].clone() if "projector_t" in s else None for s in states]
    h = _lib.galore_hparams(**hpo)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print(f"galore step: shapes={shapes} rank={rank} t={t} param={param_dtype}", flush=True)
    _lib.meo_galore_step(h, t, params, grads, states, ws)
    torch.cuda.synchronize()
    bad = []
    for k, shape in enumerate(shapes):
        if int(np.prod(shape)) == 0:
            continue
        want_x, want_s = ga.galore_step_tensor(x0[k], g0[k], s0[k], hpo, t,
                                               param_bf16=param_dtype == torch.bfloat16)
        got_x = to64(params[k])
        kind = "f32" if param_dtype == torch.float32 else "rounded"
        checks = [(kind, "param", got_x, want_x),
                  ("f32", "exp_avg", to64(states[k]["exp_avg"]), want_s["exp_avg"]),
                  ("f32", "exp_avg_sq", to64(states[k]["exp_avg_sq"]), want_s["exp_avg_sq"])]
        b1 = ga.galore_hparams(hpo)["betas"][0]
        for kd, key, a, b in checks:
            ok, err, over, n = check_bar(kd, key, a, b, x0=x0[k], prev=s0[k]["exp_avg"], beta1=b1,
                                         step_tol=TOL_UPDATE)
            if not ok:
                bad.append(f"tensor {k} {shape} {key}: err {err:.3g} ({over}/{n} above 1e-5)")
        if param_dtype == torch.float32 and check_update:
            # floored at RMS of the update, one fp32 spacing of the stored parameter
            # forgiven per element (its rounding, as in the other optimizers' step check)
            errs, _ = dx_errs(got_x, x0[k], want_x, x0[k], floor=1.0)
            e = float(np.max(errs)) if errs.size else 0.0
            if e > TOL_UPDATE:
                bad.append(f"tensor {k} {shape} update: err {e:.3g}")
        if "projector" in states[k]:
            assert torch.equal(states[k]["projector"].cpu(), torch.from_numpy(s0[k]["projector"]).to(torch.bfloat16))
            assert torch.equal(states[k]["projector_t"], pt0[k])
    assert not bad, "; ".join(bad)
    return params, states


@pytest.mark.parametrize("shape,rank", [
    ((256, 128), 32),     # m >= n, whole tiles, one active wave
    ((128, 320), 64),     # m < n (transposed gradient tile)
    ((300, 136), 40),     # ragged rows, r not a multiple of 32
    ((72, 333), 24),      # ragged, odd columns: element-wise loads
    ((200, 96), 13),      # r not a multiple of 8
    ((200, 192), 13),     # wide projection: ragged rows, r not a multiple of 8, 3 contraction steps
    ((1000, 256), 100),   # wide projection: second column wave partly past r
    ((300, 64), 64),      # wide projection: a single contraction step
    ((128, 328), 64),     # m < n wide projection (transpose reads): ragged last tile of 72 rows
    ((192, 1000), 100),   # m < n wide projection: 3 contraction steps, a wave partly past r
    ((64, 296), 32),      # m < n wide projection: a single contraction step
    ((40, 24), 256),      # rank clamped to min(m, n)
    ((512, 384), 256),    # full rank-256 tile, several contraction blocks
    ((300, 600), 256),    # m < n at rank 256
    ((64, 64), 64),       # square: projects the columns' space
    ((1, 48), 8),         # a single row: rank 1
])
def test_step_shapes(shape, rank):
    run_case([shape], rank)


@pytest.mark.parametrize("shape", [(256, 200), (96, 400)])
def test_step_bf16_param(shape):
    run_case([shape], 64, param_dtype=torch.bfloat16)


def test_step_weight_decay_and_late_step():
    run_case([(260, 130), (130, 260)], 48, t=187, hp=dict(weight_decay=0.1, lr=0.02, betas=(0.8, 0.95)))


def test_step_mixed_list():
    """2-D tensors of both sides with 1-D, 3-D (flat AdamW) and empty tensors."""
    run_case([(192, 64), (0, 5), (64, 500), (777,), (3, 5, 7), (1,), (8, 8)], 32, seed=3)


def test_step_llama_sized():
    """One Llama-7B-shaped MLP pair at rank 256 (rows of 4096 and 11008)."""
    run_case([(1024, 4096), (4096, 1024)], 256, seed=4)


def test_list_equals_singles():
    """Every block reads only its own tensor: a list step equals per-tensor steps bitwise."""
    shapes = [(200, 72), (72, 300), (129,)]
    dev = "cuda"
    h = _lib.galore_hparams(lr=0.05, rank=32)
    p1, g1, s1 = workloads.galore_inputs(shapes, 32, 9, device=dev)
    p2, g2, s2 = workloads.galore_inputs(shapes, 32, 9, device=dev)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, p1, g1), dev)
    _lib.meo_galore_step(h, 3, p1, g1, s1, ws)
    for k in range(len(shapes)):
        wk = _lib.workspace(_lib.meo_galore_workspace_size(h, [p2[k]], [g2[k]]), dev)
        _lib.meo_galore_step(h, 3, [p2[k]], [g2[k]], [s2[k]], wk)
    torch.cuda.synchronize()
    for k in range(len(shapes)):
        assert torch.equal(p1[k], p2[k])
        for key in s1[k]:
            assert torch.equal(s1[k][key], s2[k][key])



def test_direct_staging_equals_register_staging():
    """The kernels are chosen per list: the wide projection and the U-register
    back-projection (operands staged by global_load_lds) when every contraction
    length of the list is a multiple of 64, the register-staged ones otherwise. All
    feed the MFMAs the same fragments in the same order (the m < n wide projection
    through LDS transpose reads), so a tensor's step is bitwise the same on either.
    (256, 128) and (128, 320) at rank 64 take the wide and U-register kernels alone
    and the register-staged ones beside (200, 40) and (40, 200), whose rank 40 and
    contraction length 40 are not multiples of 64."""
    shapes = [(256, 128), (200, 40), (128, 320), (40, 200)]
    dev = "cuda"
    h = _lib.galore_hparams(lr=0.05, rank=64)
    p1, g1, s1 = workloads.galore_inputs(shapes, 64, 23, device=dev)
    p2, g2, s2 = workloads.galore_inputs(shapes, 64, 23, device=dev)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, p1, g1), dev)
    _lib.meo_galore_step(h, 5, p1, g1, s1, ws)
    for k in (0, 2):
        wk = _lib.workspace(_lib.meo_galore_workspace_size(h, [p2[k]], [g2[k]]), dev)
        _lib.meo_galore_step(h, 5, [p2[k]], [g2[k]], [s2[k]], wk)
    torch.cuda.synchronize()
    for k in (0, 2):
        assert not torch.equal(p1[k], workloads.galore_inputs(shapes, 64, 23, device=dev)[0][k])
        assert torch.equal(p1[k], p2[k])
        for key in s1[k]:
            assert torch.equal(s1[k][key], s2[k][key])


@pytest.mark.parametrize("shapes,direct", [([(256, 128), (40, 200)], 0), ([(200, 40), (128, 320)], 1)],
                         ids=["right-direct", "left-direct"])
def test_one_direct_side_equals_singles(shapes, direct):
    """With only one side of a list direct, the projection launches the wide kernel for
    that side and the register-staged one for the other; alone, the direct tensor
    takes the one launch for both sides. Its step is bitwise the same either way."""
    dev = "cuda"
    h = _lib.galore_hparams(lr=0.05, rank=64)
    p1, g1, s1 = workloads.galore_inputs(shapes, 64, 29, device=dev)
    p2, g2, s2 = workloads.galore_inputs(shapes, 64, 29, device=dev)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, p1, g1), dev)
    _lib.meo_galore_step(h, 4, p1, g1, s1, ws)
    for k in range(len(shapes)):
        wk = _lib.workspace(_lib.meo_galore_workspace_size(h, [p2[k]], [g2[k]]), dev)
        _lib.meo_galore_step(h, 4, [p2[k]], [g2[k]], [s2[k]], wk)
    torch.cuda.synchronize()
    x0 = workloads.galore_inputs(shapes, 64, 29, device=dev)[0]
    for k in range(len(shapes)):
        assert not torch.equal(p1[k], x0[k])
        assert torch.equal(p1[k], p2[k]), (shapes[k], k == direct)
        for key in s1[k]:
            assert torch.equal(s1[k][key], s2[k][key]), (shapes[k], key)


@pytest.mark.parametrize("pdt,offset", [(torch.float32, 1), (torch.float32, 3), (torch.bfloat16, 5)])
def test_offset_parameter_views(pdt, offset):
    """Parameters carved from one buffer at element offsets that keep their dtype's
    alignment but not 16 bytes (flat-parameter frameworks hand them over so): the
    back-projection must take its element-wise edges for them. Against the same step on
    fresh (aligned) parameters: bitwise equal, the same values computed either way."""
    dev = "cuda"
    shapes = [(256, 128), (128, 320), (320, 256)]
    h = _lib.galore_hparams(lr=0.05, rank=64)
    pa, ga_, sa = workloads.galore_inputs(shapes, 64, 41, param_dtype=pdt, device=dev)
    pb, gb, sb = workloads.galore_inputs(shapes, 64, 41, param_dtype=pdt, device=dev)
    sizes = [int(np.prod(sh)) for sh in shapes]
    buf = torch.zeros(offset + sum(sizes) + 16, dtype=pdt, device=dev)
    views, o = [], offset
    for n_, sh, p in zip(sizes, shapes, pb):
        v = buf[o:o + n_].view(sh)
        v.copy_(p)
        views.append(v)
        o += n_
    assert all(v.data_ptr() % 16 != 0 for v in views)
    for params, grads, states in ((pa, ga_, sa), (views, gb, sb)):
        ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
        _lib.meo_galore_step(h, 3, params, grads, states, ws)
    torch.cuda.synchronize()
    for k in range(len(shapes)):
        assert not torch.equal(pa[k], workloads.galore_inputs(shapes, 64, 41, param_dtype=pdt, device=dev)[0][k])
        assert torch.equal(pa[k], views[k]), k
        for key in sa[k]:
            assert torch.equal(sa[k][key], sb[k][key]), (k, key)


def test_mixed_parameter_dtypes_list():
    """A list whose parameters mix fp32 and bf16 takes the direct-staged back-projection
    (the U-register kernel is compiled per parameter dtype); each tensor alone takes the
    U-register kernel. Both run the same MFMA sequence, so the steps agree bitwise."""
    dev = "cuda"
    h = _lib.galore_hparams(lr=0.05, rank=64)
    f_shapes, b_shapes = [(256, 128), (128, 320)], [(192, 256), (256, 192)]
    runs = []
    for _ in range(2):
        pf, gf, sf = workloads.galore_inputs(f_shapes, 64, 31, device=dev)
        pb, gb, sb = workloads.galore_inputs(b_shapes, 64, 32, param_dtype=torch.bfloat16, device=dev)
        runs.append((pf + pb, gf + gb, sf + sb))
    (p1, g1, s1), (p2, g2, s2) = runs
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, p1, g1), dev)
    _lib.meo_galore_step(h, 4, p1, g1, s1, ws)
    for k in range(len(p2)):
        wk = _lib.workspace(_lib.meo_galore_workspace_size(h, [p2[k]], [g2[k]]), dev)
        _lib.meo_galore_step(h, 4, [p2[k]], [g2[k]], [s2[k]], wk)
    torch.cuda.synchronize()
    for k in range(len(p1)):
        assert torch.equal(p1[k], p2[k]), k
        for key in s1[k]:
            assert torch.equal(s1[k][key], s2[k][key]), (k, key)


def _views(shapes, dtype):
    """Views of `shapes` into one device buffer, each 256-byte aligned (the layout
    the 7B benchmark times)."""
    es = torch.empty((), dtype=dtype).element_size()
    al = 256 // es
    sizes = [int(np.prod(s)) for s in shapes]
    offs, o = [], 0
    for n in sizes:
        offs.append(o)
        o += (n + al - 1) // al * al
    buf = torch.empty(o, dtype=dtype, device="cuda")
    return [buf[a:a + n].view(sh) for a, n, sh in zip(offs, sizes, shapes)]


@pytest.mark.parametrize("param_dtype", [torch.float32, torch.bfloat16])
def test_full_llama7b_sampled(param_dtype):
    """The Llama-7B-shaped list (291 tensors, 6.74e9 parameters, 226 of them
    projected at rank 256, scale 0.25) in one call, as the benchmark runs it:
    the embedding (m >= n, D = 32000), a q projection, a gate projection (D = 11008)
    and a down projection (m < n, d = 4096 rows of G contracted) checked in full
    against the oracle with a final norm (flat AdamW). Not a refresh step: the
    projector is an input (bf16 values of a scaled Gaussian, U^T its transpose).
    The moments are those of a mid-run step, as workloads.galore_inputs seeds them:
    exp_avg ~ N(0, (g/2)^2) and exp_avg_sq in g^2 [0.5, 1.5) for gradients of scale
    g = 1e-3. (A second moment near zero would be dominated by the square of a
    projected value that cancels over d = 4096 terms, whose fp32 sum has an absolute,
    not a relative, error.)"""
    specs = workloads.llama_specs()
    shapes = [s.shape for s in specs]
    names = [s.name for s in specs]
    rank, t = 256, 5
    # lr 2e-2: updates ~1e-3, far above the fp32 rounding of the parameter (~4e-9)
    hp = dict(lr=2e-2, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, scale=0.25, rank=rank,
              update_proj_gap=200)
    gen = torch.Generator(device="cuda").manual_seed(31)
    params = _views(shapes, param_dtype)
    grads = _views(shapes, torch.bfloat16)
    states = []
    for p, g in zip(params, grads):
        p.copy_(0.02 * torch.randn(p.shape, generator=gen, device="cuda"))
        g.copy_(1e-3 * torch.randn(g.shape, generator=gen, device="cuda"))
        st = {}
        for key, shp in _lib.galore_state_shapes(p.shape, rank).items():
            if key == "exp_avg":
                st[key] = 0.5e-3 * torch.randn(shp, generator=gen, device="cuda")
            elif key == "exp_avg_sq":
                st[key] = 1e-6 * (0.5 + torch.rand(shp, generator=gen, device="cuda"))
            elif key == "projector":
                st[key] = (torch.randn(shp, generator=gen, device="cuda") / np.sqrt(shp[0])).to(torch.bfloat16)
        if "projector" in st:
            st["projector_t"] = st["projector"].t().contiguous()
        states.append(st)
    idx = [0, names.index("model.layers.0.self_attn.q_proj.weight"),
           names.index("model.layers.15.mlp.gate_proj.weight"),
           names.index("model.layers.31.mlp.down_proj.weight"), names.index("model.norm.weight")]
    x0 = {k: to64(params[k]) for k in idx}
    g0 = {k: to64(grads[k]) for k in idx}
    s0 = {k: {key: to64(v) for key, v in states[k].items() if key != "projector_t"} for k in idx}
    pt0 = {k: states[k]["projector_t"].clone() for k in idx if "projector_t" in states[k]}
    h = _lib.galore_hparams(**hp)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), "cuda")
    print(f"galore 7B step: param={param_dtype}", flush=True)
    _lib.meo_galore_step(h, t, params, grads, states, ws)
    torch.cuda.synchronize()
    bad = []
    for k in idx:
        want_x, want_s = ga.galore_step_tensor(x0[k], g0[k], s0[k], hp, t,
                                               param_bf16=param_dtype == torch.bfloat16)
        got_x = to64(params[k])
        kind = "f32" if param_dtype == torch.float32 else "rounded"
        for kd, key, a, b in [(kind, "param", got_x, want_x),
                              ("f32", "exp_avg", to64(states[k]["exp_avg"]), want_s["exp_avg"]),
                              ("f32", "exp_avg_sq", to64(states[k]["exp_avg_sq"]), want_s["exp_avg_sq"])]:
            ok, err, over, n = check_bar(kd, key, a, b, x0=x0[k], prev=s0[k]["exp_avg"],
                                         beta1=ga.galore_hparams(hp)["betas"][0], step_tol=TOL_UPDATE)
            print(f"  {names[k]} {key}: worst {err:.3g}", flush=True)
            if not ok:
                bad.append(f"{names[k]} {key}: err {err:.3g} ({over}/{n} above the bar)")
        if param_dtype == torch.float32:
            errs, _ = dx_errs(got_x, x0[k], want_x, x0[k], floor=1.0)  # as in run_case
            e = float(np.max(errs)) if errs.size else 0.0
            if e > TOL_UPDATE:
                bad.append(f"{names[k]} update: err {e:.3g}")
        if k in pt0:
            assert torch.equal(states[k]["projector_t"], pt0[k])
    assert not bad, "; ".join(bad)

# ----------------------------------------------------------------------------- projector refresh
#
# The refresh computes the leading r singular vectors by subspace iteration; it
# equals the SVD up to (sigma_{r+1} / sigma_r)^8 and fp32 rounding. The inputs are
# rank-r signals plus noise (workloads.galore_inputs with `spectrum`), whose gap
# after the r-th singular value (sigma_{r+1} / sigma_r ~ 0.04-0.06 here) is the
# structure the projection relies on. Bar for the stored bf16 projector against
# the oracle's exact basis E (fp64 SVD, canonical signs, not rounded): per element
# |U - E| <= 2^-8 |E| (nearest bf16) + 1e-4 max_j |E[j, c]| (the iteration and the
# fp32 products, ~1e-6 on these inputs; margin for the tail vectors, whose
# neighbours are 1% apart). U^T must be U transposed, bit for bit.

TOL_BASIS = 1e-4


def check_projector(u_got, g, rank):
    e = ga.galore_projector(g, rank, projector_bf16=False)
    u = u_got.to("cpu", torch.float64).numpy()
    assert u.shape == e.shape
    bound = 2.0 ** -8 * np.abs(e) + TOL_BASIS * np.max(np.abs(e), axis=0, keepdims=True)
    excess = np.abs(u - e) - bound
    worst = np.unravel_index(np.argmax(excess), e.shape)
    assert np.all(excess <= 0), f"projector off at {worst}: got {u[worst]}, want {e[worst]}"


# The last two are the Llama-7B MLP shapes at rank 256 (d = 4096); the oracle's fp64
# SVD of such a matrix takes about half a minute on the host. Their noise's largest
# singular value is about 0.04 of the 256th signal value.
REFRESH_CASES = [((512, 384), 64, (0.97, 0.005)), ((300, 600), 32, (0.95, 0.005)),
                 ((200, 96), 13, (0.9, 0.01)), ((72, 333), 24, (0.9, 0.005)),
                 ((1024, 4096), 256, (0.99, 0.002)), ((4096, 1024), 256, (0.99, 0.002)),
                 ((4096, 11008), 256, (0.99, 0.002)), ((11008, 4096), 256, (0.99, 0.002))]


@pytest.mark.parametrize("shape,rank,spec", REFRESH_CASES, ids=lambda v: str(v))
def test_refresh_matches_svd(shape, rank, spec):
    dev = "cuda"
    params, grads, states = workloads.galore_inputs([shape], rank, 11, device=dev, state="zero",
                                                    spectrum=(spec[0], spec[1], rank))
    h = _lib.galore_hparams(rank=rank)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    x0 = params[0].clone()
    print(f"galore refresh: shape={shape} rank={rank}", flush=True)
    _lib.meo_galore_refresh(h, params, grads, states, ws)
    torch.cuda.synchronize()
    check_projector(states[0]["projector"], to64(grads[0]), rank)
    assert torch.equal(states[0]["projector_t"], states[0]["projector"].T.contiguous())
    assert torch.equal(params[0], x0)
    assert not torch.any(states[0]["exp_avg"] != 0)


def test_refresh_list():
    """Both sides, a flat tensor and an empty one in one call."""
    dev = "cuda"
    shapes = [(256, 96), (1, 7), (96, 320), (50,), (0, 4), (128, 128)]
    params, grads, states = workloads.galore_inputs(shapes, 24, 12, device=dev, state="zero",
                                                    spectrum=(0.95, 0.005, 24))
    h = _lib.galore_hparams(rank=24)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print(f"galore refresh list: {shapes}", flush=True)
    _lib.meo_galore_refresh(h, params, grads, states, ws)
    torch.cuda.synchronize()
    for k in (0, 2, 5):
        check_projector(states[k]["projector"], to64(grads[k]), 24)
    # (1, 7): rank 1, the gradient row itself, normalized and signed
    g = to64(grads[1])
    np.testing.assert_allclose(to64(states[1]["projector"]), ga.galore_projector(g, 24), rtol=0, atol=2.0 ** -8)


def test_refresh_zero_gradient_is_finite():
    dev = "cuda"
    params, grads, states = workloads.galore_inputs([(128, 64)], 16, 13, device=dev, state="zero")
    grads[0].zero_()
    h = _lib.galore_hparams(rank=16)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print("galore refresh: zero gradient", flush=True)
    _lib.meo_galore_step(h, 1, params, grads, states, ws)
    torch.cuda.synchronize()
    for v in list(states[0].values()) + [params[0]]:
        assert torch.isfinite(v.float()).all()


@pytest.mark.parametrize("shape", [(384, 160), (160, 384)])
def test_due_step_end_to_end(shape):
    """A refresh step mid-run (t = 201, gap 200, seeded moments and projector): the
    refresh, then the step, against the oracle's SVD-based step. The library's
    projector may differ from the oracle's in the last bf16 bit of a few entries
    (both round values within 1e-4 of each other), which moves the rest of the step
    by up to ~1e-3 relative: every output is checked elementwise at 2e-2, floored
    at its RMS. (At t = 1 from zero moments the direction is sign(R), whose flips
    at R ~ 0 such a last-bit difference can decide, so no elementwise bar holds.)"""
    dev = "cuda"
    rank = 32
    hpo = dict(lr=0.05, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, scale=0.25, rank=rank)
    params, grads, states = workloads.galore_inputs([shape], rank, 14, device=dev, state="seeded",
                                                    spectrum=(0.95, 0.005, rank))
    x0, g0 = to64(params[0]), to64(grads[0])
    s0 = {k: to64(v) for k, v in states[0].items() if k != "projector_t"}
    h = _lib.galore_hparams(**hpo)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print(f"galore due step: shape={shape}", flush=True)
    _lib.meo_galore_step(h, 201, params, grads, states, ws)
    torch.cuda.synchronize()
    want_x, want_s = ga.galore_step_tensor(x0, g0, s0, hpo, 201)
    check_projector(states[0]["projector"], g0, rank)
    for key, a, b in (("update", to64(params[0]) - x0, want_x - x0),
                      ("exp_avg", to64(states[0]["exp_avg"]), want_s["exp_avg"]),
                      ("exp_avg_sq", to64(states[0]["exp_avg_sq"]), want_s["exp_avg_sq"])):
        e = floored_rel_err(a, b)
        assert e <= 2e-2, f"{key}: {e:.3g}"


def test_refresh_schedule():
    """update_proj_gap: t = 1 + k * gap refreshes the projector, other steps keep it."""
    dev = "cuda"
    params, grads, states = workloads.galore_inputs([(96, 64)], 8, 15, device=dev, state="seeded",
                                                    spectrum=(0.9, 0.005, 8))
    u0 = states[0]["projector"].clone()
    h = _lib.galore_hparams(rank=8, update_proj_gap=3)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print("galore schedule", flush=True)
    for t in (2, 3):
        _lib.meo_galore_step(h, t, params, grads, states, ws)
        torch.cuda.synchronize()
        assert torch.equal(states[0]["projector"], u0)
    _lib.meo_galore_step(h, 4, params, grads, states, ws)
    torch.cuda.synchronize()
    assert not torch.equal(states[0]["projector"], u0)
    check_projector(states[0]["projector"], to64(grads[0]), 8)


def test_torch_front_end():
    """GaLoreAdamW over a model's groups equals the binding called directly (bit for
    bit) on the projected weights, and torch.optim.AdamW on the others."""
    dev = "cuda"
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(96, 64), torch.nn.LayerNorm(64), torch.nn.Linear(64, 160)).to(dev)
    names = [n for n, _ in model.named_parameters()]  # 0.weight 0.bias 1.weight 1.bias 2.weight 2.bias
    twin = [p.detach().clone() for p in model.parameters()]
    opt = GaLoreAdamW(get_galore_param_groups_named(model), lr=0.02, weight_decay=0.01)
    ref = [p.detach().clone().requires_grad_(True) for p in model.parameters()]
    # torch reference for the groups without a rank: 1.weight decays, the biases do not
    torch_opt = torch.optim.AdamW([dict(params=[ref[2]], weight_decay=0.01),
                                   dict(params=[ref[1], ref[3], ref[5]], weight_decay=0.0)], lr=0.02)
    grads = []
    for t in range(1, 4):
        gs = []
        for k, p in enumerate(model.parameters()):
            g = workloads.galore_inputs([tuple(p.shape)], 8, 100 * t + k, device=dev, state="zero",
                                        spectrum=(0.9, 0.005, 8) if p.dim() == 2 else None)[1][0].float()
            p.grad = g
            gs.append(g)
        grads.append(gs)
        opt.step()
        for r, g in zip(ref, gs):
            r.grad = g.clone()
        torch_opt.step()
    # the binding directly, on copies of the two projected weights
    hp2 = _lib.galore_hparams(lr=0.02, weight_decay=0.01, rank=8)
    w2 = [twin[0], twin[4]]
    st2 = [_lib.galore_init_state(w, 8) for w in w2]
    for t in range(1, 4):
        g2 = [grads[t - 1][0].to(torch.bfloat16), grads[t - 1][4].to(torch.bfloat16)]
        ws = _lib.workspace(_lib.meo_galore_workspace_size(hp2, w2, g2), dev)
        _lib.meo_galore_step(hp2, t, w2, g2, st2, ws)
    torch.cuda.synchronize()
    ps = list(model.parameters())
    assert torch.equal(ps[0].detach(), w2[0]) and torch.equal(ps[4].detach(), w2[1])
    assert torch.equal(opt.state[ps[0]]["projector"], st2[0]["projector"])
    for k in (1, 2, 3, 5):
        e = floored_rel_err(to64(ps[k].detach()), to64(ref[k].detach()))
        assert e < 1e-5, (names[k], e)


def get_galore_param_groups_named(model):
    from memory_efficient_optimizers_amd import get_galore_param_groups
    return get_galore_param_groups(model, weight_decay=0.01, rank=8)


def test_refresh_full_rank():
    """rank >= min(m, n): the basis is the whole space, every vector still the SVD's."""
    dev = "cuda"
    params, grads, states = workloads.galore_inputs([(160, 48), (40, 120)], 256, 21, device=dev, state="zero",
                                                    spectrum=(0.93, 0.0, 256))
    h = _lib.galore_hparams(rank=256)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print("galore refresh: full rank", flush=True)
    _lib.meo_galore_refresh(h, params, grads, states, ws)
    torch.cuda.synchronize()
    for k in range(2):
        check_projector(states[k]["projector"], to64(grads[k]), 256)


def test_refresh_rank_deficient_gradient():
    """A gradient of rank 3 with r = 8: the leading 3 vectors are the SVD's; the rest
    (which the SVD leaves free) are finite and complete an orthonormal basis."""
    dev = "cuda"
    params, grads, states = workloads.galore_inputs([(200, 96)], 8, 22, device=dev, state="zero",
                                                    spectrum=(0.8, 0.0, 3))
    h = _lib.galore_hparams(rank=8)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print("galore refresh: rank-deficient gradient", flush=True)
    _lib.meo_galore_refresh(h, params, grads, states, ws)
    torch.cuda.synchronize()
    u = to64(states[0]["projector"])
    assert np.all(np.isfinite(u))
    e = ga.galore_projector(to64(grads[0]), 8, projector_bf16=False)
    bound = 2.0 ** -8 * np.abs(e[:, :3]) + TOL_BASIS * np.max(np.abs(e[:, :3]), axis=0, keepdims=True)
    assert np.all(np.abs(u[:, :3] - e[:, :3]) <= bound)
    np.testing.assert_allclose(u.T @ u, np.eye(8), atol=2e-2)  # bf16-rounded orthonormal columns


@pytest.mark.parametrize("param_dtype", [torch.float32, torch.bfloat16])
def test_refresh_every_step(param_dtype):
    """update_proj_gap = 1 over 3 steps mid-run (a refresh before each), against the
    oracle's SVD-based steps; the bar of the due step above (the projectors may
    differ in a last bf16 bit)."""
    dev = "cuda"
    rank = 16
    hpo = dict(lr=0.01, rank=rank, update_proj_gap=1, weight_decay=0.01)
    shapes = [(192, 96), (96, 256)]
    params, grads, states = workloads.galore_inputs(shapes, rank, 23, device=dev, state="seeded",
                                                    param_dtype=param_dtype, spectrum=(0.9, 0.005, rank))
    ox = [to64(p) for p in params]
    ost = [{k: to64(v) for k, v in s.items() if k != "projector_t"} for s in states]
    h = _lib.galore_hparams(**hpo)
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print(f"galore refresh every step: {param_dtype}", flush=True)
    for t in range(11, 14):  # mid-run, seeded moments (see the due-step test on t = 1)
        g = workloads.galore_inputs(shapes, rank, 30 + t, device=dev, state="zero", spectrum=(0.9, 0.005, rank))[1]
        _lib.meo_galore_step(h, t, params, g, states, ws)
        for k in range(2):
            ox[k], ost[k] = ga.galore_step_tensor(ox[k], to64(g[k]), ost[k], hpo, t,
                                                  param_bf16=param_dtype == torch.bfloat16)
    torch.cuda.synchronize()
    for k in range(2):
        check_projector(states[k]["projector"], to64(g[k]), rank)
        for key, a, b in (("param", to64(params[k]), ox[k]), ("exp_avg", to64(states[k]["exp_avg"]), ost[k]["exp_avg"])):
            e = floored_rel_err(a, b)
            assert e <= 2e-2, f"tensor {k} {key}: {e:.3g}"


@pytest.mark.parametrize("shape,rank", [((256, 128), 32), ((128, 320), 64), ((300, 136), 40), ((72, 333), 24),
                                        ((512, 384), 256)])
def test_step_reverse_std(shape, rank):
    """proj_type reverse_std: the projector on the longer side."""
    run_case([shape], rank, hp=dict(proj_type="reverse_std"))


def test_step_reverse_std_list():
    """reverse_std over a list with tensors of both sides and both shapes: the tall
    (256, 128) and (512, 384) are projected on the left, the wide (128, 320) and
    (192, 448) on the right; with every contraction length a multiple of 64 they share
    the one projection launch, which takes each tile's side from its descriptor."""
    run_case([(256, 128), (128, 320), (512, 384), (192, 448)], 64, hp=dict(proj_type="reverse_std"), seed=6)


@pytest.mark.parametrize("shape", [(384, 160), (160, 384)])
def test_refresh_reverse_std(shape):
    dev = "cuda"
    rank = 24
    params, grads, states = workloads.galore_inputs([shape], rank, 41, device=dev, state="zero",
                                                    spectrum=(0.93, 0.005, rank), proj_type="reverse_std")
    h = _lib.galore_hparams(rank=rank, proj_type="reverse_std")
    ws = _lib.workspace(_lib.meo_galore_workspace_size(h, params, grads), dev)
    print(f"galore refresh reverse_std: {shape}", flush=True)
    _lib.meo_galore_refresh(h, params, grads, states, ws)
    torch.cuda.synchronize()
    e = ga.galore_projector(to64(grads[0]), rank, projector_bf16=False, proj_type="reverse_std")
    u = to64(states[0]["projector"])
    assert u.shape == (max(shape), rank)
    bound = 2.0 ** -8 * np.abs(e) + TOL_BASIS * np.max(np.abs(e), axis=0, keepdims=True)
    assert np.all(np.abs(u - e) <= bound)
