"""GPU parity: the HIP library (called through its C ABI via the ctypes
binding) against the fp64 CPU oracle, element by element, on the same seeded
inputs.

Tolerances (max abs error <= tol * (1 + |ref|), elementwise):
  forward, fp32 value ........ 1e-5
  forward, bf16 value ........ 2e-2 (the oracle consumes the bf16-rounded value)
  backward (all three) ....... 1e-4
  reference points, sampling locations, softmax ... 1e-6 (a few fp32 ulps)
"""
import numpy as np
import pytest
import torch

import oracle
import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.core_inputs import build, tolerance_check

pytestmark = pytest.mark.gpu

FWD_TOL, BF16_TOL, BWD_TOL, PRO_TOL = 1e-5, 2e-2, 1e-4, 1e-6


def dev(t):
    return t.to("cuda")


def run_forward(ci, loc=None, attn=None):
    loc = ci.loc if loc is None else loc
    attn = ci.attn if attn is None else attn
    out = msda.msda_forward(dev(ci.value), ci.shapes, ci.lsi, dev(loc), dev(attn))
    torch.cuda.synchronize()
    return out.cpu()


def run_backward(ci, loc=None, attn=None, grad_value=None):
    loc = ci.loc if loc is None else loc
    attn = ci.attn if attn is None else attn
    gv, gl, ga = msda.msda_backward(dev(ci.value), ci.shapes, ci.lsi, dev(loc), dev(attn),
                                    dev(ci.grad_output), grad_value=grad_value)
    torch.cuda.synchronize()
    return gv.cpu(), gl.cpu(), ga.cpu()


def check_forward(ci, tol=FWD_TOL, loc=None, attn=None, name=""):
    loc = ci.loc if loc is None else loc
    attn = ci.attn if attn is None else attn
    out = run_forward(ci, loc, attn)
    ref = oracle.forward(ci.value, ci.shapes, ci.lsi, loc, attn)
    return tolerance_check(out, ref, tol, f"forward {name}")


def check_backward(ci, loc=None, attn=None, name="", repeats=1):
    loc = ci.loc if loc is None else loc
    attn = ci.attn if attn is None else attn
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, loc, attn, ci.grad_output)
    for r in range(repeats):
        gv, gl, ga = run_backward(ci, loc, attn)
        tolerance_check(gv, rgv, BWD_TOL, f"grad_value {name} run {r}")
        tolerance_check(gl, rgl, BWD_TOL, f"grad_loc {name} run {r}")
        tolerance_check(ga, rga, BWD_TOL, f"grad_attn {name} run {r}")


# ---------------------------------------------------------------- the workloads

@pytest.mark.parametrize("name", ["tiny", "encoder", "decoder"])
def test_forward_workloads(gpu_lib, name):
    print(f"[forward parity] {name}", flush=True)
    check_forward(build(name), name=name)


def test_forward_bf16_large_every_element(gpu_lib):
    """B=8, S=Nq=22223 bf16 value (177,784 queries, 22.8M samples), in the
    launch configuration the bench times (the kernel with the coarse levels
    staged in LDS): every output element against the oracle."""
    print("[forward parity] encoder_bf16_large (every element)", flush=True)
    ci = build("encoder_bf16_large")
    out = run_forward(ci)
    ref = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn)
    tolerance_check(out, ref, BF16_TOL, "forward bf16 large")
    # context only: with fp32 accumulation the bf16 path is far inside its bound
    assert float(np.abs(out.numpy() - ref).max()) < 1e-4


@pytest.mark.parametrize("name", ["tiny", "encoder_backward"])
def test_backward_workloads(gpu_lib, name):
    print(f"[backward parity] {name}", flush=True)
    check_backward(build(name), name=name, repeats=2)


def test_backward_bf16_large(gpu_lib):
    """The backward at the large-batch bf16 shape (B=8, S=Nq=22223): 22.8M
    samples, so the 32-bit record and row offsets run at four times the
    encoder's range; every element against the oracle."""
    wl = workloads.custom(name="bf16_large_backward", batch=8, heads=8, channels=32, points=4,
                          spatial_shapes=workloads.WORKLOADS["encoder_bf16_large"].spatial_shapes,
                          num_query=None, offset_sigma_px=2.0, value_dtype=torch.bfloat16, backward=True)
    print("[backward parity] bf16 large", flush=True)
    check_backward(build(wl), name="bf16 large")


# ------------------------------------------------- shapes: fast path and generic

GEOMS = [
    # C = 256 fast path: (M, D) in {(8,32), (4,64), (16,16)}, several (L, K)
    dict(batch=3, heads=8, channels=32, points=4, spatial_shapes=((9, 13), (5, 7), (3, 4), (1, 2)), num_query=37),
    dict(batch=2, heads=4, channels=64, points=4, spatial_shapes=((9, 13), (5, 7), (3, 4), (1, 2)), num_query=None),
    dict(batch=1, heads=16, channels=16, points=4, spatial_shapes=((9, 13), (5, 7), (3, 4), (1, 2)), num_query=21),
    dict(batch=2, heads=8, channels=32, points=4, spatial_shapes=((11, 6),), num_query=None),
    dict(batch=2, heads=8, channels=32, points=8, spatial_shapes=((9, 13), (5, 7), (3, 4), (1, 2)), num_query=5),
    dict(batch=1, heads=8, channels=32, points=4, spatial_shapes=((12, 10), (6, 5), (3, 3)), num_query=None),
    dict(batch=2, heads=8, channels=32, points=1, spatial_shapes=((9, 13), (5, 7), (3, 4), (1, 2)), num_query=7),
    # generic path
    dict(batch=2, heads=3, channels=5, points=3, spatial_shapes=((7, 9), (4, 5)), num_query=11),
    dict(batch=1, heads=8, channels=32, points=2, spatial_shapes=((9, 13), (5, 7)), num_query=None),
    dict(batch=1, heads=1, channels=1, points=1, spatial_shapes=((1, 1),), num_query=3),
    dict(batch=2, heads=2, channels=8, points=5, spatial_shapes=((6, 4), (3, 2), (2, 1), (1, 1), (1, 1)), num_query=None),
    # more compiled shapes: five levels (L*K = 20 does not divide the wave); two points
    dict(batch=2, heads=8, channels=32, points=4, spatial_shapes=((12, 10), (6, 5), (3, 3), (2, 2), (1, 1)),
         num_query=None),
    dict(batch=2, heads=8, channels=32, points=2, spatial_shapes=((9, 13), (5, 7), (3, 4), (1, 2)), num_query=23),
]


@pytest.mark.parametrize("geom", GEOMS, ids=[f"g{i}" for i in range(len(GEOMS))])
@pytest.mark.parametrize("vdtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_shapes_forward_backward(gpu_lib, geom, vdtype):
    wl = workloads.custom(name="geom", offset_sigma_px=2.5, value_dtype=vdtype, random_valid_ratios=True,
                          backward=True, **geom)
    print(f"[shape parity] {geom} {vdtype}", flush=True)
    ci = build(wl, seed=3)
    check_forward(ci, tol=FWD_TOL if vdtype == torch.float32 else BF16_TOL, name=str(geom))
    check_backward(ci, name=str(geom))


@pytest.mark.parametrize("geom", [GEOMS[11], GEOMS[12]], ids=["m8l5k4", "m8l4k2"])
def test_compiled_shapes_take_the_fast_path(gpu_lib, geom):
    """The added compiled shapes run the per-query forward and the tiled
    backward (not the generic kernels) and match the oracle."""
    print(f"[shape parity] compiled shape {geom}", flush=True)
    wl = workloads.custom(name="geom", offset_sigma_px=2.5, random_valid_ratios=True, backward=True, **geom)
    ci = build(wl, seed=7)
    value, loc, attn, go = dev(ci.value), dev(ci.loc), dev(ci.attn), dev(ci.grad_output)
    out, ran = _kernels_run(lambda: msda.msda_forward(value, ci.shapes, ci.lsi, loc, attn))
    assert ran == {"forward_c256_kernel"}, ran
    tolerance_check(out.cpu(), oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn), FWD_TOL, "forward")
    (gv, gl, ga), ran = _kernels_run(lambda: msda.msda_backward(value, ci.shapes, ci.lsi, loc, attn, go))
    assert "backward_c256_kernel" in ran and not any("generic" in k for k in ran), ran
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    tolerance_check(gv.cpu(), rgv, BWD_TOL, "grad_value")
    tolerance_check(gl.cpu(), rgl, BWD_TOL, "grad_loc")
    tolerance_check(ga.cpu(), rga, BWD_TOL, "grad_attn")


def _kernels_run(fn):
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    res = fn()
    torch.cuda.synchronize()
    msda.msda_timing_enable(False)
    ran = set(msda.msda_timing_read())
    msda.msda_timing_reset()
    return res, ran


@pytest.mark.parametrize("geom,aligned,fwd,bwd", [
    (GEOMS[10], True, "forward_generic4_kernel", "backward_generic4_kernel"),      # D = 8
    (GEOMS[10], False, "forward_generic_kernel", "backward_generic_kernel"),       # value 4 bytes off
    (dict(GEOMS[10], channels=12), True, "forward_generic4_kernel", "backward_generic_kernel"),  # D/4 = 3
    (GEOMS[7], True, "forward_generic_kernel", "backward_generic_kernel"),         # D = 5
], ids=["d8", "d8_misaligned", "d12", "d5"])
def test_generic_kernel_choice(gpu_lib, geom, aligned, fwd, bwd):
    """Shapes without compiled kernels: four channels per thread when D is a
    multiple of 4 and the operands are 16-byte aligned (in the backward also
    D/4 a power of two, a head's lanes adding their sums by lane exchange),
    else one channel (forward) or one head (backward) per thread; each matches
    the oracle."""
    print(f"[shape parity] generic kernel choice {geom} aligned={aligned}", flush=True)
    wl = workloads.custom(name="geom", offset_sigma_px=2.5, random_valid_ratios=True, backward=True, **geom)
    ci = build(wl, seed=5)
    value = dev(ci.value)
    if not aligned:
        # the same values 4 bytes past a 16-byte boundary
        buf = torch.zeros(ci.value.numel() + 1, dtype=ci.value.dtype, device="cuda")
        value = buf[1:].view(ci.value.shape)
        value.copy_(dev(ci.value))
        assert value.data_ptr() % 16 == 4
    loc, attn, go = dev(ci.loc), dev(ci.attn), dev(ci.grad_output)
    out, ran = _kernels_run(lambda: msda.msda_forward(value, ci.shapes, ci.lsi, loc, attn))
    assert ran == {fwd}, ran
    tolerance_check(out.cpu(), oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn), FWD_TOL,
                    "forward generic")
    (gv, gl, ga), ran = _kernels_run(lambda: msda.msda_backward(value, ci.shapes, ci.lsi, loc, attn, go))
    assert bwd in ran, ran
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    tolerance_check(gv.cpu(), rgv, BWD_TOL, "grad_value generic")
    tolerance_check(gl.cpu(), rgl, BWD_TOL, "grad_loc generic")
    tolerance_check(ga.cpu(), rga, BWD_TOL, "grad_attn generic")


# ------------------------------------------------------------------ edge cases

def _edge_case():
    wl = workloads.custom(name="edge", batch=2, heads=8, channels=32, points=4,
                          spatial_shapes=((8, 8), (4, 4), (2, 2), (1, 1)), num_query=24,
                          offset_sigma_px=1.0, backward=True)
    return build(wl, seed=5)


def test_all_samples_outside_map(gpu_lib):
    ci = _edge_case()
    for v in (5.0, -3.0, 1e6):
        loc = torch.full_like(ci.loc, v)
        out = run_forward(ci, loc=loc)
        assert torch.count_nonzero(out) == 0, v
        gv, gl, ga = run_backward(ci, loc=loc)
        assert torch.count_nonzero(gv) == 0 and torch.count_nonzero(gl) == 0 and torch.count_nonzero(ga) == 0


def test_samples_on_the_border(gpu_lib):
    """Locations on and around the map border (pixel coordinate -1, 0, W-1, W
    and just inside/outside): zero padding and the right-derivative convention
    at the kink, as the oracle has them."""
    ci = _edge_case()
    for v in (-1.0 / 16, 0.0, 1.0 / 16, 1.0 - 1.0 / 16, 1.0, 1.0 + 1.0 / 16, 1e-7, 1.0 - 1e-7):
        loc = torch.full_like(ci.loc, v)
        loc[..., 1] = torch.linspace(-0.1, 1.1, loc[..., 1].numel()).reshape(loc[..., 1].shape)
        check_forward(ci, loc=loc, name=f"border {v}")
        check_backward(ci, loc=loc, name=f"border {v}")


def test_non_finite_and_huge_locations(gpu_lib):
    ci = _edge_case()
    loc = ci.loc.clone()
    flat = loc.view(-1)
    n = flat.numel()
    specials = torch.tensor([float("nan"), float("inf"), -float("inf"), 1e30, -1e30, 3.0e9, -2.5e9])
    idx = torch.arange(0, n, 7)
    flat[idx] = specials[torch.arange(idx.numel()) % specials.numel()]
    check_forward(ci, loc=loc, name="non-finite")
    check_backward(ci, loc=loc, name="non-finite")


def test_pixel_centres_and_integer_coordinates(gpu_lib):
    """Samples exactly on pixel centres (integer pixel coordinates, the kink of
    bilinear sampling): forward is an exact gather and grad_loc takes the
    cell to the right, as the oracle does."""
    ci = _edge_case()
    shapes = ci.shapes
    g = torch.Generator().manual_seed(1)
    loc = ci.loc.clone()
    for l, (H, W) in enumerate(shapes.tolist()):
        xi = torch.randint(-1, W + 1, loc[:, :, :, l, :, 0].shape, generator=g).float()
        yi = torch.randint(-1, H + 1, loc[:, :, :, l, :, 1].shape, generator=g).float()
        loc[:, :, :, l, :, 0] = (xi + 0.5) / W   # exact in fp32 for these W
        loc[:, :, :, l, :, 1] = (yi + 0.5) / H
    check_forward(ci, loc=loc, name="pixel centres")
    check_backward(ci, loc=loc, name="pixel centres")


def test_backward_accumulate_flag(gpu_lib):
    ci = _edge_case()
    base = torch.linspace(-1, 1, ci.value.numel()).reshape(ci.value.shape)
    gv, _, _ = run_backward(ci, grad_value=dev(base.clone()))
    gv0, _, _ = run_backward(ci)
    np.testing.assert_allclose(gv.numpy(), (base + gv0).numpy(), rtol=0, atol=1e-5)


def test_empty_batch_and_queries(gpu_lib):
    shapes = [[4, 4], [2, 2]]
    v = torch.randn(2, 20, 8, 32, device="cuda")
    loc = torch.rand(2, 0, 8, 2, 4, 2, device="cuda")
    a = torch.rand(2, 0, 8, 2, 4, device="cuda")
    out = msda.msda_forward(v, shapes, [0, 16], loc, a)
    assert out.shape == (2, 0, 256)
    gv, gl, ga = msda.msda_backward(v, shapes, [0, 16], loc, a, torch.zeros(2, 0, 256, device="cuda"))
    torch.cuda.synchronize()
    assert gv.shape == v.shape and torch.count_nonzero(gv) == 0


# ----------------------------------------------- reference points, locations, softmax

@pytest.mark.parametrize("name", ["tiny", "encoder", "encoder_bf16_large"])
def test_reference_points_encoder(gpu_lib, name):
    d = workloads.draw(name)
    ref = msda.msda_reference_points(d.spatial_shapes, valid_ratios=dev(d.valid_ratios))
    torch.cuda.synchronize()
    want = oracle.reference_points_encoder(d.spatial_shapes, d.valid_ratios)
    tolerance_check(ref.cpu(), want, PRO_TOL, f"reference points {name}")


def test_reference_points_encoder_per_level_ratios_and_defaults(gpu_lib):
    shapes = [[9, 13], [5, 7], [3, 4], [1, 2]]
    vr = workloads.draw_level_valid_ratios(3, 4, seed=2)
    ref = msda.msda_reference_points(shapes, valid_ratios=dev(vr))
    tolerance_check(ref.cpu(), oracle.reference_points_encoder(shapes, vr), PRO_TOL, "per-level ratios")
    ref1 = msda.msda_reference_points(shapes, batch=2)
    tolerance_check(ref1.cpu(), oracle.reference_points_encoder(shapes, np.ones((2, 4, 2))), PRO_TOL, "no ratios")


def test_reference_points_decoder(gpu_lib):
    d = workloads.draw("decoder")
    ref = msda.msda_reference_points(d.spatial_shapes, valid_ratios=dev(d.valid_ratios), query_ref=dev(d.query_ref))
    want = oracle.reference_points_decoder(d.query_ref, d.valid_ratios)
    tolerance_check(ref.cpu(), want, PRO_TOL, "decoder reference points")


@pytest.mark.parametrize("name", ["tiny", "encoder", "decoder"])
def test_sampling_locations(gpu_lib, name):
    ci = build(name)
    ref32 = torch.from_numpy(ci.ref64).to(torch.float32)
    loc = msda.msda_sampling_locations(ci.shapes, dev(ref32), dev(ci.draws.offsets_px))
    want = oracle.sampling_locations(ci.shapes, ref32, ci.draws.offsets_px)
    tolerance_check(loc.cpu(), want, PRO_TOL, f"locations {name}")


@pytest.mark.parametrize("name", ["tiny", "encoder"])
def test_softmax(gpu_lib, name):
    d = workloads.draw(name)
    w = d.workload
    A = msda.msda_attention_softmax(d.spatial_shapes, dev(d.logits), w.points)
    want = oracle.softmax(d.logits, w.levels * w.points).reshape(A.shape)
    tolerance_check(A.cpu(), want, PRO_TOL, f"softmax {name}")
    big = d.logits * 40.0
    A = msda.msda_attention_softmax(d.spatial_shapes, dev(big), w.points)
    tolerance_check(A.cpu(), oracle.softmax(big, w.levels * w.points).reshape(A.shape), PRO_TOL, "softmax x40")


@pytest.mark.parametrize("name", ["tiny", "decoder"])
def test_whole_path_end_to_end(gpu_lib, name):
    """Reference points -> locations -> softmax -> core, all on the GPU from the
    raw draws, against the oracle's fp64 chain. The bound adds to the core's
    1e-5 the effect of the fp32 rounding of the locations (at most 2^-21 in
    normalised units, a few ulps of the reference point and of the sum):
    |d out / d loc| <= sum_{l,k} A * (W_l + H_l) * 2 max|V| per head."""
    ci = build(name)
    d = ci.draws
    w = d.workload
    vr = dev(d.valid_ratios)
    if w.encoder:
        ref = msda.msda_reference_points(d.spatial_shapes, valid_ratios=vr)
    else:
        ref = msda.msda_reference_points(d.spatial_shapes, valid_ratios=vr, query_ref=dev(d.query_ref))
    out = msda.ms_deform_attn(dev(d.value), d.spatial_shapes, ref, dev(d.offsets_px), dev(d.logits), w.points)
    torch.cuda.synchronize()
    want = oracle.forward(d.value, ci.shapes, ci.lsi, ci.loc64, ci.attn64)
    B, Nq, M, L, K = ci.attn64.shape
    span = (ci.shapes[:, 0] + ci.shapes[:, 1]).astype(np.float64)            # H_l + W_l
    vmax = float(d.value.abs().max())
    slope = (ci.attn64 * span[None, None, None, :, None]).sum(axis=(3, 4)) * 2 * vmax   # [B,Nq,M]
    bound = FWD_TOL * (1 + np.abs(want)) + 2.0 ** -21 * np.repeat(slope, w.channels, axis=-1).reshape(want.shape)
    err = np.abs(out.cpu().numpy() - want)
    assert np.all(err <= bound), float((err / bound).max())


def test_autograd_function(gpu_lib):
    ci = _edge_case()
    v = dev(ci.value).requires_grad_(True)
    loc = dev(ci.loc).requires_grad_(True)
    a = dev(ci.attn).requires_grad_(True)
    out = msda.MSDeformAttnFunction.apply(v, ci.shapes, ci.lsi, loc, a)
    out.backward(dev(ci.grad_output))
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    tolerance_check(v.grad.cpu(), rgv, BWD_TOL, "autograd grad_value")
    tolerance_check(loc.grad.cpu(), rgl, BWD_TOL, "autograd grad_loc")
    tolerance_check(a.grad.cpu(), rga, BWD_TOL, "autograd grad_attn")
