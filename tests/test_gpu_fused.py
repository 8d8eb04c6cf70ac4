"""GPU parity of the fused path (locations and the L*K softmax formed inside
the core, gradients carried back to the offsets, logits and reference points)
against the oracle's chain: sampling locations -> softmax -> core, and back.

The fused forward returns the locations and weights it formed; they are
compared with the oracle's fp64 steps (1e-6 (1+|ref|)), and the core output
with the oracle's core evaluated at exactly those fp32 locations and weights
(1e-5 (1+|ref|)). The backward is compared with the oracle's core backward at
the same inputs followed by its softmax and location backward (1e-4 (1+|ref|)
for grad_value and grad_offsets; for grad_logits and grad_ref the bound adds
the propagated core tolerance, see below)."""
import numpy as np
import pytest
import torch

import oracle
import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.core_inputs import build, tolerance_check
from tests.test_gpu_parity import GEOMS

pytestmark = pytest.mark.gpu

FWD_TOL, BF16_TOL, BWD_TOL, PRO_TOL = 1e-5, 2e-2, 1e-4, 1e-6


def dev(t):
    return torch.as_tensor(t).to("cuda")


def fused_case(ci):
    d = ci.draws
    w = d.workload
    ref32 = torch.from_numpy(ci.ref64).to(torch.float32)
    logits = d.logits.reshape(w.batch, w.nq, w.heads, w.levels * w.points)
    return ref32, d.offsets_px, logits


def box_case(ci, seed=11):
    """4-d references: the point as (cx, cy), box sizes drawn in [0.05, 0.5]."""
    ref32, off, logits = fused_case(ci)
    g = torch.Generator().manual_seed(seed)
    wh = 0.05 + 0.45 * torch.rand(ref32.shape, generator=g)
    return torch.cat([ref32, wh], dim=-1), off, logits


def check_fused(ci, vtol, name, box=False, mask=None):
    """mask: a [B,S] key padding mask for the fused pair; the oracle chain then
    fills the value with zeros at the padded rows before its core and zeroes
    its grad_value there (the module's masked_fill and its backward)."""
    w = ci.draws.workload
    ref32, off, logits = box_case(ci) if box else fused_case(ci)
    dmask = None if mask is None else dev(mask)
    value_o = ci.value if mask is None else oracle.masked_fill(ci.value, mask)
    out, loc, A = msda.msda_forward_fused(dev(ci.value), ci.shapes, ci.lsi, dev(ref32), dev(off), dev(logits),
                                          key_padding_mask=dmask)
    torch.cuda.synchronize()
    loc, A = loc.cpu(), A.cpu()
    want_loc = (oracle.sampling_locations_box(ref32, off) if box
                else oracle.sampling_locations(ci.shapes, ref32, off))
    tolerance_check(loc, want_loc, PRO_TOL, f"fused loc {name}")
    tolerance_check(A, oracle.softmax(logits, w.levels * w.points).reshape(A.shape), PRO_TOL, f"fused A {name}")
    tolerance_check(out.cpu(), oracle.forward(value_o, ci.shapes, ci.lsi, loc, A), vtol, f"fused out {name}")
    # the core is the same code as msda_forward: identical output at the same locations and weights
    plain_value = ci.value if mask is None else ci.value.masked_fill(mask[..., None, None], 0)
    plain = msda.msda_forward(dev(plain_value), ci.shapes, ci.lsi, dev(loc), dev(A))
    torch.cuda.synchronize()
    assert torch.equal(plain.cpu(), out.cpu()), f"fused and plain forward differ {name}"
    if ci.grad_output is None:
        return
    G = ci.grad_output
    gv, goff, glog, gref = msda.msda_backward_fused(dev(ci.value), ci.shapes, ci.lsi, dev(loc), dev(A), dev(G),
                                                    box_references=dev(ref32) if box else None,
                                                    sampling_offsets=dev(off) if box else None,
                                                    key_padding_mask=dmask)
    torch.cuda.synchronize()
    rgv, rgl, rga = oracle.backward(value_o, ci.shapes, ci.lsi, loc, A, G)
    if mask is not None:
        rgv = oracle.masked_fill(rgv, mask)
    if box:
        rgref, rgoff = oracle.sampling_locations_box_backward(ref32, off, rgl)
    else:
        rgref, rgoff = oracle.sampling_locations_backward(ci.shapes, rgl)
    LK = w.levels * w.points
    rglog = oracle.softmax_backward(A, rga, LK).reshape(glog.shape)
    tolerance_check(gv.cpu(), rgv, BWD_TOL, f"fused grad_value {name}")
    tolerance_check(goff.cpu(), rgoff, BWD_TOL, f"fused grad_offsets {name}")
    # grad_logit_i = A_i (ga_i - sum_j A_j ga_j): a core error e_j <= 1e-4 (1+|ga_j|)
    # reaches it as A_i (e_i + sum_j A_j e_j) <= A_i 1e-4 (2 + |ga_i| + max_j |ga_j|)
    a = A.numpy().astype(np.float64).reshape(glog.shape)
    ga = np.abs(rga).reshape(glog.shape)
    extra = BWD_TOL * a * (2.0 + ga + ga.max(axis=-1, keepdims=True))
    err = np.abs(glog.cpu().numpy() - rglog)
    assert np.all(err <= BWD_TOL * (1 + np.abs(rglog)) + extra), f"fused grad_logits {name}"
    # grad_ref sums M*K grad_loc entries (for box sizes times |offset| / (2K)),
    # each entry within 1e-4 (1+|entry|)
    e = BWD_TOL * (1 + np.abs(rgl))                                   # [B,Nq,M,L,K,2]
    span = e.sum(axis=(2, 4))                                         # [B,Nq,L,2]
    if box:
        span = np.concatenate([span, (e * np.abs(off.numpy()) * 0.5 / w.points).sum(axis=(2, 4))], axis=-1)
    err = np.abs(gref.cpu().numpy() - rgref)
    assert np.all(err <= span + BWD_TOL * (1 + np.abs(rgref))), f"fused grad_ref {name}"


@pytest.mark.parametrize("name", ["tiny", "encoder_backward", "decoder"])
def test_fused_workloads(gpu_lib, name):
    print(f"[fused] {name}", flush=True)
    check_fused(build(name), FWD_TOL, name)


@pytest.mark.parametrize("geom", GEOMS, ids=[f"g{i}" for i in range(len(GEOMS))])
def test_fused_shapes(gpu_lib, geom):
    """Fast shapes (L*K dividing 64: in-kernel fusion), the 3-level shape
    (L*K = 12: plain kernels, then the conversion kernel) and generic shapes."""
    wl = workloads.custom(name="geom", offset_sigma_px=2.5, random_valid_ratios=True, backward=True, **geom)
    print(f"[fused shape] {geom}", flush=True)
    check_fused(build(wl, seed=5), FWD_TOL, str(geom))


@pytest.mark.parametrize("name", ["tiny", "encoder_backward"])
def test_fused_box_references(gpu_lib, name):
    print(f"[fused box] {name}", flush=True)
    check_fused(build(name), FWD_TOL, name, box=True)


@pytest.mark.parametrize("geom", [GEOMS[0], GEOMS[5], GEOMS[7]], ids=["fast", "lk12", "generic"])
def test_fused_box_shapes(gpu_lib, geom):
    wl = workloads.custom(name="geom", offset_sigma_px=2.5, random_valid_ratios=True, backward=True, **geom)
    check_fused(build(wl, seed=6), FWD_TOL, str(geom), box=True)


@pytest.mark.parametrize("heads,channels,points,shapes", [
    (8, 32, 4, ((9, 13), (5, 7), (3, 4), (1, 2))),   # fast kernels
    (4, 16, 3, ((9, 13), (5, 7))),                   # generic, 4-channel loads
], ids=["fast", "generic4"])
def test_fused_bf16_value(gpu_lib, heads, channels, points, shapes):
    wl = workloads.custom(name="bf16", batch=2, heads=heads, channels=channels, points=points,
                          spatial_shapes=shapes, num_query=None,
                          value_dtype=torch.bfloat16, offset_sigma_px=2.0, random_valid_ratios=True, backward=True)
    check_fused(build(wl, seed=2), BF16_TOL, "bf16")


def test_fused_autograd(gpu_lib):
    ci = build("tiny")
    w = ci.draws.workload
    ref32, off, logits = fused_case(ci)
    v = dev(ci.value).requires_grad_(True)
    r = dev(ref32).requires_grad_(True)
    o = dev(off).requires_grad_(True)
    lg = dev(logits).requires_grad_(True)
    out = msda.MSDeformAttnFusedFunction.apply(v, ci.shapes, ci.lsi, r, o, lg)
    out.backward(dev(ci.grad_output))
    loc = oracle.sampling_locations(ci.shapes, ref32, off)
    A = oracle.softmax(logits, w.levels * w.points).reshape(w.batch, w.nq, w.heads, w.levels, w.points)
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, loc, A, ci.grad_output)
    rgref, rgoff = oracle.sampling_locations_backward(ci.shapes, rgl)
    rglog = oracle.softmax_backward(A, rga, w.levels * w.points).reshape(logits.shape)
    tolerance_check(v.grad.cpu(), rgv, BWD_TOL, "autograd fused grad_value")
    tolerance_check(o.grad.cpu(), rgoff, BWD_TOL, "autograd fused grad_offsets")
    tolerance_check(lg.grad.cpu(), rglog, 3 * BWD_TOL, "autograd fused grad_logits")
    tolerance_check(r.grad.cpu(), rgref, 2 * w.heads * w.points * BWD_TOL, "autograd fused grad_ref")


def test_fused_empty_queries(gpu_lib):
    ci = build("tiny")
    ref32, off, logits = fused_case(ci)
    out, loc, A = msda.msda_forward_fused(dev(ci.value), ci.shapes, ci.lsi, dev(ref32[:, :0]), dev(off[:, :0]),
                                          dev(logits[:, :0]))
    assert out.shape[1] == 0 and loc.shape[1] == 0 and A.shape[1] == 0
    gv, goff, glog, gref = msda.msda_backward_fused(dev(ci.value), ci.shapes, ci.lsi, loc, A,
                                                    torch.zeros(out.shape, device="cuda"))
    torch.cuda.synchronize()
    assert float(gv.abs().max()) == 0.0


MASK_CASES = {
    "encoder_backward": None,                      # staged kernels, binned backward with dense levels
    "tiny": None,                                  # generic kernels (M*D = 8; 4-channel loads)
    "generic4": dict(batch=2, heads=4, channels=16, points=3, spatial_shapes=((9, 13), (5, 7)),
                     num_query=23),                # generic 4-channel forward (no fast kernel for L=2, K=3)
    "fast": GEOMS[0],                              # per-query kernel, 37 queries
    "lk12": GEOMS[5],                              # L*K = 12: plain kernels, then the conversion kernel
    "split": dict(batch=1, heads=8, channels=32, points=4, spatial_shapes=((46, 46),),
                  num_query=50000),                # direct-mode tiles merged by float atomics
}


@pytest.mark.parametrize("case", list(MASK_CASES), ids=list(MASK_CASES))
def test_fused_key_padding_mask(gpu_lib, case):
    """The fused pair with a key padding mask shaped like an image batch's
    (the bottom and right parts of every level padded, from valid ratios
    drawn in [0.6, 0.9]) plus 5% of positions at random."""
    geom = MASK_CASES[case]
    if geom is None:
        ci = build(case)
    else:
        wl = workloads.custom(name="mask", offset_sigma_px=2.5, random_valid_ratios=True, backward=True, **geom)
        ci = build(wl, seed=8)
    B = ci.value.shape[0]
    g = torch.Generator().manual_seed(4)
    vr = 0.6 + 0.3 * torch.rand(B, len(ci.shapes), 2, generator=g)
    mask = workloads.padding_mask(ci.shapes, vr, seed=9, extra=0.05)
    assert mask.any() and not mask.all()
    print(f"[fused mask] {case}: {int(mask.sum())} of {mask.numel()} positions padded", flush=True)
    check_fused(ci, FWD_TOL, f"mask {case}", mask=mask)


def test_fused_key_padding_mask_accumulate_and_bf16(gpu_lib):
    """With MSDA_BWD_ACCUMULATE the padded rows keep what grad_value held;
    bf16 value with a mask."""
    wl = workloads.custom(name="maskacc", batch=2, heads=8, channels=32, points=4,
                          spatial_shapes=((17, 21), (9, 11), (5, 6), (3, 3)), num_query=None,
                          value_dtype=torch.bfloat16, offset_sigma_px=2.5, random_valid_ratios=True, backward=True)
    ci = build(wl, seed=12)
    mask = workloads.padding_mask(ci.shapes, ci.draws.valid_ratios * 0.8, seed=3, extra=0.05)
    check_fused(ci, BF16_TOL, "mask bf16", mask=mask)
    ref32, off, logits = fused_case(ci)
    _, loc, A = msda.msda_forward_fused(dev(ci.value), ci.shapes, ci.lsi, dev(ref32), dev(off), dev(logits),
                                        key_padding_mask=dev(mask))
    base = torch.randn(tuple(ci.value.shape), generator=torch.Generator().manual_seed(2))
    gv, _, _, _ = msda.msda_backward_fused(dev(ci.value), ci.shapes, ci.lsi, loc, A, dev(ci.grad_output),
                                           grad_value=dev(base), key_padding_mask=dev(mask))
    torch.cuda.synchronize()
    rgv, _, _ = oracle.backward(oracle.masked_fill(ci.value, mask), ci.shapes, ci.lsi, loc.cpu(), A.cpu(),
                                ci.grad_output)
    tolerance_check(gv.cpu(), base.double().numpy() + oracle.masked_fill(rgv, mask), BWD_TOL, "mask accumulate")
    assert torch.equal(gv.cpu()[mask], base[mask])
