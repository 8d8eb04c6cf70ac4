"""GPU parity of msda_prologue: reference points, sampling locations and the
L*K softmax in one call. Its three outputs must be the same bits as
msda_reference_points, msda_sampling_locations and msda_attention_softmax
called in turn, and within 1e-6 * (1 + |ref|) of the fp64 oracle. Covered:
the named workloads; shapes it takes in one kernel launch (K in {2, 4, 8} and
L*K in {4, 8, 16, 32}; one query, ragged counts); and shapes it hands to the
three kernels in turn (L*K = 12, odd K, an offsets view that is 8- but not
16-byte aligned), with the kernels that ran checked by name.
"""
import pytest
import torch

import oracle
import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import _binding as B, workloads
from tests.core_inputs import build, tolerance_check

pytestmark = pytest.mark.gpu

PRO_TOL = 1e-6
ONE_LAUNCH = {"prologue_kernel"}


def _separate(d, vr, u, off, logits):
    w = d.workload
    ref = msda.msda_reference_points(d.spatial_shapes, valid_ratios=vr, query_ref=u)
    loc = msda.msda_sampling_locations(d.spatial_shapes, ref, off)
    A = msda.msda_attention_softmax(d.spatial_shapes, logits, w.points)
    return ref, loc, A


def _kernels(fn):
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        msda.msda_timing_enable(False)
    ran = set(msda.msda_timing_read())
    msda.msda_timing_reset()
    return out, ran


def _check(ci, name, one_launch, misalign=False):
    print(f"[prologue] {name}", flush=True)
    d = ci.draws
    w = d.workload
    vr = d.valid_ratios.cuda()
    u = None if w.encoder else d.query_ref.cuda()
    off = d.offsets_px.cuda()
    if misalign:
        # the same offsets two floats into a larger buffer: 8-byte aligned only
        buf = torch.empty(off.numel() + 2, dtype=torch.float32, device="cuda")
        buf[2:] = off.reshape(-1)
        off = buf[2:].view(off.shape)
        assert off.data_ptr() % 16 == 8
    logits = d.logits.cuda()
    (ref, loc, A), ran = _kernels(lambda: msda.msda_prologue(d.spatial_shapes, off, logits, valid_ratios=vr,
                                                             query_ref=u))
    if one_launch:
        assert ran == ONE_LAUNCH, ran
    else:
        assert "prologue_kernel" not in ran and "reference_points_kernel" in ran, ran
    ref0, loc0, A0 = _separate(d, vr, u, off, logits)
    torch.cuda.synchronize()
    assert torch.equal(ref, ref0), f"reference points {name}"
    assert torch.equal(loc, loc0), f"locations {name}"
    assert torch.equal(A, A0), f"weights {name}"
    tolerance_check(ref.cpu(), ci.ref64, PRO_TOL, f"reference points {name}")
    tolerance_check(loc.cpu(), ci.loc64, PRO_TOL, f"locations {name}")
    tolerance_check(A.cpu(), ci.attn64, PRO_TOL, f"weights {name}")


@pytest.mark.parametrize("name", ["tiny", "encoder", "decoder"])
def test_prologue_workloads(gpu_lib, name):
    _check(build(name), name, one_launch=True)


ONE = [
    # (name, batch, heads, points, shapes, num_query or None for the encoder)
    ("enc_L1K4", 3, 4, 4, ((7, 9),), None),
    ("enc_L2K8", 2, 2, 8, ((11, 13), (5, 7)), None),
    ("enc_L4K2", 1, 8, 2, ((13, 17), (7, 9), (4, 5), (2, 3)), None),
    ("dec_L4K8", 2, 8, 8, ((20, 30), (10, 15), (5, 8), (3, 4)), 37),
    ("dec_L2K2_one_query", 1, 3, 2, ((9, 9), (4, 4)), 1),
    ("dec_L1K8", 2, 1, 8, ((6, 5),), 301),
]

TURN = [
    ("dec_L3K4_n12", 2, 8, 4, ((12, 10), (6, 5), (3, 3)), 45),
    ("enc_L3K3", 2, 2, 3, ((9, 7), (5, 4), (2, 2)), None),
]


@pytest.mark.parametrize("case", ONE, ids=[c[0] for c in ONE])
def test_prologue_one_launch(gpu_lib, case):
    name, batch, heads, points, shapes, nq = case
    wl = workloads.custom(name=name, batch=batch, heads=heads, channels=4, points=points, spatial_shapes=shapes,
                          num_query=nq, random_valid_ratios=True, backward=False)
    _check(build(wl, seed=21), name, one_launch=True)


@pytest.mark.parametrize("case", TURN, ids=[c[0] for c in TURN])
def test_prologue_in_turn(gpu_lib, case):
    name, batch, heads, points, shapes, nq = case
    wl = workloads.custom(name=name, batch=batch, heads=heads, channels=4, points=points, spatial_shapes=shapes,
                          num_query=nq, random_valid_ratios=True, backward=False)
    _check(build(wl, seed=22), name, one_launch=False)


def test_prologue_unaligned_offsets_in_turn(gpu_lib):
    _check(build("tiny", seed=3), "tiny, offsets 8-byte aligned", one_launch=False, misalign=True)


def test_prologue_weights_alias_logits(gpu_lib):
    """weights_out may be the logits buffer (softmax in place), through the C ABI."""
    print("[prologue] in-place weights", flush=True)
    ci = build("tiny", seed=4)
    d = ci.draws
    w = d.workload
    off = d.offsets_px.cuda()
    x = d.logits.cuda().contiguous()
    ref = torch.empty(w.batch, w.nq, w.levels, 2, dtype=torch.float32, device="cuda")
    loc = torch.empty_like(off)
    sh = B._shape(d.spatial_shapes, w.batch, w.heads, 1, w.points, w.nq)
    st = B.load().msda_prologue(sh.ptr, B._p(d.valid_ratios.cuda()), None, B._p(off), B._p(x), B._p(ref),
                                B._p(loc), B._p(x), B._stream(x))
    assert st == 0, st
    torch.cuda.synchronize()
    tolerance_check(x.cpu().reshape(ci.attn64.shape), ci.attn64, PRO_TOL, "in-place weights")
    tolerance_check(loc.cpu(), ci.loc64, PRO_TOL, "locations")


def test_prologue_errors(gpu_lib):
    d = workloads.draw("tiny")
    w = d.workload
    off = d.offsets_px.cuda()
    with pytest.raises(ValueError):
        msda.msda_prologue(d.spatial_shapes, off, d.logits.cuda()[..., :-1])
    # encoder reference points need Nq == S
    dec = workloads.draw("decoder")
    with pytest.raises(msda.MSDAError):
        msda.msda_prologue(dec.spatial_shapes, dec.offsets_px.cuda(), dec.logits.cuda())
    assert w.encoder
