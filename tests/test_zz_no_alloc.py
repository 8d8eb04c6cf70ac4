"""msda_backward_noalloc (the backward for callers that cannot allocate: its
scratch is the library's own device array) against msda_backward, called
through the C ABI on buffers allocated beforehand, on two calls in a row with
the second one smaller; every gradient within the backward's parity bound
1e-4 * (1 + |ref|) of the workspace entry point's, and grad_sampling_locations
/ grad_attention_weights (summed in a fixed order) bit for bit."""
import ctypes

import pytest
import torch

import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import _binding as B
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.core_inputs import build, tolerance_check

pytestmark = pytest.mark.gpu


def _noalloc(ci, accumulate_into=None):
    value = ci.value.cuda()
    loc, attn, go = ci.loc.cuda(), ci.attn.cuda(), ci.grad_output.cuda()
    Bq, Nq, M, L, K, _ = loc.shape
    S = value.shape[1]
    sh = B.Shape(ci.shapes, Bq, M, value.shape[3], K, Nq, ci.lsi)
    sh.c.num_value = S
    if accumulate_into is None:
        gv = torch.full((Bq, S, M, value.shape[3]), float("nan"), device="cuda")
        flags = 0
    else:
        gv = accumulate_into.clone()
        flags = B.MSDA_BWD_ACCUMULATE
    gl = torch.full_like(loc, float("nan"))
    ga = torch.full_like(attn, float("nan"))
    vt = B.MSDA_BF16 if value.dtype == torch.bfloat16 else B.MSDA_F32
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    torch.cuda.synchronize()
    st = B.raw_call("msda_backward_noalloc", sh.ptr, p(value), vt, p(loc), p(attn), p(go), p(gv), p(gl), p(ga),
                    flags, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == B.MSDA_OK, B.load().msda_last_error().decode()
    torch.cuda.synchronize()
    return gv.cpu(), gl.cpu(), ga.cpu()


def _with_workspace(ci, accumulate_into=None):
    gv = None if accumulate_into is None else accumulate_into.clone()
    out = msda.msda_backward(ci.value.cuda(), ci.shapes, ci.lsi, ci.loc.cuda(), ci.attn.cuda(),
                             ci.grad_output.cuda(), grad_value=gv)
    torch.cuda.synchronize()
    return tuple(t.cpu() for t in out)


def _compare(got, want, name):
    for g, w, what in zip(got, want, ("grad_value", "grad_loc", "grad_attn")):
        tolerance_check(g, w.double(), 1e-4, f"{what} {name}")
    assert torch.equal(got[1], want[1]), f"grad_loc {name} not bit-identical"
    assert torch.equal(got[2], want[2]), f"grad_attn {name} not bit-identical"


def test_noalloc_matches_backward_twice_second_smaller(gpu_lib):
    big = build("encoder_backward")  # the encoder step's backward: 135 MiB of scratch
    small = build(workloads.custom(name="small", batch=1, heads=8, channels=32, points=4,
                                   spatial_shapes=((23, 31), (12, 16), (6, 8), (3, 4)), num_query=None,
                                   offset_sigma_px=2.0, random_valid_ratios=True), seed=7)
    for ci, name in ((big, "encoder"), (small, "smaller pyramid after it")):
        print(f"[no-alloc] {name}", flush=True)
        _compare(_noalloc(ci), _with_workspace(ci), name)


def test_noalloc_accumulate_and_generic_path(gpu_lib):
    ci = build(workloads.custom(name="acc", batch=2, heads=8, channels=32, points=4,
                                spatial_shapes=((17, 21), (9, 11), (5, 6), (3, 3)), num_query=None,
                                offset_sigma_px=2.5), seed=3)
    base = torch.randn(tuple(ci.value.shape), generator=torch.Generator().manual_seed(1)).cuda()
    print("[no-alloc] accumulate", flush=True)
    _compare(_noalloc(ci, base), _with_workspace(ci, base), "accumulate")
    gen = build(workloads.custom(name="generic", batch=2, heads=3, channels=5, points=3,
                                 spatial_shapes=((7, 9), (4, 5)), num_query=11, offset_sigma_px=2.0), seed=5)
    print("[no-alloc] generic path", flush=True)
    got, want = _noalloc(gen), _with_workspace(gen)
    for g, w, what in zip(got, want, ("grad_value", "grad_loc", "grad_attn")):
        tolerance_check(g, w.double(), 1e-4, f"{what} generic")
