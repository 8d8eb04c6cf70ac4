"""GPU parity of the backward's internal paths that the named workloads do not
all reach, each on sizes the planner is checked (host side) to send down that
path, against the fp64 oracle at the backward tolerance 1e-4 * (1 + |ref|):

  - sorted tiles whose records overflow one LDS chunk (a hotspot: every query
    samples around one point, so one tile gets many chunks of records);
  - tiles too small to sort (about 80 samples per pixel), one workgroup each;
  - the same with the records split over two workgroups whose partial sums
    meet in float atomics (about 94 samples per pixel), with the split
    levels zeroed first, and with the accumulate flag (no zeroing);
  - dense levels split over queries, with the accumulate flag;
  - only the last run of adjacent dense levels summed from the samples;
  - three dense levels numbered across two pixel parts, beside the per-head
    main kernel;
  - sparse levels (a decoder's few queries on large maps): tiles with a few
    records or none, with the accumulate flag.
"""
import numpy as np
import pytest
import torch

import oracle
import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import _binding as B, workloads
from tests.core_inputs import build, tolerance_check

pytestmark = pytest.mark.gpu

BWD_TOL = 1e-4


def _plan(ci):
    """The planner's per-level paths; asserts the sizes take the tiled fast
    path at all (it needs a workspace; the generic path needs none)."""
    w = ci.draws.workload
    sh = B.Shape(ci.shapes, w.batch, w.heads, w.channels, w.points, w.nq)
    assert B.msda_backward_workspace_size(sh) > 0
    return B.msda_backward_plan(sh)


def _run(ci, grad_value=None):
    gv, gl, ga = msda.msda_backward(ci.value.cuda(), ci.shapes, ci.lsi, ci.loc.cuda(), ci.attn.cuda(),
                                    ci.grad_output.cuda(), grad_value=grad_value)
    torch.cuda.synchronize()
    return gv.cpu(), gl.cpu(), ga.cpu()


def _check(ci, name, accumulate_too=True):
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    gv, gl, ga = _run(ci)
    tolerance_check(gv, rgv, BWD_TOL, f"grad_value {name}")
    tolerance_check(gl, rgl, BWD_TOL, f"grad_loc {name}")
    tolerance_check(ga, rga, BWD_TOL, f"grad_attn {name}")
    if accumulate_too:
        base = torch.linspace(-1.0, 1.0, ci.value.numel(), dtype=torch.float32).reshape(ci.value.shape)
        gva, _, _ = _run(ci, grad_value=base.cuda())
        tolerance_check(gva, base.numpy().astype(np.float64) + rgv, BWD_TOL, f"grad_value accumulated {name}")


def _decoder(name, shapes, nq, sigma, seed, query_ref=None, batch=1):
    wl = workloads.custom(name=name, batch=batch, heads=8, channels=32, points=4, spatial_shapes=shapes,
                          num_query=nq, offset_sigma_px=sigma, backward=True)
    return build(wl, seed=seed, query_ref=query_ref)


def test_hotspot_tile_spans_many_chunks(gpu_lib):
    print("[backward paths] hotspot", flush=True)
    nq = 3000
    g = torch.Generator().manual_seed(11)
    u = (0.5 + 0.002 * torch.randn(1, nq, 2, generator=g)).to(torch.float32)
    ci = _decoder("hotspot", ((40, 40),), nq, 0.5, seed=5, query_ref=u)
    assert _plan(ci) == {"dense": [], "direct": [], "split": []}  # sorted tiles
    # nearly every sample of a head lands within a few pixels of the centre:
    # the centre tile holds many times the 1024 records of one LDS chunk
    x = ci.loc[..., 0, :, 0].numpy() * 40 - 0.5
    assert np.mean(np.abs(x - 19.5) < 3) > 0.95
    _check(ci, "hotspot")


def test_small_tiles_one_workgroup(gpu_lib):
    print("[backward paths] direct tiles", flush=True)
    ci = _decoder("direct", ((46, 46),), 42320, 2.0, seed=6)
    assert _plan(ci) == {"dense": [], "direct": [0], "split": []}
    _check(ci, "direct")


def test_small_tiles_split_over_workgroups(gpu_lib):
    print("[backward paths] direct split tiles", flush=True)
    ci = _decoder("split", ((46, 46),), 50000, 2.0, seed=7)
    assert _plan(ci) == {"dense": [], "direct": [0], "split": [0]}
    _check(ci, "split")


def test_dense_levels_split_over_queries(gpu_lib):
    print("[backward paths] dense split", flush=True)
    # 16x16 and 8x8 levels with 4000 queries: over 24 samples per pixel, a
    # few thousand samples per head, so each level is dense and split over
    # queries; a 48x48 level stays tiled
    ci = _decoder("dense", ((48, 48), (16, 16), (8, 8)), 4000, 2.0, seed=8, batch=2)
    plan = _plan(ci)
    assert plan["dense"] == [1, 2], plan
    _check(ci, "dense")


def test_dense_levels_last_run_only(gpu_lib):
    print("[backward paths] dense: last run of levels", flush=True)
    # levels 0 and 2 both have hundreds of samples per pixel, but only the
    # last run of adjacent dense levels is summed from the samples (the dense
    # samples of a query must be adjacent in memory): level 0 is tiled
    ci = _decoder("dense_last", ((4, 4), (40, 40), (6, 6)), 3000, 1.5, seed=9, batch=2)
    plan = _plan(ci)
    assert plan["dense"] == [2], plan
    _check(ci, "dense last run")


def test_dense_levels_over_several_parts(gpu_lib):
    print("[backward paths] dense: three levels over two pixel parts", flush=True)
    # levels 1-3 are dense (896 pixels numbered across them: two pixel parts of
    # at most 640), level 0 is tiled; 8 heads, 4 levels, 4 points and 12000
    # queries take the per-head main kernel with levels 2-3 staged in LDS
    ci = _decoder("dense_parts", ((64, 64), (24, 24), (16, 16), (8, 8)), 12000, 2.0, seed=10, batch=2)
    plan = _plan(ci)
    assert plan["dense"] == [1, 2, 3], plan
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    _run(ci)
    msda.msda_timing_enable(False)
    ran = set(msda.msda_timing_read())
    msda.msda_timing_reset()
    assert {"backward_head_kernel", "dense_accum_kernel", "dense_reduce_kernel", "tile_accum_kernel"} <= ran, ran
    _check(ci, "dense parts")


def test_sparse_levels(gpu_lib):
    print("[backward paths] sparse levels", flush=True)
    # 300 queries on a 100x150 level: under 0.1 samples per pixel, about 3
    # records per 32-pixel tile and some tiles without any
    ci = _decoder("sparse", ((100, 150), (50, 75), (25, 38), (13, 19)), 300, 2.0, seed=12, batch=2)
    assert _plan(ci) == {"dense": [], "direct": [], "split": []}
    _check(ci, "sparse")
