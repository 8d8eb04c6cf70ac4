"""GPU parity of the forward whose coarse levels are staged in LDS (one head
per workgroup; the C = 256 shapes with 8 heads, 4 levels and 4 points, at
least 1024 queries): each split between levels read from memory and levels
read from LDS, bf16 value, a ragged query count, samples off the map and the
fused form (point and box references), against the fp64 oracle element by
element."""
import pytest
import torch

import oracle
import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.core_inputs import build, tolerance_check

pytestmark = pytest.mark.gpu

FWD_TOL, BF16_TOL = 1e-5, 2e-2

CASES = {
    # levels 1-3 fit in LDS: one level from memory
    "split1_encoder": dict(batch=1, spatial_shapes=((40, 48), (12, 16), (6, 8), (3, 4)), num_query=None,
                           offset_sigma_px=2.0, value_dtype=torch.float32),
    # only level 3 fits: three levels from memory
    "split3_decoder": dict(batch=1, spatial_shapes=((96, 96), (48, 48), (30, 30), (20, 24)), num_query=1500,
                           offset_sigma_px=3.0, value_dtype=torch.float32),
    # levels 2-3 in LDS (the encoder pyramid's split), ragged query count, two images
    "split2_ragged": dict(batch=2, spatial_shapes=((48, 64), (30, 40), (12, 16), (6, 8)), num_query=1031,
                          offset_sigma_px=2.0, value_dtype=torch.float32),
    # most coarse samples off the map
    "far_offsets": dict(batch=1, spatial_shapes=((38, 53), (19, 27), (10, 14), (5, 7)), num_query=1100,
                        offset_sigma_px=12.0, value_dtype=torch.float32),
    "bf16_encoder": dict(batch=2, spatial_shapes=((40, 48), (20, 24), (10, 12), (5, 6)), num_query=None,
                         offset_sigma_px=2.0, value_dtype=torch.bfloat16),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_staged_forward_matches_oracle(gpu_lib, name):
    c = CASES[name]
    wl = workloads.custom(name=name, heads=8, channels=32, points=4, random_valid_ratios=True,
                          backward=False, **c)
    print(f"[staged forward] {name}", flush=True)
    ci = build(wl, seed=11)
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    try:
        out = msda.msda_forward(ci.value.cuda(), ci.shapes, ci.lsi, ci.loc.cuda(), ci.attn.cuda())
        torch.cuda.synchronize()
    finally:
        msda.msda_timing_enable(False)
    ran = msda.msda_timing_read()
    msda.msda_timing_reset()
    assert set(ran) == {"forward_staged_kernel"}, ran
    ref = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn)
    tol = FWD_TOL if c["value_dtype"] == torch.float32 else BF16_TOL
    tolerance_check(out.cpu(), ref, tol, f"staged forward {name}")


def test_few_queries_keep_the_per_query_kernel(gpu_lib):
    # below 1024 queries the staging does not pay: the per-query kernel runs
    wl = workloads.custom(name="few", batch=1, heads=8, channels=32, points=4,
                          spatial_shapes=((38, 53), (19, 27), (10, 14), (5, 7)), num_query=1000,
                          offset_sigma_px=2.0, backward=False)
    ci = build(wl, seed=12)
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    try:
        out = msda.msda_forward(ci.value.cuda(), ci.shapes, ci.lsi, ci.loc.cuda(), ci.attn.cuda())
        torch.cuda.synchronize()
    finally:
        msda.msda_timing_enable(False)
    ran = msda.msda_timing_read()
    msda.msda_timing_reset()
    assert set(ran) == {"forward_c256_kernel"}, ran
    ref = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn)
    tolerance_check(out.cpu(), ref, FWD_TOL, "per-query forward")


@pytest.mark.parametrize("box", [False, True], ids=["points", "boxes"])
def test_staged_fused_forward(gpu_lib, box):
    from tests.test_gpu_fused import check_fused
    wl = workloads.custom(name="staged_fused", batch=1, heads=8, channels=32, points=4,
                          spatial_shapes=((48, 64), (30, 40), (12, 16), (6, 8)), num_query=1200,
                          offset_sigma_px=2.0, random_valid_ratios=True, backward=True)
    print(f"[staged fused forward] box={box}", flush=True)
    ci = build(wl, seed=13)
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    try:
        check_fused(ci, FWD_TOL, f"staged fused box={box}", box=box)
    finally:
        msda.msda_timing_enable(False)
    ran = msda.msda_timing_read()
    msda.msda_timing_reset()
    assert "forward_fused_staged_kernel" in ran and "forward_fused_c256_kernel" not in ran, ran
