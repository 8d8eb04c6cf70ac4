"""The per-kernel timing aid on the GPU: event pairs around every launch of
the library, none while a stream is being captured, and results unchanged."""
import pytest
import torch

import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import workloads

pytestmark = pytest.mark.gpu


def test_timing_counts_each_kernel_launch_and_skips_capture(gpu_lib):
    d = workloads.draw("encoder", 0)
    w = d.workload
    shapes = d.spatial_shapes
    lsi, _ = msda.level_start_index_host(shapes)
    value = d.value.cuda()
    loc = msda.msda_sampling_locations(shapes, msda.msda_reference_points(shapes, valid_ratios=d.valid_ratios.cuda()),
                                       d.offsets_px.cuda())
    A = msda.msda_attention_softmax(shapes, d.logits.cuda(), w.points)
    G = torch.randn(w.batch, w.nq, w.heads * w.channels, device="cuda")
    ref_out = msda.msda_forward(value, shapes, lsi, loc, A)
    ref_gv = msda.msda_backward(value, shapes, lsi, loc, A, G)[0]
    torch.cuda.synchronize()

    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    try:
        for _ in range(3):
            out = msda.msda_forward(value, shapes, lsi, loc, A)
            gv = msda.msda_backward(value, shapes, lsi, loc, A, G)[0]
        # launches on a capturing stream are not timed (and still work)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            msda.msda_forward(value, shapes, lsi, loc, A)
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            msda.msda_forward(value, shapes, lsi, loc, A)
        torch.cuda.synchronize()
    finally:
        msda.msda_timing_enable(False)
    t = msda.msda_timing_read()
    msda.msda_timing_reset()
    assert torch.equal(out, ref_out)
    assert torch.allclose(gv, ref_gv, rtol=0, atol=1e-4)
    # 3 timed forwards + 1 on the side stream (not capturing); the captured one is not timed
    # (this shape takes the forward with the coarse levels staged in LDS)
    assert t["forward_staged_kernel"][1] == 4
    assert "forward_c256_kernel" not in t
    # (and the backward the per-head path with its own binning and main kernel)
    assert "bin_count_kernel" not in t and "backward_c256_kernel" not in t
    for name in ("bin_count_head_kernel", "backward_head_kernel", "tile_accum_kernel"):
        ms, n = t[name]
        assert n == 3 and ms > 0.0, (name, t[name])
    assert msda.msda_timing_read() == {}
