"""The backward's binning run ahead of it (msda_backward_prepare, then the
backward with the prepared workspace): the same gradients as the backward
that bins for itself, whether the preparation ran on the same stream or on a
second stream beside the forward, under graph capture, for the fused backward,
and for sizes without a fast path (where there is nothing to prepare).

grad_loc and grad_attn are summed in a fixed order and must be equal bit for
bit; grad_value's summation order is not fixed (LDS atomics racing between
waves), so it is compared within 1e-5 * (1 + |x|), a tenth of the parity
tolerance. One case also goes against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.core_inputs import build, tolerance_check

pytestmark = pytest.mark.gpu


def _same(got, want):
    gv, gl, ga = got[:3]
    wgv, wgl, wga = want[:3]
    assert torch.allclose(gv, wgv, rtol=1e-5, atol=1e-5)
    assert torch.equal(gl, wgl)
    assert torch.equal(ga, wga)


def _encoder():
    d = workloads.draw("encoder_backward", 0)
    shapes = d.spatial_shapes
    lsi, _ = msda.level_start_index_host(shapes)
    ref = msda.msda_reference_points(shapes, valid_ratios=d.valid_ratios.cuda())
    loc = msda.msda_sampling_locations(shapes, ref, d.offsets_px.cuda())
    A = msda.msda_attention_softmax(shapes, d.logits.cuda(), d.workload.points)
    return d, shapes, lsi, ref, loc, A, d.value.cuda(), d.grad_output.cuda()


def test_prepared_backward_same_stream(gpu_lib):
    d, shapes, lsi, ref, loc, A, v, G = _encoder()
    want = msda.msda_backward(v, shapes, lsi, loc, A, G)
    ws = msda.msda_backward_prepare(v, shapes, lsi, loc)
    got = msda.msda_backward(v, shapes, lsi, loc, A, G, prepared=ws)
    torch.cuda.synchronize()
    _same(got, want)
    # the same workspace serves again for the same locations (the backward
    # only reads the binning)
    again = msda.msda_backward(v, shapes, lsi, loc, A, G, prepared=ws)
    torch.cuda.synchronize()
    _same(again, want)


def test_prepared_beside_the_forward(gpu_lib):
    d, shapes, lsi, ref, loc, A, v, G = _encoder()
    want_out = msda.msda_forward(v, shapes, lsi, loc, A)
    want = msda.msda_backward(v, shapes, lsi, loc, A, G)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for _ in range(3):
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            ws = msda.msda_backward_prepare(v, shapes, lsi, loc)
        out = msda.msda_forward(v, shapes, lsi, loc, A)
        cur.wait_stream(side)
        ws.record_stream(cur)
        got = msda.msda_backward(v, shapes, lsi, loc, A, G, prepared=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, want_out)
        _same(got, want)


def test_prepared_step_under_graph_capture(gpu_lib):
    d, shapes, lsi, ref, loc, A, v, G = _encoder()
    want = [t.clone() for t in msda.msda_backward(v, shapes, lsi, loc, A, G)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()

    def step():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            ws = msda.msda_backward_prepare(v, shapes, lsi, loc)
        msda.msda_forward(v, shapes, lsi, loc, A)
        cur.wait_stream(side)
        return msda.msda_backward(v, shapes, lsi, loc, A, G, prepared=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _same(out, want)
        msda.msda_forward(v, shapes, lsi, loc, A)  # eager work between the replays
        torch.cuda.synchronize()


def test_prepared_fused_backward(gpu_lib):
    d, shapes, lsi, ref, loc, A, v, G = _encoder()
    w = d.workload
    logits = d.logits.cuda().reshape(w.batch, w.nq, w.heads, w.levels * w.points)
    _, loc_f, A_f = msda.msda_forward_fused(v, shapes, lsi, ref, d.offsets_px.cuda(), logits)
    want = msda.msda_backward_fused(v, shapes, lsi, loc_f, A_f, G)
    ws = msda.msda_backward_prepare(v, shapes, lsi, loc_f)
    got = msda.msda_backward_fused(v, shapes, lsi, loc_f, A_f, G, prepared=ws)
    torch.cuda.synchronize()
    assert torch.allclose(got[0], want[0], rtol=1e-5, atol=1e-5)
    for a, b in zip(got[1:], want[1:]):
        assert torch.equal(a, b)


def test_prepared_against_the_oracle_and_without_fast_path(gpu_lib):
    # a small pyramid on the fast path (sparse and dense levels), against the oracle
    wl = workloads.custom(name="prep", batch=2, heads=8, channels=32, points=4,
                          spatial_shapes=((12, 16), (6, 8), (3, 4), (2, 2)), num_query=None,
                          offset_sigma_px=2.0, backward=True)
    ci = build(wl, seed=4)
    v, loc, A, G = ci.value.cuda(), ci.loc.cuda(), ci.attn.cuda(), ci.grad_output.cuda()
    ws = msda.msda_backward_prepare(v, ci.shapes, ci.lsi, loc)
    gv, gl, ga = msda.msda_backward(v, ci.shapes, ci.lsi, loc, A, G, prepared=ws)
    torch.cuda.synchronize()
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    tolerance_check(gv.cpu(), rgv, 1e-4, "grad_value prepared")
    tolerance_check(gl.cpu(), rgl, 1e-4, "grad_loc prepared")
    tolerance_check(ga.cpu(), rga, 1e-4, "grad_attn prepared")
    # sizes off the fast path (M*D != 256): the preparation does nothing and
    # the backward ignores the flag
    wl2 = workloads.custom(name="prep_generic", batch=1, heads=3, channels=5, points=3,
                           spatial_shapes=((7, 9), (4, 5)), num_query=11, backward=True)
    c2 = build(wl2, seed=2)
    v2, l2, a2, g2 = c2.value.cuda(), c2.loc.cuda(), c2.attn.cuda(), c2.grad_output.cuda()
    ws2 = msda.msda_backward_prepare(v2, c2.shapes, c2.lsi, l2)
    got = msda.msda_backward(v2, c2.shapes, c2.lsi, l2, a2, g2, prepared=ws2)
    want = msda.msda_backward(v2, c2.shapes, c2.lsi, l2, a2, g2)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        np.testing.assert_allclose(a.cpu().numpy(), b.cpu().numpy(), rtol=0, atol=1e-6)
