"""The backward (and the one-launch prologue) under HIP graph capture. On the fast path its dense levels run
on a stream of the library's own, forked from and joined back into the
caller's stream by events; a graph captured from the caller's stream must
take that branch in, and every replay must match the eager call. Replays are
interleaved with eager work and synchronisation (a replay is checked against
the eager result each time, not only the first).

grad_loc and grad_attn are summed in a fixed order and must be equal bit for
bit. grad_value sums each pixel's contributions in an order set by LDS atomics
racing between waves, so its last bits may differ from run to run: it is
compared within 1e-5 * (1 + |x|), a tenth of the parity tolerance. (On the
coarsest level a pixel sums about 1600 terms; reordering them moves the
result by up to about 2e-6 here.)"""
import pytest
import torch

import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import workloads

pytestmark = pytest.mark.gpu


def _inputs():
    d = workloads.draw("encoder_backward", 0)
    w = d.workload
    shapes = d.spatial_shapes
    lsi, _ = msda.level_start_index_host(shapes)
    ref = msda.msda_reference_points(shapes, valid_ratios=d.valid_ratios.cuda())
    loc = msda.msda_sampling_locations(shapes, ref, d.offsets_px.cuda())
    A = msda.msda_attention_softmax(shapes, d.logits.cuda(), w.points)
    return d, w, shapes, lsi, ref, loc, A, d.value.cuda(), d.grad_output.cuda()


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on a side stream, as torch recommends before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    return graph, out


def test_backward_graph_replays_equal_eager(gpu_lib):
    d, w, shapes, lsi, ref, loc, A, value, G = _inputs()
    eager = [t.clone() for t in msda.msda_backward(value, shapes, lsi, loc, A, G)]
    torch.cuda.synchronize()
    graph, out = _capture(lambda: msda.msda_backward(value, shapes, lsi, loc, A, G))
    for i in range(3):
        for t in out:
            t.fill_(float("nan"))  # a replay that skipped a kernel would leave NaNs
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("grad_value", "grad_loc", "grad_attn"), out, eager):
            if name == "grad_value":
                assert torch.allclose(a, b, rtol=1e-5, atol=1e-5), (i, name)
            else:
                assert torch.equal(a, b), (i, name)
        # eager work between the replays, on the same stream
        msda.msda_forward(value, shapes, lsi, loc, A)
        torch.cuda.synchronize()


def test_fused_backward_graph_replays_equal_eager(gpu_lib):
    d, w, shapes, lsi, ref, loc, A, value, G = _inputs()
    off = d.offsets_px.cuda()
    logits = d.logits.cuda().reshape(w.batch, w.nq, w.heads, w.levels * w.points)
    _, loc_f, A_f = msda.msda_forward_fused(value, shapes, lsi, ref, off, logits)
    eager = [t.clone() for t in msda.msda_backward_fused(value, shapes, lsi, loc_f, A_f, G)]
    torch.cuda.synchronize()
    graph, out = _capture(lambda: msda.msda_backward_fused(value, shapes, lsi, loc_f, A_f, G))
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(out, eager)):
            if k == 0:  # grad_value
                assert torch.allclose(a, b, rtol=1e-5, atol=1e-5), (i, k)
            else:
                assert torch.equal(a, b), (i, k)
        msda.msda_backward(value, shapes, lsi, loc, A, G)
        torch.cuda.synchronize()


def test_backward_on_two_streams_in_turn(gpu_lib):
    """Calls on different caller streams share the library's stream and its
    events; each call's results must still be complete when its own stream
    is synchronised."""
    d, w, shapes, lsi, ref, loc, A, value, G = _inputs()
    want = msda.msda_backward(value, shapes, lsi, loc, A, G)[0].clone()
    G2 = (2.0 * G).contiguous()
    want2 = msda.msda_backward(value, shapes, lsi, loc, A, G2)[0].clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        r1 = msda.msda_backward(value, shapes, lsi, loc, A, G)[0]
    with torch.cuda.stream(s2):
        r2 = msda.msda_backward(value, shapes, lsi, loc, A, G2)[0]
    s1.synchronize()
    assert torch.allclose(r1, want, rtol=1e-5, atol=1e-5)
    s2.synchronize()
    assert torch.allclose(r2, want2, rtol=1e-5, atol=1e-5)


def test_prologue_graph_replays_equal_eager(gpu_lib):
    """The step's first call, captured: every replay writes the same bits as
    the eager call (reference points, locations and weights have one writer
    per element and a fixed order of operations)."""
    d = workloads.draw("encoder_backward", 0)
    shapes = d.spatial_shapes
    vr, off, logits = d.valid_ratios.cuda(), d.offsets_px.cuda(), d.logits.cuda()
    eager = [t.clone() for t in msda.msda_prologue(shapes, off, logits, valid_ratios=vr)]
    torch.cuda.synchronize()
    graph, out = _capture(lambda: msda.msda_prologue(shapes, off, logits, valid_ratios=vr))
    for i in range(3):
        for t in out:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("ref", "loc", "weights"), out, eager):
            assert torch.equal(a, b), (i, name)
        msda.msda_attention_softmax(shapes, logits, d.workload.points)  # eager work between the replays
        torch.cuda.synchronize()
