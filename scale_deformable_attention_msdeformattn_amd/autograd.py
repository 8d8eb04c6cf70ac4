"""torch.autograd wrapper over the HIP core (allocation and calls only).

``MSDeformAttnFunction.apply(value, spatial_shapes, level_start_index,
sampling_locations, attention_weights)`` keeps the argument order of the core
op on the walkthrough page ("encoder" section), minus its batch-chunk knob,
which these kernels do not need.
"""
import torch

from . import _binding as B


class MSDeformAttnFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, sampling_locations, attention_weights):
        out = B.msda_forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights)
        ctx.save_for_backward(value, sampling_locations, attention_weights)
        ctx.shapes = spatial_shapes
        ctx.lsi = level_start_index
        return out

    @staticmethod
    def backward(ctx, grad_output):
        value, loc, attn = ctx.saved_tensors
        gv, gl, ga = B.msda_backward(value, ctx.shapes, ctx.lsi, loc, attn, grad_output.contiguous())
        if value.dtype != torch.float32:
            gv = gv.to(value.dtype)
        return gv, None, None, gl, ga


class MSDeformAttnFusedFunction(torch.autograd.Function):
    """value, reference points (2-d points or 4-d boxes), offsets, logits and
    an optional key padding mask [B,S] (True = padded: those value rows read
    as zero) -> output, with the location formation and the L*K softmax
    inside the core; gradients for all four float tensor inputs."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                attention_logits, key_padding_mask=None):
        out, loc, attn = B.msda_forward_fused(value, spatial_shapes, level_start_index, reference_points,
                                              sampling_offsets, attention_logits, key_padding_mask)
        box = reference_points.shape[-1] == 4
        ctx.save_for_backward(value, loc, attn, reference_points if box else None, sampling_offsets if box else None,
                              key_padding_mask)
        ctx.shapes = spatial_shapes
        ctx.lsi = level_start_index
        return out

    @staticmethod
    def backward(ctx, grad_output):
        value, loc, attn, box, off, mask = ctx.saved_tensors
        gv, goff, glog, gref = B.msda_backward_fused(value, ctx.shapes, ctx.lsi, loc, attn,
                                                     grad_output.contiguous(),
                                                     reference_grad=ctx.needs_input_grad[3],
                                                     box_references=box, sampling_offsets=off,
                                                     key_padding_mask=mask)
        if value.dtype != torch.float32:
            gv = gv.to(value.dtype)
        return gv, None, None, gref, goff, glog, None


def ms_deform_attn(value, spatial_shapes, reference_points, offsets_px, logits, points):
    """Location formation + L*K softmax + core forward, all in the HIP library
    (no autograd through the first two steps)."""
    loc = B.msda_sampling_locations(spatial_shapes, reference_points, offsets_px)
    attn = B.msda_attention_softmax(spatial_shapes, logits, points)
    lsi, _ = B.level_start_index_host(spatial_shapes)
    return B.msda_forward(value, spatial_shapes, lsi, loc, attn)
