"""Multi-scale deformable attention (MSDeformAttn) core for AMD MI355X (gfx950).

The computation runs in the hand-written HIP kernels of ``libmsda.so`` behind
the C ABI in ``include/msda.h``; this package only marshals torch tensors into
that ABI. Entry points (same names as the C ABI):

    msda_reference_points, msda_sampling_locations, msda_attention_softmax,
    msda_prologue (the three in one launch), msda_forward, msda_backward, msda_forward_fused, msda_backward_fused,
    msda_backward_plan

and the per-kernel timing aid msda_timing_enable / msda_timing_read /
msda_timing_reset, plus ``MSDeformAttnFunction`` and ``MSDeformAttnFusedFunction``
(autograd over the plain and the fused forward/backward) and ``ms_deform_attn``
(location formation + softmax + core in three calls).
"""
from ._binding import (MSDAError, declared_symbols, level_start_index_host, load, msda_attention_softmax,
                       msda_backward, msda_backward_fused, msda_backward_plan, msda_forward,
                       msda_forward_fused, msda_prologue, msda_reference_points, msda_sampling_locations,
                       msda_timing_enable, msda_timing_read, msda_timing_reset)
from .autograd import MSDeformAttnFunction, MSDeformAttnFusedFunction, ms_deform_attn

__all__ = [
    "MSDAError", "MSDeformAttnFunction", "MSDeformAttnFusedFunction", "declared_symbols",
    "level_start_index_host", "load", "ms_deform_attn", "msda_attention_softmax", "msda_backward",
    "msda_backward_fused", "msda_backward_plan", "msda_forward", "msda_forward_fused", "msda_prologue",
    "msda_reference_points",
    "msda_sampling_locations", "msda_timing_enable", "msda_timing_read", "msda_timing_reset",
]
