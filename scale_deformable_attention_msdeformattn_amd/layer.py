"""A full MSDeformAttn layer and a Deformable-DETR encoder stack around the
HIP core, as a workload that shows the core's share of a real layer.

The dense parts (the value, offset, weight and output projections, the FFN and
the layer norms) are plain library GEMMs and elementwise ops through torch
(hipBLASLt / rocBLAS on this GPU); the sampling core, with the location
formation and the L*K softmax fused into it, is the fused op of libmsda.

Layer structure and initialisation follow the MSDeformAttn module source and
its parameter reset on the walkthrough page ("encoder" section): offsets bias
initialised to a ring of K growing steps per head, direction theta_m =
2 pi m / M scaled so that its larger component is 1; attention weights zero;
value and output projections Xavier-uniform. The encoder layer (paper notes,
"Engineering details"; walkthrough page, "encoder") is attention + residual +
layer norm, then a d -> 4d -> d ReLU FFN + residual + layer norm.
"""
import math

import torch
from torch import nn

from .autograd import MSDeformAttnFusedFunction


class MSDeformAttnLayer(nn.Module):
    def __init__(self, d_model=256, n_levels=4, n_heads=8, n_points=4):
        super().__init__()
        if d_model % n_heads:
            raise ValueError("d_model must be a multiple of n_heads")
        self.d_model, self.n_levels, self.n_heads, self.n_points = d_model, n_levels, n_heads, n_points
        self.sampling_offsets = nn.Linear(d_model, n_heads * n_levels * n_points * 2)
        self.attention_weights = nn.Linear(d_model, n_heads * n_levels * n_points)
        self.value_proj = nn.Linear(d_model, d_model)
        self.output_proj = nn.Linear(d_model, d_model)
        self.reset_parameters()

    def reset_parameters(self):
        M, L, K = self.n_heads, self.n_levels, self.n_points
        nn.init.zeros_(self.sampling_offsets.weight)
        theta = torch.arange(M, dtype=torch.float32) * (2.0 * math.pi / M)
        ring = torch.stack([theta.cos(), theta.sin()], dim=-1)
        ring = ring / ring.abs().max(dim=-1, keepdim=True).values          # larger component = 1
        steps = torch.arange(1, K + 1, dtype=torch.float32).view(1, 1, K, 1)
        bias = ring.view(M, 1, 1, 2).expand(M, L, K, 2) * steps             # point k at k+1 ring steps
        with torch.no_grad():
            self.sampling_offsets.bias.copy_(bias.reshape(-1))
        nn.init.zeros_(self.attention_weights.weight)
        nn.init.zeros_(self.attention_weights.bias)
        nn.init.xavier_uniform_(self.value_proj.weight)
        nn.init.xavier_uniform_(self.output_proj.weight)

    def forward(self, query, reference_points, input_flatten, spatial_shapes, level_start_index,
                padding_mask=None):
        """query [B,Nq,d], reference_points [B,Nq,L,2] (or boxes [B,Nq,L,4]),
        input_flatten [B,S,d], padding_mask [B,S] (True = padding) or None."""
        B, Nq, _ = query.shape
        S = input_flatten.shape[1]
        M, L, K = self.n_heads, self.n_levels, self.n_points
        # the padded positions of the value are filled with zeros inside the
        # core (the mask goes to the fused op instead of a masked_fill pass)
        value = self.value_proj(input_flatten).view(B, S, M, self.d_model // M)
        offsets = self.sampling_offsets(query).view(B, Nq, M, L, K, 2)
        logits = self.attention_weights(query).view(B, Nq, M, L * K)
        out = MSDeformAttnFusedFunction.apply(value, spatial_shapes, level_start_index, reference_points,
                                              offsets, logits, padding_mask)
        return self.output_proj(out)


class EncoderLayer(nn.Module):
    def __init__(self, d_model=256, d_ffn=1024, n_levels=4, n_heads=8, n_points=4):
        super().__init__()
        self.self_attn = MSDeformAttnLayer(d_model, n_levels, n_heads, n_points)
        self.norm1 = nn.LayerNorm(d_model)
        self.linear1 = nn.Linear(d_model, d_ffn)
        self.linear2 = nn.Linear(d_ffn, d_model)
        self.norm2 = nn.LayerNorm(d_model)

    def forward(self, src, pos, reference_points, spatial_shapes, level_start_index, padding_mask=None):
        q = src + pos
        src = self.norm1(src + self.self_attn(q, reference_points, src, spatial_shapes, level_start_index,
                                              padding_mask))
        return self.norm2(src + self.linear2(torch.relu(self.linear1(src))))


class Encoder(nn.Module):
    """n_layers encoder layers sharing the reference points of every pixel."""

    def __init__(self, n_layers=6, **kw):
        super().__init__()
        self.layers = nn.ModuleList(EncoderLayer(**kw) for _ in range(n_layers))

    def forward(self, src, pos, reference_points, spatial_shapes, level_start_index, padding_mask=None):
        for layer in self.layers:
            src = layer(src, pos, reference_points, spatial_shapes, level_start_index, padding_mask)
        return src
