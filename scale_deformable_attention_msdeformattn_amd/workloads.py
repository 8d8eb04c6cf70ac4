"""Seeded synthetic workloads for the multi-scale deformable attention core.

This module only draws random numbers with fixed shapes, distributions and a
fixed draw order. It holds none of the method's arithmetic: reference points,
location formation, softmax and sampling are done by the library (on the GPU)
or by the oracle (on the CPU), each on its own.

Shapes follow the pages:
  * 76x106 / 38x53 / 19x27 / 8x13 is the four-level pyramid whose per-level
    token counts (8056 / 2014 / 513 / 104) are printed in the juhe.plus notes,
    "Key point 1: get_reference_points".
  * 100x167 / 50x84 / 25x42 / 13x21 is an 800x1333 input (short side <= 800,
    long side <= 1333, "Engineering practice / training configuration" of the
    phdsky.com paper notes) at strides 8/16/32/64, rounded up.
  * M=8 heads, K=4 points, L=4 levels, C=256 channels and 300 decoder queries
    come from the same training configuration table.
Synthetic draws stand in for COCO images: no dataset item is used.

Draw order (one ``torch.Generator`` seeded per workload):
  1. value ~ N(0, 1) [B,S,M,D] (cast to bf16 for the bf16-value workload)
  2. valid ratios ~ U[0.7, 1] per image and axis, [B,1,2] broadcast over L
     (only where the workload says so; otherwise all ones)
  3. decoder reference inputs u ~ U(0, 1)^2 [B,Nq,2] (decoder workload only)
  4. sampling offsets ~ N(0, sigma) in level pixels [B,Nq,M,L,K,2]
  5. attention logits ~ N(0, 1) [B,Nq,M,L*K]
  6. grad_output ~ N(0, 1) [B,Nq,M*D] (backward workloads only)
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import torch

PYRAMID_76x106: List[Tuple[int, int]] = [(76, 106), (38, 53), (19, 27), (8, 13)]
PYRAMID_800x1333: List[Tuple[int, int]] = [(100, 167), (50, 84), (25, 42), (13, 21)]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    channels: int              # D, channels per head
    points: int                # K
    spatial_shapes: Tuple[Tuple[int, int], ...]
    num_query: Optional[int]   # None: encoder, every pixel is a query (Nq = S)
    offset_sigma_px: float
    value_dtype: torch.dtype = torch.float32
    random_valid_ratios: bool = False
    backward: bool = False
    description: str = ""

    @property
    def levels(self) -> int:
        return len(self.spatial_shapes)

    @property
    def num_value(self) -> int:
        return sum(h * w for h, w in self.spatial_shapes)

    @property
    def encoder(self) -> bool:
        return self.num_query is None

    @property
    def nq(self) -> int:
        return self.num_value if self.num_query is None else self.num_query


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", batch=1, heads=2, channels=4, points=2,
        spatial_shapes=((8, 8), (4, 4)), num_query=None, offset_sigma_px=1.5,
        backward=True,
        description="tiny fwd+bwd fp32: B=1 M=2 D=4 L=2 {8x8,4x4} S=Nq=80 K=2"),
    "encoder": Workload(
        "encoder", batch=2, heads=8, channels=32, points=4,
        spatial_shapes=tuple(PYRAMID_76x106), num_query=None, offset_sigma_px=2.0,
        random_valid_ratios=True,
        description="encoder self-attention fwd fp32: B=2 M=8 D=32 L=4 76x106..8x13 "
                    "S=Nq=10687 K=4"),
    "decoder": Workload(
        "decoder", batch=2, heads=8, channels=32, points=4,
        spatial_shapes=tuple(PYRAMID_76x106), num_query=300, offset_sigma_px=4.0,
        random_valid_ratios=True,
        description="decoder cross-attention fwd fp32: B=2 M=8 D=32 L=4 Nq=300 K=4"),
    "encoder_bf16_large": Workload(
        "encoder_bf16_large", batch=8, heads=8, channels=32, points=4,
        spatial_shapes=tuple(PYRAMID_800x1333), num_query=None, offset_sigma_px=2.0,
        value_dtype=torch.bfloat16,
        description="large-batch encoder fwd, bf16 value: B=8 M=8 D=32 L=4 "
                    "100x167..13x21 S=Nq=22223 K=4"),
    "encoder_backward": Workload(
        "encoder_backward", batch=2, heads=8, channels=32, points=4,
        spatial_shapes=tuple(PYRAMID_76x106), num_query=None, offset_sigma_px=2.0,
        random_valid_ratios=True, backward=True,
        description="encoder bwd fp32: B=2 M=8 D=32 L=4 76x106..8x13 S=Nq=10687 K=4"),
}


def custom(name="custom", batch=1, heads=2, channels=4, points=2,
           spatial_shapes=((8, 8), (4, 4)), num_query=None, offset_sigma_px=1.5,
           value_dtype=torch.float32, random_valid_ratios=False, backward=True) -> Workload:
    """A workload of arbitrary shape with the same recipe (for tests)."""
    return Workload(name, batch, heads, channels, points, tuple(tuple(s) for s in spatial_shapes),
                    num_query, offset_sigma_px, value_dtype, random_valid_ratios, backward)


@dataclass
class Draws:
    workload: Workload
    spatial_shapes: torch.Tensor        # [L,2] int64 (H, W), host
    value: torch.Tensor                 # [B,S,M,D] fp32 or bf16
    valid_ratios: torch.Tensor          # [B,L,2] fp32, (x=width, y=height)
    offsets_px: torch.Tensor            # [B,Nq,M,L,K,2] fp32, level pixels
    logits: torch.Tensor                # [B,Nq,M,L*K] fp32
    query_ref: Optional[torch.Tensor] = None    # [B,Nq,2] decoder inputs u
    grad_output: Optional[torch.Tensor] = None  # [B,Nq,M*D]
    extra: dict = field(default_factory=dict)


def draw(wl, seed: int = 0) -> Draws:
    """Draw one workload's raw inputs on the CPU, in the fixed order above."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    B, M, D, K, L = wl.batch, wl.heads, wl.channels, wl.points, wl.levels
    S, Nq = wl.num_value, wl.nq
    value = torch.randn(B, S, M, D, generator=g, dtype=torch.float32)
    if wl.value_dtype != torch.float32:
        value = value.to(wl.value_dtype)
    if wl.random_valid_ratios:
        vr = torch.empty(B, 1, 2, dtype=torch.float32).uniform_(0.7, 1.0, generator=g)
        valid_ratios = vr.expand(B, L, 2).contiguous()
    else:
        valid_ratios = torch.ones(B, L, 2, dtype=torch.float32)
    query_ref = None
    if not wl.encoder:
        query_ref = torch.rand(B, Nq, 2, generator=g, dtype=torch.float32)
    offsets_px = torch.randn(B, Nq, M, L, K, 2, generator=g, dtype=torch.float32) * wl.offset_sigma_px
    logits = torch.randn(B, Nq, M, L * K, generator=g, dtype=torch.float32)
    grad_output = None
    if wl.backward:
        grad_output = torch.randn(B, Nq, M * D, generator=g, dtype=torch.float32)
    shapes = torch.tensor(wl.spatial_shapes, dtype=torch.int64)
    return Draws(wl, shapes, value, valid_ratios, offsets_px, logits, query_ref, grad_output)


def draw_level_valid_ratios(batch: int, levels: int, seed: int = 0) -> torch.Tensor:
    """Valid ratios that differ per level and axis, U[0.5, 1] (unit tests only)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.empty(batch, levels, 2, dtype=torch.float32).uniform_(0.5, 1.0, generator=g)


def padding_mask(spatial_shapes, valid_ratios: torch.Tensor, seed: Optional[int] = None,
                 extra: float = 0.0) -> torch.Tensor:
    """A key padding mask [B,S] (True = padded) shaped like an image batch's:
    on level l of image b the columns from ceil(vr[b,l,0] * W_l) and the rows
    from ceil(vr[b,l,1] * H_l) on are padding (the valid region is the
    top-left part, as for images padded to a common size). With `extra` > 0
    a further random fraction of positions is masked too (seeded), so that
    padded rows also sit inside the maps in tests."""
    shapes = [(int(h), int(w)) for h, w in torch.as_tensor(spatial_shapes).tolist()]
    B = valid_ratios.shape[0]
    parts = []
    for l, (H, W) in enumerate(shapes):
        vw = torch.ceil(valid_ratios[:, l, 0].double() * W).long().clamp(1, W)
        vh = torch.ceil(valid_ratios[:, l, 1].double() * H).long().clamp(1, H)
        xs = torch.arange(W).view(1, 1, W)
        ys = torch.arange(H).view(1, H, 1)
        parts.append(((xs >= vw.view(B, 1, 1)) | (ys >= vh.view(B, 1, 1))).reshape(B, H * W))
    mask = torch.cat(parts, dim=1)
    if extra > 0:
        g = torch.Generator(device="cpu")
        g.manual_seed(0 if seed is None else seed)
        mask |= torch.rand(mask.shape, generator=g) < extra
    return mask
