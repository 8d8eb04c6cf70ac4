"""Inputs of the core op for parity tests, built from the seeded raw draws by
the ORACLE only (reference points, sampling locations and softmax in fp64,
then rounded once to fp32). The same fp32 tensors go to the HIP library and to
the oracle's core, so the core is compared on identical inputs. Nothing here
comes from the HIP path."""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import oracle
from scale_deformable_attention_msdeformattn_amd import workloads


@dataclass
class CoreInputs:
    draws: workloads.Draws
    shapes: np.ndarray              # [L,2] int64
    lsi: np.ndarray                 # [L] int64
    ref64: np.ndarray               # [B,Nq,L,2] oracle reference points
    loc64: np.ndarray               # [B,Nq,M,L,K,2] oracle locations (from ref64)
    attn64: np.ndarray              # [B,Nq,M,L,K] oracle softmax
    value: torch.Tensor             # [B,S,M,D] fp32 / bf16 (CPU)
    loc: torch.Tensor               # fp32 rounding of loc64 (CPU)
    attn: torch.Tensor              # fp32 rounding of attn64 (CPU)
    grad_output: Optional[torch.Tensor]


def build(wl, seed: int = 0, valid_ratios: Optional[torch.Tensor] = None,
          query_ref: Optional[torch.Tensor] = None) -> CoreInputs:
    """query_ref (decoder workloads only) replaces the drawn [B,Nq,2] inputs u,
    to place the queries where a test needs them."""
    d = workloads.draw(wl, seed)
    if query_ref is not None:
        assert d.query_ref is not None and query_ref.shape == d.query_ref.shape
        d.query_ref = query_ref
    w = d.workload
    shapes = d.spatial_shapes.numpy()
    lsi, S = oracle.level_start_index(shapes)
    assert S == w.num_value
    vr = d.valid_ratios if valid_ratios is None else valid_ratios
    if w.encoder:
        ref64 = oracle.reference_points_encoder(shapes, vr)
    else:
        ref64 = oracle.reference_points_decoder(d.query_ref, vr)
    loc64 = oracle.sampling_locations(shapes, ref64, d.offsets_px)
    B, Nq, M, L, K = w.batch, w.nq, w.heads, w.levels, w.points
    attn64 = oracle.softmax(d.logits, L * K).reshape(B, Nq, M, L, K)
    return CoreInputs(d, shapes, lsi, ref64, loc64, attn64, d.value,
                      torch.from_numpy(loc64).to(torch.float32), torch.from_numpy(attn64).to(torch.float32),
                      d.grad_output)


def tolerance_check(got, ref, atol_scale, name=""):
    """max |got - ref| <= atol_scale * (1 + |ref|), elementwise; returns the
    worst ratio |err| / (atol_scale*(1+|ref|))."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    bound = atol_scale * (1.0 + np.abs(ref))
    err = np.abs(got - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(err / bound)), err.shape)
        raise AssertionError(f"{name}: max err ratio {worst:.3g} at {idx}: got {got[idx]!r} ref {ref[idx]!r} "
                             f"(max abs err {err.max():.3g})")
    return worst
