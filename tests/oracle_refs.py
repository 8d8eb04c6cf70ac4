"""Independent references used only to pin the oracle (CPU, fp64).

Each one computes the same quantity as the oracle by a different route, so a
plausible slip in the oracle (a dropped term, a wrong sign or index, swapped x
and y, swapped H and W) shows up as a mismatch:

* ``tent_forward``: bilinear sampling with zero padding written as the sum over
  every pixel of V[y][x] * max(0, 1-|x-px|) * max(0, 1-|y-py|); no floor, no
  corner enumeration.
* ``grid_sample_forward``: the per-level composition through
  ``torch.nn.functional.grid_sample`` (bilinear, zeros, align_corners=False)
  that the walkthrough page's "encoder" section describes for the pure-PyTorch
  core; written from that description, in float64, differentiable, so torch
  autograd gives independent gradients.
"""
import numpy as np
import torch
import torch.nn.functional as F


def tent_forward(value, shapes, loc, attn):
    value = np.asarray(value, dtype=np.float64)
    loc = np.asarray(loc, dtype=np.float64)
    attn = np.asarray(attn, dtype=np.float64)
    B, S, M, D = value.shape
    _, Nq, _, L, K, _ = loc.shape
    out = np.zeros((B, Nq, M, D))
    start = 0
    for l in range(L):
        H, W = int(shapes[l][0]), int(shapes[l][1])
        vmap = value[:, start:start + H * W].reshape(B, H, W, M, D)
        start += H * W
        cols = np.arange(W, dtype=np.float64)
        rows = np.arange(H, dtype=np.float64)
        for b in range(B):
            for q in range(Nq):
                for m in range(M):
                    for k in range(K):
                        px = loc[b, q, m, l, k, 0] * W - 0.5
                        py = loc[b, q, m, l, k, 1] * H - 0.5
                        if not (np.isfinite(px) and np.isfinite(py)):
                            continue
                        wx = np.maximum(0.0, 1.0 - np.abs(px - cols))
                        wy = np.maximum(0.0, 1.0 - np.abs(py - rows))
                        samp = np.einsum("i,j,ijd->d", wy, wx, vmap[b, :, :, m, :])
                        out[b, q, m] += attn[b, q, m, l, k] * samp
    return out.reshape(B, Nq, M * D)


def grid_sample_forward(value, shapes, loc, attn):
    """value [B,S,M,D], loc [B,Nq,M,L,K,2], attn [B,Nq,M,L,K] -> [B,Nq,M*D] (torch fp64)."""
    B, S, M, D = value.shape
    _, Nq, _, L, K, _ = loc.shape
    out = torch.zeros(B * M, D, Nq, dtype=value.dtype)
    start = 0
    for l in range(L):
        H, W = int(shapes[l][0]), int(shapes[l][1])
        # level l as images [B*M, D, H, W]
        img = value[:, start:start + H * W].reshape(B, H, W, M, D).permute(0, 3, 4, 1, 2)
        img = img.reshape(B * M, D, H, W)
        start += H * W
        # grid in [-1, 1]: [B*M, Nq, K, 2]
        grid = (loc[:, :, :, l] * 2.0 - 1.0).permute(0, 2, 1, 3, 4).reshape(B * M, Nq, K, 2)
        samp = F.grid_sample(img, grid, mode="bilinear", padding_mode="zeros", align_corners=False)
        w = attn[:, :, :, l].permute(0, 2, 1, 3).reshape(B * M, 1, Nq, K)
        out = out + (samp * w).sum(-1)
    return out.reshape(B, M, D, Nq).permute(0, 3, 1, 2).reshape(B, Nq, M * D)


def random_case(B=2, M=2, D=3, shapes=((5, 7), (3, 4)), Nq=6, K=3, spread=0.3, seed=0):
    """Random value/loc/attn in float64 with locations spread beyond [0,1]."""
    rng = np.random.default_rng(seed)
    L = len(shapes)
    S = sum(h * w for h, w in shapes)
    value = rng.standard_normal((B, S, M, D))
    loc = rng.uniform(-spread, 1 + spread, size=(B, Nq, M, L, K, 2))
    attn = rng.uniform(0.0, 1.0, size=(B, Nq, M, L, K))
    attn /= attn.sum(axis=(3, 4), keepdims=True)
    grad = rng.standard_normal((B, Nq, M * D))
    return value, np.array(shapes, dtype=np.int64), loc, attn, grad
