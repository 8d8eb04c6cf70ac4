"""The 32-bit index edge: one batch of value close to the library's cap of
2^31 bytes (as fp32), on the 256-channel path.

One level of 1400 x 1470 pixels plus three small ones gives S = 2,058,336
rows of 1 KB: 2,107,736,064 bytes, 98.2% of 2^31. The kernels address value
rows with 32-bit byte offsets (row * 1024 up to 2.1e9) and mark off-map
corners with the offset 2^31, so the last rows are the ones that would break
first. Decoder-style queries are placed on the last rows and columns, in the
bottom-right corner and across the map; the forward runs both the per-query
kernel (300 queries) and the kernel with the coarse levels staged in LDS
(1200 queries). The backward at this size takes the generic path (the tiled
path's per-workgroup tile cursors cannot hold the 64K tiles of such a level:
msda_backward_plan reports no plan), so its int64 row arithmetic and the
grad_value zero fill over 2.1 GB are checked too. Every element of every
output is compared with the oracle, the forward and grad_value / grad_attn
within the usual bounds. grad_sampling_locations is the gradient with respect
to the normalised location, i.e. the pixel-coordinate gradient times W_l
(H_l): at 1470 x 1400 pixels the fp32 rounding of the four corner dot
products (32 channels each) is multiplied by a map size 14 times the encoder
workload's, so its bound adds that rounding, A * W_l * 2^-20 *
sum_c sum_d |G_d| |v_c,d| (and likewise with H_l)."""
import numpy as np
import pytest
import torch

import oracle
import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import _binding as B
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.core_inputs import build, tolerance_check

pytestmark = pytest.mark.gpu

SHAPES = ((1400, 1470), (16, 16), (8, 8), (4, 4))


def _queries(nq, seed):
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(1, nq, 2, generator=g)
    third = nq // 3
    u[0, :third, 1] = 1.0 - torch.rand(third, generator=g) * 0.003      # the last rows
    u[0, third:2 * third, 0] = 1.0 - torch.rand(third, generator=g) * 0.003  # the last columns
    u[0, :8] = torch.tensor([1.0, 1.0])                                  # the bottom-right corner
    return u


def _corner_dot_abs(ci):
    """sum over a sample's in-map corners of sum_d |G_d| |v_c,d|, [B,Nq,M,L,K]
    (the size of the terms of its corner dot products; for the bound only)."""
    v = ci.value.numpy()
    G = np.abs(ci.grad_output.numpy().astype(np.float64))
    B, Nq, M, L, K, _ = ci.loc.shape
    D = v.shape[-1]
    G = G.reshape(B, Nq, M, 1, D)
    loc = ci.loc.numpy().astype(np.float64)
    out = np.zeros((B, Nq, M, L, K))
    for l, (H, W) in enumerate(SHAPES):
        x = loc[:, :, :, l, :, 0] * W - 0.5
        y = loc[:, :, :, l, :, 1] * H - 0.5
        x0, y0 = np.floor(x), np.floor(y)
        for dy in (0, 1):
            for dx in (0, 1):
                xi, yi = x0 + dx, y0 + dy
                ok = (xi >= 0) & (xi < W) & (yi >= 0) & (yi < H)
                row = (int(ci.lsi[l]) + np.where(ok, yi, 0) * W + np.where(ok, xi, 0)).astype(np.int64)
                rows = np.abs(v[0][row[0], np.arange(M).reshape(1, M, 1)].astype(np.float64))  # [Nq,M,K,D]
                out[0, :, :, l, :] += np.where(ok[0], (rows * G[0]).sum(-1), 0.0)
    return out


def _chunked_check(got, want, tol, name, chunk=1 << 25):
    got = got.reshape(-1)
    want = want.reshape(-1)
    worst = 0.0
    for i in range(0, got.numel(), chunk):
        worst = max(worst, tolerance_check(got[i:i + chunk].numpy(), want[i:i + chunk], tol, f"{name}[{i}:]"))
    return worst


@pytest.mark.parametrize("nq", [300, 1200])
def test_value_batch_near_the_32bit_cap(gpu_lib, nq):
    S = sum(h * w for h, w in SHAPES)
    assert S * 256 * 4 > 0.95 * 2 ** 31 and S * 256 * 4 < 2 ** 31
    wl = workloads.custom(name="cap", batch=1, heads=8, channels=32, points=4, spatial_shapes=SHAPES,
                          num_query=nq, offset_sigma_px=2.0, random_valid_ratios=False)
    print(f"[index width] building inputs, S={S}, Nq={nq}", flush=True)
    ci = build(wl, seed=11, query_ref=_queries(nq, seed=11))
    sh = B.Shape(ci.shapes, 1, 8, 32, 4, nq, ci.lsi)
    assert B.msda_backward_plan(sh) == {"dense": [], "direct": [], "split": []}
    # the queries do reach the last rows of the big level
    ylast = ci.loc64[..., 0, :, 1] * SHAPES[0][0] - 0.5
    assert float(ylast.max()) > SHAPES[0][0] - 1.5
    value = ci.value.cuda()
    print("[index width] forward", flush=True)
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    out = msda.msda_forward(value, ci.shapes, ci.lsi, ci.loc.cuda(), ci.attn.cuda())
    torch.cuda.synchronize()
    msda.msda_timing_enable(False)
    ran = set(msda.msda_timing_read())
    msda.msda_timing_reset()
    assert ran == {"forward_c256_kernel" if nq < 1024 else "forward_staged_kernel"}, ran
    ref = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn)
    tolerance_check(out.cpu(), ref, 1e-5, f"forward near the cap, Nq={nq}")
    print("[index width] backward", flush=True)
    gv, gl, ga = msda.msda_backward(value, ci.shapes, ci.lsi, ci.loc.cuda(), ci.attn.cuda(), ci.grad_output.cuda())
    torch.cuda.synchronize()
    del value
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    size = np.array([[w, h] for h, w in SHAPES], dtype=np.float64)                  # [L, 2] = (W_l, H_l)
    A = ci.attn.numpy().astype(np.float64)
    extra = (A * _corner_dot_abs(ci))[..., None] * size[None, None, None, :, None, :] * 2.0 ** -20
    err = np.abs(gl.cpu().numpy().astype(np.float64) - rgl)
    bound = 1e-4 * (1 + np.abs(rgl)) + extra
    assert np.all(err <= bound), f"grad_loc near the cap: worst ratio {float((err / bound).max()):.3g}"
    tolerance_check(ga.cpu(), rga, 1e-4, "grad_attn near the cap")
    gv = gv.cpu()
    # the last rows of the big level did receive gradient
    last = gv[0, (SHAPES[0][0] - 2) * SHAPES[0][1]:SHAPES[0][0] * SHAPES[0][1]]
    assert torch.count_nonzero(last) > 0
    _chunked_check(gv, rgv, 1e-4, "grad_value near the cap")
    print("[index width] ok", flush=True)
