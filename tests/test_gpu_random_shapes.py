"""GPU parity on seeded random shapes of the 256-channel fast path: map sizes,
level counts, query counts and offset spreads drawn from a fixed seed, so
that tile edges, narrow edge tiles, levels that turn dense or stay sparse,
and small maps that many samples leave, all come up. Every case is checked
against the oracle at the stated tolerances, forward and backward; the
planner's choice per level is printed with the case."""
import numpy as np
import pytest
import torch

import oracle
import scale_deformable_attention_msdeformattn_amd as msda
from scale_deformable_attention_msdeformattn_amd import _binding as B, workloads
from tests.core_inputs import build, tolerance_check

pytestmark = pytest.mark.gpu

# (M, L, K) combinations the fast path is compiled for
COMBOS = [(8, 4, 4), (4, 4, 4), (16, 4, 4), (8, 1, 4), (8, 4, 8), (8, 3, 4), (8, 4, 1), (8, 5, 4), (8, 4, 2)]


def _case(i):
    rng = np.random.default_rng(1000 + i)
    M, L, K = COMBOS[i % len(COMBOS)]
    h0, w0 = int(rng.integers(3, 40)), int(rng.integers(3, 40))
    shapes = [(max(1, h0 >> l), max(1, w0 >> l)) for l in range(L)]
    encoder = bool(rng.integers(0, 2))
    nq = None if encoder else int(rng.integers(1, 3000))
    return dict(batch=int(rng.integers(1, 3)), heads=M, channels=256 // M, points=K,
                spatial_shapes=tuple(shapes), num_query=nq, offset_sigma_px=float(rng.choice([0.5, 2.0, 6.0])))


@pytest.mark.parametrize("i", range(18))
def test_random_shape(gpu_lib, i):
    geom = _case(i)
    wl = workloads.custom(name=f"random{i}", backward=True, random_valid_ratios=True, **geom)
    ci = build(wl, seed=i)
    w = ci.draws.workload
    sh = B.Shape(ci.shapes, w.batch, w.heads, w.channels, w.points, w.nq)
    print(f"[random shape {i}] {geom} plan {B.msda_backward_plan(sh)} "
          f"workspace {B.msda_backward_workspace_size(sh)}", flush=True)
    v, loc, A, G = ci.value.cuda(), ci.loc.cuda(), ci.attn.cuda(), ci.grad_output.cuda()
    out = msda.msda_forward(v, ci.shapes, ci.lsi, loc, A)
    gv, gl, ga = msda.msda_backward(v, ci.shapes, ci.lsi, loc, A, G)
    torch.cuda.synchronize()
    tolerance_check(out.cpu(), oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn), 1e-5, f"forward {i}")
    rgv, rgl, rga = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    tolerance_check(gv.cpu(), rgv, 1e-4, f"grad_value {i}")
    tolerance_check(gl.cpu(), rgl, 1e-4, f"grad_loc {i}")
    tolerance_check(ga.cpu(), rga, 1e-4, f"grad_attn {i}")
