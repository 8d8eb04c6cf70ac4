"""Pins for the oracle's forward (CPU only).

The forward has a plain definition (the MSDeformAttn equation of the phdsky.com
paper notes, "Insight 2", with the bilinear / zero-padding / align_corners=False
sampling of the xdnf.cn walkthrough's "encoder" section), so it is pinned by
independent routes to the same number: brute-force tent sums, torch's
grid_sample, hand-worked values, and closed-form special cases.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.conftest import golden
from tests.oracle_refs import grid_sample_forward, random_case, tent_forward

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _lsi(shapes):
    return oracle.level_start_index(shapes)[0]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("geom", [
    dict(B=1, M=1, D=1, shapes=((4, 5),), Nq=7, K=2),
    dict(B=2, M=2, D=3, shapes=((5, 7), (3, 4)), Nq=6, K=3),
    dict(B=1, M=3, D=2, shapes=((6, 3), (3, 2), (1, 1)), Nq=5, K=4),
])
def test_forward_matches_tent_brute_force(seed, geom):
    value, shapes, loc, attn, _ = random_case(seed=seed, **geom)
    got = oracle.forward(value, shapes, _lsi(shapes), loc, attn)
    want = tent_forward(value, shapes, loc, attn)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 5])
def test_forward_matches_grid_sample_composition(seed):
    value, shapes, loc, attn, _ = random_case(B=2, M=3, D=4, shapes=((9, 11), (5, 6), (2, 3)),
                                              Nq=13, K=4, seed=seed)
    got = oracle.forward(value, shapes, _lsi(shapes), loc, attn)
    want = grid_sample_forward(torch.from_numpy(value), shapes, torch.from_numpy(loc),
                               torch.from_numpy(attn)).numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_bilinear_hand_worked_values():
    g = golden("bilinear_2x2.json")
    vmap = np.array(g["map"], dtype=np.float64)           # [H=2, W=2]
    value = vmap.reshape(1, 4, 1, 1)
    shapes = np.array([[2, 2]])
    for case in g["cases"]:
        loc = np.array(case["loc_xy"], dtype=np.float64).reshape(1, 1, 1, 1, 1, 2)
        attn = np.ones((1, 1, 1, 1, 1))
        out = oracle.forward(value, shapes, _lsi(shapes), loc, attn)
        assert out[0, 0, 0] == pytest.approx(case["expected"], abs=1e-15), case


def test_pixel_centre_is_exact_gather():
    """K=1, L=1, A=1, location at a pixel centre (j+.5)/W, (i+.5)/H: exactly V[i, j]."""
    rng = np.random.default_rng(3)
    H, W, M, D = 6, 9, 2, 5
    value = rng.standard_normal((1, H * W, M, D))
    ii, jj = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    loc = np.zeros((1, H * W, M, 1, 1, 2))
    loc[0, :, :, 0, 0, 0] = ((jj.reshape(-1) + 0.5) / W)[:, None]
    loc[0, :, :, 0, 0, 1] = ((ii.reshape(-1) + 0.5) / H)[:, None]
    attn = np.ones((1, H * W, M, 1, 1))
    out = oracle.forward(value, np.array([[H, W]]), [0], loc, attn)
    np.testing.assert_array_equal(out.reshape(1, H * W, M, D), value)


def test_page2_offset_example_lands_on_pixels():
    """A point at pixel (30,30) with pixel offsets (1,1),(1,2),(-2,-1) samples
    (31,31),(31,32),(28,29) (walkthrough page, "overall flow")."""
    g = golden("offset_example_p2.json")
    H, W = g["map_hw"]
    rng = np.random.default_rng(4)
    value = rng.standard_normal((1, H * W, 1, 3))
    px, py = g["point_xy"]
    ref = np.array([[[[(px + 0.5) / W, (py + 0.5) / H]]]])           # [1,1,1,2]
    offs = np.array(g["offsets_xy"], dtype=np.float64).reshape(1, 1, 1, 1, 3, 2)
    loc = oracle.sampling_locations([[H, W]], ref, offs)
    for k, (sx, sy) in enumerate(g["sampled_xy"]):
        attn = np.zeros((1, 1, 1, 1, 3))
        attn[..., k] = 1.0
        out = oracle.forward(value, [[H, W]], [0], loc, attn)
        np.testing.assert_allclose(out[0, 0], value[0, sy * W + sx, 0], rtol=0, atol=1e-12)


def test_constant_map_interior_gives_constant():
    """With every corner inside, a constant map c gives c * sum(A) (sum(A)=1
    for softmaxed weights)."""
    rng = np.random.default_rng(5)
    shapes = np.array([[7, 9], [4, 5]])
    S = 63 + 20
    B, M, D, Nq, K, L = 2, 3, 4, 11, 3, 2
    c = 1.7
    value = np.full((B, S, M, D), c)
    loc = np.empty((B, Nq, M, L, K, 2))
    for l, (H, W) in enumerate(shapes):
        # interior: x in [0, W-1], i.e. u in [0.5/W, (W-0.5)/W]
        loc[:, :, :, l, :, 0] = rng.uniform(0.5 / W, (W - 0.5) / W, size=(B, Nq, M, K))
        loc[:, :, :, l, :, 1] = rng.uniform(0.5 / H, (H - 0.5) / H, size=(B, Nq, M, K))
    logits = rng.standard_normal((B, Nq, M, L * K))
    attn = oracle.softmax(logits, L * K).reshape(B, Nq, M, L, K)
    out = oracle.forward(value, shapes, _lsi(shapes), loc, attn)
    expect = c * attn.sum(axis=(3, 4))                                 # [B,Nq,M]
    np.testing.assert_allclose(out.reshape(B, Nq, M, D), np.repeat(expect[..., None], D, -1),
                               rtol=0, atol=1e-13)


def test_zero_padding_and_non_finite():
    value, shapes, loc, attn, _ = random_case(seed=7)
    far = loc.copy()
    far[..., 0] = 5.0                   # x far right of every level
    np.testing.assert_array_equal(oracle.forward(value, shapes, _lsi(shapes), far, attn), 0.0)
    far[..., 0] = -3.0
    np.testing.assert_array_equal(oracle.forward(value, shapes, _lsi(shapes), far, attn), 0.0)
    bad = loc.copy()
    bad[0, 0, 0, 0, 0, 0] = np.nan
    bad[0, 1, 0, 0, 0, 1] = np.inf
    bad[0, 2, 0, 0, 0, 0] = 1e30
    clean = attn.copy()
    clean[0, 0, 0, 0, 0] = clean[0, 1, 0, 0, 0] = clean[0, 2, 0, 0, 0] = 0.0
    np.testing.assert_allclose(oracle.forward(value, shapes, _lsi(shapes), bad, attn),
                               oracle.forward(value, shapes, _lsi(shapes), loc, clean), atol=0)


def test_linearity_in_value_and_weights():
    value, shapes, loc, attn, _ = random_case(seed=8)
    v2 = np.random.default_rng(9).standard_normal(value.shape)
    a2 = np.random.default_rng(10).uniform(size=attn.shape)
    lsi = _lsi(shapes)
    f = lambda v, a: oracle.forward(v, shapes, lsi, loc, a)
    np.testing.assert_allclose(f(2 * value - 3 * v2, attn), 2 * f(value, attn) - 3 * f(v2, attn), atol=1e-12)
    np.testing.assert_allclose(f(value, attn + a2), f(value, attn) + f(value, a2), atol=1e-12)


def test_query_subset_matches_full():
    value, shapes, loc, attn, _ = random_case(seed=11)
    lsi = _lsi(shapes)
    full = oracle.forward(value, shapes, lsi, loc, attn)
    B, Nq = loc.shape[:2]
    ids = np.array([0, 3, Nq + 2, 2 * Nq - 1])
    sub = oracle.forward(value, shapes, lsi, loc, attn, query_ids=ids)
    np.testing.assert_array_equal(sub, full.reshape(B * Nq, -1)[ids])


def test_bf16_value_upcasts_exactly():
    t = torch.randn(1, 4, 1, 2).to(torch.bfloat16)
    loc = np.array([0.25, 0.25]).reshape(1, 1, 1, 1, 1, 2)
    out = oracle.forward(t, [[2, 2]], [0], loc, np.ones((1, 1, 1, 1, 1)))
    np.testing.assert_array_equal(out[0, 0], t[0, 0, 0].to(torch.float64).numpy())
