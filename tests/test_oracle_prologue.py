"""Pins for the oracle's reference points, level start indices, sampling
locations and softmax (CPU only)."""
import numpy as np
import pytest
import scipy.special

import oracle
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.conftest import golden


def test_pyramid_counts_from_page1():
    g = golden("pyramid_76x106.json")
    lsi, S = oracle.level_start_index(g["spatial_shapes"])
    assert [h * w for h, w in g["spatial_shapes"]] == g["tokens_per_level"]
    assert lsi.tolist() == g["level_start_index"]
    assert S == g["S"]
    assert workloads.WORKLOADS["encoder"].num_value == g["S"]


def test_encoder_refs_at_unit_ratio_are_pixel_centres():
    """valid ratios all 1: every query's point on every level is its own pixel
    centre, (linspace(0.5, W-0.5, W)/W, linspace(0.5, H-0.5, H)/H)."""
    shapes = [[5, 7], [3, 4], [1, 2]]
    L = len(shapes)
    ref = oracle.reference_points_encoder(shapes, np.ones((2, L, 2)))
    start = 0
    for (H, W) in shapes:
        yy, xx = np.meshgrid(np.linspace(0.5, H - 0.5, H) / H, np.linspace(0.5, W - 0.5, W) / W,
                             indexing="ij")
        want = np.stack([xx.reshape(-1), yy.reshape(-1)], -1)        # [H*W, 2]
        for l in range(L):
            np.testing.assert_allclose(ref[:, start:start + H * W, l], np.broadcast_to(want, (2, H * W, 2)),
                                       rtol=0, atol=1e-15)
        start += H * W


def test_encoder_refs_keep_valid_relative_position():
    """The notes' identity h2/H2 = (h1/HE1) * (HE2/H2): a point keeps its
    position relative to the valid region of every level, and on its own level
    it is its own pixel centre, whatever the ratios."""
    shapes = [[6, 8], [3, 4], [2, 2]]
    L = len(shapes)
    vr = workloads.draw_level_valid_ratios(3, L, seed=1).double().numpy()
    ref = oracle.reference_points_encoder(shapes, vr)               # [B,S,L,2]
    rel = ref / vr[:, None, :, :]                                    # position / valid extent
    np.testing.assert_allclose(rel, np.broadcast_to(rel[:, :, :1], rel.shape), rtol=1e-14, atol=0)
    start = 0
    for lq, (H, W) in enumerate(shapes):
        q = np.arange(H * W)
        own_x = (q % W + 0.5) / W
        own_y = (q // W + 0.5) / H
        np.testing.assert_allclose(ref[:, start + q, lq, 0], np.broadcast_to(own_x, (3, H * W)), rtol=1e-14)
        np.testing.assert_allclose(ref[:, start + q, lq, 1], np.broadcast_to(own_y, (3, H * W)), rtol=1e-14)
        start += H * W


def test_decoder_refs_scaled_by_valid_ratio_page2():
    g = golden("decoder_valid_ratio_p2.json")
    for case in g["cases"]:
        u = np.array(case["u"]).reshape(1, 1, 2)
        vr = np.array(case["valid_ratio_xy"]).reshape(1, 1, 2).repeat(3, axis=1)
        ref = oracle.reference_points_decoder(u, vr)
        for l in range(3):
            np.testing.assert_allclose(ref[0, 0, l], case["ref_xy"], rtol=0, atol=1e-15)


def test_locations_zero_offset_is_reference_and_pixel_steps():
    shapes = [[5, 7], [3, 4]]
    rng = np.random.default_rng(0)
    ref = rng.uniform(size=(2, 3, 2, 2))
    off = np.zeros((2, 3, 4, 2, 3, 2))
    loc = oracle.sampling_locations(shapes, ref, off)
    np.testing.assert_array_equal(loc, np.broadcast_to(ref[:, :, None, :, None, :], loc.shape))
    # one pixel along x on level l moves the normalised x by exactly 1/W_l
    off[..., 0] = 1.0
    off[..., 1] = -2.0
    loc = oracle.sampling_locations(shapes, ref, off)
    for l, (H, W) in enumerate(shapes):
        np.testing.assert_allclose(loc[:, :, :, l, :, 0] - ref[:, :, None, l, None, 0], 1.0 / W, atol=1e-15)
        np.testing.assert_allclose(loc[:, :, :, l, :, 1] - ref[:, :, None, l, None, 1], -2.0 / H, atol=1e-15)


def test_softmax_matches_scipy_and_sums_to_one_over_levels_and_points():
    rng = np.random.default_rng(1)
    B, Nq, M, L, K = 2, 5, 3, 4, 4
    logits = rng.standard_normal((B, Nq, M, L * K)) * 3
    got = oracle.softmax(logits, L * K)
    np.testing.assert_allclose(got, scipy.special.softmax(logits, axis=-1), rtol=1e-14, atol=1e-16)
    # normalised jointly over all L*K samples, not per level (paper notes, "Insight 2")
    A = got.reshape(B, Nq, M, L, K)
    np.testing.assert_allclose(A.sum(axis=(3, 4)), 1.0, atol=1e-14)
    assert not np.allclose(A.sum(axis=4), 1.0)


def test_softmax_shift_invariant_and_stable():
    x = np.array([[1000.0, 1001.0, 999.0, -1e4]])
    y = oracle.softmax(x, 4)
    assert np.all(np.isfinite(y))
    np.testing.assert_allclose(y, oracle.softmax(x - 1000.0, 4), rtol=1e-15)
