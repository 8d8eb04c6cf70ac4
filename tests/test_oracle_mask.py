"""Pins for the oracle's padding-mask step (the module fills the projected
value with zeros at padded positions before the core: phdsky.com notes, "Key
code", MSDeformAttn.forward; xdnf.cn walkthrough, "encoder"), alone and
composed with the core (CPU only)."""
import numpy as np

import oracle
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.core_inputs import build


def _case(seed=3, num_query=None):
    # power-of-two maps: pixel centres (i + 0.5) / W are exact in fp32
    wl = workloads.custom(name="mask", batch=2, heads=2, channels=3, points=2,
                          spatial_shapes=((8, 8), (4, 4)), num_query=num_query, offset_sigma_px=1.5)
    return build(wl, seed=seed)


def test_mask_fill_identity_zero_idempotent_and_self_adjoint():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(2, 9, 4, 3))
    y = rng.normal(size=x.shape)
    none = np.zeros((2, 9), dtype=bool)
    every = np.ones((2, 9), dtype=bool)
    some = rng.random((2, 9)) < 0.4
    assert np.array_equal(oracle.masked_fill(x, none), x)
    assert not np.any(oracle.masked_fill(x, every))
    once = oracle.masked_fill(x, some)
    assert np.array_equal(oracle.masked_fill(once, some), once)
    # an orthogonal projection: <P x, y> = <x, P y>, and it keeps the unmasked part of the norm
    assert abs(np.vdot(once, y) - np.vdot(x, oracle.masked_fill(y, some))) < 1e-12
    assert np.count_nonzero(once) == np.count_nonzero(~some) * 12


def test_masking_rows_no_corner_touches_changes_nothing():
    ci = _case(num_query=3)
    B, S = ci.value.shape[:2]
    plain = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn)
    # the rows that some in-map corner reads: the adjoint of the forward with
    # grad_output = 1 is nonzero exactly there (up to exact cancellation)
    gv, _, _ = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn,
                               np.ones((B, ci.loc.shape[1], ci.value.shape[2] * ci.value.shape[3])))
    touched = np.abs(gv).sum(axis=(2, 3)) > 0
    untouched = ~touched
    assert untouched.any()
    masked = oracle.forward(oracle.masked_fill(ci.value, untouched), ci.shapes, ci.lsi, ci.loc, ci.attn)
    assert np.array_equal(masked, plain)


def test_masked_pixel_centre_reads_zero():
    """A sample exactly on a pixel centre reads that pixel alone: with the
    pixel masked it contributes nothing."""
    ci = _case()
    loc = ci.loc.clone()
    H, W = int(ci.shapes[0, 0]), int(ci.shapes[0, 1])
    loc[...] = -5.0                                          # every other sample off the map
    loc[0, 0, 0, 0, 0, 0] = (2 + 0.5) / W                    # pixel (row 3, column 2) of level 0
    loc[0, 0, 0, 0, 0, 1] = (3 + 0.5) / H
    mask = np.zeros(ci.value.shape[:2], dtype=bool)
    out = oracle.forward(ci.value, ci.shapes, ci.lsi, loc, ci.attn)
    a = float(ci.attn[0, 0, 0, 0, 0])
    np.testing.assert_allclose(out[0, 0, :3], a * ci.value[0, 3 * W + 2, 0].double().numpy(), rtol=1e-15)
    mask[0, 3 * W + 2] = True
    out = oracle.forward(oracle.masked_fill(ci.value, mask), ci.shapes, ci.lsi, loc, ci.attn)
    assert not np.any(out)


def test_masked_chain_gradient_by_central_differences():
    """d/d value of <G, forward(masked_fill(value))> is
    masked_fill(grad_value) of the core backward at the filled value."""
    ci = _case(seed=5)
    rng = np.random.default_rng(1)
    mask = rng.random(ci.value.shape[:2]) < 0.3
    v = ci.value.double().numpy()
    G = ci.grad_output.double().numpy()
    filled = oracle.masked_fill(v, mask)
    gv, _, _ = oracle.backward(filled, ci.shapes, ci.lsi, ci.loc, ci.attn, G)
    want = oracle.masked_fill(gv, mask)
    h = 1e-3
    for idx in [tuple(rng.integers(0, n) for n in v.shape) for _ in range(40)]:
        vp, vm = v.copy(), v.copy()
        vp[idx] += h
        vm[idx] -= h
        fp = np.vdot(G, oracle.forward(oracle.masked_fill(vp, mask), ci.shapes, ci.lsi, ci.loc, ci.attn))
        fm = np.vdot(G, oracle.forward(oracle.masked_fill(vm, mask), ci.shapes, ci.lsi, ci.loc, ci.attn))
        assert abs((fp - fm) / (2 * h) - want[idx]) < 1e-9, idx
