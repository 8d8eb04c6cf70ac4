"""Pins for the oracle's backward (CPU only).

The pages train the op end to end through autograd and print no backward
formula, so the backward is read as the exact derivative of the forward. It is
pinned by: the adjoint identities (the forward is linear in value and in the
weights), central finite differences of the oracle's own forward away from the
bilinear kinks, and torch autograd through an independent fp64 grid_sample
composition.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.oracle_refs import grid_sample_forward, random_case

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

GEOMS = [
    dict(B=1, M=1, D=2, shapes=((4, 5),), Nq=5, K=2),
    dict(B=2, M=2, D=3, shapes=((5, 7), (3, 4)), Nq=6, K=3),
    dict(B=1, M=3, D=4, shapes=((6, 8), (3, 4), (2, 2)), Nq=4, K=2),
]


def _lsi(shapes):
    return oracle.level_start_index(shapes)[0]


@pytest.mark.parametrize("geom", GEOMS)
def test_adjoint_identities(geom):
    value, shapes, loc, attn, G = random_case(seed=21, **geom)
    lsi = _lsi(shapes)
    out = oracle.forward(value, shapes, lsi, loc, attn)
    gv, gl, ga = oracle.backward(value, shapes, lsi, loc, attn, G)
    lhs = float((G * out).sum())
    assert lhs == pytest.approx(float((gv * value).sum()), abs=1e-11)
    assert lhs == pytest.approx(float((ga * attn).sum()), abs=1e-11)


def _kink_distance(loc, shapes):
    """Distance in pixels from each coordinate to the nearest integer pixel
    coordinate (where bilinear sampling has a kink)."""
    L = len(shapes)
    d = np.full(loc.shape, np.inf)
    for l in range(L):
        H, W = shapes[l]
        x = loc[:, :, :, l, :, 0] * W - 0.5
        y = loc[:, :, :, l, :, 1] * H - 0.5
        d[:, :, :, l, :, 0] = np.abs(x - np.round(x))
        d[:, :, :, l, :, 1] = np.abs(y - np.round(y))
    return d


@pytest.mark.parametrize("geom", GEOMS)
def test_grad_loc_central_differences(geom):
    value, shapes, loc, attn, G = random_case(seed=22, **geom)
    lsi = _lsi(shapes)
    _, gl, _ = oracle.backward(value, shapes, lsi, loc, attn, G)
    h = 1e-7
    kink = _kink_distance(loc, shapes)
    checked = 0
    it = np.nditer(loc, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        l = idx[3]
        scale = shapes[l][1] if idx[5] == 0 else shapes[l][0]
        if kink[idx] < 10 * h * scale:
            continue
        lp, lm = loc.copy(), loc.copy()
        lp[idx] += h
        lm[idx] -= h
        fp = (G * oracle.forward(value, shapes, lsi, lp, attn)).sum()
        fm = (G * oracle.forward(value, shapes, lsi, lm, attn)).sum()
        fd = (fp - fm) / (2 * h)
        assert gl[idx] == pytest.approx(fd, rel=1e-6, abs=1e-6), idx
        checked += 1
    assert checked > 0.9 * loc.size


@pytest.mark.parametrize("geom", GEOMS)
def test_grad_attn_and_value_finite_differences(geom):
    value, shapes, loc, attn, G = random_case(seed=23, **geom)
    lsi = _lsi(shapes)
    gv, _, ga = oracle.backward(value, shapes, lsi, loc, attn, G)
    f = lambda v, a: (G * oracle.forward(v, shapes, lsi, loc, a)).sum()
    rng = np.random.default_rng(0)
    for _ in range(10):
        idx = tuple(rng.integers(0, n) for n in attn.shape)
        e = np.zeros_like(attn)
        e[idx] = 1.0
        # linear in attn: a unit step is exact
        assert ga[idx] == pytest.approx(f(value, attn + e) - f(value, attn), abs=1e-11)
        vidx = tuple(rng.integers(0, n) for n in value.shape)
        ev = np.zeros_like(value)
        ev[vidx] = 1.0
        assert gv[vidx] == pytest.approx(f(value + ev, attn) - f(value, attn), abs=1e-11)


@pytest.mark.parametrize("seed", [24, 25])
def test_backward_matches_grid_sample_autograd(seed):
    value, shapes, loc, attn, G = random_case(B=2, M=2, D=3, shapes=((7, 9), (4, 5), (2, 3)),
                                              Nq=9, K=3, seed=seed)
    # keep away from the kinks, where the one-sided derivatives may differ
    kink = _kink_distance(loc, shapes)
    loc = np.where(kink < 1e-6, loc + 1e-4, loc)
    lsi = _lsi(shapes)
    gv, gl, ga = oracle.backward(value, shapes, lsi, loc, attn, G)
    tv = torch.from_numpy(value).requires_grad_(True)
    tl = torch.from_numpy(loc).requires_grad_(True)
    ta = torch.from_numpy(attn).requires_grad_(True)
    out = grid_sample_forward(tv, shapes, tl, ta)
    out.backward(torch.from_numpy(G))
    np.testing.assert_allclose(gv, tv.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(ga, ta.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(gl, tl.grad.numpy(), rtol=1e-9, atol=1e-9)


def test_grad_loc_right_derivative_at_integer_pixel():
    """At an integer pixel coordinate the oracle takes the cell to the right:
    d/dx at x=0 on a 1-row map [a, b] is (b - a) * W (times A and G)."""
    value = np.array([2.0, 7.0, -1.0]).reshape(1, 3, 1, 1)       # H=1, W=3
    loc = np.array([0.5 / 3, 0.5]).reshape(1, 1, 1, 1, 1, 2)       # x = 0 exactly, y = 0
    attn = np.ones((1, 1, 1, 1, 1))
    G = np.ones((1, 1, 1))
    _, gl, ga = oracle.backward(value, [[1, 3]], [0], loc, attn, G)
    assert ga[0, 0, 0, 0, 0] == 2.0
    assert gl[0, 0, 0, 0, 0, 0] == pytest.approx((7.0 - 2.0) * 3)


def test_non_finite_location_has_zero_gradients():
    value, shapes, loc, attn, G = random_case(seed=26)
    loc[0, 0, 0, 0, 0, 0] = np.nan
    loc[0, 1, 0, 0, 0, 1] = -np.inf
    _, gl, ga = oracle.backward(value, shapes, _lsi(shapes), loc, attn, G)
    assert gl[0, 0, 0, 0, 0].tolist() == [0.0, 0.0] and ga[0, 0, 0, 0, 0] == 0.0
    assert gl[0, 1, 0, 0, 0].tolist() == [0.0, 0.0] and ga[0, 1, 0, 0, 0] == 0.0
