"""Pins for the oracle's backward of the two steps next to the core: the L*K
softmax and the location formation (CPU only). Both are pinned against
numerical derivatives of the oracle's own forward steps and against textbook
forms written independently of the oracle's code."""
import numpy as np
import pytest

import oracle


def test_softmax_backward_matches_explicit_jacobian():
    """The textbook Jacobian of softmax is diag(A) - A A^T; its transpose
    applied to grad_A must equal the oracle's grad_logits."""
    rng = np.random.default_rng(3)
    for n in (4, 16, 32):
        x = rng.normal(size=(5, n)) * 2.0
        g = rng.normal(size=(5, n))
        A = oracle.softmax(x, n)
        got = oracle.softmax_backward(A, g, n)
        for r in range(5):
            J = np.diag(A[r]) - np.outer(A[r], A[r])
            np.testing.assert_allclose(got[r], J.T @ g[r], rtol=1e-12, atol=1e-14)


def test_softmax_backward_central_differences():
    rng = np.random.default_rng(4)
    n = 16
    x = rng.normal(size=(3, n))
    g = rng.normal(size=(3, n))
    got = oracle.softmax_backward(oracle.softmax(x, n), g, n)
    h = 1e-6
    num = np.zeros_like(x)
    for r in range(3):
        for i in range(n):
            xp, xm = x.copy(), x.copy()
            xp[r, i] += h
            xm[r, i] -= h
            num[r, i] = ((oracle.softmax(xp, n) * g).sum() - (oracle.softmax(xm, n) * g).sum()) / (2 * h)
    np.testing.assert_allclose(got, num, rtol=1e-7, atol=1e-9)


def test_softmax_backward_rows_sum_to_zero_and_ignore_constant_gradients():
    """Shift invariance of softmax: every row of grad_logits sums to 0, and a
    grad_A that is constant over a row gives zero."""
    rng = np.random.default_rng(5)
    A = oracle.softmax(rng.normal(size=(4, 16)), 16)
    got = oracle.softmax_backward(A, rng.normal(size=(4, 16)), 16)
    np.testing.assert_allclose(got.sum(axis=1), 0.0, atol=1e-14)
    const = oracle.softmax_backward(A, np.full((4, 16), 2.5), 16)
    np.testing.assert_allclose(const, 0.0, atol=1e-14)


def _loc_case(seed=6):
    rng = np.random.default_rng(seed)
    shapes = [[5, 7], [3, 4]]
    B, Nq, M, L, K = 2, 3, 2, 2, 3
    ref = rng.uniform(size=(B, Nq, L, 2))
    off = rng.normal(size=(B, Nq, M, L, K, 2)) * 1.5
    gl = rng.normal(size=(B, Nq, M, L, K, 2))
    return shapes, ref, off, gl


def test_locations_backward_central_differences():
    """loc is affine in (ref, offset): central differences of <grad_loc, loc>
    give the exact gradients."""
    shapes, ref, off, gl = _loc_case()
    gref, goff = oracle.sampling_locations_backward(shapes, gl)

    def f(r, o):
        return float((oracle.sampling_locations(shapes, r, o) * gl).sum())

    h = 1e-3
    num_off = np.zeros_like(off)
    it = np.nditer(off, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        op, om = off.copy(), off.copy()
        op[i] += h
        om[i] -= h
        num_off[i] = (f(ref, op) - f(ref, om)) / (2 * h)
    np.testing.assert_allclose(goff, num_off, rtol=1e-9, atol=1e-11)
    num_ref = np.zeros_like(ref)
    it = np.nditer(ref, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        rp, rm = ref.copy(), ref.copy()
        rp[i] += h
        rm[i] -= h
        num_ref[i] = (f(rp, off) - f(rm, off)) / (2 * h)
    np.testing.assert_allclose(gref, num_ref, rtol=1e-9, atol=1e-11)


def test_locations_backward_scales_by_level_size():
    """One offset pixel is 1/W_l of the normalised x axis and 1/H_l of the y
    axis: on level (H, W) = (5, 7) a unit grad_loc gives (1/7, 1/5)."""
    shapes = [[5, 7]]
    gl = np.ones((1, 1, 1, 1, 1, 2))
    gref, goff = oracle.sampling_locations_backward(shapes, gl)
    np.testing.assert_allclose(goff.reshape(2), [1 / 7, 1 / 5], rtol=0, atol=1e-16)
    np.testing.assert_allclose(gref.reshape(2), [1.0, 1.0], rtol=0, atol=0)


def test_box_locations_reduce_to_pixel_offsets():
    """With one level and a box of size (2K/W, 2K/H), offset / K * wh * 0.5 is
    offset / (W, H): the 4-d form must equal the 2-d form."""
    rng = np.random.default_rng(7)
    H, W, K = 6, 9, 3
    B, Nq, M = 2, 4, 2
    xy = rng.uniform(size=(B, Nq, 1, 2))
    box = np.concatenate([xy, np.broadcast_to([2.0 * K / W, 2.0 * K / H], (B, Nq, 1, 2))], axis=-1)
    off = rng.normal(size=(B, Nq, M, 1, K, 2))
    np.testing.assert_allclose(oracle.sampling_locations_box(box, off),
                               oracle.sampling_locations([[H, W]], xy, off), rtol=0, atol=1e-15)


def test_box_locations_worked_value():
    """cx = 0.5, w = 0.2, K = 4, offset 2.0: 0.5 + 2/4 * 0.2 * 0.5 = 0.55."""
    ref = np.array([0.5, 0.25, 0.2, 0.4]).reshape(1, 1, 1, 4)
    off = np.array([2.0, -1.0]).reshape(1, 1, 1, 1, 1, 2)
    off = np.repeat(off, 4, axis=4)
    loc = oracle.sampling_locations_box(ref, off)
    np.testing.assert_allclose(loc[0, 0, 0, 0, 0], [0.55, 0.25 - 1.0 / 4 * 0.4 * 0.5], rtol=0, atol=1e-15)


def test_box_locations_backward_central_differences():
    rng = np.random.default_rng(8)
    B, Nq, M, L, K = 2, 3, 2, 2, 3
    ref = np.concatenate([rng.uniform(size=(B, Nq, L, 2)), rng.uniform(0.05, 0.5, size=(B, Nq, L, 2))], axis=-1)
    off = rng.normal(size=(B, Nq, M, L, K, 2))
    gl = rng.normal(size=(B, Nq, M, L, K, 2))
    gref, goff = oracle.sampling_locations_box_backward(ref, off, gl)

    def f(r, o):
        return float((oracle.sampling_locations_box(r, o) * gl).sum())

    h = 1e-4
    for arr, got in ((off, goff), (ref, gref)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            p_, m_ = arr.copy(), arr.copy()
            p_[i] += h
            m_[i] -= h
            if arr is off:
                num[i] = (f(ref, p_) - f(ref, m_)) / (2 * h)
            else:
                num[i] = (f(p_, off) - f(m_, off)) / (2 * h)
        np.testing.assert_allclose(got, num, rtol=1e-7, atol=1e-10)
