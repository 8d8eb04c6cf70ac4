"""The oracle's threaded loops (used by the host-core baseline) give results
bit-identical to its serial loops, which the other oracle tests pin: every
output element is computed by one thread with the same operations in the same
order."""
import numpy as np
import pytest

import oracle
from scale_deformable_attention_msdeformattn_amd import workloads
from tests.core_inputs import build


@pytest.mark.parametrize("threads", [2, 5, 16])
def test_threaded_oracle_is_bit_identical_to_serial(threads):
    wl = workloads.custom(name="thr", batch=3, heads=4, channels=8, points=3,
                          spatial_shapes=((9, 13), (5, 7), (3, 4)), num_query=None,
                          offset_sigma_px=2.5, random_valid_ratios=True)
    ci = build(wl, seed=4)
    ids = np.array([0, 5, ci.loc.shape[1], 3 * ci.loc.shape[1] - 1])
    serial_f = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn)
    serial_q = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, query_ids=ids)
    serial_b = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    with oracle.threads(threads):
        f = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn)
        fq = oracle.forward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, query_ids=ids)
        b = oracle.backward(ci.value, ci.shapes, ci.lsi, ci.loc, ci.attn, ci.grad_output)
    assert np.array_equal(f, serial_f)
    assert np.array_equal(fq, serial_q)
    for got, want in zip(b, serial_b):
        assert np.array_equal(got, want)
