"""The oracle's pins have teeth: plant one plausible mistake at a time in a copy
of the oracle source (on the CPU), build it, and check that at least one pin
fails against it. The shipped oracle is never modified."""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle_backward as tb
from tests import test_oracle_forward as tf
from tests import test_oracle_fused_grads as tg
from tests import test_oracle_mask as tmk
from tests import test_oracle_prologue as tp


def _forward_pins():
    tf.test_forward_matches_tent_brute_force(0, dict(B=2, M=2, D=3, shapes=((5, 7), (3, 4)), Nq=6, K=3))
    tf.test_bilinear_hand_worked_values()
    tf.test_pixel_centre_is_exact_gather()
    tf.test_page2_offset_example_lands_on_pixels()
    tf.test_zero_padding_and_non_finite()


def _backward_pins():
    for g in tb.GEOMS:
        tb.test_adjoint_identities(g)
        tb.test_grad_loc_central_differences(g)
    tb.test_grad_loc_right_derivative_at_integer_pixel()


def _prologue_pins():
    tp.test_pyramid_counts_from_page1()
    tp.test_encoder_refs_at_unit_ratio_are_pixel_centres()
    tp.test_encoder_refs_keep_valid_relative_position()
    tp.test_decoder_refs_scaled_by_valid_ratio_page2()
    tp.test_locations_zero_offset_is_reference_and_pixel_steps()
    tp.test_softmax_matches_scipy_and_sums_to_one_over_levels_and_points()


def _fused_grad_pins():
    tg.test_softmax_backward_matches_explicit_jacobian()
    tg.test_softmax_backward_central_differences()
    tg.test_locations_backward_central_differences()
    tg.test_locations_backward_scales_by_level_size()
    tg.test_box_locations_reduce_to_pixel_offsets()
    tg.test_box_locations_worked_value()
    tg.test_box_locations_backward_central_differences()


def _mask_pins():
    tmk.test_mask_fill_identity_zero_idempotent_and_self_adjoint()
    tmk.test_masking_rows_no_corner_touches_changes_nothing()
    tmk.test_masked_pixel_centre_reads_zero()
    tmk.test_masked_chain_gradient_by_central_differences()


MUTANTS = [
    # (name, text in msda_oracle.c, replacement, pins expected to catch it)
    ("swapped_x_weights", "(dx ? fx : 1.0 - fx)", "(dx ? 1.0 - fx : fx)", _forward_pins),
    ("no_half_pixel_shift", "lx * (double)W - 0.5", "lx * (double)W", _forward_pins),
    ("align_corners_true", "lx * (double)W - 0.5", "lx * (double)(W - 1)", _forward_pins),
    ("transposed_row_index", "lsi[l] + yi * W + xi;\n                        const double *v",
     "lsi[l] + xi * H + yi;\n                        const double *v", _forward_pins),
    ("h_w_swapped", "const int64_t H = shapes[2 * l + 0];\n            const int64_t W = shapes[2 * l + 1];\n"
     "            for (int k = 0; k < K; ++k) {\n                const int64_t sidx = (((b * Nq + q) * M + m) * L + l) * K + k;\n"
     "                const double a = attn[sidx];\n                int64_t x0",
     "const int64_t H = shapes[2 * l + 1];\n            const int64_t W = shapes[2 * l + 0];\n"
     "            for (int k = 0; k < K; ++k) {\n                const int64_t sidx = (((b * Nq + q) * M + m) * L + l) * K + k;\n"
     "                const double a = attn[sidx];\n                int64_t x0", _forward_pins),
    ("edge_corner_kept", "return xi >= 0 && xi < W", "return xi >= 0 && xi <= W", _forward_pins),
    ("dropped_attention_weight", "acc[d] += a * w * v[d]", "acc[d] += w * v[d]", _forward_pins),
    ("wrong_grad_sign", "const double dwx = dx ? 1.0 : -1.0;", "const double dwx = dx ? -1.0 : 1.0;", _backward_pins),
    ("grad_loc_wrong_scale", "a * (double)W * glx", "a * (double)H * glx", _backward_pins),
    ("grad_value_drops_weight", "gv[d] += a * wx * wy * g[d]", "gv[d] += a * wx * g[d]", _backward_pins),
    ("grad_attn_wrong_corner_weight", "ga += wx * wy * gdotv", "ga += wx * gdotv", _backward_pins),
    ("ref_no_half_pixel", "((double)j + 0.5) / (vr_x_own", "((double)j) / (vr_x_own", _prologue_pins),
    ("ref_own_ratio_missing", "/ (vr_y_own * (double)H)", "/ ((double)H)", _prologue_pins),
    ("loc_normaliser_swapped", "offset_px[idx + 0] / W", "offset_px[idx + 0] / H", _prologue_pins),
    ("lsi_inclusive", "lsi_out[l] = start;\n        start += shapes[2 * l + 0] * shapes[2 * l + 1];",
     "start += shapes[2 * l + 0] * shapes[2 * l + 1];\n        lsi_out[l] = start;", _prologue_pins),
    ("softmax_no_normalise", "for (int i = 0; i < n; ++i) y[i] /= sum;", "", _prologue_pins),
    ("softmax_grad_drops_mean", "a[i] * (ga[i] - dot)", "a[i] * ga[i]", _fused_grad_pins),
    ("softmax_grad_wrong_factor", "a[i] * (ga[i] - dot)", "(ga[i] - dot)", _fused_grad_pins),
    ("offset_grad_swapped_normaliser", "grad_offset_px[idx + 0] = grad_loc[idx + 0] / W;",
     "grad_offset_px[idx + 0] = grad_loc[idx + 0] / H;", _fused_grad_pins),
    ("ref_grad_one_term", "gr[0] += grad_loc[idx + 0];\n                            gr[1] += grad_loc[idx + 1];\n                        }",
     "gr[0] = grad_loc[idx + 0];\n                            gr[1] += grad_loc[idx + 1];\n                        }", _fused_grad_pins),
    ("box_wh_swapped", "offset[idx + 0] / (double)K * r[2] * 0.5", "offset[idx + 0] / (double)K * r[3] * 0.5",
     _fused_grad_pins),
    ("box_no_half", "offset[idx + 1] / (double)K * r[3] * 0.5", "offset[idx + 1] / (double)K * r[3]",
     _fused_grad_pins),
    ("box_grad_wh_term", "gr[2] += grad_loc[idx + 0] * offset[idx + 0] * 0.5 / (double)K;",
     "gr[2] += grad_loc[idx + 0] * offset[idx + 0] / (double)K;", _fused_grad_pins),
    ("mask_inverted", "mask[b * S + s] ? 0.0 : x[(b * S + s) * C + c]", "mask[b * S + s] ? x[(b * S + s) * C + c] : 0.0",
     _mask_pins),
    ("mask_wrong_row", "mask[b * S + s] ? 0.0", "mask[s] ? 0.0", _mask_pins),
]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, pins):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in the oracle source"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-ffp-contract=off",
                    "-I", os.path.dirname(obuild.SRC), "-o", str(lib), str(mutated), "-lm"], check=True)
    with oracle.swapped_library(str(lib)):
        with pytest.raises(AssertionError):
            pins()
    # and the shipped oracle still passes the same pins
    pins()
