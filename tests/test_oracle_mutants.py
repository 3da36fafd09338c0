"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/dcn_oracle.c, builds it into a
temporary library, routes the oracle wrappers to it, and runs the pin battery
of test_oracle_pins / test_oracle_grad.  At least one pin must fail.  Nothing
here touches the HIP library or a GPU.
"""
import json
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_grad as tg
from tests import test_oracle_pins as tp

SRC = os.path.join(os.path.dirname(oracle.__file__), "dcn_oracle.c")

MUTANTS = {
    "x_y_fractions_swapped": ("double lx = x - fx, ly = y - fy;\n                for (int cy",
                              "double ly = x - fx, lx = y - fy;\n                for (int cy"),
    "corner_weight_flipped": ("double w = (cy ? ly : 1.0 - ly) * (cx ? lx : 1.0 - lx);",
                              "double w = (cy ? 1.0 - ly : ly) * (cx ? lx : 1.0 - lx);"),
    "centre_c0_dropped": ("return (double)(o * s - pad + c0) + alpha * ((double)(tap * d - c0) + delta);",
                          "return (double)(o * s - pad + c0) + alpha * ((double)(tap * d) + delta);"),
    "alpha_not_on_grid": ("return (double)(o * s - pad + c0) + alpha * ((double)(tap * d - c0) + delta);",
                          "return (double)(o * s - pad + c0) + (double)(tap * d - c0) + alpha * delta;"),
    "half_pixel_shift": ("return (double)(o * s - pad + c0) + alpha * ((double)(tap * d - c0) + delta);",
                         "return (double)(o * s - pad + c0) - 0.5 + alpha * ((double)(tap * d - c0) + delta);"),
    "skip_rule_too_strict": ("return x > -1.0 && x < (double)W && y > -1.0 && y < (double)H;",
                             "return x >= 0.0 && x < (double)W && y > -1.0 && y < (double)H;"),
    "softmax_unnormalised": ("for (int p = 0; p < P; ++p) m[p] /= sum;", ""),
    "point_order_transposed": ("int p = i * K + j, centre = (K * K - 1) / 2;",
                               "int p = j * K + i, centre = (K * K - 1) / 2;"),
    "removed_tap_not_centre": ("int p = i * K + j, centre = (K * K - 1) / 2;",
                               "int p = i * K + j, centre = (K * K - 1) / 2 + 1;"),
    "right_edge_off_by_one": ("if (yy < 0 || yy >= H || xx < 0 || xx >= W) continue;\n                    double w =",
                              "if (yy < 0 || yy >= H || xx < 0 || xx > W) continue;\n                    double w ="),
    "offset_pair_swapped": ("alpha, off[2 * p], coord_mode);\n                double y = coord(ho, stride, pad, c0, j, dil, alpha, off[2 * p + 1], coord_mode);\n                if (!sample",
                            "alpha, off[2 * p + 1], coord_mode);\n                double y = coord(ho, stride, pad, c0, j, dil, alpha, off[2 * p], coord_mode);\n                if (!sample"),
    "bwd_dwx_sign": ("double dwx = (cx ? 1.0 : -1.0) * wy;", "double dwx = (cx ? -1.0 : 1.0) * wy;"),
    "bwd_dwy_wrong_factor": ("double dwy = (cy ? 1.0 : -1.0) * wx;", "double dwy = (cy ? 1.0 : -1.0) * wy;"),
    "bwd_softmax_jacobian_missing_m": ("gmk[p] = m[p] * (gm[p] - dot);", "gmk[p] = gm[p] - dot;"),
    "bwd_scatter_wrong_pixel": ("long base = (((long)n * H + yy) * W + xx) * C + (long)g * Cg;",
                                "long base = (((long)n * H + yy) * W + (W - 1 - xx)) * C + (long)g * Cg;"),
    "bwd_alpha_missing": ("god[2 * p] = touches ? alpha * m[p] * gdx : 0.0;", "god[2 * p] = touches ? m[p] * gdx : 0.0;"),
    "bwd_skipped_offset_grad_uses_mask": ("god[2 * p] = touches ? alpha * m[p] * gdx : 0.0;",
                                          "god[2 * p] = alpha * m[p] * gdx;"),
}


def battery():
    """All pins, as zero-argument callables."""
    checks = []
    for geom in tp.RC_GEOMS:
        checks.append(lambda g=geom: tp.test_bruteforce_remove_center(g))
        checks.append(lambda g=geom: tp.test_remove_center_is_full_grid_without_centre(g))
    for geom in tp.GEOMS:
        checks.append(lambda g=geom: tp.test_bruteforce_normalised_form_exact_coords(g))
        checks.append(lambda g=geom: tp.test_bruteforce_binary32_coords_dyadic(g))
        checks.append(lambda g=geom: tp.test_grid_sample_construction(g))
    for case in json.load(open(tp.GOLDEN))["cases"]:
        checks.append(lambda c=case: tp.test_hand_worked_golden(c))
    checks += [lambda: tp.test_identity_bit_exact(False), lambda: tp.test_identity_bit_exact(True),
               tp.test_integer_offsets_are_pure_shifts, tp.test_far_outside_is_zero_and_nonfinite_coords_skip,
               tp.test_constant_input_softmax_closed_form, tp.test_linearity_in_input_and_raw_mask,
               tp.test_transpose_consistency, tp.test_absum_bounds_output, tp.test_out_size_matches_conv2d]
    for geom in tg.GEOMS:
        checks.append(lambda g=geom: tg.test_grad_input_adjoint(g))
        checks.append(lambda g=geom: tg.test_grad_offset_finite_difference(g))
    checks += [tg.test_grad_mask_raw_adjoint, lambda: tg.test_grad_mask_finite_difference(False),
               lambda: tg.test_grad_mask_finite_difference(True), tg.test_skipped_samples_have_zero_gradient]
    for bad in (float("inf"), float("nan")):
        checks.append(lambda b=bad: tg.test_skipped_sample_gradients_ignore_its_mask_value(b))
    return checks


def failures(lib_path):
    n = 0
    with oracle.library_override(lib_path):
        for chk in battery():
            try:
                chk()
            except (AssertionError, ValueError):
                n += 1
    return n


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: " + name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99",
                    "-o", str(lib), str(mutated), "-lm"], check=True)
    assert failures(str(lib)) > 0, "no pin caught mutant " + name


def test_unmutated_copy_passes_every_pin(tmp_path):
    lib = tmp_path / "libsame.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99",
                    "-o", str(lib), SRC, "-lm"], check=True)
    assert failures(str(lib)) == 0
