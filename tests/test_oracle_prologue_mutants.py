"""Planted mistakes in the producer-step oracle must be caught by its pins
(CPU only): each case copies oracle/prologue.py, plants one plausible mistake
(group sizes swapped, frequency sign or denominator wrong, rotation
direction, rotate-half pairing instead of adjacent pairs, axes swapped, eps
outside the root, sum instead of mean, means taken before rounding), loads
the mutant and runs the pins of tests/test_oracle_prologue.py against it.
The unmutated source must pass the same pins."""
import os
import types

import pytest

from tests import test_oracle_prologue as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "prologue.py")

MUTANTS = {
    "group_sizes_swapped": [("return D - 2 * dy, dy, dy", "return dy, dy, D - 2 * dy")],
    "frequency_sign": [("theta = base ** (-2.0 * j / d_a)", "theta = base ** (2.0 * j / d_a)")],
    "frequency_over_head_dim": [("theta = base ** (-2.0 * j / d_a)",
                                 "theta = base ** (-2.0 * j / (d_t + d_y + d_x))"),
                                ("dt, dy, dx = rope_split(D)", "dt, dy, dx = rope_split(D)\n    d_t, d_y, d_x = dt, dy, dx")],
    "rotation_direction": [("out[..., 0::2] = a * c - b * s", "out[..., 0::2] = a * c + b * s"),
                           ("out[..., 1::2] = a * s + b * c", "out[..., 1::2] = -a * s + b * c")],
    "rotate_half_pairs": [("a, b = x[..., 0::2], x[..., 1::2]",
                           "a, b = x[..., :x.shape[-1] // 2], x[..., x.shape[-1] // 2:]"),
                          ("out[..., 0::2] = a * c - b * s", "out[..., :x.shape[-1] // 2] = a * c - b * s"),
                          ("out[..., 1::2] = a * s + b * c", "out[..., x.shape[-1] // 2:] = a * s + b * c")],
    "rows_and_columns_swapped": [("pos = (tok // (Hg * Wg), (tok // Wg) % Hg, tok % Wg)",
                                  "pos = (tok // (Hg * Wg), tok % Wg, (tok // Wg) % Hg)")],
    "eps_outside_root": [("np.sqrt(ms + eps)", "(np.sqrt(ms) + eps)")],
    "sum_instead_of_mean": [("ms = (x * x).mean(axis=-1, keepdims=True)", "ms = (x * x).sum(axis=-1, keepdims=True)")],
    "means_before_rounding": [("pos = yb if order is None else yb[np.asarray(order)]",
                               "pos = y if order is None else y[np.asarray(order)]")],
}

PINS = [
    lambda: pins.test_group_split(),
    lambda: pins.test_closed_form_d6(),
    lambda: pins.test_closed_form_d12_second_frequency(),
    lambda: pins.test_rotation_is_complex_multiplication(),
    lambda: pins.test_scores_depend_on_relative_position_only(),
    lambda: pins.test_rms_norm_scale_invariance_and_unit_mean_square(),
    lambda: pins.test_prologue_means_are_block_means_of_rounded_output(),
    lambda: pins.test_rms_norm_eps_closed_form(),
]


def _load(src):
    mod = types.ModuleType("prologue_mutant")
    exec(compile(src, "prologue_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    saved = pins.pro
    pins.pro = mod
    try:
        for pin in PINS:
            pin()
        return True
    except (AssertionError, ValueError, IndexError, ZeroDivisionError):
        return False
    finally:
        pins.pro = saved


def _source():
    with open(SRC) as f:
        return f.read()


def test_unmutated_oracle_passes():
    assert _pins_pass(_load(_source()))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    src = _source()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
        src = src.replace(old, new)
    assert not _pins_pass(_load(src)), f"pins accept the mutant {name}"
