"""Pins of the attention acceptance rule (oracle.acceptance.check_attention):
every attention decision of the GPU parity tests passes through it, so each
plausible slip in it (one bar instead of both, a signed instead of an
absolute error, a NaN that compares false, a broadcast between mismatched
shapes) must fail one of these.

The bars are the stated tolerance of the attention output: max-abs 2e-2 and
mean-abs 2e-3 against the oracle on identical FP8 operands."""
import numpy as np
import pytest

from oracle.acceptance import (ATTN_MAX_ABS, ATTN_MEAN_ABS, attention_error,
                               check_attention)

SHAPE = (32, 128)


def _ref(seed=0):
    return np.random.default_rng(seed).standard_normal(SHAPE) * 0.05


def test_bars_are_the_stated_tolerance():
    assert ATTN_MAX_ABS == 2e-2 and ATTN_MEAN_ABS == 2e-3


def test_identical_and_small_errors_accepted():
    ref = _ref()
    assert check_attention(ref, ref) is None
    assert attention_error(ref, ref) == (0.0, 0.0)
    rng = np.random.default_rng(1)
    out = ref + rng.uniform(-1e-3, 1e-3, SHAPE)
    assert check_attention(out, ref) is None


def test_max_bar_alone_rejects():
    # one element past 2e-2, every other exact: mean 2.1e-2 / 4096 is far
    # below 2e-3, so only the max bar can reject it
    ref = _ref()
    out = ref.copy()
    out[3, 7] += 2.1e-2
    mx, mean = attention_error(out, ref)
    assert mx > ATTN_MAX_ABS and mean < ATTN_MEAN_ABS
    assert check_attention(out, ref) is not None
    out[3, 7] = ref[3, 7] + 1.9e-2
    assert check_attention(out, ref) is None


def test_mean_bar_alone_rejects():
    # every element off by 3e-3: max 3e-3 is within 2e-2, mean 3e-3 is not
    ref = _ref()
    out = ref + 3e-3
    mx, mean = attention_error(out, ref)
    assert mx <= ATTN_MAX_ABS and mean > ATTN_MEAN_ABS
    assert check_attention(out, ref) is not None


def test_mean_is_of_absolute_errors():
    # +3e-3 and -3e-3 alternating: the signed mean is 0, the absolute 3e-3
    ref = _ref()
    sign = np.where(np.arange(ref.size).reshape(SHAPE) % 2 == 0, 1.0, -1.0)
    out = ref + 3e-3 * sign
    assert abs(float(np.mean(out - ref))) < 1e-12
    assert attention_error(out, ref)[1] == pytest.approx(3e-3)
    assert check_attention(out, ref) is not None


def test_error_is_symmetric():
    ref = _ref()
    out = ref.copy()
    out[0, 0] -= 5e-2
    assert attention_error(out, ref) == attention_error(ref, out)
    assert check_attention(ref, out) is not None


def test_bars_are_inclusive():
    # errors exactly at the bars pass (<=), just past them fail; the values
    # are chosen exact in binary so the comparison is not decided by rounding
    ref = np.zeros(SHAPE)
    out = np.zeros(SHAPE)
    out[0, 0] = 2.0 ** -6                      # 0.0156 < 2e-2
    assert check_attention(out, ref, max_abs=2.0 ** -6, mean_abs=1.0) is None
    assert check_attention(out, ref, max_abs=2.0 ** -7, mean_abs=1.0) is not None
    m = float(np.mean(np.abs(out - ref)))
    assert check_attention(out, ref, max_abs=1.0, mean_abs=m) is None
    assert check_attention(out, ref, max_abs=1.0, mean_abs=m / 2) is not None


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_rejected(bad):
    ref = _ref()
    out = ref.copy()
    out[5, 9] = bad
    assert check_attention(out, ref) is not None
    # also when the oracle side holds it
    assert check_attention(ref, out) is not None
    assert attention_error(out, ref) == (float("inf"), float("inf"))


def test_shape_mismatch_rejected():
    # broadcasting a single head row against all heads must not pass
    ref = _ref()
    assert check_attention(ref[:1], ref) is not None
    assert check_attention(ref.reshape(-1), ref) is not None
    assert check_attention(np.zeros((0, 128)), np.zeros((0, 128))) is not None


def test_a_wrong_head_mapping_is_caught():
    # the kind of error a kernel could make: two query heads' outputs swapped.
    # Attention outputs of N(0,1) data over ~2,000 keys are ~0.03 RMS, so a
    # swap moves elements by ~0.05, far past the max bar.
    rng = np.random.default_rng(7)
    ref = rng.standard_normal(SHAPE) * 0.035
    out = ref.copy()
    out[[4, 12]] = out[[12, 4]]
    assert check_attention(out, ref) is not None
