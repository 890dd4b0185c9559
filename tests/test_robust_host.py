"""Host-only checks of the training-loop robustness pieces of libgpt2.so: the
rolling z-score detector behind the loss / gradient-norm spike skip (llm.c
GPT-2 1.5B post, dszhyy.com: the training log's z-scores and the restart
that skips updates whose z-score exceeds 5).  No GPU calls."""
import math

import numpy as np
import pytest

import transformer_lm_pretraining_train_amd as g


def closed_form_z(window_vals, x):
    """z of x against the population mean and standard deviation of the
    window, in float64, from the definition."""
    w = np.asarray(window_vals, dtype=np.float64)
    sd = math.sqrt(((w - w.mean()) ** 2).mean())
    return (x - w.mean()) / sd if sd > 0 else float("nan")


def test_zscore_is_nan_until_the_window_is_full_then_the_closed_form():
    zs = g.ZScore(4)
    seq = [3.0, 1.0, 4.0, 1.5, 9.0, 2.6, 5.0, -3.5, 5.8, 9.7]
    for i, x in enumerate(seq):
        z = zs.update(x)
        if i < 4:
            assert math.isnan(z)
        else:
            want = closed_form_z(seq[i - 4:i], x)  # the four values before x
            assert z == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_zscore_skips_non_finite_values_and_flat_windows():
    zs = g.ZScore(3)
    for x in (2.0, 2.0, 2.0):
        zs.update(x)
    assert math.isnan(zs.update(5.0))  # std of (2, 2, 2) is 0
    assert math.isnan(zs.update(float("nan")))  # not finite: NaN, not added
    assert math.isnan(zs.update(float("inf")))
    # the window now holds 2, 2, 5 (the NaN and inf never entered it)
    assert zs.update(1.0) == pytest.approx(closed_form_z([2.0, 2.0, 5.0], 1.0), rel=1e-12)


def test_zscore_spike_against_a_noisy_history():
    """A value far above a noisy history scores far above 5, one inside it
    scores near 0: the detector the guarded step uses to skip an update."""
    rng = np.random.default_rng(7)
    hist = 3.0 + 0.05 * rng.standard_normal(128)
    zs = g.ZScore(128)
    for x in hist:
        zs.update(x)
    assert zs.update(3.0 + 100 * 0.05) > 5.0
    assert abs(zs.update(float(hist[-1]))) < 5.0


@pytest.mark.parametrize("window", [0, 1, 65537])
def test_zscore_window_bounds(window):
    with pytest.raises(g.GPT2Error):
        g.ZScore(window)


def test_zscore_state_round_trip_continues_bit_for_bit():
    """A detector rebuilt from another's state (get_state / set_state, the
    values held, oldest first) scores every later value with the same bits,
    before and after the window has wrapped; bad states are refused."""
    rng = np.random.default_rng(3)
    xs = list(rng.standard_normal(40) * 0.1 + 3.0)
    for cut in (3, 5, 17):  # part-full, just full, wrapped
        a = g.ZScore(5)
        for x in xs[:cut]:
            a.update(x)
        st = a.get_state()
        assert st == xs[max(0, cut - 5):cut]
        b = g.ZScore(5)
        b.set_state(st)
        assert b.get_state() == st
        for x in xs[cut:]:
            za, zb = a.update(x), b.update(x)
            assert (math.isnan(za) and math.isnan(zb)) or za == zb
    c = g.ZScore(4)
    for bad in ([1.0] * 5, [1.0, float("nan")]):
        with pytest.raises(g.GPT2Error) as ei:
            c.set_state(bad)
        assert ei.value.name == "EINVAL"
