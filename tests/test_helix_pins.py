"""Pins of the coupled update's scalar schedule in the oracle (oracle/helix.py;
"Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the Active
Set", sections 2.4, 2.5, 2.6 and 2.8).  The page's equations are lost, so the
schedule is pinned by what its prose fixes: the Fibonacci ladder capped at 21
and walked one rung per step, the restart at 1 after a rewind, 36 degrees per
rung of stride, ten steps a turn at stride 1, a blend running from the own
gradient alone to the full coupling strength over each turn, the 1.833 : 1
channel ratio and the 10% / 5% modulation bounds; the trend is checked
against its closed form for constant loss decrements."""
import math

import pytest

from oracle import helix as hx


def test_trend_of_constant_decrements_is_the_decrement():
    h = hx.Helix()
    for k in range(40):
        h.step(10.0 - 0.1 * k)
    assert h.trend == pytest.approx(0.1, rel=1e-9)
    assert h.smooth == pytest.approx(0.1, rel=1e-9)


def test_trend_weights_decay_with_length_ten():
    # decrements 1 then 0, 0, ...: the mean is r^k / sum_{i<=k} r^i
    h = hx.Helix()
    h.step(1.0)
    h.step(0.0)
    for k in range(1, 6):
        h.step(0.0)
        r = math.exp(-0.1)
        assert h.trend == pytest.approx(r ** k / sum(r ** i for i in range(k + 1)), rel=1e-12)


def test_steady_descent_walks_the_fibonacci_ladder_to_21():
    h = hx.Helix()
    strides = []
    for k in range(12):
        h.step(10.0 - 0.1 * k)
        strides.append(h.stride)
    # no trend on the first loss; then one rung per step, capped at 21
    assert strides == [1, 1, 2, 3, 5, 8, 13, 21, 21, 21, 21, 21]
    assert h.rotation == pytest.approx(36.0 * sum(strides))


def test_rising_loss_steps_the_stride_down_one_rung_at_a_time():
    h = hx.Helix()
    for k in range(10):
        h.step(10.0 - 0.1 * k)
    assert h.stride == 21
    seen = []
    x = h.last_loss
    for _ in range(30):
        x += 0.5
        h.step(x)
        seen.append(h.rung)
    # once the smoothed trend turns negative the rung falls by one per step
    first = next(i for i, r in enumerate(seen) if r < 7)
    assert seen[first:first + 7] == [6, 5, 4, 3, 2, 1, 0]
    assert all(r == 0 for r in seen[first + 7:])


def test_rewind_restarts_the_stride_at_one():
    h = hx.Helix()
    for k in range(8):
        h.step(10.0 - 0.1 * k)
    assert h.stride == 21
    h.step(9.0, rewind=True)
    assert h.rung == 0 and h.stride == 1


def test_ten_steps_at_stride_one_make_one_turn():
    h = hx.Helix()
    for _ in range(10):
        h.step(5.0)          # flat loss: trend 0, the rung stays on the first 1
        assert h.stride == 1
    assert h.rotation == pytest.approx(360.0)
    assert h.phase == pytest.approx(0.0, abs=1e-9)


def test_blend_runs_from_own_gradient_to_full_coupling_over_a_turn():
    h = hx.Helix(mod_plus=0.0, mod_minus=0.0)
    b = 0.6
    vals = []
    for k in range(10):
        a_own, a_cross = h.coupling(b)
        assert a_own == 1.0
        e = (1 + math.cos(math.radians(36.0 * k))) / 2
        assert a_cross == pytest.approx(b * (1 - e) / (1.833 * e + (1 - e)), rel=1e-12, abs=1e-15)
        vals.append(a_cross)
        h.step(5.0)
    assert vals[0] == pytest.approx(0.0, abs=1e-15)     # phase 0: own gradient only
    assert vals[5] == pytest.approx(b)                  # phase 180: full coupling strength
    assert all(0.0 <= v <= b for v in vals)
    assert vals[1:5] == pytest.approx(vals[9:5:-1])     # symmetric about half a turn
    assert all(vals[i] < vals[i + 1] for i in range(5))


def test_zero_coupling_strength_gives_no_cross_term_and_psi_shifts_the_phase():
    h = hx.Helix()
    assert h.coupling(0.0) == (1.0, 0.0)
    assert h.coupling(0.4, psi_deg=180.0)[1] == pytest.approx(0.4)


def test_channel_weight_modulation_bounds_and_periods():
    h = hx.Helix()
    for R, wp, wm in ((0.0, 1.10, 1.05), (180.0, 0.90, None), (1800.0, 1.10, 0.95), (3600.0, 1.10, 1.05)):
        h.rotation = R
        p, m = h.weights()
        assert p == pytest.approx(wp)
        if wm is not None:
            assert m == pytest.approx(wm)
    for R in range(0, 7200, 37):
        h.rotation = float(R)
        p, m = h.weights()
        assert 0.9 - 1e-12 <= p <= 1.1 + 1e-12 and 0.95 - 1e-12 <= m <= 1.05 + 1e-12


def test_descent_channel_dominates_at_equal_exposure():
    """Section 2.8: the two channels have unequal weights, 1.833 to 1, so that
    descent stays dominant.  At equal exposure of the two channels (phase 90
    degrees, e = 1/2) and unmodulated channel weights, the cross term must
    take less than half of the coupling strength; with the weights the other
    way round it would take more.  Pins the direction of M : mu."""
    h = hx.Helix(mod_plus=0.0, mod_minus=0.0)
    h.rotation = 90.0
    b = 0.6
    a_own, a_cross = h.coupling(b)
    assert a_own == 1.0
    assert a_cross < b / 2
    swapped = hx.Helix(M=1.0, mu=1.833, mod_plus=0.0, mod_minus=0.0)
    swapped.rotation = 90.0
    assert swapped.coupling(b)[1] > b / 2
    # over a whole turn at stride 1 the cross term averages below half of b too
    h = hx.Helix(mod_plus=0.0, mod_minus=0.0)
    vals = []
    for _ in range(10):
        vals.append(h.coupling(b)[1])
        h.step(5.0)
    assert sum(vals) / len(vals) < b / 2
