"""The library's checkpoint-and-rewind controller (host code, section 2.6 of
"Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the Active
Set") against the oracle: on the hand-worked pin sequences and on long
seeded loss runs with spikes and NaNs, every action and every state field
must agree exactly (both compare in double precision)."""
import math

import numpy as np
import pytest

from oracle import rewind as rw
from sparse_full_weight_amd import _lib


def _run(losses):
    c = rw.Rewind()
    return [c.observe(x) for x in losses]


def _random_losses(seed, n):
    g = np.random.default_rng(seed)
    x, out = 5.0, []
    for _ in range(n):
        x *= math.exp(g.normal(-0.01, 0.04))
        y = x * (1.0 + (g.random() < 0.05) * g.uniform(0.1, 0.6))   # occasional spikes
        if g.random() < 0.01:
            y = float("nan")
        out.append(y)
    return out


def test_library_controller_matches_the_pins():
    cases = [[10.0, 9.0, 8.0, 7.0], [10.0, 8.0] + [8.5] * 9 + [9.3],
             [10.0, 8.0] + [8.5] * 9 + [9.3] + [9.3] * 40,
             [10.0, 8.0] + [8.5] * 9 + [9.1, 8.7, 9.5, 8.0],
             [10.0, 8.0] + [9.0] * 5 + [7.0] + [9.0] * 10, [10.0, float("nan")] + [math.inf] * 9,
             [math.inf, 5.0]]
    for losses in cases:
        want = _run(losses)
        ctl = _lib.Rewind()
        assert [ctl.observe(x) for x in losses] == want


def test_library_controller_reproduces_the_page_rewind():
    """Section 4.2's event: the first restore of the run comes at step 356
    and brings back the checkpoint of step 336."""
    losses = [6.17 * math.exp(-0.00322 * k) for k in range(336)]
    l336 = losses[-1] * 0.99
    l346 = l336 * 0.98
    losses += [l336] + [l336 * 1.03] * 9 + [l346] + [l346 * 1.05] * 9 + [l346 * 1.2]
    c = _lib.Rewind()
    acts = [c.observe(x) for x in losses]
    assert acts.index(_lib.SFT_REWIND_RESTORE) == 356
    assert c.state().checkpoint_step == 336 and c.state().min_step == 346


def _fields(c, o):
    st = c.state()
    got = (st.has_checkpoint, st.watch_left, st.recoveries, st.checkpoint_loss, st.min_loss, st.step,
           st.checkpoint_step, st.min_step)
    want = (int(o.has_checkpoint), o.watch_left, o.recoveries, o.checkpoint_loss, o.min_loss, o.step,
            o.checkpoint_step, o.min_step)
    return got, want


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_library_controller_matches_oracle_on_long_runs(seed):
    losses = _random_losses(seed, 3000)
    o = rw.Rewind()
    c = _lib.Rewind()
    seen = set()
    for x in losses:
        a = c.observe(x)
        assert a == o.observe(x)
        seen.add(a)
        got, want = _fields(c, o)
        assert got == want
    # the runs exercise every kind of step
    assert {0, rw.RESTORE, rw.PROMOTE, rw.PROMOTE | rw.SAVE_MIN, rw.SAVE} <= seen


def test_library_controller_rejects_bad_settings():
    c = _lib.Rewind()
    c.st.watch_steps = 0
    with pytest.raises(_lib.SftError) as e:
        c.observe(1.0)
    assert e.value.code == _lib.SFT_EINVAL
