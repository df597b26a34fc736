"""Pins of the checkpoint-and-rewind oracle ("Sparse-First Fine-Tuning: Full-
Weight Training at the Cost of the Active Set", section 2.6).

The expected action sequences below were worked out by hand from the rule
the section states (copy while the loss stays within a 10% margin of the
last copy's loss, a 10-step watch after each new minimum, restore when the
watch closes with a loss over 1.15 times the minimum, at most 3 restores per
minimum, else keep the minimum), under the readings listed in
oracle/rewind.py; each case names the step that decides it.
"""
import math

import numpy as np

import oracle
from oracle import rewind as rw
from sparse_full_weight_amd import synth

S, R = rw.SAVE, rw.RESTORE


def _run(losses, ctl=None):
    ctl = ctl or rw.Rewind()
    return [ctl.observe(x) for x in losses], ctl


def test_defaults_are_the_page_values():
    c = rw.Rewind()
    assert (c.save_within, c.rise_above, c.watch_steps, c.max_recoveries) == (0.10, 0.15, 10, 3)


def test_steady_descent_saves_every_step():
    acts, c = _run([10.0, 9.0, 8.0, 7.0])
    assert acts == [S, S, S, S]
    assert c.min_loss == 7.0 and c.watch_left == 10 and c.checkpoint_loss == 7.0


def test_rise_above_15_percent_at_end_of_watch_restores():
    # minimum 8 at step 1; steps 2..10 at 8.5 stay under 1.1 times the last copy
    # (8.8, then 9.35) and are saved; step 11 is the 10th after the minimum and
    # 9.3 > 1.15 * 8 = 9.2
    acts, c = _run([10.0, 8.0] + [8.5] * 9 + [9.3])
    assert acts == [S, S] + [S] * 9 + [R]
    assert c.recoveries == 1 and c.watch_left == 10 and c.min_loss == 8.0


def test_rise_within_15_percent_accepts_the_minimum():
    # 9.1 <= 9.2: the minimum is accepted, the copy reference drops to 8, and
    # 9.1 > 1.1 * 8 = 8.8 is not saved; the next step at 8.7 <= 8.8 is
    acts, c = _run([10.0, 8.0] + [8.5] * 9 + [9.1, 8.7])
    assert acts == [S, S] + [S] * 9 + [0, S]
    assert c.watch_left == 0 and c.recoveries == 0


def test_three_recoveries_per_minimum_then_accept():
    # after the first restore the watch re-opens on the same minimum; a loss of
    # 9.3 stays within 10% of the copies (first 8.5: 9.35) so it is saved, and
    # each 10th step restores again until 3 restores were made; the 4th rise
    # accepts the minimum (reference 8: 9.3 > 8.8, no copy)
    first = [10.0, 8.0] + [8.5] * 9 + [9.3]
    acts, c = _run(first + [9.3] * 30)
    assert acts[:12] == [S, S] + [S] * 9 + [R]
    assert acts[12:22] == [S] * 9 + [R]
    assert acts[22:32] == [S] * 9 + [R]
    assert acts[32:42] == [S] * 9 + [0]
    assert c.recoveries == 3 and c.watch_left == 0 and c.checkpoint_loss == 8.0
    # no watch is open and 9.3 is not within 10% of 8: nothing more happens
    assert [c.observe(9.3) for _ in range(12)] == [0] * 12


def test_new_minimum_restarts_the_watch():
    # minimum 8 at step 1, then 9 (no copy: 9 > 8.8); a new minimum 7 at step
    # 7 restarts the watch, so step 11 decides nothing; step 17 (10th after
    # step 7) has 9 > 1.15 * 7 = 8.05 and restores
    acts, c = _run([10.0, 8.0] + [9.0] * 5 + [7.0] + [9.0] * 10)
    assert acts == [S, S] + [0] * 5 + [S] + [0] * 9 + [R]
    assert c.min_loss == 7.0


def test_non_finite_loss_is_a_rise_and_never_saved():
    acts, c = _run([10.0, float("nan")] + [math.inf] * 9)
    assert acts == [S, 0] + [0] * 8 + [R]
    assert c.min_loss == 10.0


def test_infinite_first_loss_is_not_saved_the_first_finite_one_is():
    acts, _ = _run([math.inf, 5.0])
    assert acts == [0, S]


def _state(R_, C, n_slots, seed):
    q, s, delta = synth.quant_state(R_, C, seed)
    m, v, t = synth.moments(n_slots, C, seed + 1, mid_run=True)
    w = np.zeros((R_, C), np.uint16)
    return oracle.MatState(q, s, delta, m, v, t, w)


def test_rows_save_restore_round_trip():
    st = _state(40, 24, 12, 31)
    rows = np.array([1, 5, 6, 30], np.int32)
    slot = np.array([3, 0, 11, 7], np.int32)
    before = st.copy()
    ck = rw.rows_save(st, rows, slot)
    assert np.array_equal(ck.q, before.q[rows]) and np.array_equal(ck.m, before.m[slot])
    # scramble the live state, restore, compare
    st.q[:] = 0
    st.s[:] = 1.0
    st.delta[:] = 2.0
    st.m[:] = 7
    st.v[:] = 9
    st.t[:] = 99
    rw.rows_restore(st, ck, rows, slot)
    assert np.array_equal(st.q[rows], before.q[rows])
    assert np.array_equal(st.s[rows], before.s[rows])
    assert np.array_equal(st.delta[rows].view(np.uint32), before.delta[rows].view(np.uint32))
    assert np.array_equal(st.m[slot], before.m[slot]) and np.array_equal(st.v[slot], before.v[slot])
    assert np.array_equal(st.t[slot], before.t[slot])
    others = np.setdiff1d(np.arange(40), rows)
    assert np.all(st.q[others] == 0) and np.all(st.s[others] == 1.0)
    assert np.all(np.delete(st.m, slot, axis=0) == 7)
    # the restored rows' live weights are bf16(fl(s*q) + delta)
    w = oracle.bf16_to_f32(st.w_live[rows])
    want = (before.s[rows, None] * before.q[rows].astype(np.float32)).astype(np.float32) + before.delta[rows]
    assert np.array_equal(st.w_live[rows], oracle.f32_to_bf16(want))
    assert np.allclose(w, want, rtol=2 ** -8, atol=0)
    assert not st.w_live[others].any()
