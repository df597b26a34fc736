"""Checkpoint and rewind, as plain Python: the controller's decisions and the
row copies a checkpoint makes.

TEST INFRASTRUCTURE ONLY: the test-suite and the smoke check use this module
to state what the library's checkpoint calls must do.  The GPU library never
imports it, and it imports nothing from the GPU library.

Source: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
Active Set", section 2.6 (checkpoint and rewind).  The section gives the rule
in prose only; the readings taken here are:
  1. a copy of the active rows is taken when no copy exists yet, or when the
     step's loss is at most (1 + 0.10) times the loss recorded with the last
     copy (a lower loss qualifies); the copy records its loss;
  2. a new minimum is a loss strictly below every loss seen before; it opens
     a watch of the 10 following steps and clears the recovery count;
  3. the 10th step after the minimum ends the watch: if its loss is more than
     (1 + 0.15) times the minimum and fewer than 3 recoveries were made for
     this minimum, the rows are restored, the stride restarts and the step
     is dropped (nothing else happens on it), and the watch starts again on
     the same minimum; in every other case the minimum stands and later
     copies are compared with it;
  4. within one step: end of watch first, then the new-minimum test, then
     the copy test;
  5. a NaN or infinite loss is taken as +infinity.
All comparisons are in double precision (Python floats).
"""
from __future__ import annotations

import math

import numpy as np

SAVE = 1
RESTORE = 2


class Rewind:
    """The controller's state and its per-step decision."""

    def __init__(self, save_within: float = 0.10, rise_above: float = 0.15, watch_steps: int = 10,
                 max_recoveries: int = 3):
        self.save_within = save_within
        self.rise_above = rise_above
        self.watch_steps = watch_steps
        self.max_recoveries = max_recoveries
        self.has_checkpoint = False
        self.checkpoint_loss = 0.0
        self.min_loss = math.inf
        self.watch_left = 0
        self.recoveries = 0

    def observe(self, loss: float) -> int:
        """Returns 0, SAVE or RESTORE for the step whose loss is ``loss``."""
        x = float(loss)
        if not math.isfinite(x):
            x = math.inf
        # reading 3: the end of an open watch
        if self.watch_left > 0:
            self.watch_left -= 1
            if self.watch_left == 0:
                risen = x > (1.0 + self.rise_above) * self.min_loss
                if risen and self.recoveries < self.max_recoveries:
                    self.recoveries += 1
                    self.watch_left = self.watch_steps
                    return RESTORE
                self.checkpoint_loss = self.min_loss
        # reading 2: a new minimum
        if x < self.min_loss:
            self.min_loss = x
            self.watch_left = self.watch_steps
            self.recoveries = 0
        # reading 1: the copy
        if x != math.inf and (not self.has_checkpoint or x <= (1.0 + self.save_within) * self.checkpoint_loss):
            self.has_checkpoint = True
            self.checkpoint_loss = x
            return SAVE
        return 0


class RowCopy:
    """The saved rows of one matrix: row k belongs to rows[k]."""

    def __init__(self, q, s, delta, m, v, t):
        self.q, self.s, self.delta, self.m, self.v, self.t = q, s, delta, m, v, t


def rows_save(st, rows, slot) -> RowCopy:
    """Copies rows (q, s, delta) and the moment slots (m, v, t) of a matrix
    state (an ``oracle.MatState``)."""
    rows = np.asarray(rows, np.int64)
    slot = np.asarray(slot, np.int64)
    return RowCopy(st.q[rows].copy(), st.s[rows].copy(), st.delta[rows].copy(), st.m[slot].copy(),
                   st.v[slot].copy(), st.t[slot].copy())


def rows_restore(st, ck: RowCopy, rows, slot) -> None:
    """Writes a copy back (rows and slots) and rebuilds those rows of the live
    bf16 weights when the state has them (section 2.3's write-back)."""
    import oracle
    rows = np.asarray(rows, np.int64)
    slot = np.asarray(slot, np.int64)
    st.q[rows] = ck.q
    st.s[rows] = ck.s
    st.delta[rows] = ck.delta
    st.m[slot] = ck.m
    st.v[slot] = ck.v
    st.t[slot] = ck.t
    if st.w_live is not None:
        oracle.masked_writeback(st.q, st.s, st.delta, rows.astype(np.int32), st.w_live)
