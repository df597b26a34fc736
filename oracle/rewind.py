"""Checkpoint and rewind, as plain Python: the controller's decisions and the
row copies a checkpoint makes.

TEST INFRASTRUCTURE ONLY: the test-suite and the smoke check use this module
to state what the library's checkpoint calls must do.  The GPU library never
imports it, and it imports nothing from the GPU library.

Source: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
Active Set", section 2.6 (checkpoint and rewind) and section 4.2 (the one
rewind the page reports: at step 356 the loss had rebounded past the
threshold and the checkpoint restored was the one of step 336).  Section 2.6
gives the rule in prose only.  The readings taken here are:
  1. two row copies exist: the checkpoint (what a restore brings back) and
     the copy of the current minimum (taken when the minimum is seen, so
     that the minimum itself can become the checkpoint once accepted);
  2. a new minimum is a loss strictly below every loss seen before; its rows
     are copied into the minimum's copy, it opens a watch of the 10
     following steps and clears the recovery count.  A new minimum that
     arrives while the watch of an earlier minimum is open accepts that
     earlier minimum first (the loss has fallen below it, so it cannot have
     risen 15% above it);
  3. the 10th step after the minimum ends the watch: if its loss is more
     than (1 + 0.15) times the minimum and fewer than 3 recoveries were made
     for this minimum, the checkpoint is restored, the stride restarts and
     the step is dropped (nothing else happens on it), and the watch starts
     again on the same minimum; otherwise the minimum is accepted;
  4. an accepted minimum becomes the checkpoint: its copy takes the
     checkpoint's place, with the minimum's loss;
  5. outside a watch the checkpoint is refreshed with the current rows when
     the loss is within (1 + 0.10) times the checkpoint's loss (a lower loss
     qualifies) and not more than (1 + 0.15) times the minimum (a state the
     rise test would reject is never kept); the first finite loss always
     makes the first checkpoint; during a watch the checkpoint is left as
     it is, so that a restore brings back a state from before the watched
     minimum;
  6. within one step: end of watch first, then the new-minimum test, then
     the refresh; a loss that is NaN or infinite is taken as +infinity;
  7. every copy carries the loss of the rows it holds; the rows copied are
     the ones that produced the step's loss (the caller applies the actions
     before the step's update).
With these readings the page's section 4.2 event is one restore: a minimum
at step 336 passes its watch at step 346 and becomes the checkpoint, step
346 is a new minimum whose watch ends at step 356 with a rebound, and the
restore brings back the rows of step 336.
All comparisons are in double precision (Python floats).
"""
from __future__ import annotations

import math

import numpy as np

# action bits; a step's actions are applied in the order PROMOTE, SAVE_MIN, SAVE
SAVE = 1        # copy the current rows into the checkpoint
RESTORE = 2     # bring the checkpoint back and drop the step (always alone)
SAVE_MIN = 4    # copy the current rows into the minimum's copy
PROMOTE = 8     # the minimum's copy becomes the checkpoint (the two copies swap roles)


class Rewind:
    """The controller's state and its per-step decision."""

    def __init__(self, save_within: float = 0.10, rise_above: float = 0.15, watch_steps: int = 10,
                 max_recoveries: int = 3):
        self.save_within = save_within
        self.rise_above = rise_above
        self.watch_steps = watch_steps
        self.max_recoveries = max_recoveries
        self.step = 0                 # index of the next observed step
        self.has_checkpoint = False
        self.checkpoint_loss = 0.0
        self.checkpoint_step = -1     # step whose rows the checkpoint holds
        self.min_loss = math.inf
        self.min_step = -1            # step whose rows the minimum's copy holds
        self.watch_left = 0
        self.recoveries = 0

    def _accept(self) -> int:
        self.has_checkpoint = True
        self.checkpoint_loss = self.min_loss
        self.checkpoint_step = self.min_step
        return PROMOTE

    def observe(self, loss: float) -> int:
        """Returns the action bits for the step whose loss is ``loss``."""
        x = float(loss)
        if not math.isfinite(x):
            x = math.inf
        k = self.step
        self.step += 1
        act = 0
        # reading 3: the end of an open watch
        if self.watch_left > 0:
            self.watch_left -= 1
            if self.watch_left == 0:
                if x > (1.0 + self.rise_above) * self.min_loss and self.recoveries < self.max_recoveries:
                    self.recoveries += 1
                    self.watch_left = self.watch_steps
                    return RESTORE
                act |= self._accept()
        # reading 2: a new minimum (accepting a minimum still being watched)
        if x < self.min_loss:
            if self.watch_left > 0:
                act |= self._accept()
            self.min_loss = x
            self.min_step = k
            self.watch_left = self.watch_steps
            self.recoveries = 0
            act |= SAVE_MIN
        # reading 5: the refresh
        if x != math.inf:
            if not self.has_checkpoint:
                take = True
            else:
                take = (self.watch_left == 0 and x <= (1.0 + self.save_within) * self.checkpoint_loss
                        and x <= (1.0 + self.rise_above) * self.min_loss)
            if take:
                self.has_checkpoint = True
                self.checkpoint_loss = x
                self.checkpoint_step = k
                act |= SAVE
        return act


class RowCopy:
    """The saved rows of one matrix: row k belongs to rows[k]."""

    def __init__(self, q, s, delta, m, v, t, e):
        self.q, self.s, self.delta, self.m, self.v, self.t, self.e = q, s, delta, m, v, t, e


def rows_save(st, rows, slot) -> RowCopy:
    """Copies rows (q, s, delta) and the moment slots (m, v, t and the
    moments' exponents) of a matrix state (an ``oracle.MatState``)."""
    rows = np.asarray(rows, np.int64)
    slot = np.asarray(slot, np.int64)
    return RowCopy(st.q[rows].copy(), st.s[rows].copy(), st.delta[rows].copy(), st.m[slot].copy(),
                   st.v[slot].copy(), st.t[slot].copy(), st.e[slot].copy())


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
    st.e[slot] = ck.e
    if st.w_live is not None:
        oracle.masked_writeback(st.q, st.s, st.delta, rows.astype(np.int32), st.w_live)
