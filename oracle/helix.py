"""The coupled update's scalar schedule, as plain Python: loss trend, Fibonacci
stride, phase, channel weights and the two mixing coefficients of a pair.

TEST INFRASTRUCTURE ONLY: the test-suite uses this module to state what the
library's schedule calls must return.  The GPU library never imports it, and
it imports nothing from the GPU library.

Source: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
Active Set", sections 2.4 (each step a phase moves on by 36 degrees per unit
of stride and divides the update between a primary and a secondary channel,
weighted 1.833 to 1, with a slow phase term that never repeats), 2.5 (the
loss changes are averaged with exponential weights that fall off over ten
steps; a smoothed copy of that average moves the stride over the Fibonacci
numbers up to 21; slower counters vary the channel weights by 10% and 5%),
2.6 (a rewind starts the stride again at 1) and 2.8 (over a turn a pair's
mix goes from nearly its own gradient to fully coupled).  The
page's equations are lost; the readings taken here are:
  1. trend C_t = sum_i r^i dL_{t-i} / sum_i r^i over the steps seen so far,
     r = exp(-1/10), dL_t = L_{t-1} - L_t (positive while the loss falls); no
     change is recorded for the first loss;
  2. the smoothed trend is the same mean taken over the series of C;
  3. each step the rung goes up by one (at most to 21) if the smoothed trend
     is above `up_threshold`, down by one (at least to the first 1) if it is
     below zero, and otherwise stays; a rewind puts it back on the first rung
     instead; the stride is the rung's Fibonacci number;
  4. the rotation grows by 36 degrees times the stride; the phase is the
     rotation modulo 360;
  5. channel weights w+ = 1 + 0.10 cos(2 pi R / 360), w- = 1 + 0.05 cos(2 pi R /
     3600) for the accumulated rotation R in degrees (periods of one and of
     ten turns);
  6. exposure e = (1 + cos(phase + psi)) / 2 with psi the slow phase term (an
     input: the page's elliptic-curve walk is not specified), a_own = 1 and
     a_cross = b mu w- (1 - e) / (M w+ e + mu w- (1 - e)), M : mu = 1.833 : 1;
  7. all arithmetic in double precision.

Parity unpinned: the page prints none of these formulas' values, so readings
1-6 are checked only by their invariants (closed forms of the trend, the
ladder's moves, the turn's sweep of the blend from 0 to b, the bounds of the
weights) and by section 2.8's statement that the 1.833 : 1 weighting keeps
descent dominant, not by a printed number.
"""
from __future__ import annotations

import math

FIB = (1, 1, 2, 3, 5, 8, 13, 21)


class Helix:
    def __init__(self, decay_len: float = 10.0, up_threshold: float = 1e-4, rung_deg: float = 36.0,
                 M: float = 1.833, mu: float = 1.0, mod_plus: float = 0.10, mod_minus: float = 0.05):
        self.decay_len = decay_len
        self.up_threshold = up_threshold
        self.rung_deg = rung_deg
        self.M, self.mu = M, mu
        self.mod_plus, self.mod_minus = mod_plus, mod_minus
        self.trend_sum = self.trend_w = 0.0
        self.smooth_sum = self.smooth_w = 0.0
        self.last_loss = 0.0
        self.has_loss = False
        self.rung = 0
        self.rotation = 0.0

    @property
    def trend(self) -> float:
        return self.trend_sum / self.trend_w if self.trend_w > 0.0 else 0.0

    @property
    def smooth(self) -> float:
        return self.smooth_sum / self.smooth_w if self.smooth_w > 0.0 else 0.0

    @property
    def stride(self) -> int:
        return FIB[self.rung]

    @property
    def phase(self) -> float:
        return math.fmod(self.rotation, 360.0)

    def step(self, loss: float, rewind: bool = False) -> None:
        r = math.exp(-1.0 / self.decay_len)
        x = float(loss)
        if self.has_loss:
            d = self.last_loss - x
            self.trend_sum = d + r * self.trend_sum
            self.trend_w = 1.0 + r * self.trend_w
            self.smooth_sum = self.trend + r * self.smooth_sum
            self.smooth_w = 1.0 + r * self.smooth_w
        self.last_loss = x
        self.has_loss = True
        if rewind:
            self.rung = 0
        elif self.smooth > self.up_threshold:
            self.rung = min(self.rung + 1, len(FIB) - 1)
        elif self.smooth < 0.0:
            self.rung = max(self.rung - 1, 0)
        self.rotation += self.rung_deg * self.stride

    def weights(self):
        R = self.rotation
        wp = 1.0 + self.mod_plus * math.cos(2.0 * math.pi * R / 360.0)
        wm = 1.0 + self.mod_minus * math.cos(2.0 * math.pi * R / 3600.0)
        return wp, wm

    def coupling(self, b: float, psi_deg: float = 0.0):
        """(a_own, a_cross) of a pair with coupling strength b."""
        e = (1.0 + math.cos(math.radians(self.phase + psi_deg))) / 2.0
        wp, wm = self.weights()
        sec = self.mu * wm * (1.0 - e)
        return 1.0, b * sec / (self.M * wp * e + sec)
