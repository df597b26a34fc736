"""The library's coupled-update schedule (host code, sections 2.4-2.6 and 2.8
of "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the Active
Set") against the oracle: on seeded loss runs with plateaus, spikes and
rewinds every stride, phase, coupling coefficient and state field must be
the same double (both sides evaluate the same expressions in the same order
with the same C math library)."""
import math

import numpy as np
import pytest

from oracle import helix as hx
from sparse_full_weight_amd import _lib


def _losses(seed, n):
    g = np.random.default_rng(seed)
    x, out = 8.0, []
    for k in range(n):
        phase = (k // 200) % 3          # descent, plateau, rise
        drift = (-0.01, 0.0, 0.004)[phase]
        x = max(0.05, x * math.exp(drift + g.normal(0, 0.01)))
        out.append(x * (1.0 + (g.random() < 0.03) * g.uniform(0.1, 0.5)))
    return out


@pytest.mark.parametrize("seed", [1, 2])
def test_library_schedule_matches_oracle(seed):
    o = hx.Helix()
    c = _lib.Helix()
    g = np.random.default_rng(seed + 100)
    for x in _losses(seed, 1500):
        rw = bool(g.random() < 0.01)
        o.step(x, rewind=rw)
        stride, phase = c.step(x, rewind=rw)
        assert stride == o.stride and phase == o.phase
        for b in (0.6, 0.4):
            psi = float(g.uniform(-5, 5))
            assert c.coupling(b, psi) == o.coupling(b, psi)
        st = c.st
        assert (st.trend_sum, st.trend_w, st.smooth_sum, st.smooth_w, st.rotation, st.rung) == \
            (o.trend_sum, o.trend_w, o.smooth_sum, o.smooth_w, o.rotation, o.rung)


def test_library_schedule_rejects_bad_input():
    c = _lib.Helix()
    with pytest.raises(_lib.SftError):
        c.step(float("nan"))
    with pytest.raises(_lib.SftError):
        c.coupling(float("inf"))
    c.st.mu = 0.0
    with pytest.raises(_lib.SftError):
        c.coupling(0.6)
