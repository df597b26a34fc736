"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test checks an oracle function against something other than the oracle
itself: a closed form the method implies, a library routine (numpy, torch),
brute force on tiny inputs, or an invariant that a plausible slip (a dropped
term, a wrong sign or index, a transposed operand) would break.

Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
Active Set", sections 2.1 (conductor/tracker), 2.2 (masked dW), 2.3 (int8 +
residual state, fp16 moments) and 2.4 (Adam with bias correction; coupled
pairs).  Adam as in Kingma and Ba, restated in the SparseLeaf post, section 4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_full_weight_amd import synth

# ---------------------------------------------------------------- formats


def test_f16_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = oracle.f16_to_f32(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_to_f32(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))


def _conversion_probe_values():
    g = synth.rng(7)
    parts = [
        g.standard_normal(200000).astype(np.float32) * np.float32(1e-3),
        g.standard_normal(200000).astype(np.float32) * np.float32(10.0),
        (g.uniform(-1, 1, 100000) * 2.0 ** -20).astype(np.float32),      # fp16 subnormal range
        (g.uniform(-1, 1, 100000) * 2.0 ** -126).astype(np.float32),     # fp32 subnormal range
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8],
                 np.float32),
    ]
    # exact ties between neighbouring fp16 values: midpoints have one extra bit
    h = g.integers(0, 0x7bff, 50000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    return np.concatenate(parts)


def test_f16_encode_vs_numpy():
    x = _conversion_probe_values()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(x), ref)


def test_bf16_encode_vs_torch():
    x = _conversion_probe_values()
    g = synth.rng(8)
    # ties between neighbouring bf16 values
    b = g.integers(0, 0x7f00, 50000).astype(np.uint32)
    mid = ((b << 16) | 0x8000).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, mid, -mid])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), ref)


# ---------------------------------------------------------------- section 2.1 conductor


def test_conductor_busiest_row_closed_form():
    # The busiest row's share is exactly 1 in every window, so from zero the
    # charge after n windows is 1 - 2^-n exactly (all operations exact).
    ch = np.zeros(3, np.float32)
    for n in range(1, 25):
        act = oracle.conductor_window(ch, [0, 0, 1])
        assert ch[0] == np.float32(1.0 - 2.0 ** -n)
        assert act[0] == 1


def test_conductor_share_is_hits_over_busiest():
    ch = np.zeros(4, np.float32)
    act = oracle.conductor_window(ch, [0, 0, 0, 1, 2, 2])
    # hits 3, 1, 2, 0; busiest 3 -> shares 1, 1/3, 2/3, 0; charge = share / 2
    assert ch[0] == np.float32(0.5)
    assert ch[1] == np.float32(0.5) * np.float32(np.float32(1) / np.float32(3))
    assert ch[2] == np.float32(0.5) * np.float32(np.float32(2) / np.float32(3))
    assert ch[3] == 0.0
    assert act.tolist() == [1, 1, 1, 0]


def test_conductor_silent_row_fades_after_six_windows():
    # A row at full charge that is never seen again halves every window:
    # 2^-6 = 0.0156 >= 0.01 > 2^-7, so it stays active exactly six windows.
    ch = np.array([1.0, 0.0], np.float32)
    states = []
    for n in range(1, 9):
        act = oracle.conductor_window(ch, [1])
        assert ch[0] == np.float32(2.0 ** -n)
        states.append(int(act[0]))
    assert states == [1, 1, 1, 1, 1, 1, 0, 0]


def test_conductor_constant_share_closed_form():
    # At a constant share sigma the charge tends to sigma: ch_n = sigma (1 - 2^-n).
    ch = np.zeros(2, np.float32)
    for n in range(1, 20):
        oracle.conductor_window(ch, [0, 0, 0, 0, 1])  # row 1 share = 1/4
        want = 0.25 * (1 - 2.0 ** -n)
        assert abs(float(ch[1]) - want) <= 4 * np.spacing(np.float32(want))


def test_conductor_threshold_inclusive_and_empty_window():
    ch = np.array([0.02, 0.0200001, 0.5], np.float32)
    act = oracle.conductor_window(ch, [])  # empty window: charges only halve
    assert ch[0] == np.float32(0.01) and act[0] == 1  # 0.01f >= 0.01f
    assert ch[2] == np.float32(0.25)


def test_conductor_relabel_equivariance():
    g = synth.rng(3)
    toks = synth.zipf_tokens(2000, 300, 1.1, 4)
    perm = g.permutation(300).astype(np.int32)
    ch1 = np.zeros(300, np.float32)
    ch2 = np.zeros(300, np.float32)
    for w in range(3):
        t = toks[w * 600:(w + 1) * 600]
        a1 = oracle.conductor_window(ch1, t)
        a2 = oracle.conductor_window(ch2, perm[t])
        assert np.array_equal(ch2[perm], ch1)
        assert np.array_equal(a2[perm], a1)


def test_conductor_rejects_bad_token():
    with pytest.raises(ValueError):
        oracle.conductor_window(np.zeros(4, np.float32), [0, 4])


def test_tracker_matches_conductor_on_counts():
    # The tracker applies the same recurrence to magnitudes: feeding it hit
    # counts as magnitudes must reproduce the conductor exactly.
    toks = synth.zipf_tokens(3000, 500, 1.1, 11)
    ch1 = np.zeros(500, np.float32)
    ch2 = np.zeros(500, np.float32)
    for w in range(3):
        t = toks[w * 1000:(w + 1) * 1000]
        a1 = oracle.conductor_window(ch1, t)
        a2 = oracle.tracker_window(ch2, np.bincount(t, minlength=500).astype(np.float32))
        assert np.array_equal(ch1, ch2) and np.array_equal(a1, a2)


def test_tracker_seeded_magnitudes_give_exact_k():
    R, k = 4096, 41
    hot = synth.clustered_rows(R, k, 5)
    a = synth.tracker_magnitudes(R, hot, 6)
    act = oracle.tracker_window(np.zeros(R, np.float32), a)
    assert np.array_equal(np.nonzero(act)[0], hot)


# ---------------------------------------------------------------- plans


@pytest.mark.parametrize("R", [1, 31, 32, 33, 100, 512, 4096, 11008])
def test_plan_round_trip(R):
    g = synth.rng(R)
    mask = (g.random(R) < 0.07).astype(np.uint8)
    mask[-1] = 1                       # the last (possibly one-row) tile is active
    p = oracle.plan_rows(mask)
    back = np.zeros(R, np.uint8)
    for j, w in enumerate(p["bits"]):
        for i in range(32):
            if (int(w) >> i) & 1:
                back[32 * j + i] = 1
    assert np.array_equal(back, mask)
    assert np.array_equal(p["active_rows"], np.nonzero(mask)[0])
    assert np.array_equal(p["active_tiles"], np.nonzero(p["bits"])[0])
    assert p["bits"].size == (R + 31) // 32


def test_plan_embedding_vs_nonzero():
    toks = synth.zipf_tokens(4096, 1000, 1.1, 2)
    rows = np.array([0, 1, 5, 17, 999, 500], np.int32)
    rows.sort()
    row_ptr, pos = oracle.plan_embedding(rows, toks)
    for k, r in enumerate(rows):
        assert np.array_equal(pos[row_ptr[k]:row_ptr[k + 1]], np.nonzero(toks == r)[0])


def test_slots_assignment_rules():
    R, n_slots = 10, 4
    rs = np.full(R, -1, np.int32)
    slot, fresh = oracle.slots_update(rs, n_slots, [1, 3, 7])
    assert slot.tolist() == [0, 1, 2] and fresh.tolist() == [1, 1, 1]
    # 3 leaves (frees slot 1), 7 stays (keeps 2), 2 and 9 arrive (lowest free: 0? no, 1 rows)
    slot, fresh = oracle.slots_update(rs, n_slots, [1, 2, 7, 9])
    assert slot.tolist() == [0, 1, 2, 3]
    assert fresh.tolist() == [0, 1, 0, 1]
    assert rs[3] == -1 and rs[1] == 0 and rs[7] == 2
    with pytest.raises(ValueError):
        oracle.slots_update(rs, n_slots, [0, 1, 2, 3, 4])


def test_slots_random_invariants():
    g = synth.rng(99)
    R, n_slots = 200, 40
    rs = np.full(R, -1, np.int32)
    prev = {}
    for step in range(30):
        rows = np.sort(g.choice(R, size=int(g.integers(0, n_slots + 1)), replace=False)).astype(np.int32)
        slot, fresh = oracle.slots_update(rs, n_slots, rows)
        assert len(set(slot.tolist())) == rows.size          # distinct slots
        for r, s_, f in zip(rows, slot, fresh):
            if r in prev:
                assert s_ == prev[r] and f == 0                  # kept while active
            else:
                assert f == 1
        prev = {int(r): int(s_) for r, s_ in zip(rows, slot)}


# ---------------------------------------------------------------- section 2.2 masked dW


def _f32(bits):
    return oracle.bf16_to_f32(bits)


def test_masked_dw_vs_numpy_float64():
    T, R, Cc = 37, 70, 24
    dY = synth.normal_bf16((T, R), 0.01, 1)
    X = synth.normal_bf16((T, Cc), 1.0, 2)
    rows = np.array([0, 3, 31, 32, 64, 69], np.int32)
    got = oracle.masked_dw(dY, X, rows)
    ref = (_f32(dY)[:, rows].astype(np.float64).T @ _f32(X).astype(np.float64)).astype(np.float32)
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(got - ref) <= ulp)


def test_masked_dw_integer_inputs_exact():
    T, R, Cc = 64, 40, 16
    dY = synth.integer_bf16((T, R), -3, 3, 5)
    X = synth.integer_bf16((T, Cc), -3, 3, 6)
    rows = np.arange(0, 40, 3, dtype=np.int32)
    got = oracle.masked_dw(dY, X, rows)
    ref = (_f32(dY)[:, rows].astype(np.int64).T @ _f32(X).astype(np.int64)).astype(np.float32)
    assert np.array_equal(got, ref)


def test_masked_dw_single_token_is_outer_product():
    # One token: dW is the outer product of dY and X (SparseLeaf post,
    # Appendix B); a bf16 x bf16 product is exact in fp32.
    dY = synth.normal_bf16((1, 50), 0.01, 7)
    X = synth.normal_bf16((1, 8), 1.0, 8)
    rows = np.array([2, 9, 40], np.int32)
    got = oracle.masked_dw(dY, X, rows)
    ref = np.outer(_f32(dY)[0, rows], _f32(X)[0]).astype(np.float32)
    assert np.array_equal(got, ref)


def test_masked_dw_linear_and_full_mask():
    T, R, Cc = 20, 33, 8
    dY = synth.normal_bf16((T, R), 0.01, 9)
    X = synth.normal_bf16((T, Cc), 1.0, 10)
    allrows = np.arange(R, dtype=np.int32)
    full = oracle.masked_dw(dY, X, allrows)
    sub = oracle.masked_dw(dY, X, allrows[5:9])
    assert np.array_equal(full[5:9], sub)
    dY2 = synth.to_bf16_bits(_f32(dY) * 2)      # exact power-of-two scaling
    assert np.array_equal(oracle.masked_dw(dY2, X, allrows), full * 2)
    assert oracle.masked_dw(dY, X, np.zeros(0, np.int32)).shape == (0, Cc)


def test_embedding_dw_vs_onehot_product():
    T, V, d = 300, 50, 16
    toks = synth.zipf_tokens(T, V, 1.1, 12)
    dY = synth.normal_bf16((T, d), 0.01, 13)
    rows = np.array([0, 1, 2, 7, 49], np.int32)
    got = oracle.embedding_dw(dY, toks, rows)
    onehot = np.zeros((T, V), np.float64)
    onehot[np.arange(T), toks] = 1.0
    ref = (onehot.T @ _f32(dY).astype(np.float64))[rows].astype(np.float32)
    assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref)))
    dYi = synth.integer_bf16((T, d), -3, 3, 14)
    got = oracle.embedding_dw(dYi, toks, rows)
    ref = (onehot.T @ _f32(dYi).astype(np.float64))[rows].astype(np.float32)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- sections 2.3-2.4 update

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)


def _state(R, Cc, seed, n_slots, mid_run):
    q, s, delta = synth.quant_state(R, Cc, seed)
    m, v, t, e = synth.moments(n_slots, Cc, seed + 1, mid_run)
    w_live = np.full((R, Cc), 0xA5A5, np.uint16)
    return oracle.MatState(q, s, delta, m, v, t, w_live, e=e)


def _rebuild(st):
    """w = s*q + delta in fp32 with two roundings (numpy, no FMA)."""
    sq = (st.s[:, None] * st.q.astype(np.float32)).astype(np.float32)
    return (sq + st.delta).astype(np.float32)


def _torch_adam(w0, g, m0, v0, step0, wd=0.0, **hp):
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    cls = torch.optim.AdamW if wd else torch.optim.Adam
    opt = cls([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=wd,
              foreach=False)
    p.grad = torch.from_numpy(g.copy())
    if step0:
        opt.state[p] = {"step": torch.tensor(float(step0)), "exp_avg": torch.from_numpy(m0.copy()),
                        "exp_avg_sq": torch.from_numpy(v0.copy())}
    opt.step()
    st = opt.state[p]
    return p.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()


def _check_quantised(st, rows):
    """The stored (q, s, delta) of each row is a canonical quantisation of
    w = s*q + delta: s = max|w|/127, every code a nearest integer of w/s (up
    to the rounding of the reciprocal scale near a .5 tie: within 1/2 + 2^-16,
    in fp64), the largest code 127, and delta = w - s*q with |delta| at most
    s/2 plus that slack and one ulp of w."""
    w = _rebuild(st)
    for r in rows:
        amax = np.max(np.abs(w[r]))
        assert st.s[r] == np.float32(amax / np.float32(127.0))
        if st.s[r] == 0:
            assert not st.q[r].any()
            continue
        assert np.max(np.abs(st.q[r].astype(np.int32))) == 127
        x = w[r].astype(np.float64) / np.float64(st.s[r])
        assert np.all(np.abs(x - st.q[r]) <= 0.5 + 2.0 ** -16)
        assert np.all((np.abs(x) <= 127.5) | (np.abs(st.q[r]) == 127))
        bound = np.float64(st.s[r]) * (0.5 + 2.0 ** -16) + np.spacing(np.abs(w[r]))
        assert np.all(np.abs(st.delta[r]) <= bound)
    return w


@pytest.mark.parametrize("mid_run", [False, True])
def test_update_matches_torch_adam(mid_run):
    R, Cc = 96, 64
    rows = np.array([3, 4, 40, 95], np.int32)
    n_slots = 6
    st = _state(R, Cc, 21, n_slots, mid_run)
    slot = np.array([5, 0, 2, 3], np.int32)
    G = synth.gradient_rows(rows.size, Cc, 0.16, 22)
    before = st.copy()
    w0 = _rebuild(before)
    oracle.sparse_update(st, G, rows, slot, None, **HP)
    w1 = _check_quantised(st, rows)
    m_before, v_before = before.moments()
    m_after, v_after = st.moments()
    for k, r in enumerate(rows):
        sl = slot[k]
        wt, mt, vt = _torch_adam(w0[r], G[k], m_before[sl], v_before[sl], int(before.t[sl]), **HP)
        tol = 2 * np.spacing(np.abs(wt)) + 1e-6 * HP["lr"]
        assert np.all(np.abs(w1[r] - wt) <= tol)
        # stored moments: torch's fp32 moments as fp16 rows scaled by 2^e (1 ulp
        # of the scaled fp16 value as slack for torch's operation order)
        for got, want, e in ((m_after[sl], mt, st.e[sl, 0]), (v_after[sl], vt, st.e[sl, 1])):
            scaled = np.abs(want.astype(np.float64)) * 2.0 ** int(e)
            ulp = (np.spacing(scaled.astype(np.float16)).astype(np.float64) + 2 ** -24) * 2.0 ** -int(e)
            assert np.all(np.abs(got.astype(np.float64) - want) <= ulp)
        assert st.t[sl] == before.t[sl] + 1
        assert np.array_equal(st.w_live[r], synth.to_bf16_bits(w1[r]))


def test_update_first_step_moves_by_lr_against_gradient():
    # From zero moments at t = 1, mhat = g and vhat = g^2 (to rounding), so every
    # element moves by lr * |g| / (|g| + eps) against the sign of its gradient.
    R, Cc = 64, 128
    rows = np.array([7, 33], np.int32)
    st = _state(R, Cc, 31, 2, False)
    G = synth.gradient_rows(2, Cc, 0.16, 32)
    w0 = _rebuild(st)
    oracle.sparse_update(st, G, rows, np.array([0, 1], np.int32), None, **HP)
    w1 = _rebuild(st)
    for k, r in enumerate(rows):
        step = (w0[r] - w1[r]).astype(np.float64)
        want = HP["lr"] * G[k] / (np.abs(G[k]) + HP["eps"])
        assert np.all(np.abs(step - want) <= 1e-5 * HP["lr"] + 2 * np.spacing(np.abs(w0[r])))


def test_update_decoupled_weight_decay_matches_adamw():
    R, Cc = 40, 32
    rows = np.array([1, 38], np.int32)
    st = _state(R, Cc, 41, 2, True)
    G = synth.gradient_rows(2, Cc, 0.1, 42)
    before = st.copy()
    w0 = _rebuild(before)
    wd = 0.01 * math.cos(math.radians(28.4))
    oracle.sparse_update(st, G, rows, np.array([0, 1], np.int32), None, weight_decay=wd, **HP)
    w1 = _rebuild(st)
    m_before, v_before = before.moments()
    for k, r in enumerate(rows):
        wt, _, _ = _torch_adam(w0[r], G[k], m_before[k], v_before[k], int(before.t[k]), wd=wd, **HP)
        assert np.all(np.abs(w1[r] - wt) <= 2 * np.spacing(np.abs(wt)) + 1e-6 * HP["lr"])


def test_update_decay_order_at_large_step():
    # With lr * lambda = 0.1 the order of decay and step is visible: AdamW
    # shrinks the weight first, then subtracts the Adam step.
    R, Cc = 32, 64
    rows = np.array([4], np.int32)
    st = _state(R, Cc, 45, 1, False)
    G = synth.gradient_rows(1, Cc, 0.1, 46)
    hp = dict(HP, lr=0.05)
    w0 = _rebuild(st)
    oracle.sparse_update(st, G, rows, np.array([0], np.int32), None, weight_decay=2.0, **hp)
    wt, _, _ = _torch_adam(w0[4], G[0], None, None, 0, wd=2.0, **hp)
    w1 = _rebuild(st)[4]
    assert np.all(np.abs(w1 - wt) <= 4 * np.spacing(np.abs(wt)))


def test_update_leaves_inactive_rows_and_slots_untouched():
    R, Cc = 100, 48
    rows = np.array([10, 11, 50], np.int32)
    st = _state(R, Cc, 51, 8, True)
    before = st.copy()
    G = synth.gradient_rows(3, Cc, 0.1, 52)
    oracle.sparse_update(st, G, rows, np.array([1, 4, 6], np.int32), None, **HP)
    others = np.setdiff1d(np.arange(R), rows)
    for a, b in ((st.q, before.q), (st.delta, before.delta), (st.w_live, before.w_live)):
        assert np.array_equal(a[others], b[others])
    assert np.array_equal(st.s[others], before.s[others])
    free = np.setdiff1d(np.arange(8), [1, 4, 6])
    assert np.array_equal(st.m[free], before.m[free]) and np.array_equal(st.v[free], before.v[free])
    assert np.array_equal(st.t[free], before.t[free]) and np.array_equal(st.e[free], before.e[free])


def test_update_fresh_slot_ignores_stale_moments():
    R, Cc = 32, 16
    rows = np.array([5], np.int32)
    a = _state(R, Cc, 61, 1, True)       # stale garbage moments, t = 6
    b = a.copy()
    b.m[:] = 0
    b.v[:] = 0
    b.t[:] = 0
    b.e[:] = 0
    G = synth.gradient_rows(1, Cc, 0.1, 62)
    oracle.sparse_update(a, G, rows, np.array([0], np.int32), np.array([1], np.uint8), **HP)
    oracle.sparse_update(b, G, rows, np.array([0], np.int32), None, **HP)
    for x, y in ((a.q, b.q), (a.s, b.s), (a.delta, b.delta), (a.m, b.m), (a.v, b.v), (a.t, b.t), (a.e, b.e)):
        assert np.array_equal(x, y)


def test_update_zero_row_edge():
    R, Cc = 32, 16
    st = _state(R, Cc, 71, 1, False)
    st.q[3] = 0
    st.delta[3] = 0
    oracle.sparse_update(st, np.zeros((1, Cc), np.float32), np.array([3], np.int32),
                         np.array([0], np.int32), None, **HP)
    assert st.s[3] == 0 and not st.q[3].any() and not st.delta[3].any()


# ---------------------------------------------------------------- scaled fp16 moment rows


def test_moment_row_maximum_lands_in_the_top_binade():
    """A stored row's largest moment is an fp16 value in [2^14, 2^15] whatever
    the row's magnitude (numpy's float16 decodes the stored bits)."""
    g = synth.rng(80)
    for amax in np.concatenate([[1.0, 2.0 ** -20, 3.0e4, 1e-30, 5e30],
                                np.exp(g.uniform(-60, 60, 200))]).astype(np.float32):
        e = oracle.moment_exponent(amax)
        h = oracle.moment_encode(np.array([amax, -amax], np.float32), e)
        top = np.abs(h.view(np.float16).astype(np.float64))
        assert np.all((2.0 ** 14 <= top) & (top <= 2.0 ** 15)), (amax, e, top)
    assert oracle.moment_exponent(0.0) == 0


def test_moment_encoding_is_fp16_of_the_power_of_two_scaled_value():
    """Encode and decode against numpy's float16 rounding of x * 2^e (round to
    nearest even), with saturation at 65504 where numpy overflows to inf."""
    g = synth.rng(81)
    x = (g.standard_normal(4000) * np.exp(g.uniform(-20, 10, 4000))).astype(np.float32)
    for e in (-30, -5, 0, 7, 19, 60):
        scaled = x.astype(np.float64) * 2.0 ** e
        with np.errstate(over="ignore"):
            want = scaled.astype(np.float16)
            want = np.where(np.isinf(want), np.copysign(np.float16(65504), scaled), want).astype(np.float16)
        got = oracle.moment_encode(x, e)
        assert np.array_equal(got, want.view(np.uint16)), e
        back = oracle.moment_decode(got, e)
        assert np.array_equal(back, (want.astype(np.float64) * 2.0 ** -e).astype(np.float32))


def _adam_fp32_displacement(g, steps, **hp):
    """Displacement of a weight row after `steps` Adam steps with fp32 moments
    (numpy, every operation rounded to fp32)."""
    f = np.float32
    b1, b2, lr, eps = f(hp["beta1"]), f(hp["beta2"]), f(hp["lr"]), f(hp["eps"])
    m = np.zeros_like(g)
    v = np.zeros_like(g)
    d = np.zeros(g.shape, np.float64)
    for t in range(1, steps + 1):
        m = b1 * m + (f(1) - b1) * g
        v = b2 * v + (f(1) - b2) * (g * g)
        bc1 = f(1.0 - float(b1) ** t)
        bc2 = f(1.0 - float(b2) ** t)
        d += lr * ((m / bc1) / (np.sqrt(v / bc2) + eps))
    return d


@pytest.mark.parametrize("gmag", [1e-5, 1e-3, 300.0])
def test_thousand_steps_follow_fp32_moment_adam(gmag):
    """With the moments stored as scaled fp16 rows, 1000 steps on a constant
    gradient move every weight within 2% of what Adam with fp32 moments moves
    it, at gradients far below and far above fp16's comfortable range (plain
    fp16 moments move the |g| = 1e-5 and 1e-3 rows about 17x too far, and
    overflow v to infinity near |g| = 300 after a few thousand steps)."""
    R, Cc, steps = 32, 64, 1000
    g = synth.rng(82)
    grad = (gmag * np.where(g.random(Cc) < 0.5, -1.0, 1.0) * g.uniform(0.5, 1.0, Cc)).astype(np.float32)
    st = _state(R, Cc, 83, 1, False)
    st.s[5] = np.float32(1.0)           # a weight row of order 1 keeps the displacement visible
    rows, slot = np.array([5], np.int32), np.array([0], np.int32)
    w0 = _rebuild(st)[5].astype(np.float64)
    for _ in range(steps):
        oracle.sparse_update(st, grad[None, :], rows, slot, None, **HP)
    got = w0 - _rebuild(st)[5].astype(np.float64)
    want = _adam_fp32_displacement(grad, steps, **HP)
    assert np.all(np.abs(got / want - 1.0) <= 0.02), (gmag, np.abs(got / want - 1.0).max())
    m, v = st.moments()
    assert np.all(np.isfinite(m)) and np.all(np.isfinite(v)) and np.all(v > 0)


def test_huge_gradient_moments_saturate_nowhere_and_stay_finite():
    R, Cc = 32, 16
    st = _state(R, Cc, 84, 1, False)
    grad = np.full((1, Cc), 3.0e4, np.float32)
    grad[0, ::2] *= -1
    for _ in range(20):
        oracle.sparse_update(st, grad, np.array([2], np.int32), np.array([0], np.int32), None, **HP)
    m, v = st.moments()
    assert np.all(np.isfinite(v)) and np.all(np.abs(v - 9.0e8 * (1 - 0.999 ** 20)) <= 1e-3 * 9.0e8)
    assert np.all(np.abs(np.abs(m) - 3.0e4 * (1 - 0.9 ** 20)) <= 1e-3 * 3.0e4)


def test_update_tiny_row_divides_when_the_reciprocal_scale_overflows():
    """A row whose new scale is below 2^-128 (its reciprocal overflows fp32)
    is quantised by division: the codes are rint(w'/s'), the largest 127, and
    the rebuild is exact."""
    R, Cc = 8, 16
    st = _state(R, Cc, 91, 1, False)
    st.q[2] = 0
    st.delta[2] = (synth.rng(92).uniform(-1, 1, Cc) * 2.0 ** -122).astype(np.float32)
    st.delta[2, 3] = np.float32(2.0 ** -122)
    w0 = _rebuild(st)[2]
    oracle.sparse_update(st, np.zeros((1, Cc), np.float32), np.array([2], np.int32), np.array([0], np.int32), None,
                         **HP)
    s2 = st.s[2]
    with np.errstate(over="ignore"):
        assert 0 < s2 < 2.0 ** -128 and np.isinf(np.float32(1.0) / s2)
    w1 = _rebuild(st)[2]
    assert np.array_equal(w1.view(np.uint32), w0.view(np.uint32))      # zero gradient: w' = w
    assert np.array_equal(st.q[2], np.rint((w0 / s2).astype(np.float32)).astype(np.int8))
    assert np.max(np.abs(st.q[2].astype(np.int32))) == 127


def test_update_step_against_float64_adam():
    """Every element's step against Adam's formula evaluated in float64 from
    the same fp32 moments (bias corrections from the same fp32 betas): within
    a few parts in 10^7 of the step, whatever order the fp32 operations take."""
    R, Cc = 16, 512
    st = _state(R, Cc, 93, 4, True)
    rows, slot = np.array([1, 5, 9, 14], np.int32), np.array([3, 1, 0, 2], np.int32)
    G = synth.gradient_rows(4, Cc, 0.3, 94)
    before = st.copy()
    w0 = _rebuild(before).astype(np.float64)
    oracle.sparse_update(st, G, rows, slot, None, **HP)
    m_old, v_old = before.moments()
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    for k, r in enumerate(rows):
        t = int(before.t[slot[k]]) + 1
        g = G[k].astype(np.float64)
        m = b1 * m_old[slot[k]] + (1 - b1) * g
        v = b2 * v_old[slot[k]] + (1 - b2) * g * g
        u = HP["lr"] * (m / (1 - b1 ** t)) / (np.sqrt(v / (1 - b2 ** t)) + HP["eps"])
        step = w0[r] - _rebuild(st)[r].astype(np.float64)
        assert np.all(np.abs(step - u) <= 4e-7 * np.abs(u) + 2 * np.spacing(np.abs(w0[r]).astype(np.float32)))


def test_bias_table_closed_form():
    bc1, bc2 = oracle.bias_table(0.9, 0.999, 40000)
    b1 = np.float32(0.9)
    assert bc1[1] == np.float32(1) - b1                    # exact (Sterbenz)
    assert np.all(np.diff(bc1[1:]) >= 0) and np.all(np.diff(bc2[1:]) >= 0)
    assert bc1[-1] == 1.0 and bc2[-1] == 1.0
    assert bc2[2] == np.float32(1 - float(np.float32(0.999)) ** 2)


# ---------------------------------------------------------------- section 2.4 coupled pairs


def _pair_inputs(seed, R=64, Cc=32):
    A = _state(R, Cc, seed, 8, True)
    B = _state(R, Cc, seed + 10, 8, True)
    ra = np.array([1, 2, 20, 40], np.int32)
    rb = np.array([2, 3, 40, 63], np.int32)
    GA = synth.gradient_rows(ra.size, Cc, 0.1, seed + 20)
    GB = synth.gradient_rows(rb.size, Cc, 0.1, seed + 21)
    sa = np.array([0, 1, 2, 3], np.int32)
    sb = np.array([4, 5, 6, 7], np.int32)
    return A, B, ra, rb, GA, GB, sa, sb


def _same(x: oracle.MatState, y: oracle.MatState):
    return all(np.array_equal(a, b) for a, b in
               ((x.q, y.q), (x.s, y.s), (x.delta, y.delta), (x.m, y.m), (x.v, y.v), (x.t, y.t),
                (x.e, y.e), (x.w_live, y.w_live)))


def test_coupled_without_cross_term_is_two_plain_updates():
    A, B, ra, rb, GA, GB, sa, sb = _pair_inputs(100)
    A2, B2 = A.copy(), B.copy()
    oracle.coupled_update(A, GA, ra, sa, None, B, GB, rb, sb, None, a_own=1.0, a_cross=0.0, **HP)
    oracle.sparse_update(A2, GA, ra, sa, None, **HP)
    oracle.sparse_update(B2, GB, rb, sb, None, **HP)
    assert _same(A, A2) and _same(B, B2)


def test_coupled_cross_only_feeds_partner_gradient():
    # a_own = 0, a_cross = 1: matrix A steps with B's gradient (zero where B is inactive).
    A, B, ra, rb, GA, GB, sa, sb = _pair_inputs(200)
    A2 = A.copy()
    oracle.coupled_update(A, GA, ra, sa, None, B, GB, rb, sb, None, a_own=0.0, a_cross=1.0, **HP)
    GfromB = np.zeros_like(GA)
    for k, r in enumerate(ra):
        hit = np.nonzero(rb == r)[0]
        if hit.size:
            GfromB[k] = GB[hit[0]]
    oracle.sparse_update(A2, GfromB, ra, sa, None, **HP)
    assert _same(A, A2)


def test_coupled_swap_symmetry_and_partner_isolation():
    A, B, ra, rb, GA, GB, sa, sb = _pair_inputs(300)
    A1, B1, A2, B2 = A.copy(), B.copy(), A.copy(), B.copy()
    kw = dict(a_own=0.8, a_cross=0.35, clip_a=0.9, clip_b=0.7, weight_decay=0.0088, **HP)
    oracle.coupled_update(A1, GA, ra, sa, None, B1, GB, rb, sb, None, **kw)
    kw2 = dict(kw, clip_a=0.7, clip_b=0.9)
    oracle.coupled_update(B2, GB, rb, sb, None, A2, GA, ra, sa, None, **kw2)
    assert _same(A1, A2) and _same(B1, B2)
    # rows active only in A leave B's rows bit-unchanged
    only_a = np.setdiff1d(ra, rb)
    for r in only_a:
        assert np.array_equal(B1.q[r], B.q[r]) and np.array_equal(B1.delta[r], B.delta[r])
        assert B1.s[r] == B.s[r]


def test_coupled_blend_direction_vs_float64():
    # At t = 1 from zero moments each element moves by ~lr against the sign of
    # its effective gradient, so the direction exposes the blend
    # a_own * clip_a * gA + a_cross * clip_b * gB element by element.
    R, Cc = 32, 256
    A = _state(R, Cc, 400, 1, False)
    B = _state(R, Cc, 410, 1, False)
    rows = np.array([9], np.int32)
    GA = synth.gradient_rows(1, Cc, 0.1, 420)
    GB = synth.gradient_rows(1, Cc, 0.1, 421)
    a_own, a_cross, ca, cb = 0.5, 0.45, 0.8, 1.0
    wa0, wb0 = _rebuild(A)[9], _rebuild(B)[9]
    oracle.coupled_update(A, GA, rows, [0], None, B, GB, rows, [0], None, a_own=a_own,
                          a_cross=a_cross, clip_a=ca, clip_b=cb, **HP)
    ea = a_own * ca * GA[0].astype(np.float64) + a_cross * cb * GB[0].astype(np.float64)
    eb = a_own * cb * GB[0].astype(np.float64) + a_cross * ca * GA[0].astype(np.float64)
    da = (wa0 - _rebuild(A)[9]).astype(np.float64)
    db = (wb0 - _rebuild(B)[9]).astype(np.float64)
    big_a = np.abs(ea) > 1e-4
    big_b = np.abs(eb) > 1e-4
    assert np.array_equal(np.sign(da[big_a]), np.sign(ea[big_a]))
    assert np.array_equal(np.sign(db[big_b]), np.sign(eb[big_b]))
    # and the blend is not the plain own gradient somewhere
    assert np.any(np.sign(ea[big_a]) != np.sign(GA[0][big_a]))


def test_writeback_rebuilds_live_rows_only():
    R, Cc = 50, 24
    q, s, delta = synth.quant_state(R, Cc, 501)
    w_live = np.full((R, Cc), 0x1234, np.uint16)
    rows = np.array([0, 17, 49], np.int32)
    oracle.masked_writeback(q, s, delta, rows, w_live)
    w = ((s[:, None] * q.astype(np.float32)).astype(np.float32) + delta).astype(np.float32)
    assert np.array_equal(w_live[rows], synth.to_bf16_bits(w[rows]))
    others = np.setdiff1d(np.arange(R), rows)
    assert np.all(w_live[others] == 0x1234)
