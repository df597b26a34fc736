"""GPU parity of the sparse update, the coupled update and the write-back.

The HIP kernels and the oracle receive the same state and the same gradient
rows; every stored result (q, s, delta, fp16 m and v, step counts, live bf16
weights) must match bit for bit, and rows outside the list must keep their
canary bytes.  Method: "Sparse-First Fine-Tuning: Full-Weight Training at the
Cost of the Active Set", sections 2.3 (int8 + residual state, fp16 moments
for active rows, sparse write-back) and 2.4 (Adam with bias correction,
coupled pairs).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_full_weight_amd import _lib, synth
from tests.gpu_helpers import GpuMat, adam_dev, assert_state_equal, dev, make_state

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)


def _case(R, C, n_rows, n_slots, seed, mid_run, fresh_frac=0.0, gstd=0.16):
    g = synth.rng(seed)
    st = make_state(R, C, seed, n_slots, mid_run)
    rows = np.sort(g.choice(R, size=n_rows, replace=False)).astype(np.int32)
    slot = g.choice(n_slots, size=n_rows, replace=False).astype(np.int32)
    fresh = (g.random(n_rows) < fresh_frac).astype(np.uint8) if fresh_frac else None
    G = synth.gradient_rows(n_rows, C, gstd, seed + 7)
    return st, rows, slot, fresh, G


@pytest.mark.parametrize("mid_run", [False, True])
def test_sparse_update_bit_exact_many_shapes(gpu_lib, mid_run):
    # one launch over matrices of several widths: exercises every chunk count
    shapes = [(512, 512, 51), (40, 8, 5), (33, 24, 33), (300, 4096, 7), (64, 11008, 3), (50, 6000, 4)]
    cases = [_case(R, C, n, n + 3, 100 + i, mid_run, fresh_frac=0.3 if mid_run else 0.0)
             for i, (R, C, n) in enumerate(shapes)]
    gm = [GpuMat(st, G, rows, slot, fresh) for st, rows, slot, fresh, G in cases]
    hp = adam_dev(**HP)
    _lib.sft_sparse_update([m.upd() for m in gm], hp)
    torch.cuda.synchronize()
    for i, ((st, rows, slot, fresh, G), m) in enumerate(zip(cases, gm)):
        want = st.copy()
        oracle.sparse_update(want, G, rows, slot, fresh, **HP)
        assert_state_equal(m.to_state(), want, f"shape {shapes[i]}")


def test_sparse_update_two_rows_per_workgroup(gpu_lib):
    # more rows than CUs with one row wider than 4096 columns: rows of up to
    # 8192 columns go two to a 1024-lane workgroup (odd counts leave a
    # workgroup's second half without a row)
    shapes = [(64, 6000, 21), (700, 4096, 301), (300, 2048, 33)]
    cases = [_case(R, C, n, n + 5, 900 + i, True, fresh_frac=0.2) for i, (R, C, n) in enumerate(shapes)]
    gm = [GpuMat(st, G, rows, slot, fresh) for st, rows, slot, fresh, G in cases]
    _lib.sft_sparse_update([m.upd() for m in gm], adam_dev(**HP))
    torch.cuda.synchronize()
    for i, ((st, rows, slot, fresh, G), m) in enumerate(zip(cases, gm)):
        want = st.copy()
        oracle.sparse_update(want, G, rows, slot, fresh, **HP)
        assert_state_equal(m.to_state(), want, f"shape {shapes[i]}")


@pytest.mark.parametrize("C", [20000, 40000, 65536])
def test_sparse_update_wide_rows(gpu_lib, C):
    st, rows, slot, fresh, G = _case(6, C, 3, 3, 200 + C, True)
    m = GpuMat(st, G, rows, slot, fresh)
    _lib.sft_sparse_update([m.upd()], adam_dev(**HP))
    torch.cuda.synchronize()
    want = st.copy()
    oracle.sparse_update(want, G, rows, slot, fresh, **HP)
    assert_state_equal(m.to_state(), want, f"C={C}")


def test_sparse_update_weight_decay_and_no_writeback(gpu_lib):
    st, rows, slot, fresh, G = _case(96, 256, 20, 24, 300, True)
    wd = float(np.float32(0.01 * math.cos(math.radians(28.4))))
    m = GpuMat(st, G, rows, slot, fresh, with_live=False)
    empty = GpuMat(make_state(32, 64, 301, 2, False), np.zeros((0, 64), np.float32), np.zeros(0, np.int32),
                   np.zeros(0, np.int32), None)
    _lib.sft_sparse_update([empty.upd(), m.upd()], adam_dev(weight_decay=wd, **HP))
    torch.cuda.synchronize()
    want = st.copy()
    want.w_live = None
    oracle.sparse_update(want, G, rows, slot, fresh, weight_decay=wd, **HP)
    got = m.to_state()
    assert_state_equal(got, want, "wd")


def test_sparse_update_second_step_and_large_lr(gpu_lib):
    # Two consecutive steps (t goes 1 -> 2) with a step size that moves rows far.
    st, rows, slot, fresh, G = _case(128, 128, 16, 16, 400, False)
    hp = dict(HP, lr=0.05)
    m = GpuMat(st, G, rows, slot, fresh)
    want = st.copy()
    for step in range(2):
        Gs = synth.gradient_rows(rows.size, 128, 0.5, 410 + step)
        m.G.copy_(dev(Gs))
        _lib.sft_sparse_update([m.upd()], adam_dev(**hp))
        oracle.sparse_update(want, Gs, rows, slot, fresh, **hp)
    torch.cuda.synchronize()
    assert_state_equal(m.to_state(), want, "two steps")


@pytest.mark.parametrize("C", [64, 8200])
def test_sparse_update_zero_row(gpu_lib, C):
    # an all-zero row keeps a zero scale (at 8200 columns also through the
    # piecewise update and its requantisation)
    st, rows, slot, fresh, G = _case(32, C, 2, 2, 500, False)
    st.q[rows[0]] = 0
    st.delta[rows[0]] = 0
    G[0] = 0
    m = GpuMat(st, G, rows, slot, fresh)
    _lib.sft_sparse_update([m.upd()], adam_dev(**HP))
    torch.cuda.synchronize()
    want = st.copy()
    oracle.sparse_update(want, G, rows, slot, fresh, **HP)
    assert_state_equal(m.to_state(), want, "zero row")


@pytest.mark.parametrize("C", [512, 8200, 11008])
def test_coupled_update_bit_exact(gpu_lib, C):
    # 8200 and 11008 columns go in 4096-column pieces (the last one 8 and 2816
    # columns wide) and a separate requantisation
    R = 200
    g = synth.rng(600)
    pairs_np = []
    for pi, (a_own, a_cross) in enumerate([(1.0, 0.0), (0.9, 0.37), (0.0, 1.0)]):
        A = make_state(R, C, 610 + pi, 40, True)
        B = make_state(R, C, 620 + pi, 40, True)
        ra = np.sort(g.choice(R, 25, replace=False)).astype(np.int32)
        rb = np.sort(np.unique(np.concatenate([ra[:10], g.choice(R, 15, replace=False)]))).astype(np.int32)
        sa = g.choice(40, ra.size, replace=False).astype(np.int32)
        sb = g.choice(40, rb.size, replace=False).astype(np.int32)
        fa = (g.random(ra.size) < 0.2).astype(np.uint8)
        GA = synth.gradient_rows(ra.size, C, 0.2, 630 + pi)
        GB = synth.gradient_rows(rb.size, C, 0.2, 640 + pi)
        clip = np.array([0.75, 1.0], np.float32) if pi == 1 else None
        pairs_np.append((A, B, ra, rb, sa, sb, fa, GA, GB, a_own, a_cross, clip))
    wd = float(np.float32(0.01 * math.cos(math.radians(28.4))))
    gpu_pairs, mats = [], []
    for A, B, ra, rb, sa, sb, fa, GA, GB, a_own, a_cross, clip in pairs_np:
        ma, mb = GpuMat(A, GA, ra, sa, fa), GpuMat(B, GB, rb, sb, None)
        mats.append((ma, mb))
        gpu_pairs.append(_lib.Pair(ma.upd(), mb.upd(), a_own, a_cross, None if clip is None else dev(clip)))
    _lib.sft_coupled_update(gpu_pairs, adam_dev(weight_decay=wd, **HP))
    torch.cuda.synchronize()
    for (A, B, ra, rb, sa, sb, fa, GA, GB, a_own, a_cross, clip), (ma, mb) in zip(pairs_np, mats):
        wa, wb = A.copy(), B.copy()
        ca, cb = (1.0, 1.0) if clip is None else (float(clip[0]), float(clip[1]))
        oracle.coupled_update(wa, GA, ra, sa, fa, wb, GB, rb, sb, None, a_own=a_own, a_cross=a_cross,
                              clip_a=ca, clip_b=cb, weight_decay=wd, **HP)
        assert_state_equal(ma.to_state(), wa, f"pair A ({a_own},{a_cross})")
        assert_state_equal(mb.to_state(), wb, f"pair B ({a_own},{a_cross})")


def test_coupled_update_two_rows_per_workgroup(gpu_lib):
    # a wide pair and a 4096-column pair with more rows than CUs: the narrow
    # pair's rows go two to a 1024-lane workgroup
    g = synth.rng(950)
    specs = [(300, 8200, 31), (700, 4096, 163)]
    pairs_np = []
    for pi, (R, C, k) in enumerate(specs):
        A = make_state(R, C, 960 + pi, k + 4, True)
        B = make_state(R, C, 970 + pi, k + 4, True)
        ra = np.sort(g.choice(R, k, replace=False)).astype(np.int32)
        rb = np.sort(g.choice(R, k, replace=False)).astype(np.int32)
        sa = g.choice(k + 4, ra.size, replace=False).astype(np.int32)
        sb = g.choice(k + 4, rb.size, replace=False).astype(np.int32)
        GA = synth.gradient_rows(ra.size, C, 0.2, 980 + pi)
        GB = synth.gradient_rows(rb.size, C, 0.2, 990 + pi)
        pairs_np.append((A, B, ra, rb, sa, sb, GA, GB))
    gpu_pairs, mats = [], []
    for A, B, ra, rb, sa, sb, GA, GB in pairs_np:
        ma, mb = GpuMat(A, GA, ra, sa, None), GpuMat(B, GB, rb, sb, None)
        mats.append((ma, mb))
        gpu_pairs.append(_lib.Pair(ma.upd(), mb.upd(), 0.8, 0.3, None))
    _lib.sft_coupled_update(gpu_pairs, adam_dev(**HP))
    torch.cuda.synchronize()
    for (A, B, ra, rb, sa, sb, GA, GB), (ma, mb) in zip(pairs_np, mats):
        wa, wb = A.copy(), B.copy()
        oracle.coupled_update(wa, GA, ra, sa, None, wb, GB, rb, sb, None, a_own=0.8, a_cross=0.3,
                              clip_a=1.0, clip_b=1.0, weight_decay=0.0, **HP)
        assert_state_equal(ma.to_state(), wa, f"pair A C={A.q.shape[1]}")
        assert_state_equal(mb.to_state(), wb, f"pair B C={A.q.shape[1]}")


def test_masked_writeback_bit_exact(gpu_lib):
    R, C = 333, 1032
    q, s, delta = synth.quant_state(R, C, 700)
    rows = np.sort(synth.rng(701).choice(R, 40, replace=False)).astype(np.int32)
    w0 = np.full((R, C), 0x5A5A, np.uint16)
    wl = torch.from_numpy(w0.view(np.int16)).cuda()
    _lib.sft_masked_writeback(dev(q), dev(s), dev(delta), dev(rows), rows.size, wl)
    torch.cuda.synchronize()
    want = w0.copy()
    oracle.masked_writeback(q, s, delta, rows, want)
    assert np.array_equal(wl.cpu().numpy().view(np.uint16), want)


def _wb_case(R, C, k, seed):
    q, s, delta = synth.quant_state(R, C, seed)
    rows = np.sort(synth.rng(seed + 1).choice(R, k, replace=False)).astype(np.int32)
    w0 = np.full((R, C), 0x5A5A, np.uint16)
    return q, s, delta, rows, w0


def test_masked_writeback_many_bit_exact(gpu_lib):
    # 19 matrices (two launches of at most 16), mixed widths, one with no
    # active row and one with every row active; every listed row bit-exact
    # against the oracle and every other row untouched
    shapes = [(333, 1032, 40), (64, 8, 64), (500, 4096, 0), (40, 2056, 7)] + [(96, 264, 5 + i) for i in range(15)]
    cases = [_wb_case(R, C, k, 900 + 10 * i) for i, (R, C, k) in enumerate(shapes)]
    dev_wl = [torch.from_numpy(w0.view(np.int16)).cuda() for *_, w0 in cases]
    mats = [(dev(q), dev(s), dev(d), dev(rows), rows.size, wl) for (q, s, d, rows, _), wl in zip(cases, dev_wl)]
    _lib.sft_masked_writeback_many(mats)
    torch.cuda.synchronize()
    for i, ((q, s, d, rows, w0), wl) in enumerate(zip(cases, dev_wl)):
        want = w0.copy()
        oracle.masked_writeback(q, s, d, rows, want)
        assert np.array_equal(wl.cpu().numpy().view(np.uint16), want), f"matrix {i}"


def test_masked_writeback_many_matches_single_calls_and_rejects(gpu_lib):
    cases = [_wb_case(200, 520, 30, 960), _wb_case(120, 1000, 120, 970)]
    one = [torch.from_numpy(w0.view(np.int16)).cuda() for *_, w0 in cases]
    many = [torch.from_numpy(w0.view(np.int16)).cuda() for *_, w0 in cases]
    for (q, s, d, rows, _), wl in zip(cases, one):
        _lib.sft_masked_writeback(dev(q), dev(s), dev(d), dev(rows), rows.size, wl)
    _lib.sft_masked_writeback_many([(dev(q), dev(s), dev(d), dev(rows), rows.size, wl)
                                    for (q, s, d, rows, _), wl in zip(cases, many)])
    torch.cuda.synchronize()
    for a, b in zip(one, many):
        assert torch.equal(a, b)
    _lib.sft_masked_writeback_many([])
    q, s, d, rows, w0 = _wb_case(16, 12, 2, 980)       # C = 12: not a multiple of 8
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_masked_writeback_many([(dev(q), dev(s), dev(d), dev(rows), rows.size,
                                         torch.zeros((16, 12), dtype=torch.int16, device="cuda"))])
    assert e.value.code == _lib.SFT_ESHAPE


def test_update_rejects_bad_arguments(gpu_lib):
    st, rows, slot, fresh, G = _case(16, 12, 2, 2, 800, False)   # C = 12: not a multiple of 8
    m = GpuMat(st, G, rows, slot, fresh)
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_sparse_update([m.upd()], adam_dev(**HP))
    assert e.value.code == _lib.SFT_ESHAPE


def test_coupled_update_driven_by_the_schedule(gpu_lib):
    """Six steps of a gate-up-like pair (b = 0.6) whose a_own / a_cross come
    from the library's schedule at each step (falling loss, so the stride
    climbs and the phase sweeps part of a turn): the GPU state equals the
    oracle's after every step, both fed the schedule's coefficients rounded
    to fp32 and the same gradients."""
    import oracle.helix as hx
    R, C = 160, 264
    g = synth.rng(1500)
    A = make_state(R, C, 1510, 40, True)
    B = make_state(R, C, 1520, 40, True)
    ra = np.sort(g.choice(R, 30, replace=False)).astype(np.int32)
    rb = np.sort(np.unique(np.concatenate([ra[:12], g.choice(R, 18, replace=False)]))).astype(np.int32)
    sa = g.choice(40, ra.size, replace=False).astype(np.int32)
    sb = g.choice(40, rb.size, replace=False).astype(np.int32)
    wa, wb = A.copy(), B.copy()
    ma = GpuMat(A, np.zeros((ra.size, C), np.float32), ra, sa, None)
    mb = GpuMat(B, np.zeros((rb.size, C), np.float32), rb, sb, None)
    sched, ref = _lib.Helix(), hx.Helix()
    hp = adam_dev(**HP)
    for step in range(6):
        loss = 5.0 - 0.2 * step
        sched.step(loss)
        ref.step(loss)
        a_own, a_cross = sched.coupling(0.6)
        assert (a_own, a_cross) == ref.coupling(0.6)
        GA = synth.gradient_rows(ra.size, C, 0.2, 1530 + step)
        GB = synth.gradient_rows(rb.size, C, 0.2, 1540 + step)
        ma.G.copy_(torch.from_numpy(GA))
        mb.G.copy_(torch.from_numpy(GB))
        _lib.sft_coupled_update([_lib.Pair(ma.upd(), mb.upd(), a_own, a_cross, None)], hp)
        torch.cuda.synchronize()
        oracle.coupled_update(wa, GA, ra, sa, None, wb, GB, rb, sb, None, a_own=float(np.float32(a_own)),
                              a_cross=float(np.float32(a_cross)), clip_a=1.0, clip_b=1.0, weight_decay=0.0, **HP)
        assert_state_equal(ma.to_state(), wa, f"step {step} A")
        assert_state_equal(mb.to_state(), wb, f"step {step} B")


def test_binding_rejects_mismatched_tensors(gpu_lib):
    """The binding checks every tensor's dtype and shape before the library
    sees the pointers (the kernels trust the sizes)."""
    st, rows, slot, fresh, G = _case(64, 32, 4, 6, 1600, True)
    m = GpuMat(st, G, rows, slot, fresh)
    ok = m.upd()
    bad_cases = [
        ("m", m.m[:, :16], ValueError),                                   # wrong width
        ("v", m.v[:3], ValueError),                                       # slot count disagrees with m
        ("t", m.t[:2], ValueError),
        ("mv_exp", m.e[:, :1].contiguous(), ValueError),
        ("G", m.G.to(torch.float64), TypeError),                          # wrong dtype
        ("G", m.G[:2], ValueError),                                       # fewer rows than n_active
        ("delta", m.delta[:, :16].contiguous(), ValueError),
        ("s", m.s[:10], ValueError),
        ("active_rows", m.rows.to(torch.int64), TypeError),
        ("q", m.q.to(torch.int16), TypeError),
        ("w_live", m.w_live.to(torch.float32), TypeError),
    ]
    import dataclasses
    for field, value, exc in bad_cases:
        bad = dataclasses.replace(ok, **{field: value})
        with pytest.raises(exc):
            _lib.sft_sparse_update([bad], adam_dev(**HP))
    _lib.sft_sparse_update([ok], adam_dev(**HP))       # the unchanged matrix still runs
    torch.cuda.synchronize()


@pytest.mark.parametrize("gmag", [1e-5, 3e4], ids=["tiny", "huge"])
@pytest.mark.parametrize("C", [264, 20000], ids=["C264", "C20000"])
def test_scaled_moments_over_many_steps_at_extreme_gradients(gpu_lib, gmag, C):
    """Forty steps with gradients far below and far above fp16's range (the
    moments stored as scaled fp16 rows, their exponents moving step by step;
    at 20000 columns through the wide rows' two passes): bit-exact with the
    oracle after every fifth step."""
    st, rows, slot, fresh, _ = _case(24, C, 5, 7, 1700 + C, False)
    m = GpuMat(st, np.zeros((rows.size, C), np.float32), rows, slot, fresh)
    want = st.copy()
    hp = adam_dev(**HP)
    for step in range(40):
        Gs = (synth.gradient_rows(rows.size, C, 1.0, 1710 + step) * np.float32(gmag)).astype(np.float32)
        m.G.copy_(dev(Gs))
        _lib.sft_sparse_update([m.upd()], hp)
        oracle.sparse_update(want, Gs, rows, slot, fresh if step == 0 else None, **HP)
        if step == 0:
            m.fresh = None
        if step % 5 == 4:
            torch.cuda.synchronize()
            assert_state_equal(m.to_state(), want, f"step {step}")
    mo, vo = want.moments()
    assert np.all(np.isfinite(vo[slot])) and np.all(vo[slot] > 0)


def test_fresh_rows_ignore_stale_slot_contents(gpu_lib):
    """A fresh row's slot still holds what its previous owner left (or
    garbage): step counts below zero and past the bias table, NaN and
    infinite fp16 moments, extreme exponents.  The update reads them (its
    loads are unconditional) but must start the row from zero moments and
    step 1, bit for bit like the oracle; a step count that is never a valid
    table index must not be used as one.  Plain and coupled update, 256- and
    1024-lane launches."""
    hp = adam_dev(**HP, t_max=100)
    for C, seed in ((512, 3100), (11008, 3101)):
        st, rows, slot, _, G = _case(96, C, 40, 48, seed, True)
        fresh = np.ones(rows.size, np.uint8)
        fresh[::3] = 0                                     # a third continue from their stored state
        g = synth.rng(seed + 1)
        stale = np.array([-7, -2 ** 31, 2 ** 31 - 1, 101, 5000], np.int32)
        for i in np.nonzero(fresh)[0]:
            s = slot[i]
            st.t[s] = stale[i % stale.size]
            st.m[s, : C // 2] = 0x7E00                     # NaN
            st.v[s, C // 2:] = 0x7C00                      # +inf
            st.e[s] = (-128, 127)
        st.t[slot[fresh == 0]] = np.minimum(st.t[slot[fresh == 0]], 90)
        gm = GpuMat(st, G, rows, slot, fresh)
        _lib.sft_sparse_update([gm.upd()], hp)
        torch.cuda.synchronize()
        want = st.copy()
        oracle.sparse_update(want, G, rows, slot, fresh, **HP)
        assert_state_equal(gm.to_state(), want, f"plain C={C}")
        # coupled: the same state on both sides of a pair, partner rows shifted by one
        a_st, b_st = st.copy(), st.copy()
        ga, gb = GpuMat(a_st, G, rows, slot, fresh), GpuMat(b_st, G[::-1].copy(), rows, slot, fresh)
        _lib.sft_coupled_update([_lib.Pair(ga.upd(), gb.upd(), 1.0, 0.25, None)], hp)
        torch.cuda.synchronize()
        wa, wb = a_st.copy(), b_st.copy()
        oracle.coupled_update(wa, G, rows, slot, fresh, wb, G[::-1].copy(), rows, slot, fresh,
                              a_own=1.0, a_cross=0.25, **HP)
        assert_state_equal(ga.to_state(), wa, f"coupled a C={C}")
        assert_state_equal(gb.to_state(), wb, f"coupled b C={C}")
