"""GPU parity of the active-row checkpoint calls (sft_rows_save,
sft_rows_restore) against the oracle's row copies: "Sparse-First
Fine-Tuning: Full-Weight Training at the Cost of the Active Set", section 2.6
(the checkpoint holds the active rows only) and section 2.3 (the restored rows'
live bf16 weights are rebuilt as the write-back does).  Every comparison is
bit for bit, over whole arrays: the checkpoint buffers, the live state after a
restore (rows outside the checkpoint must be untouched) and the live weights.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import rewind as rw
from sparse_full_weight_amd import _lib, synth
from tests.gpu_helpers import GpuMat, adam_dev, assert_state_equal, host_u16, make_state

pytestmark = pytest.mark.gpu


def _case(R, C, n_rows, n_slots, seed):
    """A mid-run state, an ascending row list and a permutation of slots."""
    st = make_state(R, C, seed, n_slots, True)
    g = synth.rng(seed + 5)
    rows = np.sort(g.choice(R, size=n_rows, replace=False)).astype(np.int32)
    slot = g.choice(n_slots, size=n_rows, replace=False).astype(np.int32)
    return st, rows, slot


def _gpu(st, rows, slot, with_live=True):
    gm = GpuMat(st, np.zeros((max(rows.size, 1), st.q.shape[1]), np.float32), rows, slot, None, with_live)
    ck = _lib.CkptMat.alloc(gm.q, gm.s, gm.delta, gm.m, gm.v, gm.t, gm.e, gm.rows, gm.slot, rows.size, gm.w_live)
    return gm, ck


def _ck_host(ck, n):
    return rw.RowCopy(ck.ck_q.cpu().numpy()[:n], ck.ck_s.cpu().numpy()[:n], ck.ck_delta.cpu().numpy()[:n],
                      host_u16(ck.ck_m)[:n], host_u16(ck.ck_v)[:n], ck.ck_t.cpu().numpy()[:n],
                      ck.ck_mv_exp.cpu().numpy()[:n])


def _assert_copy_equal(got: rw.RowCopy, want: rw.RowCopy, what):
    for name in ("q", "s", "delta", "m", "v", "t", "e"):
        a, b = getattr(got, name), getattr(want, name)
        assert a.shape == b.shape, (what, name)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{what}: checkpoint {name} differs"


SHAPES = [(40, 8, 5, 9), (300, 264, 37, 64), (96, 4096, 20, 24), (64, 11008, 9, 16), (50, 16, 0, 4)]


def test_rows_save_matches_oracle(gpu_lib):
    cases = [_case(R, C, n, ns, 4000 + i) for i, (R, C, n, ns) in enumerate(SHAPES)]
    gpus = [_gpu(*c) for c in cases]
    _lib.sft_rows_save([ck for _, ck in gpus])
    torch.cuda.synchronize()
    for i, ((st, rows, slot), (gm, ck)) in enumerate(zip(cases, gpus)):
        _assert_copy_equal(_ck_host(ck, rows.size), rw.rows_save(st, rows, slot), f"matrix {i}")
        assert_state_equal(gm.to_state(), st, f"matrix {i} live state after save")


@pytest.mark.parametrize("with_live", [True, False], ids=["live", "no_live"])
def test_rows_restore_after_updates_matches_oracle(gpu_lib, with_live):
    """Save, take two sparse update steps on the GPU (rows inside and outside
    the checkpoint), restore: the live state must equal the oracle's restore
    applied to the GPU's post-update state, with the oracle's own copy."""
    cases = [_case(R, C, n, ns, 4100 + i) for i, (R, C, n, ns) in enumerate(SHAPES)]
    gpus = [_gpu(st, rows, slot, with_live) for st, rows, slot in cases]
    cks = [ck for _, ck in gpus]
    _lib.sft_rows_save(cks)
    hp = adam_dev()
    upd = []
    for i, ((st, rows, slot), (gm, _)) in enumerate(zip(cases, gpus)):
        # the update's rows: half of the checkpointed rows plus a few others
        R, C = st.q.shape
        extra = np.setdiff1d(np.arange(R), rows)[: 3]
        urows = np.union1d(rows[::2], extra).astype(np.int32)
        uslot = np.setdiff1d(np.arange(st.m.shape[0]), slot[1::2])[: urows.size].astype(np.int32)
        if urows.size > uslot.size:
            urows, uslot = urows[: uslot.size], uslot
        G = synth.gradient_rows(urows.size, C, 1e-3, 4300 + i)
        um = GpuMat(st, G, urows, uslot, None, with_live)
        for name in ("q", "s", "delta", "m", "v", "t", "e", "w_live"):
            setattr(um, name, getattr(gm, name))
        upd.append(um.upd())
    _lib.sft_sparse_update(upd, hp)
    _lib.sft_sparse_update(upd, hp)
    torch.cuda.synchronize()
    mid = [gm.to_state() for gm, _ in gpus]
    _lib.sft_rows_restore(cks)
    torch.cuda.synchronize()
    for i, ((st, rows, slot), (gm, _), after) in enumerate(zip(cases, gpus, mid)):
        want = after.copy()
        rw.rows_restore(want, rw.rows_save(st, rows, slot), rows, slot)
        assert_state_equal(gm.to_state(), want, f"matrix {i}")


def test_rows_copy_more_matrices_than_one_launch(gpu_lib):
    cases = [_case(64, 8 * (1 + i % 5), 3 + i, 12 + i, 4400 + i) for i in range(19)]
    gpus = [_gpu(*c) for c in cases]
    cks = [ck for _, ck in gpus]
    _lib.sft_rows_save(cks)
    for gm, _ in gpus:
        gm.q.zero_()
        gm.s.fill_(1.0)
        gm.m.fill_(3)
    _lib.sft_rows_restore(cks)
    torch.cuda.synchronize()
    for i, ((st, rows, slot), (gm, ck)) in enumerate(zip(cases, gpus)):
        _assert_copy_equal(_ck_host(ck, rows.size), rw.rows_save(st, rows, slot), f"matrix {i}")
        want = st.copy()
        want.q[:] = 0
        want.s[:] = 1.0
        want.m[:] = 3
        rw.rows_restore(want, rw.rows_save(st, rows, slot), rows, slot)
        assert_state_equal(gm.to_state(), want, f"matrix {i}")


def test_rewind_cycle_returns_the_accepted_checkpoint(gpu_lib):
    """The controller drives a short run with two copy buffers (the
    checkpoint and the minimum's copy): each step the loss of the current rows
    is observed, then PROMOTE swaps the buffers' roles, SAVE_MIN and SAVE copy
    the rows into the minimum's buffer and the checkpoint, and the update is
    applied unless the step is dropped by a RESTORE.  Losses 10, 8, then 8.5
    for nine steps and 9.3 (section 2.6: 9.3 > 1.15 * 8 at the end of the
    minimum's watch): the restore brings back the step-0 rows, the last
    accepted state, bit for bit."""
    st, rows, slot = _case(128, 264, 24, 32, 4500)
    gm, ck_a = _gpu(st, rows, slot)
    ck_b = _lib.CkptMat.alloc(gm.q, gm.s, gm.delta, gm.m, gm.v, gm.t, gm.e, gm.rows, gm.slot, rows.size,
                              gm.w_live)
    hp = adam_dev(lr=1e-3)
    G = synth.gradient_rows(rows.size, 264, 1e-2, 4501)
    gm.G = torch.from_numpy(G).cuda()
    ctl = _lib.Rewind()
    bufs = {"ckpt": ck_a, "min": ck_b}
    states = {}
    losses = [10.0, 8.0] + [8.5] * 9 + [9.3]
    for k, x in enumerate(losses):
        torch.cuda.synchronize()
        states[k] = gm.to_state()          # the rows that produced loss x
        act = ctl.observe(x)
        if act & _lib.SFT_REWIND_RESTORE:
            assert act == _lib.SFT_REWIND_RESTORE and k == len(losses) - 1
            _lib.sft_rows_restore([bufs["ckpt"]])
            break
        if act & _lib.SFT_REWIND_PROMOTE:
            bufs["ckpt"], bufs["min"] = bufs["min"], bufs["ckpt"]
        if act & _lib.SFT_REWIND_SAVE_MIN:
            _lib.sft_rows_save([bufs["min"]])
        if act & _lib.SFT_REWIND_SAVE:
            _lib.sft_rows_save([bufs["ckpt"]])
        _lib.sft_sparse_update([gm.upd()], hp)
    torch.cuda.synchronize()
    assert ctl.state().checkpoint_step == 0
    got, saved = gm.to_state(), states[0]
    for name in ("q", "s", "delta"):
        assert np.array_equal(getattr(got, name)[rows].view(np.uint8), getattr(saved, name)[rows].view(np.uint8))
    for name in ("m", "v", "t", "e"):
        assert np.array_equal(getattr(got, name)[slot], getattr(saved, name)[slot])
    # the step-1 rows (the watched minimum's copy) differ from what came back
    assert not np.array_equal(states[1].delta[rows], got.delta[rows])
    want_w = np.zeros_like(got.w_live)
    oracle.masked_writeback(got.q, got.s, got.delta, rows, want_w)
    assert np.array_equal(got.w_live[rows], want_w[rows])


def test_rows_copy_rejects_bad_input(gpu_lib):
    st, rows, slot = _case(40, 24, 6, 8, 4600)
    gm, ck = _gpu(st, rows, slot)
    rows9 = torch.arange(0, 36, 4, dtype=torch.int32, device="cuda")
    bad = _lib.CkptMat.alloc(gm.q, gm.s, gm.delta, gm.m, gm.v, gm.t, gm.e, rows9, rows9, 9, gm.w_live)
    with pytest.raises(_lib.SftError) as e:                         # 9 rows, 8 slots: the library's check
        _lib.sft_rows_save([bad])
    assert e.value.code == _lib.SFT_EINVAL
    short = _lib.CkptMat(**{**ck.__dict__, "n_rows": 9})            # row list shorter than n_rows
    with pytest.raises(ValueError):
        _lib.sft_rows_save([short])
    st12, rows12, slot12 = _case(40, 12, 6, 8, 4601)                 # C = 12: the library's own check
    _, ck12 = _gpu(st12, rows12, slot12)
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_rows_restore([ck12])
    assert e.value.code == _lib.SFT_ESHAPE
    odd = torch.zeros((40, 12), dtype=torch.int8, device="cuda")
    bad = _lib.CkptMat(**{**ck.__dict__, "q": odd})               # q's columns disagree with delta's
    with pytest.raises(ValueError):
        _lib.sft_rows_restore([bad])
    shifted = torch.zeros(6 * 24 + 4, dtype=torch.float32, device="cuda")[4:].view(6, 24)
    ok = _lib.CkptMat(**{**ck.__dict__, "ck_delta": shifted})     # 16 bytes past an allocation: aligned
    _lib.sft_rows_save([ok])
    mis = torch.zeros(6 * 24 + 1, dtype=torch.float32, device="cuda")[1:].view(6, 24)
    bad = _lib.CkptMat(**{**ck.__dict__, "ck_delta": mis})        # 4 bytes past: not aligned
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_rows_save([bad])
    assert e.value.code == _lib.SFT_EALIGN
    torch.cuda.synchronize()
