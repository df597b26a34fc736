"""CPU tests of the C-ABI library: every declared symbol is exported, and the
host-side logic (conductor, row tracker, row plans, embedding CSR, moment
slots, bias table, argument checks) matches the oracle bit for bit.

No GPU is needed: these calls run on the host.  Method: "Sparse-First
Fine-Tuning: Full-Weight Training at the Cost of the Active Set", sections
2.1 (conductor and tracker, masks once a step on the CPU) and 2.2 (32-row
tiles).
"""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import oracle
from sparse_full_weight_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(sft_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(_lib.LIB_PATH)
    declared = _declared()
    assert len(declared) >= 14
    missing = [n for n in declared if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(_lib.EXPORTS) == declared
    want = int(re.search(r"#define SFT_ABI_VERSION (\d+)", open(os.path.join(ROOT, "include", "sft.h")).read())[1])
    assert _lib.sft_abi_version() == want


def test_conductor_matches_oracle_over_windows():
    V = 32000
    ch_l = np.zeros(V, np.float32)
    ch_o = np.zeros(V, np.float32)
    for w in range(4):
        toks = synth.zipf_tokens(4096, V, 1.1, 2000 + w)
        a_l = _lib.sft_conductor_window(ch_l, toks)
        a_o = oracle.conductor_window(ch_o, toks)
        assert np.array_equal(ch_l.view(np.uint32), ch_o.view(np.uint32))
        assert np.array_equal(a_l, a_o)
    # the embedding config's conductor yields a sparse mask (about 0.2% of rows)
    assert 20 <= a_l.sum() <= 200


def test_tracker_matches_oracle():
    R = 11008
    hot = synth.clustered_rows(R, 110, 2100)
    ch_l = np.zeros(R, np.float32)
    ch_o = np.zeros(R, np.float32)
    for w in range(3):
        a = synth.tracker_magnitudes(R, hot, 2101 + w)
        a_l = _lib.sft_tracker_window(ch_l, a)
        a_o = oracle.tracker_window(ch_o, a)
        assert np.array_equal(ch_l.view(np.uint32), ch_o.view(np.uint32))
        assert np.array_equal(a_l, a_o)
    with pytest.raises(_lib.SftError):
        _lib.sft_tracker_window(ch_l, -np.ones(R, np.float32))


@pytest.mark.parametrize("R", [1, 31, 33, 512, 4097, 11008])
def test_plan_rows_matches_oracle(R):
    mask = (synth.rng(R).random(R) < 0.05).astype(np.uint8)
    mask[-1] = 1
    p = _lib.sft_plan_rows(mask)
    o = oracle.plan_rows(mask)
    assert np.array_equal(p.tile_bits, o["bits"])
    assert np.array_equal(p.active_rows, o["active_rows"])
    assert np.array_equal(p.active_tiles, o["active_tiles"])
    # per active tile: its bits, and where its first active row sits in the row list
    assert np.array_equal(p.active_bits, o["bits"][o["active_tiles"]])
    assert np.array_equal(p.tile_first, np.searchsorted(o["active_rows"], 32 * o["active_tiles"]))


def test_plan_embedding_matches_oracle():
    V = 5000
    toks = synth.zipf_tokens(4096, V, 1.1, 2200)
    mask = np.zeros(V, np.uint8)
    mask[np.unique(toks)[:40]] = 1
    mask[V - 1] = 1                       # an active row with no hits
    p = _lib.sft_plan_rows(mask)
    rp, pos = _lib.sft_plan_embedding(p, toks)
    orp, opos = oracle.plan_embedding(p.active_rows, toks)
    assert np.array_equal(rp, orp) and np.array_equal(pos, opos)


def test_slots_match_oracle_over_steps():
    g = synth.rng(2300)
    R, n_slots = 500, 60
    rs_l = np.full(R, -1, np.int32)
    rs_o = np.full(R, -1, np.int32)
    for _ in range(40):
        rows = np.sort(g.choice(R, size=int(g.integers(0, n_slots + 1)), replace=False)).astype(np.int32)
        s_l, f_l = _lib.sft_slots_update(rs_l, n_slots, rows)
        s_o, f_o = oracle.slots_update(rs_o, n_slots, rows)
        assert np.array_equal(s_l, s_o) and np.array_equal(f_l, f_o) and np.array_equal(rs_l, rs_o)
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_slots_update(rs_l, 2, np.arange(3, dtype=np.int32))
    assert e.value.code == _lib.SFT_ECAPACITY


def test_bias_table_matches_oracle():
    for b1, b2 in [(0.9, 0.999), (0.8, 0.95), (0.0, 0.5)]:
        l1, l2 = _lib.sft_bias_table(b1, b2, 20000)
        o1, o2 = oracle.bias_table(b1, b2, 20000)
        assert np.array_equal(l1.view(np.uint32), o1.view(np.uint32))
        assert np.array_equal(l2.view(np.uint32), o2.view(np.uint32))
    assert _lib.sft_bias_table(0.9, 0.999, 20000)[1][-1] == 1.0   # table reaches 1.0f


def test_host_calls_reject_bad_input_before_writing():
    ch = np.full(4, 0.5, np.float32)
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_conductor_window(ch, np.array([0, 4], np.int32))
    assert e.value.code == _lib.SFT_EINVAL
    assert np.all(ch == 0.5)
    with pytest.raises(_lib.SftError):
        _lib.sft_bias_table(1.0, 0.9, 10)
    assert "beta" in _lib.lib().sft_last_error().decode()


def _layer_case(step, shapes, density=0.01, seed=2400):
    """Magnitudes of one window per matrix: clustered hot rows that drift
    from step to step."""
    mags = []
    for i, R in enumerate(shapes):
        if R == 0:
            mags.append(np.zeros(0, np.float32))
            continue
        hot = synth.clustered_rows(R, max(1, round(density * R)), seed + 10 * i + step)
        mags.append(synth.tracker_magnitudes(R, hot, seed + 10 * i + 5 + step))
    return mags


def test_plan_layer_matches_oracle_over_steps():
    """sft_plan_layer equals the oracle's tracker window, row plan and moment
    slots of each matrix, step after step (charges and slots carried), with
    the sections where the offsets say; matrices of ragged sizes, an empty
    one, and slot pools both larger than the rows and only as large as
    needed (the staged path)."""
    shapes = [4096, 4096, 4096, 4096, 11008, 11008, 4096, 33, 0, 1000]
    slots = [R for R in shapes[:7]] + [40, 0, 900]
    pl = _lib.LayerPlanner(shapes, slots)
    ch_o = [np.zeros(R, np.float32) for R in shapes]
    rs_o = [np.full(R, -1, np.int32) for R in shapes]
    for step in range(5):
        mags = _layer_case(step, shapes)
        got = pl.plan(mags)
        offs = sorted(o for mp in got for o in mp.off.values())
        assert all(o % 4 == 0 for o in offs) and pl.length <= pl.words
        for i, R in enumerate(shapes):
            act = oracle.tracker_window(ch_o[i], mags[i])
            assert np.array_equal(pl.charge[i].view(np.uint32), ch_o[i].view(np.uint32)), (step, i)
            want = oracle.plan_rows(act)
            slot, fresh = oracle.slots_update(rs_o[i], slots[i], want["active_rows"])
            mp = got[i]
            assert np.array_equal(pl.section(mp, "rows"), want["active_rows"]), (step, i)
            assert np.array_equal(pl.section(mp, "tiles"), want["active_tiles"]), (step, i)
            assert np.array_equal(pl.section(mp, "bits"), want["bits"][want["active_tiles"]]), (step, i)
            first = np.searchsorted(want["active_rows"], 32 * want["active_tiles"]).astype(np.int32)
            assert np.array_equal(pl.section(mp, "first"), first), (step, i)
            assert np.array_equal(pl.section(mp, "slot"), slot) and np.array_equal(pl.section(mp, "fresh"), fresh)
            assert np.array_equal(pl.row_slot[i], rs_o[i]), (step, i)


def test_plan_layer_checks_everything_before_writing():
    shapes = [4096, 11008, 64]
    pl = _lib.LayerPlanner(shapes, [4096, 11008, 2])
    mags = _layer_case(0, shapes)
    mags[2] = np.zeros(64, np.float32)
    pl.plan(mags)
    before = ([c.copy() for c in pl.charge], [r.copy() for r in pl.row_slot], pl.packed.copy())

    def unchanged():
        return (all(np.array_equal(a.view(np.uint32), b.view(np.uint32)) for a, b in zip(pl.charge, before[0]))
                and all(np.array_equal(a, b) for a, b in zip(pl.row_slot, before[1]))
                and np.array_equal(pl.packed, before[2]))

    bad = _layer_case(1, shapes)
    bad[2] = np.zeros(64, np.float32)
    bad[1] = bad[1].copy()
    bad[1][77] = np.nan                                   # a bad magnitude in the second matrix
    with pytest.raises(_lib.SftError) as e:
        pl.plan(bad)
    assert e.value.code == _lib.SFT_EINVAL and unchanged()
    full = _layer_case(1, shapes)
    full[2] = np.ones(64, np.float32)                      # 64 active rows, 2 slots
    with pytest.raises(_lib.SftError) as e:
        pl.plan(full)
    assert e.value.code == _lib.SFT_ECAPACITY and unchanged()
    pl.row_slot[0][5] = 4096                               # a slot outside the pool
    with pytest.raises(_lib.SftError) as e:
        pl.plan(_layer_case(1, shapes))
    assert e.value.code == _lib.SFT_EINVAL
    pl.row_slot[0][5] = before[1][0][5]
    small = _lib.LayerPlanner(shapes, [4096, 11008, 2], packed_ptr=pl.packed.ctypes.data, packed_words=pl.words)
    small._cap = pl.words - 1                             # one word short
    with pytest.raises(_lib.SftError) as e:
        small.plan(mags)
    assert e.value.code == _lib.SFT_ECAPACITY
    small._cap, small._ptr = pl.words, pl.packed.ctypes.data + 4
    with pytest.raises(_lib.SftError) as e:
        small.plan(mags)
    assert e.value.code == _lib.SFT_EALIGN and unchanged()
