"""The masked-dW launch planner, on the host (no GPU): which launch shape and
which tile shape per group sft_masked_dw takes for the benchmark's layer at
each row density, the adversarial one-row-per-tile layer and the shapes the
GPU tests rely on to reach each path.  The planner only decides how the
active 32-row tiles of section 2.2 ("Sparse-First Fine-Tuning: Full-Weight
Training at the Cost of the Active Set") are laid over the CUs; the GPU
parity tests check that every shape computes the same dW.
"""
import math

import numpy as np
import pytest

from sparse_full_weight_amd import _lib, synth

CUS = 256   # MI355X


def _plan(R, rows):
    return _lib.sft_plan_rows(synth.mask_from_rows(R, np.asarray(rows, np.int64)))


def _layer(density, T=4096, layout=_lib.SFT_DW_PACKED, one_per_tile=False):
    groups = []
    for gi, (_, members) in enumerate(synth.LLAMA7B_GROUPS):
        C = synth.LLAMA7B[members[0]][1]
        plans = []
        for j, m in enumerate(members):
            R = synth.LLAMA7B[m][0]
            rows = (synth.one_per_tile_rows(R, 300 + 10 * gi + j) if one_per_tile
                    else synth.clustered_rows(R, round(density * R), 100 + 10 * gi + j))
            plans.append(_plan(R, rows))
        groups.append((T, C, layout, plans))
    return groups


def _check_invariants(groups, launches):
    for L in launches:
        if L["kind"] == "narrow":
            assert CUS // 2 <= L["workgroups"] <= 2 * CUS
            if L["workgroups"] > CUS:   # two rounds keep at least 70% of the CUs busy
                assert 10 * L["workgroups"] >= 14 * CUS
        for (T, C, layout, plans), (shape, n_mblk, n_nblk) in zip(groups, L["groups"]):
            rows = sum(p.n_active if layout == _lib.SFT_DW_PACKED else 32 * p.n_active_tiles for p in plans)
            ptiles = (rows + 31) // 32
            if shape == 0:
                assert n_mblk == math.ceil(ptiles / 4)
            else:                       # one wave per packed tile: only past 4 tiles, at most 8 an M-block
                assert L["kind"] == "narrow" and ptiles > 4 and n_mblk == math.ceil(ptiles / 8)
            bn = 64 if shape == 1 else 128 if L["kind"] == "narrow" else 256
            assert n_nblk == math.ceil(C / bn)
        if L["kind"] == "narrow":
            assert L["workgroups"] == sum(m * n for _, m, n in L["groups"])


@pytest.mark.parametrize("density, workgroups, shapes", [
    # q/k/v, o, gate/up, down: (shape, M-blocks, column blocks)
    (0.005, 182, [(0, 1, 32), (0, 1, 32), (0, 1, 32), (0, 1, 86)]),
    (0.01, 214, [(0, 1, 32), (0, 1, 32), (1, 1, 64), (0, 1, 86)]),
    (0.02, 246, [(1, 1, 64), (0, 1, 32), (2, 2, 32), (0, 1, 86)]),
    (0.05, 374, [(2, 3, 32), (2, 1, 32), (2, 5, 32), (2, 1, 86)]),
])
def test_layer_densities_take_narrow_whole_tiles(density, workgroups, shapes):
    groups = _layer(density)
    launches = _lib.sft_probe_dw_plan(groups, CUS)
    assert launches == [{"kind": "narrow", "workgroups": workgroups, "groups": shapes}]
    _check_invariants(groups, launches)


def test_adversarial_layer_takes_team_slices():
    # one active row per 32-row tile: 12 / 4 / 22 / 4 packed tiles; 278 whole
    # tiles would leave 54% of two rounds busy, so the launch takes teams
    groups = _layer(0.0, one_per_tile=True)
    launches = _lib.sft_probe_dw_plan(groups, CUS)
    assert len(launches) == 1 and launches[0]["kind"] == "teams"
    assert [g[1] for g in launches[0]["groups"]] == [3, 1, 6, 1]
    _check_invariants(groups, launches)


def test_tile_layout_at_one_percent():
    # whole active tiles instead of packed rows: more tiles per group, still
    # one round of narrow whole tiles
    groups = _layer(0.01, layout=_lib.SFT_DW_TILES)
    launches = _lib.sft_probe_dw_plan(groups, CUS)
    assert len(launches) == 1 and launches[0]["kind"] == "narrow"
    _check_invariants(groups, launches)


def test_gpu_test_shapes_reach_their_paths():
    # the GPU tests' shapes for team slices, two rounds, 128-column one-wave
    # tiles and tile-aligned slices
    def tiles(R, ts):
        return _plan(R, [32 * t + r for t in ts for r in range(32)])

    team = [(4096, 1496, _lib.SFT_DW_PACKED, [_plan(900, synth.clustered_rows(900, 330, 2110)),
                                               _plan(600, synth.clustered_rows(600, 200, 2111))]),
            (4096, 1496, _lib.SFT_DW_PACKED, [_plan(512, synth.clustered_rows(512, 200, 2122))])]
    assert _lib.sft_probe_dw_plan(team, CUS)[0]["kind"] == "teams"
    two = [(200, 180 * 128, _lib.SFT_DW_PACKED, [tiles(320, [0, 1, 2, 4, 5, 6, 7, 8, 9])])]
    assert _lib.sft_probe_dw_plan(two, CUS) == [{"kind": "narrow", "workgroups": 360, "groups": [(2, 2, 180)]}]
    wide = [(700, 150 * 128 + 40, _lib.SFT_DW_PACKED, [tiles(256, range(8))])]
    assert _lib.sft_probe_dw_plan(wide, CUS) == [{"kind": "narrow", "workgroups": 151, "groups": [(2, 1, 151)]}]
    aligned = [(1024, 50 * 256, _lib.SFT_DW_PACKED, [_plan(96, synth.clustered_rows(96, 40, 1603))])]
    assert _lib.sft_probe_dw_plan(aligned, CUS) == [{"kind": "aligned", "workgroups": 200, "groups": [(0, 1, 50)]}]
    small = [(256, 512, _lib.SFT_DW_PACKED, [_plan(512, synth.clustered_rows(512, 51, 1501))])]
    assert _lib.sft_probe_dw_plan(small, CUS)[0]["kind"] == "stream-k"
    for g in (team, two, wide, aligned, small):
        _check_invariants(g, _lib.sft_probe_dw_plan(g, CUS))


def test_rounds_differ_or_too_few_tiles_leave_narrow():
    # narrow tiles need every group on the same 512-token rounds
    a = (4096, 4096, _lib.SFT_DW_PACKED, [_plan(4096, synth.clustered_rows(4096, 41, 11))])
    b = (600, 11008, _lib.SFT_DW_PACKED, [_plan(4096, synth.clustered_rows(4096, 41, 12))])
    assert _lib.sft_probe_dw_plan([a, b], CUS)[0]["kind"] != "narrow"
    # on 1024 CUs the same 214 tiles fill less than half of them
    assert _lib.sft_probe_dw_plan(_layer(0.01), 1024)[0]["kind"] != "narrow"


def test_empty_groups_launch_nothing_and_bad_arguments_fail():
    empty = [(4096, 4096, _lib.SFT_DW_PACKED, [_plan(4096, [])])]
    assert _lib.sft_probe_dw_plan(empty, CUS) == []
    with pytest.raises(_lib.SftError):
        _lib.sft_probe_dw_plan(_layer(0.01), -1)
