"""GPU parity of the masked dW with the update fused in (sft_masked_dw_update).

The fused call adds the partial rows of split output tiles inside the update,
in the same slice order as the fix-up kernel, so every state array it leaves
must be bit-identical to sft_masked_dw followed by sft_sparse_update on the
same inputs; one case is also checked against the oracle directly.  Method:
"Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the Active
Set", sections 2.2 (masked dW) and 2.3 (sparse int8 + residual Adam update).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_full_weight_amd import _lib, synth
from tests.gpu_helpers import GpuMat, adam_dev, assert_state_equal, bf16_dev, dw_close, make_state

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)
LAYOUTS = pytest.mark.parametrize("layout", [_lib.SFT_DW_TILES, _lib.SFT_DW_PACKED], ids=["tiles", "packed"])


def _case(spec, seed):
    """spec: [(T, C, [(R, k_active), ...]), ...] -> numpy inputs of every group and matrix."""
    g = synth.rng(seed)
    groups = []
    for gi, (T, C, mats) in enumerate(spec):
        X = synth.normal_bf16((T, C), 1.0, seed + 10 * gi)
        ms = []
        for mi, (R, k) in enumerate(mats):
            s = seed + 1000 + 100 * gi + mi
            dY = synth.normal_bf16((T, R), 0.01, s)
            mask = synth.mask_from_rows(R, synth.clustered_rows(R, k, s + 1))
            plan = _lib.sft_plan_rows(mask)
            n = plan.n_active
            st = make_state(R, C, s + 2, n + 3, True)
            slot = g.choice(n + 3, size=n, replace=False).astype(np.int32)
            ms.append((dY, plan, st, slot))
        groups.append((X, ms))
    return groups


def _run(case, layout, fused):
    """Runs one path on fresh device copies; returns the final states."""
    groups, mats, gm = [], [], []
    for X, ms in case:
        dws = []
        for dY, plan, st, slot in ms:
            dplan = plan.to_device()
            C = X.shape[1]
            m = GpuMat(st, np.zeros((plan.n_active, C), np.float32), plan.active_rows, slot, None)
            m.rows = dplan.active_rows          # the update reads the dW plan's row list
            dws.append(_lib.DwMat(bf16_dev(dY), dplan, m.G))
            mats.append(m.upd())
            gm.append(m)
        groups.append(_lib.DwGroup(bf16_dev(X), dws, layout))
    nbytes = _lib.sft_masked_dw_workspace(groups)
    ws = torch.zeros(max(nbytes // 4, 1), dtype=torch.int32, device="cuda")
    hp = adam_dev(**HP)
    if fused:
        _lib.sft_masked_dw_update(groups, ws, mats, hp)
    else:
        _lib.sft_masked_dw(groups, ws)
        _lib.sft_sparse_update(mats, hp)
    torch.cuda.synchronize()
    return [m.to_state() for m in gm]


def _check_equal(case, layout):
    want = _run(case, layout, fused=False)
    got = _run(case, layout, fused=True)
    for i, (a, b) in enumerate(zip(got, want)):
        assert_state_equal(a, b, f"matrix {i}")


@LAYOUTS
def test_fused_matches_two_calls(gpu_lib, layout):
    # three matrices on one input spanning two M-blocks, plus a second group
    case = _case([(192, 264, [(320, 100), (128, 40), (96, 10)]), (192, 96, [(200, 20)])], 2100)
    _check_equal(case, layout)


@LAYOUTS
def test_fused_long_token_axis(gpu_lib, layout):
    # few output tiles, many tokens: tiles cut by more than four slices (the
    # update adds the fifth and later partial rows after the first four)
    case = _case([(4096, 128, [(128, 70)])], 2200)
    _check_equal(case, layout)


def test_fused_wide_and_narrow_rows(gpu_lib):
    # 4096- and 11008-column matrices (the 1024-lane update), 512 tokens
    case = _case([(512, 4096, [(1024, 20), (1024, 20)]), (512, 11008, [(1024, 12)])], 2300)
    _check_equal(case, _lib.SFT_DW_PACKED)


@LAYOUTS
def test_fused_tile_aligned_slices(gpu_lib, layout):
    # 50 output tiles of 4 rounds, each cut in quarters by the slices (too few
    # 128-column tiles for the whole-tile shape)
    case = _case([(1024, 50 * 256, [(96, 40)])], 2350)
    _check_equal(case, layout)


@LAYOUTS
def test_fused_narrow_whole_tiles(gpu_lib, layout):
    # 200 whole 128-column tiles: no partial sums, the update reads dW_act
    case = _case([(700, 199 * 128 + 40, [(96, 70)])], 2360)
    _check_equal(case, layout)


def test_fused_narrow_wave_per_tile(gpu_lib):
    # a group of 7 packed tiles (one M-block of 64-column tiles, one wave per
    # packed tile) beside a 2-tile group of 128-column tiles, one narrow
    # launch: the update reads dW_act
    case = _case([(1000, 4096, [(512, 110), (512, 110)]), (600, 8192, [(256, 40)])], 2370)
    _check_equal(case, _lib.SFT_DW_PACKED)


def test_fused_falls_back_beyond_one_launch(gpu_lib):
    # ten groups need two product launches: the call runs the two calls
    case = _case([(128, 64 + 8 * i, [(40 + 13 * i, 5 + i)]) for i in range(10)], 2400)
    _check_equal(case, _lib.SFT_DW_PACKED)


def test_fused_against_oracle(gpu_lib):
    # the oracle's update, fed the GPU's own dW rows (within the dW tolerance
    # of the oracle's fp64 sums), gives the fused call's states bit for bit
    case = _case([(320, 136, [(200, 30), (96, 12)])], 2500)
    got = _run(case, _lib.SFT_DW_PACKED, fused=True)
    X, ms = case[0]
    dws, bufs = [], []
    for dY, plan, st, slot in ms:
        buf = torch.zeros((plan.n_active, X.shape[1]), dtype=torch.float32, device="cuda")
        dws.append(_lib.DwMat(bf16_dev(dY), plan.to_device(), buf))
        bufs.append(buf)
    groups = [_lib.DwGroup(bf16_dev(X), dws, _lib.SFT_DW_PACKED)]
    ws = torch.zeros(max(_lib.sft_masked_dw_workspace(groups) // 4, 1), dtype=torch.int32, device="cuda")
    _lib.sft_masked_dw(groups, ws)
    torch.cuda.synchronize()
    for i, ((dY, plan, st, slot), buf, g) in enumerate(zip(ms, bufs, got)):
        G = buf.cpu().numpy()
        dw_close(G, oracle.masked_dw(dY, X, plan.active_rows))
        want = st.copy()
        oracle.sparse_update(want, G, plan.active_rows, slot, None, **HP)
        assert_state_equal(g, want, f"matrix {i}")


def test_fused_rejects_mismatched_gradient(gpu_lib):
    case = _case([(64, 64, [(64, 8)])], 2600)
    X, ms = case[0]
    dY, plan, st, slot = ms[0]
    dplan = plan.to_device()
    m = GpuMat(st, np.zeros((plan.n_active, 64), np.float32), plan.active_rows, slot, None)
    m.rows = dplan.active_rows
    other = torch.zeros((plan.n_active, 64), dtype=torch.float32, device="cuda")
    groups = [_lib.DwGroup(bf16_dev(X), [_lib.DwMat(bf16_dev(dY), dplan, other)], _lib.SFT_DW_PACKED)]
    ws = torch.zeros(max(_lib.sft_masked_dw_workspace(groups) // 4, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_masked_dw_update(groups, ws, [m.upd()], adam_dev(**HP))
    assert e.value.code == _lib.SFT_EINVAL


@LAYOUTS
def test_fused_many_mblocks(gpu_lib, layout):
    # 4 and more M-blocks (output tiles numbered column block by column block)
    case = _case([(256, 520, [(700, 300), (400, 150)]), (256, 136, [(300, 170)])], 2700)
    _check_equal(case, layout)


@LAYOUTS
def test_fused_team_slices_cut_tiles(gpu_lib, layout):
    # team slicing with tiles cut at ragged rounds (5- and 2-M-block groups,
    # too few columns for whole narrow tiles, 16 rounds a tile, teams of 3-4
    # rounds): the update adds each cut tile's partial rows, one slice per
    # team, in the fix-up's order
    case = _case([(4096, 1496, [(900, 330), (600, 200)]), (4096, 1496, [(512, 200)])], 2800)
    _check_equal(case, layout)


def test_fused_million_token_axis(gpu_lib):
    # 2^20 tokens over one 32-row tile and 8 columns: every output tile is cut
    # into one slice per CU, so each updated row adds 256 partial rows
    case = _case([(1 << 20, 8, [(32, 7)])], 2900)
    _check_equal(case, _lib.SFT_DW_PACKED)
