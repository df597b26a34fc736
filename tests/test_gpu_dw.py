"""GPU parity of the masked weight gradient and the embedding gradient.

The HIP path (sft_masked_dw, sft_embedding_dw) and the oracle get the same
seeded bf16 inputs; dW rows of active rows must agree within the stated
tolerance (fp32 accumulation against an fp64 sum rounded once), exactly where
the arithmetic is exact (one token, small integers), and no byte outside the
active rows may be written.  Method: "Sparse-First Fine-Tuning: Full-Weight
Training at the Cost of the Active Set", section 2.2.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_full_weight_amd import _lib, synth
from tests.gpu_helpers import bf16_dev, dev, dw_close

pytestmark = pytest.mark.gpu

CANARY = float("nan")


LAYOUTS = pytest.mark.parametrize("layout", [_lib.SFT_DW_TILES, _lib.SFT_DW_PACKED], ids=["tiles", "packed"])


def _run(groups_np, repeat=1, layout=_lib.SFT_DW_PACKED):
    """groups_np: list of (X_bits [T x C], [(dY_bits [T x R], mask [R]), ...])."""
    groups, outs, plans = [], [], []
    for X, mats in groups_np:
        C = X.shape[1]
        ms = []
        for dY, mask in mats:
            plan = _lib.sft_plan_rows(mask)
            buf = torch.full((plan.n_active + 3, C), CANARY, dtype=torch.float32, device="cuda")
            ms.append(_lib.DwMat(bf16_dev(dY), plan.to_device(), buf[:plan.n_active]))
            outs.append(buf)
            plans.append(plan)
        groups.append(_lib.DwGroup(bf16_dev(X), ms, layout))
    nbytes = _lib.sft_masked_dw_workspace(groups)
    ws = torch.zeros(max(nbytes // 4, 1), dtype=torch.int32, device="cuda") if nbytes else None
    results = []
    for _ in range(repeat):
        _lib.sft_masked_dw(groups, ws)
        torch.cuda.synchronize()
        results.append([b.cpu().numpy() for b in outs])
    for res in results:
        for b, plan in zip(res, plans):
            assert np.all(np.isnan(b[plan.n_active:])), "write past the last active row"
    return results[-1] if repeat == 1 else results, plans


def _check(groups_np, exact=False, repeat=1, layout=_lib.SFT_DW_PACKED):
    res, plans = _run(groups_np, repeat, layout)
    if repeat > 1:
        for r in res[1:]:
            for a, b in zip(res[0], r):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "not deterministic"
        res = res[0]
    i = 0
    for X, mats in groups_np:
        for dY, mask in mats:
            want = oracle.masked_dw(dY, X, np.nonzero(mask)[0].astype(np.int32))
            got = res[i][:plans[i].n_active]
            if exact:
                assert np.array_equal(got, want)
            else:
                dw_close(got, want)
            i += 1


def _mask_rows(R, rows):
    return synth.mask_from_rows(R, np.asarray(rows, np.int64))


@LAYOUTS
def test_dw_small_projection_10pct_clustered(gpu_lib, layout):
    # 512 x 512 projection, 256 tokens, 10% of rows active in clustered tiles
    T, R, C = 256, 512, 512
    X = synth.normal_bf16((T, C), 1.0, 1001)
    dY = synth.normal_bf16((T, R), 0.01, 1002)
    mask = _mask_rows(R, synth.clustered_rows(R, round(0.10 * R), 1501))
    _check([(X, [(dY, mask)])], repeat=2, layout=layout)


@LAYOUTS
def test_dw_ragged_everything(gpu_lib, layout):
    # R % 32 != 0 and R % 8 != 0 (unaligned dY rows), C not a multiple of 128,
    # T not a multiple of the token chunk; last row active
    T, R, C = 100, 70, 200
    X = synth.normal_bf16((T, C), 1.0, 1011)
    dY = synth.normal_bf16((T, R), 0.01, 1012)
    mask = _mask_rows(R, [0, 5, 31, 32, 40, 63, 64, 69])
    _check([(X, [(dY, mask)])], layout=layout)


@LAYOUTS
def test_dw_single_token_is_exact_outer_product(gpu_lib, layout):
    T, R, C = 1, 96, 136
    X = synth.normal_bf16((T, C), 1.0, 1021)
    dY = synth.normal_bf16((T, R), 0.01, 1022)
    mask = _mask_rows(R, [1, 2, 33, 95])
    _check([(X, [(dY, mask)])], exact=True, layout=layout)


@LAYOUTS
def test_dw_integer_inputs_exact_under_split(gpu_lib, layout):
    # small integers: every partial sum is exact, so any order or split agrees
    T, R, C = 2048, 64, 128
    X = synth.integer_bf16((T, C), -3, 3, 1031)
    dY = synth.integer_bf16((T, R), -3, 3, 1032)
    mask = _mask_rows(R, list(range(0, 64, 3)))
    _check([(X, [(dY, mask)])], exact=True, repeat=2, layout=layout)


@LAYOUTS
def test_dw_empty_full_and_one_per_tile(gpu_lib, layout):
    T, R, C = 128, 256, 64
    X = synth.normal_bf16((T, C), 1.0, 1041)
    dY = synth.normal_bf16((T, R), 0.01, 1042)
    empty = np.zeros(R, np.uint8)
    full = np.ones(R, np.uint8)
    one = _mask_rows(R, synth.one_per_tile_rows(R, 1543))
    _check([(X, [(dY, empty), (dY, full), (dY, one)])], layout=layout)


@LAYOUTS
def test_dw_groups_share_x_and_span_mblocks(gpu_lib, layout):
    # three matrices on one input with 11 active tiles (two M-blocks), plus a
    # second group with its own input
    T, C = 192, 264
    X1 = synth.normal_bf16((T, C), 1.0, 1051)
    X2 = synth.normal_bf16((T, 96), 1.0, 1052)
    mats1 = []
    for i, (R, k) in enumerate([(320, 100), (128, 40), (96, 10)]):
        mats1.append((synth.normal_bf16((T, R), 0.01, 1060 + i), _mask_rows(R, synth.clustered_rows(R, k, 1560 + i))))
    mats2 = [(synth.normal_bf16((T, 200), 0.01, 1070), _mask_rows(200, synth.clustered_rows(200, 20, 1570)))]
    _check([(X1, mats1), (X2, mats2)], layout=layout)


@LAYOUTS
def test_dw_long_token_axis_split(gpu_lib, layout):
    # few tiles and many tokens: the launch splits the token axis many ways
    T, R, C = 4096, 128, 128
    X = synth.normal_bf16((T, C), 1.0, 1081)
    dY = synth.normal_bf16((T, R), 0.01, 1082)
    mask = _mask_rows(R, synth.clustered_rows(R, 70, 1581))
    _check([(X, [(dY, mask)])], repeat=3, layout=layout)


@LAYOUTS
def test_dw_tile_aligned_quarter_slices(gpu_lib, layout):
    # 50 output tiles of 4 rounds: 200 workgroups each take exactly a quarter
    # of a 256-column tile (slices aligned to the tiles, four partial sums a
    # tile); the 128-column shape would have 100 tiles, too few for half of
    # 256 CUs
    T, R, C = 1024, 96, 50 * 256
    X = synth.normal_bf16((T, C), 1.0, 1601)
    dY = synth.normal_bf16((T, R), 0.01, 1602)
    mask = _mask_rows(R, synth.clustered_rows(R, 40, 1603))
    _check([(X, [(dY, mask)])], repeat=2, layout=layout)


@LAYOUTS
def test_dw_narrow_whole_tiles(gpu_lib, layout):
    # 200 output tiles of 128 columns (the last one ragged), each one
    # workgroup's over a ragged token axis (700 of 1024 padded tokens; odd
    # workgroups start halfway and wrap); three packed tiles, so two of the
    # eight waves only copy
    T, R, C = 700, 96, 199 * 128 + 40
    X = synth.normal_bf16((T, C), 1.0, 1621)
    dY = synth.normal_bf16((T, R), 0.01, 1622)
    mask = _mask_rows(R, synth.clustered_rows(R, 70, 1623))
    _check([(X, [(dY, mask)])], repeat=2, layout=layout)


@LAYOUTS
def test_dw_narrow_tiles_two_groups_exact(gpu_lib, layout):
    # 128-column tiles over two groups (100 tiles of a 4-tile M-block and 94
    # of a 1-tile one; 1000 and 600 tokens, one round count) on small
    # integers: the two token halves' sums add exactly, so the result is the
    # exact product
    g1 = (synth.integer_bf16((1000, 100 * 128), -3, 3, 1631),
          [(synth.integer_bf16((1000, 128), -3, 3, 1632), _mask_rows(128, synth.clustered_rows(128, 100, 1633)))])
    g2 = (synth.integer_bf16((600, 12000), -3, 3, 1634),
          [(synth.integer_bf16((600, 64), -3, 3, 1635), _mask_rows(64, synth.clustered_rows(64, 20, 1636)))])
    _check([g1, g2], exact=True, layout=layout)


@LAYOUTS
@pytest.mark.parametrize("n_tiles", [5, 7, 8])
def test_dw_narrow_wave_per_tile(gpu_lib, layout, n_tiles):
    # 5-8 packed tiles in a narrow launch: one M-block of 64-column tiles,
    # one wave per packed tile (151 tiles, the last one ragged; 700 of 1024
    # padded tokens, odd workgroups start halfway and wrap); rows spread over
    # exactly n_tiles 32-row tiles, so both layouts take this shape
    T, R, C = 700, 8 * 32, 150 * 64 + 40
    rng = np.random.default_rng(1640 + n_tiles)
    rows = []
    for t in range(n_tiles):
        rows += list(32 * t + np.sort(rng.choice(32, 31 if t % 2 else 32, replace=False)))
    X = synth.normal_bf16((T, C), 1.0, 1641)
    dY = synth.normal_bf16((T, R), 0.01, 1642)
    _check([(X, [(dY, _mask_rows(R, rows))])], repeat=2, layout=layout)


@LAYOUTS
def test_dw_narrow_wave_per_tile_beside_narrow_exact(gpu_lib, layout):
    # the 1% layer's shape in small: a group of 7 packed tiles over two
    # matrices (64 tiles of 64 columns) beside a 2-tile group (64 tiles of 128
    # columns) in one narrow launch, on small integers (exact products)
    g1 = (synth.integer_bf16((1000, 4096), -3, 3, 1651),
          [(synth.integer_bf16((1000, 128), -3, 3, 1652), _mask_rows(128, list(range(0, 128)))),
           (synth.integer_bf16((1000, 160), -3, 3, 1653), _mask_rows(160, list(range(0, 90)) + [100, 127]))])
    g2 = (synth.integer_bf16((600, 8192), -3, 3, 1654),
          [(synth.integer_bf16((600, 64), -3, 3, 1655), _mask_rows(64, synth.clustered_rows(64, 40, 1656)))])
    _check([g1, g2], exact=True, layout=layout)


def _tile_rows(tiles, seed, drop=(1, 3)):
    """Rows of the given 32-row tiles, all but a row or two of some, so that
    both layouts see exactly those tiles."""
    rng = np.random.default_rng(seed)
    rows = []
    for i, t in enumerate(tiles):
        keep = 32 - drop[i % len(drop)] if i % 2 else 32
        rows += list(32 * t + np.sort(rng.choice(32, keep, replace=False)))
    return rows


@LAYOUTS
def test_dw_narrow_wave_per_tile_128_columns(gpu_lib, layout):
    # 8 packed tiles over 19240 columns: one wave per tile over 64 columns
    # would need 301 workgroups, so the group takes 128-column tiles (151,
    # the last one ragged) with one wave per packed tile over all 128 tokens
    # of a chunk; ragged token axis, odd workgroups start halfway
    T, R, C = 700, 256, 150 * 128 + 40
    X = synth.normal_bf16((T, C), 1.0, 1661)
    dY = synth.normal_bf16((T, R), 0.01, 1662)
    _check([(X, [(dY, _mask_rows(R, _tile_rows(range(8), 1663)))])], repeat=2, layout=layout)


@LAYOUTS
def test_dw_narrow_three_shapes_exact(gpu_lib, layout):
    # one narrow launch with all three whole-tile shapes, on small integers
    # (exact products): 14 packed tiles over two matrices (two M-blocks of 7,
    # 128-column tiles, one wave per packed tile: 64 workgroups), 8 tiles
    # (one M-block of 64-column tiles: 64) and 3 tiles over 11008 columns
    # (two waves per packed tile: 86)
    T = 600
    ga = (synth.integer_bf16((T, 4096), -3, 3, 1671),
          [(synth.integer_bf16((T, 320), -3, 3, 1672), _mask_rows(320, _tile_rows([0, 2, 3, 5, 6, 8, 9], 1673))),
           (synth.integer_bf16((T, 256), -3, 3, 1674), _mask_rows(256, _tile_rows([0, 1, 2, 4, 5, 6, 7], 1675)))])
    gb = (synth.integer_bf16((T, 4096), -3, 3, 1676),
          [(synth.integer_bf16((T, 256), -3, 3, 1677), _mask_rows(256, _tile_rows(range(8), 1678)))])
    gc = (synth.integer_bf16((T, 11008), -3, 3, 1679),
          [(synth.integer_bf16((T, 128), -3, 3, 1680), _mask_rows(128, _tile_rows([0, 1, 3], 1681)))])
    _check([ga, gb, gc], exact=True, layout=layout)


@LAYOUTS
def test_dw_narrow_two_rounds(gpu_lib, layout):
    # 9 packed tiles (3 M-blocks of 4 would take team slices) over 23040
    # columns: two M-blocks of 128-column tiles, one wave per packed tile,
    # 360 whole tiles, so two rounds of workgroups (more tiles than CUs);
    # ragged token axis
    T, R, C = 200, 320, 180 * 128
    X = synth.normal_bf16((T, C), 1.0, 1691)
    dY = synth.normal_bf16((T, R), 0.01, 1692)
    _check([(X, [(dY, _mask_rows(R, _tile_rows([0, 1, 2, 4, 5, 6, 7, 8, 9], 1693)))])], repeat=2, layout=layout)


@LAYOUTS
def test_dw_narrow_one_wave_two_mblocks_64_columns(gpu_lib, layout):
    # 10 packed tiles over 8192 columns: two M-blocks of 5 with one wave per
    # packed tile over 64 columns (256 whole tiles, every CU), ragged tokens;
    # the planner's choice is checked first so the case keeps its shape
    T, R, C = 300, 320, 8192
    rows = _tile_rows(range(10), 1695)
    plan = _lib.sft_plan_rows(_mask_rows(R, rows))
    got = _lib.sft_probe_dw_plan([(T, C, layout, [plan])], 256)
    assert got == [{"kind": "narrow", "workgroups": 256, "groups": [(1, 2, 128)]}]
    X = synth.normal_bf16((T, C), 1.0, 1696)
    dY = synth.normal_bf16((T, R), 0.01, 1697)
    _check([(X, [(dY, _mask_rows(R, rows))])], repeat=2, layout=layout)


@LAYOUTS
def test_dw_one_tile_per_workgroup(gpu_lib, layout):
    # 200 output tiles of one round: every workgroup computes one whole tile
    # (no partial sums at all)
    T, R, C = 256, 64, 200 * 256
    X = synth.normal_bf16((T, C), 1.0, 1611)
    dY = synth.normal_bf16((T, R), 0.01, 1612)
    mask = _mask_rows(R, synth.clustered_rows(R, 30, 1613))
    _check([(X, [(dY, mask)])], layout=layout)


def test_dw_layouts_agree_bitwise_on_integer_inputs(gpu_lib):
    # packed and whole-tile layouts sum the same exact products: bit-identical
    T, R, C = 640, 200, 136
    X = synth.integer_bf16((T, C), -3, 3, 1091)
    dY = synth.integer_bf16((T, R), -3, 3, 1092)
    mask = _mask_rows(R, synth.one_per_tile_rows(R, 1591))
    a, plans = _run([(X, [(dY, mask)])], layout=_lib.SFT_DW_TILES)
    b, _ = _run([(X, [(dY, mask)])], layout=_lib.SFT_DW_PACKED)
    n = plans[0].n_active
    assert np.array_equal(a[0][:n], b[0][:n])
    assert np.array_equal(a[0][:n], oracle.masked_dw(dY, X, plans[0].active_rows))


@LAYOUTS
def test_dw_more_groups_than_one_launch(gpu_lib, layout):
    # ten groups of one matrix: the call splits into two launches that reuse
    # one workspace in stream order
    T = 320
    groups = []
    for i in range(10):
        C, R = 64 + 8 * i, 40 + 13 * i
        X = synth.normal_bf16((T, C), 1.0, 1200 + i)
        dY = synth.normal_bf16((T, R), 0.01, 1300 + i)
        groups.append((X, [(dY, _mask_rows(R, synth.clustered_rows(R, 5 + i, 1400 + i)))]))
    _check(groups, layout=layout)


@LAYOUTS
def test_dw_many_rows_tiny_shape(gpu_lib, layout):
    # 2^22 + 96 active rows of one token and 8 columns: 131075 packed tiles in
    # 32769 M-blocks, so an M-block's first packed tile (block * packed tiles /
    # blocks) needs more than 32 bits on the way; one token of small integers
    # makes the product exact
    T, R, C = 1, (1 << 22) + 96, 8
    X = synth.integer_bf16((T, C), -3, 3, 1501)
    dY = synth.integer_bf16((T, R), -3, 3, 1502)
    _check([(X, [(dY, np.ones(R, np.uint8))])], exact=True, layout=layout)


def test_dw_rejects_bad_shapes(gpu_lib):
    T, R, C = 16, 32, 12
    X = bf16_dev(synth.normal_bf16((T, C), 1.0, 1))
    plan = _lib.sft_plan_rows(np.ones(R, np.uint8))
    out = torch.zeros((R, C), dtype=torch.float32, device="cuda")
    g = [_lib.DwGroup(X, [_lib.DwMat(bf16_dev(synth.normal_bf16((T, R), 0.01, 2)), plan.to_device(), out)])]
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_masked_dw(g, None)
    assert e.value.code == _lib.SFT_ESHAPE


def test_dw_rejects_c_beyond_2_24(gpu_lib):
    # one token of 2^24 + 8 columns: T*C is fine, C itself is past the limit
    T, R, C = 1, 32, (1 << 24) + 8
    X = torch.zeros((T, C), dtype=torch.bfloat16, device="cuda")
    plan = _lib.sft_plan_rows(_mask_rows(R, [0]))
    out = torch.zeros((1, C), dtype=torch.float32, device="cuda")
    g = [_lib.DwGroup(X, [_lib.DwMat(bf16_dev(synth.normal_bf16((T, R), 0.01, 3)), plan.to_device(), out)])]
    with pytest.raises(_lib.SftError):
        _lib.sft_masked_dw_workspace(g)
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_masked_dw(g, None)
    assert e.value.code == _lib.SFT_ENOTSUP


# ------------------------------------------------------------------ embedding


def _emb_case(V, T, d, seed, integer=False):
    toks_windows = [synth.zipf_tokens(T, V, 1.1, seed + w) for w in range(4)]
    ch = np.zeros(V, np.float32)
    for w in toks_windows:
        mask = _lib.sft_conductor_window(ch, w)
    tokens = toks_windows[-1]
    plan = _lib.sft_plan_rows(mask)
    row_ptr, pos = _lib.sft_plan_embedding(plan, tokens)
    dY = synth.integer_bf16((T, d), -3, 3, seed + 9) if integer else synth.normal_bf16((T, d), 0.01, seed + 9)
    return tokens, plan, row_ptr, pos, dY


@pytest.mark.parametrize("integer", [False, True])
def test_embedding_dw(gpu_lib, integer):
    V, T, d = 2000, 1024, 264
    tokens, plan, row_ptr, pos, dY = _emb_case(V, T, d, 1100, integer)
    assert plan.n_active > 0
    out = torch.full((plan.n_active + 2, d), CANARY, dtype=torch.float32, device="cuda")
    _lib.sft_embedding_dw(bf16_dev(dY), dev(row_ptr), dev(pos if pos.size else np.zeros(1, np.int32)),
                          plan.n_active, out[:plan.n_active])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isnan(got[plan.n_active:]))
    want = oracle.embedding_dw(dY, tokens, plan.active_rows)
    if integer:
        assert np.array_equal(got[:plan.n_active], want)
    else:
        dw_close(got[:plan.n_active], want)


def test_embedding_dw_hot_rows(gpu_lib):
    # a 50-row vocabulary and 2048 tokens: the hottest row has more than 512
    # positions, so each of its 8 position shares spans two 64-position reads
    # and more than one batch of 32 loads (and the 520 columns leave a ragged
    # 8-column slab); integer values make every sum exact
    V, T, d = 50, 2048, 520
    tokens, plan, row_ptr, pos, dY = _emb_case(V, T, d, 1200, integer=True)
    assert np.diff(row_ptr).max() > 8 * 64
    out = torch.full((plan.n_active + 2, d), CANARY, dtype=torch.float32, device="cuda")
    _lib.sft_embedding_dw(bf16_dev(dY), dev(row_ptr), dev(pos), plan.n_active, out[:plan.n_active])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isnan(got[plan.n_active:]))
    assert np.array_equal(got[:plan.n_active], oracle.embedding_dw(dY, tokens, plan.active_rows))


@LAYOUTS
def test_dw_many_mblocks_column_major_tiles(gpu_lib, layout):
    # groups of three and more M-blocks number their output tiles column block
    # by column block and keep X in L2: 450 active rows of two matrices on one
    # input (15 packed tiles, 4 M-blocks; tile layout more), ragged C and T,
    # beside a 2-M-block group, repeated for determinism; and an integer case
    # that must be exact
    T, C = 200, 520
    X1 = synth.normal_bf16((T, C), 1.0, 1900)
    mats1 = [(synth.normal_bf16((T, R), 0.01, 1901 + i), _mask_rows(R, synth.clustered_rows(R, k, 1910 + i)))
             for i, (R, k) in enumerate([(700, 300), (400, 150)])]
    X2 = synth.normal_bf16((T, 136), 1.0, 1920)
    mats2 = [(synth.normal_bf16((T, 300), 0.01, 1921), _mask_rows(300, synth.clustered_rows(300, 170, 1922)))]
    _check([(X1, mats1), (X2, mats2)], repeat=2, layout=layout)
    Xi = synth.integer_bf16((T, C), -3, 3, 1930)
    matsi = [(synth.integer_bf16((T, 900), -2, 2, 1931), _mask_rows(900, synth.clustered_rows(900, 420, 1932)))]
    _check([(Xi, matsi)], exact=True, layout=layout)


@LAYOUTS
def test_dw_team_slices_cut_tiles(gpu_lib, layout):
    # a group of three or more M-blocks puts the launch on team slicing (too
    # few columns for whole narrow tiles): a 5-M-block and a 2-M-block group
    # (packed; more in the tile layout), 6 column blocks each, 4096 tokens
    # (16 rounds a tile), share the CUs in teams of 3-4 rounds, so most tiles
    # are cut at ragged rounds into up to five partial sums added by the
    # fix-up; repeated for determinism
    T, C = 4096, 1496
    X1 = synth.normal_bf16((T, C), 1.0, 2100)
    mats1 = [(synth.normal_bf16((T, R), 0.01, 2101 + i), _mask_rows(R, synth.clustered_rows(R, k, 2110 + i)))
             for i, (R, k) in enumerate([(900, 330), (600, 200)])]
    X2 = synth.normal_bf16((T, C), 1.0, 2120)
    mats2 = [(synth.normal_bf16((T, 512), 0.01, 2121), _mask_rows(512, synth.clustered_rows(512, 200, 2122)))]
    _check([(X1, mats1), (X2, mats2)], repeat=2, layout=layout)


@LAYOUTS
def test_dw_million_token_axis_exact(gpu_lib, layout):
    # T = 2^20 tokens, one 32-row tile, 8 columns: the one output tile is cut
    # into one slice per CU (256 partial tiles, added by the fix-up in slice
    # order); small integers keep every partial sum exact, so the result is
    # bit for bit the oracle's
    T, R, C = 1 << 20, 32, 8
    X = synth.integer_bf16((T, C), -2, 2, 2201)
    dY = synth.integer_bf16((T, R), -2, 2, 2202)
    mask = _mask_rows(R, [0, 3, 4, 5, 17, 30, 31])
    _check([(X, [(dY, mask)])], exact=True, layout=layout)
