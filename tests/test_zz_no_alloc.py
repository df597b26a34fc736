"""The allocation-free fused call (sft_masked_dw_update_noalloc) against the
call it varies (sft_masked_dw_update with a caller workspace): the masked dW
of a group of matrices with the sparse update fused in ("Sparse-First
Fine-Tuning: Full-Weight Training at the Cost of the Active Set", sections
2.2 and 2.3), run on two inputs in a row -- the second smaller, so that it
runs over what the first left in the library's scratch array -- must leave
every state array bit-identical to the workspace call.  A call whose groups
need more workspace than the array holds is rejected before any launch."""
import numpy as np
import pytest
import torch

from sparse_full_weight_amd import _lib, synth
from tests.gpu_helpers import GpuMat, adam_dev, assert_state_equal, bf16_dev, make_state

pytestmark = pytest.mark.gpu


def _case(T, shapes, density, seed):
    """One group: matrices sharing X, clustered masks, mid-run states."""
    C = shapes[0][1]
    X = synth.normal_bf16((T, C), 1.0, seed)
    mats = []
    for i, (R, _) in enumerate(shapes):
        rows = synth.clustered_rows(R, max(1, round(density * R)), seed + 10 + i)
        plan = _lib.sft_plan_rows(synth.mask_from_rows(R, rows))
        st = make_state(R, C, seed + 20 + i, plan.n_active + 3, True)
        g = synth.rng(seed + 30 + i)
        slot = g.choice(plan.n_active + 3, size=plan.n_active, replace=False).astype(np.int32)
        dY = synth.normal_bf16((T, R), 0.01, seed + 40 + i)
        mats.append((st, plan, slot, dY))
    return X, mats


def _run(case, noalloc):
    X, mats = case
    dms, upd, gms = [], [], []
    for st, plan, slot, dY in mats:
        dplan = plan.to_device()
        out = torch.zeros((max(plan.n_active, 1), st.q.shape[1]), dtype=torch.float32, device="cuda")
        dms.append(_lib.DwMat(bf16_dev(dY), dplan, out[:plan.n_active]))
        gm = GpuMat(st, np.zeros((plan.n_active, st.q.shape[1]), np.float32), plan.active_rows, slot, None)
        gm.rows = dplan.active_rows
        gm.G = out[:plan.n_active]
        gms.append(gm)
        upd.append(gm.upd())
    groups = [_lib.DwGroup(bf16_dev(X), dms, _lib.SFT_DW_PACKED)]
    hp = adam_dev()
    if noalloc:
        _lib.sft_masked_dw_update_noalloc(groups, upd, hp)
    else:
        ws = torch.zeros(max(_lib.sft_masked_dw_workspace(groups) // 4, 1), dtype=torch.int32, device="cuda")
        _lib.sft_masked_dw_update(groups, ws, upd, hp)
    torch.cuda.synchronize()
    return [gm.to_state() for gm in gms]


def test_noalloc_call_equals_the_workspace_call_twice_in_a_row(gpu_lib):
    big = _case(1000, [(2048, 1024), (1100, 1024), (4096, 1024)], 0.04, 9100)
    small = _case(200, [(512, 256), (300, 256)], 0.10, 9200)
    for what, case in (("first (larger) call", big), ("second (smaller) call", small)):
        want = _run(case, noalloc=False)
        got = _run(case, noalloc=True)
        for i, (a, b) in enumerate(zip(got, want)):
            assert_state_equal(a, b, f"{what}, matrix {i}")


def test_noalloc_call_on_narrow_whole_tiles(gpu_lib):
    # narrow whole tiles (no partial rows): 7 packed tiles over 8192 columns
    # take one wave per packed tile over 64 columns (128 tiles), then a
    # smaller call on 4 packed tiles over 8192 columns (stream-K slices)
    narrow = _case(600, [(512, 8192), (512, 8192)], 110 / 512, 9300)
    small = _case(300, [(256, 8192)], 0.45, 9400)
    shape = [(600, 8192, _lib.SFT_DW_PACKED, [p for _, p, _, _ in narrow[1]])]
    assert _lib.sft_probe_dw_plan(shape, 256)[0]["kind"] == "narrow"
    for what, case in (("first (narrow) call", narrow), ("second (smaller) call", small)):
        want = _run(case, noalloc=False)
        got = _run(case, noalloc=True)
        for i, (a, b) in enumerate(zip(got, want)):
            assert_state_equal(a, b, f"{what}, matrix {i}")


def test_noalloc_call_rejects_groups_beyond_the_scratch_array(gpu_lib):
    T, R, C = 1 << 18, 2048, 8
    X = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    plan = _lib.sft_plan_rows(np.ones(R, np.uint8)).to_device()
    out = torch.empty((R, C), dtype=torch.float32, device="cuda")
    groups = [_lib.DwGroup(X, [_lib.DwMat(dY, plan, out)], _lib.SFT_DW_PACKED)]
    assert _lib.sft_masked_dw_workspace(groups) > _lib.sft_noalloc_scratch_bytes()
    st = make_state(R, C, 9300, R, False)
    gm = GpuMat(st, np.zeros((R, C), np.float32), np.arange(R, dtype=np.int32), np.arange(R, dtype=np.int32), None)
    gm.rows = plan.active_rows
    gm.G = out
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_masked_dw_update_noalloc(groups, [gm.upd()], adam_dev())
    assert e.value.code == _lib.SFT_ECAPACITY
    torch.cuda.synchronize()
