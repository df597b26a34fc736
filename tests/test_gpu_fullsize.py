"""GPU parity at the full size of one Llama-7B-shaped layer, in the launch
configuration the benchmark times: q, k, v, o 4096x4096, gate and up
11008x4096, down 4096x11008, 4096 tokens, 1% of each matrix's rows active
(row-tracker masks over seeded magnitudes, clustered in 32-row tiles), all
seven masked dW products in one call (q/k/v and gate/up sharing their input),
then the sparse update with fused write-back of all seven in one call.

The oracle cannot afford every row at this size, so it checks a seeded
sample of active rows of every matrix: their dW rows element by element
(same tolerance as the small cases), and their whole update (q, s, delta, m,
v, t and the live bf16 row) bit for bit, given the GPU's dW.  Rows outside
the active set are checked bit-unchanged on a sample.  Method:
"Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the Active
Set", sections 2.1-2.3.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_full_weight_amd import _lib, synth
from tests.gpu_helpers import adam_dev, bf16_dev, dev, dw_close, host_u16

pytestmark = pytest.mark.gpu

T = 4096
DENSITY = 0.01
ROWS_PER_MAT = 4          # sampled active rows per matrix


def _layer(seed):
    """Seeded inputs, masks and state of one layer (host copies)."""
    mats = {}
    X = {}
    for gi, (gname, members) in enumerate(synth.LLAMA7B_GROUPS):
        C = synth.LLAMA7B[members[0]][1]
        X[gname] = synth.normal_bf16((T, C), 1.0, seed + 10 * gi)
        for name in members:
            R, Cm = synth.LLAMA7B[name]
            mi = list(synth.LLAMA7B).index(name)
            hot = synth.clustered_rows(R, round(DENSITY * R), seed + 100 + mi)
            mag = synth.tracker_magnitudes(R, hot, seed + 200 + mi)
            mask = _lib.sft_tracker_window(np.zeros(R, np.float32), mag)
            q, s, delta = synth.quant_state(R, Cm, seed + 300 + mi)
            mats[name] = {"R": R, "C": Cm, "group": gname, "mask": mask,
                          "dY": synth.normal_bf16((T, R), 0.01, seed + 400 + mi),
                          "q": q, "s": s, "delta": delta}
    return X, mats


@pytest.fixture(scope="module")
def layer():
    return _layer(7000)


@pytest.mark.parametrize("layout", [_lib.SFT_DW_PACKED, _lib.SFT_DW_TILES], ids=["packed", "tiles"])
def test_llama7b_layer_dw_and_update_sampled(gpu_lib, layer, layout):
    X, mats = layer
    rng = synth.rng(7777)
    Xd = {g: bf16_dev(x) for g, x in X.items()}
    groups, gpu = [], {}
    for gname, members in synth.LLAMA7B_GROUPS:
        ms = []
        for name in members:
            m = mats[name]
            plan = _lib.sft_plan_rows(m["mask"])
            assert plan.n_active == round(DENSITY * m["R"])
            out = torch.full((plan.n_active + 1, m["C"]), float("nan"), dtype=torch.float32, device="cuda")
            gpu[name] = {"plan": plan, "dplan": plan.to_device(), "out": out}
            ms.append(_lib.DwMat(bf16_dev(m["dY"]), gpu[name]["dplan"], out[:plan.n_active]))
        groups.append(_lib.DwGroup(Xd[gname], ms, layout))
    nbytes = _lib.sft_masked_dw_workspace(groups)
    ws = torch.zeros(max(nbytes // 4, 1), dtype=torch.int32, device="cuda")
    _lib.sft_masked_dw(groups, ws)
    torch.cuda.synchronize()

    # dW: sampled active rows of every matrix against the fp64 oracle
    G_host = {}
    for name, m in mats.items():
        plan = gpu[name]["plan"]
        got = gpu[name]["out"].cpu().numpy()
        assert np.all(np.isnan(got[plan.n_active:])), "write past the last active row"
        G_host[name] = got[:plan.n_active]
        pick = np.sort(rng.choice(plan.n_active, size=ROWS_PER_MAT, replace=False))
        pick[-1] = plan.n_active - 1                      # the last active row, always
        want = oracle.masked_dw(m["dY"], X[m["group"]], plan.active_rows[pick])
        dw_close(G_host[name][pick], want)

    # update with fused write-back of all seven matrices in one call, fresh moments
    hp = adam_dev()
    upd, dev_state = [], {}
    for name, m in mats.items():
        plan = gpu[name]["plan"]
        n = plan.n_active
        st = {"q": dev(m["q"]), "s": dev(m["s"]), "delta": dev(m["delta"]),
              "m": torch.zeros((n, m["C"]), dtype=torch.int16, device="cuda"),
              "v": torch.zeros((n, m["C"]), dtype=torch.int16, device="cuda"),
              "t": torch.zeros(n, dtype=torch.int32, device="cuda"),
              "w": torch.zeros((m["R"], m["C"]), dtype=torch.int16, device="cuda"),
              "slot": dev(np.arange(n, dtype=np.int32)),
              "fresh": dev(np.ones(n, np.uint8))}
        dev_state[name] = st
        upd.append(_lib.UpdMat(st["q"], st["s"], st["delta"], st["m"], st["v"], st["t"], gpu[name]["dplan"].active_rows,
                               st["slot"], gpu[name]["out"][:n], n, st["fresh"], st["w"]))
    _lib.sft_sparse_update(upd, hp)
    torch.cuda.synchronize()

    for name, m in mats.items():
        plan = gpu[name]["plan"]
        n, C = plan.n_active, m["C"]
        st = dev_state[name]
        pick = np.sort(rng.choice(n, size=ROWS_PER_MAT, replace=False))
        rows = plan.active_rows[pick]
        # oracle on the sampled rows only: a state holding just those rows
        sub = oracle.MatState(m["q"][rows].copy(), m["s"][rows].copy(), m["delta"][rows].copy(),
                              np.zeros((pick.size, C), np.uint16), np.zeros((pick.size, C), np.uint16),
                              np.zeros(pick.size, np.int32), np.zeros((pick.size, C), np.uint16))
        oracle.sparse_update(sub, G_host[name][pick], np.arange(pick.size, dtype=np.int32),
                             np.arange(pick.size, dtype=np.int32), np.ones(pick.size, np.uint8),
                             lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)
        q = st["q"].cpu().numpy()
        s = st["s"].cpu().numpy()
        delta = st["delta"].cpu().numpy()
        assert np.array_equal(q[rows], sub.q), name
        assert np.array_equal(s[rows].view(np.uint32), sub.s.view(np.uint32)), name
        assert np.array_equal(delta[rows].view(np.uint32), sub.delta.view(np.uint32)), name
        assert np.array_equal(host_u16(st["m"])[pick], sub.m), name
        assert np.array_equal(host_u16(st["v"])[pick], sub.v), name
        assert np.array_equal(st["t"].cpu().numpy()[pick], sub.t), name
        assert np.array_equal(host_u16(st["w"])[rows], sub.w_live), name
        # inactive rows: bit-unchanged state, untouched live weights
        idle = np.setdiff1d(np.arange(m["R"]), plan.active_rows)
        idle = idle[rng.choice(idle.size, size=min(64, idle.size), replace=False)]
        assert np.array_equal(q[idle], m["q"][idle]), name
        assert np.array_equal(s[idle].view(np.uint32), m["s"][idle].view(np.uint32)), name
        assert np.array_equal(delta[idle].view(np.uint32), m["delta"][idle].view(np.uint32)), name
        assert not host_u16(st["w"])[idle].any(), name
