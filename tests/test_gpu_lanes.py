"""GPU test of the step schedule the benchmark uses: independent layers whose
steps alternate between three streams (the lanes) end in exactly the state
the same steps reach one after the other on one stream.  Each layer has its
own plan, workspace, gradients and optimizer state, so no two lanes share a
byte; the test checks that nothing in the library (a static buffer, a
launch's host-side state) couples them.  Method: "Sparse-First Fine-Tuning:
Full-Weight Training at the Cost of the Active Set", sections 2.2-2.3 (masked
dW and the sparse update, one call per layer step) and 2.6 (one plan upload
per step).
"""
import numpy as np
import pytest
import torch

from sparse_full_weight_amd import _lib, synth
from tests.gpu_helpers import GpuMat, adam_dev, assert_state_equal, bf16_dev, make_state

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)


class _Layer:
    """One layer: a group of two matrices on one input, its pinned plan
    (active rows of both matrices, uploaded every step), state and calls."""

    def __init__(self, seed, T, C, R, k):
        self.X = synth.normal_bf16((T, C), 1.0, seed)
        self.mats = []
        for mi in range(2):
            s = seed + 10 * (mi + 1)
            dY = synth.normal_bf16((T, R), 0.01, s)
            mask = synth.mask_from_rows(R, synth.clustered_rows(R, k, s + 1))
            plan = _lib.sft_plan_rows(mask)
            st = make_state(R, C, s + 2, plan.n_active + 2, True)
            self.mats.append((dY, plan, st))

    def build(self):
        """Fresh device copies of everything, a pinned plan buffer and the prepared fused call."""
        self.host = torch.from_numpy(np.concatenate([p.active_rows for _, p, _ in self.mats]).astype(np.int32))
        self.host = self.host.pin_memory()
        self.plan_dev = torch.zeros_like(self.host, device="cuda")
        groups, upd, self.gm = [], [], []
        dws, off = [], 0
        for dY, plan, st in self.mats:
            n = plan.n_active
            rows_dev = self.plan_dev[off:off + n]
            off += n
            dplan = plan.to_device()
            dplan = _lib.DevicePlan(plan, rows_dev, dplan.active_tiles, dplan.active_bits, dplan.tile_first)
            m = GpuMat(st, np.zeros((n, self.X.shape[1]), np.float32), plan.active_rows, np.arange(n), None)
            m.rows = rows_dev
            dws.append(_lib.DwMat(bf16_dev(dY), dplan, m.G))
            upd.append(m.upd())
            self.gm.append(m)
        groups.append(_lib.DwGroup(bf16_dev(self.X), dws, _lib.SFT_DW_PACKED))
        nbytes = _lib.sft_masked_dw_workspace(groups)
        self.ws = torch.zeros(max(nbytes // 4, 1), dtype=torch.int32, device="cuda")
        self.call = _lib.prepare_masked_dw_update(groups, self.ws, upd, adam_dev(**HP))

    def step(self, stream):
        _lib.sft_plan_upload(self.plan_dev, self.host, stream=stream)
        self.call(stream)

    def state(self):
        return [m.to_state() for m in self.gm]


@pytest.mark.parametrize("shape", [(512, 1024, 512, 60), (1024, 25000, 96, 60)], ids=["stream-k", "narrow"])
def test_lanes_reach_the_one_stream_state(gpu_lib, shape):
    T, C, R, k = shape
    layers = [_Layer(7000 + 100 * i, T, C, R, k) for i in range(3)]
    steps = 4
    # one stream
    for L in layers:
        L.build()
    main = torch.cuda.current_stream()
    for _ in range(steps):
        for L in layers:
            L.step(main)
    torch.cuda.synchronize()
    want = [L.state() for L in layers]
    for L, w in zip(layers, want):   # the steps did move every matrix
        for (_, plan, st), ws in zip(L.mats, w):
            assert not np.array_equal(ws.delta, st.delta) and np.all(ws.t[:plan.n_active] == st.t[:plan.n_active] + steps)
    # three lanes: layer i on lane i, the steps enqueued in the same order
    for L in layers:
        L.build()
    lanes = [main, torch.cuda.Stream(), torch.cuda.Stream()]
    start = torch.cuda.Event()
    start.record(main)
    for s in lanes[1:]:
        s.wait_event(start)
    for _ in range(steps):
        for i, L in enumerate(layers):
            L.step(lanes[i])
    torch.cuda.synchronize()
    for i, L in enumerate(layers):
        for j, (a, b) in enumerate(zip(L.state(), want[i])):
            assert_state_equal(a, b, f"layer {i} matrix {j}")
