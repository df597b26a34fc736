"""Shared helpers of the GPU parity tests: move seeded inputs to the GPU and
results back, so that the HIP path and the oracle see the same bytes."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_full_weight_amd import _lib, synth

DEV = "cuda"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def u16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def adam_dev(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, t_max=20000) -> _lib.Adam:
    bc1, bc2 = _lib.sft_bias_table(beta1, beta2, t_max)
    return _lib.Adam(lr, beta1, beta2, eps, dev(bc1), dev(bc2), weight_decay)


class GpuMat:
    """GPU copy of an oracle.MatState plus the step's row list and gradient."""

    def __init__(self, st: oracle.MatState, G: np.ndarray, rows: np.ndarray, slot: np.ndarray,
                 fresh: np.ndarray | None, with_live: bool = True):
        self.q = dev(st.q)
        self.s = dev(st.s)
        self.delta = dev(st.delta)
        self.m = u16_dev(st.m)
        self.v = u16_dev(st.v)
        self.t = dev(st.t)
        self.w_live = u16_dev(st.w_live) if (with_live and st.w_live is not None) else None
        self.rows = dev(np.asarray(rows, np.int32))
        self.slot = dev(np.asarray(slot, np.int32))
        self.fresh = None if fresh is None else dev(np.asarray(fresh, np.uint8))
        self.G = dev(np.ascontiguousarray(G, np.float32))
        self.n = int(np.asarray(rows).size)

    def upd(self) -> _lib.UpdMat:
        return _lib.UpdMat(self.q, self.s, self.delta, self.m, self.v, self.t, self.rows, self.slot, self.G,
                           self.n, self.fresh, self.w_live)

    def to_state(self) -> oracle.MatState:
        return oracle.MatState(self.q.cpu().numpy(), self.s.cpu().numpy(), self.delta.cpu().numpy(),
                               host_u16(self.m), host_u16(self.v), self.t.cpu().numpy(),
                               None if self.w_live is None else host_u16(self.w_live))


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view({1: np.uint8, 2: np.uint16, 4: np.uint32}[a.itemsize])


def assert_state_equal(got: oracle.MatState, want: oracle.MatState, what: str = "") -> None:
    """Bitwise equality of every state array."""
    for name in ("q", "s", "delta", "m", "v", "t", "w_live"):
        a, b = getattr(got, name), getattr(want, name)
        if a is None and b is None:
            continue
        bad = np.argwhere(_bits(a) != _bits(b))
        if bad.size:
            raise AssertionError(f"{what} {name}: {len(bad)} mismatches, first at {bad[:5].tolist()}")


def dw_close(got: np.ndarray, want: np.ndarray, rel: float = 1e-3) -> None:
    """Masked-dW tolerance: |gpu - oracle| <= rel * max(|oracle|, 1e-3 * max_c |oracle row|).

    bf16 inputs, fp32 accumulation on the GPU against an fp64 sum rounded once;
    the per-row floor keeps cancellation near zero from failing a correct kernel."""
    assert got.shape == want.shape, (got.shape, want.shape)
    if want.size == 0:
        return
    row_max = np.max(np.abs(want), axis=1, keepdims=True)
    bound = rel * np.maximum(np.abs(want), 1e-3 * row_max)
    bad = np.abs(got.astype(np.float64) - want.astype(np.float64)) > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"dW mismatch at {bad.sum()} elements, e.g. {idx.tolist()}: "
                             f"{[(float(got[i, j]), float(want[i, j])) for i, j in idx]}")


def make_state(R: int, C: int, seed: int, n_slots: int, mid_run: bool) -> oracle.MatState:
    q, s, delta = synth.quant_state(R, C, seed)
    m, v, t = synth.moments(n_slots, C, seed + 1, mid_run)
    w_live = np.full((R, C), 0xA5A5, np.uint16)
    return oracle.MatState(q, s, delta, m, v, t, w_live)
