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
        self.e = dev(st.e)
        self.w_live = u16_dev(st.w_live) if (with_live and st.w_live is not None) else None
        self.rows = dev(np.asarray(rows, np.int32))
        self.slot = dev(np.asarray(slot, np.int32))
        self.fresh = None if fresh is None else dev(np.asarray(fresh, np.uint8))
        self.G = dev(np.ascontiguousarray(G, np.float32))
        self.n = int(np.asarray(rows).size)

    def upd(self) -> _lib.UpdMat:
        return _lib.UpdMat(self.q, self.s, self.delta, self.m, self.v, self.t, self.e, self.rows, self.slot,
                           self.G, self.n, self.fresh, self.w_live)

    def to_state(self) -> oracle.MatState:
        return oracle.MatState(self.q.cpu().numpy(), self.s.cpu().numpy(), self.delta.cpu().numpy(),
                               host_u16(self.m), host_u16(self.v), self.t.cpu().numpy(),
                               None if self.w_live is None else host_u16(self.w_live), e=self.e.cpu().numpy())


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view({1: np.uint8, 2: np.uint16, 4: np.uint32}[a.itemsize])


def assert_state_equal(got: oracle.MatState, want: oracle.MatState, what: str = "") -> None:
    """Bitwise equality of every state array."""
    for name in ("q", "s", "delta", "m", "v", "t", "e", "w_live"):
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
    m, v, t, e = synth.moments(n_slots, C, seed + 1, mid_run)
    w_live = np.full((R, C), 0xA5A5, np.uint16)
    return oracle.MatState(q, s, delta, m, v, t, w_live, e=e)


def oracle_dw_threads(dY: np.ndarray, X: np.ndarray, rows: np.ndarray, workers: int | None = None) -> np.ndarray:
    """oracle.masked_dw over row chunks on several host threads (the C oracle
    releases the interpreter lock); the result is the same, row for row."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    rows = np.asarray(rows, np.int32)
    workers = workers or min(16, os.cpu_count() or 1)
    parts = [p for p in np.array_split(rows, max(1, min(workers * 4, rows.size))) if p.size]
    if not parts:
        return np.zeros((0, X.shape[1]), np.float32)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        outs = list(ex.map(lambda p: oracle.masked_dw(dY, X, p), parts))
    return np.concatenate(outs, axis=0)


def _f16_ulp_scaled(x: np.ndarray, e: np.ndarray) -> np.ndarray:
    """One unit in the last place of the scaled fp16 storage of x (exponent e
    per row), in x's units, with the fp16 subnormal spacing as the floor."""
    scale = np.exp2(e.astype(np.float64))[:, None]
    sc = np.minimum(np.abs(x.astype(np.float64)) * scale, 65504.0)
    return (np.spacing(sc.astype(np.float16)).astype(np.float64) + 2.0 ** -24) / scale


def update_gate(got: oracle.MatState, want: oracle.MatState, rows: np.ndarray, slots: np.ndarray,
                what: str, G: np.ndarray, beta1: float = 0.9, beta2: float = 0.999) -> dict:
    """The end-to-end bounds of the update, where the GPU's own dW fed the GPU
    update and the oracle's dW fed the oracle's: rows `rows` of both states
    (moment slots `slots`) are compared and the differences reported.
      - t equal;
      - q' equal except +-1 flips where the oracle's w'/s' lies at the .5
        tie between the two codes, within the rounding of the two sides'
        weights (each flip is reported with its distance to the tie);
      - the rebuilt weight s'q' + delta' and, where q' agrees, delta' within
        1e-3 s';
      - m and v within one unit of their scaled fp16 storage plus what the
        dW tolerance lets through the moment recurrences: with the oracle's
        gradient g (G, row k = rows[k]) and the dW bound
        dg = 1e-3 max(|g|, 1e-3 max|g of the row|), m may move by
        (1 - beta1) dg and v by (1 - beta2)(2|g| dg + dg^2);
      - the live bf16 weights within one bf16 unit.
    """
    rows = np.asarray(rows, np.int64)
    slots = np.asarray(slots, np.int64)
    rep = {"what": what, "rows": int(rows.size), "flips": 0, "flip_tie_dist_ulp": []}
    assert np.array_equal(got.t[slots], want.t[slots]), f"{what}: step counts differ"
    sg, so = got.s[rows].astype(np.float64), want.s[rows].astype(np.float64)
    qg, qo = got.q[rows].astype(np.int32), want.q[rows].astype(np.int32)
    wg = (got.s[rows][:, None] * got.q[rows].astype(np.float32)).astype(np.float32) + got.delta[rows]
    wo = (want.s[rows][:, None] * want.q[rows].astype(np.float32)).astype(np.float32) + want.delta[rows]
    bound = 1e-3 * so[:, None]
    dw = np.abs(wg.astype(np.float64) - wo.astype(np.float64))
    assert np.all(dw <= bound), f"{what}: rebuilt weight off by {float((dw / np.maximum(so[:, None], 1e-30)).max()):.3g} s'"
    rep["max_w_err_over_s"] = float((dw / np.maximum(so[:, None], 1e-30)).max()) if dw.size else 0.0
    same = qg == qo
    dd = np.abs(got.delta[rows].astype(np.float64) - want.delta[rows].astype(np.float64))
    assert np.all(dd[same] <= np.broadcast_to(bound, dd.shape)[same]), f"{what}: delta off by more than 1e-3 s'"
    bad = np.argwhere(~same)
    for i, c in bad:
        assert abs(qg[i, c] - qo[i, c]) == 1, f"{what}: q' differs by {qg[i, c] - qo[i, c]} at row {rows[i]} col {c}"
        x = np.float32(wo[i, c] / np.float32(so[i]))
        tie = (qg[i, c] + qo[i, c]) / 2.0
        slack = 2 * np.spacing(np.abs(x)) + dw[i, c] / so[i] + abs(sg[i] - so[i]) / so[i] * 128
        dist = abs(float(x) - tie)
        assert dist <= slack, f"{what}: q' flip at row {rows[i]} col {c} is {dist:.3g} from the tie (slack {slack:.3g})"
        rep["flip_tie_dist_ulp"].append(dist / float(np.spacing(np.abs(x))))
    rep["flips"] = int(bad.shape[0])
    mg, vg = got.moments()
    mo, vo = want.moments()
    g = np.abs(np.asarray(G, np.float64))
    dg = 1e-3 * np.maximum(g, 1e-3 * (g.max(axis=1, keepdims=True) if g.size else 0.0))
    carried = {"m": (1.0 - beta1) * dg, "v": (1.0 - beta2) * (2.0 * g * dg + dg * dg)}
    for name, a, b, col in (("m", mg, mo, 0), ("v", vg, vo, 1)):
        a, b = a[slots].astype(np.float64), b[slots].astype(np.float64)
        unit = _f16_ulp_scaled(b, want.e[slots, col]) * 1.0000001
        tol = unit + carried[name]
        err = np.abs(a - b)
        assert np.all(err <= tol), f"{what}: {name} off by {float((err / tol).max()):.3g} of its bound"
        rep[f"max_{name}_err_of_bound"] = float((err / tol).max()) if err.size else 0.0
        rep[f"{name}_beyond_one_unit"] = int(np.count_nonzero(err > unit))
    if got.w_live is not None and want.w_live is not None:
        a = bf16_to_f32_host(got.w_live[rows]).astype(np.float64)
        b = bf16_to_f32_host(want.w_live[rows]).astype(np.float64)
        tol = np.spacing(np.abs(b).astype(np.float32)).astype(np.float64) * 2 ** 16 + 2.0 ** -133
        assert np.all(np.abs(a - b) <= tol), f"{what}: live weights off by more than one bf16 unit"
    return rep


def bf16_to_f32_host(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32)
