"""Benchmark of the sparse-first step on one MI355X.

Workload: one Llama-7B-shaped decoder layer (q, k, v, o 4096x4096; gate, up
11008x4096; down 4096x11008), 4096 tokens, bf16 X ~ N(0,1) and dY ~ N(0,0.01),
row-tracker masks from seeded output magnitudes with 1% of each matrix's rows
active (clustered in 32-row tiles), int8 q + fp32 residual resident, fp16
moments for the active rows.  One step = the masked dW of all seven
matrices (one launch; q/k/v and gate/up share their input) and the sparse
update with fused write-back of all seven (one launch), every input (the
packed plan included) resident in HBM when the timed region starts.  The same
steps with the plan's host->device copy in front of each are timed too and
reported beside the value (PCIe-inclusive, never the value).  Method: "Sparse-First Fine-Tuning: Full-Weight
Training at the Cost of the Active Set", sections 2.1-2.3.

Steps cycle through a ring of distinct layers (like the layers of one model
step), so that every step reads its inputs from HBM rather than from the
256 MB last-level cache.

Prints one JSON line (rank 0).  ``--gpus`` above 1 is refused: this build
measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
COUNTERS_SUMMARY = "masked_dw_llama7b_layer_1pct_counters.txt"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--layers", type=int, default=6, help="ring of distinct layers cycled by the steps")
    ap.add_argument("--density", type=float, default=0.01)
    ap.add_argument("--layout", choices=["packed", "tiles"], default="packed",
                    help="masked-dW row layout: active rows packed 32 to a tile, or whole active tiles")
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="step with sft_masked_dw + sft_sparse_update instead of the fused sft_masked_dw_update")
    ap.add_argument("--cpu-sample-every", type=int, default=4,
                    help="oracle timing uses every n-th active row of each matrix")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the timings of the other hot-path calls (embedding, coupled pairs, write-back, "
                         "checkpoint)")
    ap.add_argument("--rows-only", action="store_true",
                    help="time only the other hot-path calls (prints their JSON object), for profiling them apart "
                         "from the layer step")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the probes of the HBM and matrix-core rates this device sustains")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


class Layer:
    """Device buffers, plans and prepared launches of one layer."""

    def __init__(self, idx: int, T: int, density: float, seed0: int, layout: str = "packed"):
        import torch

        from sparse_full_weight_amd import _lib, synth
        self.idx = idx
        self.density = density
        dev = "cuda"
        seed = seed0 + 100 * idx
        shapes = synth.LLAMA7B
        self.mats = {}
        host_chunks = []   # packed plan: int32 words, uploaded once per step
        offsets = {}      # per matrix: word offset and length of each plan part
        off = 0
        for mi, (name, (R, C)) in enumerate(shapes.items()):
            k = round(density * R)
            hot = synth.clustered_rows(R, k, seed + 10 * mi + 1)
            mag = synth.tracker_magnitudes(R, hot, seed + 10 * mi + 2)
            mask = _lib.sft_tracker_window(np.zeros(R, np.float32), mag)
            plan = _lib.sft_plan_rows(mask)
            row_slot = np.full(R, -1, np.int32)
            slot, fresh = _lib.sft_slots_update(row_slot, plan.n_active, plan.active_rows)
            fresh[:] = 0          # steady state: the moments already exist
            parts = {"rows": plan.active_rows, "tiles": plan.active_tiles,
                     "abits": plan.active_bits.view(np.int32), "first": plan.tile_first, "slot": slot,
                     "fresh": np.frombuffer(np.pad(fresh, (0, (-fresh.size) % 4)).tobytes(), np.int32)}
            offsets[name] = {}
            for key, arr in parts.items():
                offsets[name][key] = (off, arr.size)
                host_chunks.append(arr.astype(np.int32, copy=False))
                off += arr.size
            self.mats[name] = {"R": R, "C": C, "plan": plan}
        packed = np.concatenate(host_chunks) if host_chunks else np.zeros(1, np.int32)
        self.plan_host = torch.from_numpy(packed).pin_memory()
        self.plan_dev = torch.empty_like(self.plan_host, device=dev)
        self.plan_dev.copy_(self.plan_host)

        gen = torch.Generator(device=dev)
        gen.manual_seed(seed + 7)
        self.X = {}
        for gname, members in synth.LLAMA7B_GROUPS:
            C = shapes[members[0]][1]
            self.X[gname] = synth.normal_bf16_device((T, C), 1.0, seed + 1000 + len(self.X), dev)
        bc1, bc2 = _lib.sft_bias_table(0.9, 0.999, 20000)
        self.hp = _lib.Adam(1e-4, 0.9, 0.999, 1e-8, torch.from_numpy(bc1).to(dev), torch.from_numpy(bc2).to(dev))
        groups, upd = [], []
        for gi, (gname, members) in enumerate(synth.LLAMA7B_GROUPS):
            dw_mats = []
            for name in members:
                m = self.mats[name]
                R, C, plan = m["R"], m["C"], m["plan"]
                lay = offsets[name]

                def view(key, n=None, dtype=None):
                    o, sz = lay[key]
                    t = self.plan_dev[o:o + sz]
                    if dtype is not None:
                        t = t.view(dtype)[: n]
                    return t
                dplan = _lib.DevicePlan(plan, view("rows"), view("tiles"), view("abits"), view("first"))
                m["dY"] = synth.normal_bf16_device((T, R), 0.01, seed + 2000 + R + len(dw_mats) + 17 * gi, dev)
                n = plan.n_active
                m["dW"] = torch.empty((n, C), dtype=torch.float32, device=dev)
                dw_mats.append(_lib.DwMat(m["dY"], dplan, m["dW"]))
                # resident state
                m["q"] = torch.randint(-127, 128, (R, C), dtype=torch.int8, device=dev, generator=gen)
                m["s"] = torch.empty(R, dtype=torch.float32, device=dev).uniform_(1e-4, 1e-3, generator=gen)
                m["delta"] = (torch.rand((R, C), dtype=torch.float32, device=dev, generator=gen) - 0.5) * m["s"][:, None]
                m["w_live"] = torch.zeros((R, C), dtype=torch.bfloat16, device=dev)
                m["m"] = torch.zeros((n, C), dtype=torch.int16, device=dev)
                m["v"] = torch.zeros((n, C), dtype=torch.int16, device=dev)
                m["t"] = torch.zeros(n, dtype=torch.int32, device=dev)
                upd.append(_lib.UpdMat(m["q"], m["s"], m["delta"], m["m"], m["v"], m["t"], view("rows"),
                                       view("slot"), m["dW"], n, view("fresh", n, torch.uint8), m["w_live"]))
            groups.append(_lib.DwGroup(self.X[gname], dw_mats,
                                       _lib.SFT_DW_PACKED if layout == "packed" else _lib.SFT_DW_TILES))
        self.groups = groups
        self.upd = upd
        nbytes = _lib.sft_masked_dw_workspace(groups)
        self.ws = torch.zeros(max(nbytes // 4, 1), dtype=torch.int32, device=dev)
        self.dw_call = _lib.prepare_masked_dw(groups, self.ws)
        self.upd_call = _lib.prepare_sparse_update(upd, self.hp)
        # the update matrices follow the groups' matrices in order
        self.fused_call = _lib.prepare_masked_dw_update(groups, self.ws, upd, self.hp)
        self.T = T

    def upload_plan(self):
        self.plan_dev.copy_(self.plan_host, non_blocking=True)

    def dw_work(self):
        from sparse_full_weight_amd import accounting, synth
        groups = []
        for gname, members in synth.LLAMA7B_GROUPS:
            C = self.mats[members[0]]["C"]
            groups.append((self.T, C, [(self.mats[n]["plan"].n_active, self.mats[n]["plan"].n_active_tiles)
                                       for n in members]))
        return accounting.masked_dw_work(groups)

    def upd_work(self):
        from sparse_full_weight_amd import accounting
        return accounting.update_work([(m["C"], m["plan"].n_active) for m in self.mats.values()])


def cpu_baseline(layer: "Layer", every: int):
    """Time the oracle (plain C, one thread) on every n-th active row of each
    matrix of one layer: its masked dW rows and their update; scale to the
    whole layer."""
    import oracle
    import torch

    from sparse_full_weight_amd import synth
    t_total = 0.0
    rows_done = rows_all = 0
    for gname, members in synth.LLAMA7B_GROUPS:
        Xb = layer.X[gname].view(torch.int16).cpu().numpy().view(np.uint16)
        for name in members:
            m = layer.mats[name]
            plan = m["plan"]
            rows = plan.active_rows[::every].copy()
            dY = m["dY"].view(torch.int16).cpu().numpy().view(np.uint16)
            R, C = m["R"], m["C"]
            sub = np.searchsorted(plan.active_rows, rows)
            q = m["q"].cpu().numpy()
            s = m["s"].cpu().numpy()
            delta = m["delta"].cpu().numpy()
            st = oracle.MatState(q, s, delta, np.zeros((rows.size, C), np.uint16), np.zeros((rows.size, C), np.uint16),
                                 np.zeros(rows.size, np.int32), np.zeros((R, C), np.uint16))
            t0 = time.perf_counter()
            G = oracle.masked_dw(dY, Xb, rows)
            oracle.sparse_update(st, G, rows, np.arange(rows.size, dtype=np.int32), None, lr=1e-4, beta1=0.9,
                                 beta2=0.999, eps=1e-8)
            t_total += time.perf_counter() - t0
            rows_done += rows.size
            rows_all += plan.n_active
            del sub
    scale = rows_all / max(rows_done, 1)
    return t_total * scale * 1e3, rows_done, rows_all, t_total


LEAF_DENSITY = 0.001


def leaf_support(m: int, n: int, seed: int):
    """SparseLeaf support: round(0.1% of m*n) distinct coordinates, uniform,
    sorted by (row, column)."""
    from sparse_full_weight_amd import synth
    g = synth.rng(seed)
    flat = np.sort(g.choice(m * n, size=round(LEAF_DENSITY * m * n), replace=False))
    return (flat // n).astype(np.int32), (flat % n).astype(np.int32)


def _time_calls(fns, K, stream):
    """Average ms of one pass over fns (each enqueued on stream), over K back-to-back passes after 5 warm-ups."""
    import torch
    for _ in range(5):
        for f in fns:
            f(stream)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        for f in fns:
            f(stream)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / K


def _hbm(work_bytes, ms):
    gbs = work_bytes / (ms * 1e-3) / 1e9
    return {"avg_ms": round(ms, 5), "algorithmic_bytes": work_bytes, "GB_s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def other_rows(L0: "Layer", K: int, stream):
    """Timings of the hot-path calls the layer step does not run: the embedding
    scatter-gradient and its update, the coupled pair update (with the packed
    masked dW feeding it) on one-active-row-per-tile masks, the standalone
    masked write-back, the active-row checkpoint save and restore, the
    SparseLeaf connection gradients and Adam step, and the layer step at the
    full step's other row densities (0.5%, 2%, 5%).  Same event bracketing as the step: K back-to-back
    passes over prepared calls."""
    import torch

    from sparse_full_weight_amd import _lib, accounting, synth
    dev = "cuda"
    out = {}

    def state(R, C, n, seed):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        st = {"q": torch.randint(-127, 128, (R, C), dtype=torch.int8, device=dev, generator=gen),
              "s": torch.empty(R, dtype=torch.float32, device=dev).uniform_(1e-4, 1e-3, generator=gen)}
        st["delta"] = (torch.rand((R, C), dtype=torch.float32, device=dev, generator=gen) - 0.5) * st["s"][:, None]
        st["w"] = torch.zeros((R, C), dtype=torch.bfloat16, device=dev)
        st["m"] = torch.zeros((n, C), dtype=torch.int16, device=dev)
        st["v"] = torch.zeros((n, C), dtype=torch.int16, device=dev)
        st["t"] = torch.zeros(n, dtype=torch.int32, device=dev)
        st["slot"] = torch.arange(n, dtype=torch.int32, device=dev)
        return st

    def upd(st, rows_dev, G, n):
        return _lib.UpdMat(st["q"], st["s"], st["delta"], st["m"], st["v"], st["t"], rows_dev, st["slot"], G, n,
                           None, st["w"])

    hp = L0.hp

    # ---- embedding: a 32000 x 4096 table, 4 windows of 8 x 512 Zipf(1.1) ids
    V, d, Tb = 32000, 4096, 8 * 512
    windows = [synth.zipf_tokens(Tb, V, 1.1, 9000 + w) for w in range(4)]
    ch = np.zeros(V, np.float32)
    t0 = time.perf_counter()
    for tokens in windows:
        mask = _lib.sft_conductor_window(ch, tokens)
    plan = _lib.sft_plan_rows(mask)
    row_ptr, pos = _lib.sft_plan_embedding(plan, tokens)
    host_us = (time.perf_counter() - t0) * 1e6
    n = plan.n_active
    dY = synth.normal_bf16_device((Tb, d), 0.01, 9010, dev)
    G = torch.empty((max(n, 1), d), dtype=torch.float32, device=dev)
    st = state(V, d, n, 9020)
    dplan = plan.to_device()
    rp, ps = torch.from_numpy(row_ptr).to(dev), torch.from_numpy(pos).to(dev)
    emb = _lib.prepare_embedding_dw(dY, rp, ps, n, G)
    eup = _lib.prepare_sparse_update([upd(st, dplan.active_rows, G, n)], hp)
    w_emb = accounting.embedding_dw_work(d, int(pos.size), n).bytes
    w_eup = accounting.update_work([(d, n)]).bytes
    out["a3_embedding_dw"] = dict(_hbm(w_emb, _time_calls([emb], K, stream)), active_rows=n, hit_tokens=int(pos.size),
                                  table=[V, d], tokens=Tb)
    out["a3_embedding_dw_and_update"] = dict(_hbm(w_emb + w_eup, _time_calls([emb, eup], K, stream)),
                                             host_conductor_plan_us=round(host_us, 1))
    del st, dY, G

    # ---- coupled pairs on one active row per 32-row tile (every tile active)
    pairs = [("gate", "up"), ("q", "o"), ("k", "v")]
    rows = {name: synth.one_per_tile_rows(L0.mats[name]["R"], 9100 + mi) for mi, name in enumerate(L0.mats)}
    for a, b in pairs:
        rows[b][::2] = rows[a][::2]   # a pair shares the row of every other tile
    groups, plans, G = [], {}, {}
    for gname, members in synth.LLAMA7B_GROUPS:
        ms = []
        for name in members:
            m = L0.mats[name]
            plan = _lib.sft_plan_rows(synth.mask_from_rows(m["R"], rows[name]))
            plans[name] = plan.to_device()
            G[name] = torch.empty((plan.n_active, m["C"]), dtype=torch.float32, device=dev)
            ms.append(_lib.DwMat(m["dY"], plans[name], G[name]))
        groups.append(_lib.DwGroup(L0.X[gname], ms, _lib.SFT_DW_PACKED))
    ws = torch.zeros(max(_lib.sft_masked_dw_workspace(groups) // 4, 1), dtype=torch.int32, device=dev)
    dw = _lib.prepare_masked_dw(groups, ws)
    sts = {name: state(L0.mats[name]["R"], L0.mats[name]["C"], plans[name].n_active, 9200 + i)
           for i, name in enumerate(L0.mats)}
    cp = _lib.prepare_coupled_update([_lib.Pair(upd(sts[a], plans[a].active_rows, G[a], plans[a].n_active),
                                                upd(sts[b], plans[b].active_rows, G[b], plans[b].n_active), 1.0, 0.4)
                                      for a, b in pairs], hp)
    dn = _lib.prepare_sparse_update([upd(sts["down"], plans["down"].active_rows, G["down"], plans["down"].n_active)],
                                    hp)
    dw_groups = [(L0.T, L0.mats[mm[0]]["C"], [(plans[n].n_active, plans[n].n_active_tiles) for n in mm])
                 for _, mm in synth.LLAMA7B_GROUPS]
    w_dw = accounting.masked_dw_work(dw_groups)
    sides = []
    for a, b in pairs:
        shared = int(np.intersect1d(rows[a], rows[b]).size)
        sides += [(L0.mats[a]["C"], rows[a].size, shared), (L0.mats[b]["C"], rows[b].size, shared)]
    w_cp = accounting.coupled_update_work(sides).bytes
    t_dw = _time_calls([dw], K, stream)
    out["f1_packed_dw_one_row_per_tile"] = dict(
        _hbm(w_dw.bytes, t_dw), active_rows=int(sum(p.n_active for p in plans.values())),
        useful_TFLOP_s=round(w_dw.flops_useful / (t_dw * 1e-3) / 1e12, 1),
        whole_tile_TFLOP=round(w_dw.flops_issued / 1e12, 3))
    out["a5_coupled_update"] = dict(_hbm(w_cp, _time_calls([cp], K, stream)), pairs=[list(p) for p in pairs],
                                    a_own=1.0, a_cross=0.4)
    out["a5_coupled_and_down_update"] = _hbm(
        w_cp + accounting.update_work([(L0.mats["down"]["C"], plans["down"].n_active)]).bytes,
        _time_calls([cp, dn], K, stream))
    del sts, G, ws

    # ---- standalone write-back of the 1% layer's active rows (7 matrices):
    # one batched call, and the seven single-matrix calls beside it
    wb, wb_mats, w_wb = [], [], 0.0
    for name, m in L0.mats.items():
        plan = m["plan"]
        rows_dev = torch.from_numpy(plan.active_rows).to(dev)
        wb.append(_lib.prepare_masked_writeback(m["q"], m["s"], m["delta"], rows_dev, plan.n_active, m["w_live"]))
        wb_mats.append((m["q"], m["s"], m["delta"], rows_dev, plan.n_active, m["w_live"]))
        w_wb += accounting.writeback_work(m["C"], plan.n_active).bytes
    out["a6_masked_writeback"] = dict(_hbm(w_wb, _time_calls([_lib.prepare_masked_writeback_many(wb_mats)], K,
                                                             stream)), calls=1)
    out["a6_masked_writeback_single_calls"] = dict(_hbm(w_wb, _time_calls(wb, K, stream)), calls=len(wb))

    # ---- active-row checkpoint of the 1% layer (7 matrices, one call each way)
    cks = [_lib.CkptMat.alloc(u.q, u.s, u.delta, u.m, u.v, u.t, u.active_rows, u.slot, u.n_active, u.w_live)
           for u in L0.upd]
    dims = [(u.q.shape[1], u.n_active) for u in L0.upd]
    save = _lib.prepare_rows_save(cks)
    restore = _lib.prepare_rows_restore(cks)
    out["f2_rows_save"] = dict(_hbm(accounting.checkpoint_work(dims).bytes, _time_calls([save], K, stream)),
                               rows=int(sum(n for _, n in dims)))
    out["f2_rows_restore"] = _hbm(accounting.checkpoint_work(dims, restore=True).bytes,
                                  _time_calls([restore], K, stream))

    # ---- SparseLeaf connections: 0.1% of each matrix's entries, uniform random
    # coordinates (sorted), on the layer's own dY and X
    leaf, lvecs, dims = [], [], []
    for mi, (name, m) in enumerate(L0.mats.items()):
        rows, cols = leaf_support(m["R"], m["C"], 9300 + mi)
        g = torch.empty(rows.size, dtype=torch.float32, device=dev)
        X = L0.X[[gn for gn, mm in synth.LLAMA7B_GROUPS if name in mm][0]]
        leaf.append(_lib.LeafMat(m["dY"], X, torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev), g))
        z = [torch.zeros(rows.size, dtype=torch.float32, device=dev) for _ in range(3)]
        lvecs.append(_lib.LeafVec(g, z[0], z[1], z[2], torch.zeros(rows.size, dtype=torch.int16, device=dev)))
        dims.append((int(np.unique(rows).size), int(np.unique(cols).size), int(rows.size)))
    lws = torch.zeros(max(_lib.sft_leaf_grad_workspace(leaf) // 4, 1), dtype=torch.int32, device=dev)
    lgrad = _lib.prepare_leaf_grad(leaf, lws)
    ladam = _lib.prepare_leaf_adam(lvecs, 1, hp)
    wl = accounting.leaf_grad_work(L0.T, dims)
    t_l = _time_calls([lgrad], K, stream)
    out["f4_leaf_grad"] = dict(_hbm(wl.bytes, t_l), coordinates=int(sum(d[2] for d in dims)), density=LEAF_DENSITY,
                               useful_TFLOP_s=round(wl.flops_useful / (t_l * 1e-3) / 1e12, 2))
    out["f4_leaf_adam"] = _hbm(accounting.leaf_adam_work(sum(d[2] for d in dims)).bytes,
                               _time_calls([ladam], K, stream))
    del leaf, lvecs, lws

    # ---- the full step's other row densities: the same layer step (fused
    # masked dW and update, plan resident) over a ring of 3 layers at each density
    sweep = {}
    for density in (0.005, 0.02, 0.05):
        ring = [Layer(100 + i, L0.T, density, 6000, "packed") for i in range(3)]

        def step(L):
            L.fused_call(stream)
        for i in range(5):
            step(ring[i % 3])
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(K):
            step(ring[i % 3])
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / K
        work = ring[0].dw_work().bytes + ring[0].upd_work().bytes
        sweep[f"{density:g}"] = dict(_hbm(work, ms), active_rows=int(sum(m["plan"].n_active
                                                                        for m in ring[0].mats.values())))
        del ring
        torch.cuda.empty_cache()
    out["c_density_sweep_step"] = sweep

    # ---- one GPU's share of a token-sharded step: the same 1% layer step (fused
    # call, plans resident) on T/N tokens, the shape each of N GPUs would run
    # before the dW exchange (which is not built here)
    share = {}
    for n_gpu in (2, 4, 8):
        T = L0.T // n_gpu
        ring = [Layer(200 + i, T, L0.density, 7000, "packed") for i in range(3)]

        def ring_ms(fn):
            for i in range(5):
                fn(ring[i % 3])
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(K):
                fn(ring[i % 3])
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / K
        dw_b, up_b = ring[0].dw_work().bytes, ring[0].upd_work().bytes
        share[f"T{T}"] = dict(_hbm(dw_b + up_b, ring_ms(lambda L: L.fused_call(stream))), n_gpus_sharing=n_gpu,
                              tokens=T, masked_dw=_hbm(dw_b, ring_ms(lambda L: L.dw_call(stream))))
        del ring
        torch.cuda.empty_cache()
    out["e_token_share_step"] = share
    torch.cuda.synchronize()
    return out


def ceilings(stream):
    """What this device sustains beside the published peaks: an HBM read stream
    and copy over 2 GiB buffers (16-byte non-temporal accesses, 8 workgroups per
    CU) and back-to-back bf16 MFMA on register operands."""
    import torch

    from sparse_full_weight_amd import _lib
    n = 1 << 31
    a = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    sink = torch.empty(_lib.sft_probe_grid() * 256, dtype=torch.int32, device="cuda")
    t_read = _time_calls([_lib.prepare_probe_read(a, sink)], 20, stream)
    t_copy = _time_calls([_lib.prepare_probe_copy(a, b)], 20, stream)
    del a, b
    iters = 4096
    out = torch.empty(_lib.sft_probe_grid() * 256, dtype=torch.float32, device="cuda")
    t_mfma = _time_calls([_lib.prepare_probe_mfma(iters, out)], 10, stream)
    flops = _lib.sft_probe_grid() * 4 * 4 * iters * 32768
    return {"hbm_read_GB_s": round(n / (t_read * 1e-3) / 1e9, 1),
            "hbm_copy_GB_s": round(2 * n / (t_copy * 1e-3) / 1e9, 1),
            "mfma_bf16_TFLOP_s": round(flops / (t_mfma * 1e-3) / 1e12, 1),
            "peaks": {"hbm_GB_s": HBM_PEAK_GBS, "mfma_bf16_TFLOP_s": MFMA_BF16_PEAK_TFLOPS},
            "note": "read and copy over 2 GiB buffers (copy counts read + write bytes); MFMA 32x32x16 bf16 "
                    "back to back, 8 workgroups per CU"}


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": {"read": n, "write": n}, "launches": 3}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(the path would shard over token positions; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    torch.cuda.set_device(0)
    print(f"[bench] building {args.layers} layers (T={args.tokens}, density={args.density})", file=sys.stderr,
          flush=True)
    t0 = time.perf_counter()
    layers = [Layer(i, args.tokens, args.density, 5000, args.layout) for i in range(args.layers)]
    torch.cuda.synchronize()
    print(f"[bench] setup {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)

    # host plan cost of one layer (tracker windows + plans + slots), for the record
    from sparse_full_weight_amd import _lib, synth
    th0 = time.perf_counter()
    for mi, (name, (R, C)) in enumerate(synth.LLAMA7B.items()):
        mag = synth.tracker_magnitudes(R, synth.clustered_rows(R, round(args.density * R), 7 + mi), 8 + mi)
        mask = _lib.sft_tracker_window(np.zeros(R, np.float32), mag)
        plan = _lib.sft_plan_rows(mask)
        _lib.sft_slots_update(np.full(R, -1, np.int32), plan.n_active, plan.active_rows)
    host_plan_us = (time.perf_counter() - th0) * 1e6

    stream = torch.cuda.current_stream()
    if args.rows_only:
        print(json.dumps({"rows": other_rows(layers[0], min(args.steps, 100), stream)}), flush=True)
        return

    def step(L):
        if args.unfused:
            L.dw_call(stream)
            L.upd_call(stream)
        else:
            L.fused_call(stream)

    def step_with_upload(L):
        L.upload_plan()
        step(L)

    # Untimed: about 0.1 s of steps so that the clocks have settled, then the
    # W warmup steps.
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.1:
        for i in range(len(layers)):
            step(layers[i])
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()

    K = args.steps
    # The timed loop: K whole steps back to back, bracketed by one event pair
    # (per-step events would put markers between the kernels); every plan is
    # resident (uploaded when its layer was built).
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    def timed_steps(fn):
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(K):
            fn(layers[i % len(layers)])
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    ms_per_step = timed_steps(step)
    # the same steps, each behind its plan's host->device copy (PCIe-inclusive)
    ms_with_upload = timed_steps(step_with_upload)

    # Per-call durations, each timed over its own back-to-back run of K calls
    # on the same stream and inputs (the masked-dW call is the gather, product
    # and fix-up kernels; the update call is one kernel).
    def timed(fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(K):
            fn(layers[i % len(layers)])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K

    for L in layers:
        L.upload_plan()
    dw_avg = timed(lambda L: L.dw_call(stream))
    up_avg = timed(lambda L: L.upd_call(stream))
    fu_avg = timed(lambda L: L.fused_call(stream))

    L0 = layers[0]
    dw = L0.dw_work()
    up = L0.upd_work()
    dw_gbs = dw.bytes / (dw_avg * 1e-3) / 1e9
    up_gbs = up.bytes / (up_avg * 1e-3) / 1e9
    fu_gbs = (dw.bytes + up.bytes) / (fu_avg * 1e-3) / 1e9
    n_act = sum(m["plan"].n_active for m in L0.mats.values())
    n_tiles = sum(m["plan"].n_active_tiles for m in L0.mats.values())

    # HBM bytes per masked-dW call from the committed counter summary, if it
    # was taken on the current kernel source (else null).
    from sparse_full_weight_amd import profsum
    rec = profsum.read_traffic(os.path.join(ROOT, "profiles", COUNTERS_SUMMARY))
    traffic = None
    if rec and rec.get("sft_dw_sha256") == profsum.source_hash("sft_dw.hip"):
        traffic = rec["masked_dw_call_bytes"]

    rows = None
    if not args.no_rows:
        print("[bench] timing the other hot-path calls", file=sys.stderr, flush=True)
        rows = other_rows(L0, min(K, 100), stream)

    ceil = None
    if not args.no_ceilings:
        print("[bench] probing the sustained HBM and matrix-core rates", file=sys.stderr, flush=True)
        ceil = ceilings(stream)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a sample", file=sys.stderr, flush=True)
        cpu_ms, rows_done, rows_all, t_sample = cpu_baseline(L0, args.cpu_sample_every)
        cpu = {"value": round(cpu_ms, 1), "unit": "ms", "cores": 1, "kind": "oracle",
               "sample": f"every {args.cpu_sample_every}th active row of each of the 7 matrices of one layer "
                         f"({rows_done} of {rows_all} rows: masked dW rows + their update, "
                         f"{t_sample:.1f} s), scaled to the whole layer"}

    out = {
        "metric": "masked step ms per 7B-shape layer at 1% active rows; MFMA util + HBM GB/s",
        "value": round(ms_per_step, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama7b_layer_masked_step", "tokens": args.tokens, "density": args.density,
                   "matrices": {k: list(v) for k, v in synth.LLAMA7B.items()}, "active_rows": n_act,
                   "active_tiles": n_tiles, "ring_layers": args.layers, "dw_layout": args.layout,
                   "step": ("masked dW (7 matrices) + sparse update with fused write-back (7 matrices), "
                            + ("two calls" if args.unfused else
                               "one call: sft_masked_dw_update, the split tiles' fix-up done by the update")
                            + "; inputs and plans resident in HBM"),
                   "ms_per_step_with_plan_upload": round(ms_with_upload, 5)},
        "roofline": {"bound": "hbm", "kernel": "sft_masked_dw (k_dw_gather + k_masked_dw + k_dw_fixup)",
                     "achieved": round(dw_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dw_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": dw.bytes, "avg_ms": round(dw_avg, 5)},
        "cpu_baseline": cpu,
        "kernels": {
            "sft_masked_dw": {"avg_ms": round(dw_avg, 5), "GB_s": round(dw_gbs, 1),
                            "hbm_frac": round(dw_gbs / HBM_PEAK_GBS, 4),
                            "useful_TFLOP_s": round(dw.flops_useful / (dw_avg * 1e-3) / 1e12, 1),
                            "issued_TFLOP_s": round(dw.flops_issued / (dw_avg * 1e-3) / 1e12, 1),
                            "mfma_frac_issued": round(dw.flops_issued / (dw_avg * 1e-3) / 1e12 /
                                                      MFMA_BF16_PEAK_TFLOPS, 4)},
            "sft_sparse_update": {"avg_ms": round(up_avg, 5), "GB_s": round(up_gbs, 1),
                                "hbm_frac": round(up_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": up.bytes},
            "sft_masked_dw_update": {"avg_ms": round(fu_avg, 5), "GB_s": round(fu_gbs, 1),
                                     "hbm_frac": round(fu_gbs / HBM_PEAK_GBS, 4),
                                     "algorithmic_bytes": dw.bytes + up.bytes},
        },
        "rows": rows,
        "ceilings": ceil,
        "host_plan_us_per_layer": round(host_plan_us, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
