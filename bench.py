"""Benchmark of the sparse-first step on one MI355X.

Headline workload: one Llama-7B-shaped decoder layer (q, k, v, o 4096x4096;
gate, up 11008x4096; down 4096x11008), 4096 tokens, bf16 X ~ N(0,1) and
dY ~ N(0,0.01), row-tracker masks from seeded output magnitudes with 1% of
each matrix's rows active (clustered in 32-row tiles), int8 q + fp32 residual
resident, scaled fp16 moments for the active rows.  One step = the copy of
the step's packed plan (active rows, tiles, slots; a few KB made on the host,
section 2.6 and Figure 2 of the page) to the device, then the masked dW of
all seven matrices and the sparse update with fused write-back of all seven
(one call, sft_masked_dw_update).  Every other input (activations, output
gradients, optimizer state) is resident in HBM when the timed region starts.
The same steps with the plan already resident are reported beside the value.
Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
Active Set", sections 2.1-2.6.

Steps cycle through a ring of 12 distinct layers (like the layers of one
model step), so that every step reads its inputs and its active rows' state
from HBM rather than from the 256 MB last-level cache (a ring of 6 left the
state of the active rows there: 4% faster steps).  The layers' steps are independent of each other,
so consecutive layers alternate between three streams, the lanes (all of the
default priority; layer i always on lane i mod 3): one layer's launches fill
the CUs the others leave idle while they start, drain and run their updates.
The same steps on one stream are reported beside the value
(``ms_per_step_one_stream``).

Besides the headline, the JSON line carries (``rows``) the other workloads
timed as steps: the 512x512 projection (10% rows), the whole 7B-shaped model
(32 distinct layers plus the 32000x4096 embedding) at 0.5%, 1%, 2% and 5%
rows, the adversarial one-row-per-tile layer with the coupled update, and the
separate calls of the path; the oracle timed on the host on one thread and on
several; the a1 host calls timed alone.

Prints one JSON line (rank 0).  ``--gpus`` above 1 is refused: the benchmark
measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
COUNTERS_SUMMARY = "masked_dw_llama7b_layer_1pct_counters.txt"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)
CPU_THREADS = 16               # the host share of one GPU on the box


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--block", type=int, default=12,
                    help="steps between the timing events whose block means give the median and percentiles")
    ap.add_argument("--layers", type=int, default=12, help="ring of distinct layers cycled by the steps")
    ap.add_argument("--density", type=float, default=0.01)
    ap.add_argument("--layout", choices=["packed", "tiles"], default="packed",
                    help="masked-dW row layout: active rows packed 32 to a tile, or whole active tiles")
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="step with sft_masked_dw + sft_sparse_update instead of the fused sft_masked_dw_update")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other workloads and calls (model step, adversarial step, embedding, ...)")
    ap.add_argument("--rows-only", action="store_true",
                    help="time only the other calls (prints their JSON object), for profiling them apart "
                         "from the layer step")
    ap.add_argument("--no-model", action="store_true", help="skip the 32-layer model step")
    ap.add_argument("--lanes", type=int, default=3,
                    help="streams the layers' steps alternate over (layer i on lane i mod lanes); 1: one stream")
    ap.add_argument("--one-stream", action="store_true", help="the same as --lanes 1")
    ap.add_argument("--steps-only", action="store_true",
                    help="only the warm-up and the K timed steps (prints their ms per step), for kernel traces of "
                         "the step schedule")
    ap.add_argument("--model-steps", type=int, default=10)
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the probes of the HBM and matrix-core rates this device sustains")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--skip-probe", action="store_true",
                    help="run only masked dW calls with 0..16 active tiles of 128 (the skipped-tile traffic "
                         "evidence, under the HBM counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------- workloads
def layer_buffers(T, seed, dev="cuda", shapes=None, groups=None):
    """Activations, output gradients and resident state of one layer, drawn
    on the device (torch's seeded generator)."""
    import torch

    from sparse_full_weight_amd import synth
    shapes = shapes or synth.LLAMA7B
    groups = groups or synth.LLAMA7B_GROUPS
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 7)
    X = {}
    for gi, (gname, members) in enumerate(groups):
        X[gname] = synth.normal_bf16_device((T, shapes[members[0]][1]), 1.0, seed + 1000 + gi, dev)
    mats = {}
    for mi, (name, (R, C)) in enumerate(shapes.items()):
        m = {"R": R, "C": C, "dY": synth.normal_bf16_device((T, R), 0.01, seed + 2000 + mi, dev),
             "q": torch.randint(-127, 128, (R, C), dtype=torch.int8, device=dev, generator=gen),
             "s": torch.empty(R, dtype=torch.float32, device=dev).uniform_(1e-4, 1e-3, generator=gen),
             "w_live": torch.zeros((R, C), dtype=torch.bfloat16, device=dev)}
        m["delta"] = (torch.rand((R, C), dtype=torch.float32, device=dev, generator=gen) - 0.5) * m["s"][:, None]
        mats[name] = m
    return X, mats


class Layer:
    """Plans, moments and prepared launches of one layer over its buffers."""

    def __init__(self, idx: int, T: int, density: float, seed0: int, layout: str = "packed", buffers=None,
                 rows=None, shapes=None, groups=None):
        import torch

        from sparse_full_weight_amd import _lib, synth
        self.idx = idx
        self.density = density
        self.T = T
        dev = "cuda"
        seed = seed0 + 100 * idx
        self.shapes = shapes or synth.LLAMA7B
        self.groups_def = groups or synth.LLAMA7B_GROUPS
        X, bufs = buffers if buffers is not None else layer_buffers(T, seed, dev, self.shapes, self.groups_def)
        self.X = X
        self.mats = {}
        # the step's plan: one sft_plan_layer call over the seven matrices'
        # tracker windows, written into pinned host memory for one upload
        names = list(self.shapes)
        Rs = [self.shapes[n][0] for n in names]
        self.mags = []
        for mi, name in enumerate(names):
            R = Rs[mi]
            if rows is not None:
                self.mags.append(synth.mask_from_rows(R, rows[name]).astype(np.float32))
            else:
                hot = synth.clustered_rows(R, round(density * R), seed + 10 * mi + 1)
                self.mags.append(synth.tracker_magnitudes(R, hot, seed + 10 * mi + 2))
        words = _lib.LayerPlanner(Rs, Rs).words
        self.plan_host = torch.zeros(max(words, 1), dtype=torch.int32).pin_memory()
        self.planner = _lib.LayerPlanner(Rs, Rs, self.plan_host.data_ptr(), words)
        mplans = self.planner.plan(self.mags)
        host = self.plan_host.numpy()
        offsets = {}
        for mi, name in enumerate(names):
            mp = mplans[mi]
            o = mp.off
            sec = lambda k, n: host[o[k]:o[k] + n].copy()   # noqa: E731
            plan = _lib.Plan(Rs[mi], np.zeros(0, np.uint32), sec("rows", mp.n_active), sec("tiles", mp.n_active_tiles),
                             sec("bits", mp.n_active_tiles).view(np.uint32), sec("first", mp.n_active_tiles))
            # steady state: the moments already exist (no fresh rows)
            host[o["fresh"]:o["fresh"] + (mp.n_active + 3) // 4] = 0
            offsets[name] = {"rows": (o["rows"], mp.n_active), "tiles": (o["tiles"], mp.n_active_tiles),
                             "abits": (o["bits"], mp.n_active_tiles), "first": (o["first"], mp.n_active_tiles),
                             "slot": (o["slot"], mp.n_active), "fresh": (o["fresh"], (mp.n_active + 3) // 4)}
            self.mats[name] = dict(bufs[name], plan=plan)
        self.plan_len = self.planner.length
        self.plan_dev = torch.empty_like(self.plan_host, device=dev)
        self.plan_dev.copy_(self.plan_host)
        bc1, bc2 = _lib.sft_bias_table(0.9, 0.999, 20000)
        self.hp = _lib.Adam(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], torch.from_numpy(bc1).to(dev),
                            torch.from_numpy(bc2).to(dev))
        groups, upd = [], []
        self.views = {}
        for gname, members in self.groups_def:
            dw_mats = []
            for name in members:
                m = self.mats[name]
                C, plan = m["C"], m["plan"]
                lay = offsets[name]

                def view(key, n=None, dtype=None, lay=lay):
                    o, sz = lay[key]
                    t = self.plan_dev[o:o + sz]
                    if dtype is not None:
                        t = t.view(dtype)[: n]
                    return t
                n = plan.n_active
                self.views[name] = {"rows": view("rows"), "slot": view("slot")}
                dplan = _lib.DevicePlan(plan, view("rows"), view("tiles"), view("abits"), view("first"))
                m["dW"] = torch.empty((max(n, 1), C), dtype=torch.float32, device=dev)
                dw_mats.append(_lib.DwMat(m["dY"], dplan, m["dW"][:n]))
                m["m"] = torch.zeros((n, C), dtype=torch.int16, device=dev)
                m["v"] = torch.zeros((n, C), dtype=torch.int16, device=dev)
                m["t"] = torch.zeros(n, dtype=torch.int32, device=dev)
                m["e"] = torch.zeros((n, 2), dtype=torch.int8, device=dev)
                upd.append(_lib.UpdMat(m["q"], m["s"], m["delta"], m["m"], m["v"], m["t"], m["e"], view("rows"),
                                       view("slot"), m["dW"][:n], n, view("fresh", n, torch.uint8), m["w_live"]))
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

    def upload_plan(self, stream=None):
        # one kernel on the stream reads the pinned plan over the bus
        # (sft_plan_upload)
        from sparse_full_weight_amd import _lib
        _lib.sft_plan_upload(self.plan_dev, self.plan_host, 4 * self.plan_len, stream)

    def n_active(self):
        return int(sum(m["plan"].n_active for m in self.mats.values()))

    def dw_work(self):
        from sparse_full_weight_amd import accounting
        groups = []
        for gname, members in self.groups_def:
            C = self.mats[members[0]]["C"]
            groups.append((self.T, C, [(self.mats[n]["plan"].n_active, self.mats[n]["plan"].n_active_tiles)
                                       for n in members]))
        return accounting.masked_dw_work(groups)

    def upd_work(self):
        from sparse_full_weight_amd import accounting
        return accounting.update_work([(m["C"], m["plan"].n_active) for m in self.mats.values()])


class Embedding:
    """The 32000 x 4096 embedding: the conductor over four windows of 8 x 512
    Zipf(1.1) token ids sets the mask; one step uploads the step's plan (active
    rows, slots, the CSR of token positions), takes the masked scatter-gradient
    and the sparse update with fused write-back."""

    def __init__(self, seed, hp, dev="cuda"):
        import torch

        from sparse_full_weight_amd import _lib, synth
        V, d, Tb = 32000, 4096, 8 * 512
        self.V, self.d, self.Tb = V, d, Tb
        windows = [synth.zipf_tokens(Tb, V, 1.1, seed + w) for w in range(4)]
        ch = np.zeros(V, np.float32)
        row_slot = np.full(V, -1, np.int32)
        for w in range(3):
            mask = _lib.sft_conductor_window(ch, windows[w])
            _lib.sft_slots_update(row_slot, V, _lib.sft_plan_rows(mask).active_rows)
        tokens = windows[3]
        # the host work of one step, timed alone (median of 30): the
        # conductor's window, the row plan, the CSR of token positions and the
        # moment slots, from the state the first three windows left
        ch0, rs0, times = ch.copy(), row_slot.copy(), []
        for _ in range(30):
            ch[:] = ch0
            row_slot[:] = rs0
            t0 = time.perf_counter()
            mask = _lib.sft_conductor_window(ch, tokens)
            plan = _lib.sft_plan_rows(mask)
            row_ptr, pos = _lib.sft_plan_embedding(plan, tokens)
            _lib.sft_slots_update(row_slot, V, plan.active_rows)
            times.append((time.perf_counter() - t0) * 1e6)
        self.host_us = float(np.median(times))
        n = plan.n_active
        self.n, self.nnz = n, int(pos.size)
        slot = np.arange(n, dtype=np.int32)
        packed = np.concatenate([plan.active_rows, slot, row_ptr, pos]).astype(np.int32)
        self.plan_host = torch.from_numpy(packed).pin_memory()
        self.plan_dev = self.plan_host.to(dev)
        o1, o2, o3 = n, 2 * n, 2 * n + n + 1
        rows_d, slot_d = self.plan_dev[:o1], self.plan_dev[o1:o2]
        rp_d, pos_d = self.plan_dev[o2:o3], self.plan_dev[o3:]
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed + 20)
        self.dY = synth.normal_bf16_device((Tb, d), 0.01, seed + 10, dev)
        self.G = torch.empty((max(n, 1), d), dtype=torch.float32, device=dev)
        st = {"q": torch.randint(-127, 128, (V, d), dtype=torch.int8, device=dev, generator=gen),
              "s": torch.empty(V, dtype=torch.float32, device=dev).uniform_(1e-4, 1e-3, generator=gen),
              "w": torch.zeros((V, d), dtype=torch.bfloat16, device=dev),
              "m": torch.zeros((n, d), dtype=torch.int16, device=dev),
              "v": torch.zeros((n, d), dtype=torch.int16, device=dev),
              "t": torch.zeros(n, dtype=torch.int32, device=dev),
              "e": torch.zeros((n, 2), dtype=torch.int8, device=dev)}
        st["delta"] = (torch.rand((V, d), dtype=torch.float32, device=dev, generator=gen) - 0.5) * st["s"][:, None]
        self.st = st
        self.emb_call = _lib.prepare_embedding_dw(self.dY, rp_d, pos_d, n, self.G[:n])
        self.upd_call = _lib.prepare_sparse_update(
            [_lib.UpdMat(st["q"], st["s"], st["delta"], st["m"], st["v"], st["t"], st["e"], rows_d, slot_d,
                         self.G[:n], n, None, st["w"])], hp)

    def upload_plan(self, stream=None):
        from sparse_full_weight_amd import _lib
        _lib.sft_plan_upload(self.plan_dev, self.plan_host, None, stream)

    def step(self, stream):
        self.upload_plan(stream)
        self.emb_call(stream)
        self.upd_call(stream)

    def work(self):
        from sparse_full_weight_amd import accounting
        return (accounting.embedding_dw_work(self.d, self.nnz, self.n).bytes
                + accounting.update_work([(self.d, self.n)]).bytes)


# ---------------------------------------------------------------------- timing
def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def timed_blocks(fn, K: int, block: int, stream):
    """K calls of fn(i) back to back on `stream`, with an event pair around
    the whole run and an event between every `block` calls.  Returns the mean
    ms per call over all K and the block means (ms per call)."""
    return timed_blocks_lanes(fn, K, block, (stream,))


def timed_blocks_lanes(fn, K: int, block: int, lanes):
    """Exactly K calls of fn(i) (i = 0..K-1), which may enqueue on any of
    `lanes`, with an event pair around the whole run on lanes[0] and an event
    after every `block` calls (the last block may be shorter).  The other
    lanes wait for the start event, and are joined back into lanes[0] (an
    event wait) before each block's event, so that every block's interval
    covers all of its work.  Returns the mean ms per call over all K and the
    means of the full blocks (ms per call)."""
    import torch
    main, others = lanes[0], lanes[1:]
    K = max(1, K)
    block = max(1, min(block, K))
    bounds = list(range(0, K, block)) + [K]
    evs = [_ev() for _ in bounds]
    torch.cuda.synchronize()
    evs[0].record(main)
    for s in others:
        s.wait_event(evs[0])
    for b in range(len(bounds) - 1):
        for i in range(bounds[b], bounds[b + 1]):
            fn(i)
        for s in others:
            e = torch.cuda.Event()
            e.record(s)
            main.wait_event(e)
        evs[b + 1].record(main)
    torch.cuda.synchronize()
    per = [evs[b].elapsed_time(evs[b + 1]) / block for b in range(len(bounds) - 1)
           if bounds[b + 1] - bounds[b] == block]
    if not per:
        per = [evs[0].elapsed_time(evs[-1]) / K]
    return evs[0].elapsed_time(evs[-1]) / K, per


# The streams the layer steps alternate over (set by main; one stream when
# --one-stream).  A layer's launches always go to the same one.
LANES = None


def lane(L):
    return LANES[L.idx % len(LANES)]


def _stats(per):
    a = np.asarray(per, np.float64)
    return {"median_ms": round(float(np.median(a)), 5), "p10_ms": round(float(np.percentile(a, 10)), 5),
            "p90_ms": round(float(np.percentile(a, 90)), 5), "blocks": int(a.size)}


def _time_calls(fns, K, stream):
    """Average ms of one pass over fns (each enqueued on stream), over K back-to-back passes after 5 warm-ups."""
    import torch
    for _ in range(5):
        for f in fns:
            f(stream)
    torch.cuda.synchronize()
    a, b = _ev(), _ev()
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


# ---------------------------------------------------------------------- host side
def host_plan_us(density: float, reps: int = 50):
    """The a1 host work of one layer timed alone: one sft_plan_layer call
    (the row tracker's window, the row plan and the moment slots of the seven
    matrices, written into pinned memory), median over `reps` repetitions.
    Each repetition starts from the state of a run in progress -- charges from
    an earlier window of the same hot rows, and those rows holding slots --
    restored before the clock starts; the magnitudes are drawn beforehand."""
    import torch

    from sparse_full_weight_amd import _lib, synth
    names = list(synth.LLAMA7B)
    Rs = [synth.LLAMA7B[n][0] for n in names]
    mags = []
    for mi, R in enumerate(Rs):
        hot = synth.clustered_rows(R, round(density * R), 7 + mi)
        mags.append(synth.tracker_magnitudes(R, hot, 8 + mi))
    words = _lib.LayerPlanner(Rs, Rs).words
    pinned = torch.zeros(words, dtype=torch.int32).pin_memory()
    pl = _lib.LayerPlanner(Rs, Rs, pinned.data_ptr(), words)
    # an earlier window of the same hot rows (no background): those rows now
    # hold charges and slots, and the timed window keeps exactly them active
    pl.plan([np.where(m >= 0.1, m, np.float32(0)).astype(np.float32) for m in mags])
    ch0 = [c.copy() for c in pl.charge]
    rs0 = [r.copy() for r in pl.row_slot]
    pl.bind(mags)
    times = []
    for _ in range(reps):
        for i in range(len(Rs)):
            pl.charge[i][:] = ch0[i]
            pl.row_slot[i][:] = rs0[i]
        t0 = time.perf_counter()
        pl.step()
        times.append((time.perf_counter() - t0) * 1e6)
    return {"median_us": round(float(np.median(times)), 1), "p10_us": round(float(np.percentile(times, 10)), 1),
            "p90_us": round(float(np.percentile(times, 90)), 1), "reps": reps,
            "n_active": int(sum(int(np.count_nonzero(r >= 0)) for r in pl.row_slot)),
            "calls": "one sft_plan_layer call over the 7 matrices (42,496 rows): tracker windows, row plans and "
                     "moment slots into pinned memory, through the ctypes binding (magnitude arrays bound once, "
                     "refilled in place by a training loop)"}


def host_info():
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def cpu_baseline(L0: "Layer", threads: int):
    """Time the oracle (plain C) on samples of one layer's active rows: their
    masked dW rows (fp64 sums over the 4096 tokens) and their update, scaled
    to the whole layer.  Once on one thread (every 8th active row of each
    matrix) and once on `threads` host threads, each taking a share of the
    rows (every 2nd active row; the C oracle releases the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import torch
    host = {}
    for gname, members in L0.groups_def:
        Xb = L0.X[gname].view(torch.int16).cpu().numpy().view(np.uint16)
        for name in members:
            m = L0.mats[name]
            host[name] = (Xb, m["dY"].view(torch.int16).cpu().numpy().view(np.uint16), m["q"].cpu().numpy(),
                          m["s"].cpu().numpy(), m["delta"].cpu().numpy())

    def rows_work(name, rows):
        Xb, dY, q, s, delta = host[name]
        C = q.shape[1]
        st = oracle.MatState(q[rows], s[rows], delta[rows], np.zeros((rows.size, C), np.uint16),
                             np.zeros((rows.size, C), np.uint16), np.zeros(rows.size, np.int32),
                             np.zeros((rows.size, C), np.uint16))
        G = oracle.masked_dw(dY, Xb, rows)
        k = np.arange(rows.size, dtype=np.int32)
        oracle.sparse_update(st, G, k, k, None, **HP)

    def run(every, n_threads):
        jobs, done, total = [], 0, 0
        for name, m in L0.mats.items():
            rows = m["plan"].active_rows[::every].copy()
            total += m["plan"].n_active
            done += rows.size
            for part in np.array_split(rows, max(1, min(rows.size, 4 * n_threads))):
                if part.size:
                    jobs.append((name, part))
        t0 = time.perf_counter()
        if n_threads == 1:
            for j in jobs:
                rows_work(*j)
        else:
            with ThreadPoolExecutor(max_workers=n_threads) as ex:
                list(ex.map(lambda j: rows_work(*j), jobs))
        dt = time.perf_counter() - t0
        return dt * total / done * 1e3, done, total, dt

    one_ms, one_done, total, one_s = run(8, 1)
    many_ms, many_done, _, many_s = run(2, threads)
    info = host_info()
    configs = cpu_configs(L0, threads, many_ms, total)
    return {"value": round(many_ms, 1), "unit": "ms", "cores": threads, "kind": "oracle",
            "sample": (f"every 2nd active row of each of the 7 matrices of one layer ({many_done} of {total} rows: "
                       f"masked dW rows + their update, {many_s:.1f} s on {threads} threads), scaled to the "
                       f"whole layer"),
            "single_thread": {"value": round(one_ms, 1), "unit": "ms", "cores": 1,
                              "sample": f"every 8th active row ({one_done} of {total} rows, {one_s:.1f} s), scaled"},
            "configs": configs, "host": info}


def cpu_configs(L0: "Layer", threads: int, layer_ms: float, layer_rows: int):
    """The oracle on the other configurations, on the same host threads:
    the 512 x 512 projection at T = 256 (51 rows) and the 32000 x 4096
    embedding step (conductor over four windows, plan, scatter-gradient and
    the update of its rows) in full; the one-row-per-tile layer (cfg 5: its
    masked dW rows, the coupled update of the three pairs, the plain update of
    down) on every 16th row of each matrix, scaled; and the 32-layer model step
    at 0.5/1/2/5% rows, extrapolated from the 1% layer's measured time per
    active row (labelled as such)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import torch

    from sparse_full_weight_amd import synth
    out = {}
    # cfg 1
    T, R, C = 256, 512, 512
    X = synth.normal_bf16((T, C), 1.0, 11)
    dY = synth.normal_bf16((T, R), 0.01, 12)
    rows = synth.clustered_rows(R, round(0.10 * R), 13).astype(np.int32)
    q, s_, d_ = synth.quant_state(R, C, 15)
    t0 = time.perf_counter()
    mask = oracle.tracker_window(np.zeros(R, np.float32), synth.tracker_magnitudes(R, rows, 14))
    act = oracle.plan_rows(mask)["active_rows"]
    G = oracle.masked_dw(dY, X, act)
    k = np.arange(act.size, dtype=np.int32)
    st = oracle.MatState(q[act], s_[act], d_[act], np.zeros((act.size, C), np.uint16),
                         np.zeros((act.size, C), np.uint16), np.zeros(act.size, np.int32),
                         np.zeros((act.size, C), np.uint16))
    oracle.sparse_update(st, G, k, k, None, **HP)
    out["cfg1_small_projection_step"] = {"value": round((time.perf_counter() - t0) * 1e3, 2), "unit": "ms",
                                         "cores": 1, "sample": f"whole step ({act.size} rows)"}
    # cfg 2
    V, dd, Tb = 32000, 4096, 8 * 512
    windows = [synth.zipf_tokens(Tb, V, 1.1, 5100 + w) for w in range(4)]
    dYe = synth.normal_bf16((Tb, dd), 0.01, 5110)
    t0 = time.perf_counter()
    ch = np.zeros(V, np.float32)
    for w in windows:
        mask = oracle.conductor_window(ch, w)
    act = oracle.plan_rows(mask)["active_rows"]
    Ge = oracle.embedding_dw(dYe, windows[-1], act)
    k = np.arange(act.size, dtype=np.int32)
    st = oracle.MatState(np.zeros((act.size, dd), np.int8), np.full(act.size, 1e-3, np.float32),
                         np.zeros((act.size, dd), np.float32), np.zeros((act.size, dd), np.uint16),
                         np.zeros((act.size, dd), np.uint16), np.zeros(act.size, np.int32),
                         np.zeros((act.size, dd), np.uint16))
    oracle.sparse_update(st, Ge, k, k, None, **HP)
    out["cfg2_embedding_step"] = {"value": round((time.perf_counter() - t0) * 1e3, 2), "unit": "ms", "cores": 1,
                                  "sample": f"whole step ({act.size} rows, 4 conductor windows)"}
    # cfg 5, sampled on the host threads
    host = {}
    for gname, members in L0.groups_def:
        Xb = L0.X[gname].view(torch.int16).cpu().numpy().view(np.uint16)
        for name in members:
            m = L0.mats[name]
            host[name] = (Xb, m["dY"].view(torch.int16).cpu().numpy().view(np.uint16), m["C"])
    pairs = [("gate", "up"), ("q", "o"), ("k", "v")]
    adv = {name: synth.one_per_tile_rows(L0.mats[name]["R"], 9100 + mi) for mi, name in enumerate(L0.mats)}
    for a, b in pairs:
        adv[b][::2] = adv[a][::2]
    every = 16
    jobs, done, total = [], 0, 0
    for name in L0.mats:
        sample = adv[name][::every].astype(np.int32)
        total += adv[name].size
        done += sample.size
        jobs += [(name, part) for part in np.array_split(sample, 4 * threads) if part.size]

    def work(name, rws):
        Xb, dYm, Cm = host[name]
        Gm = oracle.masked_dw(dYm, Xb, rws)
        kk = np.arange(rws.size, dtype=np.int32)
        z = np.zeros((rws.size, Cm), np.uint16)
        sm = oracle.MatState(np.zeros((rws.size, Cm), np.int8), np.full(rws.size, 1e-3, np.float32),
                             np.zeros((rws.size, Cm), np.float32), z.copy(), z.copy(), np.zeros(rws.size, np.int32),
                             z.copy())
        other = oracle.MatState(np.zeros((rws.size, Cm), np.int8), np.full(rws.size, 1e-3, np.float32),
                                np.zeros((rws.size, Cm), np.float32), z.copy(), z.copy(), np.zeros(rws.size, np.int32),
                                z.copy())
        oracle.coupled_update(sm, Gm, kk, kk, None, other, Gm, kk, kk, None, a_own=1.0, a_cross=0.0318, **HP)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda j: work(*j), jobs))
    dt = time.perf_counter() - t0
    out["cfg5_adversarial_coupled_step"] = {
        "value": round(dt * total / done * 1e3, 1), "unit": "ms", "cores": threads,
        "sample": (f"every {every}th active row of each matrix ({done} of {total} rows: masked dW rows and a coupled "
                   f"update of each sampled row with itself as partner, {dt:.1f} s), scaled")}
    # cfg 4, extrapolated
    per_row = layer_ms / layer_rows
    emb = out["cfg2_embedding_step"]["value"]
    ext = {}
    for dens in (0.005, 0.01, 0.02, 0.05):
        n = sum(round(dens * Rm) for Rm, _ in synth.LLAMA7B.values())
        ext[str(dens)] = round(32 * n * per_row + emb, 1)
    out["cfg4_model_step_extrapolated"] = {
        "value": ext, "unit": "ms", "cores": threads,
        "sample": ("32 layers x the 1% layer's oracle time per active row x the density's active rows, plus the "
                   "embedding step: extrapolated, not run")}
    return out


# ---------------------------------------------------------------------- other workloads
LEAF_DENSITY = 0.001


def leaf_support(m: int, n: int, seed: int):
    """SparseLeaf support: round(0.1% of m*n) distinct coordinates, uniform,
    sorted by (row, column)."""
    from sparse_full_weight_amd import synth
    g = synth.rng(seed)
    flat = np.sort(g.choice(m * n, size=round(LEAF_DENSITY * m * n), replace=False))
    return (flat // n).astype(np.int32), (flat % n).astype(np.int32)


def _warm(fn, calls: int, seconds: float):
    """Untimed calls of fn(i): at least `calls`, and for at least `seconds`
    (after a pause on the host the first steps run slower, more so with the
    lanes overlapping)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < calls or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _ring_step_ms(ring, fn, K, stream, block=12):
    """fn(L, st) enqueues layer L's step on st; the ring's layers alternate
    over the lanes."""
    import torch

    def one(i):
        L = ring[i % len(ring)]
        st = lane(L)
        with torch.cuda.stream(st):
            fn(L, st)
    _warm(one, 5, 0.1)
    return timed_blocks_lanes(one, K, block, LANES)


def _ring_serial_ms(ring, fn, K, stream, block=10):
    """fn(L) enqueues one call of layer L on `stream`; the ring's calls one
    after the other (a call's own duration)."""
    for i in range(5):
        fn(ring[i % len(ring)])
    return timed_blocks(lambda i: fn(ring[i % len(ring)]), K, block, stream)


def small_projection_step(K, stream):
    """The 512 x 512 projection, 256 tokens, 10% of the rows active (51, in
    two clustered tiles): plan upload, masked dW and update in one call."""
    shapes = {"w": (512, 512)}
    groups = (("x", ("w",)),)
    ring = [Layer(300 + i, 256, 0.10, 8000, "packed", shapes=shapes, groups=groups) for i in range(6)]

    def fn(L, st):
        L.upload_plan()
        L.fused_call(st)
    mean, per = _ring_step_ms(ring, fn, K, stream)
    work = ring[0].dw_work().bytes + ring[0].upd_work().bytes
    return dict(_hbm(work, mean), **_stats(per), active_rows=ring[0].n_active(), tokens=256,
                note="launch-latency bound (about 1 MB of work)")


def adversarial_coupled_step(L0, K, stream):
    """One active row in every 32-row tile of every matrix (a pair's second
    matrix shares the first one's row in every other tile): plan upload, packed
    masked dW of the seven matrices, the coupled update of (gate, up), (q, o),
    (k, v) at coupling strength 0.6 with the schedule's coefficients at its
    first step, weight decay 0.01 cos(28.4 deg), and the plain update of down."""
    import torch

    from sparse_full_weight_amd import _lib, accounting, synth
    pairs = [("gate", "up"), ("q", "o"), ("k", "v")]
    rows = {name: synth.one_per_tile_rows(L0.mats[name]["R"], 9100 + mi) for mi, name in enumerate(L0.mats)}
    for a, b in pairs:
        rows[b][::2] = rows[a][::2]
    bufs = (L0.X, {n: {k: m[k] for k in ("R", "C", "dY", "q", "s", "delta", "w_live")} for n, m in L0.mats.items()})
    L = Layer(0, L0.T, 0.0, 9000, "packed", buffers=bufs, rows=rows)
    helix = _lib.Helix()
    helix.step(6.17)
    a_own, a_cross = helix.coupling(0.6, 0.0)
    wd = float(np.float32(0.01 * math.cos(math.radians(28.4))))
    bc1, bc2 = L.hp.bc1, L.hp.bc2
    hp = _lib.Adam(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], bc1, bc2, wd)
    by_name = {name: u for name, u in zip([n for _, mm in L.groups_def for n in mm], L.upd)}
    cp = _lib.prepare_coupled_update([_lib.Pair(by_name[a], by_name[b], a_own, a_cross) for a, b in pairs], hp)
    dn = _lib.prepare_sparse_update([by_name["down"]], hp)

    def step(_):
        L.upload_plan()
        L.dw_call(stream)
        cp(stream)
        dn(stream)
    for i in range(3):
        step(i)
    mean, per = timed_blocks(step, K, 10, stream)
    w_dw = L.dw_work()
    sides = []
    for a, b in pairs:
        shared = int(np.intersect1d(rows[a], rows[b]).size)
        sides += [(L.mats[a]["C"], rows[a].size, shared), (L.mats[b]["C"], rows[b].size, shared)]
    w_up = (accounting.coupled_update_work(sides).bytes
            + accounting.update_work([(L.mats["down"]["C"], rows["down"].size)]).bytes)
    t_dw = _time_calls([L.dw_call], K, stream)
    t_cp = _time_calls([cp, dn], K, stream)
    out = dict(_hbm(w_dw.bytes + w_up, mean), **_stats(per), active_rows=L.n_active(), a_own=a_own,
               a_cross=round(a_cross, 6), coupling_strength=0.6, weight_decay=wd,
               useful_TFLOP_s=round(w_dw.flops_useful / (mean * 1e-3) / 1e12, 1),
               whole_tile_TFLOP=round(w_dw.flops_issued / 1e12, 3),
               packed_dw=dict(_hbm(w_dw.bytes, t_dw),
                              useful_TFLOP_s=round(w_dw.flops_useful / (t_dw * 1e-3) / 1e12, 1)),
               coupled_and_down_update=_hbm(w_up, t_cp))
    del L
    torch.cuda.empty_cache()
    return out


def model_step(T, K, stream, densities=(0.005, 0.01, 0.02, 0.05), n_layers=32):
    """The whole 7B-shaped model: 32 layers with distinct activations,
    gradients and state, and the 32000 x 4096 embedding; fresh seeded masks
    per layer at each density.  One step = every layer's plan upload and fused
    call (consecutive layers on alternate lanes), then the embedding's plan
    upload, scatter-gradient and update."""
    import torch
    t0 = time.perf_counter()
    bufs = [layer_buffers(T, 11000 + 100 * i) for i in range(n_layers)]
    torch.cuda.synchronize()
    setup = time.perf_counter() - t0
    out = {"layers": n_layers, "tokens": T, "setup_s": round(setup, 1)}
    emb = None
    for density in densities:
        layers = [Layer(i, T, density, 12000 + int(density * 1e4) * 1000, "packed", buffers=bufs[i])
                  for i in range(n_layers)]
        if emb is None:
            emb = Embedding(13000, layers[0].hp)

        def step(_):
            for L in layers:
                st = lane(L)
                with torch.cuda.stream(st):
                    L.upload_plan()
                L.fused_call(st)
            emb.step(stream)
        _warm(step, 2, 0.3)
        mean, per = timed_blocks_lanes(step, K, 1, LANES)
        work = sum(L.dw_work().bytes + L.upd_work().bytes for L in layers) + emb.work()
        out[f"{density:g}"] = dict(_hbm(work, mean), **_stats(per),
                                   ms_per_layer=round(mean / n_layers, 5),
                                   active_rows_per_layer=round(float(np.mean([L.n_active() for L in layers])), 1),
                                   embedding_active_rows=emb.n,
                                   hbm_roofline_ms=round(work / (HBM_PEAK_GBS * 1e9) * 1e3, 4))
        del layers
        torch.cuda.empty_cache()
    del bufs, emb
    torch.cuda.empty_cache()
    return out


def other_rows(L0: "Layer", K: int, stream, with_model=True, model_steps=10):
    """The other workloads and calls, each timed over back-to-back prepared
    calls on the stream (see the module docstring)."""
    import torch

    from sparse_full_weight_amd import _lib, accounting, synth
    dev = "cuda"
    out = {}
    hp = L0.hp

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
        st["e"] = torch.zeros((n, 2), dtype=torch.int8, device=dev)
        st["slot"] = torch.arange(n, dtype=torch.int32, device=dev)
        return st

    def upd(st, rows_dev, G, n):
        return _lib.UpdMat(st["q"], st["s"], st["delta"], st["m"], st["v"], st["t"], st["e"], rows_dev, st["slot"],
                           G, n, None, st["w"])

    # ---- cfg 1: the 512 x 512 projection
    out["cfg1_small_projection_step"] = small_projection_step(K, stream)

    # ---- cfg 5: the adversarial layer with the coupled update, as one step
    out["cfg5_adversarial_coupled_step"] = adversarial_coupled_step(L0, K, stream)

    # ---- cfg 2: the embedding workload as one step, and its scatter-gradient alone
    emb = Embedding(9000, hp)
    w_emb = accounting.embedding_dw_work(emb.d, emb.nnz, emb.n).bytes
    out["a3_embedding_dw"] = dict(_hbm(w_emb, _time_calls([emb.emb_call], K, stream)), active_rows=emb.n,
                                  hit_tokens=emb.nnz, table=[emb.V, emb.d], tokens=emb.Tb)
    mean, per = timed_blocks(lambda i: emb.step(stream), K, 10, stream)
    out["cfg2_embedding_step"] = dict(_hbm(emb.work(), mean), **_stats(per),
                                      host_conductor_plan_us=round(emb.host_us, 1),
                                      note="plan upload + scatter-gradient + sparse update with write-back")
    del emb

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
    cks = [_lib.CkptMat.alloc(u.q, u.s, u.delta, u.m, u.v, u.t, u.mv_exp, u.active_rows, u.slot, u.n_active,
                              u.w_live) for u in L0.upd]
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

    # ---- the layer step at the model's other row densities (0.5%, 2%, 5%),
    # plan upload included, over a ring of 12 layers at each density (spread
    # evenly over the lanes)
    sweep = {}
    for density in (0.005, 0.02, 0.05):
        ring = [Layer(100 + i, L0.T, density, 6000, "packed") for i in range(12)]

        def fn(L, st):
            L.upload_plan()
            L.fused_call(st)
        mean, per = _ring_step_ms(ring, fn, K, stream)
        work = ring[0].dw_work().bytes + ring[0].upd_work().bytes
        sweep[f"{density:g}"] = dict(_hbm(work, mean), **_stats(per), active_rows=ring[0].n_active())
        del ring
        torch.cuda.empty_cache()
    out["c_density_sweep_step"] = sweep

    # ---- one GPU's share of a token-sharded step: the same 1% layer step (fused
    # call, plan upload included) on T/N tokens, the shape each of N GPUs would
    # run before the dW exchange (which is not built here)
    share = {}
    for n_gpu in (2, 4, 8):
        T = L0.T // n_gpu
        ring = [Layer(200 + i, T, L0.density, 7000, "packed") for i in range(12)]
        dw_b, up_b = ring[0].dw_work().bytes, ring[0].upd_work().bytes

        def fn(L, st):
            L.upload_plan()
            L.fused_call(st)
        mean, _ = _ring_step_ms(ring, fn, K, stream)
        dw_ms, _ = _ring_serial_ms(ring, lambda L: L.dw_call(stream), K, stream)
        share[f"T{T}"] = dict(_hbm(dw_b + up_b, mean), n_gpus_sharing=n_gpu, tokens=T, masked_dw=_hbm(dw_b, dw_ms))
        del ring
        torch.cuda.empty_cache()
    out["e_token_share_step"] = share

    # ---- cfg 4: the whole model (32 layers + embedding) at four densities
    if with_model:
        print("[bench] timing the 32-layer model step", file=sys.stderr, flush=True)
        out["cfg4_model_step"] = model_step(L0.T, model_steps, stream)
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


SKIP_PROBE_TILES = (0, 1, 2, 4, 8, 16)
SKIP_PROBE_CALLS = 3


def skip_probe():
    """Masked dW of one 4096 x 4096 matrix (T = 4096, whole-tile layout) with
    0, 1, 2, 4, 8 and 16 of its 128 row tiles active (every 8th tile), each
    called SKIP_PROBE_CALLS times in that order: run under rocprofv3's
    FETCH_SIZE / WRITE_SIZE counters, the dispatches show what a skipped tile
    costs (none is launched for an all-skipped call)."""
    import torch

    from sparse_full_weight_amd import _lib, synth
    T, R, C = 4096, 4096, 4096
    X = synth.normal_bf16_device((T, C), 1.0, 71, "cuda")
    dY = synth.normal_bf16_device((T, R), 0.01, 72, "cuda")
    out = []
    for k in SKIP_PROBE_TILES:
        mask = np.zeros(R, np.uint8)
        for t in range(k):
            mask[32 * 8 * t: 32 * 8 * t + 32] = 1
        plan = _lib.sft_plan_rows(mask)
        dW = torch.empty((max(plan.n_active, 1), C), dtype=torch.float32, device="cuda")
        groups = [_lib.DwGroup(X, [_lib.DwMat(dY, plan.to_device("cuda"), dW[:plan.n_active])], _lib.SFT_DW_TILES)]
        nbytes = _lib.sft_masked_dw_workspace(groups)
        ws = torch.zeros(max(nbytes // 4, 1), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        for _ in range(SKIP_PROBE_CALLS):
            _lib.sft_masked_dw(groups, ws)
        torch.cuda.synchronize()
        out.append({"active_tiles": k, "active_rows": plan.n_active, "calls": SKIP_PROBE_CALLS})
        print(f"[skip-probe] {k} active tiles done", file=sys.stderr, flush=True)
    print(json.dumps({"skip_probe": out, "T": T, "R": R, "C": C}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path would shard over "
              "token positions: each GPU the masked dW of its own tokens, then one reduce-scatter of the active rows)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    if args.skip_probe:
        skip_probe()
        return
    torch.cuda.set_device(0)
    print(f"[bench] building {args.layers} layers (T={args.tokens}, density={args.density})", file=sys.stderr,
          flush=True)
    t0 = time.perf_counter()
    layers = [Layer(i, args.tokens, args.density, 5000, args.layout) for i in range(args.layers)]
    torch.cuda.synchronize()
    print(f"[bench] setup {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)

    from sparse_full_weight_amd import synth
    stream = torch.cuda.current_stream()
    global LANES
    n_lanes = 1 if args.one_stream else max(1, args.lanes)
    LANES = (stream,) + tuple(torch.cuda.Stream() for _ in range(n_lanes - 1))
    if args.rows_only:
        print(json.dumps({"rows": other_rows(layers[0], min(args.steps, 100), stream, not args.no_model,
                                             args.model_steps)}), flush=True)
        return

    def call(L, st):
        if args.unfused:
            L.dw_call(st)
            L.upd_call(st)
        else:
            L.fused_call(st)

    def step(i, lanes=None):
        # the step: this step's plan to the device, then the masked dW and
        # update, on the layer's lane.  (Copying the next step's plan on
        # another stream during this step, ordered by events, measured slower:
        # the cross-stream waits cost more than the copy.)
        L = layers[i % len(layers)]
        st = lane(L) if lanes is None else lanes[0]
        with torch.cuda.stream(st):
            L.upload_plan()
        call(L, st)

    def step_resident(i, lanes=None):
        L = layers[i % len(layers)]
        call(L, lane(L) if lanes is None else lanes[0])

    one = (stream,)

    # Untimed: about 0.1 s of steps so that the clocks have settled, then the
    # W warmup steps.
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.1:
        for i in range(len(layers)):
            step(i)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    # The timed loop: K whole steps back to back, with an event pair around the
    # run and an event every `block` steps (between steps, never inside one).
    ms_per_step, per_block = timed_blocks_lanes(step, K, args.block, LANES)
    if args.steps_only:
        print(json.dumps({"ms_per_step": round(ms_per_step, 5), "steps": K, "lanes": len(LANES)}), flush=True)
        return
    ms_resident, per_block_res = timed_blocks_lanes(step_resident, K, args.block, LANES)
    # the same steps with every layer on one stream
    ms_one, per_one = timed_blocks_lanes(lambda i: step(i, one), K, args.block, one)
    ms_one_res, _ = timed_blocks_lanes(lambda i: step_resident(i, one), K, args.block, one)

    # Per-call durations, each timed over its own back-to-back run of K calls
    # on the same stream and inputs (the masked-dW call is the gather, product
    # and fix-up kernels; the update call is one kernel).
    for L in layers:
        L.upload_plan()
    dw_avg, _ = timed_blocks(lambda i: layers[i % len(layers)].dw_call(stream), K, K, stream)
    up_avg, _ = timed_blocks(lambda i: layers[i % len(layers)].upd_call(stream), K, K, stream)
    fu_avg, _ = timed_blocks(lambda i: layers[i % len(layers)].fused_call(stream), K, K, stream)

    L0 = layers[0]
    dw = L0.dw_work()
    up = L0.upd_work()
    dw_gbs = dw.bytes / (dw_avg * 1e-3) / 1e9
    up_gbs = up.bytes / (up_avg * 1e-3) / 1e9
    fu_gbs = (dw.bytes + up.bytes) / (fu_avg * 1e-3) / 1e9
    step_gbs = (dw.bytes + up.bytes) / (ms_per_step * 1e-3) / 1e9
    n_act = L0.n_active()
    n_tiles = sum(m["plan"].n_active_tiles for m in L0.mats.values())

    # HBM bytes per masked-dW call from the committed counter summary, if it
    # was taken on the current kernel source (else null).
    from sparse_full_weight_amd import profsum
    rec = profsum.read_traffic(os.path.join(ROOT, "profiles", COUNTERS_SUMMARY))
    traffic = None
    if rec and rec.get("sft_dw_sha256") == profsum.source_hash("sft_dw.hip"):
        traffic = rec["masked_dw_call_bytes"]
    # HBM bytes a step touches (the dW call and the update kernel the step
    # ran, from the same counters; both sources unchanged since), against the
    # step time
    step_traffic = None
    if (traffic is not None and rec.get("sft_update_sha256") == profsum.source_hash("sft_update.hip")
            and not args.unfused):
        ks = rec["kernels"]
        # split tiles (a fix-up ran) make the step's update the fused kernel
        upd = "k_fused_update" if "k_dw_fixup" in ks else "k_sparse_update"
        if upd in ks:
            b = traffic + ks[upd]["read_bytes"] + ks[upd]["write_bytes"]
            gbs = b / (ms_per_step * 1e-3) / 1e9
            step_traffic = {"bytes": b, "update_kernel": upd, "GB_s": round(gbs, 1),
                            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}

    print("[bench] timing the a1 host calls", file=sys.stderr, flush=True)
    host_plan = host_plan_us(args.density)

    rows = None
    if not args.no_rows:
        print("[bench] timing the other workloads and calls", file=sys.stderr, flush=True)
        rows = other_rows(L0, min(K, 100), stream, not args.no_model, args.model_steps)

    ceil = None
    if not args.no_ceilings:
        print("[bench] probing the sustained HBM and matrix-core rates", file=sys.stderr, flush=True)
        ceil = ceilings(stream)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on samples", file=sys.stderr, flush=True)
        cpu = cpu_baseline(L0, CPU_THREADS)

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
                   "step": ("the step's packed plan (one sft_plan_layer output, a few KB, pinned) copied host -> "
                            "device, then masked dW (7 matrices) + sparse update with fused write-back "
                            "(7 matrices), "
                            + ("two calls" if args.unfused else
                               "one call: sft_masked_dw_update, the split tiles' fix-up done by the update")
                            + "; activations, gradients and state resident in HBM; consecutive layers' steps "
                              "alternate between the lanes (streams of the default priority, a layer always on "
                              "the same one), so one layer's step overlaps the next one's"),
                   "lanes": len(LANES),
                   "step_stats": _stats(per_block),
                   "ms_per_step_plan_resident": round(ms_resident, 5),
                   "step_stats_plan_resident": _stats(per_block_res),
                   "ms_per_step_one_stream": round(ms_one, 5),
                   "step_stats_one_stream": _stats(per_one),
                   "ms_per_step_one_stream_plan_resident": round(ms_one_res, 5),
                   "step_GB_s": round(step_gbs, 1), "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
                   "step_traffic": step_traffic,
                   "hbm_roofline_ms": round((dw.bytes + up.bytes) / (HBM_PEAK_GBS * 1e9) * 1e3, 5)},
        "roofline": {"bound": "hbm", "kernel": ("sft_masked_dw (k_dw_gather + k_masked_dw, + k_dw_fixup where the "
                                                "launch splits tiles; the 1% layer's narrow tiles split none)"),
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
        "host_plan_us_per_layer": host_plan,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
