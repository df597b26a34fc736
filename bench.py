"""Benchmark of the sparse-first step on one MI355X.

Workload: one Llama-7B-shaped decoder layer (q, k, v, o 4096x4096; gate, up
11008x4096; down 4096x11008), 4096 tokens, bf16 X ~ N(0,1) and dY ~ N(0,0.01),
row-tracker masks from seeded output magnitudes with 1% of each matrix's rows
active (clustered in 32-row tiles), int8 q + fp32 residual resident, fp16
moments for the active rows.  One step = the packed plan upload (one
host->device copy), the masked dW of all seven matrices (one launch; q/k/v
and gate/up share their input), and the sparse update with fused write-back
of all seven (one launch).  Method: "Sparse-First Fine-Tuning: Full-Weight
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


class Layer:
    """Device buffers, plans and prepared launches of one layer."""

    def __init__(self, idx: int, T: int, density: float, seed0: int, layout: str = "packed"):
        import torch

        from sparse_full_weight_amd import _lib, synth
        self.idx = idx
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

    def step(L):
        L.upload_plan()
        if args.unfused:
            L.dw_call(stream)
            L.upd_call(stream)
        else:
            L.fused_call(stream)

    for i in range(args.warmup):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()

    K = args.steps
    # The timed loop: K whole steps back to back, bracketed by one event pair
    # (per-step events would put markers between the kernels).
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(layers[i % len(layers)])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K

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
                   "step": ("plan upload + masked dW (7 matrices) + sparse update with fused write-back "
                            "(7 matrices), " + ("two calls" if args.unfused else
                                                "one call: sft_masked_dw_update, the split tiles' fix-up "
                                                "done by the update"))},
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
        "host_plan_us_per_layer": round(host_plan_us, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
