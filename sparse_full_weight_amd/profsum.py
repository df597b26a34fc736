"""Summaries of rocprofv3 output for the kernels of this library.

Two summaries, both plain text meant to be kept next to the numbers they
support:

* ``stats``: per-kernel call count and average/min/max duration from a
  ``--kernel-trace --stats --output-format csv`` run, plus the sum over the
  kernels of one masked-dW call (gather, product, fix-up);
* ``counters``: HBM bytes per dispatch from two ``--pmc`` runs of the same
  program (``FETCH_SIZE``, then ``WRITE_SIZE``, both in KiB), each scaled by
  what the same counter reads for a plain device copy of known size (a
  ``bench.py --copy-calibration`` run under the same counter).  The last line
  is machine-readable (``traffic-json: {...}``) and carries the SHA-256 of the
  kernel source the counters were taken on, so that a reader can tell when
  they no longer describe the code;
* ``units``: how busy the texture address (TA) and texture data (TD) units,
  the matrix cores and the L2 read path were during one kernel, from a
  ``--pmc`` run of ``GRBM_GUI_ACTIVE TA_TA_BUSY_sum TD_TD_BUSY_sum
  SQ_VALU_MFMA_BUSY_CYCLES`` (and a second of ``TCP_TCC_READ_REQ_LATENCY_sum
  TCP_TCC_READ_REQ_sum``).  On MI355X ``GRBM_GUI_ACTIVE`` adds the 8 XCDs'
  active cycles, the TA and TD sums add the 256 CUs' and the MFMA-busy sum
  the 1024 SIMDs' busy cycles; the fractions divide by those counts.  With
  ``SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS`` collected too it
  adds the LDS's busy fraction (the 256 CUs' LDS cycles) and the bank-conflict
  cycles per LDS instruction;
* ``skip``: HBM bytes per masked-dW call against the number of active 32-row
  tiles, from ``FETCH_SIZE`` / ``WRITE_SIZE`` runs of ``bench.py
  --skip-probe`` (calls with 0, 1, 2, 4, 8, 16 active tiles of 128, three
  each, in that order), scaled like ``counters``;
* ``overlap``: how much kernels of a ``--kernel-trace`` run ran at the same
  time (from ``*_kernel_trace.csv``): the span from the first start to the
  last end, the time at least one kernel ran, the time two or more did, and
  the sum of all durations, over the dispatches of this library's kernels
  (plus the plan copies) from the named dispatch on.

Usage:
  python -m sparse_full_weight_amd.profsum stats <kernel_stats.csv> --cmd "<command>" > out.txt
  python -m sparse_full_weight_amd.profsum counters --fetch <dir> --write <dir> \\
      --copy-fetch <dir> --copy-write <dir> --cmd "<commands>" > out.txt
  python -m sparse_full_weight_amd.profsum units --runs <dir> [<dir> ...] --kernel k_masked_dw \\
      --label "<workload>" ... --cmd "<commands>" > out.txt
  python -m sparse_full_weight_amd.profsum skip --fetch <dir> --write <dir> \\
      --copy-fetch <dir> --copy-write <dir> --cmd "<commands>" > out.txt
  python -m sparse_full_weight_amd.profsum overlap <kernel_trace.csv> --cmd "<command>" > out.txt
(each <dir> holds the ``*_counter_collection.csv`` of one run).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
DW_KERNELS = ("k_dw_gather", "k_masked_dw", "k_dw_fixup")
UPDATE_KERNELS = ("k_sparse_update", "k_coupled_update", "k_fused_update")
COPY_BYTES = 1 << 30            # bench.py --copy-calibration copies 1 GiB per launch


def source_hash(name: str = "sft_dw.hip") -> str:
    with open(os.path.join(ROOT, "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short(name: str) -> str:
    """Kernel name without namespace and parameter list."""
    base = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return base.split("(")[0].strip()


def kernel_of(name: str, kernels) -> str | None:
    s = short(name)
    for k in kernels:
        if s == k or s.startswith(k + "<"):
            return k
    return None


def stats(path: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel-trace statistics", f"# command: {cmd}", "",
           f"{'kernel':40s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    dw_sum = 0.0
    for r in rows:
        s = short(r["Name"])
        if s.startswith("at::") or "at::native" in r["Name"]:
            continue
        avg = float(r["AverageNs"]) / 1e3
        out.append(f"{s[:40]:40s} {int(r['Calls']):6d} {avg:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                   f"{float(r['MaxNs']) / 1e3:9.2f}")
        if kernel_of(r["Name"], DW_KERNELS):
            dw_sum += avg
    out += ["", f"sft_masked_dw call (k_dw_gather + k_masked_dw, + k_dw_fixup where it ran), "
                f"sum of averages: {dw_sum:.2f} us"]
    return "\n".join(out) + "\n"


def _counter(dirname: str, counter: str) -> dict:
    files = glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {dirname}")
    per: dict = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def _copy_kib(per) -> float:
    """Average counter value (KiB) of the 1 GiB copies of a calibration run."""
    vals = [v for k, vs in per.items() if "copyBuffer" in k or "copy" in short(k).lower() for v in vs]
    vals = [v for v in vals if v > 1024]     # the 1 GiB copies, not small blits
    return sum(vals) / len(vals)


def counters(fetch: str, write: str, copy_fetch: str, copy_write: str, cmd: str) -> str:
    f = _counter(fetch, "FETCH_SIZE")
    w = _counter(write, "WRITE_SIZE")
    cf = _counter(copy_fetch, "FETCH_SIZE")
    cw = _counter(copy_write, "WRITE_SIZE")

    copy_kib = _copy_kib
    f_scale = (COPY_BYTES / 1024) / copy_kib(cf)
    w_scale = (COPY_BYTES / 1024) / copy_kib(cw)

    def avg_kib(per, kernels):
        res = {}
        for name, vals in per.items():
            k = kernel_of(name, kernels)
            if k:
                res.setdefault(k, []).extend(vals)
        return {k: sum(v) / len(v) for k, v in res.items()}

    out = ["# HBM traffic per dispatch from rocprofv3 counters",
           f"# commands: {cmd}", "",
           f"calibration: a 1 GiB device copy reads FETCH_SIZE {copy_kib(cf):.0f} KiB and WRITE_SIZE "
           f"{copy_kib(cw):.0f} KiB per launch -> scale FETCH_SIZE x{f_scale:.4f}, WRITE_SIZE x{w_scale:.4f}", "",
           f"{'kernel':20s} {'FETCH KiB':>12s} {'WRITE KiB':>12s} {'read MB':>10s} {'written MB':>11s}"]
    fk = avg_kib(f, DW_KERNELS + UPDATE_KERNELS)
    wk = avg_kib(w, DW_KERNELS + UPDATE_KERNELS)
    total = {}
    for k in DW_KERNELS + UPDATE_KERNELS:
        if k not in fk:
            continue
        rd = fk[k] * 1024 * f_scale
        wr = wk.get(k, 0.0) * 1024 * w_scale
        total[k] = {"read_bytes": round(rd), "write_bytes": round(wr)}
        out.append(f"{k:20s} {fk[k]:12.1f} {wk.get(k, 0.0):12.1f} {rd / 1e6:10.2f} {wr / 1e6:11.2f}")
    dw = sum(v["read_bytes"] + v["write_bytes"] for k, v in total.items() if k in DW_KERNELS)
    out += ["", f"sft_masked_dw call (gather + product + fix-up): {dw / 1e6:.2f} MB of HBM traffic per call"]
    rec = {"kernels": total, "masked_dw_call_bytes": dw, "fetch_scale": f_scale, "write_scale": w_scale,
           "sft_dw_sha256": source_hash("sft_dw.hip"), "sft_update_sha256": source_hash("sft_update.hip")}
    out.append("traffic-json: " + json.dumps(rec, sort_keys=True))
    return "\n".join(out) + "\n"


XCDS, CUS, SIMDS = 8, 256, 1024


def _kernel_avgs(dirname: str, kernel: str) -> dict:
    """Average per dispatch of every counter a run collected for `kernel`."""
    files = glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {dirname}")
    per: dict = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if kernel_of(r["Kernel_Name"], (kernel,)):
                per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {c: sum(v) / len(v) for c, v in per.items()}


def units(groups, labels, kernel: str, cmd: str) -> str:
    """groups: per workload, the run directories whose counters it combines."""
    out = [f"# unit activity of {kernel} from rocprofv3 counters", f"# commands: {cmd}",
           f"# fractions: TA and TD busy cycles / ({CUS} CUs x active cycles per XCD), MFMA busy cycles / "
           f"({SIMDS} SIMDs x active cycles per XCD), VALU busy = 4 x SQ_ACTIVE_INST_VALU (quad-cycles) / "
           f"({SIMDS} SIMDs x active cycles per XCD), active cycles per XCD = GRBM_GUI_ACTIVE / {XCDS}; "
           f"VALU inst/wave = SQ_INSTS_VALU / SQ_WAVES", "",
           f"{'workload':28s} {'cycles/XCD':>11s} {'TA busy':>8s} {'TD busy':>8s} {'MFMA busy':>10s} "
           f"{'L2 read latency (cyc)':>22s} {'LDS busy':>9s} {'conflict cyc/LDS inst':>22s} {'VALU busy':>9s} "
           f"{'VALU inst/wave':>15s}"]
    for label, dirs in zip(labels, groups):
        v: dict = {}
        for d in dirs:
            v.update(_kernel_avgs(d, kernel))
        g = v.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        frac = lambda c, n: f"{v[c] / (n * g):8.3f}" if c in v and g else f"{'-':>8s}"
        lat = (f"{v['TCP_TCC_READ_REQ_LATENCY_sum'] / v['TCP_TCC_READ_REQ_sum']:22.0f}"
               if v.get("TCP_TCC_READ_REQ_sum") else f"{'-':>22s}")
        conf = (f"{v['SQ_LDS_BANK_CONFLICT'] / v['SQ_INSTS_LDS']:22.2f}"
                if v.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in v else f"{'-':>22s}")
        valu = (f"{4.0 * v['SQ_ACTIVE_INST_VALU'] / (SIMDS * g):9.3f}" if "SQ_ACTIVE_INST_VALU" in v and g
                else f"{'-':>9s}")
        ipw = (f"{v['SQ_INSTS_VALU'] / v['SQ_WAVES']:15.0f}" if v.get("SQ_WAVES") and "SQ_INSTS_VALU" in v
               else f"{'-':>15s}")
        out.append(f"{label:28s} {g:11.0f} {frac('TA_TA_BUSY_sum', CUS)} {frac('TD_TD_BUSY_sum', CUS)} "
                   f"{frac('SQ_VALU_MFMA_BUSY_CYCLES', SIMDS):>10s} {lat} {frac('SQ_LDS_IDX_ACTIVE', CUS):>9s} {conf} "
                   f"{valu} {ipw}")
    return "\n".join(out) + "\n"


def _dispatches(dirname: str, counter: str) -> list:
    """(dispatch id, short kernel name, value) of every dispatch of a run."""
    rows = []
    for path in glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), short(r["Kernel_Name"]), float(r["Counter_Value"])))
    return sorted(rows)


def skip(fetch: str, write: str, copy_fetch: str, copy_write: str, tiles, calls: int, T: int, cmd: str) -> str:
    """Per-call HBM traffic of the masked-dW kernels against the number of
    active 32-row tiles (the skipped-tile probe: configurations in order,
    `calls` calls each; a configuration without active tiles launches
    nothing)."""
    f_scale = (COPY_BYTES / 1024) / _copy_kib(_counter(copy_fetch, "FETCH_SIZE"))
    w_scale = (COPY_BYTES / 1024) / _copy_kib(_counter(copy_write, "WRITE_SIZE"))
    # (a kernel's template instances count as the kernel)
    fd = [(i, kernel_of(k, DW_KERNELS), v) for i, k, v in _dispatches(fetch, "FETCH_SIZE") if kernel_of(k, DW_KERNELS)]
    wd = [(i, kernel_of(k, DW_KERNELS), v) for i, k, v in _dispatches(write, "WRITE_SIZE") if kernel_of(k, DW_KERNELS)]
    live = [k for k in tiles if k > 0]
    out = ["# HBM traffic of masked-dW calls against active 32-row tiles (4096 x 4096 matrix, 128 tiles)",
           f"# commands: {cmd}", "",
           f"calibration: FETCH_SIZE x{f_scale:.4f}, WRITE_SIZE x{w_scale:.4f} (a 1 GiB device copy)",
           f"dispatches: {len(fd)} FETCH and {len(wd)} WRITE records for {len(live)} configurations with active "
           f"tiles x {calls} calls; the configuration with 0 active tiles launched no kernel"
           if 0 in tiles else f"dispatches: {len(fd)}", ""]
    out.append(f"{'tiles':>5s} {'gather read MB':>15s} {'dY columns MB':>14s} {'product read MB':>16s} "
               f"{'product write MB':>17s} {'fix-up read MB':>15s}")
    # the dispatches of one call: gather, product and (if any tile was cut) fix-up
    calls_f, calls_w = [], []
    for dl, acc in ((fd, calls_f), (wd, calls_w)):
        cur = None
        for _, k, v in dl:
            if k == "k_dw_gather":
                cur = {}
                acc.append(cur)
            if cur is not None:
                cur[k] = cur.get(k, 0.0) + v
    if len(calls_f) != len(live) * calls or len(calls_w) != len(live) * calls:
        raise SystemExit(f"expected {len(live) * calls} calls, found {len(calls_f)} / {len(calls_w)}")
    rec = []
    for i, k in enumerate(live):
        cf = calls_f[i * calls:(i + 1) * calls]
        cw = calls_w[i * calls:(i + 1) * calls]

        def mean(cs, name, scale):
            return sum(c.get(name, 0.0) for c in cs) / len(cs) * 1024 * scale

        g = mean(cf, "k_dw_gather", f_scale)
        pr = mean(cf, "k_masked_dw", f_scale)
        pw = mean(cw, "k_masked_dw", w_scale)
        fx = mean(cf, "k_dw_fixup", f_scale)
        dy = k * 32 * T * 2
        rec.append({"tiles": k, "gather_read": round(g), "dY_bytes": dy, "product_read": round(pr),
                    "product_write": round(pw), "fixup_read": round(fx)})
        out.append(f"{k:5d} {g / 1e6:15.3f} {dy / 1e6:14.3f} {pr / 1e6:16.2f} {pw / 1e6:17.2f} {fx / 1e6:15.2f}")
    out.append("skip-json: " + json.dumps(rec))
    return "\n".join(out) + "\n"


def read_traffic(path: str) -> dict | None:
    """The traffic record of a counters summary, or None if missing."""
    try:
        for line in open(path):
            if line.startswith("traffic-json: "):
                return json.loads(line[len("traffic-json: "):])
    except OSError:
        return None
    return None


def _ours(name: str) -> bool:
    s = short(name)
    return s.startswith("k_") or s.startswith("__amd_rocclr_copyBuffer")


def overlap(path: str, cmd: str, first: int = 0) -> str:
    """Concurrency of the trace's kernels (dispatch id >= first): span, busy
    time (union of the intervals), time with two or more running, and the
    sum of the durations, all in microseconds."""
    rows = [r for r in csv.DictReader(open(path)) if _ours(r["Kernel_Name"]) and int(r["Dispatch_Id"]) >= first]
    iv = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows)
    ev = sorted([(a, 1) for a, _ in iv] + [(b, -1) for _, b in iv], key=lambda e: (e[0], e[1]))
    busy = multi = 0
    depth, last = 0, None
    for t, d in ev:
        if last is not None:
            if depth >= 1:
                busy += t - last
            if depth >= 2:
                multi += t - last
        depth += d
        last = t
    span = (iv[-1][1] - iv[0][0]) if iv else 0
    total = sum(b - a for a, b in iv)
    out = ["# kernel concurrency from a rocprofv3 kernel trace", f"# command: {cmd}", "",
           f"dispatches: {len(iv)} (this library's kernels and the plan copies, from dispatch {first} on)",
           f"span from first start to last end: {span / 1e3:.1f} us",
           f"time with at least one kernel running: {busy / 1e3:.1f} us",
           f"time with two or more running: {multi / 1e3:.1f} us ({(multi / busy if busy else 0):.3f} of the busy time)",
           f"sum of the kernels' durations: {total / 1e3:.1f} us ({(total / busy if busy else 0):.3f} x the busy time)"]
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--cmd", required=True)
    b = sub.add_parser("counters")
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        b.add_argument("--" + k, required=True)
    b.add_argument("--cmd", required=True)
    d = sub.add_parser("skip")
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        d.add_argument("--" + k, required=True)
    d.add_argument("--tiles", default="0,1,2,4,8,16")
    d.add_argument("--calls", type=int, default=3)
    d.add_argument("--tokens", type=int, default=4096)
    d.add_argument("--cmd", required=True)
    c = sub.add_parser("units")
    c.add_argument("--runs", nargs="+", action="append", required=True,
                   help="run directories of one workload (repeat the flag per workload)")
    c.add_argument("--label", action="append", required=True)
    c.add_argument("--kernel", default="k_masked_dw")
    c.add_argument("--cmd", required=True)
    o = sub.add_parser("overlap")
    o.add_argument("csv")
    o.add_argument("--first", type=int, default=0, help="first dispatch id to count")
    o.add_argument("--cmd", required=True)
    args = ap.parse_args(argv)
    if args.what == "stats":
        sys.stdout.write(stats(args.csv, args.cmd))
    elif args.what == "skip":
        sys.stdout.write(skip(args.fetch, args.write, args.copy_fetch, args.copy_write,
                              [int(x) for x in args.tiles.split(",")], args.calls, args.tokens, args.cmd))
    elif args.what == "overlap":
        sys.stdout.write(overlap(args.csv, args.cmd, args.first))
    elif args.what == "units":
        if len(args.runs) != len(args.label):
            raise SystemExit("one --label per --runs")
        sys.stdout.write(units(args.runs, args.label, args.kernel, args.cmd))
    else:
        sys.stdout.write(counters(args.fetch, args.write, args.copy_fetch, args.copy_write, args.cmd))


if __name__ == "__main__":
    main()
