"""Host logic of the profile summaries (sparse_full_weight_amd/profsum.py) on
small synthetic rocprofv3 counter files: the unit-busy fractions divide the
summed busy cycles by the unit counts and the per-XCD active cycles, and
average over dispatches of the named kernel only."""
import csv
import os

from sparse_full_weight_amd import profsum


def _write_run(dirname, rows):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_units_fractions(tmp_path):
    k = "(anonymous namespace)::k_masked_dw((anonymous namespace)::DwParams)"
    other = "(anonymous namespace)::k_dw_gather((anonymous namespace)::DwParams)"
    g = 8 * 1000.0                                    # 1000 active cycles per XCD
    a = str(tmp_path / "a")
    _write_run(a, [(k, "GRBM_GUI_ACTIVE", g), (k, "GRBM_GUI_ACTIVE", g),
                   (k, "TA_TA_BUSY_sum", 256 * 1000 * 0.25), (k, "TA_TA_BUSY_sum", 256 * 1000 * 0.75),
                   (k, "TD_TD_BUSY_sum", 256 * 1000 * 0.8), (k, "TD_TD_BUSY_sum", 256 * 1000 * 0.8),
                   (k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000 * 0.1), (k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000 * 0.1),
                   (other, "TD_TD_BUSY_sum", 1e12)])
    b = str(tmp_path / "b")
    _write_run(b, [(k, "TCP_TCC_READ_REQ_LATENCY_sum", 5000.0), (k, "TCP_TCC_READ_REQ_sum", 10.0)])
    text = profsum.units([[a, b]], ["layer"], "k_masked_dw", "cmd")
    row = [ln for ln in text.splitlines() if ln.startswith("layer")][0].split()
    assert row[1:] == ["1000", "0.500", "0.800", "0.100", "500", "-", "-", "-", "-"]


def test_units_missing_counters_print_dashes(tmp_path):
    k = "(anonymous namespace)::k_masked_dw((anonymous namespace)::DwParams)"
    a = str(tmp_path / "a")
    _write_run(a, [(k, "GRBM_GUI_ACTIVE", 8000.0)])
    row = [ln for ln in profsum.units([[a]], ["x"], "k_masked_dw", "c").splitlines() if ln.startswith("x")][0]
    assert row.split()[1:] == ["1000", "-", "-", "-", "-", "-", "-", "-", "-"]


def test_units_lds_columns(tmp_path):
    k = "void (anonymous namespace)::k_leaf_grad<28>((anonymous namespace)::LeafParams)"
    a = str(tmp_path / "a")
    _write_run(a, [(k, "GRBM_GUI_ACTIVE", 8000.0), (k, "SQ_LDS_IDX_ACTIVE", 256 * 1000 * 0.4),
                   (k, "SQ_LDS_BANK_CONFLICT", 300.0), (k, "SQ_INSTS_LDS", 100.0)])
    row = [ln for ln in profsum.units([[a]], ["leaf"], "k_leaf_grad", "c").splitlines() if ln.startswith("leaf")][0]
    assert row.split()[-4:] == ["0.400", "3.00", "-", "-"]


def _write_dispatches(dirname, rows):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_skip_groups_calls_by_gather_and_scales(tmp_path):
    """Calls start at each gather dispatch; configurations follow in order;
    values are per call and scaled by the copy calibration (here x2 for
    FETCH_SIZE, x1 for WRITE_SIZE)."""
    g = "(anonymous namespace)::k_dw_gather((anonymous namespace)::DwParams)"
    # (the product as one of its template instances, as rocprofv3 names it)
    p = "void (anonymous namespace)::k_masked_dw<0>((anonymous namespace)::DwParams)"
    x = "(anonymous namespace)::k_dw_fixup((anonymous namespace)::DwParams)"
    copy = "__amd_rocclr_copyBuffer"
    gib = (1 << 30) / 1024
    fetch, write = [], []
    for tiles in (1, 2):
        for _ in range(2):
            fetch += [(g, "FETCH_SIZE", 100.0 * tiles), (p, "FETCH_SIZE", 1000.0), (x, "FETCH_SIZE", 10.0)]
            write += [(g, "WRITE_SIZE", 5.0), (p, "WRITE_SIZE", 50.0 * tiles), (x, "WRITE_SIZE", 1.0)]
    d = {n: str(tmp_path / n) for n in ("f", "w", "cf", "cw")}
    _write_dispatches(d["f"], fetch)
    _write_dispatches(d["w"], write)
    _write_run(d["cf"], [(copy, "FETCH_SIZE", gib / 2)])
    _write_run(d["cw"], [(copy, "WRITE_SIZE", gib)])
    text = profsum.skip(d["f"], d["w"], d["cf"], d["cw"], [0, 1, 2], 2, 4096, "cmd")
    import json
    rec = json.loads(text.split("skip-json: ")[1])
    assert [r["tiles"] for r in rec] == [1, 2]
    assert rec[0]["gather_read"] == 100 * 1024 * 2 and rec[1]["gather_read"] == 200 * 1024 * 2
    assert rec[1]["product_write"] == 100 * 1024 and rec[0]["fixup_read"] == 10 * 1024 * 2
    assert rec[0]["product_read"] == 1000 * 1024 * 2
    assert "0 active tiles launched no kernel" in text


def test_units_valu_columns(tmp_path):
    k = "void (anonymous namespace)::k_fused_update<1024, 4>((anonymous namespace)::FusedParams)"
    a = str(tmp_path / "a")
    _write_run(a, [(k, "GRBM_GUI_ACTIVE", 8000.0), (k, "SQ_ACTIVE_INST_VALU", 1024 * 1000 * 0.3 / 4),
                   (k, "SQ_INSTS_VALU", 5000.0), (k, "SQ_WAVES", 10.0)])
    row = [ln for ln in profsum.units([[a]], ["upd"], "k_fused_update", "c").splitlines() if ln.startswith("upd")][0]
    assert row.split()[-2:] == ["0.300", "500"]


def test_overlap_counts_concurrent_time(tmp_path):
    # three kernels: [0, 10) and [5, 20) overlap for 5 us, [30, 35) alone;
    # another library's kernel is not counted
    path = str(tmp_path / "kt.csv")
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, (k, a, b) in enumerate([("void (anonymous namespace)::k_masked_dw<0>(x)", 0, 10000),
                                       ("(anonymous namespace)::k_fused_update<1024, 4>(y)", 5000, 20000),
                                       ("__amd_rocclr_copyBuffer", 30000, 35000),
                                       ("at::native::elementwise_kernel", 0, 99000)]):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Start_Timestamp": a, "End_Timestamp": b})
    text = profsum.overlap(path, "cmd")
    assert "dispatches: 3" in text
    assert "span from first start to last end: 35.0 us" in text
    assert "time with at least one kernel running: 25.0 us" in text
    assert "time with two or more running: 5.0 us (0.200 of the busy time)" in text
    assert "sum of the kernels' durations: 30.0 us (1.200 x the busy time)" in text
    # from dispatch 2 on: the first kernel is left out
    assert "time with two or more running: 0.0 us" in profsum.overlap(path, "cmd", first=2)

