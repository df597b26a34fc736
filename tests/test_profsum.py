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
    assert row[1:] == ["1000", "0.500", "0.800", "0.100", "500", "-", "-"]


def test_units_missing_counters_print_dashes(tmp_path):
    k = "(anonymous namespace)::k_masked_dw((anonymous namespace)::DwParams)"
    a = str(tmp_path / "a")
    _write_run(a, [(k, "GRBM_GUI_ACTIVE", 8000.0)])
    row = [ln for ln in profsum.units([[a]], ["x"], "k_masked_dw", "c").splitlines() if ln.startswith("x")][0]
    assert row.split()[1:] == ["1000", "-", "-", "-", "-", "-", "-"]


def test_units_lds_columns(tmp_path):
    k = "void (anonymous namespace)::k_leaf_grad<28>((anonymous namespace)::LeafParams)"
    a = str(tmp_path / "a")
    _write_run(a, [(k, "GRBM_GUI_ACTIVE", 8000.0), (k, "SQ_LDS_IDX_ACTIVE", 256 * 1000 * 0.4),
                   (k, "SQ_LDS_BANK_CONFLICT", 300.0), (k, "SQ_INSTS_LDS", 100.0)])
    row = [ln for ln in profsum.units([[a]], ["leaf"], "k_leaf_grad", "c").splitlines() if ln.startswith("leaf")][0]
    assert row.split()[-2:] == ["0.400", "3.00"]
