"""The byte accounting against the page's printed worked example (section 3,
tests/golden/memory_model.txt) and against hand-counted kernel traffic."""
import os

import pytest

from sparse_full_weight_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "memory_model.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (x.strip() for x in line.split("=", 1))
            vals[k] = float(v)
    return vals


def test_memory_model_matches_page_example():
    g = _golden()
    base, active = acc.state_bytes(g["n_params"], g["active_share"])
    assert base == pytest.approx(g["helix_base_bytes"])
    assert active == pytest.approx(g["helix_active_bytes"])
    full = acc.full_ft_bytes(g["n_params"])
    assert full == pytest.approx(g["full_ft_bytes"])
    assert full / (base + active) == pytest.approx(g["full_ft_over_helix"], rel=0.05)
    lora = acc.lora_bytes(g["n_params"], g["lora_adapter_params"])
    assert lora / (base + active) == pytest.approx(g["lora_over_helix"], rel=0.1)
    _, one_more = acc.state_bytes(g["n_params"], 0.01)
    assert one_more == pytest.approx(g["per_percent_bytes"])


def test_update_bytes_per_element():
    # 24 bytes per active element with the fused write-back, 22 without; per
    # row the scale (read + write 8) and the two moment exponents (read + write 4)
    assert acc.update_work([(1, 1)]).bytes == 24 + 12
    assert acc.update_work([(1, 1)], fused_writeback=False).bytes == 22 + 12


def test_masked_dw_work_llama_layer():
    T = 4096
    groups = [(T, 4096, [(41, 2)] * 3), (T, 4096, [(41, 2)]), (T, 4096, [(110, 4)] * 2),
              (T, 11008, [(41, 2)])]
    w = acc.masked_dw_work(groups)
    x = T * (3 * 4096 + 11008) * 2
    dy = 18 * T * 32 * 2
    dw = (41 * 4 * 4096 + 110 * 2 * 4096 + 41 * 11008) * 4
    assert w.bytes == x + dy + dw
    assert w.flops_useful == pytest.approx(16.58e9, rel=1e-3)
    assert w.flops_issued == pytest.approx(22.95e9, rel=1e-3)
    # a group with no active tile costs nothing (the tile skip)
    assert acc.masked_dw_work([(T, 4096, [(0, 0)])]).bytes == 0


def test_coupled_update_bytes():
    # one pair of 64-column matrices: 3 rows listed by a, 2 by b, 1 by both.
    # Per listed row element: read g 4, q 1, delta 4, m 2, v 2; write q 1,
    # delta 4, m 2, v 2, live bf16 2 (24 in all); per row s and the moment
    # exponents read + write (12); a shared row also reads the partner's fp32
    # gradient row.
    w = acc.coupled_update_work([(64, 3, 1), (64, 2, 1)])
    assert w.bytes == (3 + 2) * 64 * 24 + (3 + 2) * 12 + 2 * 64 * 4


def test_writeback_and_embedding_bytes():
    assert acc.writeback_work(16, 3).bytes == 3 * 16 * 7 + 3 * 4
    # 10 hit tokens of a 32-wide table into 4 rows: bf16 dY rows read, fp32
    # rows written, CSR (positions + row pointers) read
    assert acc.embedding_dw_work(32, 10, 4).bytes == 10 * 32 * 2 + 4 * 32 * 4 + (10 + 5) * 4


def test_checkpoint_bytes():
    # 3 rows of 16 columns: q 1 + delta 4 + m 2 + v 2 read and written per
    # element, s, t and the two moment exponents read and written per row; a
    # restore writes bf16 too
    assert acc.checkpoint_work([(16, 3)]).bytes == 3 * 16 * 18 + 3 * 20
    assert acc.checkpoint_work([(16, 3)], restore=True).bytes == 3 * 16 * 20 + 3 * 20
    assert acc.checkpoint_work([(16, 3)], restore=True, live=False).bytes == 3 * 16 * 18 + 3 * 20


def test_leaf_bytes():
    # 10 tokens, a support touching 3 rows and 5 columns with 7 coordinates:
    # 10 bf16 values per touched row of D and column of X, two int32 indices
    # and one fp32 gradient per coordinate
    w = acc.leaf_grad_work(10, [(3, 5, 7)])
    assert w.bytes == 10 * 2 * (3 + 5) + 7 * 12
    assert w.flops_useful == 2 * 10 * 7
    assert acc.leaf_adam_work(7).bytes == 7 * 30
