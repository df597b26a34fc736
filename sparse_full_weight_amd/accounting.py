"""Algorithmic work of the sparse-first kernels, and the page's memory model.

Algorithmic bytes are the bytes a kernel must move at minimum (each input
byte read once, each output byte written once); dividing them by a measured
time gives the achieved bandwidth used for the roofline fraction.

Sources: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
Active Set", section 2.2 (dW = dY^T X restricted to active 32-row tiles),
section 2.3 (int8 q, fp32 residual, fp16 moments, sparse write-back) and
section 3 (training-state memory: a base cost per parameter plus a cost per
active parameter; for the page's engine 1 byte per parameter plus 4 + 2 + 2 + 4
bytes per active parameter).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Sequence, Tuple

BF16 = 2
F32 = 4


@dataclass
class Work:
    bytes: float
    flops_useful: float = 0.0
    flops_issued: float = 0.0


def masked_dw_work(groups: Sequence[Tuple[int, int, Sequence[Tuple[int, int]]]]) -> Work:
    """groups: (T, C, [(n_active_rows, n_active_tiles), ...]) per shared input X.

    Bytes: X once per group (T*C bf16), the dY columns of every active tile
    (T*32 bf16), and the fp32 dW rows of the active rows.  FLOPs: 2*T*C per
    active row (useful) and per row of every active tile (issued on the
    matrix cores)."""
    b = fu = fi = 0.0
    for T, C, mats in groups:
        if not any(nt for _, nt in mats):
            continue
        b += T * C * BF16
        for n_act, n_tiles in mats:
            b += n_tiles * T * 32 * BF16 + n_act * C * F32
            fu += 2.0 * T * C * n_act
            fi += 2.0 * T * C * 32 * n_tiles
    return Work(b, fu, fi)


# Per active element of the update: read g (4), q (1), delta (4), m (2), v (2);
# write q (1), delta (4), m (2), v (2); plus the bf16 live weight (2) when the
# write-back is fused.  Per active row: the scale s (read 4, write 4) and the
# two moment exponents of its slot (read 2, write 2).
UPDATE_BYTES_PER_ELEMENT = 4 + 1 + 4 + 2 + 2 + 1 + 4 + 2 + 2
WRITEBACK_BYTES_PER_ELEMENT = 2
UPDATE_BYTES_PER_ROW = 8 + 4


def update_work(mats: Iterable[Tuple[int, int]], fused_writeback: bool = True) -> Work:
    """mats: (C, n_active_rows) per matrix."""
    per = UPDATE_BYTES_PER_ELEMENT + (WRITEBACK_BYTES_PER_ELEMENT if fused_writeback else 0)
    b = 0.0
    for C, n in mats:
        b += n * C * per + n * UPDATE_BYTES_PER_ROW
    return Work(b)


def coupled_update_work(sides: Iterable[Tuple[int, int, int]]) -> Work:
    """sides: (C, n_active_rows, n_rows_also_listed_by_the_partner) per matrix
    of every pair.  Each listed row takes the update with fused write-back and
    reads its partner's gradient row where the partner lists the row too."""
    b = 0.0
    for C, n, n_shared in sides:
        b += n * C * (UPDATE_BYTES_PER_ELEMENT + WRITEBACK_BYTES_PER_ELEMENT) + n * UPDATE_BYTES_PER_ROW
        b += n_shared * C * F32
    return Work(b)


# Section 2.6 checkpoint of one row element: q (1), delta (4), m (2), v (2),
# read on one side and written on the other; a restore also writes the live
# bf16 weight (2).  Per row: s, the slot's step count and its two moment
# exponents, read and written.
CHECKPOINT_BYTES_PER_ELEMENT = 2 * (1 + 4 + 2 + 2)
CHECKPOINT_BYTES_PER_ROW = 2 * (4 + 4 + 2)


def checkpoint_work(mats: Iterable[Tuple[int, int]], restore: bool = False, live: bool = True) -> Work:
    """mats: (C, n_rows) per matrix; restore adds the rebuilt live rows."""
    per = CHECKPOINT_BYTES_PER_ELEMENT + (WRITEBACK_BYTES_PER_ELEMENT if restore and live else 0)
    return Work(sum(n * C * per + n * CHECKPOINT_BYTES_PER_ROW for C, n in mats))


def leaf_grad_work(T: int, mats: Iterable[Tuple[int, int, int]]) -> Work:
    """SparseLeaf connection gradients. mats: (distinct rows, distinct columns,
    K) per weight.  Bytes: the bf16 columns of D and X the support touches (T
    values each), the two int32 indices and the fp32 gradient per coordinate;
    FLOPs: 2*T per coordinate."""
    b = f = 0.0
    for n_rows, n_cols, K in mats:
        b += T * BF16 * (n_rows + n_cols) + K * (4 + 4 + F32)
        f += 2.0 * T * K
    return Work(b, f, f)


# SparseLeaf Adam per coordinate: read g, theta, m, v (fp32); write theta, m,
# v (fp32) and the bf16 copy of theta.
LEAF_ADAM_BYTES = 4 * F32 + 3 * F32 + BF16


def leaf_adam_work(K: int) -> Work:
    return Work(K * LEAF_ADAM_BYTES)


def embedding_dw_work(d: int, nnz: int, n_active: int) -> Work:
    """Reads the bf16 dY row of every hit position, writes fp32 rows."""
    return Work(nnz * d * BF16 + n_active * d * F32 + (nnz + n_active + 1) * 4)


def writeback_work(C: int, n_active: int) -> Work:
    """Reads q (1) and delta (4), writes bf16 (2) per element; s per row."""
    return Work(n_active * C * (1 + 4 + 2) + n_active * 4)


# Section 3 memory model: bytes = N * b_base + h * N * b_active.
HELIX_BASE = 1            # int8 weight
HELIX_ACTIVE = 4 + 2 + 2 + 4  # residual, two fp16 moments, fp32 gradient
FULL_FT_BASE = 2 + 4 + 8 + 2  # weight, master copy, moments, gradient
LORA_BASE = 2
LORA_ADAPTER_BYTES = 16


def state_bytes(n_params: float, active_share: float) -> Tuple[float, float]:
    """(base bytes, active bytes) of the sparse-first training state."""
    return n_params * HELIX_BASE, active_share * n_params * HELIX_ACTIVE


def full_ft_bytes(n_params: float) -> float:
    return n_params * FULL_FT_BASE


def lora_bytes(n_params: float, adapter_params: float) -> float:
    return n_params * LORA_BASE + adapter_params * LORA_ADAPTER_BYTES
