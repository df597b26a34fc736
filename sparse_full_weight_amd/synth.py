"""Seeded synthetic inputs for the sparse-first step (no method arithmetic here).

This module only draws random numbers and packs them into the storage formats
the step uses (bf16 bit patterns, int8, fp16 bit patterns).  It is the one
module that both the GPU library's callers and the CPU oracle's callers share:
the same seed gives the same bytes to both sides.

Workload shapes follow the page "Sparse-First Fine-Tuning: Full-Weight
Training at the Cost of the Active Set": row masks per projection (section
2.1), int8 weights with a per-row scale and an fp32 residual (section 2.3),
Llama-7B-shaped projections.  Value distributions:
  * activations X ~ N(0, 1) and output gradients dY ~ N(0, 0.01) read as a
    standard deviation of 0.01, both rounded to bf16 (round to nearest even);
  * q ~ U{-127..127}, s_r ~ U(1e-4, 1e-3), delta ~ U(-s_r/2, s_r/2);
  * mid-run moments m ~ N(0, 1e-3), v ~ U(1e-6, 1e-4) stored as fp16 rows
    scaled by a per-slot power of two (m by 2^em, em ~ U{8..12}; v by 2^ev,
    ev ~ U{16..22}), the exponents stored beside them;
  * embedding tokens from a Zipf(1.1) law bounded to the vocabulary.
Every generator takes an explicit integer seed (numpy PCG64).  Bulk tensors for
timing can also be drawn on the GPU with torch's seeded generator
(``normal_bf16_device``).
"""
from __future__ import annotations

import numpy as np

# Llama-7B projection shapes (rows = output features, cols = input features).
LLAMA7B = {
    "q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
    "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008),
}
# Matrices that read the same layer input X (q/k/v the attention input, gate/up
# the MLP input); o and down each read their own.
LLAMA7B_GROUPS = (("attn", ("q", "k", "v")), ("o", ("o",)), ("mlp", ("gate", "up")),
                  ("down", ("down",)))


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (storage packing only)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    g = rng(seed)
    return to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


def integer_bf16(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Small-integer values in [lo, hi], exactly representable in bf16."""
    g = rng(seed)
    return to_bf16_bits(g.integers(lo, hi + 1, size=shape).astype(np.float32))


def normal_bf16_device(shape, std: float, seed: int, device):
    """Bulk bf16 N(0, std) drawn on ``device`` with torch's seeded generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(0.0, 1.0, generator=gen)
    return (x * std).to(torch.bfloat16)


# ------------------------------------------------------------------ masks
def clustered_rows(R: int, k: int, seed: int) -> np.ndarray:
    """k hot rows packed into whole 32-row tiles (the last one partly filled),
    the tiles chosen at random: the clustered activity pattern of a projection."""
    if k <= 0:
        return np.zeros(0, np.int32)
    g = rng(seed)
    n_tiles = (R + 31) // 32
    need = (k + 31) // 32
    tiles = g.choice(n_tiles, size=need, replace=False)
    rows = []
    left = k
    for j in tiles:
        lo = 32 * int(j)
        hi = min(lo + 32, R)
        take = min(left, hi - lo)
        rows.extend(range(lo, lo + take))
        left -= take
    if left > 0:  # a ragged last tile could not hold its share: fill elsewhere
        free = np.setdiff1d(np.arange(R), np.array(rows, np.int64))
        rows.extend(g.choice(free, size=left, replace=False).tolist())
    return np.sort(np.array(rows, np.int32))


def one_per_tile_rows(R: int, seed: int) -> np.ndarray:
    """Exactly one hot row in every 32-row tile, at a seeded offset."""
    g = rng(seed)
    n_tiles = (R + 31) // 32
    rows = []
    for j in range(n_tiles):
        width = min(32, R - 32 * j)
        rows.append(32 * j + int(g.integers(0, width)))
    return np.array(rows, np.int32)


def tracker_magnitudes(R: int, hot_rows: np.ndarray, seed: int) -> np.ndarray:
    """Output magnitudes for one observation window: hot rows ~ U(0.1, 1] (the
    largest forced to 1), the rest ~ U(0, 0.019)."""
    g = rng(seed)
    a = g.uniform(0.0, 0.019, size=R).astype(np.float32)
    if hot_rows.size:
        a[hot_rows] = g.uniform(0.1, 1.0, size=hot_rows.size).astype(np.float32)
        a[hot_rows[g.integers(0, hot_rows.size)]] = 1.0
    return a


def zipf_tokens(n: int, vocab: int, s: float, seed: int) -> np.ndarray:
    """n token ids drawn from a Zipf(s) law over ranks 1..vocab (id = rank - 1)."""
    g = rng(seed)
    p = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return g.choice(vocab, size=n, p=p).astype(np.int32)


def mask_from_rows(R: int, rows: np.ndarray) -> np.ndarray:
    m = np.zeros(R, np.uint8)
    m[rows] = 1
    return m


# ------------------------------------------------------------------ state
def quant_state(R: int, C: int, seed: int):
    """int8 q, per-row scale s and residual delta of one matrix."""
    g = rng(seed)
    q = g.integers(-127, 128, size=(R, C), dtype=np.int64).astype(np.int8)
    s = g.uniform(1e-4, 1e-3, size=R).astype(np.float32)
    delta = (g.uniform(-0.5, 0.5, size=(R, C)).astype(np.float32) * s[:, None]).astype(np.float32)
    return q, s, delta


def moments(n_slots: int, C: int, seed: int, mid_run: bool):
    """Stored moments: fp16 bit patterns of m and v rows, per-slot step
    counts, and per-slot exponents e (int8 [n_slots, 2]); a stored value h
    stands for h * 2^-e of its row."""
    if not mid_run:
        return (np.zeros((n_slots, C), np.uint16), np.zeros((n_slots, C), np.uint16),
                np.zeros(n_slots, np.int32), np.zeros((n_slots, 2), np.int8))
    g = rng(seed)
    em = g.integers(8, 13, size=n_slots)
    ev = g.integers(16, 23, size=n_slots)
    m = to_f16_bits(g.standard_normal((n_slots, C), dtype=np.float32) * np.float32(1e-3)
                    * np.exp2(em).astype(np.float32)[:, None])
    v = to_f16_bits(g.uniform(1e-6, 1e-4, size=(n_slots, C)).astype(np.float32)
                    * np.exp2(ev).astype(np.float32)[:, None])
    t = np.full(n_slots, 6, np.int32)
    e = np.stack([em, ev], axis=1).astype(np.int8)
    return m, v, t, e


def gradient_rows(n: int, C: int, std: float, seed: int) -> np.ndarray:
    """fp32 gradient rows (for update-only checks that bypass the product)."""
    g = rng(seed)
    return (g.standard_normal((n, C), dtype=np.float32) * np.float32(std)).astype(np.float32)
