"""ctypes shim over the plain-C oracle (``oracle/sft_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark use this module to compute what the sparse-first step
must produce.  The GPU library never imports it, and it never imports the GPU
library.  Inputs and outputs are numpy arrays; bf16/fp16 tensors travel as
``uint16`` bit patterns.

Method source: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of
the Active Set", sections 2.1-2.4, and the blog post "SparseLeaf: synaptic
sparse fine-tuning" for the gradients and Adam step of K selected
connections (each C function names the passage it follows).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sft_oracle.c")
_LIB = os.path.join(_HERE, "libsft_oracle.so")

# gcc flags: IEEE binary32 with no contraction and no fast-math, so that every
# rounding the C source writes is the rounding that happens.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (always, when ``force``)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = C.CDLL(_LIB)
        _declare(_lib)
    return _lib


class OracleMat(C.Structure):
    _fields_ = [
        ("R", C.c_int64), ("C", C.c_int64), ("n_active", C.c_int64),
        ("active_rows", C.c_void_p), ("slot", C.c_void_p), ("fresh", C.c_void_p),
        ("G", C.c_void_p), ("q", C.c_void_p), ("s", C.c_void_p), ("delta", C.c_void_p),
        ("m", C.c_void_p), ("v", C.c_void_p), ("t", C.c_void_p), ("mv_exp", C.c_void_p),
        ("n_slots", C.c_int64), ("w_live", C.c_void_p),
    ]


class OracleAdam(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float),
                ("eps", C.c_float), ("weight_decay", C.c_float)]


def _declare(L: C.CDLL) -> None:
    p, i64, i32, f32 = C.c_void_p, C.c_int64, C.c_int32, C.c_float
    L.oracle_bf16_to_f32.argtypes = [C.c_uint16]; L.oracle_bf16_to_f32.restype = f32
    L.oracle_f16_to_f32.argtypes = [C.c_uint16]; L.oracle_f16_to_f32.restype = f32
    L.oracle_f32_to_f16.argtypes = [f32]; L.oracle_f32_to_f16.restype = C.c_uint16
    L.oracle_f32_to_bf16.argtypes = [f32]; L.oracle_f32_to_bf16.restype = C.c_uint16
    L.oracle_moment_exponent.argtypes = [f32]; L.oracle_moment_exponent.restype = C.c_int
    L.oracle_moment_encode.argtypes = [f32, C.c_int]; L.oracle_moment_encode.restype = C.c_uint16
    L.oracle_moment_decode.argtypes = [C.c_uint16, C.c_int]; L.oracle_moment_decode.restype = f32
    L.oracle_moment_encode_array.argtypes = [p, i64, C.c_int, p]; L.oracle_moment_encode_array.restype = None
    L.oracle_moment_decode_array.argtypes = [p, i64, C.c_int, p]; L.oracle_moment_decode_array.restype = None
    for n in ("oracle_f32_to_f16_array", "oracle_f32_to_bf16_array", "oracle_f16_to_f32_array",
              "oracle_bf16_to_f32_array"):
        getattr(L, n).argtypes = [p, i64, p]; getattr(L, n).restype = None
    L.oracle_conductor_window.argtypes = [p, i64, p, i64, p]; L.oracle_conductor_window.restype = C.c_int
    L.oracle_tracker_window.argtypes = [p, i64, p, p]; L.oracle_tracker_window.restype = C.c_int
    L.oracle_plan_rows.argtypes = [p, i64, p, p, p, p, p]; L.oracle_plan_rows.restype = None
    L.oracle_plan_embedding.argtypes = [p, i64, p, i64, p, p, p]; L.oracle_plan_embedding.restype = None
    L.oracle_slots_update.argtypes = [p, i64, i64, p, i64, p, p]; L.oracle_slots_update.restype = C.c_int
    L.oracle_masked_dw.argtypes = [p, i64, i64, p, i64, p, i64, p]; L.oracle_masked_dw.restype = None
    L.oracle_embedding_dw.argtypes = [p, i64, i64, p, p, i64, p]; L.oracle_embedding_dw.restype = None
    L.oracle_bias_table.argtypes = [f32, f32, i32, p, p]; L.oracle_bias_table.restype = None
    L.oracle_sparse_update.argtypes = [C.POINTER(OracleMat), C.POINTER(OracleAdam)]
    L.oracle_sparse_update.restype = C.c_int
    L.oracle_coupled_update.argtypes = [C.POINTER(OracleMat), C.POINTER(OracleMat), f32, f32, f32, f32,
                                        C.POINTER(OracleAdam)]
    L.oracle_coupled_update.restype = C.c_int
    L.oracle_masked_writeback.argtypes = [p, p, p, i64, i64, p, i64, p]
    L.oracle_masked_writeback.restype = None
    L.oracle_leaf_grad.argtypes = [p, p, i64, i64, i64, p, p, i64, p]
    L.oracle_leaf_grad.restype = None
    L.oracle_leaf_adam.argtypes = [i64, p, p, p, p, p, i32, f32, f32, f32, f32]
    L.oracle_leaf_adam.restype = None


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _arr(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


# ---------------------------------------------------------------- formats
def f32_to_f16(x) -> np.ndarray:
    x = _arr(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_f16_array(_ptr(x), x.size, _ptr(out))
    return out


def f32_to_bf16(x) -> np.ndarray:
    x = _arr(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_to_f32(h) -> np.ndarray:
    h = _arr(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = _arr(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_bf16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


# ---------------------------------------------------------------- scaled fp16 moments
def moment_exponent(amax: float) -> int:
    """The exponent a moment row with largest magnitude ``amax`` is stored with."""
    return int(lib().oracle_moment_exponent(float(amax)))


def moment_encode(x, e: int) -> np.ndarray:
    """fp16 bits of x * 2^e (round to nearest even, saturating)."""
    x = _arr(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_moment_encode_array(_ptr(x), x.size, int(e), _ptr(out))
    return out


def moment_decode(h, e: int) -> np.ndarray:
    """The fp32 values fp16(h) * 2^-e."""
    h = _arr(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_moment_decode_array(_ptr(h), h.size, int(e), _ptr(out))
    return out


# ---------------------------------------------------------------- section 2.1
def conductor_window(ch: np.ndarray, tokens) -> np.ndarray:
    """One observation window of the conductor; updates ``ch`` in place, returns the mask."""
    assert ch.dtype == np.float32 and ch.flags["C_CONTIGUOUS"]
    tokens = _arr(tokens, np.int32)
    active = np.zeros(ch.shape[0], np.uint8)
    rc = lib().oracle_conductor_window(_ptr(ch), ch.shape[0], _ptr(tokens), tokens.size, _ptr(active))
    if rc:
        raise ValueError(f"oracle_conductor_window: {rc}")
    return active


def tracker_window(ch: np.ndarray, magnitude) -> np.ndarray:
    assert ch.dtype == np.float32 and ch.flags["C_CONTIGUOUS"]
    magnitude = _arr(magnitude, np.float32)
    active = np.zeros(ch.shape[0], np.uint8)
    rc = lib().oracle_tracker_window(_ptr(ch), ch.shape[0], _ptr(magnitude), _ptr(active))
    if rc:
        raise ValueError(f"oracle_tracker_window: {rc}")
    return active


# ---------------------------------------------------------------- plans
def plan_rows(active) -> dict:
    active = _arr(active, np.uint8)
    rows = active.size
    tiles = (rows + 31) // 32
    bits = np.zeros(tiles, np.uint32)
    act = np.zeros(max(rows, 1), np.int32)
    at = np.zeros(max(tiles, 1), np.int32)
    na, nt = C.c_int64(), C.c_int64()
    lib().oracle_plan_rows(_ptr(active), rows, _ptr(bits), _ptr(act), C.byref(na), _ptr(at), C.byref(nt))
    return {"bits": bits, "active_rows": act[: na.value].copy(), "active_tiles": at[: nt.value].copy()}


def plan_embedding(active_rows, tokens):
    active_rows = _arr(active_rows, np.int32)
    tokens = _arr(tokens, np.int32)
    row_ptr = np.zeros(active_rows.size + 1, np.int32)
    pos = np.zeros(max(tokens.size, 1), np.int32)
    nnz = C.c_int64()
    lib().oracle_plan_embedding(_ptr(active_rows), active_rows.size, _ptr(tokens), tokens.size,
                                _ptr(row_ptr), _ptr(pos), C.byref(nnz))
    return row_ptr, pos[: nnz.value].copy()


def slots_update(row_slot: np.ndarray, n_slots: int, active_rows):
    assert row_slot.dtype == np.int32 and row_slot.flags["C_CONTIGUOUS"]
    active_rows = _arr(active_rows, np.int32)
    slot = np.zeros(max(active_rows.size, 1), np.int32)
    fresh = np.zeros(max(active_rows.size, 1), np.uint8)
    rc = lib().oracle_slots_update(_ptr(row_slot), row_slot.size, n_slots, _ptr(active_rows),
                                   active_rows.size, _ptr(slot), _ptr(fresh))
    if rc:
        raise ValueError(f"oracle_slots_update: {rc}")
    return slot[: active_rows.size].copy(), fresh[: active_rows.size].copy()


# ---------------------------------------------------------------- section 2.2
def masked_dw(dY_bits: np.ndarray, X_bits: np.ndarray, active_rows) -> np.ndarray:
    """dW rows of the active rows: fp64 sum over tokens, rounded once. Inputs are bf16 bits."""
    dY_bits = _arr(dY_bits, np.uint16)
    X_bits = _arr(X_bits, np.uint16)
    active_rows = _arr(active_rows, np.int32)
    T, R = dY_bits.shape
    T2, Cc = X_bits.shape
    assert T == T2
    out = np.zeros((active_rows.size, Cc), np.float32)
    lib().oracle_masked_dw(_ptr(dY_bits), T, R, _ptr(X_bits), Cc, _ptr(active_rows),
                           active_rows.size, _ptr(out))
    return out


def embedding_dw(dY_bits: np.ndarray, tokens, active_rows) -> np.ndarray:
    dY_bits = _arr(dY_bits, np.uint16)
    tokens = _arr(tokens, np.int32)
    active_rows = _arr(active_rows, np.int32)
    T, d = dY_bits.shape
    out = np.zeros((active_rows.size, d), np.float32)
    lib().oracle_embedding_dw(_ptr(dY_bits), T, d, _ptr(tokens), _ptr(active_rows),
                              active_rows.size, _ptr(out))
    return out


# ---------------------------------------------------------------- sections 2.3-2.4
def bias_table(beta1: float, beta2: float, t_max: int):
    bc1 = np.zeros(t_max + 1, np.float32)
    bc2 = np.zeros(t_max + 1, np.float32)
    lib().oracle_bias_table(beta1, beta2, t_max, _ptr(bc1), _ptr(bc2))
    return bc1, bc2


class MatState:
    """Host copy of one matrix's optimizer state (all numpy, updated in place).
    ``e`` holds each slot's moment exponents (int8 [n_slots, 2]: m's, v's);
    the stored fp16 value h of a moment stands for h * 2^-e."""

    def __init__(self, q, s, delta, m, v, t, w_live=None, e=None):
        self.q = _arr(q, np.int8)
        self.s = _arr(s, np.float32)
        self.delta = _arr(delta, np.float32)
        self.m = _arr(m, np.uint16)
        self.v = _arr(v, np.uint16)
        self.t = _arr(t, np.int32)
        self.w_live = None if w_live is None else _arr(w_live, np.uint16)
        self.e = np.zeros((self.m.shape[0], 2), np.int8) if e is None else _arr(e, np.int8).reshape(-1, 2)
        assert self.e.shape[0] == self.m.shape[0]

    def copy(self) -> "MatState":
        return MatState(self.q.copy(), self.s.copy(), self.delta.copy(), self.m.copy(),
                        self.v.copy(), self.t.copy(), None if self.w_live is None else self.w_live.copy(),
                        self.e.copy())

    def moments(self):
        """The fp32 moments the stored rows stand for (m, v), slot by slot."""
        m = np.stack([moment_decode(self.m[k], self.e[k, 0]) for k in range(self.m.shape[0])])
        v = np.stack([moment_decode(self.v[k], self.e[k, 1]) for k in range(self.v.shape[0])])
        return m.reshape(self.m.shape), v.reshape(self.v.shape)


def _mat(st: MatState, G, active_rows, slot, fresh, keep):
    R, Cc = st.q.shape
    active_rows = _arr(active_rows, np.int32)
    slot = _arr(slot, np.int32)
    fresh = None if fresh is None else _arr(fresh, np.uint8)
    G = _arr(G, np.float32).reshape(active_rows.size, Cc)
    keep.extend([active_rows, slot, fresh, G])
    return OracleMat(R, Cc, active_rows.size, _ptr(active_rows), _ptr(slot), _ptr(fresh), _ptr(G),
                     _ptr(st.q), _ptr(st.s), _ptr(st.delta), _ptr(st.m), _ptr(st.v), _ptr(st.t),
                     _ptr(st.e), st.m.shape[0], _ptr(st.w_live))


def sparse_update(st: MatState, G, active_rows, slot, fresh=None, *, lr, beta1, beta2, eps,
                  weight_decay=0.0) -> None:
    keep: list = []
    M = _mat(st, G, active_rows, slot, fresh, keep)
    hp = OracleAdam(lr, beta1, beta2, eps, weight_decay)
    rc = lib().oracle_sparse_update(C.byref(M), C.byref(hp))
    if rc:
        raise ValueError(f"oracle_sparse_update: {rc}")


def coupled_update(A: MatState, GA, rows_a, slot_a, fresh_a, B: MatState, GB, rows_b, slot_b,
                   fresh_b, *, a_own, a_cross, clip_a=1.0, clip_b=1.0, lr, beta1, beta2, eps,
                   weight_decay=0.0) -> None:
    keep: list = []
    MA = _mat(A, GA, rows_a, slot_a, fresh_a, keep)
    MB = _mat(B, GB, rows_b, slot_b, fresh_b, keep)
    hp = OracleAdam(lr, beta1, beta2, eps, weight_decay)
    rc = lib().oracle_coupled_update(C.byref(MA), C.byref(MB), a_own, a_cross, clip_a, clip_b,
                                     C.byref(hp))
    if rc:
        raise ValueError(f"oracle_coupled_update: {rc}")


def masked_writeback(q, s, delta, active_rows, w_live: np.ndarray) -> None:
    q = _arr(q, np.int8)
    s = _arr(s, np.float32)
    delta = _arr(delta, np.float32)
    active_rows = _arr(active_rows, np.int32)
    assert w_live.dtype == np.uint16 and w_live.flags["C_CONTIGUOUS"]
    R, Cc = q.shape
    lib().oracle_masked_writeback(_ptr(q), _ptr(s), _ptr(delta), R, Cc, _ptr(active_rows),
                                  active_rows.size, _ptr(w_live))


def leaf_grad(D_bits: np.ndarray, X_bits: np.ndarray, rows, cols) -> np.ndarray:
    """SparseLeaf connection gradients: g[k] = sum_t D[t, rows[k]] * X[t, cols[k]]
    (bf16 inputs as uint16 bits, fp64 sum, one rounding)."""
    D = _arr(D_bits, np.uint16)
    X = _arr(X_bits, np.uint16)
    rows = _arr(rows, np.int32)
    cols = _arr(cols, np.int32)
    T, m = D.shape
    assert X.shape[0] == T and rows.size == cols.size
    g = np.zeros(rows.size, np.float32)
    lib().oracle_leaf_grad(_ptr(D), _ptr(X), T, m, X.shape[1], _ptr(rows), _ptr(cols), rows.size, _ptr(g))
    return g


def leaf_adam(g, theta: np.ndarray, m: np.ndarray, v: np.ndarray, theta_bf16, step: int, *, lr, beta1, beta2,
              eps) -> None:
    """SparseLeaf Adam step on K coordinates (theta, m, v fp32, updated in place)."""
    g = _arr(g, np.float32)
    for a in (theta, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"] and a.size == g.size
    if theta_bf16 is not None:
        assert theta_bf16.dtype == np.uint16 and theta_bf16.size == g.size
    lib().oracle_leaf_adam(g.size, _ptr(g), _ptr(theta), _ptr(m), _ptr(v), _ptr(theta_bf16), step, lr, beta1,
                           beta2, eps)
