"""ctypes binding of ``libsft.so`` (the C ABI declared in ``include/sft.h``).

Argument marshalling only: host calls take numpy arrays, device calls take
torch tensors that live on the GPU and enqueue on torch's current stream.
Every step of the computation runs in the library; there is no Python or CPU
fallback -- if the library is missing the import of this module's ``lib()``
fails loudly.

Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
Active Set" (sections 2.1-2.4); each function's C declaration states the
passage it implements.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsft.so")

SFT_OK, SFT_EINVAL, SFT_ESHAPE, SFT_EALIGN, SFT_ECAPACITY, SFT_EHIP, SFT_ENOTSUP = 0, -1, -2, -3, -4, -5, -6
_CODES = {SFT_EINVAL: "EINVAL", SFT_ESHAPE: "ESHAPE", SFT_EALIGN: "EALIGN", SFT_ECAPACITY: "ECAPACITY",
          SFT_EHIP: "EHIP", SFT_ENOTSUP: "ENOTSUP"}

# Every symbol include/sft.h declares (checked by the test-suite).
EXPORTS = (
    "sft_last_error", "sft_abi_version", "sft_conductor_window", "sft_tracker_window", "sft_plan_rows",
    "sft_plan_embedding", "sft_slots_update", "sft_bias_table", "sft_masked_dw_workspace", "sft_masked_dw",
    "sft_embedding_dw", "sft_sparse_update", "sft_coupled_update", "sft_masked_writeback", "sft_masked_dw_update",
    "sft_masked_writeback_many",
    "sft_rewind_init", "sft_rewind_observe", "sft_rows_save", "sft_rows_restore",
    "sft_leaf_grad_workspace", "sft_leaf_grad", "sft_leaf_adam", "sft_helix_init", "sft_helix_step",
    "sft_helix_coupling", "sft_probe_grid", "sft_probe_read", "sft_probe_copy", "sft_probe_mfma", "sft_probe_dw_plan",
    "sft_noalloc_scratch_bytes", "sft_masked_dw_update_noalloc", "sft_plan_layer_words", "sft_plan_layer",
    "sft_plan_upload",
)


class SftError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODES.get(code, code)}: {msg}")
        self.code = code


# ------------------------------------------------------------------ C structs
class CPlan(C.Structure):
    _fields_ = [("rows", C.c_int64), ("n_active", C.c_int64), ("n_active_tiles", C.c_int64),
                ("tile_bits", C.c_void_p), ("active_rows", C.c_void_p), ("active_tiles", C.c_void_p),
                ("active_bits", C.c_void_p), ("tile_first", C.c_void_p)]


class CLayerMat(C.Structure):
    _fields_ = [("rows", C.c_int64), ("n_slots", C.c_int64), ("charge", C.c_void_p), ("magnitude", C.c_void_p),
                ("row_slot", C.c_void_p), ("n_active", C.c_int64), ("n_active_tiles", C.c_int64),
                ("off_rows", C.c_int64), ("off_tiles", C.c_int64), ("off_bits", C.c_int64),
                ("off_first", C.c_int64), ("off_slot", C.c_int64), ("off_fresh", C.c_int64)]


class CDwMat(C.Structure):
    _fields_ = [("dY", C.c_void_p), ("R", C.c_int64), ("active_rows", C.c_void_p), ("active_tiles", C.c_void_p),
                ("active_bits", C.c_void_p), ("tile_first", C.c_void_p), ("n_active", C.c_int64),
                ("n_active_tiles", C.c_int64), ("dW_act", C.c_void_p)]


SFT_DW_TILES = 0    # whole active 32-row tiles on the matrix cores, inactive rows dropped at the store
SFT_DW_PACKED = 1   # active rows packed 32 to a tile before the product


class CDwGroup(C.Structure):
    _fields_ = [("X", C.c_void_p), ("T", C.c_int64), ("C", C.c_int64), ("n_mats", C.c_int32),
                ("layout", C.c_int32), ("mats", C.POINTER(CDwMat))]


class CAdam(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("bc1", C.c_void_p), ("bc2", C.c_void_p), ("t_max", C.c_int32)]


class CUpdMat(C.Structure):
    _fields_ = [("R", C.c_int64), ("C", C.c_int64), ("n_active", C.c_int64), ("n_slots", C.c_int64),
                ("active_rows", C.c_void_p), ("slot", C.c_void_p), ("fresh", C.c_void_p), ("G", C.c_void_p),
                ("q", C.c_void_p), ("s", C.c_void_p), ("delta", C.c_void_p), ("m", C.c_void_p),
                ("v", C.c_void_p), ("t", C.c_void_p), ("mv_exp", C.c_void_p), ("w_live", C.c_void_p)]


class CWbMat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("delta", C.c_void_p), ("R", C.c_int64), ("C", C.c_int64),
                ("active_rows", C.c_void_p), ("n_active", C.c_int64), ("w_live", C.c_void_p)]


class CPair(C.Structure):
    _fields_ = [("a", CUpdMat), ("b", CUpdMat), ("a_own", C.c_float), ("a_cross", C.c_float),
                ("clip", C.c_void_p)]


class CRewind(C.Structure):
    _fields_ = [("save_within", C.c_double), ("rise_above", C.c_double), ("watch_steps", C.c_int32),
                ("max_recoveries", C.c_int32), ("has_checkpoint", C.c_int32), ("watch_left", C.c_int32),
                ("recoveries", C.c_int32), ("reserved", C.c_int32), ("checkpoint_loss", C.c_double),
                ("min_loss", C.c_double), ("step", C.c_int64), ("checkpoint_step", C.c_int64),
                ("min_step", C.c_int64)]


class CCkptMat(C.Structure):
    _fields_ = [("R", C.c_int64), ("C", C.c_int64), ("n_rows", C.c_int64), ("n_slots", C.c_int64),
                ("rows", C.c_void_p), ("slot", C.c_void_p), ("q", C.c_void_p), ("s", C.c_void_p),
                ("delta", C.c_void_p), ("m", C.c_void_p), ("v", C.c_void_p), ("t", C.c_void_p),
                ("mv_exp", C.c_void_p), ("w_live", C.c_void_p), ("ck_q", C.c_void_p), ("ck_s", C.c_void_p),
                ("ck_delta", C.c_void_p), ("ck_m", C.c_void_p), ("ck_v", C.c_void_p), ("ck_t", C.c_void_p),
                ("ck_mv_exp", C.c_void_p)]


class CHelix(C.Structure):
    _fields_ = [(n, C.c_double) for n in ("decay_len", "up_threshold", "rung_deg", "M", "mu", "mod_plus",
                                          "mod_minus", "trend_sum", "trend_w", "smooth_sum", "smooth_w",
                                          "last_loss", "rotation")] + [("has_loss", C.c_int32), ("rung", C.c_int32)]


class CLeafMat(C.Structure):
    _fields_ = [("dY", C.c_void_p), ("X", C.c_void_p), ("m", C.c_int64), ("n", C.c_int64), ("K", C.c_int64),
                ("rows", C.c_void_p), ("cols", C.c_void_p), ("grad", C.c_void_p)]


class CLeafVec(C.Structure):
    _fields_ = [("K", C.c_int64), ("grad", C.c_void_p), ("theta", C.c_void_p), ("m", C.c_void_p),
                ("v", C.c_void_p), ("theta_bf16", C.c_void_p)]


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -c \"import __graft_entry__ as g; "
                              f"g.build()\"` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        p, i64, i32, f32 = C.c_void_p, C.c_int64, C.c_int32, C.c_float
        L.sft_last_error.restype = C.c_char_p
        L.sft_last_error.argtypes = []
        L.sft_abi_version.restype = C.c_int
        L.sft_conductor_window.argtypes = [p, i64, p, i64, p]
        L.sft_tracker_window.argtypes = [p, i64, p, p]
        L.sft_plan_rows.argtypes = [p, C.POINTER(CPlan)]
        L.sft_plan_embedding.argtypes = [C.POINTER(CPlan), p, i64, p, p, i64, C.POINTER(C.c_int64)]
        L.sft_slots_update.argtypes = [p, i64, i64, p, i64, p, p]
        L.sft_plan_layer_words.argtypes = [C.POINTER(CLayerMat), i32]
        L.sft_plan_layer_words.restype = i64
        L.sft_plan_layer.argtypes = [C.POINTER(CLayerMat), i32, p, i64, C.POINTER(C.c_int64)]
        L.sft_bias_table.argtypes = [f32, f32, i32, p, p]
        L.sft_plan_upload.argtypes = [p, p, C.c_size_t, p]
        L.sft_masked_dw_workspace.argtypes = [C.POINTER(CDwGroup), i32]
        L.sft_masked_dw_workspace.restype = C.c_size_t
        L.sft_masked_dw.argtypes = [C.POINTER(CDwGroup), i32, p, C.c_size_t, p]
        L.sft_embedding_dw.argtypes = [p, i64, i64, p, p, i64, p, p]
        L.sft_sparse_update.argtypes = [C.POINTER(CUpdMat), i32, C.POINTER(CAdam), p]
        L.sft_coupled_update.argtypes = [C.POINTER(CPair), i32, C.POINTER(CAdam), p]
        L.sft_masked_dw_update.argtypes = [C.POINTER(CDwGroup), i32, p, C.c_size_t, C.POINTER(CUpdMat), i32,
                                           C.POINTER(CAdam), p]
        L.sft_masked_dw_update_noalloc.argtypes = [C.POINTER(CDwGroup), i32, C.POINTER(CUpdMat), i32,
                                                    C.POINTER(CAdam), p]
        L.sft_noalloc_scratch_bytes.argtypes = []
        L.sft_noalloc_scratch_bytes.restype = C.c_size_t
        L.sft_masked_writeback.argtypes = [p, p, p, i64, i64, p, i64, p, p]
        L.sft_masked_writeback_many.argtypes = [C.POINTER(CWbMat), i32, p]
        L.sft_rewind_init.argtypes = [C.POINTER(CRewind)]
        L.sft_rewind_observe.argtypes = [C.POINTER(CRewind), C.c_double, C.POINTER(C.c_int32)]
        L.sft_rows_save.argtypes = [C.POINTER(CCkptMat), i32, p]
        L.sft_rows_restore.argtypes = [C.POINTER(CCkptMat), i32, p]
        L.sft_leaf_grad_workspace.argtypes = [C.POINTER(CLeafMat), i32, i64]
        L.sft_leaf_grad_workspace.restype = C.c_size_t
        L.sft_leaf_grad.argtypes = [C.POINTER(CLeafMat), i32, i64, p, C.c_size_t, p]
        L.sft_leaf_adam.argtypes = [C.POINTER(CLeafVec), i32, i32, C.POINTER(CAdam), p]
        L.sft_probe_grid.argtypes = []
        L.sft_probe_read.argtypes = [p, C.c_size_t, p, p]
        L.sft_probe_copy.argtypes = [p, p, C.c_size_t, p]
        L.sft_probe_mfma.argtypes = [i64, p, p]
        L.sft_probe_dw_plan.argtypes = [C.POINTER(CDwGroup), i32, i32, p, i32]
        L.sft_helix_init.argtypes = [C.POINTER(CHelix)]
        L.sft_helix_step.argtypes = [C.POINTER(CHelix), C.c_double, i32, C.POINTER(C.c_int32),
                                     C.POINTER(C.c_double)]
        L.sft_helix_coupling.argtypes = [C.POINTER(CHelix), C.c_double, C.c_double, C.POINTER(C.c_double),
                                         C.POINTER(C.c_double)]
        for n in EXPORTS[2:]:
            if n not in ("sft_masked_dw_workspace", "sft_leaf_grad_workspace", "sft_noalloc_scratch_bytes"):
                getattr(L, n).restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != SFT_OK:
        raise SftError(rc, lib().sft_last_error().decode())


def _np_ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "host arrays must be C-contiguous"
    return a.ctypes.data


def _dev(t, dtype=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError("device argument must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _shape(t, want, what):
    """Raise unless tensor ``t`` has shape ``want`` (entries None match any size)."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        raise ValueError(f"{what}: shape {got}, expected {tuple('*' if w is None else w for w in want)}")


def _numel_at_least(t, n, what):
    if t.numel() < n:
        raise ValueError(f"{what}: {t.numel()} elements, need at least {n}")


def _is16(t) -> bool:
    import torch
    return t.dtype in (torch.int16, torch.uint16, torch.float16, torch.bfloat16)


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------------------ host calls
def sft_abi_version() -> int:
    return lib().sft_abi_version()


def sft_conductor_window(ch: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """Section 2.1 conductor: updates ``ch`` (fp32) in place, returns the u8 mask."""
    assert ch.dtype == np.float32
    tokens = np.ascontiguousarray(tokens, np.int32)
    active = np.zeros(ch.size, np.uint8)
    _check(lib().sft_conductor_window(_np_ptr(ch), ch.size, _np_ptr(tokens), tokens.size, _np_ptr(active)))
    return active


def sft_tracker_window(ch: np.ndarray, magnitude: np.ndarray) -> np.ndarray:
    """Section 2.1 row tracker over output magnitudes."""
    assert ch.dtype == np.float32
    magnitude = np.ascontiguousarray(magnitude, np.float32)
    active = np.zeros(ch.size, np.uint8)
    _check(lib().sft_tracker_window(_np_ptr(ch), ch.size, _np_ptr(magnitude), _np_ptr(active)))
    return active


@dataclass
class Plan:
    """Host row plan of one mask (tile bitmap, active rows, active tiles and,
    per active tile, its row bits and the index of its first active row)."""
    rows: int
    tile_bits: np.ndarray
    active_rows: np.ndarray
    active_tiles: np.ndarray
    active_bits: np.ndarray
    tile_first: np.ndarray

    @property
    def n_active(self) -> int:
        return int(self.active_rows.size)

    @property
    def n_active_tiles(self) -> int:
        return int(self.active_tiles.size)

    def to_device(self, device="cuda") -> "DevicePlan":
        import torch
        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device, non_blocking=False)
        return DevicePlan(self, up(self.active_rows), up(self.active_tiles), up(self.active_bits),
                          up(self.tile_first))


@dataclass
class DevicePlan:
    host: Plan
    active_rows: "object"
    active_tiles: "object"
    active_bits: "object"
    tile_first: "object"

    @property
    def rows(self) -> int:
        return self.host.rows

    @property
    def n_active(self) -> int:
        return self.host.n_active

    @property
    def n_active_tiles(self) -> int:
        return self.host.n_active_tiles


def sft_plan_rows(mask: np.ndarray) -> Plan:
    mask = np.ascontiguousarray(mask, np.uint8)
    rows = mask.size
    tiles = (rows + 31) // 32
    bits = np.zeros(max(tiles, 1), np.uint32)
    act = np.zeros(max(rows, 1), np.int32)
    at = np.zeros(max(tiles, 1), np.int32)
    ab = np.zeros(max(tiles, 1), np.uint32)
    tf = np.zeros(max(tiles, 1), np.int32)
    cp = CPlan(rows, 0, 0, _np_ptr(bits), _np_ptr(act), _np_ptr(at), _np_ptr(ab), _np_ptr(tf))
    _check(lib().sft_plan_rows(_np_ptr(mask), C.byref(cp)))
    nt = cp.n_active_tiles
    return Plan(rows, bits[:tiles].copy(), act[:cp.n_active].copy(), at[:nt].copy(), ab[:nt].copy(), tf[:nt].copy())


def sft_plan_embedding(plan: Plan, tokens: np.ndarray):
    """CSR (row_ptr, positions) of the active embedding rows' token positions."""
    tokens = np.ascontiguousarray(tokens, np.int32)
    cp = CPlan(plan.rows, plan.n_active, plan.n_active_tiles, _np_ptr(plan.tile_bits),
               _np_ptr(plan.active_rows), _np_ptr(plan.active_tiles), _np_ptr(plan.active_bits),
               _np_ptr(plan.tile_first))
    row_ptr = np.zeros(plan.n_active + 1, np.int32)
    pos = np.zeros(max(tokens.size, 1), np.int32)
    nnz = C.c_int64()
    _check(lib().sft_plan_embedding(C.byref(cp), _np_ptr(tokens), tokens.size, _np_ptr(row_ptr), _np_ptr(pos),
                                    pos.size, C.byref(nnz)))
    return row_ptr, pos[:nnz.value].copy()


def sft_slots_update(row_slot: np.ndarray, n_slots: int, active_rows: np.ndarray):
    assert row_slot.dtype == np.int32 and row_slot.flags["C_CONTIGUOUS"]
    active_rows = np.ascontiguousarray(active_rows, np.int32)
    slot = np.zeros(max(active_rows.size, 1), np.int32)
    fresh = np.zeros(max(active_rows.size, 1), np.uint8)
    _check(lib().sft_slots_update(_np_ptr(row_slot), row_slot.size, n_slots, _np_ptr(active_rows),
                                  active_rows.size, _np_ptr(slot), _np_ptr(fresh)))
    return slot[:active_rows.size].copy(), fresh[:active_rows.size].copy()


def sft_plan_upload(dst, src, nbytes: int | None = None, stream=None) -> None:
    """Section 2.6 / Figure 2: the first nbytes (default: all of src) of a
    pinned host tensor src copied to the GPU tensor dst by a kernel on the
    stream (asynchronous; src must stay unchanged until the stream has
    passed the call)."""
    if src.is_cuda or not src.is_pinned():
        raise TypeError("src must be a pinned host tensor")
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size() or n > dst.numel() * dst.element_size():
        raise ValueError(f"{n} bytes exceed src or dst")
    _check(lib().sft_plan_upload(_dev(dst), src.data_ptr(), n, _stream(stream)))


@dataclass
class LayerMatPlan:
    """One matrix's part of a layer plan: counts, and the word offsets of its
    sections in the packed buffer."""
    n_active: int
    n_active_tiles: int
    off: dict


class LayerPlanner:
    """sft_plan_layer over a fixed list of matrices: holds each matrix's
    tracker charge and row -> slot map across steps, and the packed host
    buffer the plans are written to (a numpy array, or the address and word
    capacity of a caller's buffer, such as pinned memory)."""

    SECTIONS = ("rows", "tiles", "bits", "first", "slot", "fresh")

    def __init__(self, rows, n_slots, packed_ptr: int | None = None, packed_words: int | None = None):
        self.n = len(rows)
        assert len(n_slots) == self.n
        self.charge = [np.zeros(int(R), np.float32) for R in rows]
        self.row_slot = [np.full(int(R), -1, np.int32) for R in rows]
        self.c = (CLayerMat * max(self.n, 1))()
        for i, R in enumerate(rows):
            self.c[i].rows = int(R)
            self.c[i].n_slots = int(n_slots[i])
            self.c[i].charge = _np_ptr(self.charge[i])
            self.c[i].row_slot = _np_ptr(self.row_slot[i])
        self.words = int(lib().sft_plan_layer_words(self.c, self.n))
        if self.words < 0:
            raise ValueError("sft_plan_layer_words: bad matrix list")
        if packed_ptr is None:
            buf = np.zeros(self.words + 8, np.int32)      # 16-byte aligned view below
            start = (-buf.ctypes.data % 16) // 4
            self.packed = buf[start:start + max(self.words, 1)]
            self._ptr, self._cap = self.packed.ctypes.data, self.words
        else:
            if packed_words is None or packed_words < self.words:
                raise ValueError(f"packed buffer holds {packed_words} words, {self.words} needed")
            self.packed = None
            self._ptr, self._cap = int(packed_ptr), int(packed_words)
        self._mags = [None] * self.n
        self.length = 0

    def bind(self, magnitudes) -> None:
        """Point the matrices at their magnitude arrays (float32, one per
        matrix, kept alive here); a loop that refills them in place binds
        once and calls step()."""
        assert len(magnitudes) == self.n
        for i, mag in enumerate(magnitudes):
            mag = np.ascontiguousarray(mag, np.float32)
            if mag.shape != (self.c[i].rows,):
                raise ValueError(f"magnitudes[{i}] has shape {mag.shape}, want ({self.c[i].rows},)")
            self._mags[i] = mag
            self.c[i].magnitude = _np_ptr(mag)
        self._bound = True

    def step(self) -> int:
        """One sft_plan_layer call over the bound magnitudes; returns the
        words written."""
        if not getattr(self, "_bound", False):
            raise ValueError("LayerPlanner.step: bind() the magnitudes first")
        n = C.c_int64()
        _check(lib().sft_plan_layer(self.c, self.n, self._ptr, self._cap, C.byref(n)))
        self.length = int(n.value)
        return self.length

    def results(self) -> list[LayerMatPlan]:
        return [LayerMatPlan(self.c[i].n_active, self.c[i].n_active_tiles,
                             {k: getattr(self.c[i], "off_" + k) for k in self.SECTIONS}) for i in range(self.n)]

    def plan(self, magnitudes) -> list[LayerMatPlan]:
        """One step: the tracker window of every matrix over `magnitudes`,
        its row plan and moment slots, written into the packed buffer."""
        self.bind(magnitudes)
        self.step()
        return self.results()

    def section(self, mp: LayerMatPlan, name: str) -> np.ndarray:
        """A matrix's section of the numpy packed buffer (rows, tiles, bits,
        first, slot as int32; fresh as uint8)."""
        assert self.packed is not None
        o = mp.off[name]
        if name == "fresh":
            return self.packed[o:o + (mp.n_active + 3) // 4].view(np.uint8)[:mp.n_active]
        n = mp.n_active if name in ("rows", "slot") else mp.n_active_tiles
        a = self.packed[o:o + n]
        return a.view(np.uint32) if name == "bits" else a


def sft_bias_table(beta1: float, beta2: float, t_max: int):
    bc1 = np.zeros(t_max + 1, np.float32)
    bc2 = np.zeros(t_max + 1, np.float32)
    _check(lib().sft_bias_table(beta1, beta2, t_max, _np_ptr(bc1), _np_ptr(bc2)))
    return bc1, bc2


# ------------------------------------------------------------------ device calls
@dataclass
class DwMat:
    dY: "object"            # bf16 [T x R] GPU tensor
    plan: DevicePlan
    dW_act: "object"        # fp32 [n_active x C]


@dataclass
class DwGroup:
    X: "object"             # bf16 [T x C] GPU tensor
    mats: Sequence[DwMat]
    layout: int = SFT_DW_PACKED


def _c_groups(groups: Sequence[DwGroup]):
    import torch
    keep = []
    arr = (CDwGroup * max(len(groups), 1))()
    for i, g in enumerate(groups):
        T, Cc = g.X.shape
        mats = (CDwMat * max(len(g.mats), 1))()
        for j, m in enumerate(g.mats):
            _shape(m.dY, (T, m.plan.rows), f"group {i} matrix {j} dY")
            if m.plan.n_active:
                _shape(m.dW_act, (None, Cc), f"group {i} matrix {j} dW_act")
                _numel_at_least(m.dW_act, m.plan.n_active * Cc, f"group {i} matrix {j} dW_act")
            mats[j] = CDwMat(_dev(m.dY, torch.bfloat16), m.plan.rows, _dev(m.plan.active_rows),
                             _dev(m.plan.active_tiles), _dev(m.plan.active_bits), _dev(m.plan.tile_first),
                             m.plan.n_active, m.plan.n_active_tiles, _dev(m.dW_act, torch.float32))
        keep.append(mats)
        arr[i] = CDwGroup(_dev(g.X, torch.bfloat16), T, Cc, len(g.mats), g.layout, mats)
    return arr, keep


def sft_masked_dw_workspace(groups: Sequence[DwGroup]) -> int:
    arr, keep = _c_groups(groups)
    n = lib().sft_masked_dw_workspace(arr, len(groups))
    if n == C.c_size_t(-1).value:
        raise SftError(SFT_EINVAL, lib().sft_last_error().decode())
    return n


def sft_masked_dw(groups: Sequence[DwGroup], ws=None, stream=None) -> None:
    """Section 2.2 masked dW for every matrix of every group (async on the stream)."""
    arr, keep = _c_groups(groups)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sft_masked_dw(arr, len(groups), _dev(ws), nbytes, _stream(stream)))


def sft_embedding_dw(dY, row_ptr, positions, n_active: int, dW_act, stream=None) -> None:
    import torch
    T, d = dY.shape
    _check(lib().sft_embedding_dw(_dev(dY, torch.bfloat16), T, d, _dev(row_ptr, torch.int32),
                                  _dev(positions, torch.int32), n_active, _dev(dW_act, torch.float32),
                                  _stream(stream)))


@dataclass
class Adam:
    lr: float
    beta1: float
    beta2: float
    eps: float
    bc1: "object"           # fp32 GPU tensor [t_max + 1]
    bc2: "object"
    weight_decay: float = 0.0

    def c(self) -> CAdam:
        return CAdam(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, _dev(self.bc1),
                     _dev(self.bc2), self.bc1.numel() - 1)


@dataclass
class UpdMat:
    """One matrix's GPU state plus the gradient of its active rows."""
    q: "object"             # int8 [R x C]
    s: "object"             # fp32 [R]
    delta: "object"         # fp32 [R x C]
    m: "object"             # fp16 bits (int16/uint16 tensor) [n_slots x C]
    v: "object"
    t: "object"             # int32 [n_slots]
    mv_exp: "object"        # int8 [n_slots x 2]: exponents of the slot's m row and v row
    active_rows: "object"   # int32 [n_active] (GPU)
    slot: "object"          # int32 [n_active] (GPU)
    G: "object"             # fp32 [n_active x C]
    n_active: int
    fresh: "object" = None  # uint8 [n_active] (GPU) or None
    w_live: "object" = None  # bf16 [R x C] or None

    def c(self) -> CUpdMat:
        """The C struct, after checking every tensor's dtype and shape (the
        kernels trust the sizes: a wrong one would read or write out of
        bounds on the GPU)."""
        import torch
        _shape(self.q, (None, None), "q")
        R, Cc = self.q.shape
        n_slots = self.m.shape[0]
        n = int(self.n_active)
        _shape(self.s, (R,), "s")
        _shape(self.delta, (R, Cc), "delta")
        _shape(self.m, (n_slots, Cc), "m")
        _shape(self.v, (n_slots, Cc), "v")
        _shape(self.t, (n_slots,), "t")
        _shape(self.mv_exp, (n_slots, 2), "mv_exp")
        if not (_is16(self.m) and _is16(self.v)):
            raise TypeError("m and v must be 16-bit tensors (fp16 bit patterns)")
        _shape(self.G, (None, Cc), "G")
        for t_, what in ((self.active_rows, "active_rows"), (self.slot, "slot")):
            _numel_at_least(t_, n, what)
        _numel_at_least(self.G, n * Cc, "G")
        if self.fresh is not None:
            _numel_at_least(self.fresh, n, "fresh")
        if self.w_live is not None:
            _shape(self.w_live, (R, Cc), "w_live")
            if not _is16(self.w_live):
                raise TypeError("w_live must be a 16-bit tensor (bf16 bit patterns)")
        return CUpdMat(R, Cc, n, n_slots, _dev(self.active_rows, torch.int32), _dev(self.slot, torch.int32),
                       _dev(self.fresh, torch.uint8), _dev(self.G, torch.float32), _dev(self.q, torch.int8),
                       _dev(self.s, torch.float32), _dev(self.delta, torch.float32), _dev(self.m), _dev(self.v),
                       _dev(self.t, torch.int32), _dev(self.mv_exp, torch.int8), _dev(self.w_live))


def sft_sparse_update(mats: Sequence[UpdMat], hp: Adam, stream=None) -> None:
    """Sections 2.3-2.4 plain sparse update (+ fused write-back where w_live is set)."""
    arr = (CUpdMat * max(len(mats), 1))(*[m.c() for m in mats])
    h = hp.c()
    _check(lib().sft_sparse_update(arr, len(mats), C.byref(h), _stream(stream)))


def sft_masked_dw_update(groups: Sequence[DwGroup], ws, mats: Sequence[UpdMat], hp: Adam, stream=None) -> None:
    """Masked dW with the update of every matrix fused in (the split tiles' fix-up
    is done by the update); mats follow the groups' matrices in order, each
    with G = that matrix's dW_act."""
    arr, keep = _c_groups(groups)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    u = (CUpdMat * max(len(mats), 1))(*[m.c() for m in mats])
    h = hp.c()
    _check(lib().sft_masked_dw_update(arr, len(groups), _dev(ws), nbytes, u, len(mats), C.byref(h),
                                      _stream(stream)))


def sft_masked_dw_update_noalloc(groups: Sequence[DwGroup], mats: Sequence[UpdMat], hp: Adam, stream=None) -> None:
    """sft_masked_dw_update with the library's per-device scratch array as the
    workspace: the call allocates nothing (calls overlapping on one device race)."""
    arr, keep = _c_groups(groups)
    ua = (CUpdMat * max(len(mats), 1))(*[m.c() for m in mats])
    h = hp.c()
    _check(lib().sft_masked_dw_update_noalloc(arr, len(groups), ua, len(mats), C.byref(h), _stream(stream)))


def sft_noalloc_scratch_bytes() -> int:
    return lib().sft_noalloc_scratch_bytes()


@dataclass
class Pair:
    a: UpdMat
    b: UpdMat
    a_own: float
    a_cross: float
    clip: "object" = None   # fp32 GPU tensor [2] or None


def sft_coupled_update(pairs: Sequence[Pair], hp: Adam, stream=None) -> None:
    """Section 2.4 coupled update of matrix pairs."""
    arr = (CPair * max(len(pairs), 1))(*[CPair(p.a.c(), p.b.c(), p.a_own, p.a_cross, _dev(p.clip))
                                         for p in pairs])
    h = hp.c()
    _check(lib().sft_coupled_update(arr, len(pairs), C.byref(h), _stream(stream)))


def sft_masked_writeback(q, s, delta, active_rows, n_active: int, w_live, stream=None) -> None:
    """Section 2.3 sparse write-back of the live bf16 weights."""
    import torch
    R, Cc = q.shape
    _check(lib().sft_masked_writeback(_dev(q, torch.int8), _dev(s, torch.float32), _dev(delta, torch.float32),
                                      R, Cc, _dev(active_rows, torch.int32), n_active, _dev(w_live),
                                      _stream(stream)))


def _c_wb_mats(mats):
    """mats: (q, s, delta, active_rows, n_active, w_live) per matrix."""
    import torch
    return (CWbMat * max(len(mats), 1))(*[
        CWbMat(_dev(q, torch.int8), _dev(s, torch.float32), _dev(d, torch.float32), q.shape[0], q.shape[1],
               _dev(rows, torch.int32), n, _dev(w)) for q, s, d, rows, n, w in mats])


def sft_masked_writeback_many(mats, stream=None) -> None:
    """Section 2.3 sparse write-back of several matrices in one launch; mats
    holds (q, s, delta, active_rows, n_active, w_live) per matrix."""
    arr = _c_wb_mats(mats)
    _check(lib().sft_masked_writeback_many(arr, len(mats), _stream(stream)))


# ------------------------------------------------------------------ prepared calls
class Prepared:
    """A device call with its ctypes arguments built once (for tight loops).

    Calling it enqueues the same launch again on the given stream; the tensors
    it refers to must stay alive (the object keeps references to them)."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


def prepare_masked_dw(groups: Sequence[DwGroup], ws=None) -> Prepared:
    arr, keep = _c_groups(groups)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return Prepared(lib().sft_masked_dw, (arr, len(groups), _dev(ws), nbytes), (arr, keep, groups, ws))


def prepare_sparse_update(mats: Sequence[UpdMat], hp: Adam) -> Prepared:
    arr = (CUpdMat * max(len(mats), 1))(*[m.c() for m in mats])
    h = hp.c()
    return Prepared(lib().sft_sparse_update, (arr, len(mats), C.byref(h)), (arr, h, mats, hp))


def prepare_masked_dw_update(groups: Sequence[DwGroup], ws, mats: Sequence[UpdMat], hp: Adam) -> Prepared:
    arr, keep = _c_groups(groups)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    u = (CUpdMat * max(len(mats), 1))(*[m.c() for m in mats])
    h = hp.c()
    return Prepared(lib().sft_masked_dw_update, (arr, len(groups), _dev(ws), nbytes, u, len(mats), C.byref(h)),
                    (arr, keep, u, h, groups, ws, mats, hp))


def prepare_coupled_update(pairs: Sequence[Pair], hp: Adam) -> Prepared:
    arr = (CPair * max(len(pairs), 1))(*[CPair(p.a.c(), p.b.c(), p.a_own, p.a_cross, _dev(p.clip))
                                         for p in pairs])
    h = hp.c()
    return Prepared(lib().sft_coupled_update, (arr, len(pairs), C.byref(h)), (arr, h, pairs, hp))


def prepare_embedding_dw(dY, row_ptr, positions, n_active: int, dW_act) -> Prepared:
    import torch
    T, d = dY.shape
    args = (_dev(dY, torch.bfloat16), T, d, _dev(row_ptr, torch.int32), _dev(positions, torch.int32), n_active,
            _dev(dW_act, torch.float32))
    return Prepared(lib().sft_embedding_dw, args, (dY, row_ptr, positions, dW_act))


def prepare_masked_writeback(q, s, delta, active_rows, n_active: int, w_live) -> Prepared:
    import torch
    R, Cc = q.shape
    args = (_dev(q, torch.int8), _dev(s, torch.float32), _dev(delta, torch.float32), R, Cc,
            _dev(active_rows, torch.int32), n_active, _dev(w_live))
    return Prepared(lib().sft_masked_writeback, args, (q, s, delta, active_rows, w_live))


def prepare_masked_writeback_many(mats) -> Prepared:
    arr = _c_wb_mats(mats)
    return Prepared(lib().sft_masked_writeback_many, (arr, len(mats)), (arr, mats))


# ------------------------------------------------------------------ checkpoint and rewind
SFT_REWIND_SAVE = 1
SFT_REWIND_RESTORE = 2
SFT_REWIND_SAVE_MIN = 4
SFT_REWIND_PROMOTE = 8


class Rewind:
    """Section 2.6 controller (host, C library): observe(loss) -> an OR of
    the SFT_REWIND_* bits.  ``st`` is the C state (its settings may be
    changed before the first observation)."""

    def __init__(self):
        self.st = CRewind()
        _check(lib().sft_rewind_init(C.byref(self.st)))

    def observe(self, loss: float) -> int:
        act = C.c_int32(0)
        _check(lib().sft_rewind_observe(C.byref(self.st), float(loss), C.byref(act)))
        return act.value

    def state(self) -> CRewind:
        return self.st


@dataclass
class CkptMat:
    """One matrix's live state, its checkpointed rows and the checkpoint buffers."""
    q: "object"             # int8 [R x C]
    s: "object"             # fp32 [R]
    delta: "object"         # fp32 [R x C]
    m: "object"             # fp16 bits [n_slots x C]
    v: "object"
    t: "object"             # int32 [n_slots]
    mv_exp: "object"        # int8 [n_slots x 2]
    rows: "object"          # int32 [n_rows] (GPU)
    slot: "object"          # int32 [n_rows] (GPU)
    ck_q: "object"          # int8 [n_rows x C]
    ck_s: "object"          # fp32 [n_rows]
    ck_delta: "object"      # fp32 [n_rows x C]
    ck_m: "object"          # fp16 bits [n_rows x C]
    ck_v: "object"
    ck_t: "object"          # int32 [n_rows]
    ck_mv_exp: "object"     # int8 [n_rows x 2]
    n_rows: int
    w_live: "object" = None  # bf16 [R x C] or None

    def c(self) -> CCkptMat:
        import torch
        R, Cc = self.q.shape
        n_slots = self.m.shape[0]
        n = int(self.n_rows)
        if n > 0:
            # the sizes the C checks cannot see (n_rows within R and n_slots is checked there)
            _shape(self.s, (R,), "s")
            _shape(self.t, (n_slots,), "t")
            _shape(self.mv_exp, (n_slots, 2), "mv_exp")
            for t_, what in ((self.rows, "rows"), (self.slot, "slot"), (self.ck_s, "ck_s"), (self.ck_t, "ck_t")):
                _numel_at_least(t_, n, what)
            _numel_at_least(self.ck_mv_exp, 2 * n, "ck_mv_exp")
            for t_, what in ((self.ck_q, "ck_q"), (self.ck_delta, "ck_delta"), (self.ck_m, "ck_m"),
                             (self.ck_v, "ck_v")):
                _numel_at_least(t_, n * Cc, what)
            _shape(self.delta, (R, Cc), "delta")
            _shape(self.m, (n_slots, Cc), "m")
            _shape(self.v, (n_slots, Cc), "v")
            if self.w_live is not None:
                _shape(self.w_live, (R, Cc), "w_live")
        return CCkptMat(R, Cc, n, n_slots, _dev(self.rows), _dev(self.slot), _dev(self.q),
                        _dev(self.s), _dev(self.delta), _dev(self.m), _dev(self.v), _dev(self.t),
                        _dev(self.mv_exp, torch.int8), _dev(self.w_live), _dev(self.ck_q), _dev(self.ck_s),
                        _dev(self.ck_delta), _dev(self.ck_m), _dev(self.ck_v), _dev(self.ck_t),
                        _dev(self.ck_mv_exp, torch.int8))

    @staticmethod
    def alloc(q, s, delta, m, v, t, mv_exp, rows, slot, n_rows: int, w_live=None) -> "CkptMat":
        """Checkpoint buffers for n_rows rows of this state (device tensors)."""
        import torch
        Cc = q.shape[1]
        dev = q.device
        n = max(n_rows, 1)
        return CkptMat(q, s, delta, m, v, t, mv_exp, rows, slot, torch.empty((n, Cc), dtype=torch.int8, device=dev),
                       torch.empty(n, dtype=torch.float32, device=dev),
                       torch.empty((n, Cc), dtype=torch.float32, device=dev),
                       torch.empty((n, Cc), dtype=m.dtype, device=dev), torch.empty((n, Cc), dtype=v.dtype, device=dev),
                       torch.empty(n, dtype=torch.int32, device=dev), torch.empty((n, 2), dtype=torch.int8, device=dev),
                       n_rows, w_live)


def sft_rows_save(mats: Sequence[CkptMat], stream=None) -> None:
    """Section 2.6: copy the listed rows of every matrix into its checkpoint buffers."""
    arr = (CCkptMat * max(len(mats), 1))(*[m.c() for m in mats])
    _check(lib().sft_rows_save(arr, len(mats), _stream(stream)))


def sft_rows_restore(mats: Sequence[CkptMat], stream=None) -> None:
    """Section 2.6: write the checkpointed rows back (and rebuild their live bf16 rows)."""
    arr = (CCkptMat * max(len(mats), 1))(*[m.c() for m in mats])
    _check(lib().sft_rows_restore(arr, len(mats), _stream(stream)))


def prepare_rows_save(mats: Sequence[CkptMat]) -> Prepared:
    arr = (CCkptMat * max(len(mats), 1))(*[m.c() for m in mats])
    return Prepared(lib().sft_rows_save, (arr, len(mats)), (arr, mats))


def prepare_rows_restore(mats: Sequence[CkptMat]) -> Prepared:
    arr = (CCkptMat * max(len(mats), 1))(*[m.c() for m in mats])
    return Prepared(lib().sft_rows_restore, (arr, len(mats)), (arr, mats))


# ------------------------------------------------------------------ SparseLeaf connections
@dataclass
class LeafMat:
    """One weight's K selected connections: dY bf16 [T x m], X bf16 [T x n],
    rows/cols int32 [K] (GPU), grad fp32 [K] (GPU, written)."""
    dY: "object"
    X: "object"
    rows: "object"
    cols: "object"
    grad: "object"

    def c(self) -> CLeafMat:
        import torch
        T, m = self.dY.shape
        n = self.X.shape[1]
        return CLeafMat(_dev(self.dY, torch.bfloat16), _dev(self.X, torch.bfloat16), m, n, self.rows.numel(),
                        _dev(self.rows, torch.int32), _dev(self.cols, torch.int32), _dev(self.grad, torch.float32))


def _leaf_arr(mats: Sequence[LeafMat]):
    return (CLeafMat * max(len(mats), 1))(*[m.c() for m in mats])


def _leaf_T(mats: Sequence[LeafMat]) -> int:
    Ts = {m.dY.shape[0] for m in mats} | {m.X.shape[0] for m in mats}
    if len(Ts) > 1:
        raise SftError(SFT_EINVAL, f"sft_leaf_grad: matrices with different token counts {sorted(Ts)}")
    return Ts.pop() if Ts else 0


def sft_leaf_grad_workspace(mats: Sequence[LeafMat]) -> int:
    n = lib().sft_leaf_grad_workspace(_leaf_arr(mats), len(mats), _leaf_T(mats))
    if n == C.c_size_t(-1).value:
        raise SftError(SFT_EINVAL, lib().sft_last_error().decode())
    return n


def sft_leaf_grad(mats: Sequence[LeafMat], ws, stream=None) -> None:
    """SparseLeaf: gradients of the selected connections of every matrix (async)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sft_leaf_grad(_leaf_arr(mats), len(mats), _leaf_T(mats), _dev(ws), nbytes, _stream(stream)))


@dataclass
class LeafVec:
    """One weight's increments and their Adam state (fp32 [K] each, GPU)."""
    grad: "object"
    theta: "object"
    m: "object"
    v: "object"
    theta_bf16: "object" = None

    def c(self) -> CLeafVec:
        return CLeafVec(self.theta.numel(), _dev(self.grad), _dev(self.theta), _dev(self.m), _dev(self.v),
                        _dev(self.theta_bf16))


def sft_leaf_adam(vecs: Sequence[LeafVec], step: int, hp: Adam, stream=None) -> None:
    """SparseLeaf Adam step on every vector's increments (async)."""
    arr = (CLeafVec * max(len(vecs), 1))(*[v.c() for v in vecs])
    h = hp.c()
    _check(lib().sft_leaf_adam(arr, len(vecs), int(step), C.byref(h), _stream(stream)))


def prepare_leaf_grad(mats: Sequence[LeafMat], ws) -> Prepared:
    arr = _leaf_arr(mats)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return Prepared(lib().sft_leaf_grad, (arr, len(mats), _leaf_T(mats), _dev(ws), nbytes), (arr, mats, ws))


def prepare_leaf_adam(vecs: Sequence[LeafVec], step: int, hp: Adam) -> Prepared:
    arr = (CLeafVec * max(len(vecs), 1))(*[v.c() for v in vecs])
    h = hp.c()
    return Prepared(lib().sft_leaf_adam, (arr, len(vecs), int(step), C.byref(h)), (arr, h, vecs, hp))


# ------------------------------------------------------------------ coupled-update schedule
class Helix:
    """The coupled update's scalar schedule (host, C library): step(loss,
    rewind) -> (stride, phase in degrees); coupling(b, psi) -> (a_own, a_cross)."""

    def __init__(self):
        self.st = CHelix()
        _check(lib().sft_helix_init(C.byref(self.st)))

    def step(self, loss: float, rewind: bool = False):
        stride = C.c_int32(0)
        phase = C.c_double(0.0)
        _check(lib().sft_helix_step(C.byref(self.st), float(loss), int(bool(rewind)), C.byref(stride),
                                    C.byref(phase)))
        return stride.value, phase.value

    def coupling(self, b: float, psi_deg: float = 0.0):
        a_own = C.c_double(0.0)
        a_cross = C.c_double(0.0)
        _check(lib().sft_helix_coupling(C.byref(self.st), float(b), float(psi_deg), C.byref(a_own),
                                        C.byref(a_cross)))
        return a_own.value, a_cross.value


# ------------------------------------------------------------------ measurement probes
def sft_probe_grid() -> int:
    return lib().sft_probe_grid()


def prepare_probe_read(buf, sink) -> Prepared:
    nbytes = buf.numel() * buf.element_size()
    return Prepared(lib().sft_probe_read, (_dev(buf), nbytes, _dev(sink)), (buf, sink))


def prepare_probe_copy(src, dst) -> Prepared:
    nbytes = src.numel() * src.element_size()
    return Prepared(lib().sft_probe_copy, (_dev(src), _dev(dst), nbytes), (src, dst))


def prepare_probe_mfma(iters: int, out) -> Prepared:
    return Prepared(lib().sft_probe_mfma, (int(iters), _dev(out)), (out,))


DW_LAUNCH_KINDS = {0: "stream-k", 1: "aligned", 2: "teams", 3: "narrow"}


def sft_probe_dw_plan(groups, cus: int = 0) -> list:
    """How sft_masked_dw would launch groups of host row plans (no device
    work): groups = [(T, C, layout, [Plan, ...]), ...] with each matrix's
    Plan from sft_plan_rows.  Returns one dict per product launch: kind,
    workgroups, and per group (shape, M-blocks, column blocks)."""
    dummy = np.zeros(8, np.float32)          # stands in for X, dY and dW_act: never read
    if dummy.ctypes.data % 16:
        dummy = np.zeros(12, np.float32)[2:10]
    ptr = dummy.ctypes.data
    keep, arr = [], (CDwGroup * max(len(groups), 1))()
    for i, (T, Cc, layout, plans) in enumerate(groups):
        mats = (CDwMat * max(len(plans), 1))()
        for j, pl in enumerate(plans):
            mats[j] = CDwMat(ptr, pl.rows, _np_ptr(pl.active_rows), _np_ptr(pl.active_tiles),
                             _np_ptr(pl.active_bits), _np_ptr(pl.tile_first), pl.n_active, pl.n_active_tiles, ptr)
        keep.append(mats)
        arr[i] = CDwGroup(ptr, T, Cc, len(plans), layout, mats)
    out = np.zeros(1024, np.int32)
    n = lib().sft_probe_dw_plan(arr, len(groups), cus, _np_ptr(out), out.size)
    if n < 0:
        raise SftError(n, lib().sft_last_error().decode())
    assert n <= out.size, "plan description longer than its buffer"
    v, i, res = out[:n].tolist(), 0, []
    while i < n:
        kind, wg, ng = v[i:i + 3]
        i += 3
        res.append({"kind": DW_LAUNCH_KINDS[kind], "workgroups": wg,
                    "groups": [tuple(v[i + 3 * g:i + 3 * g + 3]) for g in range(ng)]})
        i += 3 * ng
    return res
