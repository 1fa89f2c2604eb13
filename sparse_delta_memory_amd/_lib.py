"""ctypes view of the C ABI declared in include/sdm.h (libsdm_amd.so next to this file)."""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# SDM_LIB selects another build of the same library (the host-sanitized one, libsdm_amd_san.so).
LIB_PATH = os.environ.get("SDM_LIB") or os.path.join(HERE, "libsdm_amd.so")

SDM_OK = 0
SDM_EINVAL = -1
SDM_ESHAPE = -2
SDM_EALIGN = -3
SDM_EUNSUPPORTED = -4
SDM_EWORKSPACE = -5
SDM_EHIP = -6
SDM_F32 = 0
SDM_BF16 = 1


class P1Shape(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("C", ctypes.c_int32), ("W", ctypes.c_int32), ("R", ctypes.c_int32),
        ("P", ctypes.c_int32), ("key_bits", ctypes.c_int32), ("stream_offset", ctypes.c_int64),
        ("first_partial", ctypes.c_int32), ("valid_last", ctypes.c_int32), ("tile_len", ctypes.c_int32),
        ("g_lane_stride", ctypes.c_int32), ("idx_bytes", ctypes.c_int32), ("val_bytes", ctypes.c_int32),
        ("tiled", ctypes.c_int32), ("lds_budget", ctypes.c_int32), ("pair_walk", ctypes.c_int32),
    ]


P1_IO_FIELDS = [
    "k_idx", "q_idx", "k_val", "q_val", "g",
    "log_k", "rex", "cpe", "k_eff", "is_last", "is_only", "pos_k",
    "log_q", "q_w", "pos_q", "q_last", "q_only",
    "spay_k", "spay_q", "krec", "tiles_k", "a", "qk", "repeats", "perm",
]


class P1IO(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in P1_IO_FIELDS] + [
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("events", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("gord_k", ctypes.c_void_p), ("defer_pairs", ctypes.c_int32)]


class DwIO(ctypes.Structure):
    _fields_ = [
        ("bank", ctypes.c_void_p), ("bank_dtype", ctypes.c_int32), ("rows", ctypes.c_int64),
        ("hd", ctypes.c_int32), ("dv", ctypes.c_void_p), ("dv_dtype", ctypes.c_int32),
        ("dv_step_rows", ctypes.c_int64), ("dv_rows", ctypes.c_int64), ("krec", ctypes.c_void_p),
        ("P", ctypes.c_int32), ("C", ctypes.c_int32), ("W", ctypes.c_int32), ("N", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("events", ctypes.c_void_p),
        ("snap", ctypes.c_void_p), ("snap_step_rows", ctypes.c_int64), ("snap_rows", ctypes.c_int64),
        ("snap_dtype", ctypes.c_int32), ("snap_ord", ctypes.c_void_p),
    ]


class ReadIO(ctypes.Structure):
    _fields_ = [
        ("bank", ctypes.c_void_p), ("bank_dtype", ctypes.c_int32), ("rows", ctypes.c_int64), ("hd", ctypes.c_int32),
        ("k_idx", ctypes.c_void_p), ("q_idx", ctypes.c_void_p), ("k_eff", ctypes.c_void_p), ("q_w", ctypes.c_void_p),
        ("a", ctypes.c_void_p), ("qk", ctypes.c_void_p), ("v", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("dv", ctypes.c_void_p), ("pred", ctypes.c_void_p), ("read", ctypes.c_void_p),
        ("step_rows", ctypes.c_int64), ("out_rows", ctypes.c_int64),
        ("P", ctypes.c_int32), ("C", ctypes.c_int32), ("W", ctypes.c_int32), ("R", ctypes.c_int32),
        ("N", ctypes.c_int32), ("first_partial", ctypes.c_int32), ("valid_last", ctypes.c_int32),
        ("idx_bytes", ctypes.c_int32), ("val_bytes", ctypes.c_int32), ("events", ctypes.c_void_p),
    ]


class GdsIO(ctypes.Structure):
    _fields_ = [
        ("bank", ctypes.c_void_p), ("bank_dtype", ctypes.c_int32), ("rows", ctypes.c_int64), ("hd", ctypes.c_int32),
        ("q_idx", ctypes.c_void_p), ("q_w", ctypes.c_void_p), ("spay_q", ctypes.c_void_p), ("gr", ctypes.c_void_p),
        ("step_rows", ctypes.c_int64), ("gr_rows", ctypes.c_int64), ("d_q_w", ctypes.c_void_p), ("grad", ctypes.c_void_p),
        ("grad_dtype", ctypes.c_int32), ("P", ctypes.c_int32), ("C", ctypes.c_int32), ("R", ctypes.c_int32),
        ("N", ctypes.c_int32), ("first_partial", ctypes.c_int32), ("valid_last", ctypes.c_int32),
        ("idx_bytes", ctypes.c_int32), ("val_bytes", ctypes.c_int32), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class GwrIO(ctypes.Structure):
    _fields_ = [
        ("grad", ctypes.c_void_p), ("grad_dtype", ctypes.c_int32), ("rows", ctypes.c_int64), ("hd", ctypes.c_int32),
        ("k_idx", ctypes.c_void_p), ("w", ctypes.c_void_p), ("dv", ctypes.c_void_p), ("step_rows", ctypes.c_int64),
        ("dv_rows", ctypes.c_int64), ("d_dv", ctypes.c_void_p), ("d_k_pd", ctypes.c_void_p),
        ("P", ctypes.c_int32), ("C", ctypes.c_int32), ("W", ctypes.c_int32), ("N", ctypes.c_int32),
        ("first_partial", ctypes.c_int32), ("valid_last", ctypes.c_int32), ("idx_bytes", ctypes.c_int32),
    ]


class PaIO(ctypes.Structure):
    _fields_ = [
        ("grad", ctypes.c_void_p), ("grad_dtype", ctypes.c_int32), ("bank", ctypes.c_void_p),
        ("bank_dtype", ctypes.c_int32), ("rows", ctypes.c_int64), ("hd", ctypes.c_int32), ("snap", ctypes.c_void_p),
        ("snap_step_rows", ctypes.c_int64), ("snap_rows", ctypes.c_int64), ("krec", ctypes.c_void_p),
        ("k_eff", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("d_dva", ctypes.c_void_p), ("step_rows", ctypes.c_int64),
        ("dva_rows", ctypes.c_int64), ("g_decay", ctypes.c_void_p), ("d_k_eff", ctypes.c_void_p),
        ("P", ctypes.c_int32), ("C", ctypes.c_int32), ("W", ctypes.c_int32), ("N", ctypes.c_int32),
        ("val_bytes", ctypes.c_int32), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


EXPORTS = ["sdm_phase1_workspace", "sdm_phase1", "sdm_phase1_pairs", "sdm_dw_workspace", "sdm_dw_step", "sdm_dw_step_noalloc", "sdm_read_step",
           "sdm_gds_workspace", "sdm_gds_step", "sdm_gwr_step", "sdm_pa_workspace", "sdm_pa_step", "sdm_status_string", "sdm_last_error"]

_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load libsdm_amd.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # torch first: its HIP runtime (same SONAME) is then the one this library binds to, so
        # torch's streams and device pointers are valid here.
        import torch  # noqa: F401

        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libsdm_amd.so is not built (run `python -m sparse_delta_memory_amd.build`); "
                "the SDM hot path has no CPU fallback")
        lib = ctypes.CDLL(LIB_PATH)
        lib.sdm_phase1_workspace.argtypes = [ctypes.POINTER(P1Shape)]
        lib.sdm_phase1_workspace.restype = ctypes.c_size_t
        lib.sdm_phase1.argtypes = [ctypes.POINTER(P1Shape), ctypes.POINTER(P1IO), ctypes.c_void_p]
        lib.sdm_phase1.restype = ctypes.c_int
        lib.sdm_phase1_pairs.argtypes = [ctypes.POINTER(P1Shape), ctypes.POINTER(P1IO), ctypes.c_void_p]
        lib.sdm_phase1_pairs.restype = ctypes.c_int
        lib.sdm_dw_workspace.argtypes = [ctypes.POINTER(DwIO)]
        lib.sdm_dw_workspace.restype = ctypes.c_size_t
        lib.sdm_dw_step.argtypes = [ctypes.POINTER(DwIO), ctypes.c_int64, ctypes.c_void_p]
        lib.sdm_dw_step.restype = ctypes.c_int
        lib.sdm_dw_step_noalloc.argtypes = [ctypes.POINTER(DwIO), ctypes.c_int64, ctypes.c_void_p]
        lib.sdm_dw_step_noalloc.restype = ctypes.c_int
        lib.sdm_read_step.argtypes = [ctypes.POINTER(ReadIO), ctypes.c_int64, ctypes.c_void_p]
        lib.sdm_read_step.restype = ctypes.c_int
        lib.sdm_gds_step.argtypes = [ctypes.POINTER(GdsIO), ctypes.c_int64, ctypes.c_void_p]
        lib.sdm_gds_step.restype = ctypes.c_int
        lib.sdm_gwr_step.argtypes = [ctypes.POINTER(GwrIO), ctypes.c_int64, ctypes.c_void_p]
        lib.sdm_gwr_step.restype = ctypes.c_int
        lib.sdm_gds_workspace.argtypes = [ctypes.POINTER(GdsIO)]
        lib.sdm_gds_workspace.restype = ctypes.c_size_t
        lib.sdm_pa_workspace.argtypes = [ctypes.POINTER(PaIO)]
        lib.sdm_pa_workspace.restype = ctypes.c_size_t
        lib.sdm_pa_step.argtypes = [ctypes.POINTER(PaIO), ctypes.c_int64, ctypes.c_void_p]
        lib.sdm_pa_step.restype = ctypes.c_int
        lib.sdm_status_string.argtypes = [ctypes.c_int]
        lib.sdm_status_string.restype = ctypes.c_char_p
        lib.sdm_last_error.argtypes = []
        lib.sdm_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


class SdmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d): %s" % (load().sdm_status_string(status).decode(), status, message))
        self.status = status


def check(status: int) -> None:
    if status != SDM_OK:
        raise SdmError(status, load().sdm_last_error().decode())
