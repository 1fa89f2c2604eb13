"""CPU oracle for the SDM forward hot path (Phase 1 and the DW step).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg use it; the product path never imports it. It shares no code with the HIP
implementation: the arithmetic lives in ``sdm_oracle.c`` (plain C, double precision), and this
module only marshals numpy arrays into it.

Definitions follow the page "sparse_delta_memory/cuda/phase1_cuda.py" (module docstring and the
Outputs / Records comments) and the DW definition of "sparse_delta_memory/cuda/mover_da2_cuda.py"
(module docstring). Every floating result is returned in float64.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsdm_oracle.so")
_lock = threading.Lock()
_lib = None


_SAN_LIB_PATH = os.path.join(_HERE, "libsdm_oracle_san.so")


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile sdm_oracle.c with gcc into oracle/libsdm_oracle.so (plain -O2, no fast-math).
    sanitize: with clang (the ROCm toolchain's, whose ASan runtime the sanitized HIP library also
    uses) and -fsanitize=address,undefined (UB traps) into libsdm_oracle_san.so. SDM_ORACLE_LIB,
    when set, names the library to load instead of building."""
    if os.environ.get("SDM_ORACLE_LIB") and not sanitize:
        return os.environ["SDM_ORACLE_LIB"]
    path = _SAN_LIB_PATH if sanitize else _LIB_PATH
    if force or sanitize or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        tmp = path + ".tmp%d" % os.getpid()
        if sanitize:
            cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                   "-fsanitize=address,undefined", "-fsanitize-trap=undefined", "-fno-omit-frame-pointer",
                   "-o", tmp, _SRC, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, path)
    return path


class _ChunkIn(ctypes.Structure):
    _fields_ = [
        ("C", ctypes.c_int), ("W", ctypes.c_int), ("R", ctypes.c_int), ("t_valid", ctypes.c_int),
        ("id_base", ctypes.c_int64),
        ("k_idx", ctypes.c_void_p), ("q_idx", ctypes.c_void_p), ("k_val", ctypes.c_void_p),
        ("q_val", ctypes.c_void_p), ("g", ctypes.c_void_p), ("tile_len", ctypes.c_int),
        ("g_width", ctypes.c_int), ("g_lane_stride", ctypes.c_int), ("val_bf16", ctypes.c_int),
    ]


_OUT_FIELDS = [
    "log_k", "rex", "cpe", "k_eff", "is_last", "is_only", "pos_k", "log_q", "q_w", "pos_q", "q_last", "q_only",
    "spay_k", "spay_q", "krec_slot", "krec_sc", "krec_cpe", "tiles_k", "a", "qk", "perm", "repeats",
    "a_mag", "qk_mag", "a_cnt", "qk_cnt", "gord_k",
]


class _ChunkOut(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _OUT_FIELDS]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            lib.oracle_phase1_chunk.argtypes = [ctypes.POINTER(_ChunkIn), ctypes.POINTER(_ChunkOut)]
            lib.oracle_phase1_chunk.restype = ctypes.c_int
            lib.oracle_dw_slots.argtypes = [ctypes.POINTER(_ChunkIn), ctypes.c_void_p]
            lib.oracle_dw_slots.restype = ctypes.c_int64
            lib.oracle_dw_apply.argtypes = [ctypes.POINTER(_ChunkIn), ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            lib.oracle_dw_apply.restype = ctypes.c_int64
            lib.oracle_round_bf16.argtypes = [ctypes.c_double]
            lib.oracle_round_bf16.restype = ctypes.c_double
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _chunk_in(k_idx, q_idx, k_val, q_val, g, c, P, stream_offset, first_partial, valid_last, tile_len, val_bf16=False):
    C, W = k_idx.shape[1], k_idx.shape[2]
    R = q_idx.shape[2]
    arrs = (np.ascontiguousarray(k_idx[c], dtype=np.int32), np.ascontiguousarray(q_idx[c], dtype=np.int32),
            np.ascontiguousarray(k_val[c], dtype=np.float32), np.ascontiguousarray(q_val[c], dtype=np.float32),
            np.ascontiguousarray(g[c], dtype=np.float32))
    t_valid = valid_last if c >= first_partial else C
    # gates [N, C] (one per token) or [N, C, W] (one per token and K lane)
    per_lane = np.ndim(g) == 3
    if per_lane and np.shape(g)[2] != W:
        raise ValueError("per-lane gates must be [N, C, W]")
    s = _ChunkIn(C, W, R, t_valid, (c % P) * stream_offset, *[_ptr(a) for a in arrs], tile_len,
                 W if per_lane else 1, 1 if per_lane else 0, 1 if val_bf16 else 0)
    return s, arrs


def phase1(k_idx, q_idx, k_val, q_val, g, *, P=1, stream_offset=0, first_partial=None, valid_last=None,
           tile_len=128, chunks=None, threads=1, fields=None, val_bf16=False):
    """Phase 1 of the chunks `chunks` (default: all). Arrays are [N, C, W] / [N, C, R] / [N, C].

    Returns a dict of numpy arrays whose first axis runs over the requested chunks. `fields`
    selects the outputs (default: every Phase-1 output; the per-cell term magnitudes a_mag /
    qk_mag and term counts a_cnt / qk_cnt only when named). val_bf16: the values are bfloat16
    (k_val / q_val hold their exact values); cpe, k_eff, q_w and krec_cpe are then the exact
    values rounded to bfloat16."""
    lib = _load()
    N, C, W = k_idx.shape
    R = q_idx.shape[2]
    if first_partial is None:
        first_partial = N
    if valid_last is None:
        valid_last = C
    chunks = list(range(N)) if chunks is None else [int(c) for c in chunks]
    m = len(chunks)
    nk, nq, n = C * W, C * R, C * (W + R)
    L = max(int(tile_len), 1)
    ntk = (nk + L - 1) // L
    shapes = {
        "log_k": ((C, W), np.float64), "rex": ((C, W), np.float64), "cpe": ((C, W), np.float64),
        "k_eff": ((C, W), np.float64), "is_last": ((C, W), np.int8), "is_only": ((C, W), np.int8),
        "pos_k": ((C, W), np.int32), "log_q": ((C, R), np.float64), "q_w": ((C, R), np.float64),
        "pos_q": ((C, R), np.int32), "q_last": ((C, R), np.int8), "q_only": ((C, R), np.int8),
        "spay_k": ((nk,), np.int32), "spay_q": ((nq,), np.int32), "krec_slot": ((nk,), np.int32),
        "krec_sc": ((nk,), np.float64), "krec_cpe": ((nk,), np.float64), "tiles_k": ((ntk + 1,), np.int32),
        "a": ((C, C), np.float64), "qk": ((C, C), np.float64), "perm": ((n,), np.int32), "repeats": ((1,), np.int64),
        "a_mag": ((C, C), np.float64), "qk_mag": ((C, C), np.float64), "a_cnt": ((C, C), np.int32),
        "qk_cnt": ((C, C), np.int32), "gord_k": ((nk,), np.int32),
    }
    optional = {"a_mag", "qk_mag", "a_cnt", "qk_cnt"}   # evaluation-error scales: only when asked for
    want = (set(shapes) - optional) if fields is None else set(fields)
    if "tiles_k" in want:
        want.add("spay_k")
    res = {f: np.zeros((m,) + shapes[f][0], dtype=shapes[f][1]) for f in shapes if f in want}

    def run(i):
        c = chunks[i]
        cin, keep = _chunk_in(k_idx, q_idx, k_val, q_val, g, c, P, stream_offset, first_partial, valid_last, L,
                              val_bf16)
        out = _ChunkOut(*[(_ptr(res[f][i]) if f in res else None) for f in _OUT_FIELDS])
        rc = lib.oracle_phase1_chunk(ctypes.byref(cin), ctypes.byref(out))
        del keep
        if rc != 0:
            raise MemoryError("oracle_phase1_chunk failed (%d)" % rc)

    if threads > 1 and m > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, range(m)))
    else:
        for i in range(m):
            run(i)
    if "repeats" in res:
        res["repeats"] = res["repeats"][:, 0]
    return res


def dw_slots(k_idx, q_idx, k_val, q_val, g, c, *, P=1, stream_offset=0, first_partial=None, valid_last=None):
    """Absolute slots of chunk c's valid K groups, ascending (int64)."""
    lib = _load()
    N, C, _ = k_idx.shape
    first_partial = N if first_partial is None else first_partial
    valid_last = C if valid_last is None else valid_last
    cin, keep = _chunk_in(k_idx, q_idx, k_val, q_val, g, c, P, stream_offset, first_partial, valid_last, 1)
    cnt = lib.oracle_dw_slots(ctypes.byref(cin), None)
    if cnt < 0:
        raise MemoryError("oracle_dw_slots failed")
    out = np.zeros(max(cnt, 1), dtype=np.int64)
    lib.oracle_dw_slots(ctypes.byref(cin), _ptr(out))
    del keep
    return out[:cnt]


def dw_apply(k_idx, q_idx, k_val, q_val, g, c, dv_rows, base_rows, *, P=1, stream_offset=0, first_partial=None,
             valid_last=None, with_magnitude=False, val_bf16=False):
    """New rows of chunk c's valid K groups in float64: base * exp(G) + sum k exp(rex) dv.

    dv_rows: [C, hd] token rows of the chunk; base_rows: [groups, hd] pre-step rows in the order of
    dw_slots. With with_magnitude, also returns the per-element magnitude sum of the terms. With
    val_bf16 the base row is scaled by exp(G) rounded to bfloat16 (the records' cpe)."""
    lib = _load()
    N, C, _ = k_idx.shape
    first_partial = N if first_partial is None else first_partial
    valid_last = C if valid_last is None else valid_last
    dv = np.ascontiguousarray(dv_rows, dtype=np.float64)
    base = np.ascontiguousarray(base_rows, dtype=np.float64)
    hd = dv.shape[1]
    out = np.zeros_like(base)
    mag = np.zeros_like(base) if with_magnitude else None
    cin, keep = _chunk_in(k_idx, q_idx, k_val, q_val, g, c, P, stream_offset, first_partial, valid_last, 1,
                          val_bf16)
    cnt = lib.oracle_dw_apply(ctypes.byref(cin), hd, _ptr(dv), _ptr(base), _ptr(out), _ptr(mag))
    del keep
    if cnt != base.shape[0]:
        raise ValueError("dw_apply: %d groups, %d base rows" % (cnt, base.shape[0]))
    return (out, mag) if with_magnitude else out


def round_bf16(x):
    """x (float64 array) rounded to the nearest bfloat16 value, ties to even (oracle_round_bf16)."""
    lib = _load()
    a = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_round_bf16(float(v)) for v in a.ravel()], dtype=np.float64).reshape(a.shape)
