"""MI355X (gfx950) forward hot path of the chunked sparse-delta-memory (SDM) recurrence.

Python binding of the C ABI in include/sdm.h. Everything here is argument marshalling: torch
provides device memory and the current stream; every step of the path runs in the HIP kernels of
libsdm_amd.so. There is no CPU fallback: without the built library every call raises.

    shape = P1Shape(N=..., C=..., W=..., R=..., P=..., key_bits=..., stream_offset=...)
    out = phase1(shape, k_idx, q_idx, k_val, q_val, g)          # dict of device tensors
    dw_step(bank, dv, out["krec"], shape, ti, dv_step_rows=P*C)  # bank updated in place
    read_step(bank, out, k_idx, q_idx, v, beta, dv, pred, read, shape, ti, step_rows=P*C)  # before DW
"""

from __future__ import annotations

import ctypes

from . import _lib
from ._lib import P1IO, P1Shape, SdmError  # noqa: F401

__all__ = ["P1Shape", "phase1", "phase1_pairs", "phase1_workspace_bytes", "alloc_phase1_outputs", "dw_step", "dw_workspace_bytes",
           "alloc_dw_workspace", "DwPlan", "ReadPlan", "read_step", "gds_step", "gds_workspace_bytes", "alloc_gds_workspace", "gwr_step", "pa_step", "pa_workspace_bytes",
           "alloc_pa_workspace", "SdmError", "make_shape",
           "timing_events"]


def make_shape(N, C, W, R, P=1, key_bits=16, stream_offset=0, first_partial=None, valid_last=None, tile_len=128,
               g_lane_stride=0, idx_bytes=4, val_bytes=4, tiled=False, lds_budget=0, pair_walk=False):
    """Phase-1 shape. g_lane_stride 0: gates g [N, C] (per token); 1: g [N, C, W] (per token and K lane).
    idx_bytes 4: int32 slot ids; 8: int64. val_bytes 4: float32 values; 2: bfloat16 values (and
    bfloat16 cpe, k_eff, q_w). tiled: every row through the tiled path (rows past 16384 entries
    always take it). lds_budget: LDS bytes the sort/scan kernel plans with (0: all of it; a smaller
    budget takes its narrower-digit, unstaged and multi-sweep paths, with the same bits). pair_walk:
    every slot group walked by the pair kernel (no dense hot-group contraction)."""
    return P1Shape(int(N), int(C), int(W), int(R), int(P), int(key_bits), int(stream_offset),
                   int(N if first_partial is None else first_partial), int(C if valid_last is None else valid_last),
                   int(tile_len), int(g_lane_stride), int(idx_bytes), int(val_bytes), int(bool(tiled)),
                   int(lds_budget), int(bool(pair_walk)))


def phase1_workspace_bytes(shape: P1Shape) -> int:
    return int(_lib.load().sdm_phase1_workspace(ctypes.byref(shape)))


def _ptr(t):
    return None if t is None else t.data_ptr()


def alloc_phase1_outputs(shape: P1Shape, device="cuda", fields=None):
    """Device tensors for the Phase-1 outputs (all of them, or `fields` plus the required ones)."""
    import torch

    N, C, W, R, L = shape.N, shape.C, shape.W, shape.R, shape.tile_len
    ntk = (C * W + L - 1) // L
    vt = torch.bfloat16 if shape.val_bytes == 2 else torch.float32   # value-typed fields
    spec = {
        "log_k": ((N, C, W), torch.float32), "rex": ((N, C, W), torch.float32), "cpe": ((N, C, W), vt),
        "k_eff": ((N, C, W), vt), "is_last": ((N, C, W), torch.int8), "is_only": ((N, C, W), torch.int8),
        "pos_k": ((N, C, W), torch.int32), "log_q": ((N, C, R), torch.float32), "q_w": ((N, C, R), vt),
        "pos_q": ((N, C, R), torch.int32), "q_last": ((N, C, R), torch.int8), "q_only": ((N, C, R), torch.int8),
        "spay_k": ((N, C * W), torch.int32), "spay_q": ((N, C * R), torch.int32),
        "krec": ((N, C * W, 4), torch.int32), "tiles_k": ((N, ntk + 1), torch.int32),
        "a": ((N, C, C), torch.float32), "qk": ((N, C, C), torch.float32), "repeats": ((N,), torch.int32),
        "perm": ((N, C * (W + R)), torch.int32), "gord_k": ((N, C * W), torch.int32),
    }
    # perm (the sorted order itself) and gord_k (dense group ordinals) only when asked for
    want = (set(spec) - {"perm", "gord_k"}) if fields is None else set(fields) | {"spay_k", "krec", "tiles_k"}
    return {k: torch.empty(s, dtype=dt, device=device) for k, (s, dt) in spec.items() if k in want}


def phase1(shape: P1Shape, k_idx, q_idx, k_val, q_val, g, out=None, workspace=None, stream=None, events=None,
           status=None, defer_pairs=False):
    """Enqueue Phase 1 of shape.N chunks on the current (or given) stream; returns the outputs.

    Inputs are contiguous device tensors: k_idx [N,C,W] / q_idx [N,C,R] int32 (int64 with
    shape.idx_bytes = 8), k_val / q_val
    float32 (bfloat16 with shape.val_bytes = 2) of the same shapes, g [N,C] float32 ([N,C,W] when shape.g_lane_stride = 1). `out` is a dict from alloc_phase1_outputs (a
    missing key skips that optional output). events: optional 4 torch.cuda.Events (timing_events)
    bound to the two kernels. status: optional zeroed int32 device tensor (debug): bit 0 is set
    when a valid entry's slot id is out of range. defer_pairs: leave A and QK to phase1_pairs (same
    shape, out and workspace), which may then run on another stream."""
    import torch

    lib = _lib.load()
    want = 8 if shape.idx_bytes == 8 else 4
    if k_idx.element_size() != want or q_idx.element_size() != want:
        raise TypeError("phase1: ids must be int%d (shape.idx_bytes = %d)" % (want * 8, shape.idx_bytes))
    vt = torch.bfloat16 if shape.val_bytes == 2 else torch.float32
    if k_val.dtype != vt or q_val.dtype != vt:
        raise TypeError("phase1: values must be %s (shape.val_bytes = %d)" % (vt, shape.val_bytes))
    if out is not None:
        for name in ("cpe", "k_eff", "q_w"):
            if out.get(name) is not None and out[name].dtype != vt:
                raise TypeError("phase1: %s must be %s (shape.val_bytes = %d)" % (name, vt, shape.val_bytes))
    if out is None:
        out = alloc_phase1_outputs(shape, device=k_idx.device)
    need = phase1_workspace_bytes(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=k_idx.device)
    io = P1IO()
    for name, t in (("k_idx", k_idx), ("q_idx", q_idx), ("k_val", k_val), ("q_val", q_val), ("g", g)):
        setattr(io, name, _ptr(t))
    for name in _lib.P1_IO_FIELDS[5:]:
        setattr(io, name, _ptr(out.get(name)))
    io.workspace = workspace.data_ptr()
    io.workspace_bytes = workspace.numel() * workspace.element_size()
    arr = _event_array(events, 4, "phase1")
    io.events = None if arr is None else ctypes.cast(arr, ctypes.c_void_p).value
    if status is not None:
        io.status = status.data_ptr()
    io.gord_k = _ptr(out.get("gord_k"))
    io.defer_pairs = 1 if defer_pairs else 0
    st = torch.cuda.current_stream(k_idx.device) if stream is None else stream
    _lib.check(lib.sdm_phase1(ctypes.byref(shape), ctypes.byref(io), ctypes.c_void_p(st.cuda_stream)))
    return out


def phase1_pairs(shape: P1Shape, out, workspace, stream=None, events=None):
    """Enqueue the pair sums (out["a"], out["qk"]) of an earlier phase1(..., defer_pairs=True) call
    with the same shape, out and workspace. `stream` must be ordered after that call's stream.
    events: optional 4 timing events (the pair kernel takes the last two)."""
    import torch

    lib = _lib.load()
    io = P1IO()
    io.a = _ptr(out.get("a"))
    io.qk = _ptr(out.get("qk"))
    io.workspace = workspace.data_ptr()
    io.workspace_bytes = workspace.numel() * workspace.element_size()
    arr = _event_array(events, 4, "phase1_pairs")
    io.events = None if arr is None else ctypes.cast(arr, ctypes.c_void_p).value
    dev = workspace.device
    st = torch.cuda.current_stream(dev) if stream is None else stream
    _lib.check(lib.sdm_phase1_pairs(ctypes.byref(shape), ctypes.byref(io), ctypes.c_void_p(st.cuda_stream)))
    return out


def dw_workspace_bytes(shape: P1Shape, hd: int) -> int:
    """Bytes of the (zero-filled) DW workspace that lets long groups be split across lanes."""
    io = _lib.DwIO()
    io.P, io.C, io.W, io.N, io.hd = shape.P, shape.C, shape.W, shape.N, int(hd)
    return int(_lib.load().sdm_dw_workspace(ctypes.byref(io)))


def alloc_dw_workspace(shape: P1Shape, hd: int, device="cuda"):
    """A zero-filled DW workspace (reusable by every step of the same shape)."""
    import torch

    return torch.zeros(max(dw_workspace_bytes(shape, hd), 1), dtype=torch.uint8, device=device)


def timing_events(count, stream=None):
    """`count` timing torch.cuda.Events, each recorded once on `stream` so that its HIP event exists
    (torch creates it at the first record); a kernel launch then records them again."""
    import torch

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(count)]
    for e in evs:
        e.record(stream)
    return evs


def _event_array(events, count, name):
    """A ctypes array of `count` hipEvent_t handles from torch.cuda.Event objects (read at enqueue time)."""
    if events is None:
        return None
    events = list(events)
    if len(events) != count:
        raise ValueError("%s: expected %d events, got %d" % (name, count, len(events)))
    handles = [e.cuda_event for e in events]
    if not all(handles):
        raise ValueError("%s: an event has no HIP event yet; record it once first (see timing_events)" % name)
    return (ctypes.c_void_p * count)(*handles)


class DwPlan:
    """The DW step planned once for a bank, token rows, records and shape, launched per step.

    bank [rows, hd] float32 or bfloat16 (updated in place); dv [*, hd] float32 or bfloat16 token rows,
    row ti*dv_step_rows + p*C + t; krec from phase1; workspace from alloc_dw_workspace (optional:
    without it every group is walked by one team of lanes); snapshot (optional) [*, hd] in the bank
    dtype, or bfloat16 with a float32 bank (rows rounded to bfloat16): row ti*snap_step_rows + p*C*W + j
    receives the pre-write row of the group whose FIRST is at K-row position j, or, with snap_ord (the
    Phase-1 output gord_k), row ti*snap_step_rows + p*C*W + (the group's dense ordinal). noalloc:
    step through sdm_dw_step_noalloc (the split workspace is the library's fixed device array; no
    workspace argument). The plan keeps the tensors alive."""

    def __init__(self, bank, dv, krec, shape: P1Shape, dv_step_rows: int, workspace=None, snapshot=None,
                 snap_step_rows: int = 0, snap_ord=None, noalloc: bool = False):
        import torch

        if noalloc and workspace is not None:
            raise ValueError("DwPlan: noalloc uses the library's fixed workspace; pass no workspace")
        self._noalloc = bool(noalloc)

        if bank.dtype not in (torch.float32, torch.bfloat16) or dv.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("DwPlan: bank and dv must be float32 or bfloat16")
        self._lib = _lib.load()
        self._keep = (bank, dv, krec, workspace, snapshot, snap_ord)
        if snapshot is not None and (snapshot.shape[1] != bank.shape[1] or not (
                snapshot.dtype == bank.dtype or (snapshot.dtype == torch.bfloat16 and bank.dtype == torch.float32))):
            raise TypeError("DwPlan: the snapshot must be [*, hd] in the bank dtype, or bfloat16 for a float32 bank")
        io = _lib.DwIO()
        io.bank = bank.data_ptr()
        io.bank_dtype = _lib.SDM_BF16 if bank.dtype == torch.bfloat16 else _lib.SDM_F32
        io.rows = bank.shape[0]
        io.hd = bank.shape[1]
        io.dv = dv.data_ptr()
        io.dv_dtype = _lib.SDM_BF16 if dv.dtype == torch.bfloat16 else _lib.SDM_F32
        io.dv_step_rows = int(dv_step_rows)
        io.dv_rows = dv.shape[0]
        io.krec = krec.data_ptr()
        io.P, io.C, io.W, io.N = shape.P, shape.C, shape.W, shape.N
        if workspace is not None:
            io.workspace = workspace.data_ptr()
            io.workspace_bytes = workspace.numel() * workspace.element_size()
        if snapshot is not None:
            io.snap = snapshot.data_ptr()
            io.snap_step_rows = int(snap_step_rows)
            io.snap_rows = snapshot.shape[0]
            io.snap_dtype = _lib.SDM_BF16 if snapshot.dtype == torch.bfloat16 else _lib.SDM_F32
            if snap_ord is not None:
                if snap_ord.dtype != torch.int32 or snap_ord.numel() != krec.shape[0] * krec.shape[1]:
                    raise TypeError("DwPlan: snap_ord must be the int32 [N, C*W] gord_k of these records")
                io.snap_ord = snap_ord.data_ptr()
        self.io = io
        self._io_ref = ctypes.byref(io)
        self._device = bank.device

    def step(self, ti: int, stream=None, events=None):
        """Enqueue step `ti` (chunks ti*P .. ti*P+P-1) on the current (or given) stream. events:
        optional (start, end) torch.cuda.Event pair bound to the kernel's own start and end."""
        import torch

        st = torch.cuda.current_stream(self._device) if stream is None else stream
        arr = _event_array(events, 2, "DwPlan.step")
        self.io.events = None if arr is None else ctypes.cast(arr, ctypes.c_void_p).value
        try:
            fn = self._lib.sdm_dw_step_noalloc if self._noalloc else self._lib.sdm_dw_step
            _lib.check(fn(self._io_ref, int(ti), ctypes.c_void_p(st.cuda_stream)))
        finally:
            self.io.events = None


def dw_step(bank, dv, krec, shape: P1Shape, ti: int, dv_step_rows: int, stream=None, workspace=None, events=None):
    """One DW step `ti` through a plan built for this call (see DwPlan)."""
    DwPlan(bank, dv, krec, shape, dv_step_rows, workspace).step(ti, stream=stream, events=events)


class ReadPlan:
    """The read side of a step planned once, launched per step (before that step's DW).

    bank [rows, hd] float32 or bfloat16, the memory before the step (read only); p1: the dict of
    Phase-1 outputs (k_eff, q_w: float32 or bfloat16; a, qk); k_idx / q_idx the Phase-1 id inputs; v [*, hd] float32 value
    rows and beta [N, C] float32; dv, pred, read [*, hd] float32 outputs (dv feeds DwPlan with
    dv_step_rows = step_rows). Row of (step ti, stream p, token t): ti*step_rows + p*C + t. The plan
    keeps the tensors alive."""

    def __init__(self, bank, p1, k_idx, q_idx, v, beta, dv, pred, read, shape: P1Shape, step_rows: int):
        import torch

        if bank.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("ReadPlan: bank must be float32 or bfloat16")
        for name, t in (("v", v), ("beta", beta), ("dv", dv), ("pred", pred), ("read", read)):
            if t.dtype != torch.float32:
                raise TypeError("ReadPlan: %s must be float32" % name)
        self._lib = _lib.load()
        self._keep = (bank, p1, k_idx, q_idx, v, beta, dv, pred, read)
        io = _lib.ReadIO()
        io.bank = bank.data_ptr()
        io.bank_dtype = _lib.SDM_BF16 if bank.dtype == torch.bfloat16 else _lib.SDM_F32
        io.rows = bank.shape[0]
        io.hd = bank.shape[1]
        io.k_idx, io.q_idx = k_idx.data_ptr(), q_idx.data_ptr()
        io.k_eff, io.q_w, io.a, io.qk = (p1[k].data_ptr() for k in ("k_eff", "q_w", "a", "qk"))
        io.v, io.beta, io.dv, io.pred, io.read = v.data_ptr(), beta.data_ptr(), dv.data_ptr(), pred.data_ptr(), read.data_ptr()
        io.step_rows = int(step_rows)
        io.out_rows = min(v.shape[0], dv.shape[0], pred.shape[0], read.shape[0])
        io.P, io.C, io.W, io.R, io.N = shape.P, shape.C, shape.W, shape.R, shape.N
        io.first_partial, io.valid_last = shape.first_partial, shape.valid_last
        io.idx_bytes = k_idx.element_size()
        if p1["k_eff"].dtype != p1["q_w"].dtype or p1["k_eff"].dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("ReadPlan: k_eff and q_w must both be float32 or both bfloat16")
        io.val_bytes = p1["k_eff"].element_size()
        if q_idx.dtype != k_idx.dtype or k_idx.dtype not in (torch.int32, torch.int64):
            raise TypeError("ReadPlan: k_idx and q_idx must both be int32 or both int64")
        self.io = io
        self._io_ref = ctypes.byref(io)
        self._device = bank.device

    def step(self, ti: int, stream=None, events=None):
        """Enqueue the read side of step `ti` on the current (or given) stream. events: optional 4
        torch.cuda.Events bound to the gather kernel's and the substitution kernel's start and end."""
        import torch

        st = torch.cuda.current_stream(self._device) if stream is None else stream
        arr = _event_array(events, 4, "ReadPlan.step")
        self.io.events = None if arr is None else ctypes.cast(arr, ctypes.c_void_p).value
        try:
            _lib.check(self._lib.sdm_read_step(self._io_ref, int(ti), ctypes.c_void_p(st.cuda_stream)))
        finally:
            self.io.events = None


def read_step(bank, p1, k_idx, q_idx, v, beta, dv, pred, read, shape: P1Shape, ti: int, step_rows: int, stream=None):
    """The read side of step `ti` through a plan built for this call (see ReadPlan)."""
    ReadPlan(bank, p1, k_idx, q_idx, v, beta, dv, pred, read, shape, step_rows).step(ti, stream=stream)


def gds_workspace_bytes(shape: P1Shape, hd: int) -> int:
    """Bytes of the (zero-filled) GDS workspace that lets long read groups be split across waves."""
    io = _lib.GdsIO()
    io.P, io.C, io.R, io.N, io.hd = shape.P, shape.C, shape.R, shape.N, int(hd)
    return int(_lib.load().sdm_gds_workspace(ctypes.byref(io)))


def alloc_gds_workspace(shape: P1Shape, hd: int, device="cuda"):
    """A zero-filled GDS workspace (reusable by every step of the same shape)."""
    import torch

    return torch.zeros(max(gds_workspace_bytes(shape, hd), 1), dtype=torch.uint8, device=device)


def gds_step(bank, p1, q_idx, gr, shape: P1Shape, ti: int, step_rows: int, d_q_w=None, grad=None, stream=None,
             workspace=None):
    """GDS of step `ti` (the backward of the read gather) on the current (or given) stream.

    bank [rows, hd] float32 or bfloat16, the memory before the step (read only); p1: the Phase-1
    outputs (q_w, spay_q); q_idx the Phase-1 read ids; gr [*, hd] float32 gradient rows of the reads,
    row ti*step_rows + p*C + t. d_q_w [N, C, R] float32 (optional) receives the dots of the step's
    chunks; grad [rows, hd] float32 or bfloat16 (optional) gains each read slot's sum in place.
    workspace (optional, alloc_gds_workspace): long read groups are split across waves."""
    import torch

    for name, t in (("gr", gr), ("d_q_w", d_q_w)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("gds_step: %s must be float32" % name)
    for name, t in (("bank", bank), ("grad", grad)):
        if t is not None and t.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("gds_step: %s must be float32 or bfloat16" % name)
    if grad is not None and tuple(grad.shape) != tuple(bank.shape):
        raise TypeError("gds_step: grad must have the bank's shape")
    lib = _lib.load()
    io = _lib.GdsIO()
    io.bank = bank.data_ptr()
    io.bank_dtype = _lib.SDM_BF16 if bank.dtype == torch.bfloat16 else _lib.SDM_F32
    io.rows, io.hd = bank.shape[0], bank.shape[1]
    io.q_idx = q_idx.data_ptr()
    io.q_w = p1["q_w"].data_ptr()
    io.spay_q = p1["spay_q"].data_ptr()
    io.gr = gr.data_ptr()
    io.step_rows, io.gr_rows = int(step_rows), gr.shape[0]
    io.d_q_w = _ptr(d_q_w)
    io.grad = _ptr(grad)
    io.grad_dtype = _lib.SDM_BF16 if (grad is not None and grad.dtype == torch.bfloat16) else _lib.SDM_F32
    io.P, io.C, io.R, io.N = shape.P, shape.C, shape.R, shape.N
    io.first_partial, io.valid_last = shape.first_partial, shape.valid_last
    io.idx_bytes = q_idx.element_size()
    io.val_bytes = p1["q_w"].element_size()
    if workspace is not None:
        io.workspace = workspace.data_ptr()
        io.workspace_bytes = workspace.numel() * workspace.element_size()
    st = torch.cuda.current_stream(bank.device) if stream is None else stream
    _lib.check(lib.sdm_gds_step(ctypes.byref(io), int(ti), ctypes.c_void_p(st.cuda_stream)))


def gwr_step(grad, k_idx, w, dv, shape: P1Shape, ti: int, step_rows: int, d_dv=None, d_k_pd=None, stream=None):
    """GWR of step `ti` (the backward of DW's write terms) on the current (or given) stream.

    grad [rows, hd] float32 or bfloat16 gradient of the bank rows DW wrote; k_idx the Phase-1 write
    ids; w [N, C, W] float32 write weights (k exp(rex) per entry); dv [*, hd] float32 token rows, row
    ti*step_rows + p*C + t. d_dv (same layout as dv) and d_k_pd [N, C, W] (both float32, optional)
    receive the results."""
    import torch

    for name, t in (("w", w), ("dv", dv), ("d_dv", d_dv), ("d_k_pd", d_k_pd)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("gwr_step: %s must be float32" % name)
    if grad.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("gwr_step: grad must be float32 or bfloat16")
    if d_dv is not None and d_dv.shape[0] != dv.shape[0]:
        raise TypeError("gwr_step: d_dv must have dv's rows")
    lib = _lib.load()
    io = _lib.GwrIO()
    io.grad = grad.data_ptr()
    io.grad_dtype = _lib.SDM_BF16 if grad.dtype == torch.bfloat16 else _lib.SDM_F32
    io.rows, io.hd = grad.shape[0], grad.shape[1]
    io.k_idx = k_idx.data_ptr()
    io.w = w.data_ptr()
    io.dv = dv.data_ptr()
    io.step_rows, io.dv_rows = int(step_rows), dv.shape[0]
    io.d_dv = _ptr(d_dv)
    io.d_k_pd = _ptr(d_k_pd)
    io.P, io.C, io.W, io.N = shape.P, shape.C, shape.W, shape.N
    io.first_partial, io.valid_last = shape.first_partial, shape.valid_last
    io.idx_bytes = k_idx.element_size()
    st = torch.cuda.current_stream(grad.device) if stream is None else stream
    _lib.check(lib.sdm_gwr_step(ctypes.byref(io), int(ti), ctypes.c_void_p(st.cuda_stream)))


def pa_workspace_bytes(shape: P1Shape, hd: int) -> int:
    """Bytes of the (zero-filled) PA workspace that lets long write groups be split across waves."""
    io = _lib.PaIO()
    io.P, io.C, io.W, io.N, io.hd = shape.P, shape.C, shape.W, shape.N, int(hd)
    return int(_lib.load().sdm_pa_workspace(ctypes.byref(io)))


def alloc_pa_workspace(shape: P1Shape, hd: int, device="cuda"):
    """A zero-filled PA workspace (reusable by every step of the same shape)."""
    import torch

    return torch.zeros(max(pa_workspace_bytes(shape, hd), 1), dtype=torch.uint8, device=device)


def pa_step(grad, snap, p1, beta, d_dva, shape: P1Shape, ti: int, step_rows: int, snap_step_rows: int, bank=None,
            g_decay=None, d_k_eff=None, stream=None, workspace=None):
    """PA of step `ti` (the backward of DW) on the current (or given) stream.

    grad [rows, hd] float32 or bfloat16 bank gradient, updated in place at the step's written slots;
    snap: the step's compact snapshot from DwPlan (FIRST-position layout, raw rows in the bank dtype);
    p1: the Phase-1 outputs (krec, k_eff); beta [N, C] float32; d_dva [*, hd] float32 gradient token
    rows, row ti*step_rows + p*C + t. bank (optional) gets each written slot's row restored from the
    snapshot; g_decay and d_k_eff [N, C, W] float32 (optional) receive the per-entry gradients.
    workspace (optional, alloc_pa_workspace): long write groups are split across waves."""
    import torch

    for name, t in (("beta", beta), ("d_dva", d_dva), ("g_decay", g_decay), ("d_k_eff", d_k_eff)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("pa_step: %s must be float32" % name)
    if grad.dtype not in (torch.float32, torch.bfloat16) or snap.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("pa_step: grad and snap must be float32 or bfloat16")
    if bank is not None and (bank.dtype != snap.dtype or tuple(bank.shape) != tuple(grad.shape)):
        raise TypeError("pa_step: bank must have grad's shape and the snapshot's dtype")
    lib = _lib.load()
    io = _lib.PaIO()
    io.grad = grad.data_ptr()
    io.grad_dtype = _lib.SDM_BF16 if grad.dtype == torch.bfloat16 else _lib.SDM_F32
    io.bank = _ptr(bank)
    io.bank_dtype = _lib.SDM_BF16 if snap.dtype == torch.bfloat16 else _lib.SDM_F32
    io.rows, io.hd = grad.shape[0], grad.shape[1]
    io.snap = snap.data_ptr()
    io.snap_step_rows, io.snap_rows = int(snap_step_rows), snap.shape[0]
    io.krec = p1["krec"].data_ptr()
    io.k_eff = p1["k_eff"].data_ptr()
    io.beta = beta.data_ptr()
    io.d_dva = d_dva.data_ptr()
    io.step_rows, io.dva_rows = int(step_rows), d_dva.shape[0]
    io.g_decay = _ptr(g_decay)
    io.d_k_eff = _ptr(d_k_eff)
    io.P, io.C, io.W, io.N = shape.P, shape.C, shape.W, shape.N
    io.val_bytes = p1["k_eff"].element_size()
    if workspace is not None:
        io.workspace = workspace.data_ptr()
        io.workspace_bytes = workspace.numel() * workspace.element_size()
    st = torch.cuda.current_stream(grad.device) if stream is None else stream
    _lib.check(lib.sdm_pa_step(ctypes.byref(io), int(ti), ctypes.c_void_p(st.cuda_stream)))
