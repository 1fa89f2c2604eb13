"""The allocation-free DW entry point (sdm_dw_step_noalloc) against sdm_dw_step with an allocated
workspace: the same bits, on two calls in a row (the second with a smaller input), and the size
limit refused before anything is enqueued.

sdm_dw_step_noalloc keeps the split-group workspace in a fixed device array of the library; the
comparison is with the existing entry point, which is itself checked against the oracle by
tests/test_parity_gpu.py.
"""

import ctypes
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_delta_memory_amd as sdm  # noqa: E402
from sparse_delta_memory_amd import _lib  # noqa: E402
from sparse_delta_memory_amd import workloads as W  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
import hip_harness as H  # noqa: E402


def say(*a):
    print(*a, flush=True)


def run_both(wl, steps):
    shape, out = H.run_phase1(wl)
    dv = H.device_dv(wl)
    sh = wl.shape
    bank0 = W.make_bank(wl, "cuda")
    a, b = bank0.clone(), bank0.clone()
    ref = sdm.DwPlan(a, dv, out["krec"], shape, dv_step_rows=sh.P * sh.C,
                     workspace=sdm.alloc_dw_workspace(shape, sh.hd, device="cuda"))
    nal = sdm.DwPlan(b, dv, out["krec"], shape, dv_step_rows=sh.P * sh.C, noalloc=True)
    for ti in range(steps):
        ref.step(ti)
        nal.step(ti)
    torch.cuda.synchronize()
    return a, b


def test_noalloc_matches_workspace_entry_point():
    # First call: the Zipf workload (hot slots: groups of hundreds of members, split into segments).
    wl = W.make(2, steps=2)
    say("noalloc: workload 2, 2 steps")
    a, b = run_both(wl, wl.steps)
    assert torch.equal(a.view(torch.uint16), b.view(torch.uint16))
    # Second call, smaller: a ragged shape with long groups in few slots and a tail head dim.
    sh = W.Shape("noalloc_small", P=2, T=64 * 2, C=64, W=6, R=2, S=8, hd=37, bank_dtype="bf16", dv_dtype="f32",
                 slots="uniform", valid_last=50)
    wl = W.make(sh, seed=790)
    say("noalloc: small ragged shape")
    a, b = run_both(wl, wl.steps)
    assert torch.equal(a.view(torch.uint16), b.view(torch.uint16))
    # And the uniform shape (one-member groups): the same bits again.
    wl = W.make(1, steps=2)
    say("noalloc: workload 1, 2 steps")
    a, b = run_both(wl, wl.steps)
    assert torch.equal(a.view(torch.uint16), b.view(torch.uint16))


def test_noalloc_refuses_oversized_steps():
    """Steps whose partial rows exceed the fixed array are refused on the host (nothing enqueued)."""
    lib = _lib.load()
    fake = 1 << 20
    io = _lib.DwIO()
    io.bank, io.dv, io.krec = fake, fake, fake
    io.bank_dtype, io.dv_dtype = _lib.SDM_BF16, _lib.SDM_F32
    io.rows, io.hd = 1 << 30, 1024
    io.P, io.C, io.W, io.N = 64, 256, 256, 64
    io.dv_step_rows, io.dv_rows = 0, 1 << 20
    assert lib.sdm_dw_step_noalloc(ctypes.byref(io), 0, None) == _lib.SDM_EWORKSPACE
    assert b"fixed array" in lib.sdm_last_error()
    io.workspace, io.workspace_bytes = fake, 1 << 30
    io.P, io.hd = 1, 128
    assert lib.sdm_dw_step_noalloc(ctypes.byref(io), 0, None) == _lib.SDM_EINVAL
