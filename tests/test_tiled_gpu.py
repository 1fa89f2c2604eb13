"""GPU parity of the tiled Phase-1 path (rows longer than 16384 entries, up to 2^17, or any row with
shape.tiled = 1) against the CPU oracle, and its agreement with the on-chip path.

Long rows: every Phase-1 output against the oracle (integers bit for bit, floats within
max(1e-5 |o|, 1e-6); the A / QK cells too), then the DW steps that consume their records. Forced on
short rows: every integer output (sorted order, packed positions, kind rows, record words, flags,
tile bounds, repeats, group ordinals) equals the on-chip path's bit for bit, and the float outputs
meet the oracle's tolerance. The path is bitwise reproducible run to run.
"""

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_delta_memory_amd import workloads as W  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
import hip_harness as H  # noqa: E402


def say(*a):
    print(*a, flush=True)


def long_wl(case, seed):
    sh = W.Shape("tiled", P=case["P"], T=case["C"] * case["steps"], C=case["C"], W=case["W"], R=case["R"],
                 S=case["S"], hd=case.get("hd", 64), bank_dtype=case.get("bank", "bf16"), dv_dtype="f32",
                 slots="uniform", valid_last=case.get("vl"))
    wl = W.make(sh, seed=seed, lane_gates=case.get("lg", False), val_bf16=case.get("bf", False))
    if case.get("id64", False):
        import dataclasses

        wl = dataclasses.replace(wl, k_idx=wl.k_idx.astype(np.int64), q_idx=wl.q_idx.astype(np.int64))
    return wl


@pytest.mark.parametrize("case", [
    dict(C=256, W=48, R=48, S=20000, P=1, steps=1),                 # 24576 entries: two tiles
    dict(C=256, W=48, R=48, S=300, P=2, steps=2, vl=200),           # hot groups of ~40 K entries, ragged
    dict(C=128, W=96, R=64, S=5000, P=2, steps=1, lg=True, bf=True, id64=True),   # per-lane gates, bf16, int64
    dict(C=256, W=256, R=256, S=1 << 20, P=1, steps=1, hd=32),      # the longest row, 2^17 entries
])
def test_long_rows_match_oracle(case):
    wl = long_wl(case, seed=801)
    say("tiled long row", case, "n =", wl.shape.C * (wl.shape.W + wl.shape.R))
    shape, out = H.run_phase1(wl, fields=["perm", "gord_k"])
    chunks = list(range(wl.N))
    ref = H.oracle_phase1(wl, chunks, fields=None)
    H.compare_phase1(out, ref, chunks)
    ref_p = H.oracle_phase1(wl, chunks, fields=["perm", "gord_k"])
    H.assert_exact("perm", out["perm"].cpu().numpy(), ref_p["perm"])
    H.assert_exact("gord_k", out["gord_k"].cpu().numpy(), ref_p["gord_k"])
    H.run_dw_check(wl, out, shape, set(range(wl.steps)), sample_untouched=0)


INTEGER_FIELDS = ("is_last", "is_only", "pos_k", "q_last", "q_only", "pos_q", "spay_k", "spay_q", "tiles_k", "repeats",
                  "perm", "gord_k")


@pytest.mark.parametrize("idx,steps", [(0, None), (1, 2), (2, 1), (4, 1)])
def test_forced_tiled_matches_onchip(idx, steps):
    wl = W.make(idx, steps=steps)
    say("tiled forced on workload", idx)
    _, chip = H.run_phase1(wl, fields=["perm", "gord_k"])
    _, tiled = H.run_phase1(wl, fields=["perm", "gord_k"], tiled=True)
    for k in INTEGER_FIELDS:
        assert torch.equal(chip[k], tiled[k]), k
    assert torch.equal(chip["krec"][..., :2], tiled["krec"][..., :2]), "krec element and slot"
    chunks = sorted({0, wl.N // 2, wl.N - 1})
    ref = H.oracle_phase1(wl, chunks)
    H.compare_phase1(tiled, ref, chunks)


def test_tiled_bitwise_reproducible():
    wl = long_wl(dict(C=256, W=48, R=48, S=300, P=2, steps=1, vl=200), seed=802)
    say("tiled reproducibility")
    _, o1 = H.run_phase1(wl, fields=["perm"])
    _, o2 = H.run_phase1(wl, fields=["perm"])
    for k in o1:
        assert torch.equal(o1[k].view(torch.uint8), o2[k].view(torch.uint8)), k
