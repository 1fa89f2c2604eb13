"""GPU parity of the forward read side (sdm_read_step) against the float64 oracle (oracle/read_side.py).

Per checked step the GPU and the oracle start from the same pre-step bank: the workload's seeded
initial bank (the read side is defined for any pre-step memory). The oracle works from its own
Phase-1 quantities, never from the GPU's. Tolerance: the outputs are float32 evaluations of linear
recursions whose inputs (the GPU's float32 Phase-1 fields) carry at most 1e-5 relative error; each
output element is compared against 1e-4 times the oracle's magnitude bound (the same recursion on
absolute values) plus 1e-6 (hip_harness.run_read_check).
"""

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_delta_memory_amd as sdm  # noqa: E402
from sparse_delta_memory_amd import workloads as W  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
import hip_harness as H  # noqa: E402

def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("idx,steps,checked", [(0, None, [0, 3]), (1, 2, [0, 1]), (4, 2, [1]), (2, 1, [0]), (3, 1, [0])])
def test_read_side_matches_oracle(idx, steps, checked):
    wl = W.make(idx, steps=steps)
    say("read side: workload", idx, "steps", checked)
    worst = H.run_read_check(wl, checked, chunks_per_step=4)
    say("worst relative-to-magnitude error %.3g" % worst)


@pytest.mark.parametrize("case", [
    dict(C=37, W=5, R=3, S=9, P=2, steps=2, vl=11),       # heavy sharing, ragged row and chunk
    dict(C=256, W=8, R=8, S=48, P=1, steps=1, vl=None),   # every group hot: dense A and QK
    dict(C=1, W=1, R=1, S=4, P=1, steps=2, vl=None),      # one token
    dict(C=64, W=4, R=3, S=40, P=2, steps=2, vl=21, hd=37, bank="bf16"),   # head dims 8 does not divide
    dict(C=96, W=8, R=8, S=64, P=1, steps=1, vl=None, hd=1, bank="f32"),
    dict(C=128, W=4, R=4, S=300, P=1, steps=1, vl=None, hd=100, bank="f32"),
])
def test_read_side_edge_shapes(case):
    sh = W.Shape("read_edge", P=case["P"], T=case["C"] * case["steps"], C=case["C"], W=case["W"], R=case["R"],
                 S=case["S"], hd=case.get("hd", 64), bank_dtype=case.get("bank", "f32"), dv_dtype="f32",
                 slots="uniform", valid_last=case["vl"])
    wl = W.make(sh, seed=779)
    say("read side edge", case)
    H.run_read_check(wl, list(range(wl.steps)))


def test_read_side_feeds_dw_reproducibly():
    """A forward step loop (read side, then DW, step after step) is bitwise reproducible run to run,
    and its token rows are finite."""
    wl = W.make(1, steps=3)
    sh = wl.shape
    P, C, hd = sh.P, sh.C, sh.hd
    shape, out = H.run_phase1(wl)
    ins = H.device_inputs(wl)
    v_host, beta_host = W.make_read_inputs(wl)
    res = []
    for _ in range(2):
        v = torch.from_numpy(v_host).cuda()
        beta = torch.from_numpy(beta_host).cuda()
        dv = torch.zeros((v.shape[0], hd), device="cuda")
        pred, read = torch.zeros_like(dv), torch.zeros_like(dv)
        bank = W.make_bank(wl, "cuda")
        rp = sdm.ReadPlan(bank, out, ins["k_idx"], ins["q_idx"], v, beta, dv, pred, read, shape, step_rows=P * C)
        dp = sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=P * C)
        for ti in range(wl.steps):
            rp.step(ti)
            dp.step(ti)
        torch.cuda.synchronize()
        assert torch.isfinite(dv).all() and torch.isfinite(read).all()
        res.append((bank.clone(), dv.clone(), read.clone()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("idx,steps", [(1, 1), (4, 1)])
def test_read_side_bf16_weights(idx, steps):
    """bfloat16 k_eff / q_w (bfloat16 values): the read side gives bitwise the results it gives for
    the same weights widened to float32 (the float32-weight path is checked against the oracle
    above), and those are finite for the valid tokens."""
    wl = W.make(idx, steps=steps, val_bf16=True)
    sh = wl.shape
    P, C, hd = sh.P, sh.C, sh.hd
    shape, out = H.run_phase1(wl)
    assert out["k_eff"].dtype == torch.bfloat16
    ins = H.device_inputs(wl)
    v_host, beta_host = W.make_read_inputs(wl)
    v = torch.from_numpy(v_host).cuda()
    beta = torch.from_numpy(beta_host).cuda()
    say("read side bf16 weights", idx, steps)
    res = []
    for p1 in (out, {**out, "k_eff": out["k_eff"].float(), "q_w": out["q_w"].float()}):
        dv = torch.zeros((v.shape[0], hd), device="cuda")
        pred, read = torch.zeros_like(dv), torch.zeros_like(dv)
        bank = W.make_bank(wl, "cuda")
        plan = sdm.ReadPlan(bank, p1, ins["k_idx"], ins["q_idx"], v, beta, dv, pred, read, shape, step_rows=P * C)
        for ti in range(wl.steps):
            plan.step(ti)
        torch.cuda.synchronize()
        res.append((dv, pred, read))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.isfinite(res[0][0]).all() and torch.isfinite(res[0][2]).all()   # (masked tokens: 0)


@pytest.mark.parametrize("idx,steps,checked,case", [
    (0, None, [0, 3], None), (1, 2, [1], None), (2, 1, [0], None), (3, 1, [0], None), (4, 64, [63], None),
    (None, 2, [0, 1], dict(C=37, W=5, R=3, S=9, P=2, vl=11)),             # heavy sharing, ragged
    (None, 1, [0], dict(C=256, W=8, R=8, S=48, P=1, vl=None)),            # dense A and QK
    (None, 2, [0, 1], dict(C=64, W=4, R=3, S=40, P=2, vl=21, hd=37, bank="bf16")),
])
def test_read_side_oracle_fed(idx, steps, checked, case):
    """The read kernels alone: fed the oracle's float32-rounded k_eff, q_w, A and QK, dv / pred /
    read are within the float32 evaluation bound of the oracle's float64 read side on those same
    inputs (hip_harness.read_fed_tolerance), so no Phase-1 error is in the comparison."""
    if case is None:
        wl = W.make(idx, steps=steps)
    else:
        sh = W.Shape("read_fed", P=case["P"], T=case["C"] * steps, C=case["C"], W=case["W"], R=case["R"],
                     S=case["S"], hd=case.get("hd", 64), bank_dtype=case.get("bank", "f32"), dv_dtype="f32",
                     slots="uniform", valid_last=case["vl"])
        wl = W.make(sh, seed=785)
    say("read side, oracle-fed:", idx, case, "steps", checked)
    worst = H.run_read_check_fed(wl, checked)
    say("worst error as a fraction of the bound %.3g" % worst)
