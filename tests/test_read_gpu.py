"""GPU parity of the forward read side (sdm_read_step) against the float64 oracle (oracle/read_side.py).

Per checked step the GPU and the oracle start from the same pre-step bank: the workload's seeded
initial bank (the read side is defined for any pre-step memory). The oracle works from its own
Phase-1 quantities, never from the GPU's. Tolerance: the outputs are float32 evaluations of linear
recursions whose inputs (the GPU's float32 Phase-1 fields) carry at most 1e-5 relative error; each
output element is compared against RTOL_MAG times the oracle's magnitude bound (the same recursion
on absolute values) plus 1e-6.
"""

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
import sparse_delta_memory_amd as sdm  # noqa: E402
from oracle import read_side  # noqa: E402
from sparse_delta_memory_amd import workloads as W  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
import hip_harness as H  # noqa: E402

RTOL_MAG = 1e-4


def say(*a):
    print(*a, flush=True)


def run_read(wl, steps_checked, chunks_per_step=None):
    """Phase 1, then the read side of the checked steps from the initial bank; compare with the oracle."""
    sh = wl.shape
    P, C, hd = sh.P, sh.C, sh.hd
    shape, out = H.run_phase1(wl)
    ins = H.device_inputs(wl)
    v_host, beta_host = W.make_read_inputs(wl)
    v = torch.from_numpy(v_host).cuda()
    beta = torch.from_numpy(beta_host).cuda()
    rows = v.shape[0]
    dv = torch.full((rows, hd), float("nan"), device="cuda")
    pred = torch.full_like(dv, float("nan"))
    read = torch.full_like(dv, float("nan"))
    bank = W.make_bank(wl, "cuda")
    plan = sdm.ReadPlan(bank, out, ins["k_idx"], ins["q_idx"], v, beta, dv, pred, read, shape, step_rows=P * C)
    for ti in steps_checked:
        plan.step(ti)
    torch.cuda.synchronize()
    worst = 0.0
    for ti in steps_checked:
        for p in range(P) if chunks_per_step is None else range(min(P, chunks_per_step)):
            c = ti * P + p
            o = H.oracle_phase1(wl, [c], fields=["k_eff", "q_w", "a", "qk"])
            tv = wl.valid_last if c >= wl.first_partial else C
            rows_of = lambda s: bank.index_select(0, torch.as_tensor(s, device="cuda")).float().cpu().numpy().astype(np.float64)  # noqa: E731
            r = read_side.read_step(wl.k_idx[c], wl.q_idx[c], o["k_eff"][0], o["q_w"][0], o["a"][0], o["qk"][0],
                                    v_host[c * C:(c + 1) * C], beta_host[c], rows_of, tv)
            sl = slice(ti * P * C + p * C, ti * P * C + (p + 1) * C)
            for name, got in (("dv", dv), ("pred", pred), ("read", read)):
                g = got[sl].cpu().numpy().astype(np.float64)
                want = r[name]
                tol = RTOL_MAG * r["mag_" + name] + 1e-6
                err = np.abs(g - want)
                bad = ~(err <= tol)
                if bad.any():
                    i = np.argwhere(bad)[:4]
                    raise AssertionError("%s step %d stream %d: %d of %d outside tolerance; e.g. %s" % (
                        name, ti, p, bad.sum(), bad.size,
                        ", ".join("%s gpu %r oracle %r mag %r" % (tuple(k), g[tuple(k)], want[tuple(k)],
                                                                 r["mag_" + name][tuple(k)]) for k in i)))
                worst = max(worst, float(np.max(err / (r["mag_" + name] + 1e-300))))
                # masked tokens: exactly zero
                assert np.all(g[tv:] == 0), name
    return worst


@pytest.mark.parametrize("idx,steps,checked", [(0, None, [0, 3]), (1, 2, [0, 1]), (4, 2, [1]), (2, 1, [0]), (3, 1, [0])])
def test_read_side_matches_oracle(idx, steps, checked):
    wl = W.make(idx, steps=steps)
    say("read side: workload", idx, "steps", checked)
    worst = run_read(wl, checked, chunks_per_step=4)
    say("worst relative-to-magnitude error %.3g" % worst)


@pytest.mark.parametrize("case", [
    dict(C=37, W=5, R=3, S=9, P=2, steps=2, vl=11),       # heavy sharing, ragged row and chunk
    dict(C=256, W=8, R=8, S=48, P=1, steps=1, vl=None),   # every group hot: dense A and QK
    dict(C=1, W=1, R=1, S=4, P=1, steps=2, vl=None),      # one token
])
def test_read_side_edge_shapes(case):
    sh = W.Shape("read_edge", P=case["P"], T=case["C"] * case["steps"], C=case["C"], W=case["W"], R=case["R"],
                 S=case["S"], hd=64, bank_dtype="f32", dv_dtype="f32", slots="uniform", valid_last=case["vl"])
    wl = W.make(sh, seed=779)
    say("read side edge", case)
    run_read(wl, list(range(wl.steps)))


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
