"""GPU parity of GDS (sdm_gds_step, the backward of the read gather) against the float64 oracle
(oracle/gds.py).

Inputs: the workload's Phase-1 outputs from the GPU path (q_w, spay_q) and, on the oracle side,
the oracle's own q_w; the pre-step memory is the workload's seeded initial bank; gradient rows of
the reads (seeded on the host; masked tokens' rows NaN: they must not be read) and the initial grad
rows (seeded, drawn on the device and read back as the oracle's input).
Tolerances: a dot of hd float32 products within (hd + 8) 2^-23 sum |g m| + 1e-6; a grad row within
(m + 4) 2^-23 (|grad0| + sum |q_w g|) + 1e-5 sum |q_w g| (m members; q_w carries at most 1e-5
relative error from Phase 1), plus one bf16 ulp for a bf16 grad. Untouched grad rows keep their bits.
With a workspace (read groups of more than 32 members summed in segments) the same bound holds: a
term passes through at most its segment's chain, the segment additions and the final add.
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
from oracle import gds  # noqa: E402
from sparse_delta_memory_amd import workloads as W  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
import hip_harness as H  # noqa: E402


def say(*a):
    print(*a, flush=True)


def gds_inputs(wl, grad_dtype):
    sh = wl.shape
    rng = np.random.default_rng(wl.bank_seed + 17)
    gr = rng.standard_normal((wl.steps * sh.P * sh.C, sh.hd), dtype=np.float32)
    if wl.valid_last < sh.C:
        gr.reshape(wl.steps, sh.P, sh.C, sh.hd)[wl.steps - 1, :, wl.valid_last:, :] = np.nan
    gen = torch.Generator(device="cuda")   # (banks reach tens of GB: drawn on the device)
    gen.manual_seed(wl.bank_seed + 19)
    g0 = (torch.randn((wl.rows, sh.hd), generator=gen, device="cuda") * 0.01).to(grad_dtype)
    return gr, g0


@pytest.mark.parametrize("case", [
    dict(idx=0, steps=None, checked=[0, 3]),
    dict(idx=1, steps=2, checked=[0, 1]),
    dict(idx=2, steps=1, checked=[0]),                  # Zipf: long read groups
    dict(idx=4, steps=2, checked=[1]),                  # ragged last step
    dict(shape=dict(C=37, W=5, R=3, S=9, P=2, vl=11, hd=36), steps=2, checked=[0, 1], val_bf16=True),
    dict(idx=3, steps=1, checked=[0]),                  # hd = 960: the dots' column loop, multi-block scatter
    # With a workspace: read groups of more than 32 members are split into segments.
    dict(idx=2, steps=1, checked=[0], ws=True),         # Zipf: hot slots read hundreds of times
    dict(idx=3, steps=1, checked=[0], ws=True),         # hd = 960: every column block of a split group
    dict(shape=dict(C=37, W=5, R=3, S=9, P=2, vl=11, hd=36), steps=2, checked=[0, 1], ws=True),
    # One read group of 4352 members: the in-group distance saturates, the segment starting at 4064
    # runs to the group's end.
    dict(shape=dict(C=256, W=2, R=17, S=1, P=1, vl=None, hd=64), steps=1, checked=[0], ws=True),
    # One slot per chunk and a fully masked last chunk.
    dict(shape=dict(C=64, W=2, R=2, S=1, P=1, vl=0, hd=40), steps=2, checked=[0, 1], ws=True),
])
def test_gds_matches_oracle(case):
    if "shape" in case:
        c = case["shape"]
        shp = W.Shape("gds_edge", P=c["P"], T=c["C"] * case["steps"], C=c["C"], W=c["W"], R=c["R"], S=c["S"],
                      hd=c["hd"], bank_dtype="f32", dv_dtype="f32", slots="uniform", valid_last=c["vl"])
        wl = W.make(shp, seed=787, val_bf16=case.get("val_bf16", False))
    else:
        wl = W.make(case["idx"], steps=case["steps"])
    sh = wl.shape
    P, C, R, hd = sh.P, sh.C, sh.R, sh.hd
    say("gds", case)
    shape, out = H.run_phase1(wl)
    ins = H.device_inputs(wl)
    bank = W.make_bank(wl, "cuda")
    grad_dtype = bank.dtype
    gr_host, grad0 = gds_inputs(wl, grad_dtype)
    gr = torch.from_numpy(gr_host).cuda()
    for ti in case["checked"]:
        d = torch.full((wl.N, C, R), float("nan"), device="cuda")
        grad = grad0.clone()
        ws = sdm.alloc_gds_workspace(shape, hd) if case.get("ws") else None
        sdm.gds_step(bank, out, ins["q_idx"], gr, shape, ti, step_rows=P * C, d_q_w=d, grad=grad, workspace=ws)
        torch.cuda.synchronize()
        if ws is not None:   # the arrival counters are back at zero
            assert not ws[:-(-P * C * R // 32) * 4].any()
        touched = []
        for p in range(P):
            cidx = ti * P + p
            tv = wl.valid_last if cidx >= wl.first_partial else C
            o = H.oracle_phase1(wl, [cidx], fields=["q_w"])
            rows_of = lambda s: bank.index_select(0, torch.as_tensor(s, device="cuda")).float().cpu().numpy().astype(np.float64)  # noqa: E731
            g_rows = gr_host[ti * P * C + p * C: ti * P * C + (p + 1) * C].astype(np.float64)
            dots, slots, add, mag = gds.gds_chunk(wl.q_idx[cidx], o["q_w"][0], g_rows, rows_of, tv)
            # dots
            got = d[cidx].cpu().numpy().astype(np.float64)
            dmag = np.zeros_like(dots)
            for t in range(tv):
                m0 = rows_of(wl.q_idx[cidx][t])
                dmag[t] = np.abs(m0) @ np.abs(g_rows[t])
            tol = (hd + 8) * 2.0 ** -23 * dmag + 1e-6
            bad = ~(np.abs(got - dots) <= tol)
            assert not bad.any(), ("dots", ti, p, np.argwhere(bad)[:3], got[bad][:3], dots[bad][:3])
            # grad rows
            if len(slots):
                sidx = torch.as_tensor(slots, device="cuda")
                g_new = grad.index_select(0, sidx).float().cpu().numpy().astype(np.float64)
                g_old = grad0.index_select(0, sidx).float().cpu().numpy().astype(np.float64)
                want = g_old + add
                members = np.array([(wl.q_idx[cidx][:tv] == s).sum() for s in slots], np.float64)[:, None]
                tol = (members + 4) * 2.0 ** -23 * (np.abs(g_old) + mag) + 1e-5 * mag
                if grad_dtype == torch.bfloat16:
                    tol = tol + H.ulp_bf16(np.maximum(np.abs(g_new), np.abs(want)))
                bad = ~(np.abs(g_new - want) <= tol)
                assert not bad.any(), ("grad", ti, p, int(bad.sum()), g_new[bad][:3], want[bad][:3])
                touched.append(slots)
        # rows no read of the step names keep their bits
        hit = np.unique(np.concatenate(touched)) if touched else np.zeros(0, np.int64)
        rng = np.random.default_rng(ti)
        cand = rng.integers(0, wl.rows, size=4000)
        cand = np.setdiff1d(cand, hit)
        if cand.size:
            ci = torch.as_tensor(cand, device="cuda")
            assert torch.equal(grad.index_select(0, ci).view(torch.uint8), grad0.index_select(0, ci).view(torch.uint8))


@pytest.mark.parametrize("split", [False, True])
def test_gds_reproducible(split):
    """Two runs of the same step give the same bytes (sorted-order sums, one writer per row; with a
    workspace, the long groups' partial rows added in segment order whichever segment finishes last,
    the second run reusing the workspace the first left)."""
    wl = W.make(2, steps=1)
    sh = wl.shape
    shape, out = H.run_phase1(wl)
    ins = H.device_inputs(wl)
    bank = W.make_bank(wl, "cuda")
    gr_host, grad0 = gds_inputs(wl, bank.dtype)
    gr = torch.from_numpy(gr_host).cuda()
    ws = sdm.alloc_gds_workspace(shape, sh.hd) if split else None
    res = []
    for _ in range(2):
        d = torch.zeros((wl.N, sh.C, sh.R), device="cuda")
        grad = grad0.clone()
        sdm.gds_step(bank, out, ins["q_idx"], gr, shape, 0, step_rows=sh.P * sh.C, d_q_w=d, grad=grad, workspace=ws)
        torch.cuda.synchronize()
        res.append((d, grad))
    assert torch.equal(res[0][0].view(torch.int32), res[1][0].view(torch.int32))
    assert torch.equal(res[0][1].view(torch.uint8), res[1][1].view(torch.uint8))
