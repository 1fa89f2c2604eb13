"""GPU parity of PA (sdm_pa_step, the backward of DW) against the float64 oracle (oracle/gds.py,
pa_chunk).

Per checked step: DW of that step alone from the workload's initial bank writes the compact
snapshot (so the pre-write rows are the initial rows); PA then runs with seeded gradient rows
(drawn on the device in the bank dtype), beta and gradient token rows (masked tokens NaN: never
read), and the oracle works from its own Phase-1 k_eff and cpe. Tolerances: a grad row within
(m + 4) 2^-23 mag + 1e-5 mag (+ one bf16 ulp for a bf16 grad), mag = |gdw cpe| + sum |sc d_dva|
(Phase-1 float32 inputs carry 1e-5 relative error); the dots within (hd + 8) 2^-23 of the sum of
|products| plus 1e-5 of it and 1e-6; with bfloat16 values (k_eff, cpe) both add 2^-7 of their
magnitude (either bfloat16 neighbour of the exact value is correct). Restored bank rows equal the
pre-write rows bit for bit; padding entries get zeros; gradient rows of slots the step does not
write keep their bits. With a workspace (long groups split into 32-member segments) the same bounds
hold: a member's term passes through at most its segment's chain and the segment additions, fewer
roundings than the m + 4 the bound allows. PA is also bitwise reproducible run to run.
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
from oracle import gds  # noqa: E402
from sparse_delta_memory_amd import workloads as W  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
import hip_harness as H  # noqa: E402


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("case", [
    dict(idx=0, steps=None, checked=[0, 2]),
    dict(idx=1, steps=2, checked=[1]),
    dict(idx=2, steps=1, checked=[0]),                  # Zipf: long write groups
    dict(idx=4, steps=2, checked=[1]),                  # ragged last step
    dict(shape=dict(C=37, W=5, S=9, P=2, vl=11, hd=36), steps=2, checked=[0, 1]),
    dict(idx=3, steps=1, checked=[0]),                  # hd = 960: every column block of a group's wave
    dict(idx=1, steps=2, checked=[1], val_bf16=True),   # bfloat16 k_eff (and cpe) from Phase 1
    dict(shape=dict(C=37, W=5, S=9, P=2, vl=11, hd=36), steps=2, checked=[1], val_bf16=True),
    # With a workspace: groups of more than 32 members are split into segments.
    dict(idx=2, steps=1, checked=[0], ws=True),         # Zipf: hot slots with hundreds of members
    dict(idx=0, steps=None, checked=[0, 2], ws=True),
    dict(shape=dict(C=37, W=5, S=9, P=2, vl=11, hd=36), steps=2, checked=[0, 1], ws=True),
    # One group of 4352 members: the in-group distance saturates, the segment starting at 4064 runs
    # to the group's end.
    dict(shape=dict(C=256, W=17, S=1, P=1, vl=None, hd=64), steps=1, checked=[0], ws=True),
    # One slot per chunk and a fully masked last chunk.
    dict(shape=dict(C=64, W=2, S=1, P=1, vl=0, hd=40), steps=2, checked=[0, 1], ws=True),
    dict(idx=1, steps=2, checked=[1], val_bf16=True, ws=True),
])
def test_pa_matches_oracle(case):
    vbf = case.get("val_bf16", False)
    if "shape" in case:
        c = case["shape"]
        shp = W.Shape("pa_edge", P=c["P"], T=c["C"] * case["steps"], C=c["C"], W=c["W"], R=2, S=c["S"], hd=c["hd"],
                      bank_dtype="f32", dv_dtype="f32", slots="uniform", valid_last=c["vl"])
        wl = W.make(shp, seed=791, val_bf16=vbf)
    else:
        wl = W.make(case["idx"], steps=case["steps"], val_bf16=vbf)
    # bfloat16 values: the GPU's k_eff and cpe may each be the other bfloat16 neighbour of the exact
    # value (the oracle rounds the exact value), at most one bfloat16 ulp, i.e. 2^-7 of the value;
    # every grad term and decay gradient they scale may move by 2^-7 of its magnitude.
    bf_slack = 2.0 ** -7 if vbf else 0.0
    sh = wl.shape
    P, C, Wn, hd, CW = sh.P, sh.C, sh.W, sh.hd, sh.C * sh.W
    say("pa", case)
    shape, out = H.run_phase1(wl)
    dv = H.device_dv(wl)
    bank0 = W.make_bank(wl, "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.bank_seed + 37)
    grad0 = (torch.randn(bank0.shape, generator=gen, device="cuda") * 0.01).to(bank0.dtype)
    _, beta_host = W.make_read_inputs(wl)
    beta = torch.from_numpy(beta_host).cuda()
    rng = np.random.default_rng(wl.bank_seed + 41)
    dva_host = rng.standard_normal((wl.steps * P * C, hd), dtype=np.float32)
    if wl.valid_last < C:
        dva_host.reshape(wl.steps, P, C, hd)[wl.steps - 1, :, wl.valid_last:, :] = np.nan
    d_dva = torch.from_numpy(dva_host).cuda()
    for ti in case["checked"]:
        bank = bank0.clone()
        snap = torch.zeros((P * CW, hd), dtype=bank0.dtype, device="cuda")
        sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=P * C, snapshot=snap, snap_step_rows=0).step(ti)
        grad = grad0.clone()
        g_decay = torch.full((wl.N, C, Wn), float("nan"), device="cuda")
        d_k_eff = torch.full((wl.N, C, Wn), float("nan"), device="cuda")
        ws = sdm.alloc_pa_workspace(shape, hd) if case.get("ws") else None
        sdm.pa_step(grad, snap, out, beta, d_dva, shape, ti, step_rows=P * C, snap_step_rows=0, bank=bank,
                    g_decay=g_decay, d_k_eff=d_k_eff, workspace=ws)
        torch.cuda.synchronize()
        if ws is not None:   # the arrival counters are back at zero
            assert not ws[:H.pa_counter_bytes(shape)].any()
        touched = []
        for p in range(P):
            cidx = ti * P + p
            tv = wl.valid_last if cidx >= wl.first_partial else C
            o = H.oracle_phase1(wl, [cidx], fields=["k_eff", "krec_slot", "krec_cpe", "spay_k"])
            pad = ((o["spay_k"][0].astype(np.int64) >> 17) & 1).astype(bool)
            cpe_of = dict(zip(o["krec_slot"][0][~pad].tolist(), o["krec_cpe"][0][~pad].tolist()))
            host = lambda t, s: t.index_select(0, torch.as_tensor(s, device="cuda")).float().cpu().numpy().astype(np.float64)  # noqa: E731
            rows = dva_host[ti * P * C + p * C: ti * P * C + (p + 1) * C].astype(np.float64)
            slots, new, g_dec, d_ke, mag, mag_dot = gds.pa_chunk(
                wl.k_idx[cidx], o["k_eff"][0], beta_host[cidx], lambda s: cpe_of[s], rows,
                lambda s: host(grad0, s), lambda s: host(bank0, s), tv)
            if len(slots):
                g_new = host(grad, slots)
                members = np.array([(wl.k_idx[cidx][:tv] == s).sum() for s in slots], np.float64)[:, None]
                tol = (members + 4) * 2.0 ** -23 * mag + 1e-5 * mag + bf_slack * mag
                if grad.dtype == torch.bfloat16:
                    tol = tol + H.ulp_bf16(np.maximum(np.abs(g_new), np.abs(new)))
                bad = ~(np.abs(g_new - new) <= tol)
                assert not bad.any(), ("grad", ti, p, int(bad.sum()), g_new[bad][:3], new[bad][:3])
                sidx = torch.as_tensor(slots, device="cuda")
                assert torch.equal(bank.index_select(0, sidx).view(torch.uint8), bank0.index_select(0, sidx).view(torch.uint8))
                touched.append(slots)
            gd = g_decay[cidx].cpu().numpy().astype(np.float64)
            dk = d_k_eff[cidx].cpu().numpy().astype(np.float64)
            assert np.all(gd[tv:] == 0) and np.all(dk[tv:] == 0), "masked entries"
            gmag = np.zeros_like(g_dec)
            for t in range(tv):
                for n in range(Wn):
                    s = int(wl.k_idx[cidx][t, n])
                    gmag[t, n] = cpe_of[s] * float(np.abs(host(grad0, [s])[0]) @ np.abs(host(bank0, [s])[0]))
            tol = (hd + 8) * 2.0 ** -23 * gmag + 1e-5 * gmag + bf_slack * gmag + 1e-6
            bad = ~(np.abs(gd - g_dec) <= tol)
            assert not bad.any(), ("g_decay", ti, p, np.argwhere(bad)[:3], gd[bad][:3], g_dec[bad][:3])
            tol = (hd + 8) * 2.0 ** -23 * np.abs(beta_host[cidx][:, None].astype(np.float64)) * mag_dot + 1e-6
            tol[tv:] = 0
            bad = ~(np.abs(dk - d_ke) <= tol)
            assert not bad.any(), ("d_k_eff", ti, p, np.argwhere(bad)[:3], dk[bad][:3], d_ke[bad][:3])
        hit = np.unique(np.concatenate(touched)) if touched else np.zeros(0, np.int64)
        cand = np.setdiff1d(np.random.default_rng(ti).integers(0, wl.rows, size=4000), hit)
        if cand.size:
            ci = torch.as_tensor(cand, device="cuda")
            assert torch.equal(grad.index_select(0, ci).view(torch.uint8), grad0.index_select(0, ci).view(torch.uint8))


@pytest.mark.parametrize("split", [False, True])
def test_pa_bitwise_reproducible(split):
    """Two PA runs on the same inputs (the Zipf workload: long write groups) give the same bits in
    every output: gradient rows, restored bank rows, decay and k_eff gradients. With a workspace the
    long groups are split, and whichever segment arrives last the partial sums are added in the same
    order (the workspace is reused by the second run: its counters are back at zero)."""
    wl = W.make(2, steps=1)
    sh = wl.shape
    P, C, Wn, hd, CW = sh.P, sh.C, sh.W, sh.hd, sh.C * sh.W
    say("pa reproducibility: workload 2")
    shape, out = H.run_phase1(wl)
    dv = H.device_dv(wl)
    bank0 = W.make_bank(wl, "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.bank_seed + 53)
    grad0 = (torch.randn(bank0.shape, generator=gen, device="cuda") * 0.01).to(bank0.dtype)
    beta = torch.rand((wl.N, C), generator=gen, device="cuda")
    d_dva = torch.randn((wl.steps * P * C, hd), generator=gen, device="cuda")
    ws = sdm.alloc_pa_workspace(shape, hd) if split else None
    results = []
    for _ in range(2):
        bank = bank0.clone()
        snap = torch.zeros((P * CW, hd), dtype=bank0.dtype, device="cuda")
        sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=P * C, snapshot=snap, snap_step_rows=0).step(0)
        grad = grad0.clone()
        g_decay = torch.zeros((wl.N, C, Wn), device="cuda")
        d_k_eff = torch.zeros((wl.N, C, Wn), device="cuda")
        sdm.pa_step(grad, snap, out, beta, d_dva, shape, 0, step_rows=P * C, snap_step_rows=0, bank=bank,
                    g_decay=g_decay, d_k_eff=d_k_eff, workspace=ws)
        torch.cuda.synchronize()
        results.append((grad, bank, g_decay, d_k_eff))
    for a, b in zip(*results):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
