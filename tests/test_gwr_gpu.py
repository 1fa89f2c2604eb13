"""GPU parity of GWR (sdm_gwr_step, the backward of DW's write terms) against the float64 oracle
(oracle/gds.py, gwr_chunk).

Inputs (seeded): write weights w [N, C, W] and the workload's token rows (masked tokens NaN: they
must not be read); the bank gradient drawn on the device in the bank dtype and read back as the
oracle's input. Tolerances: d_dv within (W + 4) 2^-23 sum |w grad| + 1e-6 (a W-term fma chain);
d_k_pd within (hd + 8) 2^-23 sum |dv grad| + 1e-6 (an hd-term dot with a wave reduction).
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


def gwr_inputs(wl, dtype):
    sh = wl.shape
    rng = np.random.default_rng(wl.bank_seed + 29)
    w = rng.standard_normal((wl.N, sh.C, sh.W), dtype=np.float32)
    if wl.valid_last < sh.C:
        w[wl.first_partial:, wl.valid_last:, :] = np.nan
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.bank_seed + 31)
    grad = (torch.randn((wl.rows, sh.hd), generator=gen, device="cuda") * 0.1).to(dtype)
    return w, grad


@pytest.mark.parametrize("case", [
    dict(idx=0, steps=None, checked=[0, 3]),
    dict(idx=1, steps=2, checked=[0, 1]),
    dict(idx=2, steps=1, checked=[0]),
    dict(idx=3, steps=1, checked=[0]),                  # hd = 960
    dict(idx=4, steps=2, checked=[1]),                  # ragged last step
    dict(shape=dict(C=37, W=5, S=9, P=2, vl=11, hd=36), steps=2, checked=[0, 1]),
])
def test_gwr_matches_oracle(case):
    if "shape" in case:
        c = case["shape"]
        shp = W.Shape("gwr_edge", P=c["P"], T=c["C"] * case["steps"], C=c["C"], W=c["W"], R=2, S=c["S"], hd=c["hd"],
                      bank_dtype="f32", dv_dtype="f32", slots="uniform", valid_last=c["vl"])
        wl = W.make(shp, seed=789)
    else:
        wl = W.make(case["idx"], steps=case["steps"])
    sh = wl.shape
    P, C, Wn, hd = sh.P, sh.C, sh.W, sh.hd
    say("gwr", case)
    shape = H.shape_of(wl)
    ins = H.device_inputs(wl)
    dt = torch.bfloat16 if sh.bank_dtype == "bf16" else torch.float32
    w_host, grad = gwr_inputs(wl, dt)
    w = torch.from_numpy(w_host).cuda()
    dv_host = wl.dv.reshape(-1, hd).astype(np.float32)
    dv = torch.from_numpy(dv_host).cuda()
    for ti in case["checked"]:
        d_dv = torch.full_like(dv, float("nan"))
        d_pd = torch.full((wl.N, C, Wn), float("nan"), device="cuda")
        sdm.gwr_step(grad, ins["k_idx"], w, dv, shape, ti, step_rows=P * C, d_dv=d_dv, d_k_pd=d_pd)
        torch.cuda.synchronize()
        for p in range(P):
            cidx = ti * P + p
            tv = wl.valid_last if cidx >= wl.first_partial else C
            rows_of = lambda s: grad.index_select(0, torch.as_tensor(s, device="cuda")).float().cpu().numpy().astype(np.float64)  # noqa: E731
            sl = slice(ti * P * C + p * C, ti * P * C + (p + 1) * C)
            want_dv, want_pd, mag_dv, mag_pd = gds.gwr_chunk(wl.k_idx[cidx], w_host[cidx], dv_host[sl], rows_of, tv)
            got_dv = d_dv[sl].cpu().numpy().astype(np.float64)
            tol = (Wn + 4) * 2.0 ** -23 * mag_dv + 1e-6
            bad = ~(np.abs(got_dv - want_dv) <= tol)
            assert not bad.any(), ("d_dv", ti, p, np.argwhere(bad)[:3], got_dv[bad][:3], want_dv[bad][:3])
            got_pd = d_pd[cidx].cpu().numpy().astype(np.float64)
            tol = (hd + 8) * 2.0 ** -23 * mag_pd + 1e-6
            bad = ~(np.abs(got_pd - want_pd) <= tol)
            assert not bad.any(), ("d_k_pd", ti, p, np.argwhere(bad)[:3], got_pd[bad][:3], want_pd[bad][:3])


def test_gwr_reproducible():
    wl = W.make(1, steps=1)
    sh = wl.shape
    shape = H.shape_of(wl)
    ins = H.device_inputs(wl)
    w_host, grad = gwr_inputs(wl, torch.bfloat16)
    w = torch.from_numpy(w_host).cuda()
    dv = torch.from_numpy(wl.dv.reshape(-1, sh.hd).astype(np.float32)).cuda()
    res = []
    for _ in range(2):
        d_dv = torch.zeros_like(dv)
        d_pd = torch.zeros((wl.N, sh.C, sh.W), device="cuda")
        sdm.gwr_step(grad, ins["k_idx"], w, dv, shape, 0, step_rows=sh.P * sh.C, d_dv=d_dv, d_k_pd=d_pd)
        torch.cuda.synchronize()
        res.append((d_dv, d_pd))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
