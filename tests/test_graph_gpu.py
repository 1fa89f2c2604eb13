"""Phase 1 and the DW steps captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every replay must reproduce the eager launches bit for bit: the path enqueues no memset node
(the DW arrival counters return to zero by themselves), and replays are separated by eager work
and synchronisations. The expected values are the eager results of the same library, whose
parity with the oracle the other GPU tests establish.
"""

import os
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_delta_memory_amd as sdm  # noqa: E402
from sparse_delta_memory_amd import workloads as W  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
import hip_harness as H  # noqa: E402


@pytest.mark.parametrize("idx,steps,snap", [(1, 4, False), (2, 2, False), (0, 4, True), ("tail", 2, True)])
def test_graph_replays_match_eager(idx, steps, snap):
    """snap: also the group ordinals and the dense bf16 snapshot of a float32 bank ("tail": hd = 37,
    bf16 values, so the element-access DW and the bf16-value sort/scan kernel are captured too)."""
    if idx == "tail":
        shp = W.Shape("graph_tail", P=2, T=64 * 3, C=64, W=6, R=2, S=40, hd=37, bank_dtype="f32", dv_dtype="f32",
                      slots="uniform", valid_last=50)
        wl = W.make(shp, steps=steps, seed=785, val_bf16=True)
    else:
        wl = W.make(idx, steps=steps)
    sh = wl.shape
    CW = sh.C * sh.W
    print("graph replay: workload", idx, sh.name, "N =", wl.N, "snapshot" if snap else "", flush=True)
    shape = H.shape_of(wl)
    ins = H.device_inputs(wl)
    dv = H.device_dv(wl)
    bank0 = W.make_bank(wl, "cuda")
    fields = None
    if snap:
        fields = set(sdm.alloc_phase1_outputs(sdm.make_shape(0, 1, 1, 1), device="cpu")) | {"gord_k"}

    def make_state():
        out = sdm.alloc_phase1_outputs(shape, device="cuda", fields=fields)
        ws = torch.empty(sdm.phase1_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        dw_ws = sdm.alloc_dw_workspace(shape, sh.hd, device="cuda")
        bank = bank0.clone()
        rows = torch.empty((wl.steps * wl.P * CW, sh.hd), dtype=torch.bfloat16, device="cuda") if snap else None
        plan = sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=wl.P * sh.C, workspace=dw_ws, snapshot=rows,
                          snap_step_rows=wl.P * CW, snap_ord=out["gord_k"] if snap else None)
        if snap:
            out["snapshot"] = rows   # compared with the outputs

        def step():
            sdm.phase1(shape, out=out, workspace=ws, **ins)
            for ti in range(wl.steps):
                plan.step(ti)

        return out, bank, step

    out_e, bank_e, step_e = make_state()
    step_e()
    torch.cuda.synchronize()

    out_g, bank_g, step_g = make_state()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_g()
    torch.cuda.synchronize()
    for rep in range(3):
        bank_g.copy_(bank0)
        for t in out_g.values():
            t.view(torch.uint8).fill_(0xA5)
        # Eager work of the same library between replays.
        step_e()
        bank_e.copy_(bank0)
        if snap:   # rows no group writes keep the sentinel on both sides
            out_e["snapshot"].view(torch.uint8).fill_(0xA5)
        step_e()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in out_e:
            assert torch.equal(out_g[k].view(torch.uint8), out_e[k].view(torch.uint8)), (rep, k)
        assert torch.equal(bank_g.view(torch.uint8), bank_e.view(torch.uint8)), rep


def test_kernel_bound_events():
    """Events handed to the launches are recorded at the kernels' start and end; results unchanged."""
    wl = W.make(1, steps=2)
    sh = wl.shape
    shape = H.shape_of(wl)
    ins = H.device_inputs(wl)
    dv = H.device_dv(wl)
    ref_out = sdm.phase1(shape, **ins)
    ref_bank = W.make_bank(wl, "cuda")
    for ti in range(wl.steps):
        sdm.dw_step(ref_bank, dv, ref_out["krec"], shape, ti, dv_step_rows=wl.P * sh.C)
    ev = sdm.timing_events(4)
    out = sdm.phase1(shape, events=ev, **ins)
    bank = W.make_bank(wl, "cuda")
    plan = sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=wl.P * sh.C)
    dw_ev = [sdm.timing_events(2) for _ in range(wl.steps)]
    for ti in range(wl.steps):
        plan.step(ti, events=dw_ev[ti])
    torch.cuda.synchronize()
    for a, b in ((ev[0], ev[1]), (ev[2], ev[3])) + tuple((e[0], e[1]) for e in dw_ev):
        ms = a.elapsed_time(b)
        assert 0.0 < ms < 1000.0, ms
    # The sort/scan kernel ends before the pair kernel starts (same stream).
    assert ev[1].elapsed_time(ev[2]) >= 0.0
    for k in ref_out:
        assert torch.equal(out[k].view(torch.uint8), ref_out[k].view(torch.uint8)), k
    assert torch.equal(bank.view(torch.uint8), ref_bank.view(torch.uint8))
    with pytest.raises(ValueError):
        sdm.phase1(shape, events=[torch.cuda.Event(enable_timing=True) for _ in range(4)], **ins)


def test_graph_forward_loop_with_read_side():
    """Phase 1 and, step after step, the read side then DW (the read side's dv feeding DW), captured
    once and replayed: every replay equals the eager loop bit for bit."""
    wl = W.make(1, steps=3)
    sh = wl.shape
    P, C, hd = sh.P, sh.C, sh.hd
    shape = H.shape_of(wl)
    ins = H.device_inputs(wl)
    v_host, beta_host = W.make_read_inputs(wl)
    v = torch.from_numpy(v_host).cuda()
    beta = torch.from_numpy(beta_host).cuda()
    bank0 = W.make_bank(wl, "cuda")

    def make_state():
        out = sdm.alloc_phase1_outputs(shape, device="cuda")
        ws = torch.empty(sdm.phase1_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        bank = bank0.clone()
        dv = torch.zeros((v.shape[0], hd), device="cuda")
        pred, read = torch.zeros_like(dv), torch.zeros_like(dv)
        rplan = sdm.ReadPlan(bank, out, ins["k_idx"], ins["q_idx"], v, beta, dv, pred, read, shape, step_rows=P * C)
        dplan = sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=P * C)

        def loop():
            sdm.phase1(shape, out=out, workspace=ws, **ins)
            for ti in range(wl.steps):
                rplan.step(ti)
                dplan.step(ti)

        return dict(out, bank=bank, dv=dv, pred=pred, read=read), loop

    st_e, loop_e = make_state()
    loop_e()
    torch.cuda.synchronize()
    st_g, loop_g = make_state()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop_g()
    torch.cuda.synchronize()
    for rep in range(3):
        st_g["bank"].copy_(bank0)
        for k, t in st_g.items():
            if k != "bank":
                t.view(torch.uint8).fill_(0xA5)
        st_e["bank"].copy_(bank0)
        loop_e()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in st_e:
            assert torch.equal(st_g[k].view(torch.uint8), st_e[k].view(torch.uint8)), (rep, k)


def test_graph_backward_gathers():
    """GDS and GWR of every step captured in one graph and replayed: every replay equals the eager
    calls bit for bit (both write their outputs in full or by read-modify-write from a reset grad)."""
    import numpy as np

    wl = W.make(1, steps=3)
    sh = wl.shape
    P, C, hd = sh.P, sh.C, sh.hd
    shape, out = H.run_phase1(wl)
    ins = H.device_inputs(wl)
    bank = W.make_bank(wl, "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    gr = torch.randn((wl.steps * P * C, hd), generator=gen, device="cuda")
    w = torch.randn((wl.N, C, sh.W), generator=gen, device="cuda")
    dv = torch.from_numpy(wl.dv.reshape(-1, hd).astype(np.float32)).cuda()
    g0 = (torch.randn(bank.shape, generator=gen, device="cuda") * 0.01).to(bank.dtype)

    def make_state():
        st = dict(d_q_w=torch.zeros((wl.N, C, sh.R), device="cuda"), grad=g0.clone(),
                  d_dv=torch.zeros_like(dv), d_k_pd=torch.zeros((wl.N, C, sh.W), device="cuda"))

        def run():
            for ti in range(wl.steps):
                sdm.gds_step(bank, out, ins["q_idx"], gr, shape, ti, step_rows=P * C, d_q_w=st["d_q_w"], grad=st["grad"])
                sdm.gwr_step(st["grad"], ins["k_idx"], w, dv, shape, ti, step_rows=P * C, d_dv=st["d_dv"],
                             d_k_pd=st["d_k_pd"])
        return st, run

    st_e, run_e = make_state()
    run_e()
    torch.cuda.synchronize()
    st_g, run_g = make_state()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_g()
    torch.cuda.synchronize()
    for rep in range(3):
        for k in ("d_q_w", "d_dv", "d_k_pd"):
            st_g[k].fill_(float("nan"))
        st_g["grad"].copy_(g0)
        st_e["grad"].copy_(g0)   # eager work between replays
        run_e()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in st_e:
            assert torch.equal(st_g[k].view(torch.uint8), st_e[k].view(torch.uint8)), (rep, k)
