"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Integer and index outputs must match bit for bit; float32 outputs within max(1e-5 |o|, 1e-6);
bf16 banks within one bf16 ulp plus the float32 evaluation bound (tests/hip_harness.py). Every
input comes from sparse_delta_memory_amd.workloads; every expected value from oracle/.
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

# Workload index -> steps for the full comparison (the oracle finishes each in seconds; several
# tiles of 1024 entries per chunk, the ragged last step of workload 4 included).
SMALL_STEPS = {0: None, 1: 2, 2: 1, 3: 2, 4: 2}


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_phase1_full_compare(idx):
    wl = W.make(idx, steps=SMALL_STEPS[idx])
    say("phase1 full compare: workload", idx, wl.shape.name, "N =", wl.N)
    shape, out = H.run_phase1(wl)
    ref = H.oracle_phase1(wl, list(range(wl.N)))
    H.compare_phase1(out, ref, range(wl.N))


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_phase1_full_size_sampled(idx):
    """The full workload in one call (the benchmark's launch), checked on sampled chunks."""
    wl = W.make(idx)
    say("phase1 full size: workload", idx, wl.shape.name, "N =", wl.N)
    shape, out = H.run_phase1(wl)
    chunks = sorted({0, wl.P - 1, wl.N // 2 + 1, wl.N - 1})
    ref = H.oracle_phase1(wl, chunks)
    H.compare_phase1(out, ref, chunks)
    # Properties over every chunk: sorted positions are permutations of the row.
    n = wl.shape.C * (wl.shape.W + wl.shape.R)
    pos = torch.cat([out["pos_k"].reshape(wl.N, -1), out["pos_q"].reshape(wl.N, -1)], 1) & ((1 << 17) - 1)
    srt, _ = torch.sort(pos, dim=1)
    assert torch.equal(srt, torch.arange(n, device=pos.device, dtype=pos.dtype).expand(wl.N, n))


@pytest.mark.parametrize("idx,steps,check", [
    (0, None, {0, 1, 2, 3}), (1, 4, {0, 1, 3}), (2, 2, {0, 1}), (3, 2, {0, 1}), (4, 3, {0, 2}),
])
def test_dw_steps(idx, steps, check):
    wl = W.make(idx, steps=steps)
    say("dw steps: workload", idx, wl.shape.name, "steps", wl.steps)
    shape, out = H.run_phase1(wl)
    n, _ = H.run_dw_check(wl, out, shape, check)
    assert n > 0


@pytest.mark.parametrize("idx,check", [(1, {0, 31}), (3, {0, 31}), (4, {0, 63})])
def test_dw_full_size(idx, check):
    """Every step of the full workload on the GPU; the oracle's state is carried through all steps
    and the checked steps (the first and the last, ragged in workload 4) are compared."""
    wl = W.make(idx)
    say("dw full size: workload", idx, wl.shape.name, "steps", wl.steps)
    shape, out = H.run_phase1(wl)
    n, _ = H.run_dw_check(wl, out, shape, check, sample_untouched=5000)
    assert n > 0


@pytest.mark.parametrize("idx,steps", [(2, 2), (0, None)])
def test_dw_unsplit(idx, steps):
    """Without a workspace every group is one FMA chain: also within tolerance."""
    wl = W.make(idx, steps=steps)
    say("dw without workspace: workload", idx)
    shape, out = H.run_phase1(wl)
    n, _ = H.run_dw_check(wl, out, shape, set(range(wl.steps)), split=False)
    assert n > 0


def test_bitwise_reproducible():
    wl = W.make(2, steps=1)
    say("reproducibility: workload 2")
    _, o1 = H.run_phase1(wl)
    _, o2 = H.run_phase1(wl)
    for k in o1:
        assert torch.equal(o1[k].view(torch.uint8), o2[k].view(torch.uint8)), k
    wl = W.make(1, steps=3)
    shape, out = H.run_phase1(wl)
    dv = H.device_dv(wl)
    banks = []
    for _ in range(2):
        bank = W.make_bank(wl, "cuda")
        for ti in range(wl.steps):
            sdm.dw_step(bank, dv, out["krec"], shape, ti, dv_step_rows=wl.P * wl.shape.C)
        torch.cuda.synchronize()
        banks.append(bank)
    assert torch.equal(banks[0].view(torch.uint16), banks[1].view(torch.uint16))
    # Split long groups (Zipf hot slots): whichever segment team arrives last, the same bits.
    wl = W.make(2, steps=2)
    shape, out = H.run_phase1(wl)
    dv = H.device_dv(wl)
    banks = []
    for _ in range(3):
        bank = W.make_bank(wl, "cuda")
        ws = sdm.alloc_dw_workspace(shape, wl.shape.hd)
        for ti in range(wl.steps):
            sdm.dw_step(bank, dv, out["krec"], shape, ti, dv_step_rows=wl.P * wl.shape.C, workspace=ws)
        torch.cuda.synchronize()
        banks.append(bank)
    assert torch.equal(banks[0].view(torch.uint16), banks[1].view(torch.uint16))
    assert torch.equal(banks[0].view(torch.uint16), banks[2].view(torch.uint16))


def test_masked_tokens_do_not_leak():
    """NaN in the values, gates and token rows of masked tokens changes no output bit."""
    a = W.make(4, steps=2, nan_invalid=True)
    b = W.make(4, steps=2, nan_invalid=False)
    say("masking: workload 4, 2 steps")
    shape, oa = H.run_phase1(a)
    _, ob = H.run_phase1(b)
    for k in oa:
        assert torch.equal(oa[k].view(torch.uint8), ob[k].view(torch.uint8)), k
    banks = []
    for wl, out in ((a, oa), (b, ob)):
        bank = W.make_bank(wl, "cuda")
        dv = H.device_dv(wl)
        for ti in range(wl.steps):
            sdm.dw_step(bank, dv, out["krec"], shape, ti, dv_step_rows=wl.P * wl.shape.C)
        torch.cuda.synchronize()
        banks.append(bank)
    assert torch.equal(banks[0].view(torch.uint16), banks[1].view(torch.uint16))
    assert not torch.isnan(banks[0].float()).any()


@pytest.mark.parametrize("case", [
    dict(C=37, W=5, R=3, S=9, P=2, steps=2, vl=11),       # ragged row (296 entries), heavy sharing
    dict(C=1, W=1, R=1, S=4, P=1, steps=3, vl=None),      # one token
    dict(C=64, W=2, R=3, S=1, P=1, steps=2, vl=0),        # one slot; last chunk fully masked
    # One group of 5120 entries: saturated counts. The only stress shape: its cells sum up to 289
    # terms that cancel (a 289-term cell of about 0.13 differs by 2.7e-6 in any float32 summation),
    # so A / QK take the float32 evaluation bound there (hip_harness.assert_pair_sums).
    dict(C=256, W=17, R=3, S=1, P=1, steps=1, vl=None, stress=True),
    dict(C=100, W=7, R=9, S=3000, P=3, steps=2, vl=50),   # 1600 entries: two radix tiles
    # An odd K row (8415 positions) in a DW launch wide enough for two positions per team of lanes.
    dict(C=255, W=33, R=2, S=5000, P=1, steps=1, vl=None, hd=960, bank="bf16"),
    # Every slot group hot (about 43 K entries each): more hot groups than one pair-kernel batch holds.
    dict(C=256, W=8, R=8, S=48, P=1, steps=1, vl=None),
    # Hot groups in 512-thread pair blocks (C = 120), a ragged last chunk.
    dict(C=120, W=16, R=4, S=70, P=2, steps=1, vl=100),
    # Hot groups whose log-cumsum spans more than the dense pass takes (gates near -4): walked.
    dict(C=256, W=8, R=8, S=48, P=1, steps=1, vl=None, gmu=-4.0),
    # 8192 entries (8 per thread) whose keys, values and records do not all fit in LDS together.
    dict(C=256, W=16, R=16, S=20000, P=1, steps=1, vl=200),
])
def test_edge_shapes(case):
    sh = W.Shape("edge", P=case["P"], T=case["C"] * case["steps"], C=case["C"], W=case["W"], R=case["R"],
                 S=case["S"], hd=case.get("hd", 64), bank_dtype=case.get("bank", "f32"), dv_dtype="f32",
                 slots="uniform", valid_last=case["vl"], gate_mu=case.get("gmu", 2.0))
    wl = W.make(sh, seed=777)
    say("edge shape", case)
    shape, out = H.run_phase1(wl)
    ref = H.oracle_phase1(wl, list(range(wl.N)), with_magnitudes=case.get("stress", False))
    H.compare_phase1(out, ref, range(wl.N))
    H.run_dw_check(wl, out, shape, set(range(wl.steps)), sample_untouched=0)


def test_tile_len_variants():
    # Powers of two (a mask and a shift in the kernel) and other lengths (a division), at 4 and at
    # 16 items per thread (workloads 1 and 2).
    for idx, lens in ((1, (1, 32, 100, 4096)), (2, (1, 100, 384))):
        wl = W.make(idx, steps=1)
        for L in lens:
            shape, out = H.run_phase1(wl, tile_len=L)
            ref = H.oracle_phase1(wl, list(range(wl.N)), tile_len=L)
            H.assert_exact("tiles_k w%d L=%d" % (idx, L), out["tiles_k"].cpu().numpy(), ref["tiles_k"])


def test_empty_call():
    shape = sdm.make_shape(0, 16, 2, 2, key_bits=8)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    f = torch.empty(0, dtype=torch.float32, device="cuda")
    out = sdm.phase1(shape, e, e, f, f, f)
    torch.cuda.synchronize()
    assert out["krec"].numel() == 0


@pytest.mark.parametrize("case", [
    dict(idx=0),                                           # tiny workload, one gate per (token, K lane)
    dict(C=37, W=5, R=3, S=9, P=2, steps=2, vl=11),        # heavy sharing (many repeats), ragged row and chunk
    dict(C=256, W=8, R=8, S=48, P=1, steps=1, vl=None),   # every group hot: the dense pair pass
    dict(idx=1, steps=2),                                  # the uniform bf16 shape (IPT 4)
])
def test_lane_gates(case):
    """Per-(token, K lane) gates [N, C, W]: every Phase-1 output and the DW steps match the oracle."""
    if "idx" in case:
        wl = W.make(case["idx"], steps=case.get("steps"), lane_gates=True)
    else:
        sh = W.Shape("lane_gates", P=case["P"], T=case["C"] * case["steps"], C=case["C"], W=case["W"], R=case["R"],
                     S=case["S"], hd=64, bank_dtype="f32", dv_dtype="f32", slots="uniform", valid_last=case["vl"])
        wl = W.make(sh, seed=778, lane_gates=True)
    say("lane gates", case)
    shape, out = H.run_phase1(wl)
    chunks = list(range(min(wl.N, 16)))
    ref = H.oracle_phase1(wl, chunks)
    H.compare_phase1(out, ref, chunks)
    H.run_dw_check(wl, out, shape, set(range(min(wl.steps, 2))), sample_untouched=0)


@pytest.mark.parametrize("case", [
    dict(C=37, W=5, R=3, S=9, P=2, steps=2, vl=11, lg=False),   # ragged rows: scalar value loads and stores
    dict(idx=0, lg=False),                                      # tiny shape, every chunk
    dict(idx=1, steps=2, lg=False),                             # resident layout, 4-entry vector paths
    dict(idx=2, steps=1, lg=False),                             # Zipf rows of 16384 entries (several sweeps)
    dict(idx=4, steps=1, lg=True),                              # large ragged shape, per-lane gates
])
def test_bf16_values(case):
    """bfloat16 k_val / q_val: cpe, k_eff, q_w and krec's cpe are bfloat16 within one bfloat16 ulp of
    the oracle's, every other output matches the oracle as usual, and DW (which scales by the
    bfloat16 cpe) matches the oracle's bfloat16-value DW. Also: every output that is not value-typed
    is bitwise the float32-value path's on the same (bfloat16-representable) values."""
    if "idx" in case:
        wl = W.make(case["idx"], steps=case.get("steps"), lane_gates=case["lg"], val_bf16=True)
    else:
        sh = W.Shape("bf16_values", P=case["P"], T=case["C"] * case["steps"], C=case["C"], W=case["W"], R=case["R"],
                     S=case["S"], hd=64, bank_dtype="f32", dv_dtype="f32", slots="uniform", valid_last=case["vl"])
        wl = W.make(sh, seed=781, lane_gates=case["lg"], val_bf16=True)
    say("bf16 values", case)
    shape, out = H.run_phase1(wl)
    assert out["k_eff"].dtype == torch.bfloat16 and out["cpe"].dtype == torch.bfloat16
    chunks = list(range(min(wl.N, 12))) + ([wl.N - 1] if wl.N > 12 else [])
    ref = H.oracle_phase1(wl, chunks)
    H.compare_phase1(out, ref, chunks)
    # The float32-value path on the same values: identical except the value-typed fields.
    f32_wl = W.Workload(**{**wl.__dict__, "meta": {k: v for k, v in wl.meta.items() if k != "val_bf16"}})
    _, plain = H.run_phase1(f32_wl)
    for k in plain:
        if k in H.VALUE_TYPED:
            continue
        if k == "krec":
            assert torch.equal(out[k][..., :3], plain[k][..., :3]), "krec element / slot / scale"
            continue
        assert torch.equal(out[k].view(torch.uint8), plain[k].view(torch.uint8)), k
    H.run_dw_check(wl, out, shape, set(range(min(wl.steps, 2))), sample_untouched=0)


@pytest.mark.parametrize("case", [
    dict(hd=1, bank="f32", dv="f32", S=64, C=32, W=4, P=1, vl=None, split=True),
    dict(hd=37, bank="bf16", dv="f32", S=8, C=64, W=6, P=2, vl=50, split=True),     # long groups: split path
    dict(hd=37, bank="bf16", dv="f32", S=8, C=64, W=6, P=2, vl=50, split=False),    # ... one team per group
    dict(hd=100, bank="f32", dv="bf16", S=200, C=128, W=8, P=2, vl=None, split=True),
    dict(hd=126, bank="bf16", dv="bf16", S=16, C=128, W=4, P=1, vl=None, split=True),
    dict(hd=520, bank="f32", dv="f32", S=300, C=64, W=4, P=1, vl=None, split=True),  # 16 columns per lane
    dict(hd=1000, bank="bf16", dv="f32", S=30, C=64, W=4, P=1, vl=None, split=True),
])
def test_dw_tail_head_dims(case):
    """Head dims that 16-byte vectors do not divide (element accesses, element-aligned rows): every
    checked DW step matches the oracle, and rows no group touches keep their bits."""
    sh = W.Shape("tail_hd", P=case["P"], T=case["C"] * 3, C=case["C"], W=case["W"], R=2, S=case["S"], hd=case["hd"],
                 bank_dtype=case["bank"], dv_dtype=case["dv"], slots="uniform", valid_last=case["vl"])
    wl = W.make(sh, seed=783)
    say("dw tail", case)
    shape, out = H.run_phase1(wl)
    H.run_dw_check(wl, out, shape, set(range(wl.steps)), sample_untouched=200, split=case["split"])


@pytest.mark.parametrize("idx,steps", [(0, None), (1, 2), (2, 1), (4, 1)])
def test_group_ordinals(idx, steps):
    """gord_k (dense group ordinals of the K-only row) equals the oracle's bit for bit, and asking
    for it changes no other output bit."""
    wl = W.make(idx, steps=steps)
    say("group ordinals", idx, steps)
    shape, out = H.run_phase1(wl, fields=["gord_k"])
    _, plain = H.run_phase1(wl)
    for k in plain:
        assert torch.equal(out[k].view(torch.uint8), plain[k].view(torch.uint8)), k
    chunks = list(range(min(wl.N, 8))) + [wl.N - 1]
    ref = H.oracle_phase1(wl, chunks, fields=["gord_k"])
    got = out["gord_k"].index_select(0, torch.as_tensor(chunks, device="cuda")).cpu().numpy()
    H.assert_exact("gord_k", got, ref["gord_k"])


@pytest.mark.parametrize("idx,steps", [(0, None), (2, 1), (4, 1)])
def test_perm_output(idx, steps):
    """The optional sorted order (entry index at each sorted position) equals the oracle's, and
    requesting it changes no other output bit."""
    wl = W.make(idx, steps=steps)
    say("perm", idx, steps)
    shape, out = H.run_phase1(wl, fields=["perm"])
    _, plain = H.run_phase1(wl)
    for k in plain:
        assert torch.equal(out[k].view(torch.uint8), plain[k].view(torch.uint8)), k
    chunks = list(range(min(wl.N, 8))) + [wl.N - 1]
    ref = H.oracle_phase1(wl, chunks, fields=["perm"])
    H.assert_exact("perm", out["perm"].index_select(0, torch.as_tensor(chunks, device="cuda")).cpu().numpy(), ref["perm"])


@pytest.mark.parametrize("idx,steps", [(1, 2), (4, 1)])
def test_int64_ids(idx, steps):
    """int64 slot ids give every Phase-1 output, and the read side's outputs, bit for bit as the
    same ids in int32 do."""
    import dataclasses

    wl32 = W.make(idx, steps=steps)
    wl64 = dataclasses.replace(wl32, k_idx=wl32.k_idx.astype(np.int64), q_idx=wl32.q_idx.astype(np.int64))
    say("int64 ids", idx, steps)
    outs = []
    for wl in (wl32, wl64):
        shape, out = H.run_phase1(wl, fields=["perm"])
        ins = H.device_inputs(wl)
        v_host, beta_host = W.make_read_inputs(wl32)
        v = torch.from_numpy(v_host).cuda()
        beta = torch.from_numpy(beta_host).cuda()
        dv = torch.zeros((v.shape[0], wl.shape.hd), device="cuda")
        pred, read = torch.zeros_like(dv), torch.zeros_like(dv)
        bank = W.make_bank(wl32, "cuda")
        plan = sdm.ReadPlan(bank, out, ins["k_idx"], ins["q_idx"], v, beta, dv, pred, read, shape,
                            step_rows=wl.P * wl.shape.C)
        plan.step(0)
        torch.cuda.synchronize()
        out.update(dv=dv, pred=pred, read=read)
        outs.append(out)
    for k in outs[0]:
        assert torch.equal(outs[0][k].view(torch.uint8), outs[1][k].view(torch.uint8)), k


@pytest.mark.parametrize("idx,steps,case", [(0, 2, None), (1, 2, None), (2, 1, None),
                                            (3, 1, None),   # a 7.5 GiB bank: rows loaded non-temporally
                                            (None, 1, dict(C=255, W=33, R=2, S=5000, P=1, vl=None, hd=960)),
                                            (None, 2, dict(C=64, W=6, R=2, S=8, P=2, vl=50, hd=37)),   # tail
                                            (0, 2, "bf16"),                                           # bf16 rows
                                            (None, 2, dict(C=64, W=6, R=2, S=8, P=2, vl=50, hd=37, bank="f32",
                                                           snap="bf16")),
                                            (1, 2, "dense"), (2, 1, "dense"),                         # dense rows
                                            (None, 2, dict(C=64, W=6, R=2, S=8, P=2, vl=50, hd=37, dense=True))])
def test_dw_snapshot(idx, steps, case):
    """The compact snapshot: row (ti*P*C*W + p*C*W + j) holds the raw pre-write bank row of the valid
    group whose FIRST is at K-row position j (positions from the oracle's sorted K rows), every other
    row keeps its sentinel, and writing it changes no bank bit. bf16 snapshot rows of a float32 bank:
    the pre-write row converted to bfloat16 (torch's round to nearest even). Dense layout (the Phase-1
    group ordinals as snap_ord): the chunk's groups in rows 0 .. groups - 1, ascending slot order."""
    snap_bf16 = case == "bf16" or (isinstance(case, dict) and case.get("snap") == "bf16")
    dense = case == "dense" or (isinstance(case, dict) and case.get("dense", False))
    if case in ("bf16", "dense"):
        case = None
    if case is None:
        wl = W.make(idx, steps=steps)
    else:
        sh = W.Shape("snap_edge", P=case["P"], T=case["C"] * steps, C=case["C"], W=case["W"], R=case["R"],
                     S=case["S"], hd=case["hd"], bank_dtype=case.get("bank", "bf16"), dv_dtype="f32", slots="uniform",
                     valid_last=case["vl"])
        wl = W.make(sh, seed=780)
    sh = wl.shape
    P, C, hd, CW = sh.P, sh.C, sh.hd, sh.C * sh.W
    say("dw snapshot", idx, case, "dense" if dense else "")
    shape, out = H.run_phase1(wl, fields=["gord_k"] if dense else None)
    dv = H.device_dv(wl)
    bank0 = W.make_bank(wl, "cuda")
    if snap_bf16:
        assert bank0.dtype == torch.float32
    snap = torch.empty((wl.steps * P * CW, hd), dtype=torch.bfloat16 if snap_bf16 else bank0.dtype, device="cuda")
    snap.view(torch.uint8).fill_(0xA5)
    sentinel = snap[0].clone()
    bank, bank_ref = bank0.clone(), bank0.clone()
    plan_s = sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=P * C,
                        workspace=sdm.alloc_dw_workspace(shape, hd, device="cuda"), snapshot=snap, snap_step_rows=P * CW,
                        snap_ord=out["gord_k"] if dense else None)
    plan_n = sdm.DwPlan(bank_ref, dv, out["krec"], shape, dv_step_rows=P * C,
                        workspace=sdm.alloc_dw_workspace(shape, hd, device="cuda"))
    ref = H.oracle_phase1(wl, list(range(wl.N)), fields=["spay_k", "krec_slot"])
    for ti in range(wl.steps):
        bank.copy_(bank0)
        bank_ref.copy_(bank0)
        plan_s.step(ti)
        plan_n.step(ti)
        torch.cuda.synchronize()
        assert torch.equal(bank.view(torch.uint8), bank_ref.view(torch.uint8)), ti
        for p in range(P):
            c = ti * P + p
            el = ref["spay_k"][c].astype(np.int64) & 0xFFFFFFFF
            first = ((el >> 31) & 1).astype(bool) & ~((el >> 17) & 1).astype(bool)
            js = np.flatnonzero(first)
            rows = ti * P * CW + p * CW
            got = snap[rows:rows + CW]
            want = bank0.index_select(0, torch.as_tensor(ref["krec_slot"][c][js], dtype=torch.long, device="cuda"))
            if snap_bf16:
                want = want.to(torch.bfloat16)
            at = np.arange(len(js)) if dense else js   # dense rows: the groups in FIRST (= slot) order
            assert torch.equal(got[torch.as_tensor(at, device="cuda")].view(torch.uint8), want.view(torch.uint8)), (ti, p)
            others = np.setdiff1d(np.arange(CW), at)
            if others.size:
                rest = got[torch.as_tensor(others, device="cuda")]
                assert torch.equal(rest.view(torch.uint8), sentinel.expand_as(rest).view(torch.uint8)), (ti, p)


def test_slot_id_check():
    """The debug status word: 0 for valid inputs; bit 0 once a valid entry's slot id is out of range
    (past 2^key_bits, negative, or in another stream's range); ids of masked tokens are not checked.
    Only Phase 1 runs on the planted ids (their keys are masked into range, so it stays in bounds)."""
    sh = W.Shape("idcheck", P=2, T=74, C=37, W=5, R=3, S=9, hd=64, bank_dtype="f32", dv_dtype="f32",
                 slots="uniform", valid_last=11)
    wl = W.make(sh, seed=781)
    shape = H.shape_of(wl)
    assert shape.key_bits >= 4

    def run(k_idx, q_idx):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        sdm.phase1(shape, t(k_idx), t(q_idx), t(wl.k_val), t(wl.q_val), t(wl.g), status=status)
        torch.cuda.synchronize()
        return int(status.item())

    assert run(wl.k_idx, wl.q_idx) == 0
    big = wl.k_idx.copy()
    big[1, 5, 2] = 1 * sh.S + (1 << shape.key_bits) + 3          # stream 1, local slot past 2^key_bits
    assert run(big, wl.q_idx) == 1
    neg = wl.q_idx.copy()
    neg[0, 7, 1] = -3
    assert run(wl.k_idx, neg) == 1
    other = wl.q_idx.copy()
    other[3, 2, 0] = 4                                            # chunk 3 is stream 1: local slot -5
    assert run(wl.k_idx, other) == 1
    masked = wl.k_idx.copy()
    masked[wl.first_partial, wl.valid_last + 2, 0] = -7           # a masked token of the ragged chunk
    assert run(masked, wl.q_idx) == 0


def test_fresh_process_reproducible():
    """Two fresh processes produce the same bytes: Phase 1 outputs and the bank after every DW step
    of the uniform workload, hashed in each (child processes, one after the other)."""
    import hashlib
    import subprocess

    code = r"""
import hashlib, sys, torch
sys.path.insert(0, "tests")
import hip_harness as H
import sparse_delta_memory_amd as sdm
from sparse_delta_memory_amd import workloads as W
wl = W.make(1, steps=4)
shape, out = H.run_phase1(wl)
bank = W.make_bank(wl, "cuda")
plan = sdm.DwPlan(bank, H.device_dv(wl), out["krec"], shape, dv_step_rows=wl.P * wl.shape.C,
                  workspace=sdm.alloc_dw_workspace(shape, wl.shape.hd, device="cuda"))
h = hashlib.sha256()
for k in sorted(out):
    h.update(out[k].cpu().view(torch.uint8).numpy().tobytes())
for ti in range(wl.steps):
    plan.step(ti)
    torch.cuda.synchronize()
    h.update(bank.cpu().view(torch.uint8).numpy().tobytes())
print(h.hexdigest())
"""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("fresh process: first child")
    child = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=240)
    assert child.returncode == 0, child.stderr[-2000:]
    digest_child = child.stdout.strip().splitlines()[-1]
    say("fresh process: second child")
    here = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=240)
    assert here.returncode == 0, here.stderr[-2000:]
    assert here.stdout.strip().splitlines()[-1] == digest_child
    assert len(digest_child) == 64 and hashlib.sha256(b"").hexdigest() != digest_child
