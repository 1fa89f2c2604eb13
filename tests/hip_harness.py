"""Helpers shared by the GPU tests: run the HIP path on a workload and compare with the oracle.

Inputs come from sparse_delta_memory_amd.workloads; expected values only from oracle/. The oracle
never receives a value produced by the HIP path: for the DW check, the oracle's own bank state
is copied INTO the GPU bank before a checked step, so both sides start that step from the same
rows.
"""

from __future__ import annotations

import numpy as np

import oracle
from oracle import read_side
import sparse_delta_memory_amd as sdm
from sparse_delta_memory_amd import workloads as W

F32_REL, F32_ABS = 1e-5, 1e-6
READ_RTOL_MAG = 1e-4   # read side: times the oracle's magnitude bound, plus 1e-6


def shape_of(wl: W.Workload, tile_len: int = 128, tiled: bool = False):
    s = wl.shape
    return sdm.make_shape(wl.N, s.C, s.W, s.R, P=s.P, key_bits=s.key_bits, stream_offset=s.S,
                          first_partial=wl.first_partial, valid_last=wl.valid_last, tile_len=tile_len,
                          g_lane_stride=1 if wl.g.ndim == 3 else 0, idx_bytes=wl.k_idx.dtype.itemsize,
                          val_bytes=2 if wl.val_bf16 else 4, tiled=tiled)


def device_inputs(wl: W.Workload, dev="cuda"):
    import torch

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    vt = torch.bfloat16 if wl.val_bf16 else torch.float32   # (bfloat16-representable values: exact)
    return dict(k_idx=t(wl.k_idx), q_idx=t(wl.q_idx), k_val=t(wl.k_val).to(vt), q_val=t(wl.q_val).to(vt), g=t(wl.g))


def device_dv(wl: W.Workload, dev="cuda"):
    import torch

    dv = torch.from_numpy(np.ascontiguousarray(wl.dv.reshape(-1, wl.shape.hd))).to(dev)
    return dv.to(torch.bfloat16) if wl.shape.dv_dtype == "bf16" else dv


def run_phase1(wl: W.Workload, dev="cuda", tile_len=128, fields=None, tiled=False):
    """Phase 1 of every chunk on the device; `fields` adds optional outputs (e.g. "perm"); tiled:
    through the tiled path whatever the row length."""
    import torch

    shape = shape_of(wl, tile_len, tiled)
    ins = device_inputs(wl, dev)
    out = None
    if fields is not None:
        every = set(sdm.alloc_phase1_outputs(sdm.make_shape(0, 1, 1, 1), device="cpu"))
        out = sdm.alloc_phase1_outputs(shape, device=dev, fields=every | set(fields))
    out = sdm.phase1(shape, out=out, **ins)
    torch.cuda.synchronize()
    return shape, out


def oracle_phase1(wl: W.Workload, chunks, tile_len=128, threads=8, with_magnitudes=False, fields=None):
    if with_magnitudes:
        fields = list(oracle._OUT_FIELDS)
    return oracle.phase1(wl.k_idx, wl.q_idx, wl.k_val, wl.q_val, wl.g, P=wl.P, stream_offset=wl.stream_offset,
                         first_partial=wl.first_partial, valid_last=wl.valid_last, tile_len=tile_len, chunks=chunks,
                         threads=threads, fields=fields, val_bf16=wl.val_bf16)


def f32_violations(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    tol = np.maximum(F32_REL * np.abs(r), F32_ABS)
    return ~(np.abs(g - r) <= tol)


def assert_f32(name, gpu, ref):
    bad = f32_violations(gpu, ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        g = np.asarray(gpu, np.float64)
        r = np.asarray(ref, np.float64)
        det = ", ".join("%s: gpu %r oracle %r" % (tuple(i), g[tuple(i)], r[tuple(i)]) for i in idx)
        raise AssertionError("%s: %d of %d elements outside max(1e-5|o|, 1e-6): %s" % (name, bad.sum(), bad.size, det))


def assert_exact(name, gpu, ref):
    g = np.asarray(gpu).astype(np.int64)
    r = np.asarray(ref).astype(np.int64)
    if g.shape != r.shape or not np.array_equal(g, r):
        bad = np.argwhere(g != r)[:5] if g.shape == r.shape else []
        det = ", ".join("%s: gpu %d oracle %d" % (tuple(i), g[tuple(i)], r[tuple(i)]) for i in bad)
        raise AssertionError("%s differs (%s vs %s): %s" % (name, g.shape, r.shape, det))


def assert_pair_sums(name, gpu, ref, mag, cnt):
    """A / QK cells of stress shapes: max(1e-5|o|, 1e-6), or, where larger, the float32 evaluation
    bound of an n-term sum whose terms carry a few roundings each: (n + 4) 2^-23 sum|term|."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    tol = np.maximum(np.maximum(F32_REL * np.abs(r), F32_ABS), (cnt + 4.0) * 2.0 ** -23 * mag)
    bad = ~(np.abs(g - r) <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d cells outside the bound; %s: gpu %r oracle %r (terms %d, sum|t| %r)" % (
            name, bad.sum(), i, g[i], r[i], cnt[i], mag[i]))


def assert_bf16(name, gpu, ref):
    """bfloat16 results against the oracle's (the exact value rounded to bfloat16): the GPU rounds
    its float32 evaluation, which may sit on the other side of a rounding midpoint, so either
    bfloat16 neighbour of the exact value is correct: |gpu - o| <= one bfloat16 ulp of o."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert np.array_equal(g, oracle.round_bf16(g)), name + ": not bfloat16 values"
    bad = ~(np.abs(g - r) <= ulp_bf16(r))
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d elements more than one bfloat16 ulp away; %s: gpu %r oracle %r" % (
            name, bad.sum(), bad.size, i, g[i], r[i]))


VALUE_TYPED = ("cpe", "k_eff", "q_w")


def compare_phase1(out, ref, chunks):
    """Element-by-element comparison of GPU outputs (device dict) and oracle outputs (chunk list).

    With the oracle's per-cell magnitudes in `ref` (stress shapes), A and QK use the evaluation
    bound of assert_pair_sums; otherwise every float field uses max(1e-5|o|, 1e-6). bfloat16
    outputs (bfloat16 values: cpe, k_eff, q_w and krec's cpe) use assert_bf16."""
    import torch

    idx = torch.as_tensor(list(chunks), device=out["krec"].device, dtype=torch.long)
    bf = out["k_eff"].dtype == torch.bfloat16 if "k_eff" in out else False
    host = {k: (v.index_select(0, idx).float() if v.dtype == torch.bfloat16 else v.index_select(0, idx)).cpu().numpy()
            for k, v in out.items()}
    u32 = lambda a: np.asarray(a).astype(np.int64) & 0xFFFFFFFF  # noqa: E731
    for f in ("log_k", "rex", "cpe", "k_eff", "log_q", "q_w", "a", "qk"):
        if f in host:
            if bf and f in VALUE_TYPED:
                assert_bf16(f, host[f], ref[f])
            elif f in ("a", "qk") and (f + "_mag") in ref:
                assert_pair_sums(f, host[f], ref[f], ref[f + "_mag"], ref[f + "_cnt"])
            else:
                assert_f32(f, host[f], ref[f])
    for f in ("is_last", "is_only", "q_last", "q_only", "pos_k", "pos_q", "tiles_k", "repeats", "perm"):
        if f in host:
            assert_exact(f, host[f], ref[f])
    assert_exact("spay_k", u32(host["spay_k"]), u32(ref["spay_k"]))
    if "spay_q" in host:
        assert_exact("spay_q", u32(host["spay_q"]), u32(ref["spay_q"]))
    kr = host["krec"]
    assert_exact("krec.element", u32(kr[..., 0]), u32(ref["spay_k"]))
    assert_exact("krec.slot", kr[..., 1], ref["krec_slot"])
    assert_f32("krec.scale", kr[..., 2].view(np.float32), ref["krec_sc"])
    (assert_bf16 if bf else assert_f32)("krec.cpe", kr[..., 3].view(np.float32), ref["krec_cpe"])


def ulp_bf16(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -133)))
    return 2.0 ** (np.maximum(e, -126) - 7)


def bank_violations(gpu_rows, new, mag, members, bank_dtype, cpe_slack=None):
    """Rows of the GPU bank against the oracle's new rows (float64).

    The float32 evaluation of an m-member chain with float32 scales is within
    (m + 4) 2^-23 times the sum of the term magnitudes (`mag`) of the exact value. float32 bank:
    max(1e-5|o|, 1e-6), or that evaluation bound where it is larger (long chains that cancel).
    bf16 bank: one bf16 ulp of max(|gpu|, |o|) for the final rounding plus the evaluation bound.
    cpe_slack (bfloat16 values): per element, |base| times one bfloat16 ulp of the group's cpe,
    added to both bounds (the record's cpe may be the other bfloat16 neighbour of exp(G))."""
    g = np.asarray(gpu_rows, np.float64)
    arith = (np.asarray(members, np.float64)[:, None] + 4.0) * 2.0 ** -23 * mag
    if cpe_slack is not None:
        arith = arith + cpe_slack
    if bank_dtype == "f32":
        tol = np.maximum(np.maximum(F32_REL * np.abs(new), F32_ABS), arith)
        return ~(np.abs(g - new) <= tol)
    tol = ulp_bf16(np.maximum(np.abs(g), np.abs(new))) + arith
    return ~(np.abs(g - new) <= tol)


def chunk_members(wl, c):
    """Valid K members per valid group of chunk c, in dw_slots order (counts only)."""
    C = wl.shape.C
    tv = wl.valid_last if c >= wl.first_partial else C
    ids = wl.k_idx[c, :tv].ravel().astype(np.int64)
    u, cnt = np.unique(ids, return_counts=True)
    return u, cnt


def run_dw_check(wl: W.Workload, out, shape, check_steps, dev="cuda", sample_untouched=20000, seed=0,
                 split=True):
    """Run every DW step on the GPU; at the steps in check_steps, first copy the oracle's state of
    the touched rows into the GPU bank, then compare the GPU result with the oracle's. Returns the
    number of elements compared."""
    import torch

    sh = wl.shape
    P, C, hd = sh.P, sh.C, sh.hd
    bank = W.make_bank(wl, dev)
    shadow = bank.clone()          # the oracle's bank state (generator rows, then oracle rows)
    dv = device_dv(wl, dev)
    dv_host = wl.dv.reshape(-1, hd).astype(np.float64)
    ws = sdm.alloc_dw_workspace(shape, hd, device=dev) if split else None
    touched = set()
    compared = 0
    for ti in range(wl.steps):
        check = ti in check_steps
        per = []
        for p in range(P):
            c = ti * P + p
            slots = oracle.dw_slots(wl.k_idx, wl.q_idx, wl.k_val, wl.q_val, wl.g, c, P=P, stream_offset=sh.S,
                                    first_partial=wl.first_partial, valid_last=wl.valid_last)
            per.append((c, slots))
        all_slots = torch.as_tensor(np.concatenate([s for _, s in per]), device=dev, dtype=torch.long)
        base_all = shadow.index_select(0, all_slots)
        if check:
            bank.index_copy_(0, all_slots, base_all)
        sdm.dw_step(bank, dv, out["krec"], shape, ti, dv_step_rows=P * C, workspace=ws)
        base_host = base_all.float().cpu().numpy().astype(np.float64)
        if check:
            torch.cuda.synchronize()
            got_all = bank.index_select(0, all_slots).float().cpu().numpy()
        off = 0
        news = []
        for c, slots in per:
            m = len(slots)
            rows = dv_host[c * C:(c + 1) * C]
            okw = dict(P=P, stream_offset=sh.S, first_partial=wl.first_partial, valid_last=wl.valid_last,
                       val_bf16=wl.val_bf16)
            new, mag = oracle.dw_apply(wl.k_idx, wl.q_idx, wl.k_val, wl.q_val, wl.g, c, rows, base_host[off:off + m],
                                       with_magnitude=True, **okw)
            slack = None
            if wl.val_bf16 and check:   # the groups' rounded cpe: base rows of ones, no token rows
                cpe = oracle.dw_apply(wl.k_idx, wl.q_idx, wl.k_val, wl.q_val, wl.g, c, np.zeros((C, 1)),
                                      np.ones((m, 1)), **okw)
                slack = np.abs(base_host[off:off + m]) * ulp_bf16(cpe)
            if check:
                u, cnt = chunk_members(wl, c)
                assert np.array_equal(u, slots)
                bad = bank_violations(got_all[off:off + m], new, mag, cnt, sh.bank_dtype, slack)
                if bad.any():
                    i = np.argwhere(bad)[0]
                    raise AssertionError("DW step %d chunk %d: %d of %d elements outside tolerance; slot %d col %d: "
                                         "gpu %r oracle %r" % (ti, c, bad.sum(), bad.size, slots[i[0]], i[1],
                                                               got_all[off + i[0], i[1]], new[i[0], i[1]]))
                compared += bad.size
            news.append(new)
            touched.update(slots.tolist())
            off += m
        new_all = torch.from_numpy(np.concatenate(news).astype(np.float32)).to(dev)
        shadow.index_copy_(0, all_slots, new_all.to(shadow.dtype))
    # Rows no group touched keep their initial bits.
    rng = np.random.default_rng(seed)
    cand = rng.integers(0, wl.rows, size=sample_untouched * 2)
    cand = np.array([r for r in cand if int(r) not in touched][:sample_untouched], dtype=np.int64)
    if cand.size:
        idx = torch.as_tensor(cand, device=dev)
        init = W.make_bank_rows(wl, cand, dev)
        assert torch.equal(bank.index_select(0, idx), init), "untouched rows changed"
    if ws is not None:   # the split path leaves its counters at zero
        torch.cuda.synchronize()
        cnt_bytes = (shape.P * shape.C * shape.W + 31) // 32 * 4   # one counter per block of 32 positions
        assert int(ws[:cnt_bytes].view(torch.int32).abs().sum()) == 0, "DW arrival counters not reset"
    return compared, bank


def run_read_check(wl, steps_checked, chunks_per_step=None, dev="cuda"):
    """Phase 1, then the read side of the checked steps from the initial bank; compare with the oracle
    (tolerance READ_RTOL_MAG times the oracle's magnitude bound, plus 1e-6; masked tokens exactly 0).
    Returns the worst error relative to the magnitude bound."""
    import torch

    sh = wl.shape
    P, C, hd = sh.P, sh.C, sh.hd
    shape, out = run_phase1(wl, dev=dev)
    ins = device_inputs(wl, dev)
    v_host, beta_host = W.make_read_inputs(wl)
    v = torch.from_numpy(v_host).to(dev)
    beta = torch.from_numpy(beta_host).to(dev)
    rows = v.shape[0]
    dv = torch.full((rows, hd), float("nan"), device=dev)
    pred = torch.full_like(dv, float("nan"))
    read = torch.full_like(dv, float("nan"))
    bank = W.make_bank(wl, dev)
    plan = sdm.ReadPlan(bank, out, ins["k_idx"], ins["q_idx"], v, beta, dv, pred, read, shape, step_rows=P * C)
    for ti in steps_checked:
        plan.step(ti)
    torch.cuda.synchronize()
    worst = 0.0
    for ti in steps_checked:
        for p in range(P) if chunks_per_step is None else range(min(P, chunks_per_step)):
            c = ti * P + p
            o = oracle_phase1(wl, [c], fields=["k_eff", "q_w", "a", "qk"])
            tv = wl.valid_last if c >= wl.first_partial else C
            rows_of = lambda s: bank.index_select(0, torch.as_tensor(s, device=dev)).float().cpu().numpy().astype(np.float64)  # noqa: E731
            r = read_side.read_step(wl.k_idx[c], wl.q_idx[c], o["k_eff"][0], o["q_w"][0], o["a"][0], o["qk"][0],
                                    v_host[c * C:(c + 1) * C], beta_host[c], rows_of, tv)
            sl = slice(ti * P * C + p * C, ti * P * C + (p + 1) * C)
            for name, got in (("dv", dv), ("pred", pred), ("read", read)):
                g = got[sl].cpu().numpy().astype(np.float64)
                want = r[name]
                tol = READ_RTOL_MAG * r["mag_" + name] + 1e-6
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


U32 = 2.0 ** -24   # unit roundoff of float32


def read_fed_tolerance(C, W, R, mag):
    """Float32 evaluation bound of the read side on exact float32 inputs: each output is a chain of
    dots (a gather of at most max(W, R) terms, then a forward substitution and products with A and
    QK of at most C terms) whose every rounding error is propagated by the same triangular
    recursion that builds the oracle's magnitude bound `mag` (the recursion on absolute values
    majorizes the inverse of the unit lower triangular system elementwise). So the error is at most
    gamma_n mag per stage, with n = C + max(W, R); twice that for the two stages that can compound
    (the blocked substitution applies an inverted diagonal block, then the off-diagonal products)."""
    n = C + max(W, R)
    gamma = n * U32 / (1.0 - n * U32)
    return 2.0 * gamma * mag


def run_read_check_fed(wl, steps_checked, dev="cuda"):
    """The read side fed the ORACLE's Phase-1 quantities (k_eff, q_w, A, QK, each rounded once to
    float32) instead of the GPU's, so the comparison isolates the read kernels: the oracle's read
    side is evaluated in float64 on the same float32 inputs and the same pre-step bank rows, and
    every dv / pred / read element must lie within read_fed_tolerance. Returns the worst error as a
    fraction of that tolerance."""
    import torch

    sh = wl.shape
    P, C, Wn, R, hd = sh.P, sh.C, sh.W, sh.R, sh.hd
    shape = shape_of(wl)
    ins = device_inputs(wl, dev)
    fed = {"k_eff": np.zeros((wl.N, C, Wn), np.float32), "q_w": np.zeros((wl.N, C, R), np.float32),
           "a": np.zeros((wl.N, C, C), np.float32), "qk": np.zeros((wl.N, C, C), np.float32)}
    chunks = [ti * P + p for ti in steps_checked for p in range(P)]
    o = oracle_phase1(wl, chunks, fields=["k_eff", "q_w", "a", "qk"])
    for i, c in enumerate(chunks):
        for k in fed:
            fed[k][c] = np.asarray(o[k][i], np.float64).astype(np.float32)
    p1 = {k: torch.from_numpy(v).to(dev) for k, v in fed.items()}
    v_host, beta_host = W.make_read_inputs(wl)
    v = torch.from_numpy(v_host).to(dev)
    beta = torch.from_numpy(beta_host).to(dev)
    rows = v.shape[0]
    dv = torch.full((rows, hd), float("nan"), device=dev)
    pred = torch.full_like(dv, float("nan"))
    read = torch.full_like(dv, float("nan"))
    bank = W.make_bank(wl, dev)
    plan = sdm.ReadPlan(bank, p1, ins["k_idx"], ins["q_idx"], v, beta, dv, pred, read, shape, step_rows=P * C)
    for ti in steps_checked:
        plan.step(ti)
    torch.cuda.synchronize()
    worst = 0.0
    rows_of = lambda s: bank.index_select(0, torch.as_tensor(s, device=dev)).float().cpu().numpy().astype(np.float64)  # noqa: E731
    for c in chunks:
        ti, p = divmod(c, P)
        tv = wl.valid_last if c >= wl.first_partial else C
        r = read_side.read_step(wl.k_idx[c], wl.q_idx[c], fed["k_eff"][c], fed["q_w"][c], fed["a"][c], fed["qk"][c],
                                v_host[c * C:(c + 1) * C], beta_host[c], rows_of, tv)
        sl = slice(ti * P * C + p * C, ti * P * C + (p + 1) * C)
        for name, got in (("dv", dv), ("pred", pred), ("read", read)):
            g = got[sl].cpu().numpy().astype(np.float64)
            want = r[name]
            tol = read_fed_tolerance(C, Wn, R, r["mag_" + name])
            err = np.abs(g - want)
            bad = ~(err <= tol)
            if bad.any():
                i = np.argwhere(bad)[:4]
                raise AssertionError("%s (oracle-fed) step %d stream %d: %d of %d outside the float32 bound; e.g. %s" % (
                    name, ti, p, bad.sum(), bad.size,
                    ", ".join("%s gpu %r oracle %r tol %r" % (tuple(k), g[tuple(k)], want[tuple(k)], tol[tuple(k)])
                              for k in i)))
            nz = tol > 0
            if nz.any():
                worst = max(worst, float(np.max(err[nz] / tol[nz])))
            assert np.all(g[tv:] == 0), name
    return worst


def pa_counter_bytes(shape):
    """Bytes of the PA workspace's arrival counters (its first region): one int per block of 32 K-row
    positions of a step."""
    return -(-shape.P * shape.C * shape.W // 32) * 4
