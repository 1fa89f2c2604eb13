"""Pins of the CPU oracle against facts other than itself (CPU only).

Each test checks the oracle (oracle/sdm_oracle.c) against something it does not share code
with: brute-force evaluation of the definitions on tiny inputs (O(n^2) rank counting and pair
enumeration), library routines (numpy.lexsort, numpy.cumsum, numpy.add.at), closed forms of
special cases, invariants, and a token-by-token simulation of decay-then-write whose identities
follow from the definitions on the page "sparse_delta_memory/cuda/phase1_cuda.py" (module
docstring) and the DW definition on "sparse_delta_memory/cuda/mover_da2_cuda.py" (module
docstring).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(seed, N=2, C=10, W=3, R=2, S=4, P=1, g=None, valid_last=None, distinct=False, lane_gates=False):
    rng = np.random.default_rng(seed)
    stream = (np.arange(N) % P)[:, None, None] * S
    if distinct:
        ids = rng.permutation(S)[: N * C * (W + R)].reshape(N, C, W + R)
        k_idx = (ids[:, :, :W] + stream).astype(np.int32)
        q_idx = (ids[:, :, W:] + stream).astype(np.int32)
    else:
        k_idx = (rng.integers(0, S, (N, C, W)) + stream).astype(np.int32)
        q_idx = (rng.integers(0, S, (N, C, R)) + stream).astype(np.int32)
    k_val = (rng.standard_normal((N, C, W)) / 2).astype(np.float32)
    q_val = (rng.standard_normal((N, C, R)) / 2).astype(np.float32)
    if g is None:
        # one gate per token [N, C], or per (token, K lane) [N, C, W]
        z = rng.standard_normal((N, C, W) if lane_gates else (N, C)) + 2.0
        g = (-np.log1p(np.exp(-z))).astype(np.float32)
    fp = N - P if valid_last is not None else N
    vl = C if valid_last is None else valid_last
    return dict(k_idx=k_idx, q_idx=q_idx, k_val=k_val, q_val=q_val, g=np.asarray(g, np.float32),
                P=P, stream_offset=S, first_partial=fp, valid_last=vl)


def run_oracle(d, **kw):
    return oracle.phase1(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], P=d["P"],
                         stream_offset=d["stream_offset"], first_partial=d["first_partial"],
                         valid_last=d["valid_last"], **kw)


def entries(d, c):
    """Brute-force entry table of chunk c: r, token, lane, is_q, local slot, valid, value."""
    C, W = d["k_idx"].shape[1:]
    R = d["q_idx"].shape[2]
    tv = d["valid_last"] if c >= d["first_partial"] else C
    base = (c % d["P"]) * d["stream_offset"]
    out = []
    for t in range(C):
        for j in range(W + R):
            q = j >= W
            lane = j - W if q else j
            idv = int(d["q_idx"][c, t, lane] if q else d["k_idx"][c, t, lane])
            val = float(d["q_val"][c, t, lane] if q else d["k_val"][c, t, lane])
            out.append(dict(r=t * (W + R) + j, t=t, lane=lane, q=q, s=idv - base, valid=t < tv, v=val))
    return out


def brute(d, c):
    """Everything Phase 1 defines, evaluated by brute force from the definitions (O(n^2))."""
    E = entries(d, c)
    n = len(E)
    g = d["g"][c].astype(np.float64)
    order_key = [(0 if e["valid"] else 1, e["s"] if e["valid"] else 0, e["r"]) for e in E]
    rho = [sum(1 for f in range(n) if order_key[f] < order_key[e]) for e in range(n)]
    for e in E:
        e["x"] = 0.0
    for ei, e in enumerate(E):
        if not e["valid"] or e["q"]:
            continue
        # A token's gate counts once per slot: at its lowest K lane on that slot (per-lane gates:
        # that lane's gate).
        lower = [f for f in E if f["valid"] and not f["q"] and f["t"] == e["t"] and f["s"] == e["s"]
                 and f["lane"] < e["lane"]]
        gate = float(g[e["t"]]) if g.ndim == 1 else float(g[e["t"], e["lane"]])
        e["x"] = 0.0 if lower else gate
    res = []
    for ei, e in enumerate(E):
        if not e["valid"]:
            res.append(dict(rho=rho[ei], L=0.0, rex=0.0, kb=0, ka=0, qb=0, qa=0, G=0.0))
            continue
        peers = [f for f in E if f["valid"] and f["s"] == e["s"]]
        L = sum(f["x"] for f in peers if f["r"] <= e["r"])
        rex = sum(f["x"] for f in peers if f["r"] > e["r"])
        kb = sum(1 for f in peers if not f["q"] and f["r"] < e["r"])
        ka = sum(1 for f in peers if not f["q"] and f["r"] > e["r"])
        qb = sum(1 for f in peers if f["q"] and f["r"] < e["r"])
        qa = sum(1 for f in peers if f["q"] and f["r"] > e["r"])
        res.append(dict(rho=rho[ei], L=L, rex=rex, kb=kb, ka=ka, qb=qb, qa=qa, G=L + rex))
    return E, res


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_sort_matches_brute_force_and_lexsort(seed):
    d = tiny(seed, N=3, C=9, W=3, R=2, S=5, P=1, valid_last=6)
    o = run_oracle(d, fields=["perm"])
    for c in range(3):
        E, res = brute(d, c)
        inv = np.empty(len(E), np.int64)
        inv[o["perm"][c]] = np.arange(len(E))
        assert [r["rho"] for r in res] == inv.tolist()
        # Library routine: lexsort on (invalid, slot, r) gives the same permutation.
        invalid = np.array([0 if e["valid"] else 1 for e in E])
        slot = np.array([e["s"] if e["valid"] else 0 for e in E])
        rr = np.array([e["r"] for e in E])
        assert np.array_equal(np.lexsort((rr, slot, invalid)), o["perm"][c])


@pytest.mark.parametrize("seed,lane_gates", [(4, False), (5, False), (41, True), (42, True)])
def test_scan_fields_match_brute_force(seed, lane_gates):
    d = tiny(seed, N=2, C=11, W=4, R=3, S=6, P=2, valid_last=7, lane_gates=lane_gates)
    o = run_oracle(d, fields=list(oracle._OUT_FIELDS))
    C, W = d["k_idx"].shape[1:]
    R = d["q_idx"].shape[2]
    for c in range(2):
        E, res = brute(d, c)
        # repeats: valid K entries whose token writes the same slot from a lower K lane (so the
        # entry before it in its group is a K entry of its own token, and its gate is not applied).
        reps = sum(1 for e in E if e["valid"] and not e["q"] and any(
            f["valid"] and not f["q"] and f["t"] == e["t"] and f["s"] == e["s"] and f["lane"] < e["lane"] for f in E))
        assert int(o["repeats"][c]) == reps
        for e, b in zip(E, res):
            o_idx = (e["t"], e["lane"])
            packed = b["rho"]
            before, after = (b["qb"], b["qa"]) if e["q"] else (b["kb"], b["ka"])
            if e["valid"]:
                packed |= min(after, 127) << 17 | min(before + 1 + after, 127) << 24
            if e["q"]:
                assert o["pos_q"][c][o_idx] == packed
                assert o["log_q"][c][o_idx] == pytest.approx(b["L"], abs=1e-12)
                want_qw = e["v"] * math.exp(b["L"]) if e["valid"] else 0.0
                assert o["q_w"][c][o_idx] == pytest.approx(want_qw, rel=1e-12, abs=1e-300)
                assert o["q_last"][c][o_idx] == int(e["valid"] and after == 0)
                assert o["q_only"][c][o_idx] == int(e["valid"] and after == 0 and before == 0)
            else:
                assert o["pos_k"][c][o_idx] == packed
                assert o["log_k"][c][o_idx] == pytest.approx(b["L"], abs=1e-12)
                assert o["rex"][c][o_idx] == pytest.approx(b["rex"], abs=1e-12)
                want_cpe = math.exp(b["G"]) if e["valid"] else 1.0
                assert o["cpe"][c][o_idx] == pytest.approx(want_cpe, rel=1e-12)
                want_keff = e["v"] * math.exp(b["L"]) if e["valid"] else 0.0
                assert o["k_eff"][c][o_idx] == pytest.approx(want_keff, rel=1e-12, abs=1e-300)
                assert o["is_last"][c][o_idx] == int(e["valid"] and after == 0)
                assert o["is_only"][c][o_idx] == int(e["valid"] and after == 0 and before == 0)
        # Kind rows, records and tile bounds.
        kind_rank = {}
        for q in (False, True):
            members = sorted([i for i, e in enumerate(E) if e["q"] == q], key=lambda i: res[i]["rho"])
            for j, i in enumerate(members):
                kind_rank[i] = j
        nk = C * W
        for i, e in enumerate(E):
            b = res[i]
            before, after = (b["qb"], b["qa"]) if e["q"] else (b["kb"], b["ka"])
            pay = e["lane"] | (0x100 if e["q"] else 0) | e["t"] << 9 | (0 if e["valid"] else 0x20000)
            if e["valid"]:
                elem = pay | min(before, 4095) << 18 | (0x80000000 if before == 0 else 0) | (0x40000000 if after == 0 else 0)
            else:
                elem = pay | 0x80000000 | 0x40000000
            row = o["spay_q"][c] if e["q"] else o["spay_k"][c]
            assert (int(row[kind_rank[i]]) & 0xFFFFFFFF) == elem
            if not e["q"]:
                j = kind_rank[i]
                base = (c % d["P"]) * d["stream_offset"]
                assert o["krec_slot"][c][j] == ((e["s"] + base) if e["valid"] else 0)
                want_sc = e["v"] * math.exp(b["rex"]) if e["valid"] else 0.0
                assert o["krec_sc"][c][j] == pytest.approx(want_sc, rel=1e-12, abs=1e-300)
                assert o["krec_cpe"][c][j] == pytest.approx(math.exp(b["G"]) if e["valid"] else 1.0, rel=1e-12)
        L = 128
        firsts = [j for j in range(nk) if int(o["spay_k"][c][j]) & 0x80000000]
        ntk = (nk + L - 1) // L
        want = [min([j for j in firsts if j >= t * L], default=nk) for t in range(ntk)] + [nk]
        assert o["tiles_k"][c].tolist() == want


@pytest.mark.parametrize("seed,lane_gates", [(6, False), (7, False), (61, True)])
def test_pairs_match_brute_force(seed, lane_gates):
    d = tiny(seed, N=2, C=8, W=3, R=3, S=3, P=1, valid_last=5, lane_gates=lane_gates)
    o = run_oracle(d, fields=["a", "qk", "a_mag", "qk_mag", "a_cnt", "qk_cnt"])
    C = d["k_idx"].shape[1]
    for c in range(2):
        E, res = brute(d, c)
        A = np.zeros((C, C))
        QK = np.zeros((C, C))
        cnt = {"a": np.zeros((C, C), int), "qk": np.zeros((C, C), int)}
        mag = {"a": np.zeros((C, C)), "qk": np.zeros((C, C))}
        for ei, e in enumerate(E):
            for fi, f in enumerate(E):
                if not (e["valid"] and f["valid"]) or f["q"] or e["s"] != f["s"]:
                    continue
                term = e["v"] * f["v"] * math.exp(res[ei]["L"] - res[fi]["L"])
                if e["q"] and f["t"] <= e["t"]:
                    QK[e["t"], f["t"]] += term
                    cnt["qk"][e["t"], f["t"]] += 1
                    mag["qk"][e["t"], f["t"]] += abs(term)
                if not e["q"] and f["t"] < e["t"]:
                    A[e["t"], f["t"]] += term
                    cnt["a"][e["t"], f["t"]] += 1
                    mag["a"][e["t"], f["t"]] += abs(term)
        np.testing.assert_allclose(o["a"][c], A, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(o["qk"][c], QK, rtol=1e-12, atol=1e-15)
        for k in ("a", "qk"):
            assert np.array_equal(o[k + "_cnt"][c], cnt[k])
            np.testing.assert_allclose(o[k + "_mag"][c], mag[k], rtol=1e-12, atol=1e-15)


def test_invariants_groups():
    d = tiny(11, N=3, C=40, W=6, R=5, S=13, P=1, valid_last=31)
    o = run_oracle(d)
    for c in range(3):
        G = o["log_k"][c] + o["rex"][c]
        slots = d["k_idx"][c]
        tv = d["valid_last"] if c >= d["first_partial"] else 40
        for s in np.unique(slots[:tv]):
            m = slots[:tv] == s
            # rex + log_k is the slot's total gate for every K entry of the slot.
            assert np.ptp(G[:tv][m]) < 1e-12
            assert np.allclose(o["cpe"][c][:tv][m], np.exp(G[:tv][m][0]), rtol=1e-12)
            # cpe = exp(log_k at the slot's last K entry); exactly one last entry per slot.
            last = m & (o["is_last"][c][:tv] == 1)
            assert last.sum() == 1
            assert np.allclose(o["cpe"][c][:tv][m], np.exp(o["log_k"][c][:tv][last][0]), rtol=1e-12)
        # Invalid tokens: log 0, rex 0, cpe 1, k_eff 0, no flags, position only.
        assert np.all(o["log_k"][c][tv:] == 0) and np.all(o["cpe"][c][tv:] == 1) and np.all(o["k_eff"][c][tv:] == 0)
        assert np.all(o["is_last"][c][tv:] == 0) and np.all((o["pos_k"][c][tv:] >> 17) == 0)
        # The sorted position is a permutation of the chunk's entries.
        pos = np.concatenate([o["pos_k"][c].ravel(), o["pos_q"][c].ravel()]) & ((1 << 17) - 1)
        assert np.array_equal(np.sort(pos), np.arange(pos.size))


def test_closed_form_distinct_slots():
    d = tiny(12, N=2, C=16, W=3, R=2, S=4096, P=1, distinct=True)
    o = run_oracle(d)
    g = d["g"].astype(np.float64)
    for c in range(2):
        np.testing.assert_allclose(o["log_k"][c], np.repeat(g[c][:, None], 3, 1), rtol=0, atol=0)
        assert np.all(o["rex"][c] == 0) and np.all(o["log_q"][c] == 0)
        np.testing.assert_allclose(o["cpe"][c], np.exp(np.repeat(g[c][:, None], 3, 1)), rtol=1e-15)
        assert np.array_equal(o["q_w"][c], d["q_val"][c].astype(np.float64))
        assert np.all(o["a"][c] == 0) and np.all(o["qk"][c] == 0)
        assert np.all(o["is_only"][c] == 1) and np.all(o["q_only"][c] == 1)


def test_closed_form_one_slot_cumsum():
    C = 24
    rng = np.random.default_rng(13)
    z = rng.standard_normal((1, C)) + 2.0
    g = (-np.log1p(np.exp(-z))).astype(np.float32)
    d = tiny(13, N=1, C=C, W=1, R=1, S=1, P=1, g=g)
    o = run_oracle(d)
    cs = np.cumsum(g[0].astype(np.float64))
    k = d["k_val"][0, :, 0].astype(np.float64)
    q = d["q_val"][0, :, 0].astype(np.float64)
    np.testing.assert_allclose(o["log_k"][0, :, 0], cs, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o["log_q"][0, :, 0], cs, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o["rex"][0, :, 0], cs[-1] - cs, rtol=1e-12, atol=1e-12)
    dec = np.exp(cs[:, None] - cs[None, :])
    np.testing.assert_allclose(o["a"][0], np.tril(np.outer(k, k) * dec, -1), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o["qk"][0], np.tril(np.outer(q, k) * dec, 0), rtol=1e-12, atol=1e-15)


def test_golden_worked_example():
    """A hand-worked three-token example (tests/golden/one_slot_worked.json)."""
    with open(os.path.join(GOLDEN, "one_slot_worked.json")) as f:
        gd = json.load(f)
    C = len(gd["g"])
    d = dict(k_idx=np.zeros((1, C, 1), np.int32), q_idx=np.zeros((1, C, 1), np.int32),
             k_val=np.array(gd["k"], np.float32).reshape(1, C, 1), q_val=np.array(gd["q"], np.float32).reshape(1, C, 1),
             g=np.array(gd["g"], np.float32).reshape(1, C), P=1, stream_offset=0, first_partial=1, valid_last=C)
    o = run_oracle(d)
    ev = lambda s: eval(s, {"exp": math.exp})  # noqa: E731 - fixture expressions are plain arithmetic
    np.testing.assert_allclose(o["log_k"][0, :, 0], gd["log_k"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o["rex"][0, :, 0], gd["rex"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o["cpe"][0, :, 0], [ev(s) for s in gd["cpe"]], rtol=1e-15)
    np.testing.assert_allclose(o["a"][0], [[ev(s) for s in row] for row in gd["a"]], rtol=1e-15, atol=0)
    np.testing.assert_allclose(o["qk"][0], [[ev(s) for s in row] for row in gd["qk"]], rtol=1e-15, atol=0)
    assert o["pos_k"][0, :, 0].tolist() == gd["pos_k"]
    assert (o["spay_k"][0].astype(np.int64) & 0xFFFFFFFF).tolist() == gd["spay_k"]


def test_zero_gates():
    d = tiny(14, N=2, C=20, W=4, R=3, S=5, P=1, g=np.zeros((2, 20), np.float32))
    o = run_oracle(d)
    assert np.all(o["log_k"] == 0) and np.all(o["log_q"] == 0) and np.all(o["rex"] == 0)
    assert np.all(o["cpe"] == 1)
    assert np.array_equal(o["k_eff"], d["k_val"].astype(np.float64))
    assert np.array_equal(o["q_w"], d["q_val"].astype(np.float64))


def test_dw_zero_gates_is_scatter_add():
    d = tiny(15, N=2, C=16, W=4, R=2, S=7, P=2, g=np.zeros((2, 16), np.float32))
    hd = 5
    rng = np.random.default_rng(15)
    for c in range(2):
        slots = oracle.dw_slots(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], c, P=2, stream_offset=7)
        bank = rng.standard_normal((14, hd))
        dv = rng.standard_normal((16, hd))
        new = oracle.dw_apply(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], c, dv, bank[slots],
                              P=2, stream_offset=7)
        want = bank.copy()
        k = d["k_val"][c].astype(np.float64)
        np.add.at(want, d["k_idx"][c].ravel(), (k[:, :, None] * dv[:, None, :]).reshape(-1, hd))
        assert np.array_equal(np.unique(d["k_idx"][c]), slots)
        np.testing.assert_allclose(new, want[slots], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed,S,W,R,vl,lane_gates", [(21, 3, 3, 2, None, False), (22, 5, 4, 4, 9, False),
                                                      (23, 2, 2, 1, None, False), (24, 9, 5, 3, 4, False),
                                                      (25, 3, 4, 2, None, True), (26, 6, 5, 3, 8, True)])
def test_sequential_simulation_identities(seed, S, W, R, vl, lane_gates):
    """Token-by-token decay-then-write equals DW, and its predictions / reads equal the
    Phase-1 decomposition through k_eff, q_w, A and QK. With per-lane gates a token decays each
    slot it writes once, by the gate of its lowest lane writing that slot."""
    C, hd = 14, 3
    d = tiny(seed, N=2, C=C, W=W, R=R, S=S, P=1, valid_last=vl, lane_gates=lane_gates)
    o = run_oracle(d)
    rng = np.random.default_rng(seed)
    for c in range(2):
        tv = d["valid_last"] if c >= d["first_partial"] else C
        M0 = rng.standard_normal((S, hd))
        dv = rng.standard_normal((C, hd))
        dv[tv:] = np.nan  # invalid tokens' rows are never used
        M = M0.copy()
        g = d["g"][c].astype(np.float64)
        kv = d["k_val"][c].astype(np.float64)
        qv = d["q_val"][c].astype(np.float64)
        ks, qs = d["k_idx"][c], d["q_idx"][c]
        for t in range(tv):
            for s in np.unique(ks[t]):
                lowest = int(np.flatnonzero(ks[t] == s)[0])
                M[s] *= math.exp(g[t, lowest] if lane_gates else g[t])
            pred = sum(kv[t, e] * M[ks[t, e]] for e in range(W))
            for e in range(W):
                M[ks[t, e]] += kv[t, e] * dv[t]
            read = sum(qv[t, r] * M[qs[t, r]] for r in range(R))
            want_pred = sum(o["k_eff"][c][t, e] * M0[ks[t, e]] for e in range(W)) + \
                sum(o["a"][c][t, j] * dv[j] for j in range(t))
            want_read = sum(o["q_w"][c][t, r] * M0[qs[t, r]] for r in range(R)) + \
                sum(o["qk"][c][t, j] * dv[j] for j in range(t + 1))
            np.testing.assert_allclose(pred, want_pred, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(read, want_read, rtol=1e-11, atol=1e-11)
        slots = oracle.dw_slots(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], c, P=1, stream_offset=S,
                                first_partial=d["first_partial"], valid_last=d["valid_last"])
        new = oracle.dw_apply(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], c, dv, M0[slots], P=1, stream_offset=S, first_partial=d["first_partial"], valid_last=d["valid_last"])
        np.testing.assert_allclose(new, M[slots], rtol=1e-12, atol=1e-12)
        untouched = np.setdiff1d(np.arange(S), slots)
        assert np.array_equal(M[untouched], M0[untouched])


def test_lane_gates_equal_to_token_gates():
    """Per-lane gates that repeat the token's gate on every lane give exactly the per-token result."""
    d = tiny(31, N=3, C=20, W=4, R=3, S=6, P=1, valid_last=13)
    o = run_oracle(d)
    d3 = dict(d, g=np.repeat(d["g"][:, :, None], 4, axis=2))
    o3 = run_oracle(d3)
    for k in o:
        assert np.array_equal(o[k], o3[k]), k


def test_closed_form_distinct_slots_lane_gates():
    """All slots distinct: each K entry is alone in its group, so log_k = its own lane's gate."""
    d = tiny(32, N=2, C=16, W=3, R=2, S=4096, P=1, distinct=True, lane_gates=True)
    o = run_oracle(d)
    g = d["g"].astype(np.float64)
    for c in range(2):
        np.testing.assert_array_equal(o["log_k"][c], g[c])
        assert np.all(o["rex"][c] == 0) and np.all(o["log_q"][c] == 0)
        np.testing.assert_allclose(o["cpe"][c], np.exp(g[c]), rtol=1e-15)


def test_lane_gates_lowest_lane_applies():
    """One token writing one slot from lanes 0 and 2 (lane 1 elsewhere): the slot's gate is lane 0's
    and lane 2 is a repeat; lane 1's own slot takes lane 1's gate."""
    k_idx = np.array([[[5, 7, 5]]], np.int32)
    q_idx = np.array([[[5]]], np.int32)
    g = np.array([[[-0.5, -0.25, -2.0]]], np.float32)
    d = dict(k_idx=k_idx, q_idx=q_idx, k_val=np.ones((1, 1, 3), np.float32), q_val=np.ones((1, 1, 1), np.float32),
             g=g, P=1, stream_offset=0, first_partial=1, valid_last=1)
    o = run_oracle(d)
    assert o["log_k"][0, 0].tolist() == [-0.5, -0.25, -0.5]
    assert o["log_q"][0, 0, 0] == -0.5
    assert o["repeats"][0] == 1
    assert o["cpe"][0, 0, 0] == pytest.approx(math.exp(-0.5), rel=1e-15)


@pytest.mark.parametrize("seed,S,vl", [(91, 5, None), (92, 40, 7), (93, 3000, None)])
def test_group_ordinals_brute_force(seed, S, vl):
    """gord_k: at every valid K-row position, the index of its slot among the chunk's distinct valid
    write slots in ascending order (np.unique of the valid K ids, computed here), -1 at padding."""
    rng = np.random.default_rng(seed)
    N, C, W, R = 2, 24, 3, 2
    k_idx = rng.integers(0, S, (N, C, W)).astype(np.int32)
    q_idx = rng.integers(0, S, (N, C, R)).astype(np.int32)
    k_val = rng.standard_normal((N, C, W)).astype(np.float32)
    q_val = rng.standard_normal((N, C, R)).astype(np.float32)
    g = (-rng.random((N, C)) * 0.5).astype(np.float32)
    fp = N - 1 if vl is not None else N
    o = oracle.phase1(k_idx, q_idx, k_val, q_val, g, first_partial=fp, valid_last=C if vl is None else vl,
                      fields=["gord_k", "krec_slot", "spay_k"])
    for c in range(N):
        tv = vl if (vl is not None and c >= fp) else C
        distinct = np.unique(k_idx[c, :tv].ravel())
        pad = ((o["spay_k"][c].astype(np.int64) >> 17) & 1).astype(bool)
        assert np.all(o["gord_k"][c][pad] == -1)
        want = np.searchsorted(distinct, o["krec_slot"][c][~pad])
        np.testing.assert_array_equal(o["gord_k"][c][~pad], want)
        assert (~pad).sum() == tv * W
