"""Pins of the read-side oracle (oracle/read_side.py) against facts other than itself (CPU only).

The main pin is a token-by-token evaluation of the delta rule that never forms p0, A or QK: per
token, decay the slots it writes, predict from the current memory, form the token row
dv = beta (v - prediction), write it, then read. Its predictions, token rows and reads must equal
read_step's outputs built from the Phase-1 quantities, and the memory it ends with must equal the
DW step applied with read_step's token rows. Special cases: beta = 0 (no writes: dv = 0, the reads
are the plain gather) and all slots distinct (no pair terms: dv = beta (v - p0)).
"""

import math

import numpy as np
import pytest

import oracle
from oracle import read_side


def inputs(seed, N=2, C=12, W=3, R=2, S=5, valid_last=None, lane_gates=False, distinct=False, hd=4, beta=None):
    rng = np.random.default_rng(seed)
    if distinct:
        ids = rng.permutation(S)[: N * C * (W + R)].reshape(N, C, W + R)
        k_idx, q_idx = ids[:, :, :W].astype(np.int32), ids[:, :, W:].astype(np.int32)
    else:
        k_idx = rng.integers(0, S, (N, C, W)).astype(np.int32)
        q_idx = rng.integers(0, S, (N, C, R)).astype(np.int32)
    k_val = (rng.standard_normal((N, C, W)) / 2).astype(np.float32)
    q_val = (rng.standard_normal((N, C, R)) / 2).astype(np.float32)
    z = rng.standard_normal((N, C, W) if lane_gates else (N, C)) + 2.0
    g = (-np.log1p(np.exp(-z))).astype(np.float32)
    if beta is None:
        beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((N, C))))).astype(np.float32)
    v = rng.standard_normal((N, C, hd)).astype(np.float32)
    m0 = rng.standard_normal((S, hd))
    fp = N - 1 if valid_last is not None else N
    vl = C if valid_last is None else valid_last
    return dict(k_idx=k_idx, q_idx=q_idx, k_val=k_val, q_val=q_val, g=g, beta=np.asarray(beta, np.float32), v=v,
                m0=m0, S=S, first_partial=fp, valid_last=vl)


def oracle_read(d, c):
    o = oracle.phase1(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], P=1, stream_offset=d["S"],
                      first_partial=d["first_partial"], valid_last=d["valid_last"], chunks=[c])
    tv = d["valid_last"] if c >= d["first_partial"] else d["k_idx"].shape[1]
    r = read_side.read_step(d["k_idx"][c], d["q_idx"][c], o["k_eff"][0], o["q_w"][0], o["a"][0], o["qk"][0],
                            d["v"][c], d["beta"][c], lambda s: d["m0"][s], tv)
    return r, tv


@pytest.mark.parametrize("seed,S,W,R,vl,lane_gates", [(51, 4, 3, 2, None, False), (52, 6, 4, 3, 7, False),
                                                      (53, 2, 2, 2, None, False), (54, 5, 4, 2, 9, True),
                                                      (55, 3, 5, 1, None, True)])
def test_delta_rule_simulation(seed, S, W, R, vl, lane_gates):
    d = inputs(seed, C=12, W=W, R=R, S=S, valid_last=vl, lane_gates=lane_gates)
    for c in range(2):
        r, tv = oracle_read(d, c)
        M = d["m0"].copy()
        ks, qs = d["k_idx"][c], d["q_idx"][c]
        kv, qv = d["k_val"][c].astype(np.float64), d["q_val"][c].astype(np.float64)
        g = d["g"][c].astype(np.float64)
        for t in range(tv):
            for s in np.unique(ks[t]):
                lowest = int(np.flatnonzero(ks[t] == s)[0])
                M[s] *= math.exp(g[t, lowest] if lane_gates else g[t])
            pred = sum(kv[t, e] * M[ks[t, e]] for e in range(W))
            dv = float(d["beta"][c, t]) * (d["v"][c, t].astype(np.float64) - pred)
            for e in range(W):
                M[ks[t, e]] += kv[t, e] * dv
            read = sum(qv[t, q] * M[qs[t, q]] for q in range(R))
            np.testing.assert_allclose(r["pred"][t], pred, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(r["dv"][t], dv, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(r["read"][t], read, rtol=1e-11, atol=1e-11)
        assert np.all(r["dv"][tv:] == 0) and np.all(r["read"][tv:] == 0) and np.all(r["pred"][tv:] == 0)
        # The memory the simulation ends with is the DW step applied with read_step's token rows.
        slots = oracle.dw_slots(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], c, P=1, stream_offset=S,
                                first_partial=d["first_partial"], valid_last=d["valid_last"])
        new = oracle.dw_apply(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], c, r["dv"], d["m0"][slots],
                              P=1, stream_offset=S, first_partial=d["first_partial"], valid_last=d["valid_last"])
        np.testing.assert_allclose(new, M[slots], rtol=1e-11, atol=1e-11)


def test_zero_beta_is_plain_gather():
    """beta = 0: nothing is written, so dv = 0 and a read sees M0 of its slot decayed by the gate of
    every token up to its own that writes the slot (once per token), computed here by brute force."""
    d = inputs(56, C=10, W=3, R=3, S=4, beta=np.zeros((2, 10)))
    for c in range(2):
        r, tv = oracle_read(d, c)
        assert np.all(r["dv"] == 0)
        ks, qs, g = d["k_idx"][c], d["q_idx"][c], d["g"][c].astype(np.float64)
        for t in range(tv):
            want = np.zeros(d["m0"].shape[1])
            for q in range(qs.shape[1]):
                s = qs[t, q]
                decay = sum(g[u] for u in range(t + 1) if s in ks[u])
                want += float(d["q_val"][c, t, q]) * math.exp(decay) * d["m0"][s]
            np.testing.assert_allclose(r["read"][t], want, rtol=1e-12, atol=1e-12)


def test_distinct_slots_closed_form():
    """No slot shared within the chunk: A = QK = 0, dv = beta (v - k_eff . M0), read = q_w . M0 = q . M0."""
    d = inputs(57, C=16, W=3, R=2, S=4096, distinct=True)
    for c in range(2):
        r, tv = oracle_read(d, c)
        m0 = d["m0"]
        g = d["g"][c].astype(np.float64)
        p0 = np.einsum("tw,twh->th", d["k_val"][c] * np.exp(g)[:, None], m0[d["k_idx"][c]])
        want_dv = d["beta"][c][:, None].astype(np.float64) * (d["v"][c] - p0)
        np.testing.assert_allclose(r["dv"], want_dv, rtol=1e-12, atol=1e-12)
        want_read = np.einsum("tr,trh->th", d["q_val"][c].astype(np.float64), m0[d["q_idx"][c]])
        np.testing.assert_allclose(r["read"], want_read, rtol=1e-12, atol=1e-12)
