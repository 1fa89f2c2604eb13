"""Plain float64 oracle of the forward read side of one chunk (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this module; the product
path never imports it, and it shares no code with the HIP implementation.

What it computes, per chunk, from the pre-step memory M0 (the bank rows before the chunk's DW
step) and the chunk's Phase-1 quantities (page "sparse_delta_memory/cuda/phase1_cuda.py", module
docstring: k_eff, q_w, A, QK):

  p0[t]   = sum_e k_eff[t, e] M0[k_idx[t, e]]          (the token gather of the writes)
  q0[t]   = sum_r q_w[t, r]   M0[q_idx[t, r]]          (the token gather of the reads)
  dv[t]   = beta[t] (v[t] - p0[t] - sum_{j<t} A[t, j] dv[j])     (forward substitution)
  pred[t] = p0[t] + sum_{j<t}  A[t, j]  dv[j]
  read[t] = q0[t] + sum_{j<=t} QK[t, j] dv[j]

The relation dv = beta (v - pred) is the delta rule read from the pages' records: the backward
records carry the write scale -beta * k * exp(log_k) ("sparse_delta_memory/cuda/phase1_cuda.py",
the kspa record of p1_scan_kernel; "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring), so
the token row a write adds is beta (v - pred). pred and read are then what a token-by-token
decay-then-write evaluation sees (the tests check exactly that). Tokens at or past the chunk's
valid count are masked: all their outputs are 0 and none of their inputs is read.
"""

from __future__ import annotations

import numpy as np


def read_step(k_idx, q_idx, k_eff, q_w, a, qk, v, beta, m0_rows, t_valid):
    """One chunk. k_idx [C, W] / q_idx [C, R] absolute slots; k_eff [C, W], q_w [C, R]; a, qk
    [C, C]; v [C, hd]; beta [C]; m0_rows(slots) -> [len(slots), hd] pre-step rows; t_valid tokens
    are valid. Returns float64 [C, hd] arrays p0, q0, dv, pred, read and the magnitude bounds
    mag_dv, mag_pred, mag_read (the same recursions on absolute values: the scale of the float
    evaluation error)."""
    C, W = np.shape(k_idx)
    hd = np.shape(v)[1]
    keff = np.asarray(k_eff, np.float64)
    qw = np.asarray(q_w, np.float64)
    A = np.asarray(a, np.float64)
    QK = np.asarray(qk, np.float64)
    vv = np.asarray(v, np.float64)
    bb = np.asarray(beta, np.float64)
    out = {k: np.zeros((C, hd)) for k in ("p0", "q0", "dv", "pred", "read", "mag_p0", "mag_q0", "mag_dv",
                                             "mag_pred", "mag_read")}
    for t in range(t_valid):
        kr = m0_rows(np.asarray(k_idx[t], np.int64))
        qr = m0_rows(np.asarray(q_idx[t], np.int64))
        out["p0"][t] = keff[t] @ kr
        out["q0"][t] = qw[t] @ qr
        out["mag_p0"][t] = np.abs(keff[t]) @ np.abs(kr)
        out["mag_q0"][t] = np.abs(qw[t]) @ np.abs(qr)
    for t in range(t_valid):
        prior = A[t, :t] @ out["dv"][:t]
        out["dv"][t] = bb[t] * (vv[t] - out["p0"][t] - prior)
        out["pred"][t] = out["p0"][t] + prior
        mprior = np.abs(A[t, :t]) @ out["mag_dv"][:t]
        out["mag_dv"][t] = abs(bb[t]) * (np.abs(vv[t]) + out["mag_p0"][t] + mprior)
        out["mag_pred"][t] = out["mag_p0"][t] + mprior
    for t in range(t_valid):
        out["read"][t] = out["q0"][t] + QK[t, :t + 1] @ out["dv"][:t + 1]
        out["mag_read"][t] = out["mag_q0"][t] + np.abs(QK[t, :t + 1]) @ out["mag_dv"][:t + 1]
    return out
