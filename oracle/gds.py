"""Plain float64 oracles of the backward gathers GDS and GWR (TEST INFRASTRUCTURE ONLY).

Only the tests use this module; the product path never imports it, and it shares no code with
the HIP implementation.

The read gather of a chunk is q0[t] = sum_r q_w[t, r] M0[q_idx[t, r]] over its valid tokens (the
pre-step memory M0; page "sparse_delta_memory/cuda/phase1_cuda.py", module docstring, for q_w).
Given the gradient rows gr[t] of the reads, GDS (page "sparse_delta_memory/cuda/mover_da2_cuda.py",
the GDS part of the module docstring and the comment of its scatter role) gives:

  d_q_w[t, r]  = <gr[t], M0[q_idx[t, r]]>                (the dots, token order)
  grad[s]     += sum over valid (t, r) with q_idx[t, r] = s of q_w[t, r] gr[t]   (the scatter)

Tokens at or past the chunk's valid count contribute nothing and their dots are 0.
"""

from __future__ import annotations

import numpy as np


def gds_chunk(q_idx, q_w, gr, m0_rows, t_valid):
    """One chunk. q_idx [C, R] absolute slots; q_w [C, R]; gr [C, hd] gradient rows of the reads;
    m0_rows(slots) -> [len(slots), hd] pre-step rows; t_valid valid tokens.

    Returns (d_q_w [C, R] float64, slots ascending int64, add [len(slots), hd] float64: the rows to
    add to grad at those slots, mag [len(slots), hd]: the same sum over absolute values)."""
    qi = np.asarray(q_idx, np.int64)
    w = np.asarray(q_w, np.float64)
    g = np.asarray(gr, np.float64)
    C, R = qi.shape
    hd = g.shape[1]
    dots = np.zeros((C, R))
    for t in range(t_valid):
        rows = m0_rows(qi[t])
        for r in range(R):
            dots[t, r] = float(np.dot(g[t], rows[r]))
    slots = np.unique(qi[:t_valid].ravel()) if t_valid > 0 else np.zeros(0, np.int64)
    where = {int(s): i for i, s in enumerate(slots)}
    add = np.zeros((len(slots), hd))
    mag = np.zeros((len(slots), hd))
    for t in range(t_valid):
        for r in range(R):
            i = where[int(qi[t, r])]
            add[i] += w[t, r] * g[t]
            mag[i] += np.abs(w[t, r] * g[t])
    return dots, slots, add, mag


def gwr_chunk(k_idx, w, dv, grad_rows, t_valid):
    """GWR of one chunk (page "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring: the GWR
    gather of the deterministic backward): with the DW step's write weights w[t, n] (k exp(rex) of
    the entry) and token rows dv[t],

      d_dv[t]     = sum_n w[t, n] grad[k_idx[t, n]]      (entries in order)
      d_k_pd[t,n] = <dv[t], grad[k_idx[t, n]]>

    k_idx [C, W] absolute slots; w [C, W]; dv [C, hd]; grad_rows(slots) -> rows of the gradient;
    tokens at or past t_valid give zeros. Returns float64 d_dv [C, hd], d_k_pd [C, W] and the
    magnitudes mag_dv (sum |w grad|) and mag_pd (sum |dv grad|)."""
    ki = np.asarray(k_idx, np.int64)
    ww = np.asarray(w, np.float64)
    v = np.asarray(dv, np.float64)
    C, W = ki.shape
    hd = v.shape[1]
    d_dv, mag_dv = np.zeros((C, hd)), np.zeros((C, hd))
    d_pd, mag_pd = np.zeros((C, W)), np.zeros((C, W))
    for t in range(t_valid):
        rows = grad_rows(ki[t])
        for n in range(W):
            d_dv[t] += ww[t, n] * rows[n]
            mag_dv[t] += np.abs(ww[t, n] * rows[n])
            d_pd[t, n] = float(np.dot(v[t], rows[n]))
            mag_pd[t, n] = float(np.dot(np.abs(v[t]), np.abs(rows[n])))
    return d_dv, d_pd, mag_dv, mag_pd
