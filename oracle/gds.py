"""Plain float64 oracles of the backward movers GDS, GWR and PA (TEST INFRASTRUCTURE ONLY).

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


def pa_chunk(k_idx, k_eff, beta, cpe_of_slot, d_dva, gdw_rows, snap_rows, t_valid):
    """PA of one chunk (page "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring: Phase A of
    the deterministic backward, the backward of DW): per write group (slot s, members m),

      grad[s]         = gdw[s] cpe_s + sum_m sc_m d_dva[tok_m],   sc_m = -beta[tok_m] k_eff_m
      bank[s]         = snap[s]                                    (restore)
      grad_g_decay[e] = cpe_s <gdw[s], snap[s]>,   d_k_eff[e] = -beta[tok_e] <d_dva[tok_e], snap[s]>

    with gdw the slot's gradient row before PA and snap its pre-write row. k_idx [C, W] absolute
    slots, k_eff [C, W], beta [C]; cpe_of_slot(s) the group's cpe; d_dva [C, hd]; gdw_rows(slots)
    and snap_rows(slots) -> rows. Returns (slots ascending, new grad rows, grad_g_decay [C, W],
    d_k_eff [C, W], mag_grad (|gdw cpe| + sum |sc d_dva|), mag_dot [C, W] (sum |d_dva snap|))."""
    ki = np.asarray(k_idx, np.int64)
    ke = np.asarray(k_eff, np.float64)
    b = np.asarray(beta, np.float64)
    d = np.asarray(d_dva, np.float64)
    C, W = ki.shape
    slots = np.unique(ki[:t_valid].ravel()) if t_valid > 0 else np.zeros(0, np.int64)
    gdw = gdw_rows(slots) if len(slots) else np.zeros((0, d.shape[1]))
    snap = snap_rows(slots) if len(slots) else np.zeros((0, d.shape[1]))
    where = {int(s): i for i, s in enumerate(slots)}
    cpe = np.array([cpe_of_slot(int(s)) for s in slots], np.float64)
    new = gdw * cpe[:, None]
    mag = np.abs(new)
    g_decay, d_keff, mag_dot = np.zeros((C, W)), np.zeros((C, W)), np.zeros((C, W))
    for t in range(t_valid):
        for n in range(W):
            i = where[int(ki[t, n])]
            sc = -b[t] * ke[t, n]
            new[i] += sc * d[t]
            mag[i] += np.abs(sc * d[t])
            g_decay[t, n] = cpe[i] * float(np.dot(gdw[i], snap[i]))
            d_keff[t, n] = -b[t] * float(np.dot(d[t], snap[i]))
            mag_dot[t, n] = float(np.dot(np.abs(d[t]), np.abs(snap[i])))
    return slots, new, g_decay, d_keff, mag, mag_dot
