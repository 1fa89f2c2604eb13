"""Pins of the GDS oracle (oracle/gds.py) against facts other than itself (CPU only).

GDS is the backward of the read gather q0[t] = sum_r q_w[t, r] M0[q_idx[t, r]]. The pin builds that
forward with torch float64 operations (index_select, multiply, sum) and lets autograd give the
gradients of sum_t <gr[t], q0[t]> with respect to M0 and q_w: they must equal the oracle's scatter
rows (at its slots; zero elsewhere) and its dots. Masked tokens contribute nothing.
"""

import numpy as np
import pytest

from oracle import gds

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("seed,S,C,R,tv", [(71, 5, 12, 3, 12), (72, 40, 16, 4, 9), (73, 2, 8, 5, 8), (74, 9, 6, 2, 0)])
def test_gds_is_the_gradient_of_the_read_gather(seed, S, C, R, tv):
    rng = np.random.default_rng(seed)
    hd = 6
    q_idx = rng.integers(0, S, (C, R))
    q_w = rng.standard_normal((C, R))
    gr = rng.standard_normal((C, hd))
    m0 = rng.standard_normal((S, hd))
    dots, slots, add, mag = gds.gds_chunk(q_idx, q_w, gr, lambda s: m0[s], tv)

    M = torch.tensor(m0, dtype=torch.float64, requires_grad=True)
    W = torch.tensor(q_w, dtype=torch.float64, requires_grad=True)
    idx = torch.tensor(q_idx[:tv].reshape(-1), dtype=torch.long)
    rows = M.index_select(0, idx).reshape(tv, R, hd)
    q0 = (W[:tv].unsqueeze(-1) * rows).sum(dim=1)
    (q0 * torch.tensor(gr[:tv], dtype=torch.float64)).sum().backward()

    want_grad = M.grad.numpy() if M.grad is not None else np.zeros_like(m0)
    got_grad = np.zeros_like(m0)
    got_grad[slots] = add
    np.testing.assert_allclose(got_grad, want_grad, rtol=1e-12, atol=1e-12)
    want_dots = W.grad.numpy() if W.grad is not None else np.zeros_like(q_w)
    np.testing.assert_allclose(dots, want_dots, rtol=1e-12, atol=1e-12)
    assert np.all(mag >= np.abs(add) - 1e-12)
    assert np.all(dots[tv:] == 0)


@pytest.mark.parametrize("seed,S,C,W,tv", [(81, 5, 12, 3, 12), (82, 40, 16, 4, 9), (83, 2, 8, 5, 0)])
def test_gwr_is_the_gradient_of_the_dw_writes(seed, S, C, W, tv):
    """GWR against autograd: the DW step's write terms new[s] += w[t, n] dv[t] (s = k_idx[t, n]),
    contracted with a gradient G of the new rows; the gradients with respect to dv and w are d_dv
    and d_k_pd."""
    rng = np.random.default_rng(seed)
    hd = 5
    k_idx = rng.integers(0, S, (C, W))
    w = rng.standard_normal((C, W))
    dv = rng.standard_normal((C, hd))
    G = rng.standard_normal((S, hd))
    d_dv, d_pd, mag_dv, mag_pd = gds.gwr_chunk(k_idx, w, dv, lambda s: G[s], tv)
    V = torch.tensor(dv, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    new = torch.zeros((S, hd), dtype=torch.float64)
    idx = torch.tensor(k_idx[:tv].reshape(-1), dtype=torch.long)
    terms = (Wt[:tv].unsqueeze(-1) * V[:tv].unsqueeze(1)).reshape(-1, hd)
    new = new.index_add(0, idx, terms)
    (new * torch.tensor(G)).sum().backward()
    want_dv = V.grad.numpy() if V.grad is not None else np.zeros_like(dv)
    want_w = Wt.grad.numpy() if Wt.grad is not None else np.zeros_like(w)
    np.testing.assert_allclose(d_dv, want_dv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d_pd, want_w, rtol=1e-12, atol=1e-12)
    assert np.all(mag_dv >= np.abs(d_dv) - 1e-12) and np.all(mag_pd >= np.abs(d_pd) - 1e-12)


@pytest.mark.parametrize("seed,S,C,W,tv", [(91, 5, 12, 3, 12), (92, 40, 16, 4, 9), (93, 2, 8, 5, 8)])
def test_pa_is_the_gradient_of_dw_and_the_write_prediction(seed, S, C, W, tv):
    """PA against autograd. With M0 the pre-write rows, G the gradient of the rows DW writes and
    D the gradient of the token rows, L = sum_s <G[s], M0[s] exp(T_s)> + sum_t <D[t], -beta[t] p0[t]>,
    p0[t] = sum_n k_eff[t, n] M0[k_idx[t, n]] (the token's prediction; dv = beta (v - p0 - ...)).
    dL/dM0[s] is PA's grad row, dL/dT_s its grad_g_decay (each member of the group), dL/dk_eff its
    d_k_eff; the gradient of the memory is taken only at slots the chunk writes."""
    rng = np.random.default_rng(seed)
    hd = 5
    k_idx = rng.integers(0, S, (C, W))
    k_eff = rng.standard_normal((C, W))
    beta = rng.random(C)
    m0 = rng.standard_normal((S, hd))
    G = rng.standard_normal((S, hd))
    D = rng.standard_normal((C, hd))
    T = -rng.random(S)                       # the group's total gate (cpe = exp(T))
    slots, new, g_decay, d_keff, mag, mag_dot = gds.pa_chunk(
        k_idx, k_eff, beta, lambda s: float(np.exp(T[s])), D, lambda s: G[s], lambda s: m0[s], tv)
    M = torch.tensor(m0, requires_grad=True)
    Tt = torch.tensor(T, requires_grad=True)
    Ke = torch.tensor(k_eff, requires_grad=True)
    written = torch.zeros(S, dtype=torch.float64)
    written[torch.tensor(slots, dtype=torch.long)] = 1.0
    dw_term = (torch.tensor(G) * M * torch.exp(Tt).unsqueeze(-1) * written.unsqueeze(-1)).sum()
    idx = torch.tensor(k_idx[:tv].reshape(-1), dtype=torch.long)
    p0 = (Ke[:tv].unsqueeze(-1) * M.index_select(0, idx).reshape(tv, W, hd)).sum(dim=1)
    pred_term = (torch.tensor(D[:tv]) * (-torch.tensor(beta[:tv]).unsqueeze(-1) * p0)).sum()
    (dw_term + pred_term).backward()
    np.testing.assert_allclose(new, M.grad.numpy()[slots], rtol=1e-12, atol=1e-12)
    for t in range(tv):
        for n in range(W):
            assert abs(g_decay[t, n] - Tt.grad.numpy()[k_idx[t, n]]) <= 1e-12 * (1 + abs(g_decay[t, n]))
    np.testing.assert_allclose(d_keff[:tv], Ke.grad.numpy()[:tv], rtol=1e-12, atol=1e-12)
    assert np.all(g_decay[tv:] == 0) and np.all(d_keff[tv:] == 0)
    assert np.all(mag >= np.abs(new) - 1e-12) and np.all(mag_dot >= 0)
