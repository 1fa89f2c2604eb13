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
