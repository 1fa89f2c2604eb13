"""Pins of the oracle's bfloat16-value variant (CPU only).

With bfloat16 values the page "sparse_delta_memory/cuda/phase1_cuda.py" gives cpe, k_eff and q_w
the value type, and the mover records carry cpe "as the value type widened". The oracle reads this
as: those outputs are the exact values rounded once to bfloat16 (nearest, ties to even); every other
output is unchanged; the DW step scales the base row by the rounded cpe.

Pins: the rounding against torch's float32 -> bfloat16 conversion (a library routine, round to
nearest even) on float32-exact inputs, ties and the subnormal range included; the DW step with
zero token rows and unit base rows against a brute-force sum of the gates that touch each slot.
"""

import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_library_conversion():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(4000), rng.standard_normal(1000) * 1e30, rng.standard_normal(1000) * 1e-30,
        rng.standard_normal(500) * 1e-39,                    # float32 subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 3.0 * 2.0 ** -140]),
    ]).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(x), torch_bf16(x))


def test_round_bf16_ties_to_even():
    q = 2.0 ** -7                       # bfloat16 spacing in [1, 2)
    ties = np.array([1 + q / 2, 1 + 3 * q / 2, -(1 + q / 2), 2 - q / 2, 1 + 5 * q / 2])
    want = np.array([1.0, 1 + 2 * q, -1.0, 2.0, 1 + 2 * q])
    np.testing.assert_array_equal(oracle.round_bf16(ties), want)
    np.testing.assert_array_equal(torch_bf16(ties), want)
    near = np.array([1 + q / 2 + 2.0 ** -20, 1 + q / 2 - 2.0 ** -20])   # just off the tie
    np.testing.assert_array_equal(oracle.round_bf16(near), np.array([1 + q, 1.0]))


def chunk(seed, C=16, W=3, R=2, S=6, lane_gates=False, vl=None):
    rng = np.random.default_rng(seed)
    N = 2
    k_idx = rng.integers(0, S, (N, C, W)).astype(np.int32)
    q_idx = rng.integers(0, S, (N, C, R)).astype(np.int32)
    k_val = torch_bf16(rng.standard_normal((N, C, W))).astype(np.float32)   # bfloat16-exact values
    q_val = torch_bf16(rng.standard_normal((N, C, R))).astype(np.float32)
    g = (-rng.random((N, C, W) if lane_gates else (N, C)) * 0.7).astype(np.float32)
    return dict(k_idx=k_idx, q_idx=q_idx, k_val=k_val, q_val=q_val, g=g,
                first_partial=N - 1 if vl is not None else N, valid_last=C if vl is None else vl)


@pytest.mark.parametrize("seed,lane_gates,vl", [(61, False, None), (62, True, 11)])
def test_bf16_fields_are_the_rounded_exact_values(seed, lane_gates, vl):
    d = chunk(seed, lane_gates=lane_gates, vl=vl)
    args = (d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"])
    kw = dict(first_partial=d["first_partial"], valid_last=d["valid_last"], stream_offset=6)
    f = oracle.phase1(*args, **kw)
    b = oracle.phase1(*args, val_bf16=True, **kw)
    for name in ("cpe", "k_eff", "q_w", "krec_cpe"):
        np.testing.assert_array_equal(b[name], oracle.round_bf16(f[name]), err_msg=name)
        assert not np.array_equal(b[name], f[name]), name        # the rounding is visible
    for name in set(f) - {"cpe", "k_eff", "q_w", "krec_cpe"}:
        np.testing.assert_array_equal(b[name], f[name], err_msg=name)


@pytest.mark.parametrize("seed,lane_gates", [(63, False), (64, True)])
def test_bf16_dw_scales_by_rounded_total_gate(seed, lane_gates):
    """dv = 0, base = 1: every written row is exp(G) rounded to bfloat16, G the sum of the gates of
    the valid tokens writing the slot, once per token (per-lane gates: the lowest lane's)."""
    d = chunk(seed, lane_gates=lane_gates)
    C, hd = d["k_idx"].shape[1], 4
    for c in range(2):
        slots = oracle.dw_slots(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], c)
        new = oracle.dw_apply(d["k_idx"], d["q_idx"], d["k_val"], d["q_val"], d["g"], c, np.zeros((C, hd)),
                              np.ones((len(slots), hd)), val_bf16=True)
        for gi, s in enumerate(slots):
            G = 0.0
            for t in range(C):
                lanes = np.flatnonzero(d["k_idx"][c, t] == s)
                if len(lanes):
                    G += float(d["g"][c, t, lanes[0]] if lane_gates else d["g"][c, t])
            want = torch_bf16(np.array([math.exp(G)]))[0]   # exp(G) of a few float32 gates: no tie
            np.testing.assert_array_equal(new[gi], np.full(hd, want))
