"""The Phase-1 path knobs on the GPU.

lds_budget: a smaller LDS budget makes the sort/scan kernel take other paths (narrower radix digits
and so more passes, values and ids read from global memory instead of staged in LDS, outputs in more
sweeps of token ranges); every output must be the default run's bit for bit, the pair sums included
(the pair kernel does not see the budget).

defer_pairs: the sort/scan call leaves the pair sums to a second call (sdm_phase1_pairs) that runs
on another stream; every output must be the one-call run's bit for bit.

pair_walk: every slot group walked by the pair kernel instead of the dense contraction of hot groups
(the phase1_cuda page's hot/cold note: the two forms agree within the evaluation bound, not bit for
bit). A and QK of the walked form meet the strict max(1e-5|o|, 1e-6) bound against the oracle, as
the dense form does, and every other output equals the default run's bit for bit.
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


def say(*a):
    print(*a, flush=True)


def run(wl, **knobs):
    """Phase 1 of every chunk with the given knobs; every output, perm and the group ordinals included."""
    shape = H.shape_of(wl)
    for k, v in knobs.items():
        setattr(shape, k, int(v))
    ins = H.device_inputs(wl)
    every = set(sdm.alloc_phase1_outputs(sdm.make_shape(0, 1, 1, 1), device="cpu"))
    out = sdm.alloc_phase1_outputs(shape, device="cuda", fields=every | {"perm", "gord_k"})
    out = sdm.phase1(shape, out=out, **ins)
    torch.cuda.synchronize()
    return out


def same_bits(name, a, b):
    assert a.dtype == b.dtype and a.shape == b.shape, name
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), name


def edge(C, W_, R, S, P, steps, vl=None):
    sh = W.Shape("knobs", P=P, T=C * steps, C=C, W=W_, R=R, S=S, hd=64, bank_dtype="f32", dv_dtype="f32",
                 slots="uniform", valid_last=vl)
    return W.make(sh, seed=733)


@pytest.mark.parametrize("case", [
    dict(idx=1, steps=2, budgets=[96 * 1024, 72 * 1024]),   # 4 items per thread: resident at 96 KB, unstaged at 72 KB
    dict(idx=4, steps=1, budgets=[128 * 1024, 112 * 1024]),  # 16 items: narrower digits, two K sweeps
    dict(idx=2, steps=1, budgets=[112 * 1024]),              # Zipf: hot-group lists through the sweeps
    dict(edge=(37, 5, 3, 9, 2, 2, 11), budgets=[16384]),     # a ragged 296-entry row in the smallest budget
])
def test_lds_budget_gives_the_same_bits(case):
    wl = W.make(case["idx"], steps=case["steps"]) if "idx" in case else edge(*case["edge"])
    say("lds budget", case)
    ref = run(wl)
    for b in case["budgets"]:
        say("  budget", b)
        got = run(wl, lds_budget=b)
        for k in ref:
            same_bits("%s (budget %d)" % (k, b), got[k], ref[k])


@pytest.mark.parametrize("case", [
    dict(idx=2, steps=1),   # Zipf: about 45 hot groups per chunk
    dict(idx=4, steps=1),   # the hot set of the large ragged workload
    dict(idx=1, steps=1),
])
def test_pair_walk_matches_the_oracle_and_the_dense_form(case):
    wl = W.make(case["idx"], steps=case["steps"])
    say("pair walk", case)
    dense = run(wl)
    walk = run(wl, pair_walk=1)
    for k in dense:
        if k not in ("a", "qk"):
            same_bits(k, walk[k], dense[k])
    if case["idx"] == 2:   # (hot groups there: the knob really changes the pair kernel's path)
        assert not torch.equal(walk["a"], dense["a"])
    chunks = list(range(wl.N)) if wl.N <= 16 else list(range(0, wl.N, max(1, wl.N // 16)))
    ref = H.oracle_phase1(wl, chunks)
    H.compare_phase1({k: walk[k] for k in ("a", "qk", "spay_k", "krec")}, ref, chunks)
    # The two forms differ by at most the sum of their distances to the oracle.
    idx = torch.as_tensor(chunks, device="cuda")
    for f in ("a", "qk"):
        o = np.asarray(ref[f], np.float64)
        d = dense[f].index_select(0, idx).cpu().numpy().astype(np.float64)
        w = walk[f].index_select(0, idx).cpu().numpy().astype(np.float64)
        tol = 2 * np.maximum(1e-5 * np.abs(o), 1e-6)
        assert np.all(np.abs(d - w) <= tol), f


@pytest.mark.parametrize("case", [
    dict(idx=1, steps=2),                      # uniform rows on chip
    dict(idx=2, steps=1),                      # Zipf: hot-group lists written by the first call
    dict(idx=4, steps=1, knobs=dict(pair_walk=1)),
    dict(edge=(64, 6, 3, 40, 2, 2, 50), knobs=dict(tiled=1)),   # the tiled path (32-bit entry words)
])
def test_deferred_pairs_give_the_same_bits(case):
    wl = W.make(case["idx"], steps=case["steps"]) if "idx" in case else edge(*case["edge"])
    knobs = case.get("knobs", {})
    say("deferred pairs", case)
    ref = run(wl, **knobs)
    shape = H.shape_of(wl)
    for k, v in knobs.items():
        setattr(shape, k, int(v))
    ins = H.device_inputs(wl)
    every = set(sdm.alloc_phase1_outputs(sdm.make_shape(0, 1, 1, 1), device="cpu"))
    out = sdm.alloc_phase1_outputs(shape, device="cuda", fields=every | {"perm", "gord_k"})
    for f in ("a", "qk"):
        out[f].fill_(float("nan"))
    ws = torch.empty(sdm.phase1_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    done = torch.cuda.Event()
    sdm.phase1(shape, out=out, workspace=ws, defer_pairs=True, **ins)
    done.record(main)
    side.wait_event(done)
    sdm.phase1_pairs(shape, out, ws, stream=side)
    torch.cuda.synchronize()
    for k in ref:
        same_bits(k, out[k], ref[k])
