"""Seeded synthetic workloads for the SDM forward hot path.

This module only draws random inputs; it holds none of the method's arithmetic and serves both
the HIP path and the CPU oracle (tests and benchmark pass the same arrays to both).

Five workload shapes are defined (`SHAPES`): a tiny float32 case, a uniform bf16 case, a skewed
(Zipf) slot case, a wide-row case and a large-bank case whose last chunk per stream is ragged.
Every tensor comes from its own child of ``numpy.random.SeedSequence(20261202 + index)``:

* slot ids: uniform over the S slots of the token's stream (duplicates allowed, also within a
  token), or Zipf(s) ranks mapped through a random permutation of the stream's slots, or
  uniform with a fraction of entries drawn from a shared hot set; stored as absolute ids
  ``p * S + local`` (stream p owns ``[p S, (p + 1) S)``);
* gates: ``logsigmoid(N(mu, 1))`` per token, float32;
* key / query values: ``N(0, 1) / 2`` float32;
* token rows dv: ``N(0, 1)``, rounded to bf16 (nearest even) where the shape asks for bf16;
* bank: ``N(0, 0.1)`` per element, drawn on the device that holds it in blocks of 2^20 rows
  (each block from its own seeded torch generator), rounded to bf16 where asked.

Chunk c of the flat [N, ...] arrays is step ``c // P`` of stream ``c % P``; dv is stored as
``[steps, P, C, hd]`` so the token row of (chunk c, token t) is ``c * C + t``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20261202
BANK_BLOCK_ROWS = 1 << 20


@dataclass(frozen=True)
class Shape:
    name: str
    P: int
    T: int
    C: int
    W: int
    R: int
    S: int
    hd: int
    bank_dtype: str   # "f32" | "bf16"
    dv_dtype: str     # "f32" | "bf16"
    slots: str        # "uniform" | "zipf" | "hotset"
    gate_mu: float = 2.0
    zipf_s: float = 1.1
    hot_size: int = 1024
    hot_frac: float = 0.1
    valid_last: int | None = None  # tokens valid in each stream's last chunk (None: all)

    @property
    def steps(self) -> int:
        return self.T // self.C

    @property
    def N(self) -> int:
        return self.steps * self.P

    @property
    def key_bits(self) -> int:
        return max(1, int(self.S - 1).bit_length())


SHAPES = {
    0: Shape("tiny_f32", P=1, T=256, C=64, W=4, R=4, S=4096, hd=64, bank_dtype="f32", dv_dtype="f32", slots="uniform"),
    1: Shape("uniform_bf16", P=8, T=4096, C=128, W=16, R=16, S=65536, hd=128, bank_dtype="bf16", dv_dtype="bf16",
             slots="uniform"),
    2: Shape("zipf_skewed", P=4, T=8192, C=256, W=32, R=32, S=262144, hd=120, bank_dtype="bf16", dv_dtype="f32",
             slots="zipf"),
    3: Shape("wide_rows", P=4, T=8192, C=256, W=8, R=8, S=1048576, hd=960, bank_dtype="bf16", dv_dtype="bf16",
             slots="uniform", gate_mu=3.0),
    4: Shape("large_ragged", P=16, T=16384, C=256, W=32, R=32, S=4194304, hd=128, bank_dtype="bf16",
             dv_dtype="f32", slots="hotset", valid_last=100),
}


@dataclass
class Workload:
    shape: Shape
    steps: int
    k_idx: np.ndarray   # [N, C, W] int32 absolute slot ids
    q_idx: np.ndarray   # [N, C, R] int32
    k_val: np.ndarray   # [N, C, W] float32
    q_val: np.ndarray   # [N, C, R] float32
    g: np.ndarray       # [N, C] float32 per token, or [N, C, W] per (token, K lane)
    dv: np.ndarray      # [steps, P, C, hd] float32 (bf16-representable values when dv_dtype == "bf16")
    first_partial: int
    valid_last: int
    bank_seed: int
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.k_idx.shape[0]

    @property
    def val_bf16(self) -> bool:
        """The values are bfloat16 (k_val / q_val hold bfloat16-representable float32 values)."""
        return bool(self.meta.get("val_bf16", False))

    @property
    def P(self) -> int:
        return self.shape.P

    @property
    def stream_offset(self) -> int:
        return self.shape.S

    @property
    def rows(self) -> int:
        return self.shape.P * self.shape.S


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), returned as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> 16) & 1) + np.uint32(0x7FFF)
    out = ((b + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    nan = np.isnan(x)
    out = np.where(nan, np.uint32(0x7FC00000), out)
    return out.view(np.float32)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return np.where(x >= 0, -np.log1p(np.exp(-x)), x - np.log1p(np.exp(x)))


def _slots(rng: np.random.Generator, sh: Shape, size, ctx: dict) -> np.ndarray:
    if sh.slots == "uniform":
        return rng.integers(0, sh.S, size=size, dtype=np.int64)
    if sh.slots == "zipf":
        u = rng.random(size=size)
        ranks = np.searchsorted(ctx["zipf_cdf"], u, side="right")
        ranks = np.minimum(ranks, sh.S - 1)
        return ctx["perm"][ranks]
    if sh.slots == "hotset":
        base = rng.integers(0, sh.S, size=size, dtype=np.int64)
        hot = rng.random(size=size) < sh.hot_frac
        pick = ctx["hot"][rng.integers(0, sh.hot_size, size=size)]
        return np.where(hot, pick, base)
    raise ValueError(sh.slots)


def make(index: int | Shape, steps: int | None = None, *, nan_invalid: bool = True, seed: int | None = None,
         shape_overrides: dict | None = None, lane_gates: bool = False, val_bf16: bool = False) -> Workload:
    """Draw the inputs of workload `index` (or of a Shape). `steps` truncates the step count (the
    last step stays ragged when the shape is). `shape_overrides` replaces Shape fields (tests).
    `lane_gates`: one gate per (token, K lane), g [N, C, W], instead of one per token. `val_bf16`:
    the values are drawn as before and rounded to bfloat16 (the device then takes them as bfloat16)."""
    sh = SHAPES[index] if isinstance(index, int) else index
    if shape_overrides:
        sh = Shape(**{**sh.__dict__, **shape_overrides})
    base_seed = ROOT_SEED + (index if isinstance(index, int) else 0) if seed is None else seed
    nsteps = sh.steps if steps is None else int(steps)
    P, C, W, R, hd = sh.P, sh.C, sh.W, sh.R, sh.hd
    N = nsteps * P
    ss = np.random.SeedSequence(base_seed)
    ch = dict(zip(["k_idx", "q_idx", "k_val", "q_val", "g", "dv", "bank", "perm", "hot"], ss.spawn(9)))
    ctx = {}
    if sh.slots == "zipf":
        ranks = np.arange(1, sh.S + 1, dtype=np.float64)
        w = ranks ** (-sh.zipf_s)
        cdf = np.cumsum(w)
        ctx["zipf_cdf"] = cdf / cdf[-1]
        ctx["perm"] = np.random.default_rng(ch["perm"]).permutation(sh.S).astype(np.int64)
    if sh.slots == "hotset":
        ctx["hot"] = np.random.default_rng(ch["hot"]).choice(sh.S, size=sh.hot_size, replace=False).astype(np.int64)
    stream = (np.arange(N, dtype=np.int64) % P)[:, None, None] * sh.S
    k_idx = (_slots(np.random.default_rng(ch["k_idx"]), sh, (N, C, W), ctx) + stream).astype(np.int32)
    q_idx = (_slots(np.random.default_rng(ch["q_idx"]), sh, (N, C, R), ctx) + stream).astype(np.int32)
    k_val = (np.random.default_rng(ch["k_val"]).standard_normal((N, C, W)) / 2.0).astype(np.float32)
    q_val = (np.random.default_rng(ch["q_val"]).standard_normal((N, C, R)) / 2.0).astype(np.float32)
    if val_bf16:
        k_val, q_val = round_bf16(k_val), round_bf16(q_val)
        ctx["val_bf16"] = True
    g_shape = (N, C, W) if lane_gates else (N, C)
    g = _logsigmoid(np.random.default_rng(ch["g"]).standard_normal(g_shape) + sh.gate_mu).astype(np.float32)
    dv = np.random.default_rng(ch["dv"]).standard_normal((nsteps, P, C, hd), dtype=np.float32)
    if sh.dv_dtype == "bf16":
        dv = round_bf16(dv)
    valid_last = C if sh.valid_last is None else int(sh.valid_last)
    first_partial = (nsteps - 1) * P if sh.valid_last is not None else N
    if nan_invalid and valid_last < C:
        k_val[first_partial:, valid_last:, :] = np.nan
        q_val[first_partial:, valid_last:, :] = np.nan
        g[first_partial:, valid_last:] = np.nan
        dv[nsteps - 1, :, valid_last:, :] = np.nan
    bank_seed = int(ch["bank"].generate_state(1, dtype=np.uint32)[0])
    return Workload(sh, nsteps, k_idx, q_idx, k_val, q_val, g, dv, first_partial, valid_last, bank_seed, ctx)


def make_bank(wl: Workload, device="cpu", rows: int | None = None):
    """The initial bank [P*S, hd] (torch tensor on `device`): N(0, 0.1), bf16 or float32.

    Drawn in blocks of 2^20 rows, block b from torch generator seed (bank_seed + b) on `device`,
    so the values depend on the device type that draws them."""
    import torch

    sh = wl.shape
    rows = wl.rows if rows is None else rows
    dt = torch.bfloat16 if sh.bank_dtype == "bf16" else torch.float32
    bank = torch.empty((rows, sh.hd), dtype=dt, device=device)
    for b0 in range(0, rows, BANK_BLOCK_ROWS):
        nb = min(BANK_BLOCK_ROWS, rows - b0)
        gen = torch.Generator(device=device)
        gen.manual_seed(wl.bank_seed + b0 // BANK_BLOCK_ROWS)
        blk = torch.randn((nb, sh.hd), generator=gen, device=device, dtype=torch.float32) * 0.1
        bank[b0:b0 + nb].copy_(blk.to(dt))
    return bank


def make_bank_rows(wl: Workload, rows, device="cpu"):
    """Initial values of the given bank rows, regenerated block by block exactly as make_bank."""
    import torch

    sh = wl.shape
    rows = np.asarray(rows, dtype=np.int64)
    dt = torch.bfloat16 if sh.bank_dtype == "bf16" else torch.float32
    out = torch.empty((rows.size, sh.hd), dtype=dt, device=device)
    blk_of = rows // BANK_BLOCK_ROWS
    for b in np.unique(blk_of):
        b0 = int(b) * BANK_BLOCK_ROWS
        nb = min(BANK_BLOCK_ROWS, wl.rows - b0)
        gen = torch.Generator(device=device)
        gen.manual_seed(wl.bank_seed + int(b))
        blk = (torch.randn((nb, sh.hd), generator=gen, device=device, dtype=torch.float32) * 0.1).to(dt)
        sel = np.nonzero(blk_of == b)[0]
        out[torch.as_tensor(sel, device=device)] = blk[torch.as_tensor(rows[sel] - b0, device=device)]
    return out


def make_read_inputs(wl: Workload, nan_invalid: bool = True):
    """Seeded inputs of the read side: value rows v [steps * P * C, hd] float32 ~ N(0, 1) (row
    ti*P*C + p*C + t) and write strengths beta [N, C] float32 = sigmoid(N(0, 1)); masked tokens get
    NaN (they must never be read)."""
    ss = np.random.SeedSequence([wl.bank_seed, 1])
    cv, cb = ss.spawn(2)
    sh = wl.shape
    v = np.random.default_rng(cv).standard_normal((wl.steps * sh.P * sh.C, sh.hd), dtype=np.float32)
    z = np.random.default_rng(cb).standard_normal((wl.N, sh.C))
    beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    if nan_invalid and wl.valid_last < sh.C:
        beta[wl.first_partial:, wl.valid_last:] = np.nan
        v3 = v.reshape(wl.steps, sh.P, sh.C, sh.hd)
        v3[wl.steps - 1, :, wl.valid_last:, :] = np.nan
    return v, beta
