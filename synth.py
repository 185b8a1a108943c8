"""Seeded synthetic inputs shaped like the block-diffusion workloads.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no scores, no softmax, no selection), so both the
HIP path and the float64 oracle can take their inputs from it.

Values are drawn with NumPy's PCG64 in float32 from a seed sequence keyed
by (workload seed, tensor tag, row), then rounded to the workload dtype by
torch (round to nearest even for bf16).  Tensors are returned on the CPU;
callers move them to the device.

Workloads (sizes from the five synthetic configurations the design notes
list; the shapes follow the pages: bl = 32 blocks, W = 2 windows, GQA with
G = 4, 5 % budgets and 16K-32K contexts):

* ``tiny_dense``      1 row, fp32, d=64, 4/4 heads, prefix 256, W=1.
* ``packed_wavefront`` 8 rows, C=4096, W=2, o_b multiples of 32 in [512, 3968].
* ``sparse_32k``      4 rows, 32768-token prefix, 2 % planted keys, T=8.
* ``sparse_128k``     1 row, 131072-token prefix, heavy hitters every ~64, T=16.
* ``serving_mix``     64 rows, log-uniform prefixes 1K-16K, W=4; rows with a
                      prefix over 8K are served sparsely at a 5 % budget.

The sparse workloads build the block queries as one shared per-head
direction plus a small per-position term: at selection time every block
position carries the same [MASK] embedding and the queries differ only by
position (HERALD Sec. IV-A2).  Planted keys point along the sum of the
shared directions of the KV head's query group.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

_TAGS = {"Q": 1, "K": 2, "V": 3, "W": 4, "O": 5, "PLANT": 6, "U": 7,
         "NOISE": 8, "STEPQ": 9, "STEPK": 10, "STEPV": 11, "MISC": 12}

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def rng(seed: int, tag: str, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), _TAGS[tag], *[int(e) for e in extra]])))


def normal(shape, seed: int, tag: str, *extra: int, scale: float = 1.0) -> np.ndarray:
    x = rng(seed, tag, *extra).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DTYPES[dtype])


def budget_keys(S: int, frac: float) -> int:
    """Budget in keys: ``frac * S`` rounded to the nearest integer (half up).

    0.05 * 32768 = 1638.4 -> 1638 and 0.05 * 131072 = 6553.6 -> 6554, the
    two counts the sparse workloads state; floor or ceil would miss one.
    """
    return int(math.floor(frac * S + 0.5))


@dataclass
class Workload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    d: int
    bl: int
    W: int
    C: int
    seed: int
    Kc: torch.Tensor              # [B, C, Hkv, d]; window KV at the tail [t, C)
    Vc: torch.Tensor
    o: torch.Tensor               # int32 [B] per-row offsets (prefix lengths)
    Q: torch.Tensor               # [B, q, Hq, d] window queries (step 0)
    sm_scale: float
    n_layers: int = 1
    # selection (sparse rows only)
    sparse_rows: torch.Tensor | None = None   # int32 [n_sparse]
    dense_rows: torch.Tensor | None = None    # int32 [n_dense]
    s_len: torch.Tensor | None = None         # int32 [B]: positions to select over
    k_sel: torch.Tensor | None = None         # int32 [B]: budget per row
    Qsel: torch.Tensor | None = None          # [B, nq, Hq, d] block queries for selection
    planted: dict = field(default_factory=dict)   # (b, h) -> sorted int array
    T: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def q(self) -> int:
        return self.W * self.bl

    @property
    def t(self) -> int:
        return self.C - self.q

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def k_max(self) -> int:
        return int(self.k_sel.max()) if self.k_sel is not None and len(self.k_sel) else 0

    @property
    def s_max(self) -> int:
        return int(self.s_len.max()) if self.s_len is not None and len(self.s_len) else 0


def _fill_cache(B, C, Hkv, d, dtype, o, q, seed, tag, scale, rows_fn=None):
    """Cache [B, C, Hkv, d]: prefix [0, o_b) and tail [C-q, C) drawn, the
    never-visible middle [o_b, C-q) filled with NaN sentinels."""
    t = C - q
    out = torch.full((B, C, Hkv, d), float("nan"), dtype=DTYPES[dtype])
    for b in range(B):
        ob = int(o[b])
        x = normal((ob + q, Hkv, d), seed, tag, b, scale=scale)
        if rows_fn is not None:
            rows_fn(b, x)
        xt = to_dtype(x, dtype)
        out[b, :ob] = xt[:ob]
        out[b, t:] = xt[ob:]
    return out


def _shared_queries(B, nq, Hq, d, seed, tag, step, spread=0.3):
    """Block queries = shared per-(row, head) direction + small per-position
    term.  Returns (queries float32 [B, nq, Hq, d], directions [B, Hq, d])."""
    w = normal((B, Hq, d), seed, "W", scale=1.0 / math.sqrt(d))
    e = normal((B, nq, Hq, d), seed, tag, step, scale=spread / math.sqrt(d))
    return w[:, None] + e, w


def _plant(x, positions, u, alpha, k_typ, h):
    """Overwrite key rows ``positions`` of head ``h`` in the float32 block
    ``x [n, Hkv, d]`` with ``alpha * k_typ * u + noise already in x``."""
    x[positions, h] += np.float32(alpha * k_typ) * u[None, :]


# ---------------------------------------------------------------------------
# The five workloads (and reduced copies of them for fast parity tests)
# ---------------------------------------------------------------------------

def tiny_dense(seed: int = 0, prefix: int = 256, C: int = 512) -> Workload:
    B, Hq, Hkv, d, bl, W = 1, 4, 4, 64, 32, 1
    q = W * bl
    s = 1.0 / math.sqrt(d)
    o = torch.full((B,), prefix, dtype=torch.int32)
    Kc = _fill_cache(B, C, Hkv, d, "f32", o, q, seed, "K", s)
    Vc = _fill_cache(B, C, Hkv, d, "f32", o, q, seed, "V", s)
    Q = to_dtype(normal((B, q, Hq, d), seed, "Q", scale=s), "f32")
    return Workload("tiny_dense", "f32", B, Hq, Hkv, d, bl, W, C, seed, Kc, Vc, o, Q,
                    sm_scale=s, n_layers=1)


def packed_wavefront(seed: int = 0, B: int = 8, C: int = 4096, W: int = 2,
                     o_lo: int = 512, o_hi: int = 3968, Hq: int = 32, Hkv: int = 8,
                     d: int = 128, bl: int = 32, align: int = 32,
                     dtype: str = "bf16") -> Workload:
    q = W * bl
    s = 1.0 / math.sqrt(d)
    r = rng(seed, "O")
    if align > 1:
        o = torch.from_numpy(r.integers(o_lo // align, o_hi // align + 1, size=B) * align)
    else:
        o = torch.from_numpy(r.integers(o_lo, o_hi + 1, size=B))
    o = o.to(torch.int32)
    Kc = _fill_cache(B, C, Hkv, d, dtype, o, q, seed, "K", s)
    Vc = _fill_cache(B, C, Hkv, d, dtype, o, q, seed, "V", s)
    Q = to_dtype(normal((B, q, Hq, d), seed, "Q", scale=s), dtype)
    return Workload("packed_wavefront", dtype, B, Hq, Hkv, d, bl, W, C, seed, Kc, Vc, o, Q,
                    sm_scale=s, n_layers=1)


def _sparse(name, seed, B, S, Hq, Hkv, d, bl, T, kv_scale, plant_fn,
            budget=0.05, dtype="bf16"):
    W = 1
    q = W * bl
    C = S + 2 * q            # block lands at [S, S+q); present tail at [C-q, C)
    s = 1.0 / math.sqrt(d)
    G = Hq // Hkv
    o = torch.full((B,), S, dtype=torch.int32)
    Qsel_f, w = _shared_queries(B, bl, Hq, d, seed, "Q", 0)
    # planted direction per (b, h): unit vector of the sum of the group's directions
    u = np.zeros((B, Hkv, d), np.float32)
    for b in range(B):
        for h in range(Hkv):
            v = w[b, h * G:(h + 1) * G].sum(axis=0)
            u[b, h] = v / np.linalg.norm(v)
    planted = {}
    k_typ = kv_scale * math.sqrt(d)

    def rows_fn(b, x):
        for h in range(Hkv):
            pos = plant_fn(b, h)
            planted[(b, h)] = pos
            _plant(x, pos, u[b, h], 4.0, k_typ, h)

    Kc = _fill_cache(B, C, Hkv, d, dtype, o, q, seed, "K", kv_scale, rows_fn=rows_fn)
    Vc = _fill_cache(B, C, Hkv, d, dtype, o, q, seed, "V", kv_scale)
    Qsel = to_dtype(Qsel_f, dtype)
    # denoising-step queries: same shared directions, fresh per-position terms;
    # denoising-step window KV: fresh draws per step
    steps, step_kv = [], []
    for st in range(T):
        e = normal((B, q, Hq, d), seed, "STEPQ", st, scale=0.3 / math.sqrt(d))
        steps.append(to_dtype(w[:, None] + e, dtype))
        wk = to_dtype(normal((B, q, Hkv, d), seed, "STEPK", st, scale=kv_scale), dtype)
        wv = to_dtype(normal((B, q, Hkv, d), seed, "STEPV", st, scale=kv_scale), dtype)
        step_kv.append((wk, wv))
    k = budget_keys(S, budget)
    wl = Workload(name, dtype, B, Hq, Hkv, d, bl, W, C, seed, Kc, Vc, o, steps[0],
                  sm_scale=s, n_layers=1,
                  sparse_rows=torch.arange(B, dtype=torch.int32),
                  dense_rows=torch.zeros(0, dtype=torch.int32),
                  s_len=torch.full((B,), S, dtype=torch.int32),
                  k_sel=torch.full((B,), k, dtype=torch.int32),
                  Qsel=Qsel, planted=planted, T=T)
    wl.extra["step_q"] = steps
    wl.extra["step_kv"] = step_kv
    return wl


def sparse_32k(seed: int = 0, B: int = 4, S: int = 32768, T: int = 8, Hq: int = 32,
               Hkv: int = 8, d: int = 128, plant_frac: float = 0.02) -> Workload:
    n_plant = int(math.floor(plant_frac * S + 0.5))

    def plant_fn(b, h):
        return np.sort(rng(seed, "PLANT", b, h).choice(S, size=n_plant, replace=False))

    return _sparse("sparse_32k", seed, B, S, Hq, Hkv, d, 32, T,
                   kv_scale=1.0 / math.sqrt(d), plant_fn=plant_fn)


def sparse_128k(seed: int = 0, S: int = 131072, T: int = 16, Hq: int = 32, Hkv: int = 8,
                d: int = 128, every: int = 64) -> Workload:
    n = S // every
    pos = np.arange(n) * every + rng(seed, "PLANT", 0).integers(0, every, size=n)

    def plant_fn(b, h):
        return pos           # the same heavy-hitter positions in every head

    return _sparse("sparse_128k", seed, 1, S, Hq, Hkv, d, 32, T,
                   kv_scale=1.0, plant_fn=plant_fn)


def serving_mix(seed: int = 0, B: int = 64, p_lo: int = 1024, p_hi: int = 16384,
                W: int = 4, bl: int = 32, Hq: int = 32, Hkv: int = 8, d: int = 128,
                sparse_above: int = 8192, budget: float = 0.05, C: int | None = None,
                dtype: str = "bf16") -> Workload:
    q = W * bl
    if C is None:
        C = p_hi + 2 * q
    s = 1.0 / math.sqrt(d)
    r = rng(seed, "O")
    draw = np.exp(r.uniform(math.log(p_lo), math.log(p_hi), size=B))
    o = np.clip(np.floor(draw / bl + 0.5).astype(np.int64) * bl, bl, p_hi)
    o = torch.from_numpy(o).to(torch.int32)
    Kc = _fill_cache(B, C, Hkv, d, dtype, o, q, seed, "K", s)
    Vc = _fill_cache(B, C, Hkv, d, dtype, o, q, seed, "V", s)
    Q = to_dtype(normal((B, q, Hq, d), seed, "Q", scale=s), dtype)
    sparse = (o > sparse_above)
    sparse_rows = torch.nonzero(sparse).flatten().to(torch.int32)
    dense_rows = torch.nonzero(~sparse).flatten().to(torch.int32)
    s_len = torch.where(sparse, o, torch.zeros_like(o)).to(torch.int32)
    k_sel = torch.tensor([budget_keys(int(v), budget) if sp else 0
                          for v, sp in zip(o.tolist(), sparse.tolist())], dtype=torch.int32)
    return Workload("serving_mix", dtype, B, Hq, Hkv, d, bl, W, C, seed, Kc, Vc, o, Q,
                    sm_scale=s, n_layers=1, sparse_rows=sparse_rows, dense_rows=dense_rows,
                    s_len=s_len, k_sel=k_sel, Qsel=Q, T=1)


WORKLOADS = {
    "tiny_dense": tiny_dense,
    "packed_wavefront": packed_wavefront,
    "sparse_32k": sparse_32k,
    "sparse_128k": sparse_128k,
    "serving_mix": serving_mix,
}
