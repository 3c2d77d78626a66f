"""Workload recipes: the five synthetic configurations and the tables they draw.

Each configuration fixes shapes, a seed, a plan (kind of every (loop, layer)
cell), per-cell K/V scale factors, per-(cell, head) outlier channels, sequence
lengths and a block table. Small tables are drawn with numpy's PCG64 under
fixed child seeds; the K/V/Q values themselves come from the Philox stream in
``synth.philox`` so that the GPU can draw the same bits in place.

Cell kinds: 0 = 4-bit (hi/lo planes), 1 = 2-bit, 2 = reuse of the final
loop's KV of the same layer.

Element indexing of the value streams (all uint64):
* K and V of cell ``c``: stream ``4c+1`` (K) / ``4c+2`` (V),
  index ``((b * T + t) * H + h) * D + d`` with ``T = cfg.token_stride``;
* Q of cell ``c`` at decode step ``k``: stream ``4c+3``,
  index ``((k * B + b) * H + h) * D + d``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .philox import normal_f32, f32_to_bf16_bits, scaled_bf16_bits

Q4, Q2, SHARE = 0, 1, 2
STREAM_Q, STREAM_K, STREAM_V = 3, 1, 2


@dataclass
class Config:
    name: str
    n_loops: int
    n_layers: int
    n_heads: int
    head_dim: int
    batch: int
    lengths: List[int]            # tokens per sequence at the first decode step
    taus: List[float]
    q_fp32: bool = False
    outlier_count: int = 0
    outlier_mult: float = 1.0
    cell_scales: bool = False
    shuffled: bool = False
    append_steps: int = 0         # decode steps, each preceded by a 1-token append
    seed: int = 0
    plan: Optional[np.ndarray] = field(default=None, repr=False)
    n_kv_heads: int = 0           # 0: one KV head per query head
    block_tokens: int = 16        # tokens per page of the block table (16 or 32)
    group: int = 32               # quantization group (32 or 64)

    @property
    def kv_heads(self) -> int:
        return self.n_kv_heads or self.n_heads

    @property
    def n_cells(self) -> int:
        return self.n_loops * self.n_layers

    @property
    def max_len(self) -> int:
        return max(self.lengths) + self.append_steps

    @property
    def token_stride(self) -> int:
        return self.max_len

    @property
    def bt_stride(self) -> int:
        return (self.max_len + self.block_tokens - 1) // self.block_tokens


def random_plan(n_loops: int, n_layers: int, seed: int, frac=(0.5, 0.3, 0.2)) -> np.ndarray:
    """Plan with exact counts round(frac * cells); reuse cells only in loops before the last."""
    n = n_loops * n_layers
    n_share = int(round(frac[2] * n))
    n_q4 = int(round(frac[0] * n))
    rng = np.random.default_rng([seed, 1])
    kinds = np.full(n, -1, dtype=np.int64)
    non_final = np.arange((n_loops - 1) * n_layers)
    share = rng.permutation(non_final)[:n_share]
    kinds[share] = SHARE
    rest = np.flatnonzero(kinds < 0)
    rest = rng.permutation(rest)
    kinds[rest[:n_q4]] = Q4
    kinds[rest[n_q4:]] = Q2
    return kinds.astype(np.uint8).reshape(n_loops, n_layers)


def storage_cell(plan: np.ndarray, cell: int) -> int:
    """Cell whose cache a cell reads: itself, or the final loop's cell of its layer."""
    n_loops, n_layers = plan.shape
    if plan.reshape(-1)[cell] == SHARE:
        return (n_loops - 1) * n_layers + cell % n_layers
    return cell


def make_config(name: str, seed: int = 0) -> Config:
    if name == "C1":
        cfg = Config("C1", 1, 1, 2, 64, 1, [256], [0.01], q_fp32=True,
                     outlier_count=4, outlier_mult=8.0, seed=seed)
    elif name == "C2":
        cfg = Config("C2", 1, 1, 16, 128, 8, [4096] * 8, [0.005],
                     outlier_count=int(round(0.02 * 128)), outlier_mult=10.0, seed=seed)
    elif name == "C3":
        cfg = Config("C3", 4, 24, 16, 128, 32, [8192] * 32, [0.0, 0.001, 0.01, 1.1],
                     cell_scales=True, seed=seed)
    elif name == "C4":
        cfg = Config("C4", 4, 24, 16, 128, 32, [16384] * 32, [0.0, 0.001, 0.01, 1.1],
                     cell_scales=True, shuffled=True, seed=seed)
    elif name == "C5":
        rng = np.random.default_rng([seed, 4])
        lengths = rng.integers(1024, 16384, size=128, endpoint=True).tolist()
        cfg = Config("C5", 4, 24, 16, 128, 128, lengths, [0.01],
                     cell_scales=True, shuffled=True, append_steps=64, seed=seed)
    else:
        raise ValueError(name)
    if cfg.n_cells == 1:
        cfg.plan = np.zeros((1, 1), dtype=np.uint8)
    else:
        cfg.plan = random_plan(cfg.n_loops, cfg.n_layers, seed)
    return cfg


def small_config(name: str, n_loops: int, n_layers: int, n_heads: int, head_dim: int,
                 lengths: List[int], taus: List[float], plan=None, seed: int = 0,
                 outlier_count: int = 0, outlier_mult: float = 1.0, cell_scales: bool = False,
                 shuffled: bool = False, q_fp32: bool = False, append_steps: int = 0,
                 n_kv_heads: int = 0, block_tokens: int = 16, group: int = 32) -> Config:
    """A reduced configuration with the same generators, for tests that the oracle finishes quickly."""
    cfg = Config(name, n_loops, n_layers, n_heads, head_dim, len(lengths), list(lengths), list(taus),
                 q_fp32=q_fp32, outlier_count=outlier_count, outlier_mult=outlier_mult,
                 cell_scales=cell_scales, shuffled=shuffled, append_steps=append_steps, seed=seed,
                 n_kv_heads=n_kv_heads, block_tokens=block_tokens, group=group)
    if plan is None:
        plan = np.zeros((n_loops, n_layers), dtype=np.uint8) if n_loops * n_layers == 1 \
            else random_plan(n_loops, n_layers, seed)
    cfg.plan = np.asarray(plan, dtype=np.uint8).reshape(n_loops, n_layers)
    return cfg


def factor_table(cfg: Config) -> np.ndarray:
    """float32 [cells][2 (K, V)][KV heads][D]: outlier multiplier times the cell's scale."""
    C, H, D = cfg.n_cells, cfg.kv_heads, cfg.head_dim
    f = np.ones((C, 2, H, D), dtype=np.float64)
    if cfg.cell_scales:
        rng = np.random.default_rng([cfg.seed, 2])
        sc = np.exp(rng.uniform(math.log(0.5), math.log(4.0), size=(C, 2)))
        f *= sc[:, :, None, None]
    if cfg.outlier_count:
        rng = np.random.default_rng([cfg.seed, 3])
        for c in range(C):
            for kv in range(2):
                for h in range(H):
                    ch = rng.choice(D, size=cfg.outlier_count, replace=False)
                    f[c, kv, h, ch] *= cfg.outlier_mult
    return f.astype(np.float32)


def block_table(cfg: Config) -> np.ndarray:
    """int32 [B][bt_stride]: physical page of each logical page of cfg.block_tokens tokens
    (-1 if unused).

    Each sequence owns ceil(max length it reaches / block_tokens) pages; ids are handed
    out in order (identity) or from a seeded permutation (shuffled)."""
    P = cfg.block_tokens
    need = [(n + cfg.append_steps + P - 1) // P for n in cfg.lengths]
    total = int(sum(need))
    ids = np.arange(total, dtype=np.int64)
    if cfg.shuffled:
        ids = np.random.default_rng([cfg.seed, 5]).permutation(total)
    bt = np.full((cfg.batch, cfg.bt_stride), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = ids[pos:pos + n]
        pos += n
    return bt


def num_blocks(cfg: Config) -> int:
    P = cfg.block_tokens
    return int(sum((n + cfg.append_steps + P - 1) // P for n in cfg.lengths))


def kv_index(cfg: Config, b, t, h, d):
    T, H, D = cfg.token_stride, cfg.kv_heads, cfg.head_dim
    b = np.asarray(b, dtype=np.uint64)
    t = np.asarray(t, dtype=np.uint64)
    h = np.asarray(h, dtype=np.uint64)
    d = np.asarray(d, dtype=np.uint64)
    return ((b * np.uint64(T) + t) * np.uint64(H) + h) * np.uint64(D) + d


def kv_row_bits(cfg: Config, cell: int, b: int, h: int, t0: int, t1: int, factors=None):
    """bf16 bits of K and V, each [t1-t0][D], for one (cell, sequence, KV head)."""
    if factors is None:
        factors = factor_table(cfg)
    D = cfg.head_dim
    t = np.arange(t0, t1, dtype=np.uint64)[:, None]
    d = np.arange(D, dtype=np.uint64)[None, :]
    idx = kv_index(cfg, b, t, h, d)
    k = scaled_bf16_bits(cfg.seed, 4 * cell + STREAM_K, idx, factors[cell, 0, h][None, :])
    v = scaled_bf16_bits(cfg.seed, 4 * cell + STREAM_V, idx, factors[cell, 1, h][None, :])
    return k, v


def kv_tensor_bits(cfg: Config, cell: int, t0: int, t1: int, factors=None):
    """bf16 bits of K and V, each [B][t1-t0][KV heads][D], for one cell (append input layout)."""
    if factors is None:
        factors = factor_table(cfg)
    B, H, D = cfg.batch, cfg.kv_heads, cfg.head_dim
    b = np.arange(B, dtype=np.uint64)[:, None, None, None]
    t = np.arange(t0, t1, dtype=np.uint64)[None, :, None, None]
    h = np.arange(H, dtype=np.uint64)[None, None, :, None]
    d = np.arange(D, dtype=np.uint64)[None, None, None, :]
    idx = kv_index(cfg, b, t, h, d)
    k = scaled_bf16_bits(cfg.seed, 4 * cell + STREAM_K, idx, factors[cell, 0][None, None])
    v = scaled_bf16_bits(cfg.seed, 4 * cell + STREAM_V, idx, factors[cell, 1][None, None])
    return k, v


def q_values(cfg: Config, cell: int, step: int, b=None, h=None):
    """Query of one cell at one decode step: float32 [B][H][D] (exact fp32 draws when
    ``cfg.q_fp32``, otherwise bf16-rounded and returned widened to float32), or one
    row [D] when ``b`` and ``h`` are given."""
    B, H, D = cfg.batch, cfg.n_heads, cfg.head_dim
    if b is None:
        bb = np.arange(B, dtype=np.uint64)[:, None, None]
        hh = np.arange(H, dtype=np.uint64)[None, :, None]
    else:
        bb = np.uint64(b)
        hh = np.uint64(h)
    dd = np.arange(D, dtype=np.uint64)
    idx = ((np.uint64(step) * np.uint64(B) + bb) * np.uint64(H) + hh) * np.uint64(D) + dd
    z = normal_f32(cfg.seed, 4 * cell + STREAM_Q, idx)
    if cfg.q_fp32:
        return z
    return (f32_to_bf16_bits(z).astype(np.uint32) << np.uint32(16)).view(np.float32)
