"""Seeded synthetic workloads for the KV4 decode step.

This module only draws inputs: query, key and value tensors and context
lengths with the shapes of the KV4-RL workloads (Qwen3-4B/8B attention
geometry: 32 query heads, 8 kv heads, head dim 128; 16-token pages).  It holds
none of the method's arithmetic, so the fp64 oracle and the HIP path can both
be fed from it.

Recipe (the same for every config):
  * values are drawn with numpy ``default_rng`` from a seed sequence
    ``[config seed, layer, sequence or step, stream tag]`` as float32 N(0, 1),
    then rounded to bfloat16 (round to nearest even) with torch on the CPU;
  * "outlier" key channels are picked once per config, one per distinct
    32-channel group, and their key values are multiplied (in float32, before
    the bf16 rounding) by the config's factor, in every kv head;
  * a sequence's sources cover positions [0, context + steps): the history
    plus the token(s) appended by the decode step(s); "context" is the length
    before the step's append, so a decode step attends over context + 1
    positions;
  * ragged lengths: lognormal with the stated median and sigma 0.8, rounded
    and clipped; uniform lengths are integers drawn uniformly.
Every sequence's sources depend only on (seed, layer, sequence), so any subset
can be regenerated without drawing the rest.  The 36-layer multi-step workload
is drawn on the device instead (kv_sources_device), same recipe, seeded per
(layer, sequence).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

TAG_K, TAG_V, TAG_Q, TAG_CTX, TAG_OUTLIER = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    layers: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    page: int
    group: int
    sink: int
    recent: int
    seed: int
    outliers: int
    outlier_scale: float
    ctx_kind: str                     # "fixed", "lognormal", "uniform"
    ctx_fixed: Tuple[int, ...] = ()
    ctx_median: float = 0.0
    ctx_sigma: float = 0.8
    ctx_lo: int = 0
    ctx_hi: int = 0
    steps: int = 1

    @property
    def gqa(self) -> int:
        return self.q_heads // self.kv_heads


CONFIGS = {
    # 1 layer, batch 2, 8 q / 2 kv heads, contexts 300 and 512, S=4, R=64,
    # 2 outlier K channels x8, seed 0.
    "tiny": Config("tiny", 1, 2, 8, 2, 128, 16, 32, 4, 64, 0, 2, 8.0, "fixed", (300, 512)),
    # Qwen3-4B-shaped layer, batch 64, lognormal median 2k clipped 256..8k, R=128,
    # 4 outlier K channels x10, seed 1.
    "q4b": Config("q4b", 1, 64, 32, 8, 128, 16, 32, 4, 128, 1, 4, 10.0, "lognormal",
                  ctx_median=2048, ctx_lo=256, ctx_hi=8192),
    # Qwen3-8B-shaped layer, batch 256, long-tail lognormal median 4k, max 16k,
    # R=128, seed 2 (the benchmarked workload).
    "q8b256": Config("q8b256", 1, 256, 32, 8, 128, 16, 32, 4, 128, 2, 4, 10.0, "lognormal",
                     ctx_median=4096, ctx_lo=256, ctx_hi=16384),
    # Long context: batch 16, every context 32768, R=256, seed 3.
    "long": Config("long", 1, 16, 32, 8, 128, 16, 32, 4, 256, 3, 4, 10.0, "fixed",
                   tuple([32768] * 16)),
    # One GPU's share of the Qwen3-8B layer under two-way tensor parallelism:
    # config q8b256's batch and contexts with 16 q / 4 kv heads, seed 2.
    "q8b256tp2": Config("q8b256tp2", 1, 256, 16, 4, 128, 16, 32, 4, 128, 2, 4, 10.0, "lognormal",
                        ctx_median=4096, ctx_lo=256, ctx_hi=16384),
    # 36 layers, batch 128, contexts uniform 1k..12k, R=128, seed 4, 64 steps.
    "full36": Config("full36", 36, 128, 32, 8, 128, 16, 32, 4, 128, 4, 4, 10.0, "uniform",
                     ctx_lo=1024, ctx_hi=12288, steps=64),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even) and return them as float32."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def contexts(cfg: Config) -> np.ndarray:
    """Context lengths before the step's append, one per sequence."""
    if cfg.ctx_kind == "fixed":
        c = np.array(cfg.ctx_fixed, dtype=np.int64)
        assert c.size == cfg.batch
        return c
    r = _rng(cfg.seed, TAG_CTX)
    if cfg.ctx_kind == "lognormal":
        v = r.lognormal(mean=np.log(cfg.ctx_median), sigma=cfg.ctx_sigma, size=cfg.batch)
        return np.clip(np.round(v), cfg.ctx_lo, cfg.ctx_hi).astype(np.int64)
    if cfg.ctx_kind == "uniform":
        return r.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=cfg.batch).astype(np.int64)
    raise ValueError(cfg.ctx_kind)


def outlier_channels(cfg: Config, groups_of: int = 32) -> np.ndarray:
    """Key channels scaled as outliers: one channel in each of ``outliers``
    distinct ``groups_of``-channel groups."""
    if cfg.outliers == 0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(cfg.seed, TAG_OUTLIER)
    ngroups = cfg.head_dim // groups_of
    assert cfg.outliers <= ngroups
    groups = r.choice(ngroups, size=cfg.outliers, replace=False)
    return np.sort(groups * groups_of + r.integers(0, groups_of, size=cfg.outliers))


def kv_sources(cfg: Config, layer: int, seq: int, n: int,
               outliers: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values of positions [0, n) of one sequence: float32 arrays
    [n, kv_heads, head_dim] holding bf16 values.

    The draw for position p does not depend on n (rows are drawn in order), so a
    shorter n gives a prefix of a longer one."""
    if outliers is None:
        outliers = outlier_channels(cfg)
    shape = (n, cfg.kv_heads, cfg.head_dim)
    k = _rng(cfg.seed, layer, seq, TAG_K).standard_normal(shape, dtype=np.float32)
    v = _rng(cfg.seed, layer, seq, TAG_V).standard_normal(shape, dtype=np.float32)
    if outliers.size:
        k[:, :, outliers] *= np.float32(cfg.outlier_scale)
    return to_bf16_values(k), to_bf16_values(v)


def queries(cfg: Config, layer: int, step: int = 0) -> np.ndarray:
    """Decode-step queries [batch, q_heads, head_dim] (bf16 values in float32)."""
    q = _rng(cfg.seed, layer, step, TAG_Q).standard_normal(
        (cfg.batch, cfg.q_heads, cfg.head_dim), dtype=np.float32)
    return to_bf16_values(q)


def all_kv_sources(cfg: Config, layer: int, lengths: Sequence[int],
                   seqs: Optional[Sequence[int]] = None,
                   threads: int = 8) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """Sources of many sequences, drawn on a thread pool."""
    seqs = list(range(len(lengths))) if seqs is None else list(seqs)
    out = outlier_channels(cfg)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        res = list(ex.map(lambda s: kv_sources(cfg, layer, s, int(lengths[s]), out), seqs))
    return [r[0] for r in res], [r[1] for r in res]


def device_seed(*key: int) -> int:
    """63-bit seed of a device generator, mixed from integer keys."""
    st = np.random.SeedSequence([int(k) for k in key]).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def kv_sources_device(cfg: Config, layer: int, seq: int, n: int, device,
                      outliers: Optional[np.ndarray] = None):
    """Keys and values of positions [0, n) of one sequence drawn on `device`
    with a seeded counter-based generator: bf16 tensors [n, kv_heads,
    head_dim].  Same recipe as kv_sources (N(0, 1) in float32, outlier key
    channels scaled before rounding), different stream: for the workloads too
    large to draw on the host.  A draw is reproducible for the same (n,
    device) only, so callers always pass a sequence's full length."""
    if outliers is None:
        outliers = outlier_channels(cfg)
    shape = (n, cfg.kv_heads, cfg.head_dim)
    out = []
    for tag in (TAG_K, TAG_V):
        gen = torch.Generator(device=device)
        gen.manual_seed(device_seed(cfg.seed, layer, seq, tag))
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if tag == TAG_K and outliers.size:
            x[:, :, torch.as_tensor(outliers, device=device)] *= cfg.outlier_scale
        out.append(x.to(torch.bfloat16))
    return out[0], out[1]


def queries_device(cfg: Config, layer: int, step: int, device):
    """Decode-step queries [batch, q_heads, head_dim] as bf16 on `device`."""
    gen = torch.Generator(device=device)
    gen.manual_seed(device_seed(cfg.seed, layer, step, TAG_Q))
    q = torch.randn((cfg.batch, cfg.q_heads, cfg.head_dim), generator=gen, device=device,
                    dtype=torch.float32)
    return q.to(torch.bfloat16)


def scaled(cfg: Config, **changes) -> Config:
    """A copy of a config with some fields replaced (for reduced test sizes)."""
    return dataclasses.replace(cfg, **changes)


# Group kinds of extreme_kv_sources, in the order they cycle.
EXTREME_KINDS = ("normal", "tiny", "f32_subnormal", "constant", "near_max", "int4_ties",
                 "scaled", "two_values")


def extreme_kv_sources(seed: int, n: int, kv_heads: int, head_dim: int, group: int,
                       int8_tie_rows: Sequence[int] = ()) -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values [n, kv_heads, head_dim] (bf16 values in float32) whose
    channel groups of ``group`` channels cycle through the EXTREME_KINDS value
    patterns, all inside |x| <= 65280 (the largest bf16 value below the binary16
    limit 65504):
      normal        N(0, 1);
      tiny          N(0, 1) * 1e-6 (offset and step fall in the binary16
                    subnormal range);
      f32_subnormal half the group 1e-39 (below binary32's normal range), the
                    rest N(0, 1);
      constant      one repeated value (0, -0, 3.140625, -1e-30, 65280 or -2^-20);
      near_max      values spread over [-65280, 65280], including both ends;
      int4_ties     the integers 0..15 followed by half-integers (a step of 1
                    and offset 0 put those exactly between two codes);
      scaled        N(0, 1) times 10^k, k in [-6, 3];
      two_values    a random mix of -1.5 and 2.25.
    Rows listed in ``int8_tie_rows`` hold, in every kv head, 127 followed by
    half-integers (exact ties of a symmetric 8-bit code with scale 1).
    Seeded by ``seed`` only."""
    r = _rng(seed, TAG_K, 777)
    shape = (n, kv_heads, head_dim)
    ng = head_dim // group
    consts = np.array([0.0, -0.0, 3.140625, -1e-30, 65280.0, -2.0 ** -20], np.float32)
    halves = np.array([2.5, 3.5, 4.5, 0.5, 14.5, 7.5, 8.5, 1.5, 0.25, 0.75, 13.5, 9.0, 10.0,
                       11.0, 12.0, 5.5], np.float32)
    out = []
    for tensor in range(2):
        x = np.empty(shape, np.float32)
        for t in range(n):
            for h in range(kv_heads):
                for g in range(ng):
                    kind = EXTREME_KINDS[(t * kv_heads * ng + h * ng + g + 3 * tensor) % len(EXTREME_KINDS)]
                    if kind == "normal":
                        v = r.standard_normal(group)
                    elif kind == "tiny":
                        v = r.standard_normal(group) * 1e-6
                    elif kind == "f32_subnormal":
                        v = r.standard_normal(group)
                        v[r.permutation(group)[: group // 2]] = 1e-39
                    elif kind == "constant":
                        v = np.full(group, consts[r.integers(consts.size)])
                    elif kind == "near_max":
                        v = r.uniform(-65280.0, 65280.0, group)
                        v[0], v[-1] = 65280.0, -65280.0
                    elif kind == "int4_ties":
                        base = np.concatenate([np.arange(16, dtype=np.float32), halves])
                        v = np.resize(base, group)
                    elif kind == "scaled":
                        v = r.standard_normal(group) * 10.0 ** int(r.integers(-6, 4))
                    else:
                        v = r.choice(np.array([-1.5, 2.25]), size=group)
                    x[t, h, g * group:(g + 1) * group] = v
        for t in int8_tie_rows:
            row = np.zeros(head_dim, np.float32)
            row[0] = 127.0
            ties = np.array([0.5, 1.5, 2.5, -2.5, -3.5, 100.5, 101.5, -126.5], np.float32)
            row[1:1 + ties.size] = ties
            row[1 + ties.size:] = r.integers(-120, 121, head_dim - 1 - ties.size)
            x[t, :, :] = row
        out.append(to_bf16_values(np.clip(x, -65280.0, 65280.0)))
    return out[0], out[1]
