"""Helpers for the GPU parity tests: build a paged cache on the device from
seeded sources, run the decode step, read pools back (test code only)."""
from __future__ import annotations

import math
import sys
from typing import List, Optional, Sequence

import numpy as np
import torch

from int8_mixed_precision_amd import kv4
from int8_mixed_precision_amd import workloads as W
from int8_mixed_precision_amd.paged import (PAGE, Built, append_chunks, make_cache,  # noqa: F401
                                            page_tables, to_dev_bf16)


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def build_from_sources(built: Built, layer: int, k_src, v_src, ctx: Sequence[int],
                       chunk_tokens: int = 1 << 22):
    """History [0, ctx_b) in bulk, then the step token at position ctx_b
    (a separate append, as a decode step does)."""
    B = len(k_src)
    group, tok = [], 0
    for b in range(B):
        group.append(b)
        tok += int(ctx[b])
        if tok >= chunk_tokens or b == B - 1:
            ks = [k_src[i][:int(ctx[i])] for i in group]
            vs = [v_src[i][:int(ctx[i])] for i in group]
            if sum(x.shape[0] for x in ks) > 0:
                append_chunks(built, layer, ks, vs, [0] * len(group), group)
            group, tok = [], 0
    ks = [k_src[b][int(ctx[b]):int(ctx[b]) + 1] for b in range(B)]
    vs = [v_src[b][int(ctx[b]):int(ctx[b]) + 1] for b in range(B)]
    append_chunks(built, layer, ks, vs, [int(c) for c in ctx])


def decode(built: Built, layer: int, q: np.ndarray, n: Sequence[int], max_ctx=None,
           sm_scale=None, out_dtype=kv4.KV4_OUT_F32, device="cuda") -> torch.Tensor:
    dev = torch.device(device)
    n = np.asarray(n, np.int32)
    max_ctx = int(n.max()) if max_ctx is None else max_ctx
    qd = to_dev_bf16(q, device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    return built.cache.decode(layer, qd, torch.from_numpy(n).to(dev), built.slots, built.block_tables,
                              max_ctx, sm_scale, out_dtype=out_dtype)


def pools_host(built: Built):
    torch.cuda.synchronize()
    pages = built.cache.page_pool.cpu().numpy()
    side = built.cache.side_pool.cpu().numpy() if built.cache.side_pool is not None else None
    return pages, side


def check_output(got: np.ndarray, want: np.ndarray, atol=1e-3, rtol=2e-3, rows=None):
    """max |o - o*| <= atol and, per (sequence, q head) row,
    ||o - o*||_inf / max(||o*||_inf, 1e-6) <= rtol."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    worst = float(err.max()) if err.size else 0.0
    rowmax = np.abs(want).max(axis=-1)
    rel = err.max(axis=-1) / np.maximum(rowmax, 1e-6)
    assert worst <= atol, f"max abs error {worst:.3e} > {atol} at {np.unravel_index(err.argmax(), err.shape)}"
    assert float(rel.max()) <= rtol, f"max row-relative error {float(rel.max()):.3e} > {rtol}"
    return worst, float(rel.max())


def build_streaming(built: Built, cfg: W.Config, layer: int, ctx: np.ndarray, keep=(),
                    chunk_seqs: int = 32, threads: int = 8):
    """Draw each sequence's sources (history + step token), append the history
    chunk by chunk and then every step token in one decode-style append.
    Returns {seq: (k, v)} for the sequences in `keep`."""
    keep = set(int(s) for s in keep)
    kept = {}
    step_k, step_v = [], []
    B = len(ctx)
    for lo in range(0, B, chunk_seqs):
        seqs = list(range(lo, min(B, lo + chunk_seqs)))
        ks, vs = W.all_kv_sources(cfg, layer, ctx + 1, seqs=seqs, threads=threads)
        hist = [i for i, s in enumerate(seqs) if ctx[s] > 0]
        if hist:
            append_chunks(built, layer, [ks[i][:int(ctx[seqs[i]])] for i in hist],
                          [vs[i][:int(ctx[seqs[i]])] for i in hist], [0] * len(hist),
                          [seqs[i] for i in hist])
        for i, s in enumerate(seqs):
            step_k.append(ks[i][int(ctx[s]):int(ctx[s]) + 1])
            step_v.append(vs[i][int(ctx[s]):int(ctx[s]) + 1])
            if s in keep:
                kept[s] = (ks[i], vs[i])
        torch.cuda.synchronize()
    append_chunks(built, layer, step_k, step_v, [int(c) for c in ctx])
    return kept
