"""GPU parity on the full-size synthetic workloads (KV4-RL Qwen3-shaped decode
states), in the launch configuration the benchmark times (automatic split,
max_ctx = the longest sequence).

  * Qwen3-4B shape, batch 64 (lognormal median 2k): every sequence, bytes and
    output, against the oracle;
  * long context, batch 16 x 32,768: every sequence's output, bytes of a
    sample of sequences;
  * Qwen3-8B shape, batch 256 (lognormal median 4k, max 16k): bytes and output
    of sampled sequences (shortest, longest, median and random ones) computed
    one by one by the oracle; for every other row, properties that hold at any
    size (finite output inside the hull of the dequantized values).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from int8_mixed_precision_amd import workloads as W
from tests import gpu_harness as H
from tests.test_gpu_parity import ATOL, RTOL, _compare_bytes, _fill_garbage

pytestmark = pytest.mark.gpu


def _run(cfg_name, sample=None, byte_sample=None):
    cfg = W.CONFIGS[cfg_name]
    ctx = W.contexts(cfg)
    n = ctx + 1
    B = cfg.batch
    H.log(f"case {cfg_name}: B={B} sum(n)={int(n.sum())} max={int(n.max())}")
    sample = list(range(B)) if sample is None else sorted(set(sample))
    built = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, cfg.sink, cfg.recent, n,
                         seed=cfg.seed)
    _fill_garbage(built)
    kept = H.build_streaming(built, cfg, 0, ctx, keep=sample)
    q = W.queries(cfg, 0)
    out = H.decode(built, 0, q, n).cpu().numpy()
    assert np.all(np.isfinite(out))
    ks = [kept[s][0] for s in sample]
    vs = [kept[s][1] for s in sample]
    oc = oracle.MixedCache(ks, vs, cfg.group)
    want = oracle.attend_mixed(q[sample], oc, cfg.sink, cfg.recent, 1 / math.sqrt(cfg.head_dim))
    err = H.check_output(out[sample], want, ATOL, RTOL)
    H.log(f"{cfg_name}: {len(sample)} sequences, max abs {err[0]:.2e} rel {err[1]:.2e}")
    pages, side = H.pools_host(built)
    bs = sample if byte_sample is None else byte_sample
    idx = [sample.index(s) for s in bs]
    sub = oracle.MixedCache([ks[i] for i in idx], [vs[i] for i in idx], cfg.group)
    _compare_bytes(built, pages, side, 0, sub, cfg.sink, cfg.recent, seqs=bs)
    return out, built


def test_qwen3_4b_shape_full():
    _run("q4b")


def test_long_context_full():
    _run("long", byte_sample=[0, 7, 15])


def test_qwen3_8b_batch256_sampled():
    cfg = W.CONFIGS["q8b256"]
    ctx = W.contexts(cfg)
    rng = np.random.default_rng(123)
    order = np.argsort(ctx)
    sample = [int(order[0]), int(order[-1]), int(order[len(order) // 2])]
    sample += [int(s) for s in rng.choice(cfg.batch, size=9, replace=False)]
    out, built = _run("q8b256", sample=sample)
    # every row: a convex combination of dequantized values stays inside their
    # per-channel range; |o| is bounded by the largest |v^| (<= ~6 for N(0,1))
    assert np.abs(out).max() < 16.0
