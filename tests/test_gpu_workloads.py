"""GPU parity on the full-size synthetic workloads (KV4-RL Qwen3-shaped decode
states), in the launch configuration the benchmark times (automatic wave count,
max_ctx = the longest sequence).

  * Qwen3-4B shape, batch 64 (lognormal median 2k): every sequence, bytes and
    output, against the oracle;
  * long context, batch 16 x 32,768: every sequence's output, bytes of a
    sample of sequences;
  * Qwen3-8B shape, batch 256 (lognormal median 4k, max 16k): the output of
    every (sequence, q head) row against the oracle, computed 32 sequences at a
    time; bytes of sampled sequences (shortest, longest, median, random ones);
  * the integer decode path on the same batch: every row against the oracle's
    integer path;
  * the KV8 mode on the same batch: every row's output, bytes of sampled
    sequences;
  * 36 layers x 64 decode steps, batch 128 (contexts uniform 1k..12k): every
    step appends one token per sequence and layer and decodes; the output of
    every sequence against the oracle at layers {0, 17, 35} x steps {0, 31,
    63}; bytes of sampled sequences after the last step; and, at every step,
    the pages that were full before the first step unchanged at the sampled
    layers (a position's INT4 bytes are written once, when it is appended).
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


def _q8b256_sample(seed):
    """Shortest, longest and median sequences of the Qwen3-8B batch and a few
    random ones (for byte comparisons)."""
    cfg = W.CONFIGS["q8b256"]
    ctx = W.contexts(cfg)
    order = np.argsort(ctx)
    rng = np.random.default_rng(seed)
    return sorted(set([int(order[0]), int(order[-1]), int(order[len(order) // 2])] +
                      [int(s) for s in rng.choice(cfg.batch, size=5, replace=False)]))


def _all_rows(cfg, built, out, check_chunk, chunk=32):
    """Regenerate every sequence's sources, 32 at a time, and hand each chunk
    (sequence ids, keys, values) to check_chunk."""
    ctx = W.contexts(cfg)
    n = ctx + 1
    for lo in range(0, cfg.batch, chunk):
        seqs = list(range(lo, min(cfg.batch, lo + chunk)))
        ks, vs = W.all_kv_sources(cfg, 0, n, seqs=seqs, threads=16)
        check_chunk(seqs, ks, vs)


def _build_q8b256(**kw):
    cfg = W.CONFIGS["q8b256"]
    ctx = W.contexts(cfg)
    n = ctx + 1
    H.log(f"case q8b256 {kw}: B={cfg.batch} sum(n)={int(n.sum())} max={int(n.max())}")
    S, R = (0, 0) if kw.get("kind", 0) else (cfg.sink, cfg.recent)
    built = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, S, R, n, seed=cfg.seed, **kw)
    _fill_garbage(built)
    H.build_streaming(built, cfg, 0, ctx, keep=())
    q = W.queries(cfg, 0)
    out = H.decode(built, 0, q, n).cpu().numpy()
    assert np.all(np.isfinite(out))
    return cfg, n, q, built, out


@pytest.mark.timeout(900)
def test_qwen3_8b_batch256_all_rows():
    """Every (sequence, q head) row of the benchmarked workload, in the
    benchmark's launch configuration, against the oracle; bytes of sampled
    sequences bit for bit."""
    cfg, n, q, built, out = _build_q8b256()
    pages, side = H.pools_host(built)
    sm = 1 / math.sqrt(cfg.head_dim)
    byte_seqs = set(_q8b256_sample(123))
    worst = [0.0, 0.0]

    def check(seqs, ks, vs):
        oc = oracle.MixedCache(ks, vs, cfg.group)
        want = oracle.attend_mixed(q[seqs], oc, cfg.sink, cfg.recent, sm)
        err = H.check_output(out[seqs], want, ATOL, RTOL)
        worst[0], worst[1] = max(worst[0], err[0]), max(worst[1], err[1])
        idx = [i for i, s in enumerate(seqs) if s in byte_seqs]
        if idx:
            sub = oracle.MixedCache([ks[i] for i in idx], [vs[i] for i in idx], cfg.group)
            _compare_bytes(built, pages, side, 0, sub, cfg.sink, cfg.recent, seqs=[seqs[i] for i in idx])
        H.log(f"  sequences {seqs[0]}..{seqs[-1]}: max abs {err[0]:.2e} rel {err[1]:.2e}")

    _all_rows(cfg, built, out, check)
    H.log(f"q8b256: all {cfg.batch} x {cfg.q_heads} rows, max abs {worst[0]:.2e} rel {worst[1]:.2e}")


@pytest.mark.timeout(900)
def test_qwen3_8b_batch256_integer_path_all_rows():
    """Integer decode path (KV4_FLAG_INT_PATH) on the benchmarked workload:
    every row against the oracle's integer path within 1e-4 plus the tie-flip
    bound, and an rms far below the path's own error."""
    from int8_mixed_precision_amd import kv4
    from tests.test_gpu_parity import INT_ATOL
    cfg, n, q, built, out = _build_q8b256(flags=kv4.KV4_FLAG_INT_PATH)
    out = out.astype(np.float64)
    sm = 1 / math.sqrt(cfg.head_dim)
    acc = dict(sq_dev=0.0, sq_own=0.0, cnt=0, worst=0.0)

    def check(seqs, ks, vs):
        oc = oracle.MixedCache(ks, vs, cfg.group)
        want, bound = oracle.attend_int(q[seqs], oc, cfg.sink, cfg.recent, sm)
        exact = oracle.attend_mixed(q[seqs], oc, cfg.sink, cfg.recent, sm)
        err = np.abs(out[seqs] - want)
        excess = err - (INT_ATOL + bound)
        assert excess.max() <= 0, (seqs[0], float(excess.max()))
        acc["sq_dev"] += float(np.sum((out[seqs] - want) ** 2))
        acc["sq_own"] += float(np.sum((want - exact) ** 2))
        acc["cnt"] += want.size
        acc["worst"] = max(acc["worst"], float(err.max()))
        H.log(f"  sequences {seqs[0]}..{seqs[-1]}: max |o - o_int| {err.max():.2e}")

    _all_rows(cfg, built, out, check)
    dev = math.sqrt(acc["sq_dev"] / acc["cnt"])
    own = math.sqrt(acc["sq_own"] / acc["cnt"])
    H.log(f"q8b256 integer path: all rows, max |o - o_int| {acc['worst']:.2e}, rms {dev:.2e}; "
          f"path vs exact rms {own:.2e}")
    assert dev <= 0.1 * own + 1e-6


@pytest.mark.timeout(900)
def test_qwen3_8b_batch256_kv8_all_rows():
    """KV8 mode on the benchmarked batch: every row's output against the
    oracle's attention with every position protected; bytes of sampled
    sequences against its INT8 copies."""
    from int8_mixed_precision_amd import kv4
    from tests import layout as L
    cfg, n, q, built, out = _build_q8b256(kind=kv4.KV4_KIND_KV8)
    pages, _ = H.pools_host(built)
    sm = 1 / math.sqrt(cfg.head_dim)
    byte_seqs = set(_q8b256_sample(125))

    def check(seqs, ks, vs):
        oc = oracle.MixedCache(ks, vs, cfg.group)
        want = oracle.attend_mixed(q[seqs], oc, 0, int(n.max()), sm)
        err = H.check_output(out[seqs], want, ATOL, RTOL)
        for i, b in enumerate(seqs):
            if b not in byte_seqs:
                continue
            got = L.gather_kv8(pages, layer=0, num_pages=built.desc.num_pages, Hkv=cfg.kv_heads,
                               d=cfg.head_dim, block_tables=built.bt_host,
                               slot=int(built.slots_host[b]), n=int(n[b]))
            for name in ("k8", "v8", "k8s", "v8s"):
                assert np.array_equal(got[name], getattr(oc, name)[oc.seq(i)]), (b, name)
        H.log(f"  sequences {seqs[0]}..{seqs[-1]}: max abs {err[0]:.2e} rel {err[1]:.2e}")

    _all_rows(cfg, built, out, check)


def test_qwen3_4b_shape_full():
    _run("q4b")


def test_long_context_full():
    _run("long", byte_sample=[0, 7, 15])


def test_full36_decode_steps():
    from tests import layout as L
    from int8_mixed_precision_amd import kv4
    cfg = W.CONFIGS["full36"]
    dev = torch.device("cuda")
    ctx = W.contexts(cfg)
    B, steps, Lyr = cfg.batch, cfg.steps, cfg.layers
    total = ctx + steps                          # positions each sequence ends with
    H.log(f"case full36: {Lyr} layers x {steps} steps, B={B}, sum(ctx)={int(ctx.sum())}")
    built = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, cfg.sink, cfg.recent, total,
                         layers=Lyr, seed=cfg.seed)
    c = built.cache
    out_ch = W.outlier_channels(cfg)
    sample_layers, sample_steps = (0, 17, 35), (0, 31, 63)
    cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
    # ---- history of every layer, and the step tokens kept on the device
    step_k = torch.empty((Lyr, steps, B, cfg.kv_heads, cfg.head_dim), dtype=torch.bfloat16, device=dev)
    step_v = torch.empty_like(step_k)
    for layer in range(Lyr):
        for lo in range(0, B, 16):
            seqs = list(range(lo, min(B, lo + 16)))
            ks, vs = [], []
            for b in seqs:
                k, v = W.kv_sources_device(cfg, layer, b, int(total[b]), dev, out_ch)
                ks.append(k[:int(ctx[b])])
                vs.append(v[:int(ctx[b])])
                step_k[layer, :, b] = k[int(ctx[b]):]
                step_v[layer, :, b] = v[int(ctx[b]):]
            cnt = np.array([int(ctx[b]) for b in seqs])
            cu = torch.from_numpy(np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)).to(dev)
            kv4.kv4_append(c.handle, layer, torch.cat(ks).contiguous(), torch.cat(vs).contiguous(),
                           cu, torch.zeros(len(seqs), dtype=torch.int32, device=dev),
                           built.slots[lo:lo + len(seqs)].contiguous(), built.block_tables,
                           len(seqs), int(cnt.sum()))
        torch.cuda.synchronize()
        if layer % 6 == 5:
            H.log(f"  built layer {layer}")
    # ---- snapshot of the pages that are full before the first step
    pages4 = c.page_pool.view(Lyr, built.desc.num_pages, -1)
    full_ids = np.concatenate([built.bt_host[built.slots_host[b], :int(ctx[b]) // 16] for b in range(B)])
    full_ids = torch.from_numpy(full_ids.astype(np.int64)).to(dev)
    snap = {layer: pages4[layer].index_select(0, full_ids).clone() for layer in sample_layers}
    # ---- decode steps: append + decode on every layer
    outs = {}
    sm = 1.0 / math.sqrt(cfg.head_dim)
    for step in range(steps):
        before = torch.from_numpy((ctx + step).astype(np.int32)).to(dev)
        n_d = before + 1
        max_ctx = int(ctx.max()) + step + 1
        for layer in range(Lyr):
            kv4.kv4_append(c.handle, layer, step_k[layer, step].contiguous(),
                           step_v[layer, step].contiguous(), cu1, before, built.slots,
                           built.block_tables, B, B)
            q = W.queries_device(cfg, layer, step, dev)
            o = c.decode(layer, q, n_d, built.slots, built.block_tables, max_ctx, sm)
            if layer in sample_layers and step in sample_steps:
                outs[(layer, step)] = (q.float().cpu().numpy(), o.cpu().numpy())
        for layer in sample_layers:
            assert torch.equal(pages4[layer].index_select(0, full_ids), snap[layer]), \
                f"full pages of layer {layer} changed at step {step}"
        if step % 16 == 15:
            H.log(f"  step {step} done")
    torch.cuda.synchronize()
    # ---- oracle: every sequence at the sampled (layer, step) pairs; bytes of
    # four sequences per sampled layer after the last step
    order = np.argsort(ctx)
    byte_seqs = {int(order[0]), int(order[-1]), int(order[B // 2]), 7}
    side4 = c.side_pool.view(Lyr, built.desc.max_slots, -1)
    worst = 0.0
    for layer in sample_layers:
        reps = []
        for b in range(B):
            k, v = W.kv_sources_device(cfg, layer, b, int(total[b]), dev, out_ch)
            kf, vf = k.float().cpu().numpy(), v.float().cpu().numpy()
            k4, k4d, k4m = oracle.quant_int4(kf, cfg.group)
            v4, v4d, v4m = oracle.quant_int4(vf, cfg.group)
            k8, k8s = oracle.quant_int8(kf)
            v8, v8s = oracle.quant_int8(vf)
            reps.append((k4, k4d, k4m, v4, v4d, v4m, k8, k8s, v8, v8s))
            if b in byte_seqs:
                nb = int(total[b])
                npg = -(-nb // 16)
                ids = built.bt_host[built.slots_host[b], :npg].astype(np.int64)
                pg = pages4[layer].index_select(0, torch.from_numpy(ids).to(dev)).cpu().numpy().ravel()
                sd = side4[layer, int(built.slots_host[b])].cpu().numpy().ravel()
                pm = L.protected_mask(nb, cfg.sink, cfg.recent)
                gm = L.gather_mixed(pg, sd, layer=0, num_pages=npg, Hkv=cfg.kv_heads, d=cfg.head_dim,
                                    G=cfg.group, S=cfg.sink, R=cfg.recent, max_slots=1,
                                    block_tables=np.arange(npg, dtype=np.int32)[None], slot=0, n=nb,
                                    protected_mask=pm)
                for name, want in zip(("k4", "k4d", "k4m", "v4", "v4d", "v4m"), reps[-1][:6]):
                    assert np.array_equal(gm[name], want), f"layer {layer} seq {b}: {name} differs"
                for name, want in zip(("k8", "k8s", "v8", "v8s"), reps[-1][6:]):
                    assert np.array_equal(gm[name][pm], want[pm]), f"layer {layer} seq {b}: {name} differs"
        for step in sample_steps:
            q, got = outs[(layer, step)]
            want = np.empty(got.shape, np.float64)
            for b in range(B):
                nb = int(ctx[b]) + step + 1
                r = [x[:nb] for x in reps[b]]
                want[b] = oracle.attend_mixed_raw(q[b:b + 1], [nb], [0], cfg.kv_heads, cfg.group,
                                                  cfg.sink, cfg.recent, sm, *r)[0]
            err = H.check_output(got, want, ATOL, RTOL)
            worst = max(worst, err[0])
            H.log(f"  layer {layer} step {step}: max abs {err[0]:.2e} row rel {err[1]:.2e}")
    H.log(f"full36: worst max abs {worst:.2e}")
