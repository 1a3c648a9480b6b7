#!/usr/bin/env python3
"""Benchmark of the KV4 decode step on one MI355X.

A step is one pass of the hot path over one batch: kv4_append of the batch's
new token (INT4 pages + INT8 ring) followed by kv4_decode_attn (GQA attention
over the ragged paged contexts, cut by a balanced partition over the GPU's
waves, + the log-sum-exp merge), each bracketed by HIP events.  The
workload is the Qwen3-8B-shaped layer (32 q / 8 kv heads, d = 128) at batch
256 with long-tail lognormal contexts (median 4k, max 16k), 16-token pages,
INT4 group 32, S = 4, R = 128.  Inputs are seeded synthetic data, resident in
HBM before the timed region.  Every step re-appends the same token at the same
position (idempotent) and decodes over the same contexts, so each timed step
does the full work on identical state.

Output: one JSON line: the metric and its value (algorithmic bytes of the step
per second), the step time, the dominant kernel's roofline (achieved vs peak HBM
bandwidth, measured traffic), the comparators, the populate rate and the oracle's
CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0             # dense bf16 matrix-core peak of MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=90,
                    help="timed steps (reported also as three blocks of a third each)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="q8b256")
    ap.add_argument("--waves", type=int, default=0,
                    help="waves of the decode partition (0 = the library's choice, 16 per CU)")
    ap.add_argument("--pool-chunks", type=int, default=0,
                    help="most chunks of the decode's dynamic pool (0 = none, the default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-kv8", action="store_true",
                    help="skip the KV8 comparator (INT8 pages for every position)")
    ap.add_argument("--group", type=int, default=0,
                    help="INT4 group size of the KV4 cache (0 = the config's, 32)")
    ap.add_argument("--populate-reps", type=int, default=10,
                    help="timed bulk appends of the first 32 sequences' histories (0 = skip)")
    ap.add_argument("--no-valu", action="store_true",
                    help="skip the vector-ALU decode of the same KV4 bytes (KV4_FLAG_VALU_DECODE)")
    ap.add_argument("--valu-decode", action="store_true",
                    help="run the KV4 cache's decode on the vector-ALU kernel (KV4_FLAG_VALU_DECODE; "
                         "for profiling it)")
    ap.add_argument("--no-int-path", action="store_true",
                    help="skip the integer decode path (KV4_FLAG_INT_PATH) over the same KV4 bytes")
    ap.add_argument("--prefill-reps", type=int, default=3,
                    help="timed prefill attentions over the populate histories (0 = skip)")
    ap.add_argument("--only-kv4", action="store_true",
                    help="time the KV4 decode only (no comparators, sub-records, populate, prefill or "
                         "CPU baseline): the command the counter profiles run")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill attention over the first 32 histories of the workload "
                         "as prompts (the command the prefill profiles run)")
    ap.add_argument("--populate-only", action="store_true",
                    help="time only the bulk populate of the first 32 histories of the workload (the "
                         "command the append profiles run)")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the sub-records (G = 128 rotated, Qwen3-4B shape, long context) and "
                         "the read ceilings")
    ap.add_argument("--rotate", action="store_true",
                    help="store keys in the rotated basis (KV4_FLAG_ROTATE_K) in the KV4 cache")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "decode_kv4_mfma_kernel_qwen3-8b_b256_counters.json"))
    # summaries of rocprofv3 output (no GPU work): kernel durations from a
    # --kernel-trace csv directory; counters and HBM traffic from --pmc csv
    # directories
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="rocprofv3 --pmc output directories (one per counter pass)")
    ap.add_argument("--summary-out", metavar="FILE")
    ap.add_argument("--summary-cmd", default="", help="command that produced the profile")
    ap.add_argument("--summary-bench", metavar="JSON",
                    help="bench line printed by the profiled run (live event timings)")
    ap.add_argument("--summary-kernel", default="decode_kv4_mfma_kernel",
                    help="kernel-name substring whose counters are summarised")
    ap.add_argument("--summary-last", type=int, default=0,
                    help="summarise only the last N dispatches of that kernel (0 = all)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def region_counts(n, S, R):
    sink_end = np.minimum(S, n)
    rec_start = np.maximum(S, n - R)
    n4 = np.maximum(rec_start - S, 0)
    n8 = sink_end + np.maximum(n - rec_start, 0)
    return n4, n8


def partial_bytes_kv4(n, cfg):
    """Algorithmic bytes of the attention phase (kv4_decode_partials, one
    kernel): payload + metadata of both regions, q, block-table entries of the
    INT4 pages.  160 B per (INT4 token, kv head) and 260 B per (protected
    token, kv head) at d = 128, G = 32."""
    n4, n8 = region_counts(n, cfg.sink, cfg.recent)
    ng = cfg.head_dim // cfg.group
    per4 = cfg.head_dim + 2 * 2 * 2 * ng            # K+V codes (d/2 each) + K,V (Delta, m) fp16
    per8 = 2 * cfg.head_dim + 2 * 2                 # K+V int8 + two fp16 scales
    kv = int(np.sum(cfg.kv_heads * (per4 * n4 + per8 * n8)))
    qb = len(n) * cfg.q_heads * cfg.head_dim * 2
    bt = int(np.sum(4 * np.ceil(n4 / 16)))
    return kv + qb + bt


def decode_bytes_kv4(n, cfg):
    """Algorithmic bytes of one kv4_decode_attn call: the attention phase's
    plus the fp32 output."""
    return partial_bytes_kv4(n, cfg) + len(n) * cfg.q_heads * cfg.head_dim * 4


def decode_bytes_bf16(n, cfg):
    kv = int(np.sum(cfg.kv_heads * 2 * cfg.head_dim * 2 * n))
    return kv + len(n) * cfg.q_heads * cfg.head_dim * (2 + 4) + int(np.sum(4 * np.ceil(n / 16)))


def partial_bytes_kv8(n, cfg):
    """KV8 kind: 2 d int8 codes + two fp16 scales per (token, kv head), q,
    block-table entries."""
    kv = int(np.sum(cfg.kv_heads * (2 * cfg.head_dim + 4) * n))
    return kv + len(n) * cfg.q_heads * cfg.head_dim * 2 + int(np.sum(4 * np.ceil(n / 16)))


def append_bytes_kv4(n, cfg):
    """Reads bf16 k, v of the new tokens; writes their INT4 entries and (every
    new token is recent when R >= 1) their INT8 entries."""
    B = len(n)
    rd = B * cfg.kv_heads * cfg.head_dim * 2 * 2
    ng = cfg.head_dim // cfg.group
    wr = B * cfg.kv_heads * (cfg.head_dim + 8 * ng + (2 * cfg.head_dim + 4 if cfg.recent > 0 else 0))
    return rd + wr


def populate_bytes_kv4(hist, cfg):
    """Bulk append of whole histories (prefill populate): reads bf16 k, v;
    writes every position's INT4 entry and the INT8 entries of the positions
    protected at the new length."""
    T = int(np.sum(hist))
    ng = cfg.head_dim // cfg.group
    rd = T * cfg.kv_heads * cfg.head_dim * 2 * 2
    wr4 = T * cfg.kv_heads * (cfg.head_dim + 8 * ng)
    wr8 = int(np.sum(np.minimum(hist, cfg.sink + cfg.recent))) * cfg.kv_heads * (2 * cfg.head_dim + 4)
    return rd + wr4 + wr8


def prefill_flops(lens, cfg):
    """Causal attention of every prompt position over its prefix: 2 d flops per
    (query, key, q head) for the scores and as many for the values."""
    lens = np.asarray(lens, np.float64)
    return float(np.sum(cfg.q_heads * 2 * cfg.head_dim * lens * (lens + 1)))


def append_bytes_bf16(n, cfg):
    return len(n) * cfg.kv_heads * cfg.head_dim * 2 * 2 * 2


DOMINANT = "decode_kv4_mfma_kernel"
TP_NOTE = {"q8b256tp2": " (one GPU's share under two-way tensor parallelism)"}


def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        rows.extend(csv.DictReader(open(f)))
    return rows


def _short(name):
    return name.split("(")[0].replace("void ", "").replace("kv4::", "")


def summarize_trace(args):
    """Per-kernel launch count and duration statistics from a kernel trace."""
    rows = _csv_rows(args.summarize_trace, "kernel_trace.csv")
    per = {}
    for r in rows:
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        per.setdefault(_short(r["Kernel_Name"]), []).append(dur)
    total = sum(sum(v) for v in per.values())
    lines = [f"# rocprofv3 kernel trace summary: {args.summary_cmd}", "",
             f"{'kernel':44s} {'calls':>6s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s} "
             f"{'max_us':>10s} {'total_%':>8s}"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(v) / 1e3
        k = k if len(k) <= 44 else k[:41] + "..."
        lines.append(f"{k:44s} {len(v):6d} {a.mean():10.2f} {np.median(a):10.2f} {a.min():10.2f} "
                     f"{a.max():10.2f} {100 * a.sum() * 1e3 / total:8.2f}")
    bench_line = json.loads(open(args.summary_bench).read().strip().splitlines()[-1]) if args.summary_bench else {}
    if "populate" in bench_line and "decode_attn_us" not in bench_line:
        p = bench_line["populate"]
        lines += ["", "live HIP-event timing of the same run (mean over the timed calls):",
                  f"  kv4_append (append_kv4_kernel): {p['us']} us for {p['tokens']} tokens in "
                  f"{p['sequences']} histories: {p['gbs']} GB/s of algorithmic bytes "
                  f"= {p['frac_hbm_peak']} of the HBM peak",
                  "kernel counts include the untimed call"]
    elif args.summary_bench and "prefill" in bench_line and "decode_attn_us" not in bench_line:
        p = json.loads(open(args.summary_bench).read().strip().splitlines()[-1])["prefill"]
        lines += ["", "live HIP-event timing of the same run (mean over the timed calls):",
                  f"  kv4_prefill_attn (prefill_attn_kernel): {p['us']} us for {p['tokens']} tokens in "
                  f"{p['sequences']} prompts (longest {p['max_prompt']}): {p['tflops']} TFLOP/s "
                  f"= {p['frac_mfma_bf16_peak']} of the bf16 matrix-core peak",
                  "kernel counts include the warm-up call"]
    elif args.summary_bench:
        b = json.loads(open(args.summary_bench).read().strip().splitlines()[-1])
        lines += ["", "live HIP-event timings of the same run (mean over the timed steps):",
                  f"  kv4_decode_attn (the whole call, partials + merge back to back): {b['decode_attn_us']} us",
                  f"  kv4_decode_partials ({DOMINANT}) alone: {b['decode_partials_us']} us",
                  f"  kv4_decode_merge (merge_parts_kernel) alone: {b['decode_merge_us']} us",
                  f"  kv4_append (append_kv4_kernel<32>): {b['append_us']} us"]
        if "bf16_comparator" in b:
            lines.append(f"  BF16 comparator partials (decode_bf16_mfma_kernel): "
                         f"{b['bf16_comparator']['decode_partials_us']} us")
        if "int_path" in b:
            lines.append(f"  integer path partials (decode_int_mfma_kernel): "
                         f"{b['int_path']['decode_partials_us']} us")
        if "kv8_comparator" in b:
            lines.append(f"  KV8 comparator partials (decode_kv8_mfma_kernel): "
                         f"{b['kv8_comparator']['decode_partials_us']} us")
        lines.append("kernel counts include warm-up steps, the cache build's bulk appends and one "
                     "kv4_decode_attn check call")
    text = "\n".join(lines) + "\n"
    if args.summary_out:
        open(args.summary_out, "w").write(text)
    print(text)


def summarize_counters(args):
    """Per-launch counters of the dominant kernel from rocprofv3 --pmc runs
    (one directory per pass), averaged over its dispatches, and the HBM
    traffic they give:
      read bytes  = 32 TCC_EA0_RDREQ_32B + 64 TCC_EA0_RDREQ_64B + 128 TCC_EA0_RDREQ_128B
                    (the L2's read requests to memory by size);
      write bytes = 64 TCC_EA0_WRREQ_64B + 32 (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B);
    and the factor by which the FETCH_SIZE / WRITE_SIZE metrics of this
    rocprofv3 build differ from those request-size sums."""
    vals = {}
    kernel = args.summary_kernel
    for d in args.summarize_counters:
        rows = [r for r in _csv_rows(d, "counter_collection.csv") if kernel in r["Kernel_Name"]]
        keep = sorted({int(r["Dispatch_Id"]) for r in rows})
        last = getattr(args, "summary_last", 0)
        keep = set(keep[-last:] if last > 0 else keep)
        for r in rows:
            if int(r["Dispatch_Id"]) not in keep:
                continue
            key = (r["Counter_Name"], d, int(r["Dispatch_Id"]))
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    per = {}
    for (name, _, _), v in vals.items():
        per.setdefault(name, []).append(v)
    mean = {k: float(np.mean(v)) for k, v in per.items()}
    launches = {k: len(v) for k, v in per.items()}
    out = dict(kernel=kernel, kernel_source_hash=_kernel_hash(kernel), commands=args.summary_cmd,
               counters_per_launch=mean, launches=launches)
    if all(k in mean for k in ("TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B")):
        rd = 32 * mean["TCC_EA0_RDREQ_32B"] + 64 * mean["TCC_EA0_RDREQ_64B"] + 128 * mean["TCC_EA0_RDREQ_128B"]
        out["read_bytes_per_launch"] = rd
        if "FETCH_SIZE" in mean:
            out["fetch_size_factor"] = rd / (mean["FETCH_SIZE"] * 1024.0)
    if all(k in mean for k in ("TCC_EA0_WRREQ", "TCC_EA0_WRREQ_64B")):
        wr = 64 * mean["TCC_EA0_WRREQ_64B"] + 32 * (mean["TCC_EA0_WRREQ"] - mean["TCC_EA0_WRREQ_64B"])
        out["write_bytes_per_launch"] = wr
        if "WRITE_SIZE" in mean:
            out["write_size_factor"] = wr / (mean["WRITE_SIZE"] * 1024.0)
    if "read_bytes_per_launch" in out and "write_bytes_per_launch" in out:
        out["bytes_per_launch"] = int(round(out["read_bytes_per_launch"] + out["write_bytes_per_launch"]))
    if "TCC_HIT" in mean and "TCC_MISS" in mean:
        out["l2_hit_rate"] = mean["TCC_HIT"] / max(1.0, mean["TCC_HIT"] + mean["TCC_MISS"])
    if args.summary_out:
        json.dump(out, open(args.summary_out, "w"), indent=1)
    print(json.dumps(out, indent=1))


class Timer:
    """HIP events on the stream every launch goes to (torch's current stream)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e


def build_caches(cfg, specs, H, W, kv4, dev, keep_first=0):
    """Build every cache in `specs` ({name: make_cache kwargs}) from the same
    seeded sources, 32 sequences at a time; return the caches, the step
    tokens on the device, and the histories of the first `keep_first`
    sequences (for the populate and prefill timings)."""
    ctx = W.contexts(cfg)
    n = ctx + 1
    B = cfg.batch
    caches = {name: H.make_cache(cfg.q_heads, cfg.kv_heads, kw.pop("group", cfg.group),
                                 kw.pop("sink", cfg.sink), kw.pop("recent", cfg.recent), n,
                                 seed=cfg.seed, device=str(dev), **kw)
              for name, kw in ((k, dict(v)) for k, v in specs.items())}
    step_k, step_v, first = [], [], None
    for lo in range(0, B, 32):
        seqs = list(range(lo, min(B, lo + 32)))
        ks, vs = W.all_kv_sources(cfg, 0, n, seqs=seqs, threads=16)
        if lo == 0 and keep_first:
            first = [(ks[i][:int(ctx[s])], vs[i][:int(ctx[s])]) for i, s in enumerate(seqs[:keep_first])]
        hist = [i for i, s in enumerate(seqs) if ctx[s] > 0]
        for c in caches.values():
            H.append_chunks(c, 0, [ks[i][:int(ctx[seqs[i]])] for i in hist],
                            [vs[i][:int(ctx[seqs[i]])] for i in hist], [0] * len(hist),
                            [seqs[i] for i in hist], device=str(dev))
        for i, s in enumerate(seqs):
            step_k.append(ks[i][int(ctx[s]):int(ctx[s]) + 1])
            step_v.append(vs[i][int(ctx[s]):int(ctx[s]) + 1])
        kv4_sync(dev)
    knew = H.to_dev_bf16(np.concatenate(step_k, 0), str(dev))
    vnew = H.to_dev_bf16(np.concatenate(step_v, 0), str(dev))
    return caches, knew, vnew, first


def kv4_sync(dev):
    import torch
    torch.cuda.synchronize(dev)


def time_step(c, cfg, n, knew, vnew, q, kv4, torch, tm, steps, warmup, flush=None,
              clock_warm_s=0.0):
    """`warmup` untimed steps, then `steps` timed steps of (append,
    kv4_decode_attn) on cache c, each bracketed by events (the append and the
    attention call apart); then `steps` more with the two phases of the
    attention (kv4_decode_partials, kv4_decode_merge) bracketed apart, for the
    split.  Every step re-appends the same token at the same position
    (idempotent), so each does the full work on identical state.  `flush`
    (untimed, between steps) evicts the caches for workloads that fit in
    them.  Returns per-step milliseconds."""
    dev = knew.device
    B = len(n)
    ctx = n - 1
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    ctx_d = torch.from_numpy(ctx.astype(np.int32)).to(dev)
    n_d = torch.from_numpy(n.astype(np.int32)).to(dev)
    max_ctx = int(n.max())
    sm = 1.0 / math.sqrt(cfg.head_dim)
    out = torch.empty((B, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    whole = torch.empty_like(out)
    ws = c.cache.workspace(B, max_ctx)
    st = tm.stream

    def append():
        kv4.kv4_append(c.cache.handle, 0, knew, vnew, cu, ctx_d, c.slots, c.block_tables, B, B, st)

    def attn():
        kv4.kv4_decode_attn(c.cache.handle, 0, q, n_d, c.slots, c.block_tables, B, max_ctx, sm, whole,
                            kv4.KV4_OUT_F32, ws, st)

    def partials():
        kv4.kv4_decode_partials(c.cache.handle, 0, q, n_d, c.slots, c.block_tables, B, max_ctx, sm, ws, st)

    def merge():
        kv4.kv4_decode_merge(c.cache.handle, n_d, B, max_ctx, out, kv4.KV4_OUT_F32, ws, st)

    if clock_warm_s > 0:
        # untimed: bring the clocks up before the first timed launch
        t_end = time.perf_counter() + clock_warm_s
        while time.perf_counter() < t_end:
            for _ in range(8):
                append(); attn()
            torch.cuda.synchronize()
    for _ in range(warmup):
        if flush:
            flush()
        append(); attn()
    torch.cuda.synchronize()

    def timed(phases):
        evs = []
        for i in range(steps):
            if flush:
                flush()
            e = [tm.ev()]
            for f in phases:
                f()
                e.append(tm.ev())
            evs.append(e)
        torch.cuda.synchronize()
        return np.array([[e[k].elapsed_time(e[k + 1]) for k in range(len(e) - 1)] for e in evs])

    t = timed((append, attn))                 # the step as a caller runs it
    ph = timed((append, partials, merge))     # the attention's two phases apart
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(whole, out), "kv4_decode_attn differs from partials + merge"
    waves, chunks = kv4.kv4_decode_partition(c.cache.handle)
    ta, td = t[:, 0], t[:, 1]
    tp, tmg = ph[:, 1], ph[:, 2]
    return dict(append_ms=float(ta.mean()), partials_ms=float(tp.mean()), merge_ms=float(tmg.mean()),
                decode_ms=float(td.mean()), decode_ms_median=float(np.median(td)),
                decode_ms_p10=float(np.percentile(td, 10)), decode_ms_p90=float(np.percentile(td, 90)),
                decode_ms_block_medians=[float(np.median(x)) for x in np.array_split(td, 3) if len(x)],
                partials_ms_median=float(np.median(tp)), waves=waves, pool_chunks=chunks)


class _SharedPools:
    """A second library handle over a built cache's pools with another q head
    count (the pools depend on the kv heads only), in the shape time_step
    expects of a cache."""

    def __init__(self, built, num_q_heads, kv4, torch):
        d = kv4.kv4_cache_desc.from_buffer_copy(built.desc)
        d.num_q_heads = num_q_heads
        self.desc, self.device, self._kv4, self._torch = d, built.cache.device, kv4, torch
        self.handle = kv4.kv4_cache_create(d, built.cache.page_pool, built.cache.side_pool)
        self._ws = None

    def workspace(self, batch, max_ctx):
        nb = self._kv4.kv4_decode_workspace_bytes(self.handle, batch, max_ctx)
        if self._ws is None or self._ws.numel() < nb:
            self._ws = self._torch.empty(max(nb, 16), dtype=self._torch.uint8, device=self.device)
        return self._ws

    def close(self):
        self._kv4.kv4_cache_free(self.handle)


def ratio8_record(c, cfg, n, knew, vnew, H, W, kv4, torch, tm, args, dev):
    """The same batch and pools decoded with 8 q heads per kv head (64 q / 8
    kv: the Qwen3-32B head shape) on the matrix core (two four-head halves
    per tile)."""
    from types import SimpleNamespace
    c8 = W.scaled(cfg, q_heads=8 * cfg.kv_heads)
    q8 = H.to_dev_bf16(W.queries(c8, 0), str(dev))
    sp = _SharedPools(c, c8.q_heads, kv4, torch)
    try:
        r = time_step(SimpleNamespace(cache=sp, slots=c.slots, block_tables=c.block_tables), c8, n, knew,
                      vnew, q8, kv4, torch, tm, args.steps, args.warmup, clock_warm_s=0.3)
    finally:
        sp.close()
    p8, d8 = partial_bytes_kv4(n, c8), decode_bytes_kv4(n, c8)
    return {"workload": f"the same batch and pools with {c8.q_heads} q heads ({c8.q_heads}q/{c8.kv_heads}kv, "
                        f"q/kv ratio 8: the Qwen3-32B head shape)",
            "kernel": "decode_kv4_mfma8_kernel", "waves": r["waves"],
            "decode_attn_us": round(r["decode_ms"] * 1e3, 2),
            "decode_partials_us": round(r["partials_ms"] * 1e3, 2),
            "decode_merge_us": round(r["merge_ms"] * 1e3, 2),
            "partials_alg_bytes": p8,
            "partials_frac_hbm_peak": round(p8 / (r["partials_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_attn_frac_hbm_peak": round(d8 / (r["decode_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def read_ceiling(torch, dev, st, partial_bytes):
    """The read ceilings of this GPU (libkv4_roof.so): a 4 GiB stream, and
    random 2,560-byte blocks (one (page, kv head) block of the INT4 pool) in
    the decode's own launch shape -- 4,096 one-wave workgroups, two blocks in
    flight, nontemporal loads -- over as many bytes as the decode's tiles."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "int8_mixed_precision_amd", "libkv4_roof.so"))
    lib.kv4_roof_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.kv4_roof_block_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    tm = Timer(torch, st)
    sp = ctypes.c_void_p(st.cuda_stream)
    res = {}
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)

    def timed(fn, reps=10):
        for _ in range(3):
            assert fn() == 0
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = tm.ev(); assert fn() == 0; e1 = tm.ev()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    ms = timed(lambda: lib.kv4_roof_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, 32 * cus,
                                                ctypes.c_void_p(sink.data_ptr()), sp))
    res["stream_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    waves, blk = 16 * cus, 2560
    per = max(2, int(partial_bytes // blk // waves) // 2 * 2)
    nb = per * waves
    ids = torch.from_numpy(np.random.default_rng(7).permutation(nb).astype(np.int32)).to(dev)
    ms = timed(lambda: lib.kv4_roof_block_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                               ctypes.c_void_p(ids.data_ptr()), waves, per, blk,
                                               ctypes.c_void_p(sink.data_ptr()), sp))
    res["block2560_gbs"] = round(nb * blk / (ms * 1e-3) / 1e9, 1)
    res["block2560_us"] = round(ms * 1e3, 1)
    res["block2560_bytes"] = nb * blk
    res["kernels"] = ("libkv4_roof.so: stream_read_kernel (4 GiB, 8 x 16 B loads in flight per lane), "
                      f"block_read_kernel ({waves} one-wave workgroups x {per} random 2,560 B blocks, "
                      "2 in flight); nontemporal loads")
    del buf, ids
    torch.cuda.empty_cache()
    return res


def sub_record(name, cfg, kv4c_kw, H, W, kv4, torch, dev, tm, args, flush_bytes=0, bf16=True):
    """Decode-attention time, bandwidth and fraction of the HBM peak of one
    more workload (KV4 cache, and the BF16 comparator for the ratio)."""
    ctx = W.contexts(cfg)
    n = ctx + 1
    specs = {"kv4": dict(kv4c_kw)}
    if bf16:
        specs["bf16"] = dict(kind=kv4.KV4_KIND_BF16, sink=0, recent=0)
    caches, knew, vnew, _ = build_caches(cfg, specs, H, W, kv4, dev)
    q = H.to_dev_bf16(W.queries(cfg, 0), str(dev))
    flush = None
    if flush_bytes:
        # reading 1 GiB of other data evicts the 256 MB Infinity Cache (MALL)
        # with clean lines, so the timed decode neither hits it nor pays for
        # writing dirty flush data back
        scratch = torch.ones(flush_bytes // 4, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)

        def flush():
            torch.amax(scratch, dim=0, out=sink)
    res = {}
    for k, c in caches.items():
        res[k] = time_step(c, cfg, n, knew, vnew, q, kv4, torch, tm, args.steps, args.warmup, flush=flush)
    g = kv4c_kw.get("group", cfg.group)
    cg = W.scaled(cfg, group=g)
    db = decode_bytes_kv4(n, cg)
    pb = partial_bytes_kv4(n, cg)
    r = res["kv4"]
    out = {"workload": f"{cfg.name}: batch {cfg.batch}, {cfg.q_heads}q/{cfg.kv_heads}kv, group {g}, "
                       f"S={cfg.sink}, R={cfg.recent}, sum n {int(n.sum())}, max n {int(n.max())}",
           "decode_attn_us": round(r["decode_ms"] * 1e3, 2),
           "decode_attn_us_median": round(r["decode_ms_median"] * 1e3, 2),
           "decode_partials_us": round(r["partials_ms"] * 1e3, 2),
           "decode_merge_us": round(r["merge_ms"] * 1e3, 2),
           "append_us": round(r["append_ms"] * 1e3, 2),
           "decode_alg_bytes": db,
           "decode_attn_gbs": round(db / (r["decode_ms"] * 1e-3) / 1e9, 1),
           "decode_attn_frac_hbm_peak": round(db / (r["decode_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "partials_frac_hbm_peak": round(pb / (r["partials_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "layer_tokens_per_s": round(cfg.batch / ((r["append_ms"] + r["decode_ms"]) * 1e-3), 1)}
    if flush_bytes:
        out["cache_flush"] = f"{flush_bytes >> 20} MiB of other data read between steps (untimed)"
    if "bf16" in res:
        rb = res["bf16"]
        out["bf16_decode_attn_us"] = round(rb["decode_ms"] * 1e3, 2)
        out["speedup_vs_bf16_decode"] = round(rb["decode_ms"] / r["decode_ms"], 3)
        out["speedup_vs_bf16_step"] = round((rb["append_ms"] + rb["decode_ms"]) /
                                            (r["append_ms"] + r["decode_ms"]), 3)
    del caches, knew, vnew, q
    torch.cuda.empty_cache()
    log(f"{name}: decode {out['decode_attn_us']} us, {out['decode_attn_gbs']} GB/s "
        f"({100 * out['decode_attn_frac_hbm_peak']:.1f}% of peak)")
    return out


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1 "
                                   "(the decode step shards by sequence or kv head with no "
                                   "exchange inside the op)"}))
        sys.exit(2)

    import torch
    from int8_mixed_precision_amd import kv4
    from int8_mixed_precision_amd import paged as H
    from int8_mixed_precision_amd import workloads as W

    if args.config == "full36":
        return run_full36(args, torch, kv4, H, W)
    if args.prefill_only:
        return run_prefill_only(args, torch, kv4, H, W)
    if args.populate_only:
        return run_populate_only(args, torch, kv4, H, W)
    cfg = W.CONFIGS[args.config]
    if args.group:
        cfg = W.scaled(cfg, group=args.group)
    ctx = W.contexts(cfg)
    n = ctx + 1
    B = cfg.batch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    tm = Timer(torch, stream)
    t0 = time.time()
    log(f"config {cfg.name}: B={B} sum(n)={int(n.sum())} max n={int(n.max())}")

    common = dict(waves=args.waves, pool_chunks=args.pool_chunks)
    specs = {"kv4": dict(common, flags=(kv4.KV4_FLAG_ROTATE_K if args.rotate else 0) |
                                       (kv4.KV4_FLAG_VALU_DECODE if args.valu_decode else 0))}
    if not args.only_kv4:
        if not args.no_bf16:
            specs["bf16"] = dict(common, kind=kv4.KV4_KIND_BF16, sink=0, recent=0)
        if not args.no_valu and not args.valu_decode:
            specs["valu"] = dict(common, flags=kv4.KV4_FLAG_VALU_DECODE |
                                 (kv4.KV4_FLAG_ROTATE_K if args.rotate else 0))
        if not args.no_int_path:
            specs["int"] = dict(common, flags=kv4.KV4_FLAG_INT_PATH |
                                (kv4.KV4_FLAG_ROTATE_K if args.rotate else 0))
        if not args.no_kv8:
            specs["kv8"] = dict(common, kind=kv4.KV4_KIND_KV8, sink=0, recent=0)
        if not args.no_sub and cfg.name == "q8b256" and cfg.group == 32 and not args.rotate:
            # the pages' default representation: head-wise groups, rotated keys
            specs["g128_rot"] = dict(common, group=128, flags=kv4.KV4_FLAG_ROTATE_K)
    keep = 32 if (args.populate_reps > 0 and not args.only_kv4) else 0
    caches, knew, vnew, first = build_caches(cfg, specs, H, W, kv4, dev, keep_first=keep)
    q = H.to_dev_bf16(W.queries(cfg, 0), str(dev))
    log(f"caches built in {time.time() - t0:.1f}s")

    # the headline first, after an untimed clock warm-up; then the comparators
    results = {}
    for name, c in caches.items():
        results[name] = time_step(c, cfg, n, knew, vnew, q, kv4, torch, tm, args.steps, args.warmup,
                                  clock_warm_s=0.3 if name == "kv4" else 0.0)
        r = results[name]
        log(f"{name}: append {r['append_ms'] * 1e3:.1f} us, partials {r['partials_ms'] * 1e3:.1f} us, "
            f"merge {r['merge_ms'] * 1e3:.1f} us, decode {r['decode_ms'] * 1e3:.1f} us "
            f"(median {r['decode_ms_median'] * 1e3:.1f}), waves {r['waves']}, pool chunks {r['pool_chunks']}")

    ratio8 = None
    if (not args.only_kv4 and not args.no_sub and cfg.name == "q8b256" and not args.rotate
            and not args.valu_decode):
        ratio8 = ratio8_record(caches["kv4"], cfg, n, knew, vnew, H, W, kv4, torch, tm, args, dev)
        log(f"ratio 8: decode {ratio8['decode_attn_us']} us, partials {ratio8['decode_partials_us']} us "
            f"({ratio8['partials_frac_hbm_peak']} of the HBM peak)")

    # bulk populate: the first 32 sequences' histories re-appended whole (after
    # every decode timing: it rewrites ring entries the step token owns)
    populate = prefill = None
    if first is not None:
        c = caches["kv4"]
        hist = np.array([k.shape[0] for k, _ in first])
        pcu = np.zeros(len(first) + 1, np.int32)
        pcu[1:] = np.cumsum(hist)
        pk = H.to_dev_bf16(np.concatenate([k for k, _ in first], 0), str(dev))
        pv = H.to_dev_bf16(np.concatenate([v for _, v in first], 0), str(dev))
        cu = torch.from_numpy(pcu).to(dev)
        slots = torch.from_numpy(c.slots_host[:len(first)].copy()).to(dev)
        T = int(hist.sum())
        populate = time_populate(c.cache.handle, slots, c.block_tables, hist, pk, pv, cu, cfg, kv4, torch,
                                 tm, args.populate_reps, stream)
        log(f"populate: {T} tokens in {populate['us']} us ({populate['gbs']} GB/s)")
        if args.prefill_reps > 0:
            # the same histories as prompts: causal BF16 attention (synthetic queries)
            prefill = time_prefill(c, hist, pk, pv, cu, cfg, kv4, torch, tm, args.prefill_reps)
            log(f"prefill: {T} tokens in {prefill['us']} us ({prefill['tflops']} TFLOP/s)")
        del pk, pv


    r = results["kv4"]
    db = decode_bytes_kv4(n, cfg)
    pb = partial_bytes_kv4(n, cfg)
    ab = append_bytes_kv4(n, cfg)
    step_ms = r["append_ms"] + r["decode_ms"]
    value = (db + ab) / (step_ms * 1e-3) / 1e9
    decode_gbs = db / (r["decode_ms"] * 1e-3) / 1e9
    achieved = pb / (r["partials_ms"] * 1e-3) / 1e9
    traffic = None
    # the stored counters are those of the default workload (unrotated, group 32)
    if (os.path.exists(args.traffic_json) and not args.rotate and not args.valu_decode and cfg.group == 32
            and cfg.name == "q8b256"):
        try:
            tj = json.load(open(args.traffic_json))
            if tj.get("kernel_source_hash") == _kernel_hash():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None
    line = {
        "metric": "decode-attn KV GB/s (% of HBM peak) and tokens/s vs BF16-KV, Qwen3-8B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded N(0,1) bf16 q/K/V, 4 outlier K channels x10)",
        "config": {
            "workload": (f"Qwen3-8B-shaped attention layer{TP_NOTE.get(cfg.name, '')}, "
                         f"batch {B} ragged decode step (lognormal contexts median 4k, max 16k), "
                         f"{cfg.q_heads}q/{cfg.kv_heads}kv heads, d=128, "
                         f"page 16, INT4 group {cfg.group}, S={cfg.sink}, R={cfg.recent}")
            if cfg.ctx_kind == "lognormal" else f"workload {cfg.name}",
            "global_batch": B, "seq_len_mean": float(n.mean()), "seq_len_max": int(n.max()),
            "tokens_in_context": int(n.sum()), "parallelism": "single GPU",
            "waves": r["waves"], "pool_chunks": r["pool_chunks"], "rotate_k": bool(args.rotate),
        },
        "decode_attn_gbs": round(decode_gbs, 2),
        "decode_attn_pct_hbm_peak": round(100 * decode_gbs / HBM_PEAK_GBS, 2),
        "decode_attn_us": round(r["decode_ms"] * 1e3, 2),
        "decode_partials_us": round(r["partials_ms"] * 1e3, 2),
        "decode_merge_us": round(r["merge_ms"] * 1e3, 2),
        "decode_attn_us_block_medians": [round(x * 1e3, 2) for x in r["decode_ms_block_medians"]],
        "decode_attn_median_over_mean": round(r["decode_ms_median"] / r["decode_ms"], 4),
        "decode_attn_us_median_p10_p90": [round(r["decode_ms_median"] * 1e3, 2),
                                          round(r["decode_ms_p10"] * 1e3, 2),
                                          round(r["decode_ms_p90"] * 1e3, 2)],
        "append_us": round(r["append_ms"] * 1e3, 2),
        "decode_alg_bytes": db,
        "partials_alg_bytes": pb,
        "append_alg_bytes": ab,
        "layer_tokens_per_s": round(B / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": ("decode_valu_kv4_kernel" if args.valu_decode else
                                                "decode_kv4_mfma_kernel") + " (kv4_decode_partials)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": pb,
                     "launch_us": round(r["partials_ms"] * 1e3, 2)},
    }
    if "bf16" in results:
        rb = results["bf16"]
        bstep = rb["append_ms"] + rb["decode_ms"]
        line["bf16_comparator"] = {
            "decode_attn_us": round(rb["decode_ms"] * 1e3, 2),
            "decode_partials_us": round(rb["partials_ms"] * 1e3, 2),
            "append_us": round(rb["append_ms"] * 1e3, 2),
            "decode_attn_gbs": round(decode_bytes_bf16(n, cfg) / (rb["decode_ms"] * 1e-3) / 1e9, 2),
            "layer_tokens_per_s": round(B / (bstep * 1e-3), 1),
        }
        line["speedup_vs_bf16_step"] = round(bstep / step_ms, 3)
        line["speedup_vs_bf16_decode"] = round(rb["decode_ms"] / r["decode_ms"], 3)
    if ratio8 is not None:
        line["ratio8"] = ratio8
    if populate is not None:
        line["populate"] = populate
    if prefill is not None:
        line["prefill"] = prefill
    if "valu" in results:
        rv = results["valu"]
        line["valu_comparator"] = {
            "kernel": "decode_valu_kv4_kernel<4> (KV4_FLAG_VALU_DECODE: the floating-point decode on the "
                      "vector ALU at GQA 4, same KV4 bytes)",
            "waves": rv["waves"],
            "decode_attn_us": round(rv["decode_ms"] * 1e3, 2),
            "decode_partials_us": round(rv["partials_ms"] * 1e3, 2),
            "partials_gbs": round(pb / (rv["partials_ms"] * 1e-3) / 1e9, 2),
            "partials_frac_hbm_peak": round(pb / (rv["partials_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "matrix_core_speedup": round(rv["partials_ms"] / r["partials_ms"], 3),
        }
    if "int" in results:
        ri = results["int"]
        line["int_path"] = {
            "kernel": "decode_int_mfma_kernel (KV4_FLAG_INT_PATH at GQA 4, same KV4 bytes)",
            "decode_attn_us": round(ri["decode_ms"] * 1e3, 2),
            "decode_partials_us": round(ri["partials_ms"] * 1e3, 2),
            "partials_gbs": round(pb / (ri["partials_ms"] * 1e-3) / 1e9, 2),
            "partials_frac_hbm_peak": round(pb / (ri["partials_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
    if "kv8" in results:
        r8 = results["kv8"]
        p8 = partial_bytes_kv8(n, cfg)
        line["kv8_comparator"] = {
            "decode_attn_us": round(r8["decode_ms"] * 1e3, 2),
            "decode_partials_us": round(r8["partials_ms"] * 1e3, 2),
            "append_us": round(r8["append_ms"] * 1e3, 2),
            "partials_alg_bytes": p8,
            "partials_gbs": round(p8 / (r8["partials_ms"] * 1e-3) / 1e9, 2),
            "partials_frac_hbm_peak": round(p8 / (r8["partials_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "layer_tokens_per_s": round(B / ((r8["append_ms"] + r8["decode_ms"]) * 1e-3), 1),
        }
        line["speedup_vs_kv8_decode"] = round(r8["decode_ms"] / r["decode_ms"], 3)
    if "g128_rot" in results:
        rg = results["g128_rot"]
        cg = W.scaled(cfg, group=128)
        pg, dg = partial_bytes_kv4(n, cg), decode_bytes_kv4(n, cg)
        line["g128_rot"] = {
            "workload": "the same batch, head-wise INT4 groups (G = 128, 136 B per token and kv head) "
                        "with keys in the rotated basis (KV4_FLAG_ROTATE_K): the pages' default",
            "decode_attn_us": round(rg["decode_ms"] * 1e3, 2),
            "decode_partials_us": round(rg["partials_ms"] * 1e3, 2),
            "partials_alg_bytes": pg,
            "partials_frac_hbm_peak": round(pg / (rg["partials_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_attn_frac_hbm_peak": round(dg / (rg["decode_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "append_us": round(rg["append_ms"] * 1e3, 2),
        }
        if "bf16" in results:
            line["g128_rot"]["speedup_vs_bf16_decode"] = round(results["bf16"]["decode_ms"] / rg["decode_ms"], 3)
    del caches, knew, vnew, q
    torch.cuda.empty_cache()

    if not args.only_kv4 and not args.no_sub and cfg.name == "q8b256":
        sub = {}
        sub["q4b"] = sub_record("q4b", W.CONFIGS["q4b"], dict(common), H, W, kv4, torch, dev, tm, args,
                                flush_bytes=1 << 30)
        sub["long"] = sub_record("long", W.CONFIGS["long"], dict(common), H, W, kv4, torch, dev, tm, args)
        line["sub_records"] = sub
        f36 = measure_full36(args, torch, kv4, H, W, cpu_seconds=5.0)
        sub["full36"] = {k: f36[k] for k in ("metric", "value", "unit", "ms_per_step", "config",
                                             "step_ms_median_p10_p90", "step_gbs", "step_frac_hbm_peak",
                                             "bf16_comparator", "speedup_vs_bf16_step", "cpu_baseline")
                         if k in f36}
        rc = read_ceiling(torch, dev, stream, pb)
        rc["decode_partials_frac_of_block_ceiling"] = round(achieved / rc["block2560_gbs"], 4)
        rc["decode_attn_frac_of_block_ceiling"] = round(decode_gbs / rc["block2560_gbs"], 4)
        line["read_ceiling"] = rc
        log(f"read ceiling: stream {rc['stream_gbs']} GB/s, random 2.5 KB blocks {rc['block2560_gbs']} GB/s")

    if not args.no_cpu_baseline and not args.only_kv4:
        line["cpu_baseline"] = cpu_baseline(cfg, ctx, n, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def time_prefill(c, hist, pk, pv, cu, cfg, kv4, torch, tm, reps):
    """kv4_prefill_attn over the histories `hist` packed as prompts (synthetic
    seeded queries), the mean of `reps` event-timed calls after one untimed."""
    dev = pk.device
    T = int(hist.sum())
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    qp = torch.randn((T, cfg.q_heads, cfg.head_dim), generator=gen, device=dev).to(torch.bfloat16)
    po = torch.empty((T, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    sm = 1.0 / math.sqrt(cfg.head_dim)

    def pre():
        kv4.kv4_prefill_attn(c.cache.handle, qp, pk, pv, cu, len(hist), int(hist.max()), sm, po,
                             kv4.KV4_OUT_F32, tm.stream)

    pre()
    torch.cuda.synchronize()
    fe = []
    for _ in range(reps):
        e0 = tm.ev(); pre(); e1 = tm.ev()
        fe.append((e0, e1))
    torch.cuda.synchronize()
    fms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in fe]))
    fl = prefill_flops(hist, cfg)
    return {"sequences": len(hist), "tokens": T, "max_prompt": int(hist.max()),
            "us": round(fms * 1e3, 2), "alg_flops": fl, "tflops": round(fl / (fms * 1e-3) / 1e12, 2),
            "frac_mfma_bf16_peak": round(fl / (fms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(T / (fms * 1e-3), 1)}


def time_populate(handle, slots, block_tables, hist, pk, pv, cu, cfg, kv4, torch, tm, reps, stream):
    """kv4_append of the histories `hist` (packed in pk, pv; offsets cu) into
    the slots `slots` from position 0: the mean (and median) of `reps`
    event-timed calls after 0.2 s of untimed ones."""
    dev = pk.device
    B = len(hist)
    T = int(hist.sum())
    ctx0 = torch.zeros(B, dtype=torch.int32, device=dev)

    def bulk():
        kv4.kv4_append(handle, 0, pk, pv, cu, ctx0, slots, block_tables, B, T, stream)

    # untimed calls for 0.2 s first, as before the headline's timing, so that
    # the timed calls start at full clocks
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        for _ in range(8):
            bulk()
        torch.cuda.synchronize()
    pe = []
    for _ in range(max(1, reps)):
        e0 = tm.ev(); bulk(); e1 = tm.ev()
        pe.append((e0, e1))
    torch.cuda.synchronize()
    pts = [e0.elapsed_time(e1) for e0, e1 in pe]
    pms = float(np.mean(pts))
    pbytes = populate_bytes_kv4(hist, cfg)
    return {"sequences": B, "tokens": T, "us": round(pms * 1e3, 2), "us_median": round(float(np.median(pts)) * 1e3, 2),
            "alg_bytes": pbytes, "gbs": round(pbytes / (pms * 1e-3) / 1e9, 2),
            "frac_hbm_peak": round(pbytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(T / (pms * 1e-3), 1)}


def run_populate_only(args, torch, kv4, H, W):
    """The bulk populate timing alone: the first 32 histories of the workload
    appended whole into a KV4 cache of the workload's shape (the same inputs
    as the default line's populate record)."""
    cfg = W.CONFIGS[args.config]
    ctx = W.contexts(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    tm = Timer(torch, stream)
    seqs = list(range(min(32, cfg.batch)))
    ks, vs = W.all_kv_sources(cfg, 0, ctx + 1, seqs=seqs, threads=16)
    hist = np.array([int(ctx[s]) for s in seqs])
    pk = H.to_dev_bf16(np.concatenate([ks[i][:hist[i]] for i in range(len(seqs))], 0), str(dev))
    pv = H.to_dev_bf16(np.concatenate([vs[i][:hist[i]] for i in range(len(seqs))], 0), str(dev))
    pcu = np.zeros(len(seqs) + 1, np.int32)
    pcu[1:] = np.cumsum(hist)
    cu = torch.from_numpy(pcu).to(dev)
    c = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, cfg.sink, cfg.recent, list(hist), device=str(dev))
    rec = time_populate(c.cache.handle, c.slots, c.block_tables, hist, pk, pv, cu, cfg, kv4, torch, tm,
                        args.populate_reps, stream)
    log(f"populate: {rec['tokens']} tokens in {rec['us']} us ({rec['gbs']} GB/s)")
    print(json.dumps({"populate": rec}), flush=True)


def run_prefill_only(args, torch, kv4, H, W):
    """The prefill timing alone: the first 32 histories of the workload as
    prompts (the same inputs as the default line's prefill record)."""
    cfg = W.CONFIGS[args.config]
    ctx = W.contexts(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tm = Timer(torch, torch.cuda.current_stream())
    seqs = list(range(min(32, cfg.batch)))
    ks, vs = W.all_kv_sources(cfg, 0, ctx + 1, seqs=seqs, threads=16)
    hist = np.array([int(ctx[s]) for s in seqs])
    pk = H.to_dev_bf16(np.concatenate([ks[i][:hist[i]] for i in range(len(seqs))], 0), str(dev))
    pv = H.to_dev_bf16(np.concatenate([vs[i][:hist[i]] for i in range(len(seqs))], 0), str(dev))
    pcu = np.zeros(len(seqs) + 1, np.int32)
    pcu[1:] = np.cumsum(hist)
    cu = torch.from_numpy(pcu).to(dev)
    c = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, cfg.sink, cfg.recent, [16], device=str(dev))
    rec = time_prefill(c, hist, pk, pv, cu, cfg, kv4, torch, tm, max(1, args.prefill_reps))
    log(f"prefill: {rec['tokens']} tokens in {rec['us']} us ({rec['tflops']} TFLOP/s)")
    print(json.dumps({"prefill": rec}), flush=True)


def run_full36(args, torch, kv4, H, W):
    line = measure_full36(args, torch, kv4, H, W, cpu_seconds=args.cpu_seconds)
    print(json.dumps(line), flush=True)


def measure_full36(args, torch, kv4, H, W, cpu_seconds):
    """The full decode step of a Qwen3-8B-shaped model, attention only: 36
    layers x (32 q / 8 kv heads), batch 128, contexts uniform 1k..12k, 64
    consecutive steps; every step appends one token per sequence and layer
    (crossing the recent window's demotion boundary) and decodes every layer.
    KV4 and the BF16 comparator are built one at a time (about 40 GB and
    126 GB resident).  tokens/s = batch / mean step time over the 64 steps
    (all timed: each step changes the caches, so none is repeated)."""
    cfg = W.CONFIGS["full36"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    tm = Timer(torch, stream)
    ctx = W.contexts(cfg)
    B, steps, Lyr, Hkv, d = cfg.batch, cfg.steps, cfg.layers, cfg.kv_heads, cfg.head_dim
    total = ctx + steps
    out_ch = W.outlier_channels(cfg)
    sm = 1.0 / math.sqrt(d)
    cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
    qs = torch.stack([torch.stack([W.queries_device(cfg, layer, st, dev) for st in range(steps)])
                      for layer in range(Lyr)])                  # [L, steps, B, Hq, d] bf16
    res = {}
    for name, kind in (("kv4", kv4.KV4_KIND_MIXED), ("bf16", kv4.KV4_KIND_BF16)):
        t0 = time.time()
        S, R = (cfg.sink, cfg.recent) if kind == kv4.KV4_KIND_MIXED else (0, 0)
        built = H.make_cache(cfg.q_heads, Hkv, cfg.group, S, R, total, layers=Lyr, kind=kind,
                             seed=cfg.seed, device="cuda:0")
        c = built.cache
        step_k = torch.empty((Lyr, steps, B, Hkv, d), dtype=torch.bfloat16, device=dev)
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
                kv4.kv4_append(c.handle, layer, torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), cu,
                               torch.zeros(len(seqs), dtype=torch.int32, device=dev),
                               built.slots[lo:lo + len(seqs)].contiguous(), built.block_tables,
                               len(seqs), int(cnt.sum()), stream)
            torch.cuda.synchronize()
        log(f"full36 {name}: {Lyr} layers built in {time.time() - t0:.1f}s")
        befores = [torch.from_numpy((ctx + st).astype(np.int32)).to(dev) for st in range(steps)]
        out = torch.empty((B, cfg.q_heads, d), dtype=torch.float32, device=dev)
        ws = c.workspace(B, int(total.max()))
        # untimed clock warm-up: decodes of layer 0 at the first step's lengths
        # (decoding does not change the cache)
        n0 = befores[0] + 1
        t_end = time.perf_counter() + 0.3
        while time.perf_counter() < t_end:
            for _ in range(8):
                kv4.kv4_decode_attn(c.handle, 0, qs[0, 0], n0, built.slots, built.block_tables, B,
                                    int(ctx.max()) + 1, sm, out, kv4.KV4_OUT_F32, ws, stream)
            torch.cuda.synchronize()
        evs = []
        for st in range(steps):
            n_d = befores[st] + 1
            max_ctx = int(ctx.max()) + st + 1
            e0 = tm.ev()
            for layer in range(Lyr):
                kv4.kv4_append(c.handle, layer, step_k[layer, st], step_v[layer, st], cu1, befores[st],
                               built.slots, built.block_tables, B, B, stream)
                kv4.kv4_decode_attn(c.handle, layer, qs[layer, st], n_d, built.slots, built.block_tables,
                                    B, max_ctx, sm, out, kv4.KV4_OUT_F32, ws, stream)
            evs.append((e0, tm.ev()))
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        t = np.array([a.elapsed_time(b) for a, b in evs])
        res[name] = dict(step_ms=float(t.mean()), step_ms_median=float(np.median(t)),
                         step_ms_p10=float(np.percentile(t, 10)), step_ms_p90=float(np.percentile(t, 90)))
        log(f"full36 {name}: step {t.mean():.3f} ms (median {np.median(t):.3f})")
        del built, c, step_k, step_v, ws, out
        torch.cuda.empty_cache()
    r, rb = res["kv4"], res["bf16"]
    # algorithmic bytes of a whole step: 36 layers of (append + decode) at the
    # mean length over the 64 steps
    nbar = ctx + (steps + 1) / 2.0
    per_layer = decode_bytes_kv4(np.round(nbar).astype(np.int64), cfg) + append_bytes_kv4(nbar, cfg)
    step_bytes = Lyr * per_layer
    line = {
        "metric": "36-layer attention-only decode tokens/s (KV4 vs BF16-KV), Qwen3-8B shape",
        "value": round(B / (r["step_ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": 0,
        "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded N(0,1) bf16 q/K/V drawn on the device, 4 outlier K channels x10)",
        "config": {"workload": "Qwen3-8B-shaped decode step, attention only: 36 layers x (32q/8kv heads, "
                               "d=128), batch 128, contexts uniform 1k..12k, page 16, group 32, S=4, R=128, "
                               "64 consecutive steps (append + decode per layer), each step timed",
                   "global_batch": B, "layers": Lyr, "seq_len_mean_first_step": float(ctx.mean() + 1),
                   "parallelism": "single GPU"},
        "step_ms_median_p10_p90": [round(r["step_ms_median"], 4), round(r["step_ms_p10"], 4),
                                   round(r["step_ms_p90"], 4)],
        "step_alg_bytes": int(step_bytes),
        "step_gbs": round(step_bytes / (r["step_ms"] * 1e-3) / 1e9, 1),
        "step_frac_hbm_peak": round(step_bytes / (r["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bf16_comparator": {"step_ms": round(rb["step_ms"], 4),
                            "tokens_per_s": round(B / (rb["step_ms"] * 1e-3), 1)},
        "speedup_vs_bf16_step": round(rb["step_ms"] / r["step_ms"], 3),
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(W.scaled(cfg, layers=1, steps=1), ctx, ctx + 1, cpu_seconds)
        # one layer-step of the sample, scaled to the whole batch, x 36 layers
        per_seq_layer = cb["seconds"] / cb["sequences"]
        cpu_step = per_seq_layer * B * Lyr
        line["cpu_baseline"] = {"value": round(B / cpu_step, 3), "unit": "tokens/s", "cores": cb["cores"],
                                "kind": "oracle",
                                "sample": cb["sample"] + f"; one layer-step of {cb['sequences']} sequences "
                                          f"scaled to {B} sequences x {Lyr} layers (x36 extrapolation)"}
    return line


def _kernel_hash(kernel=DOMINANT):
    """Hash of what a kernel's code is made from: the headers that define it
    and the compiler flags (so that an edit elsewhere in the library does not
    retire the kernel's counters)."""
    import hashlib
    from int8_mixed_precision_amd import build as hb
    csrc = os.path.join(ROOT, "int8_mixed_precision_amd", "csrc")
    parts = (["kv4_common.hpp", "kv4_decode.hpp", "kv4_decode_mfma.hpp"] if "decode" in kernel else
             ["kv4_common.hpp", "kv4_decode_mfma.hpp", "kv4_prefill.hpp"] if "prefill" in kernel else
             ["kv4_common.hpp", "kv4_append.hpp"] if "append" in kernel else
             [os.path.basename(f) for f in hb.sources() if f.startswith(csrc)])
    h = hashlib.sha256()
    for f in parts:
        h.update(open(os.path.join(csrc, f), "rb").read())
    h.update(" ".join(f for f in hb.HIPFLAGS if not os.path.isabs(f)).encode())   # not the include path
    return h.hexdigest()[:16]


def cpu_baseline(cfg, ctx, n, seconds):
    """The fp64 oracle's decode step (quantize the new token, attend over the
    dequantized cache) on a bounded sample of the same workload: the first
    sequences of the batch, as many as take about `seconds` of CPU time."""
    import oracle
    from int8_mixed_precision_amd import workloads as W

    q = W.queries(cfg, 0)

    def run(k):
        seqs = list(range(k))
        ks, vs = W.all_kv_sources(cfg, 0, n, seqs=seqs, threads=16)
        cache = oracle.MixedCache(ks, vs, cfg.group, protect=(cfg.sink, cfg.recent))
        newk = np.stack([x[-1] for x in ks])
        newv = np.stack([x[-1] for x in vs])
        t0 = time.perf_counter()
        # the step: quantize the new token into both representations ...
        oracle.quant_int4(newk, cfg.group)
        oracle.quant_int4(newv, cfg.group)
        oracle.quant_int8(newk)
        oracle.quant_int8(newv)
        # ... and attend over the whole context (history + new token)
        oracle.attend_mixed(q[seqs], cache, cfg.sink, cfg.recent, 1 / math.sqrt(cfg.head_dim))
        return time.perf_counter() - t0

    k = 2
    elapsed = run(k)
    k = int(min(cfg.batch, max(1, round(k * seconds / max(elapsed, 1e-3)))))
    elapsed = run(k)
    sub = n[:k]
    nb = decode_bytes_kv4(sub, cfg) + append_bytes_kv4(sub, cfg)
    return {"value": round(nb / elapsed / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {k} of {cfg.batch} sequences ({int(sub.sum())} context tokens), "
                      f"one decode step (quantize new token + fp64 attention), {elapsed:.1f} s",
            "seconds": round(elapsed, 2), "sequences": k}


if __name__ == "__main__":
    main()
