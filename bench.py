#!/usr/bin/env python3
"""Benchmark of the KV4 decode step on one MI355X.

A step is one pass of the hot path over one batch: kv4_append of the batch's
new token (INT4 pages + INT8 ring) followed by kv4_decode_attn (GQA attention
over the ragged paged contexts, cut by a balanced partition over the GPU's
waves, + the log-sum-exp merge).  The
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
    ap.add_argument("--steps", type=int, default=30)
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
    ap.add_argument("--populate-reps", type=int, default=5,
                    help="timed bulk appends of the first 32 sequences' histories (0 = skip)")
    ap.add_argument("--no-int-path", action="store_true",
                    help="skip the integer decode path (KV4_FLAG_INT_PATH) over the same KV4 bytes")
    ap.add_argument("--prefill-reps", type=int, default=3,
                    help="timed prefill attentions over the populate histories (0 = skip)")
    ap.add_argument("--rotate", action="store_true",
                    help="store keys in the rotated basis (KV4_FLAG_ROTATE_K) in the KV4 cache")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "decode_kv4_mfma_kernel_qwen3-8b_b256_traffic.json"))
    # summaries of rocprofv3 output (no GPU work): kernel durations from a
    # --kernel-trace csv directory; HBM traffic from a FETCH_SIZE and a
    # WRITE_SIZE --pmc csv directory of runs made with --copy-calibration
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summary-out", metavar="FILE")
    ap.add_argument("--summary-cmd", default="", help="command that produced the profile")
    ap.add_argument("--summary-bench", metavar="JSON",
                    help="bench line printed by the profiled run (live event timings)")
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
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


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
    if args.summary_bench:
        b = json.loads(open(args.summary_bench).read().strip().splitlines()[-1])
        lines += ["", "live HIP-event timings of the same run (mean over the timed steps):",
                  f"  kv4_decode_partials ({DOMINANT}): {b['decode_partials_us']} us",
                  f"  kv4_decode_merge (merge_parts_kernel, incl. launch gap): {b['decode_merge_us']} us",
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


def summarize_pmc(args):
    """HBM bytes per launch of the dominant kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for the
    1 GiB device-to-device copies that --copy-calibration issues."""
    out = {}
    for counter, d in zip(("FETCH_SIZE", "WRITE_SIZE"), args.summarize_pmc):
        rows = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        dom = [float(r["Counter_Value"]) for r in rows if DOMINANT in r["Kernel_Name"]]
        last_dom = max(int(r["Dispatch_Id"]) for r in rows if DOMINANT in r["Kernel_Name"])
        # the calibration copies are the device copies issued after every decode
        cal = [float(r["Counter_Value"]) for r in rows
               if r["Kernel_Name"].startswith(COPY_KERNEL) and int(r["Dispatch_Id"]) > last_dom]
        cal = [c for c in cal if cal and c >= 0.5 * max(cal)]     # the 1 GiB copies only
        if not dom or not cal:
            raise SystemExit(f"{counter}: {len(dom)} decode dispatches, {len(cal)} copy dispatches")
        scale = COPY_BYTES / (np.median(cal) * 1024.0)
        out[counter] = dict(kib_per_launch=float(np.mean(dom)), launches=len(dom),
                            kib_spread=[float(np.min(dom)), float(np.max(dom))],
                            copy_kib=float(np.median(cal)), copy_launches=len(cal), scale=scale,
                            bytes_per_launch=float(np.mean(dom)) * 1024.0 * scale)
    fetch, write = out["FETCH_SIZE"], out["WRITE_SIZE"]
    total = fetch["bytes_per_launch"] + write["bytes_per_launch"]
    res = dict(kernel=DOMINANT, kernel_source_hash=_kernel_hash(), command=args.summary_cmd,
               fetch=fetch, write=write, bytes_per_launch=int(round(total)))
    if args.summary_out:
        json.dump(res, open(args.summary_out, "w"), indent=1)
    print(json.dumps(res, indent=1))


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1 "
                                   "(the decode step shards by sequence or kv head with no "
                                   "exchange inside the op)"}))
        sys.exit(2)

    import torch
    from int8_mixed_precision_amd import kv4
    from int8_mixed_precision_amd import workloads as W
    from tests import gpu_harness as H

    cfg = W.CONFIGS[args.config]
    if args.group:
        cfg = W.scaled(cfg, group=args.group)
    ctx = W.contexts(cfg)
    n = ctx + 1
    B = cfg.batch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    log(f"config {cfg.name}: B={B} sum(n)={int(n.sum())} max n={int(n.max())}")

    kv4c = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, cfg.sink, cfg.recent, n,
                        seed=cfg.seed, waves=args.waves, pool_chunks=args.pool_chunks,
                        flags=kv4.KV4_FLAG_ROTATE_K if args.rotate else 0, device="cuda:0")
    caches = [("kv4", kv4c)]
    if not args.no_bf16:
        bfc = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, 0, 0, n, seed=cfg.seed,
                           kind=kv4.KV4_KIND_BF16, waves=args.waves,
                           pool_chunks=args.pool_chunks, device="cuda:0")
        caches.append(("bf16", bfc))
    if not args.no_int_path:
        ipc = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, cfg.sink, cfg.recent, n,
                           seed=cfg.seed, waves=args.waves, pool_chunks=args.pool_chunks,
                           flags=kv4.KV4_FLAG_INT_PATH | (kv4.KV4_FLAG_ROTATE_K if args.rotate else 0),
                           device="cuda:0")
        caches.append(("int", ipc))
    if not args.no_kv8:
        k8c = H.make_cache(cfg.q_heads, cfg.kv_heads, cfg.group, 0, 0, n, seed=cfg.seed,
                           kind=kv4.KV4_KIND_KV8, waves=args.waves,
                           pool_chunks=args.pool_chunks, device="cuda:0")
        caches.append(("kv8", k8c))
    # build every cache from the same sources, sequence chunk by chunk
    step_k, step_v = [], []
    pop = None
    for lo in range(0, B, 32):
        seqs = list(range(lo, min(B, lo + 32)))
        ks, vs = W.all_kv_sources(cfg, 0, n, seqs=seqs, threads=16)
        if lo == 0 and args.populate_reps > 0:
            # the first chunk's histories, kept on the device for the populate timing
            hist = np.array([int(ctx[s]) for s in seqs])
            pcu = np.zeros(len(seqs) + 1, np.int32)
            pcu[1:] = np.cumsum(hist)
            pop = dict(hist=hist,
                       k=H.to_dev_bf16(np.concatenate([ks[i][:hist[i]] for i in range(len(seqs))], 0), "cuda:0"),
                       v=H.to_dev_bf16(np.concatenate([vs[i][:hist[i]] for i in range(len(seqs))], 0), "cuda:0"),
                       cu=torch.from_numpy(pcu).to(dev),
                       ctx0=torch.zeros(len(seqs), dtype=torch.int32, device=dev),
                       slots=torch.from_numpy(kv4c.slots_host[seqs]).to(dev))
        for _, c in caches:
            H.append_chunks(c, 0, [ks[i][:int(ctx[s])] for i, s in enumerate(seqs)],
                            [vs[i][:int(ctx[s])] for i, s in enumerate(seqs)], [0] * len(seqs),
                            seqs, device="cuda:0")
        for i, s in enumerate(seqs):
            step_k.append(ks[i][int(ctx[s]):int(ctx[s]) + 1])
            step_v.append(vs[i][int(ctx[s]):int(ctx[s]) + 1])
        torch.cuda.synchronize()
        log(f"built sequences {seqs[0]}..{seqs[-1]}")
    knew = H.to_dev_bf16(np.concatenate(step_k, 0), "cuda:0")
    vnew = H.to_dev_bf16(np.concatenate(step_v, 0), "cuda:0")
    q = H.to_dev_bf16(W.queries(cfg, 0), "cuda:0")
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    ctx_d = torch.from_numpy(ctx.astype(np.int32)).to(dev)
    n_d = torch.from_numpy(n.astype(np.int32)).to(dev)
    max_ctx = int(n.max())
    sm = 1.0 / math.sqrt(cfg.head_dim)
    log(f"caches built in {time.time() - t0:.1f}s")

    # every launch goes to torch's current stream, which the events record on
    stream = torch.cuda.current_stream()
    results = {}
    for name, c in caches:
        out = torch.empty((B, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
        ws = c.cache.workspace(B, max_ctx)
        waves, chunks = kv4.kv4_decode_partition(c.cache.handle)

        def append():
            kv4.kv4_append(c.cache.handle, 0, knew, vnew, cu, ctx_d, c.slots, c.block_tables, B,
                           B, stream)

        def partials():
            kv4.kv4_decode_partials(c.cache.handle, 0, q, n_d, c.slots, c.block_tables, B,
                                    max_ctx, sm, ws, stream)

        def merge():
            kv4.kv4_decode_merge(c.cache.handle, n_d, B, max_ctx, out, kv4.KV4_OUT_F32, ws, stream)

        for _ in range(args.warmup):
            append()
            partials()
            merge()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            append()
            ev[i][1].record(stream)
            partials()
            ev[i][2].record(stream)
            merge()
            ev[i][3].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        t = np.array([[ev[i][k].elapsed_time(ev[i][k + 1]) for k in range(3)]
                      for i in range(args.steps)])
        ta, tp, tm = t[:, 0], t[:, 1], t[:, 2]
        td = tp + tm
        assert torch.isfinite(out).all()
        # the two phases are kv4_decode_attn exactly
        whole = torch.empty_like(out)
        kv4.kv4_decode_attn(c.cache.handle, 0, q, n_d, c.slots, c.block_tables, B, max_ctx, sm,
                            whole, kv4.KV4_OUT_F32, ws, stream)
        torch.cuda.synchronize()
        assert torch.equal(whole, out), "kv4_decode_attn differs from partials + merge"
        results[name] = dict(append_ms=float(ta.mean()), partials_ms=float(tp.mean()),
                             merge_ms=float(tm.mean()), decode_ms=float(td.mean()),
                             decode_ms_median=float(np.median(td)),
                             decode_ms_p10=float(np.percentile(td, 10)),
                             decode_ms_p90=float(np.percentile(td, 90)),
                             wall_ms_per_step=wall * 1e3 / args.steps,
                             waves=waves, pool_chunks=chunks)
        log(f"{name}: append {ta.mean() * 1e3:.1f} us, partials {tp.mean() * 1e3:.1f} us, "
            f"merge {tm.mean() * 1e3:.1f} us, decode {td.mean() * 1e3:.1f} us "
            f"(median {np.median(td) * 1e3:.1f}), waves {waves}, pool chunks {chunks}")

    # bulk populate: the first 32 sequences' histories re-appended whole (after
    # every decode timing: it rewrites ring entries the step token owns)
    populate = prefill = None
    if pop is not None:
        c = kv4c
        T = int(pop["hist"].sum())

        def bulk():
            kv4.kv4_append(c.cache.handle, 0, pop["k"], pop["v"], pop["cu"], pop["ctx0"],
                           pop["slots"], c.block_tables, len(pop["hist"]), T, stream)

        bulk()
        torch.cuda.synchronize()
        pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.populate_reps)]
        for e0, e1 in pe:
            e0.record(stream)
            bulk()
            e1.record(stream)
        torch.cuda.synchronize()
        pms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in pe]))
        pbytes = populate_bytes_kv4(pop["hist"], cfg)
        populate = {"sequences": len(pop["hist"]), "tokens": T, "us": round(pms * 1e3, 2),
                    "alg_bytes": pbytes, "gbs": round(pbytes / (pms * 1e-3) / 1e9, 2),
                    "frac_hbm_peak": round(pbytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "tokens_per_s": round(T / (pms * 1e-3), 1)}
        log(f"populate: {T} tokens in {pms * 1e3:.1f} us ({populate['gbs']} GB/s)")
        if args.prefill_reps > 0:
            # the same histories as prompts: causal BF16 attention (synthetic queries)
            gen = torch.Generator(device=dev)
            gen.manual_seed(cfg.seed)
            qp = torch.randn((T, cfg.q_heads, cfg.head_dim), generator=gen, device=dev).to(torch.bfloat16)
            po = torch.empty((T, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device=dev)

            def pre():
                kv4.kv4_prefill_attn(c.cache.handle, qp, pop["k"], pop["v"], pop["cu"],
                                     len(pop["hist"]), int(pop["hist"].max()), sm, po, kv4.KV4_OUT_F32,
                                     stream)

            pre()
            torch.cuda.synchronize()
            fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.prefill_reps)]
            for e0, e1 in fe:
                e0.record(stream)
                pre()
                e1.record(stream)
            torch.cuda.synchronize()
            fms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in fe]))
            fl = prefill_flops(pop["hist"], cfg)
            prefill = {"sequences": len(pop["hist"]), "tokens": T, "us": round(fms * 1e3, 2),
                       "alg_flops": fl, "tflops": round(fl / (fms * 1e-3) / 1e12, 2),
                       "frac_mfma_bf16_peak": round(fl / (fms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                       "tokens_per_s": round(T / (fms * 1e-3), 1)}
            log(f"prefill: {T} tokens in {fms * 1e3:.1f} us ({prefill['tflops']} TFLOP/s)")
            del qp, po
        del pop

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies")

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
    if (os.path.exists(args.traffic_json) and not args.rotate and cfg.group == 32
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
        "decode_attn_us_median_p10_p90": [round(r["decode_ms_median"] * 1e3, 2),
                                          round(r["decode_ms_p10"] * 1e3, 2),
                                          round(r["decode_ms_p90"] * 1e3, 2)],
        "append_us": round(r["append_ms"] * 1e3, 2),
        "decode_alg_bytes": db,
        "partials_alg_bytes": pb,
        "append_alg_bytes": ab,
        "layer_tokens_per_s": round(B / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "decode_kv4_mfma_kernel (kv4_decode_partials)",
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

    if populate is not None:
        line["populate"] = populate
    if prefill is not None:
        line["prefill"] = prefill
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

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, ctx, n, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def _kernel_hash():
    import hashlib
    from int8_mixed_precision_amd import build as hb
    h = hashlib.sha256()
    for f in hb.sources():
        h.update(open(f, "rb").read())
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
            "seconds": round(elapsed, 2)}


if __name__ == "__main__":
    main()
