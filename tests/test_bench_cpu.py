"""CPU checks of bench.py's host logic (no GPU): the one-GPU refusal, the
algorithmic byte models behind every roofline figure, and the HBM-traffic
summary of rocprofv3 counter files.

The byte models are checked against the pool layouts of include/kv4.h (as read
back by tests/layout.py) and against the region definition (sink S, recent R),
not against a retyped copy of their formulas.
"""
import argparse
import csv
import json
import os
import subprocess
import sys

import numpy as np

import bench
from int8_mixed_precision_amd import workloads as W
from tests import layout as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout


def test_region_counts_partition_every_context():
    for S, R in ((0, 0), (4, 128), (16, 3)):
        n = np.arange(0, 400)
        n4, n8 = bench.region_counts(n, S, R)
        assert np.array_equal(n4 + n8, n)
        # the protected positions: the first min(n, S) and the last R of the rest
        assert np.array_equal(n8, np.minimum(n, S) + np.minimum(np.maximum(n - S, 0), R))


def test_byte_models_follow_the_layouts():
    cfg = W.CONFIGS["q8b256"]
    d, G, Hkv = cfg.head_dim, cfg.group, cfg.kv_heads
    per4 = L.pb_bytes(d, G) // L.PAGE                 # INT4 bytes per (token, kv head)
    per8 = L.rb_bytes(d, 32) // 32                    # INT8 ring bytes per entry
    assert (per4, per8) == (160, 260)
    n = np.array([1, 4, 5, 132, 133, 1000, 5000])
    n4, n8 = bench.region_counts(n, cfg.sink, cfg.recent)
    q = len(n) * cfg.q_heads * d * 2
    bt = int(np.sum(np.ceil(n4 / L.PAGE))) * 4
    assert bench.partial_bytes_kv4(n, cfg) == Hkv * int(np.sum(per4 * n4 + per8 * n8)) + q + bt
    assert bench.decode_bytes_kv4(n, cfg) - bench.partial_bytes_kv4(n, cfg) == len(n) * cfg.q_heads * d * 4
    # KV8 pages: 16 tokens per 4,160-byte block; BF16 pages: 16 tokens per 8,192 bytes
    per_kv8 = L.pb_kv8_bytes(d) // L.PAGE
    bt_all = int(np.sum(np.ceil(n / L.PAGE))) * 4
    assert bench.partial_bytes_kv8(n, cfg) == Hkv * per_kv8 * int(n.sum()) + q + bt_all
    assert bench.decode_bytes_bf16(n, cfg) == (Hkv * (L.PAGE * d * 2 * 2 // L.PAGE) * int(n.sum())
                                               + len(n) * cfg.q_heads * d * 6 + bt_all)


def test_populate_and_append_bytes():
    cfg = W.CONFIGS["q8b256"]
    Hkv, d = cfg.kv_heads, cfg.head_dim
    src = 2 * d * 2                                  # bf16 K and V read per (token, kv head)
    # histories no longer than S + R: every position also gets its INT8 entry
    hist = np.array([3, 50, 132])
    assert bench.populate_bytes_kv4(hist, cfg) == int(hist.sum()) * Hkv * (src + 160 + 260)
    # longer histories: the INT8 entries of S + R positions each
    hist = np.array([1000, 5000])
    assert bench.populate_bytes_kv4(hist, cfg) == (int(hist.sum()) * Hkv * (src + 160)
                                                   + 2 * (cfg.sink + cfg.recent) * Hkv * 260)
    # a decode step appends one (protected) token per sequence
    n = np.array([10, 2000])
    assert bench.append_bytes_kv4(n, cfg) == len(n) * Hkv * (src + 160 + 260)


def _counter_dir(tmp_path, name, rows):
    d = tmp_path / name
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, kernel, counter, value in rows:
            w.writerow(dict(Dispatch_Id=disp, Kernel_Name=kernel, Counter_Name=counter, Counter_Value=value))
    return str(d)


def test_counter_summary_bytes_from_request_sizes(tmp_path):
    """Traffic from the L2's request counts by size, averaged over the dominant
    kernel's dispatches (other kernels ignored), and the factor FETCH_SIZE /
    WRITE_SIZE would need to match it."""
    dom = "void kv4::decode_kv4_mfma_kernel<32, false>(kv4::DecodeArgs)"
    other = "void kv4::merge_parts_kernel(kv4::DecodeArgs)"
    rd = _counter_dir(tmp_path, "r", [
        (1, dom, "TCC_EA0_RDREQ_32B", 10.0), (1, dom, "TCC_EA0_RDREQ_64B", 20.0),
        (1, dom, "TCC_EA0_RDREQ_128B", 1000.0), (1, other, "TCC_EA0_RDREQ_128B", 5e9),
        (2, dom, "TCC_EA0_RDREQ_32B", 12.0), (2, dom, "TCC_EA0_RDREQ_64B", 22.0),
        (2, dom, "TCC_EA0_RDREQ_128B", 1002.0)])
    fs = _counter_dir(tmp_path, "f", [(3, dom, "FETCH_SIZE", 64.0), (4, dom, "FETCH_SIZE", 64.0)])
    wr = _counter_dir(tmp_path, "w", [
        (5, dom, "TCC_EA0_WRREQ", 100.0), (5, dom, "TCC_EA0_WRREQ_64B", 60.0), (5, dom, "WRITE_SIZE", 4.0),
        (5, dom, "TCC_HIT", 30.0), (5, dom, "TCC_MISS", 90.0)])
    out = tmp_path / "c.json"
    args = argparse.Namespace(summarize_counters=[rd, fs, wr], summary_cmd="cmd", summary_out=str(out),
                              summary_kernel="decode_kv4_mfma_kernel")
    bench.summarize_counters(args)
    res = json.load(open(out))
    read = 32 * 11.0 + 64 * 21.0 + 128 * 1001.0
    write = 64 * 60.0 + 32 * 40.0
    assert res["read_bytes_per_launch"] == read and res["write_bytes_per_launch"] == write
    assert res["bytes_per_launch"] == round(read + write)
    assert abs(res["fetch_size_factor"] - read / (64.0 * 1024)) < 1e-12
    assert abs(res["write_size_factor"] - write / (4.0 * 1024)) < 1e-12
    assert abs(res["l2_hit_rate"] - 0.25) < 1e-12
    assert res["launches"]["TCC_EA0_RDREQ_128B"] == 2
    assert res["kernel_source_hash"] == bench._kernel_hash()


def test_counter_summary_last_dispatches(tmp_path):
    """--summary-last N keeps only the kernel's last N dispatches of each pass
    (the timed calls after the cache build's own launches of the kernel)."""
    k = "void kv4::append_kv4_kernel<32>(kv4::AppendArgs)"
    d = _counter_dir(tmp_path, "a", [(1, k, "SQ_INSTS_VALU", 1e9), (7, k, "SQ_INSTS_VALU", 10.0),
                                     (9, k, "SQ_INSTS_VALU", 30.0)])
    out = tmp_path / "a.json"
    args = argparse.Namespace(summarize_counters=[d], summary_cmd="cmd", summary_out=str(out),
                              summary_kernel="append_kv4_kernel", summary_last=2)
    bench.summarize_counters(args)
    res = json.load(open(out))
    assert res["counters_per_launch"]["SQ_INSTS_VALU"] == 20.0 and res["launches"]["SQ_INSTS_VALU"] == 2
    assert res["kernel_source_hash"] == bench._kernel_hash("append_kv4_kernel")
