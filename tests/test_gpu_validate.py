"""The validating build (libkv4_validate.so, compiled with KV4_VALIDATE; the
kinds are listed in include/kv4.h): on valid inputs it records nothing and its
outputs equal the product library's bit for bit, and each kind of bad device
value is reported.  Every bad value used here is one the kernels clamp into
range (tests/test_gpu_contract.py shows that no access then leaves the
buffers); the duplicate-write case makes two waves write the same bytes, which
is a race on the values but not an access fault."""
import math

import numpy as np
import pytest
import torch

from int8_mixed_precision_amd import kv4
from int8_mixed_precision_amd import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

HQ, HKV, S, R = 8, 2, 4, 16
CTX = [40, 17, 64, 5]                   # history lengths; the step token follows


@pytest.fixture
def vlib():
    prev = kv4._lib
    kv4._lib = kv4._load(kv4.VALIDATE_LIB_PATH)
    try:
        kv4.kv4_validate_report()       # start from an empty record
        yield kv4._lib
    finally:
        kv4._lib = prev


def _inputs(seed=700):
    n = np.asarray(CTX, np.int64) + 1
    cfg = W.scaled(W.CONFIGS["tiny"], q_heads=HQ, kv_heads=HKV, seed=seed, batch=len(CTX),
                   ctx_kind="fixed", ctx_fixed=tuple(CTX))
    ks, vs = W.all_kv_sources(cfg, 0, list(n))
    return cfg, n, ks, vs, W.queries(cfg, 0)


def _i32(x):
    return torch.tensor(x, dtype=torch.int32, device="cuda")


def _decode(built, q, n, slots=None, bt=None, max_ctx=None):
    B = len(n)
    max_ctx = int(max(CTX)) + 1 if max_ctx is None else max_ctx
    out = torch.empty((B, HQ, 128), dtype=torch.float32, device="cuda")
    kv4.kv4_decode_attn(built.cache.handle, 0, H.to_dev_bf16(q), _i32(list(n)),
                        built.slots if slots is None else slots,
                        built.block_tables if bt is None else bt, B, max_ctx, 1 / math.sqrt(128), out,
                        kv4.KV4_OUT_F32, built.cache.workspace(B, max_ctx))
    torch.cuda.synchronize()
    return out


def _report():
    torch.cuda.synchronize()
    return kv4.kv4_validate_report()


def test_valid_calls_record_nothing_and_match_the_product_library(vlib):
    cfg, n, ks, vs, q = _inputs()
    H.log("case validate: valid append, decode and prefill")
    built = H.make_cache(HQ, HKV, 32, S, R, n, seed=700)
    H.build_from_sources(built, 0, ks, vs, CTX)
    out_v = _decode(built, q, n)
    T = int(n.sum())
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    kp = H.to_dev_bf16(np.concatenate(ks), "cuda")
    vp = H.to_dev_bf16(np.concatenate(vs), "cuda")
    qp = torch.randn((T, HQ, 128), device="cuda").to(torch.bfloat16)
    pre_v = torch.empty((T, HQ, 128), dtype=torch.float32, device="cuda")
    kv4.kv4_prefill_attn(built.cache.handle, qp, kp, vp, _i32(list(cu)), len(n), int(n.max()),
                         1 / math.sqrt(128), pre_v)
    assert _report() == 0
    # the product library on the same pools and inputs
    P = kv4._load(kv4.LIB_PATH)
    saved, kv4._lib = kv4._lib, P
    try:
        h = kv4.kv4_cache_create(built.desc, built.cache.page_pool, built.cache.side_pool)
        try:
            B, max_ctx = len(n), int(n.max())
            out_p = torch.empty_like(out_v)
            ws = torch.empty(kv4.kv4_decode_workspace_bytes(h, B, max_ctx), dtype=torch.uint8, device="cuda")
            kv4.kv4_decode_attn(h, 0, H.to_dev_bf16(q), _i32(list(n)), built.slots, built.block_tables, B,
                                max_ctx, 1 / math.sqrt(128), out_p, kv4.KV4_OUT_F32, ws)
            pre_p = torch.empty_like(pre_v)
            kv4.kv4_prefill_attn(h, qp, kp, vp, _i32(list(cu)), len(n), int(n.max()), 1 / math.sqrt(128), pre_p)
            torch.cuda.synchronize()
        finally:
            kv4.kv4_cache_free(h)
    finally:
        kv4._lib = saved
    assert torch.equal(out_v, out_p) and torch.equal(pre_v, pre_p)


def test_decode_violations(vlib):
    cfg, n, ks, vs, q = _inputs()
    built = H.make_cache(HQ, HKV, 32, S, R, n, seed=701)
    H.build_from_sources(built, 0, ks, vs, CTX)
    assert _report() == 0
    max_ctx = int(n.max())
    H.log("case validate decode: length past max_ctx, zero length")
    _decode(built, q, [n[0], max_ctx + 1, n[2], n[3]], max_ctx=max_ctx)
    assert _report() == kv4.KV4_VIOLATION_SEQ_LEN
    _decode(built, q, [n[0], 0, n[2], n[3]], max_ctx=max_ctx)
    assert _report() == kv4.KV4_VIOLATION_SEQ_LEN
    H.log("case validate decode: slot id past max_slots")
    slots = built.slots_host.copy()
    slots[2] = built.desc.max_slots
    _decode(built, q, n, slots=_i32(list(slots)), max_ctx=max_ctx)
    assert _report() & kv4.KV4_VIOLATION_SLOT
    H.log("case validate decode: block-table entry past num_pages in a used page")
    bt = built.bt_host.copy()
    bt[built.slots_host[0], 1] = built.desc.num_pages
    _decode(built, q, n, bt=torch.from_numpy(bt).cuda(), max_ctx=max_ctx)
    assert _report() == kv4.KV4_VIOLATION_PAGE


def test_append_violations(vlib):
    cfg, n, ks, vs, q = _inputs()
    built = H.make_cache(HQ, HKV, 32, S, R, n, seed=702)
    H.build_from_sources(built, 0, ks, vs, CTX)
    assert _report() == 0
    B = len(n)
    k1 = H.to_dev_bf16(np.concatenate([k[-1:] for k in ks]), "cuda")
    v1 = H.to_dev_bf16(np.concatenate([v[-1:] for v in vs]), "cuda")

    def append(cu, ctx, slots=None, bt=None):
        kv4.kv4_append(built.cache.handle, 0, k1, v1, _i32(cu), _i32(ctx),
                       built.slots if slots is None else _i32(slots),
                       built.block_tables if bt is None else bt, B, B)
        return _report()

    H.log("case validate append: valid step, rows, positions, slot, page, duplicate")
    assert append([0, 1, 2, 3, 4], CTX) == 0
    assert append([0, 2, 1, 3, 4], CTX) == kv4.KV4_VIOLATION_ROWS        # decreasing
    assert append([0, 1, 2, 3, 3], CTX) == kv4.KV4_VIOLATION_ROWS        # does not end at total_new
    cap = built.desc.max_pages_per_seq * 16
    assert append([0, 1, 2, 3, 4], [CTX[0], -1, CTX[2], CTX[3]]) == kv4.KV4_VIOLATION_POSITION
    assert append([0, 1, 2, 3, 4], [CTX[0], CTX[1], cap, CTX[3]]) == kv4.KV4_VIOLATION_POSITION
    slots = built.slots_host.copy()
    slots[3] = -1
    assert append([0, 1, 2, 3, 4], CTX, slots=list(slots)) & kv4.KV4_VIOLATION_SLOT
    bt = built.bt_host.copy()
    bt[built.slots_host[1], CTX[1] // 16] = -1
    assert append([0, 1, 2, 3, 4], CTX, bt=torch.from_numpy(bt).cuda()) == kv4.KV4_VIOLATION_PAGE
    # two sequences of one append in the same slot: the same ring, the same pages
    slots = built.slots_host.copy()
    slots[1] = slots[0]
    assert append([0, 1, 2, 3, 4], [CTX[0], CTX[0], CTX[2], CTX[3]], slots=list(slots)) == \
        kv4.KV4_VIOLATION_DUPLICATE_WRITE


def test_prefill_violations(vlib):
    cfg, n, ks, vs, q = _inputs()
    built = H.make_cache(HQ, HKV, 32, S, R, n, seed=703)
    T = int(n.sum())
    kp = H.to_dev_bf16(np.concatenate(ks), "cuda")
    vp = H.to_dev_bf16(np.concatenate(vs), "cuda")
    qp = torch.randn((T, HQ, 128), device="cuda").to(torch.bfloat16)
    out = torch.empty((T, HQ, 128), dtype=torch.float32, device="cuda")
    cu = [0] + list(np.cumsum(n))
    H.log("case validate prefill: valid, offsets that end short of the total, a prompt past max_seqlen")
    kv4.kv4_prefill_attn(built.cache.handle, qp, kp, vp, _i32(cu), len(n), int(n.max()), 0.1, out)
    assert _report() == 0
    bad = list(cu)
    bad[-1] -= 1
    kv4.kv4_prefill_attn(built.cache.handle, qp, kp, vp, _i32(bad), len(n), int(n.max()), 0.1, out)
    assert _report() == kv4.KV4_VIOLATION_ROWS
    bad = [cu[0], cu[2], cu[1], cu[3], cu[4]]                 # decreasing at sequence 1
    kv4.kv4_prefill_attn(built.cache.handle, qp, kp, vp, _i32(bad), len(n), T, 0.1, out)
    assert _report() == kv4.KV4_VIOLATION_ROWS
    kv4.kv4_prefill_attn(built.cache.handle, qp, kp, vp, _i32(cu), len(n), int(n.max()) - 1, 0.1, out)
    assert _report() == kv4.KV4_VIOLATION_SEQ_LEN
