"""kv4_decode_attn_noalloc (the decode with its workspace in a static device
array, for callers that cannot allocate) against kv4_decode_attn with a
caller-provided workspace, through the C ABI: outputs bit-identical on two
calls in a row, the second with a smaller batch and shorter contexts (the
array keeps the first call's contents), for the floating-point path, the
integer path and the KV8 mode; a batch whose workspace exceeds the array is
rejected before anything is launched."""
import ctypes
import math

import numpy as np
import pytest
import torch

from int8_mixed_precision_amd import kv4
from int8_mixed_precision_amd import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _both(built, q, n, out_dtype):
    dev = torch.device("cuda")
    B = len(n)
    qd = H.to_dev_bf16(q)
    nd = torch.from_numpy(np.asarray(n, np.int32)).to(dev)
    max_ctx = int(max(n))
    sm = 1 / math.sqrt(128)
    dt = torch.float32 if out_dtype == kv4.KV4_OUT_F32 else torch.bfloat16
    ref = torch.empty((B, q.shape[1], 128), dtype=dt, device=dev)
    ws = torch.empty(kv4.kv4_decode_workspace_bytes(built.cache.handle, B, max_ctx), dtype=torch.uint8,
                     device=dev)
    kv4.kv4_decode_attn(built.cache.handle, 0, qd, nd, built.slots[:B], built.block_tables, B, max_ctx,
                        sm, ref, out_dtype, ws)
    got = torch.full((B, q.shape[1], 128), float("nan"), dtype=dt, device=dev)
    # straight through the C entry point (ctypes), as a caller without torch would
    L = kv4.lib()
    rc = L.kv4_decode_attn_noalloc(built.cache.handle, 0, ctypes.c_void_p(qd.data_ptr()),
                                   ctypes.c_void_p(nd.data_ptr()), ctypes.c_void_p(built.slots.data_ptr()),
                                   ctypes.c_void_p(built.block_tables.data_ptr()), B, max_ctx,
                                   ctypes.c_float(sm), ctypes.c_void_p(got.data_ptr()), out_dtype,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == kv4.KV4_OK, kv4.kv4_status_string(rc)
    torch.cuda.synchronize()
    return ref.float().cpu().numpy(), got.float().cpu().numpy()


@pytest.mark.parametrize("mode", ["fp", "int_path", "kv8"])
def test_noalloc_matches_workspace_entry_point(mode):
    Hq, Hkv, G, S, R = 32, 8, 32, 4, 64
    kind = kv4.KV4_KIND_KV8 if mode == "kv8" else kv4.KV4_KIND_MIXED
    flags = kv4.KV4_FLAG_INT_PATH if mode == "int_path" else 0
    if kind == kv4.KV4_KIND_KV8:
        S, R = 0, 0
    ctx = np.array([3000, 17, 700, 64, 1, 2500])
    n = ctx + 1
    H.log(f"case noalloc {mode}: ctx {list(ctx)}")
    cfg = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, group=G, sink=S, recent=R, seed=900,
                   batch=len(ctx), ctx_kind="fixed", ctx_fixed=tuple(int(c) for c in ctx))
    ks, vs = W.all_kv_sources(cfg, 0, n)
    built = H.make_cache(Hq, Hkv, G, S, R, n, kind=kind, flags=flags, seed=900)
    H.build_from_sources(built, 0, ks, vs, ctx)
    q = W.queries(cfg, 0)
    # first call: the whole batch
    ref, got = _both(built, q, n, kv4.KV4_OUT_F32)
    assert np.isfinite(ref).all()
    assert np.array_equal(ref, got)
    # second call: a smaller batch over shorter contexts (the first three
    # sequences, their lengths cut), bf16 output
    n2 = np.array([1200, 18, 300])
    ref2, got2 = _both(built, q[:3], n2, kv4.KV4_OUT_BF16)
    assert np.isfinite(ref2).all()
    assert np.array_equal(ref2, got2)
    H.log("  bit-identical to kv4_decode_attn on both calls")


def test_noalloc_rejects_batches_beyond_the_array():
    """A batch whose workspace exceeds KV4_NOALLOC_SCRATCH_BYTES is refused
    with KV4_ERR_CAPACITY before anything is launched."""
    Hq, Hkv = 32, 8
    B = 2000
    desc = kv4.make_desc(1, Hq, Hkv, 128, 16, 32, 4, 64, 4, B, 4)
    cache = kv4.Cache(desc, "cuda")
    need = kv4.kv4_decode_workspace_bytes(cache.handle, B, 64)
    assert need > kv4.KV4_NOALLOC_SCRATCH_BYTES
    L = kv4.lib()
    rc = L.kv4_decode_attn_noalloc(cache.handle, 0, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                   ctypes.c_void_p(16), ctypes.c_void_p(16), B, 64, ctypes.c_float(0.1),
                                   ctypes.c_void_p(16), kv4.KV4_OUT_F32, None)
    assert rc == kv4.KV4_ERR_CAPACITY
    cache.close()
