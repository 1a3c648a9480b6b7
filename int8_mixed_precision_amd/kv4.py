"""Python binding of the KV4 C ABI (include/kv4.h), argument marshalling only.

Every function here has the name of the C entry point it calls and passes
torch tensors through as raw device pointers; all the work happens in the HIP
kernels of ``libkv4.so``.  torch supplies device memory and the stream.  If
the library has not been built, importing this module raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KV4_LIB selects another build of the library (for example the host-side
# sanitizer build of tests/sanitize_cpu.py)
LIB_PATH = os.environ.get("KV4_LIB") or os.path.join(_HERE, "libkv4.so")
# the validating build (KV4_VALIDATE device-side checks; include/kv4.h)
VALIDATE_LIB_PATH = os.path.join(_HERE, "libkv4_validate.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "kv4.h")

KV4_OK = 0
KV4_ERR_INVALID_ARG = 1
KV4_ERR_UNSUPPORTED = 2
KV4_ERR_CAPACITY = 3
KV4_ERR_WORKSPACE = 4
KV4_ERR_HIP = 5
KV4_KIND_MIXED = 0
KV4_KIND_BF16 = 1
KV4_KIND_KV8 = 2
KV4_FLAG_ROTATE_K = 0x1
KV4_FLAG_INT_PATH = 0x2
KV4_FLAG_VALU_DECODE = 0x4
KV4_OUT_F32 = 0
KV4_OUT_BF16 = 1
KV4_VIOLATION_SEQ_LEN = 0x01
KV4_VIOLATION_SLOT = 0x02
KV4_VIOLATION_PAGE = 0x04
KV4_VIOLATION_ROWS = 0x08
KV4_VIOLATION_POSITION = 0x10
KV4_VIOLATION_DUPLICATE_WRITE = 0x20


class kv4_cache_desc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_layers", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "group_size",
        "sink", "recent", "num_pages", "max_slots", "max_pages_per_seq", "kind", "flags",
        "num_waves", "pool_chunks")]


class KV4Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {kv4_status_string(code)} (code {code})")


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m int8_mixed_precision_amd.build`")
    L = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    pdesc = ctypes.POINTER(kv4_cache_desc)
    psz = ctypes.POINTER(sz)
    pi32 = ctypes.POINTER(ctypes.c_int)
    L.kv4_cache_required_bytes.argtypes = [pdesc, psz, psz, psz]
    L.kv4_cache_create.argtypes = [pdesc, P, sz, P, sz, ctypes.POINTER(P)]
    L.kv4_append.argtypes = [P, i32, P, P, P, P, P, P, i32, i32, P]
    L.kv4_decode_workspace_bytes.argtypes = [P, i32, i32, psz]
    L.kv4_decode_attn.argtypes = [P, i32, P, P, P, P, i32, i32, ctypes.c_float, P, i32, P, sz, P]
    L.kv4_decode_partials.argtypes = [P, i32, P, P, P, P, i32, i32, ctypes.c_float, P, sz, P]
    L.kv4_decode_merge.argtypes = [P, P, i32, i32, P, i32, P, sz, P]
    L.kv4_decode_attn_noalloc.argtypes = [P, i32, P, P, P, P, i32, i32, ctypes.c_float, P, i32, P]
    L.kv4_cache_free.argtypes = [P]
    L.kv4_status_string.argtypes = [i32]
    L.kv4_status_string.restype = ctypes.c_char_p
    L.kv4_decode_partition.argtypes = [P, pi32, pi32]
    L.kv4_prefill_attn.argtypes = [P, P, P, P, P, i32, i32, i32, ctypes.c_float, P, i32, P]
    L.kv4_validate_report.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    for f in ("kv4_cache_required_bytes", "kv4_cache_create", "kv4_append",
              "kv4_decode_workspace_bytes", "kv4_decode_attn", "kv4_decode_partials",
              "kv4_decode_merge", "kv4_cache_free", "kv4_decode_partition", "kv4_prefill_attn",
              "kv4_decode_attn_noalloc", "kv4_validate_report"):
        getattr(L, f).restype = i32
    return L


_lib = _load()


def lib():
    return _lib


def declared_functions():
    """Names of the functions include/kv4.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(kv4_\w+)\s*\(", text, flags=re.M)))


def _check(code: int, where: str):
    if code != KV4_OK:
        raise KV4Error(code, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def make_desc(num_layers, num_q_heads, num_kv_heads, head_dim=128, page_size=16, group_size=32,
              sink=4, recent=128, num_pages=1, max_slots=1, max_pages_per_seq=1,
              kind=KV4_KIND_MIXED, flags=0, num_waves=0, pool_chunks=0) -> kv4_cache_desc:
    return kv4_cache_desc(num_layers, num_q_heads, num_kv_heads, head_dim, page_size, group_size,
                          sink, recent, num_pages, max_slots, max_pages_per_seq, kind, flags,
                          num_waves, pool_chunks)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def kv4_status_string(code: int) -> str:
    return _lib.kv4_status_string(int(code)).decode()


def kv4_cache_required_bytes(desc: kv4_cache_desc) -> Tuple[int, int, int]:
    """(page_pool_bytes, side_pool_bytes, page_bytes_per_layer)."""
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.kv4_cache_required_bytes(ctypes.byref(desc), ctypes.byref(a), ctypes.byref(b),
                                         ctypes.byref(c)), "kv4_cache_required_bytes")
    return a.value, b.value, c.value


def kv4_cache_create(desc: kv4_cache_desc, page_pool: torch.Tensor,
                     side_pool: Optional[torch.Tensor]) -> ctypes.c_void_p:
    _need(page_pool, "page_pool", torch.uint8)
    if side_pool is not None:
        _need(side_pool, "side_pool", torch.uint8)
    h = ctypes.c_void_p()
    _check(_lib.kv4_cache_create(ctypes.byref(desc), _ptr(page_pool), page_pool.numel(),
                                 _ptr(side_pool), 0 if side_pool is None else side_pool.numel(),
                                 ctypes.byref(h)), "kv4_cache_create")
    return h


def kv4_append(cache, layer: int, k: torch.Tensor, v: torch.Tensor, cu_new: torch.Tensor,
               ctx_before: torch.Tensor, slot_ids: torch.Tensor, block_tables: torch.Tensor,
               batch: int, total_new: int, stream=None) -> None:
    dev = k.device
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    for name, t in (("cu_new", cu_new), ("ctx_before", ctx_before), ("slot_ids", slot_ids),
                    ("block_tables", block_tables)):
        _need(t, name, torch.int32, dev)
    if k.shape != v.shape or k.dim() != 3 or k.shape[0] != total_new:
        raise ValueError("k and v must be [total_new, Hkv, d] of the same shape")
    if cu_new.numel() != batch + 1 or ctx_before.numel() < batch or slot_ids.numel() < batch:
        raise ValueError("cu_new must have batch+1 entries; ctx_before and slot_ids batch entries")
    _check(_lib.kv4_append(cache, int(layer), _ptr(k), _ptr(v), _ptr(cu_new), _ptr(ctx_before),
                           _ptr(slot_ids), _ptr(block_tables), int(batch), int(total_new),
                           _stream(stream)), "kv4_append")


def kv4_decode_workspace_bytes(cache, batch: int, max_ctx: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.kv4_decode_workspace_bytes(cache, int(batch), int(max_ctx), ctypes.byref(n)),
           "kv4_decode_workspace_bytes")
    return n.value


def kv4_decode_partition(cache) -> tuple:
    """(W, C): waves of the decode partition and most chunks of its pool."""
    w, c = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.kv4_decode_partition(cache, ctypes.byref(w), ctypes.byref(c)), "kv4_decode_partition")
    return w.value, c.value


def kv4_decode_attn(cache, layer: int, q: torch.Tensor, seq_lens: torch.Tensor,
                    slot_ids: torch.Tensor, block_tables: torch.Tensor, batch: int, max_ctx: int,
                    sm_scale: float, out: torch.Tensor, out_dtype: int, workspace: torch.Tensor,
                    stream=None) -> None:
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    for name, t in (("seq_lens", seq_lens), ("slot_ids", slot_ids), ("block_tables", block_tables)):
        _need(t, name, torch.int32, dev)
    _need(out, "out", torch.float32 if out_dtype == KV4_OUT_F32 else torch.bfloat16, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if q.dim() != 3 or q.shape[0] < batch or out.shape != q.shape:
        raise ValueError("q and out must be [batch, Hq, d]")
    _check(_lib.kv4_decode_attn(cache, int(layer), _ptr(q), _ptr(seq_lens), _ptr(slot_ids),
                                _ptr(block_tables), int(batch), int(max_ctx), float(sm_scale),
                                _ptr(out), int(out_dtype), _ptr(workspace), workspace.numel(),
                                _stream(stream)), "kv4_decode_attn")


KV4_NOALLOC_SCRATCH_BYTES = 32 << 20


def kv4_decode_attn_noalloc(cache, layer: int, q: torch.Tensor, seq_lens: torch.Tensor,
                            slot_ids: torch.Tensor, block_tables: torch.Tensor, batch: int,
                            max_ctx: int, sm_scale: float, out: torch.Tensor, out_dtype: int,
                            stream=None) -> None:
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    for name, t in (("seq_lens", seq_lens), ("slot_ids", slot_ids), ("block_tables", block_tables)):
        _need(t, name, torch.int32, dev)
    _need(out, "out", torch.float32 if out_dtype == KV4_OUT_F32 else torch.bfloat16, dev)
    if q.dim() != 3 or q.shape[0] < batch or out.shape != q.shape:
        raise ValueError("q and out must be [batch, Hq, d]")
    _check(_lib.kv4_decode_attn_noalloc(cache, int(layer), _ptr(q), _ptr(seq_lens), _ptr(slot_ids),
                                        _ptr(block_tables), int(batch), int(max_ctx),
                                        float(sm_scale), _ptr(out), int(out_dtype),
                                        _stream(stream)), "kv4_decode_attn_noalloc")


def kv4_prefill_attn(cache, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     cu_seqlens: torch.Tensor, batch: int, max_seqlen: int, sm_scale: float,
                     out: torch.Tensor, out_dtype: int = KV4_OUT_F32, stream=None) -> None:
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(out, "out", torch.float32 if out_dtype == KV4_OUT_F32 else torch.bfloat16, dev)
    if q.dim() != 3 or k.shape != v.shape or k.shape[0] != q.shape[0] or out.shape != q.shape:
        raise ValueError("q, out [total, Hq, d]; k, v [total, Hkv, d]")
    if cu_seqlens.numel() != batch + 1:
        raise ValueError("cu_seqlens must have batch + 1 entries")
    _check(_lib.kv4_prefill_attn(cache, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), int(batch),
                                 int(q.shape[0]), int(max_seqlen), float(sm_scale), _ptr(out),
                                 int(out_dtype), _stream(stream)), "kv4_prefill_attn")


def kv4_decode_partials(cache, layer: int, q: torch.Tensor, seq_lens: torch.Tensor,
                        slot_ids: torch.Tensor, block_tables: torch.Tensor, batch: int,
                        max_ctx: int, sm_scale: float, workspace: torch.Tensor,
                        stream=None) -> None:
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    for name, t in (("seq_lens", seq_lens), ("slot_ids", slot_ids), ("block_tables", block_tables)):
        _need(t, name, torch.int32, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if q.dim() != 3 or q.shape[0] < batch:
        raise ValueError("q must be [batch, Hq, d]")
    _check(_lib.kv4_decode_partials(cache, int(layer), _ptr(q), _ptr(seq_lens), _ptr(slot_ids),
                                    _ptr(block_tables), int(batch), int(max_ctx), float(sm_scale),
                                    _ptr(workspace), workspace.numel(), _stream(stream)),
           "kv4_decode_partials")


def kv4_decode_merge(cache, seq_lens: torch.Tensor, batch: int, max_ctx: int, out: torch.Tensor,
                     out_dtype: int, workspace: torch.Tensor, stream=None) -> None:
    dev = out.device
    _need(seq_lens, "seq_lens", torch.int32, dev)
    _need(out, "out", torch.float32 if out_dtype == KV4_OUT_F32 else torch.bfloat16, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if out.dim() != 3 or out.shape[0] < batch:
        raise ValueError("out must be [batch, Hq, d]")
    _check(_lib.kv4_decode_merge(cache, _ptr(seq_lens), int(batch), int(max_ctx), _ptr(out),
                                 int(out_dtype), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "kv4_decode_merge")


def kv4_validate_report(library=None) -> int:
    """The violation kinds the validating build recorded on the current device
    since the last report (and clears them); raises KV4Error with
    KV4_ERR_UNSUPPORTED on a library built without KV4_VALIDATE."""
    L = library if library is not None else _lib
    v = ctypes.c_uint32(0)
    _check(L.kv4_validate_report(ctypes.byref(v)), "kv4_validate_report")
    return int(v.value)


def kv4_cache_free(cache) -> None:
    _check(_lib.kv4_cache_free(cache), "kv4_cache_free")


# ---------------------------------------------------------------------------
# convenience owner of pools + handle
# ---------------------------------------------------------------------------

class Cache:
    """Pools (torch uint8 on ``device``) plus a library handle."""

    def __init__(self, desc: kv4_cache_desc, device="cuda"):
        self.desc = desc
        self.device = torch.device(device)
        pb, sb, self.page_bytes_per_layer = kv4_cache_required_bytes(desc)
        self.page_pool = torch.empty(pb, dtype=torch.uint8, device=self.device)
        self.side_pool = torch.empty(sb, dtype=torch.uint8, device=self.device) if sb else None
        self.handle = kv4_cache_create(desc, self.page_pool, self.side_pool)
        self._ws = None

    def close(self):
        if self.handle is not None:
            kv4_cache_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, batch: int, max_ctx: int) -> torch.Tensor:
        n = kv4_decode_workspace_bytes(self.handle, batch, max_ctx)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(max(n, 16), dtype=torch.uint8, device=self.device)
        return self._ws

    def append(self, layer, k, v, cu_new, ctx_before, slot_ids, block_tables, stream=None):
        batch = cu_new.numel() - 1
        kv4_append(self.handle, layer, k, v, cu_new, ctx_before, slot_ids, block_tables, batch,
                   k.shape[0], stream)

    def decode(self, layer, q, seq_lens, slot_ids, block_tables, max_ctx, sm_scale=None,
               out=None, out_dtype=KV4_OUT_F32, stream=None):
        batch = q.shape[0]
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(q.shape[-1])
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32 if out_dtype == KV4_OUT_F32
                              else torch.bfloat16, device=q.device)
        ws = self.workspace(batch, max_ctx)
        kv4_decode_attn(self.handle, layer, q, seq_lens, slot_ids, block_tables, batch, max_ctx,
                        sm_scale, out, out_dtype, ws, stream)
        return out
