"""Host-side set-up of a paged KV4 cache on one device.

Assigns 16-token pages to sequences (shuffled, so the kernels' block-table
indirection is exercised), places sequences in request slots, creates the
library handle over torch-allocated pools, and appends token chunks through
kv4_append.  Used by the benchmark and the GPU tests; no kernel work happens
here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from int8_mixed_precision_amd import kv4

PAGE = 16


@dataclass
class Built:
    cache: kv4.Cache
    desc: kv4.kv4_cache_desc
    block_tables: torch.Tensor      # device int32 [max_slots, max_pages]
    bt_host: np.ndarray
    slots: torch.Tensor             # device int32 [B]
    slots_host: np.ndarray
    lengths: np.ndarray             # positions stored per sequence


def page_tables(lengths, max_pages, rng, num_pages=None, shuffle=True):
    """Assign distinct pages to each sequence (slot b = sequence b), shuffled."""
    need = [(int(n) + PAGE - 1) // PAGE for n in lengths]
    total = sum(need)
    num_pages = max(total, 1) if num_pages is None else num_pages
    ids = rng.permutation(num_pages)[:total] if shuffle else np.arange(total)
    bt = np.zeros((len(lengths), max_pages), dtype=np.int32)
    o = 0
    for b, k in enumerate(need):
        bt[b, :k] = ids[o:o + k]
        # unused entries point at random valid pages (never read)
        bt[b, k:] = rng.integers(0, num_pages, size=max_pages - k)
        o += k
    return bt, num_pages


def make_cache(Hq, Hkv, G, S, R, lengths, *, layers=1, kind=kv4.KV4_KIND_MIXED, waves=0,
               pool_chunks=0, flags=0, seed=0, max_pages=None, extra_pages=3, slot_perm=True, device="cuda"):
    rng = np.random.default_rng(seed + 1000)
    B = len(lengths)
    if max_pages is None:
        max_pages = max(1, (int(max(lengths)) + PAGE - 1) // PAGE)
    need = sum((int(n) + PAGE - 1) // PAGE for n in lengths)
    bt_seq, num_pages = page_tables(lengths, max_pages, rng, num_pages=need + extra_pages)
    max_slots = B + 2
    # sequence b lives in slot slots[b]
    slots = rng.permutation(max_slots)[:B].astype(np.int32) if slot_perm else np.arange(B, dtype=np.int32)
    bt = np.zeros((max_slots, max_pages), dtype=np.int32)
    bt[slots] = bt_seq
    desc = kv4.make_desc(layers, Hq, Hkv, 128, PAGE, G, S, R, num_pages, max_slots, max_pages,
                         kind, flags, waves, pool_chunks)
    cache = kv4.Cache(desc, device)
    dev = torch.device(device)
    return Built(cache, desc, torch.from_numpy(bt).to(dev), bt,
                 torch.from_numpy(slots).to(dev), slots, np.asarray(lengths, np.int64))


def to_dev_bf16(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(device)


def append_chunks(built: Built, layer: int, k_list, v_list, ctx_before, seqs=None,
                  device="cuda"):
    """Append k_list[i]/v_list[i] (float32 [new_i, Hkv, d]) to sequence seqs[i]
    at positions ctx_before[i].. in one kv4_append call."""
    seqs = list(range(len(k_list))) if seqs is None else list(seqs)
    counts = np.array([k.shape[0] for k in k_list], dtype=np.int64)
    cu = np.zeros(len(k_list) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(counts)
    k = to_dev_bf16(np.concatenate(k_list, 0), device)
    v = to_dev_bf16(np.concatenate(v_list, 0), device)
    dev = torch.device(device)
    built.cache.append(layer, k, v, torch.from_numpy(cu).to(dev),
                       torch.from_numpy(np.asarray(ctx_before, np.int32)).to(dev),
                       torch.from_numpy(built.slots_host[seqs]).to(dev), built.block_tables)
