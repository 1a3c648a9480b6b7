"""Read the library's pools back into per-position arrays (test code only).

Written from the pool layout stated in include/kv4.h, independently of the
kernels, so that the GPU's bytes can be compared with the oracle's codes.
"""
from __future__ import annotations

import numpy as np

PAGE = 16


def pb_bytes(d: int, G: int) -> int:
    ng = d // G
    return PAGE * d // 2 + PAGE * d // 2 + 4 * 2 * PAGE * ng


def sr32(SR: int) -> int:
    """Ring entries, padded to a multiple of 32."""
    return -(-SR // 32) * 32


def rb_bytes(d: int, SR: int) -> int:
    return 0 if SR == 0 else sr32(SR) * (2 * d + 4)


def ring_vbyte(e, c, d: int = 128):
    """Byte of channel c of ring entry e in the V code region: blocks of 8
    entries, channel-major, channels ordered c % 16 then c // 16."""
    e = np.asarray(e, np.int64)
    c = np.asarray(c, np.int64)
    return (e // 8) * (8 * d) + ((c % 16) * 8 + c // 16) * 8 + e % 8


def ring_entry(p: np.ndarray, S: int, R: int) -> np.ndarray:
    p = np.asarray(p, dtype=np.int64)
    return np.where(p < S, p, S + ((p - S) % R if R > 0 else 0))


def gather_mixed(pages: np.ndarray, side, *, layer, num_pages, Hkv, d, G, S, R, max_slots,
                 block_tables: np.ndarray, slot: int, n: int, protected_mask=None):
    """Codes and metadata of positions [0, n) of the sequence in `slot`.

    Returns a dict with k4, v4 (uint8 [n, Hkv, d]), k4d, k4m, v4d, v4m
    (uint16 [n, Hkv, d/G]); and, for the positions where protected_mask is
    true, k8, v8 (int8 [n, Hkv, d]) and k8s, v8s (uint16 [n, Hkv]) -- other
    rows of those arrays are zero.
    """
    ng = d // G
    PB = pb_bytes(d, G)
    p = np.arange(n, dtype=np.int64)
    page = block_tables[slot, p // PAGE].astype(np.int64)
    tp = p % PAGE
    h = np.arange(Hkv, dtype=np.int64)
    base = ((layer * num_pages + page[:, None]) * Hkv + h[None, :]) * PB          # [n, Hkv]
    # K codes: token-major bytes, channel 2i low nibble, 2i+1 high nibble
    # natural byte i (channels 2i, 2i+1) of word i/4 sits in word 4 (w % 4) + w / 4 of the row
    i = np.arange(d // 2)
    kbyte = 4 * (4 * ((i // 4) % 4) + (i // 4) // 4) + i % 4
    kb = pages[base[:, :, None] + (tp[:, None, None] * (d // 2)) + kbyte[None, None, :]]
    k4 = np.empty((n, Hkv, d), dtype=np.uint8)
    k4[:, :, 0::2] = kb & 0xF
    k4[:, :, 1::2] = kb >> 4
    # V codes: half h's word for channel c at index 64(c/64) + 4(c%16) + 2((c/32)%2) + (c/16)%2,
    # token 8h+e in bits 4e..4e+3
    voff = PAGE * d // 2
    c = np.arange(d)
    vpos = 64 * (c // 64) + 4 * (c % 16) + 2 * ((c // 32) % 2) + (c // 16) % 2
    widx = base[:, :, None] + voff + 4 * ((tp[:, None, None] // 8) * d + vpos[None, None, :])
    words = (pages[widx].astype(np.uint32) | (pages[widx + 1].astype(np.uint32) << 8) |
             (pages[widx + 2].astype(np.uint32) << 16) | (pages[widx + 3].astype(np.uint32) << 24))
    v4 = ((words >> (4 * (tp[:, None, None] % 8)).astype(np.uint32)) & 0xF).astype(np.uint8)

    def u16(idx):
        return pages[idx].astype(np.uint16) | (pages[idx + 1].astype(np.uint16) << 8)

    grp = np.arange(ng)[None, None, :]
    off_kdm = PAGE * d                      # K (Delta, m) token-major: [token][group][2]
    off_vm = off_kdm + 4 * PAGE * ng        # V m token-major: [token][group]
    off_vd = off_vm + 2 * PAGE * ng         # V Delta group-major: [group][token]
    kdm = base[:, :, None] + off_kdm + tp[:, None, None] * 4 * ng + 4 * grp
    out = dict(k4=k4, v4=v4, k4d=u16(kdm), k4m=u16(kdm + 2),
               v4d=u16(base[:, :, None] + off_vd + 2 * (grp * PAGE + tp[:, None, None])),
               v4m=u16(base[:, :, None] + off_vm + tp[:, None, None] * 2 * ng + 2 * grp))
    SR = S + R
    k8 = np.zeros((n, Hkv, d), np.int8)
    v8 = np.zeros((n, Hkv, d), np.int8)
    k8s = np.zeros((n, Hkv), np.uint16)
    v8s = np.zeros((n, Hkv), np.uint16)
    if SR > 0 and protected_mask is not None and np.any(protected_mask):
        RB = rb_bytes(d, SR)
        pp = p[protected_mask]
        e = ring_entry(pp, S, R)
        rbase = ((layer * max_slots + slot) * Hkv + h[None, :]) * RB                  # [1, Hkv]
        E = sr32(SR)
        kk = side[rbase[:, :, None] + (e[:, None, None] * d) + np.arange(d)[None, None, :]]
        vv = side[rbase[:, :, None] + E * d + ring_vbyte(e[:, None, None], np.arange(d)[None, None, :], d)]
        k8[protected_mask] = kk.view(np.int8)
        v8[protected_mask] = vv.view(np.int8)
        sb = rbase + 2 * E * d
        ks = side[sb + 2 * e[:, None]].astype(np.uint16) | (side[sb + 2 * e[:, None] + 1].astype(np.uint16) << 8)
        vs = side[sb + 2 * (E + e)[:, None]].astype(np.uint16) | (
            side[sb + 2 * (E + e)[:, None] + 1].astype(np.uint16) << 8)
        k8s[protected_mask] = ks
        v8s[protected_mask] = vs
    out.update(k8=k8, v8=v8, k8s=k8s, v8s=v8s)
    return out


def protected_mask(n: int, S: int, R: int) -> np.ndarray:
    p = np.arange(n)
    return (p < min(S, n)) | (p >= max(S, n - R))


def pb_kv8_bytes(d: int) -> int:
    return PAGE * (2 * d + 4)


def gather_kv8(pages: np.ndarray, *, layer, num_pages, Hkv, d, block_tables, slot, n):
    """KV8 kind: k8, v8 (int8 [n, Hkv, d]) and k8s, v8s (uint16 [n, Hkv]) of
    positions [0, n) of the sequence in `slot`."""
    PB = pb_kv8_bytes(d)
    p = np.arange(n, dtype=np.int64)
    page = block_tables[slot, p // PAGE].astype(np.int64)
    tp = p % PAGE
    h = np.arange(Hkv, dtype=np.int64)
    base = ((layer * num_pages + page[:, None]) * Hkv + h[None, :]) * PB          # [n, Hkv]
    c = np.arange(d)[None, None, :]
    k8 = pages[base[:, :, None] + tp[:, None, None] * d + c].view(np.int8)
    v8 = pages[base[:, :, None] + PAGE * d + ring_vbyte(tp[:, None, None], c, d)].view(np.int8)

    def u16(idx):
        return pages[idx].astype(np.uint16) | (pages[idx + 1].astype(np.uint16) << 8)

    k8s = u16(base + 2 * PAGE * d + 2 * tp[:, None])
    v8s = u16(base + 2 * PAGE * d + 2 * PAGE + 2 * tp[:, None])
    return dict(k8=k8, v8=v8, k8s=k8s, v8s=v8s)


def gather_bf16(pages: np.ndarray, *, layer, num_pages, Hkv, d, block_tables, slot, n):
    """K and V (float32 [n, Hkv, d]) of the BF16 kind's pages."""
    PB = PAGE * d * 2 * 2
    p = np.arange(n, dtype=np.int64)
    page = block_tables[slot, p // PAGE].astype(np.int64)
    tp = p % PAGE
    h = np.arange(Hkv, dtype=np.int64)
    base = ((layer * num_pages + page[:, None]) * Hkv + h[None, :]) * PB
    c = np.arange(d)[None, None, :]
    idx = base[:, :, None] + 2 * (tp[:, None, None] * d + c)
    k = (pages[idx].astype(np.uint32) | (pages[idx + 1].astype(np.uint32) << 8)) << 16
    # V value (t, c) at ((t/8)*d + c)*8 + t%8 after the K block
    vi = base[:, :, None] + PAGE * d * 2 + 2 * (((tp[:, None, None] // 8) * d + c) * 8 + tp[:, None, None] % 8)
    v = (pages[vi].astype(np.uint32) | (pages[vi + 1].astype(np.uint32) << 8)) << 16
    return k.view(np.float32), v.view(np.float32)
