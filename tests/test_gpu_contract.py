"""The header's contract for device arrays (include/kv4.h, "Conventions"):
lengths, slot ids, block-table entries and append offsets cannot be checked on
the host, so the kernels clamp them into their declared ranges; out-of-range
values give wrong results but never an access outside the buffers.

Every buffer the library touches -- page pool, side pool, block table, keys and
values, append offsets, lengths, slot ids, queries, output, workspace -- is
carved out of a larger allocation whose guard bands hold a canary pattern.
The chosen values lie one step past each bound (page id = num_pages and -1,
slot = max_slots and -1, length = max_ctx + 1 and -1, cu_new past total_new,
ctx_before past the block table's capacity and -1), and each guard band is
larger than the furthest access such a value could make even without its
clamp, so this test cannot fault whatever the kernels do.  After valid
appends, appends with those values and decodes with those values, every guard
band is unchanged and every output is finite.
"""
import math

import numpy as np
import pytest
import torch

from int8_mixed_precision_amd import kv4
from int8_mixed_precision_amd import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

GUARD = 1 << 16            # bytes of every guard band
CANARY = 0xA5


class Guarded:
    """A tensor view with guard bands of GUARD bytes on both sides."""

    def __init__(self, shape, dtype, fill, dev):
        esz = torch.tensor([], dtype=dtype).element_size()
        g = GUARD // esz
        n = int(np.prod(shape)) if len(shape) else 1
        self.big = torch.empty(2 * g + n, dtype=dtype, device=dev)
        self.big.view(torch.uint8).fill_(CANARY)
        self.g, self.n = g, n
        self.view = self.big[g:g + n].view(*shape)
        self.view.copy_(fill if isinstance(fill, torch.Tensor) else
                        torch.full(shape, fill, dtype=dtype, device=dev))
        self.guards = self._guards()

    def _guards(self):
        b = self.big.view(torch.uint8)
        esz = self.big.element_size()
        return (b[:self.g * esz].clone(), b[(self.g + self.n) * esz:].clone())

    def intact(self):
        now = self._guards()
        return all(torch.equal(a, b) for a, b in zip(now, self.guards))


def _i32(vals, dev):
    return Guarded((len(vals),), torch.int32, torch.tensor(vals, dtype=torch.int32, device=dev), dev)


@pytest.mark.parametrize("case", ["mixed_gqa4", "mixed_gqa2", "mixed_int_path", "kv8", "bf16", "mixed_gqa5",
                                  "mixed_gqa8", "mixed_gqa16", "mixed_int_gqa8", "bf16_gqa8"])
def test_out_of_range_device_values_stay_inside_buffers(case):
    dev = torch.device("cuda")
    kind = {"kv8": kv4.KV4_KIND_KV8, "bf16": kv4.KV4_KIND_BF16,
            "bf16_gqa8": kv4.KV4_KIND_BF16}.get(case, kv4.KV4_KIND_MIXED)
    Hkv = 2
    Hq = {"mixed_gqa2": 4, "mixed_gqa5": 10, "mixed_gqa8": 16, "mixed_gqa16": 32, "mixed_int_gqa8": 16,
          "bf16_gqa8": 16}.get(case, 8)
    flags = kv4.KV4_FLAG_INT_PATH if case in ("mixed_int_path", "mixed_int_gqa8") else 0
    S, R = (4, 16) if kind == kv4.KV4_KIND_MIXED else (0, 0)
    B, max_slots, max_pages, num_pages = 4, 5, 4, 16
    cap = max_pages * 16
    H.log(f"case clamp contract {case}: Hq={Hq} Hkv={Hkv} S={S} R={R}")
    desc = kv4.make_desc(1, Hq, Hkv, 128, 16, 32, S, R, num_pages, max_slots, max_pages, kind, flags)
    pb, sb, _ = kv4.kv4_cache_required_bytes(desc)
    pages = Guarded((pb,), torch.uint8, 0, dev)          # zeros: every clamped read is finite
    side = Guarded((max(sb, 1),), torch.uint8, 0, dev)
    handle = kv4.kv4_cache_create(desc, pages.view, side.view if sb else None)
    guarded = [pages, side]
    try:
        # block table: slots 0..3 get pages 4 s .. 4 s + 3; the guard entries
        # (int32 num_pages: one page row past the pool) are never meant to be read
        bt_host = np.arange(max_slots * max_pages, dtype=np.int32).reshape(max_slots, max_pages) % num_pages
        bt_host[3, :2] = [num_pages, -1]                 # out-of-range page ids
        bt = Guarded((max_slots, max_pages), torch.int32, torch.from_numpy(bt_host).to(dev), dev)
        bt.big[:bt.g] = num_pages
        bt.big[bt.g + bt.n:] = num_pages
        bt.guards = bt._guards()
        guarded.append(bt)
        # ---- valid history: 40 tokens for slots 0..3
        cfg = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, seed=600, batch=B,
                       ctx_kind="fixed", ctx_fixed=(40,) * B)
        ks, vs = W.all_kv_sources(cfg, 0, [41] * B)
        kh = np.concatenate([k[:40] for k in ks])
        vh = np.concatenate([v[:40] for v in vs])
        kbuf = Guarded(kh.shape, torch.bfloat16, H.to_dev_bf16(kh, dev), dev)
        vbuf = Guarded(vh.shape, torch.bfloat16, H.to_dev_bf16(vh, dev), dev)
        cu = _i32([0, 40, 80, 120, 160], dev)
        c0 = _i32([0] * B, dev)
        sl = _i32([0, 1, 2, 3], dev)
        guarded += [kbuf, vbuf, cu, c0, sl]
        kv4.kv4_append(handle, 0, kbuf.view, vbuf.view, cu.view, c0.view, sl.view, bt.view, B, 160)
        # ---- step append with out-of-range offsets, positions and slots
        kn = np.concatenate([k[40:41] for k in ks])
        vn = np.concatenate([v[40:41] for v in vs])
        kstep = Guarded(kn.shape, torch.bfloat16, H.to_dev_bf16(kn, dev), dev)
        vstep = Guarded(vn.shape, torch.bfloat16, H.to_dev_bf16(vn, dev), dev)
        cu2 = _i32([0, 1, 2, B + 1, B + 5], dev)          # past total_new = B
        ctx2 = _i32([cap + 1, -1, 40, cap - 1], dev)      # past the table's capacity, negative
        sl2 = _i32([max_slots, -1, 2, 3], dev)            # one slot past, negative
        guarded += [kstep, vstep, cu2, ctx2, sl2]
        kv4.kv4_append(handle, 0, kstep.view, vstep.view, cu2.view, ctx2.view, sl2.view, bt.view, B, B)
        # ---- decodes with out-of-range lengths and slots
        max_ctx = 41
        q = W.queries(cfg, 0)
        qd = Guarded(q.shape, torch.bfloat16, H.to_dev_bf16(q, dev), dev)
        n_bad = _i32([max_ctx + 1, -1, 41, 30], dev)
        sl3 = _i32([max_slots, -1, 2, 3], dev)
        nb = kv4.kv4_decode_workspace_bytes(handle, B, max_ctx)
        ws = Guarded((nb,), torch.uint8, 0, dev)
        out = Guarded((B, Hq, 128), torch.float32, 0.0, dev)
        guarded += [qd, n_bad, sl3, ws, out]
        sm = 1 / math.sqrt(128)
        kv4.kv4_decode_attn(handle, 0, qd.view, n_bad.view, sl3.view, bt.view, B, max_ctx, sm,
                            out.view, kv4.KV4_OUT_F32, ws.view)
        outb = Guarded((B, Hq, 128), torch.bfloat16, 0.0, dev)
        guarded.append(outb)
        kv4.kv4_decode_attn(handle, 0, qd.view, n_bad.view, sl3.view, bt.view, B, max_ctx, sm,
                            outb.view, kv4.KV4_OUT_BF16, ws.view)
        torch.cuda.synchronize()
        for i, gb in enumerate(guarded):
            assert gb.intact(), f"guard band of buffer {i} changed"
        o = out.view.cpu().numpy()
        assert np.isfinite(o).all()
        assert np.isfinite(outb.view.float().cpu().numpy()).all()
        # a clamped length of -1 is an empty context: its rows are zero
        assert np.all(o[1] == 0)
        H.log(f"  {len(guarded)} guarded buffers intact, outputs finite")
    finally:
        kv4.kv4_cache_free(handle)
