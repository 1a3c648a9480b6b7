"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (KV4-RL decode step; tolerances fixed in advance):
  * quantized bytes -- INT4 codes, Delta, m of every stored position and the
    INT8 codes and scale of every protected position -- equal the oracle's
    bit for bit;
  * fp32 attention output: max |o - o*| <= 1e-3 and per-row
    ||o - o*||_inf / max(||o*||_inf, 1e-6) <= 2e-3 against the oracle's fp64
    attention over its own quantized cache.
Pools are filled with 0xFF bytes (binary16 NaN patterns) before use, so any
read of a position that was never written shows up as a mismatch or a NaN.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from int8_mixed_precision_amd import kv4
from int8_mixed_precision_amd import workloads as W
from tests import gpu_harness as H
from tests import layout as L
from tests import partition as PT

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-3, 2e-3


def _fill_garbage(built):
    built.cache.page_pool.fill_(0xFF)
    if built.cache.side_pool is not None:
        built.cache.side_pool.fill_(0xFF)


def _compare_bytes(built, pages, side, layer, oc, S, R, seqs=None, n_of=None):
    d, G, Hkv = 128, built.desc.group_size, built.desc.num_kv_heads
    seqs = range(len(oc.seq_lens)) if seqs is None else seqs
    for i, b in enumerate(seqs):
        n = int(oc.seq_lens[i]) if n_of is None else int(n_of[i])
        pm = L.protected_mask(n, S, R)
        gm = L.gather_mixed(pages, side, layer=layer, num_pages=built.desc.num_pages, Hkv=Hkv,
                            d=d, G=G, S=S, R=R, max_slots=built.desc.max_slots,
                            block_tables=built.bt_host, slot=int(built.slots_host[b]), n=n,
                            protected_mask=pm)
        sl = oc.seq(i)
        rows = slice(sl.start, sl.start + n)
        for name in ("k4", "v4", "k4d", "k4m", "v4d", "v4m"):
            want = getattr(oc, name)[rows]
            got = gm[name]
            if not np.array_equal(got, want):
                bad = np.argwhere(got != want)[0]
                raise AssertionError(f"seq {b} {name} mismatch at {tuple(bad)}: "
                                     f"got {got[tuple(bad)]} want {want[tuple(bad)]}")
        for name in ("k8", "v8", "k8s", "v8s"):
            want = getattr(oc, name)[rows][pm]
            got = gm[name][pm]
            if not np.array_equal(got, want):
                bad = np.argwhere(got != want)[0]
                raise AssertionError(f"seq {b} {name} mismatch at protected row {tuple(bad)}")


def _run_case(Hq, Hkv, G, S, R, ctx, seed, waves=0, layers=1, layer=0, check_bytes=True,
              garbage=True, pool_chunks=0, rotate=False, flags=0):
    """Build a cache for contexts ctx (history + one step token), decode, and
    compare with the oracle.  Returns (built, output, oracle cache).  With
    ``rotate`` the cache stores keys in the rotated basis (KV4_FLAG_ROTATE_K)
    and the oracle quantizes wht(k) and attends with wht(q)."""
    cfg = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, group=G, sink=S, recent=R,
                   seed=seed, batch=len(ctx), ctx_kind="fixed", ctx_fixed=tuple(int(c) for c in ctx))
    n = np.asarray(ctx, np.int64) + 1
    ks, vs = W.all_kv_sources(cfg, layer, n)
    q = W.queries(cfg, layer)
    built = H.make_cache(Hq, Hkv, G, S, R, n, layers=layers, waves=waves, pool_chunks=pool_chunks,
                         flags=flags | (kv4.KV4_FLAG_ROTATE_K if rotate else 0), seed=seed)
    if garbage:
        _fill_garbage(built)
    H.build_from_sources(built, layer, ks, vs, ctx)
    out = H.decode(built, layer, q, n).cpu().numpy()
    oc = oracle.MixedCache(ks, vs, G, rotate=rotate)
    want = oracle.attend_mixed(oracle.wht(q) if rotate else q, oc, S, R, 1 / math.sqrt(128))
    if check_bytes:
        pages, side = H.pools_host(built)
        _compare_bytes(built, pages, side, layer, oc, S, R)
    err = H.check_output(out, want, ATOL, RTOL)
    H.log(f"  max abs {err[0]:.2e} row rel {err[1]:.2e}")
    return built, out, oc, q, want


def test_tiny_config():
    c = W.CONFIGS["tiny"]
    H.log("case tiny: B=2 8q/2kv ctx 300,512 G=32 S=4 R=64 seed 0")
    ctx = W.contexts(c)
    n = ctx + 1
    ks, vs = W.all_kv_sources(c, 0, n)
    q = W.queries(c, 0)
    built = H.make_cache(c.q_heads, c.kv_heads, c.group, c.sink, c.recent, n, seed=c.seed)
    _fill_garbage(built)
    H.build_from_sources(built, 0, ks, vs, ctx)
    out = H.decode(built, 0, q, n).cpu().numpy()
    oc = oracle.MixedCache(ks, vs, c.group)
    pages, side = H.pools_host(built)
    _compare_bytes(built, pages, side, 0, oc, c.sink, c.recent)
    want = oracle.attend_mixed(q, oc, c.sink, c.recent, 1 / math.sqrt(128))
    err = H.check_output(out, want, ATOL, RTOL)
    H.log(f"tiny: max abs {err[0]:.2e} rel {err[1]:.2e}")
    # bf16 output is the fp32 result rounded to bf16
    outb = H.decode(built, 0, q, n, out_dtype=kv4.KV4_OUT_BF16).float().cpu().numpy()
    ref = torch.from_numpy(out).to(torch.bfloat16).float().numpy()
    assert np.array_equal(outb, ref)


@pytest.mark.parametrize("waves,pool", [(7, 0), (7, 8), (0, 0), (0, 16), (64, 16)])
def test_decode_phases_and_workspace_layout(waves, pool):
    """kv4_decode_partials followed by kv4_decode_merge equals kv4_decode_attn
    bit for bit, and the workspace holds what its header documents: the runs of
    (b, h) at records b*Hkv + h + s for the shares s = first .. last (as the
    documented partition gives them, static shares and pool chunks), the
    protected part at its own record, float d the base-2 log-normaliser.
    Merging the parts on the host by eq. A1 in fp64 reproduces the output, and
    the merged log-normaliser equals the oracle's log2 sum of 2^(sm_scale
    log2(e) q.k^) over the whole context."""
    Hq, Hkv, G, S, R = 8, 2, 32, 4, 64
    ctx = [0, 3, 40, 67, 68, 69, 300, 1000, 2500]
    H.log(f"case decode phases: 8q/2kv G=32 S=4 R=64 waves {waves} pool {pool}")
    built, out, oc, q, want = _run_case(Hq, Hkv, G, S, R, ctx, seed=11, waves=waves,
                                        pool_chunks=pool)
    n = np.asarray(ctx) + 1
    B, d, gqa = len(n), 128, Hq // Hkv
    dev = torch.device("cuda")
    qd = H.to_dev_bf16(q)
    nd = torch.from_numpy(n.astype(np.int32)).to(dev)
    max_ctx = int(n.max())
    sm = 1 / math.sqrt(d)
    ws = built.cache.workspace(B, max_ctx)
    ws.fill_(0xFF)                       # parts that are never written stay NaN
    kv4.kv4_decode_partials(built.cache.handle, 0, qd, nd, built.slots, built.block_tables, B,
                            max_ctx, sm, ws)
    o2 = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    kv4.kv4_decode_merge(built.cache.handle, nd, B, max_ctx, o2, kv4.KV4_OUT_F32, ws)
    torch.cuda.synchronize()
    assert np.array_equal(o2.cpu().numpy(), out)
    W, C = kv4.kv4_decode_partition(built.cache.handle)
    if waves:
        assert W == waves
    nrec = 2 * B * Hkv + W + C
    rec = ws[:nrec * gqa * (d + 4) * 4].view(torch.float32).cpu().numpy()
    rec = rec.reshape(nrec, gqa, d + 4).astype(np.float64)
    hdr = ws[nrec * gqa * (d + 4) * 4:nrec * gqa * (d + 4) * 4 + B * Hkv * 8].view(torch.int32)
    hdr = hdr.cpu().numpy().reshape(B * Hkv, 2)
    want_hdr, tiles, prot, pl = PT.header(n, S, R, Hkv, W, C)
    if pool > 0:
        assert pl["Cd"] > 0          # the case exercises the pool
    c2 = sm / math.log(2.0)
    for b in range(B):
        nb = int(n[b])
        sl = oc.seq(b)
        prot_mask = np.array([oracle.is_protected(p, nb, S, R) for p in range(nb)])
        k_hat = np.where(prot_mask[:, None, None],
                         oracle.dequant_int8(oc.k8[sl][:nb], oc.k8s[sl][:nb]),
                         oracle.dequant_int4(oc.k4[sl][:nb], oc.k4d[sl][:nb], oc.k4m[sl][:nb], G))
        for h in range(Hkv):
            bh = b * Hkv + h
            used = []
            if tiles[b]:
                first, last = (int(v) for v in hdr[bh])
                assert (first, last) == want_hdr[(b, h)], (b, h, first, last, want_hdr[(b, h)])
                used += [bh + w for w in range(first, last + 1)]
            if prot[b]:
                used.append(B * Hkv + W + C + bh)
            for j in range(gqa):
                z = rec[used, j, d]
                o = rec[used, j, :d]
                assert np.all(np.isfinite(z)) and np.all(np.isfinite(o))
                w = np.exp2(z - z.max())
                merged = (w[:, None] * o).sum(0) / w.sum()
                assert np.abs(merged - out[b, h * gqa + j]).max() <= 1e-5
                qq = H.to_dev_bf16(q[b, h * gqa + j]).float().cpu().numpy().astype(np.float64)
                s = c2 * (k_hat[:, h, :] @ qq)
                z_ref = s.max() + np.log2(np.exp2(s - s.max()).sum())
                z_got = z.max() + np.log2(w.sum())
                assert abs(z_got - z_ref) <= 1e-4 * max(1.0, abs(z_ref)), (b, h, j, z_got, z_ref)


@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("S", [0, 1, 4, 16])
def test_edge_grid(G, S):
    """n in [1, 40] x R in {0, 1, 3, 8, 64}: every case against the oracle."""
    for R in (0, 1, 3, 8, 64):
        H.log(f"case edge grid G={G} S={S} R={R} n=1..40")
        ctx = np.arange(0, 40)
        _run_case(8, 2, G, S, R, ctx, seed=S * 131 + R * 7 + G)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (16, 2), (32, 8)])
def test_gqa_ratios(Hq, Hkv):
    H.log(f"case gqa Hq={Hq} Hkv={Hkv}")
    _run_case(Hq, Hkv, 32, 4, 16, [0, 5, 19, 20, 21, 100, 257, 700], seed=Hq * 10 + Hkv)


def test_ratio8_matrix_core():
    """q/kv ratio 8 on the matrix core (two four-head halves per tile): group
    sizes 32, 64 and 128, rotated keys, edge lengths around S + R, several
    waves, and a 64 q / 8 kv layer with long contexts; the integer path too."""
    edge = [0, 1, 3, 4, 5, 19, 20, 21, 67, 68, 69, 100, 257, 700, 2500]
    for G, rotate, waves in ((32, False, 0), (64, False, 5), (128, False, 0), (32, True, 0), (128, True, 7)):
        H.log(f"case ratio 8 Hq=16 Hkv=2 G={G} rotate={rotate} waves={waves}")
        _run_case(16, 2, G, 4, 64, edge, seed=170 + G + rotate, rotate=rotate, waves=waves)
    H.log("case ratio 8 Hq=64 Hkv=8 G=32, long contexts")
    _run_case(64, 8, 32, 4, 128, [9000, 17, 4000, 131, 133], seed=178)
    ictx = [0, 3, 7, 8, 9, 40, 67, 68, 69, 300, 1000, 2500]
    for G, rotate in ((32, False), (64, True)):
        H.log(f"case ratio 8, integer path, G={G} rotate={rotate}")
        _int_case(16, 2, G, 4, 64, ictx, seed=180 + G + rotate, rotate=rotate)
    H.log("case ratio 8, integer path, Hq=64 Hkv=8, long contexts")
    _int_case(64, 8, 32, 4, 128, [9000, 17, 4000], seed=183)


def test_other_ratios():
    """q/kv ratios that are not powers of two, and 16: the matrix core runs the q
    heads of a kv head in halves of four with the heads past the ratio padded
    (3: one half, 5-7: two, 16: four), on the floating-point and integer paths
    and the BF16 kind (ratio 3), against the oracle."""
    edge = [0, 3, 19, 20, 21, 67, 68, 69, 300, 1000, 2500]
    for Hq, Hkv, G, rotate in ((12, 4, 32, False), (40, 8, 32, False), (12, 2, 64, True), (14, 2, 128, False),
                               (64, 4, 32, False), (32, 2, 128, True)):
        H.log(f"case ratio {Hq // Hkv}: Hq={Hq} Hkv={Hkv} G={G} rotate={rotate}")
        _run_case(Hq, Hkv, G, 4, 64, edge, seed=190 + Hq + Hkv + G, rotate=rotate)
    for Hq, Hkv, G in ((12, 4, 32), (40, 8, 32), (14, 2, 64)):
        H.log(f"case ratio {Hq // Hkv}, integer path: Hq={Hq} Hkv={Hkv} G={G}")
        _int_case(Hq, Hkv, G, 4, 64, edge, seed=195 + Hq + Hkv + G)
    H.log("case ratio 3, BF16 kind")
    ctx = np.array([0, 15, 16, 17, 300, 1000, 3000])
    n = ctx + 1
    cfg = W.scaled(W.CONFIGS["tiny"], seed=37, batch=len(ctx), ctx_kind="fixed", ctx_fixed=tuple(ctx),
                   q_heads=12, kv_heads=4)
    ks, vs = W.all_kv_sources(cfg, 0, n)
    q = W.queries(cfg, 0)
    built = H.make_cache(12, 4, 32, 0, 0, n, kind=kv4.KV4_KIND_BF16, seed=6)
    H.build_from_sources(built, 0, ks, vs, ctx)
    out = H.decode(built, 0, q, n).cpu().numpy()
    H.check_output(out, oracle.attend_dense(q, ks, vs, 1 / math.sqrt(128)), ATOL, RTOL)


def test_group_64_and_multi_layer():
    H.log("case G=64, 3 layers, layer 2")
    _run_case(8, 2, 64, 4, 32, [33, 150, 401], seed=77, layers=3, layer=2)


# Self-agreement bound across wave counts.  The merge (eq. A1) is exact up to
# rounding; what changes with the cut is the fp32 rounding order.  The PV
# accumulator sums w * code (codes enter the matrix core exactly) over up to
# n/32 tile additions, so one path deviates from the exact value by about
# sqrt(n/32) * 2^-24 * 15 * max(Delta_V) <= ~1e-5 at n = 2,500, plus 2^-18
# relative rounding of the bf16 hi+lo operand.  Two paths: 5e-5.
SPLIT_SELF_TOL = 5e-5


def test_wave_invariance():
    """The partition's pieces merged by eq. A1 give the same output for any
    number of waves (one wave running everything, to more waves than units)."""
    ctx = [0, 3, 70, 300, 1000, 2500]
    outs = {}
    for waves, pool in ((1, 0), (1, 8), (2, 0), (7, 0), (7, 8), (64, 0), (64, 16), (0, 0),
                        (0, 4096), (5000, 0)):
        H.log(f"case waves={waves} pool={pool}")
        _, out, _, _, _ = _run_case(8, 2, 32, 4, 64, ctx, seed=5, waves=waves, pool_chunks=pool)
        outs[(waves, pool)] = out
    ref = outs[(1, 0)]        # one wave, no pool: one run per (sequence, kv head)
    for waves, o in outs.items():
        assert np.abs(o - ref).max() <= SPLIT_SELF_TOL, (waves, float(np.abs(o - ref).max()))


def test_bulk_equals_token_by_token():
    """Re-prefill path: a cache built in one bulk append equals the cache grown
    one token per append (the quantization is per token)."""
    Hq, Hkv, G, S, R = 8, 2, 32, 4, 16
    n = np.array([1, 9, 40, 77])
    cfg = W.scaled(W.CONFIGS["tiny"], seed=9, batch=4, ctx_kind="fixed", ctx_fixed=tuple(n))
    ks, vs = W.all_kv_sources(cfg, 0, n)
    H.log("case bulk vs token-by-token")
    a = H.make_cache(Hq, Hkv, G, S, R, n, seed=1, slot_perm=False)
    b = H.make_cache(Hq, Hkv, G, S, R, n, seed=1, slot_perm=False)
    _fill_garbage(a)
    _fill_garbage(b)
    H.append_chunks(a, 0, ks, vs, [0] * 4)
    for t in range(int(n.max())):
        seqs = [i for i in range(4) if n[i] > t]
        H.append_chunks(b, 0, [ks[i][t:t + 1] for i in seqs], [vs[i][t:t + 1] for i in seqs],
                        [t] * len(seqs), seqs)
    pa, sa = H.pools_host(a)
    pb, sb = H.pools_host(b)
    assert np.array_equal(a.bt_host, b.bt_host) and np.array_equal(a.slots_host, b.slots_host)
    for i in range(4):
        kw = dict(layer=0, num_pages=a.desc.num_pages, Hkv=Hkv, d=128, G=G, S=S, R=R,
                  max_slots=a.desc.max_slots, block_tables=a.bt_host, slot=int(a.slots_host[i]),
                  n=int(n[i]), protected_mask=L.protected_mask(int(n[i]), S, R))
        ga = L.gather_mixed(pa, sa, **kw)
        gb = L.gather_mixed(pb, sb, **kw)
        for k in ga:
            assert np.array_equal(ga[k], gb[k]), (i, k)


@pytest.mark.parametrize("G,rotate", [(32, False), (128, True)])
def test_bulk_append_long_history_in_two_unaligned_parts(G, rotate):
    """Bulk appends at the extremes of the launch's shape, bytes bit-exact
    against the oracle (KV4-RL eq. 3.3; Appendix A.3 "Encoding and
    allocation"): one 20,003-token history appended in two calls, the second
    starting at position 4,003 (each call then has a partial first or last
    half page beside hundreds of waves of whole ones, and the second rewrites
    the whole side ring), and 64 short histories of 1 to 299 tokens in one
    call (few whole half pages per sequence)."""
    Hq, Hkv, S, R = 8, 2, 4, 128
    flags = kv4.KV4_FLAG_ROTATE_K if rotate else 0
    n = np.array([20003])
    H.log(f"case bulk long history G={G} rotate={rotate}")
    cfg = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, group=G, sink=S, recent=R, seed=77,
                   batch=1, ctx_kind="fixed", ctx_fixed=(int(n[0]),))
    ks, vs = W.all_kv_sources(cfg, 0, n)
    built = H.make_cache(Hq, Hkv, G, S, R, n, flags=flags, seed=77)
    _fill_garbage(built)
    cut = 4003
    H.append_chunks(built, 0, [ks[0][:cut]], [vs[0][:cut]], [0])
    H.append_chunks(built, 0, [ks[0][cut:]], [vs[0][cut:]], [cut])
    pages, side = H.pools_host(built)
    _compare_bytes(built, pages, side, 0, oracle.MixedCache(ks, vs, G, rotate=rotate), S, R)

    n2 = np.random.default_rng(5).integers(1, 300, 64)
    H.log(f"case bulk 64 short histories G={G} rotate={rotate}")
    cfg2 = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, group=G, sink=S, recent=R, seed=78,
                    batch=64, ctx_kind="fixed", ctx_fixed=tuple(int(x) for x in n2))
    ks2, vs2 = W.all_kv_sources(cfg2, 0, n2)
    b2 = H.make_cache(Hq, Hkv, G, S, R, n2, flags=flags, seed=78)
    _fill_garbage(b2)
    H.append_chunks(b2, 0, ks2, vs2, [0] * len(n2))
    pages2, side2 = H.pools_host(b2)
    _compare_bytes(b2, pages2, side2, 0, oracle.MixedCache(ks2, vs2, G, rotate=rotate), S, R)


def test_decode_steps_cross_demotion_boundary():
    """64 consecutive steps of (append, decode) starting at n = S+R-32, so the
    cache goes from all-INT8 to mixed and positions are demoted every step;
    INT4 bytes of a position never change after its append."""
    Hq, Hkv, G, S, R = 8, 2, 32, 4, 64
    steps = 64
    start = S + R - 32
    ctx0 = np.array([start, start + 5, start + 40, 300])
    cfg = W.scaled(W.CONFIGS["tiny"], seed=21, batch=4, ctx_kind="fixed", ctx_fixed=tuple(ctx0))
    total = ctx0 + steps
    ks, vs = W.all_kv_sources(cfg, 0, total)
    built = H.make_cache(Hq, Hkv, G, S, R, total, seed=3)
    _fill_garbage(built)
    H.append_chunks(built, 0, [k[:c] for k, c in zip(ks, ctx0)], [v[:c] for v, c in zip(vs, ctx0)],
                    [0] * 4)
    oc = oracle.MixedCache(ks, vs, G)
    first = None
    for t in range(steps):
        H.log(f"case demotion step {t}")
        ctx = ctx0 + t
        H.append_chunks(built, 0, [k[c:c + 1] for k, c in zip(ks, ctx)],
                        [v[c:c + 1] for v, c in zip(vs, ctx)], list(ctx))
        q = W.queries(cfg, 0, step=t)
        out = H.decode(built, 0, q, ctx + 1).cpu().numpy()
        want = oracle.attend_mixed(q, oc, S, R, 1 / math.sqrt(128), seq_lens=ctx + 1)
        H.check_output(out, want, ATOL, RTOL)
        if t in (0, 31, 63):
            pages, side = H.pools_host(built)
            _compare_bytes(built, pages, side, 0, oc, S, R, n_of=ctx + 1)
            snap = pages.copy()
            if first is None:
                first = (snap, ctx + 1)
            else:
                # lifetime: INT4 bytes of positions present at step 0 are unchanged
                n0 = first[1]
                for i in range(4):
                    kw = dict(layer=0, num_pages=built.desc.num_pages, Hkv=Hkv, d=128, G=G, S=S,
                              R=R, max_slots=built.desc.max_slots, block_tables=built.bt_host,
                              slot=int(built.slots_host[i]), n=int(n0[i]))
                    g0 = L.gather_mixed(first[0], None, **kw)
                    g1 = L.gather_mixed(snap, None, **kw)
                    for k in ("k4", "v4", "k4d", "k4m", "v4d", "v4m"):
                        assert np.array_equal(g0[k], g1[k]), (t, i, k)


@pytest.mark.parametrize("vscale", [1.0, 300.0, 1e-3])
def test_extreme_scales(vscale):
    """Inputs far from N(0, 1): per-head q magnitudes from 1e-30 to 100
    (one head all zero), keys x 10 and values x vscale.  The matrix-core path
    scales q by a power of two per head and carries codes and weights as
    subnormal / power-of-two-scaled numbers; the errors scale with the
    values, so the absolute bar is 1e-3 * max(vscale, 1)."""
    Hq, Hkv, G, S, R = 32, 8, 32, 4, 64
    ctx = [70, 333, 1200, 2500]
    H.log(f"case extreme scales: vscale {vscale} ctx {ctx}")
    cfg = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, group=G, sink=S, recent=R,
                   seed=11, batch=len(ctx), ctx_kind="fixed", ctx_fixed=tuple(ctx))
    n = np.asarray(ctx, np.int64) + 1
    ks, vs = W.all_kv_sources(cfg, 0, n)
    ks = [W.to_bf16_values(k * 10.0) for k in ks]
    vs = [W.to_bf16_values(v * vscale) for v in vs]
    q = W.queries(cfg, 0).astype(np.float64)
    head_scale = np.array([1e-30, 1e-6, 1e-2, 1.0, 3.0, 10.0, 100.0, 0.0] * (Hq // 8))
    q = W.to_bf16_values((q * head_scale[None, :, None]).astype(np.float32))
    built = H.make_cache(Hq, Hkv, G, S, R, n, seed=11)
    _fill_garbage(built)
    H.build_from_sources(built, 0, ks, vs, ctx)
    out = H.decode(built, 0, q, n).cpu().numpy()
    oc = oracle.MixedCache(ks, vs, G)
    pages, side = H.pools_host(built)
    _compare_bytes(built, pages, side, 0, oc, S, R)
    want = oracle.attend_mixed(q, oc, S, R, 1 / math.sqrt(128))
    assert np.isfinite(out).all()
    err = H.check_output(out, want, ATOL * max(vscale, 1.0), RTOL)
    H.log(f"  max abs {err[0]:.2e} row rel {err[1]:.2e}")


@pytest.mark.parametrize("G", [32, 128])
def test_append_extreme_values(G):
    """Quantizer edge cases through the HIP append, bytes against the oracle
    bit for bit (KV4-RL eq. 3.3 and Appendix A.3; readings Q-1 .. Q-4): groups
    of magnitude 1e-6 (offset and step binary16 subnormals), bf16 values below
    binary32's normal range mixed with N(0, 1), constant groups (step 0),
    values out to +-65280, INT4 groups whose values sit exactly between two
    codes, whole kv-head vectors whose INT8 codes are exact ties, and groups
    scaled by 10^-6 .. 10^3.  These are the cases where the append's binary32
    code decision hands over to its exact binary64 test.  Most positions are
    protected (S = 4, R = 24), so both encodings are compared.

    The attention over this cache is then checked against the oracle with a
    bar derived from binary32 score arithmetic: keys near 65280 give scores of
    1e4 .. 1e5 nats, where one binary32 ulp is already 2^-24 of that, so the
    workloads' fixed 2e-3 cannot hold.  With every partial sum of a score
    bounded by A = sm_scale * max_t sum_c |q_c k^_{t,c}| and at most 16
    roundings of 2^-24 each, every score is within delta = 2^-20 A, every
    normalised weight within a factor e^(2 delta), and every output within
    (e^(2 delta) - 1) * 2 max|v^| of the oracle's, plus the value path's
    1e-3 * max|v^|.  The queries are scaled by 2^-12 so that this bar stays
    near 3e-3 * max|v^| (it is checked per row)."""
    Hq, Hkv, S, R = 8, 2, 4, 24
    ctx = [0, 5, 27, 28, 29, 90, 200]
    n = np.asarray(ctx, np.int64) + 1
    H.log(f"case append extreme values G={G} ctx {ctx}")
    ks, vs = [], []
    for b, nb in enumerate(n):
        k, v = W.extreme_kv_sources(1000 + 10 * G + b, int(nb), Hkv, 128, G,
                                    int8_tie_rows=(0, int(nb) - 1))
        ks.append(k)
        vs.append(v)
    cfg = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, group=G, sink=S, recent=R,
                   seed=1000 + G, batch=len(ctx), ctx_kind="fixed", ctx_fixed=tuple(ctx))
    q = W.to_bf16_values(W.queries(cfg, 0) * np.float32(2.0 ** -12))
    built = H.make_cache(Hq, Hkv, G, S, R, n, seed=1000 + G)
    _fill_garbage(built)
    H.build_from_sources(built, 0, ks, vs, ctx)
    out = H.decode(built, 0, q, n).cpu().numpy()
    oc = oracle.MixedCache(ks, vs, G)
    pages, side = H.pools_host(built)
    _compare_bytes(built, pages, side, 0, oc, S, R)
    # the cases are really present in the oracle's bytes
    d16 = oracle.f16_bits_to_f64(oc.k4d)
    assert np.any((d16 > 0) & (d16 < 2.0 ** -14))          # subnormal steps
    assert np.any(oc.k4d == 0)                              # constant groups
    assert np.any(oc.k8s == 0x3C00)                         # INT8 scale 1 (the tie rows)
    assert np.isfinite(out).all()
    sm = 1 / math.sqrt(128)
    want = oracle.attend_mixed(q, oc, S, R, sm)
    worst = 0.0
    for b in range(len(ctx)):
        nb = int(n[b])
        sl = oc.seq(b)
        prot = np.array([oracle.is_protected(p, nb, S, R) for p in range(nb)])
        khat = np.where(prot[:, None, None], oracle.dequant_int8(oc.k8[sl][:nb], oc.k8s[sl][:nb]),
                        oracle.dequant_int4(oc.k4[sl][:nb], oc.k4d[sl][:nb], oc.k4m[sl][:nb], G))
        vhat = np.where(prot[:, None, None], oracle.dequant_int8(oc.v8[sl][:nb], oc.v8s[sl][:nb]),
                        oracle.dequant_int4(oc.v4[sl][:nb], oc.v4d[sl][:nb], oc.v4m[sl][:nb], G))
        for j in range(Hq):
            h = j // (Hq // Hkv)
            A = sm * float((np.abs(khat[:, h, :]) @ np.abs(q[b, j].astype(np.float64))).max())
            vmax = float(np.abs(vhat[:, h, :]).max())
            tol = ATOL * max(vmax, 1.0) + math.expm1(2 * 2.0 ** -20 * A) * 2 * vmax
            e = float(np.abs(out[b, j] - want[b, j]).max())
            assert e <= tol, (b, j, e, tol, A)
            worst = max(worst, e / max(vmax, 1.0))
    H.log(f"  bytes bit-exact; outputs within the derived bar, worst error {worst:.2e} of max|v^|")


def test_valu_decode_flag():
    """KV4_FLAG_VALU_DECODE: the decode runs on the vector-ALU kernels at every
    q/kv ratio (without the flag the mixed kind runs on the matrix-core
    kernels), against the same oracle (floating-point and integer paths,
    rotated keys, G = 32 and 128, edge lengths, the BF16 kind)."""
    ctx = [0, 3, 4, 5, 19, 20, 21, 100, 257, 700, 2500]
    for Hq, Hkv, G, rotate in ((8, 2, 32, False), (8, 2, 128, False), (8, 2, 32, True), (4, 4, 32, False),
                               (8, 4, 64, True), (16, 2, 32, False)):
        H.log(f"case vector-ALU decode Hq={Hq} Hkv={Hkv} G={G} rotate={rotate}")
        _run_case(Hq, Hkv, G, 4, 16, ctx, seed=140 + G + Hq + Hkv, rotate=rotate,
                  flags=kv4.KV4_FLAG_VALU_DECODE)
    ictx = [0, 3, 7, 8, 9, 40, 67, 68, 69, 300, 1000, 2500]
    for Hq, Hkv in ((8, 2), (8, 8), (8, 4), (16, 2)):
        H.log(f"case vector-ALU decode, integer path, Hq={Hq} Hkv={Hkv}")
        _int_case(Hq, Hkv, 32, 4, 64, ictx, seed=150 + Hq + Hkv, flags=kv4.KV4_FLAG_VALU_DECODE)
    ctxb = np.array([0, 15, 16, 17, 300, 1000, 3000])
    n = ctxb + 1
    for Hq, Hkv in ((8, 2), (8, 4), (16, 2)):
        H.log(f"case vector-ALU decode, BF16 kind, Hq={Hq} Hkv={Hkv}")
        cfg = W.scaled(W.CONFIGS["tiny"], seed=33, batch=len(ctxb), ctx_kind="fixed", ctx_fixed=tuple(ctxb),
                       q_heads=Hq, kv_heads=Hkv)
        ks, vs = W.all_kv_sources(cfg, 0, n)
        q = W.queries(cfg, 0)
        built = H.make_cache(Hq, Hkv, 32, 0, 0, n, kind=kv4.KV4_KIND_BF16, flags=kv4.KV4_FLAG_VALU_DECODE,
                             seed=5)
        H.build_from_sources(built, 0, ks, vs, ctxb)
        out = H.decode(built, 0, q, n).cpu().numpy()
        H.check_output(out, oracle.attend_dense(q, ks, vs, 1 / math.sqrt(128)), ATOL, RTOL)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 4), (4, 4), (16, 2), (10, 2)])
def test_bf16_comparator(Hq, Hkv):
    """BF16 kind: pages hold the bf16 values exactly; output matches the
    oracle's dense attention (q/kv ratios 4, 2, 1, 8 and 5, all on the
    matrix core: one four-head half up to 4, two above)."""
    ctx = np.array([0, 15, 16, 17, 300, 1000, 3000])
    n = ctx + 1
    cfg = W.scaled(W.CONFIGS["tiny"], seed=31, batch=len(ctx), ctx_kind="fixed", ctx_fixed=tuple(ctx),
                   q_heads=Hq, kv_heads=Hkv)
    ks, vs = W.all_kv_sources(cfg, 0, n)
    q = W.queries(cfg, 0)
    for waves in (0, 3):
        H.log(f"case bf16 comparator Hq={Hq} Hkv={Hkv} waves={waves}")
        built = H.make_cache(Hq, Hkv, 32, 0, 0, n, kind=kv4.KV4_KIND_BF16, waves=waves, seed=4)
        _fill_garbage(built)
        H.build_from_sources(built, 0, ks, vs, ctx)
        out = H.decode(built, 0, q, n).cpu().numpy()
        pages, _ = H.pools_host(built)
        for b in range(len(ctx)):
            k, v = L.gather_bf16(pages, layer=0, num_pages=built.desc.num_pages, Hkv=Hkv, d=128,
                                 block_tables=built.bt_host, slot=int(built.slots_host[b]), n=int(n[b]))
            assert np.array_equal(k, ks[b]) and np.array_equal(v, vs[b])
        want = oracle.attend_dense(q, ks, vs, 1 / math.sqrt(128))
        H.check_output(out, want, ATOL, RTOL)


# ---------------------------------------------------------------------------
# KV8 kind (KV4-RL Fig. 3b / Fig. 4a comparison point): every position holds
# the side entries' INT8 encoding; bytes are compared with the oracle's INT8
# copies of every position, outputs with its fp64 attention when every
# position is protected (S = 0, R >= n).
# ---------------------------------------------------------------------------

def _kv8_case(Hkv, ctx, seed, waves=0, layers=1, layer=0, pool_chunks=0, ratio=4):
    Hq = ratio * Hkv
    n = np.asarray(ctx, np.int64) + 1
    cfg = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, seed=seed, batch=len(ctx),
                   ctx_kind="fixed", ctx_fixed=tuple(int(c) for c in ctx))
    ks, vs = W.all_kv_sources(cfg, layer, n)
    q = W.queries(cfg, layer)
    built = H.make_cache(Hq, Hkv, 32, 0, 0, n, layers=layers, kind=kv4.KV4_KIND_KV8, waves=waves,
                         seed=seed, pool_chunks=pool_chunks)
    _fill_garbage(built)
    H.build_from_sources(built, layer, ks, vs, ctx)
    out = H.decode(built, layer, q, n).cpu().numpy()
    oc = oracle.MixedCache(ks, vs, 32)
    pages, _ = H.pools_host(built)
    for b in range(len(ctx)):
        got = L.gather_kv8(pages, layer=layer, num_pages=built.desc.num_pages, Hkv=Hkv, d=128,
                           block_tables=built.bt_host, slot=int(built.slots_host[b]), n=int(n[b]))
        sl = oc.seq(b)
        for name in ("k8", "v8", "k8s", "v8s"):
            want = getattr(oc, name)[sl]
            if not np.array_equal(got[name], want):
                bad = np.argwhere(got[name] != want)[0]
                raise AssertionError(f"seq {b} {name} mismatch at {tuple(bad)}")
    want = oracle.attend_mixed(q, oc, 0, int(n.max()), 1 / math.sqrt(128))
    err = H.check_output(out, want, ATOL, RTOL)
    H.log(f"  max abs {err[0]:.2e} row rel {err[1]:.2e}")
    return out


@pytest.mark.parametrize("Hkv", [1, 2, 8])
def test_kv8_kind(Hkv):
    ctx = [0, 14, 15, 16, 30, 31, 32, 33, 63, 64, 300, 1000, 2500]
    H.log(f"case kv8 Hkv={Hkv}")
    out = _kv8_case(Hkv, ctx, seed=80 + Hkv)
    for waves in (1, 5):
        H.log(f"case kv8 Hkv={Hkv} waves={waves}")
        o2 = _kv8_case(Hkv, ctx, seed=80 + Hkv, waves=waves)
        assert np.abs(o2 - out).max() <= 5e-5


@pytest.mark.parametrize("ratio", [1, 2, 3, 5, 8])
def test_kv8_ratios(ratio):
    """KV8 kind at q/kv ratios other than 4 (the four-head matrix-core layout
    with the heads past the ratio padded; 5 and 8 in two four-head halves per
    staged tile)."""
    H.log(f"case kv8 ratio {ratio}")
    _kv8_case(2, [0, 15, 16, 31, 32, 300, 1000, 2500], seed=90 + ratio, ratio=ratio)


def test_kv8_layers_and_long_context():
    H.log("case kv8, 3 layers, layer 2, waves 7")
    _kv8_case(2, [33, 150, 401, 1200], seed=91, layers=3, layer=2, waves=7)
    H.log("case kv8 long 9000 + short")
    _kv8_case(4, [9000, 1, 47], seed=92)
    H.log("case kv8, dynamic pool of 16 chunks, 64 waves")
    _kv8_case(2, [1000, 2500, 40, 3000], seed=93, waves=64, pool_chunks=16)


# ---------------------------------------------------------------------------
# Integer decode path (KV4_FLAG_INT_PATH; KV4-RL Appendix A.3), against the
# oracle's integer path.  Where the kernel's binary32 probabilities and the
# oracle's binary64 ones lie on two sides of a rounding tie of the 8-bit
# operand, either code is a correct reading: the oracle's bound (every code
# within 2^-6 of a tie moved by one) covers those; all else agrees to 1e-4.
# And the kernel is much closer to the integer oracle than the integer path is
# to the exact attention over the same cache (no systematic deviation).
# ---------------------------------------------------------------------------

INT_ATOL = 1e-4


def _int_case(Hq, Hkv, G, S, R, ctx, seed, rotate=False, waves=0, layers=1, layer=0, pool_chunks=0,
              qscale=1.0, flags=0):
    cfg = W.scaled(W.CONFIGS["tiny"], q_heads=Hq, kv_heads=Hkv, group=G, sink=S, recent=R,
                   seed=seed, batch=len(ctx), ctx_kind="fixed", ctx_fixed=tuple(int(c) for c in ctx))
    n = np.asarray(ctx, np.int64) + 1
    ks, vs = W.all_kv_sources(cfg, layer, n)
    q = W.queries(cfg, layer)
    if qscale != 1.0:
        q = W.to_bf16_values((q * qscale).astype(np.float32))
    flags |= kv4.KV4_FLAG_INT_PATH | (kv4.KV4_FLAG_ROTATE_K if rotate else 0)
    built = H.make_cache(Hq, Hkv, G, S, R, n, layers=layers, waves=waves, flags=flags, seed=seed,
                         pool_chunks=pool_chunks)
    _fill_garbage(built)
    H.build_from_sources(built, layer, ks, vs, ctx)
    out = H.decode(built, layer, q, n).cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()
    oc = oracle.MixedCache(ks, vs, G, rotate=rotate)
    qq = oracle.wht(q) if rotate else q
    want, bound = oracle.attend_int(qq, oc, S, R, 1 / math.sqrt(128))
    exact = oracle.attend_mixed(qq, oc, S, R, 1 / math.sqrt(128))
    err = np.abs(out - want)
    excess = err - (INT_ATOL + bound)
    assert excess.max() <= 0, (f"|o - o_int| exceeds 1e-4 + bound by {excess.max():.3e} at "
                               f"{np.unravel_index(excess.argmax(), excess.shape)}")
    own = float(np.sqrt(np.mean((want - exact) ** 2)))
    dev = float(np.sqrt(np.mean((out - want) ** 2)))
    H.log(f"  max |o - o_int| {err.max():.2e}, rms {dev:.2e}; integer path vs exact: "
          f"rms {own:.2e}, max {np.abs(want - exact).max():.2e}")
    assert dev <= 0.1 * own + 1e-6
    return out


@pytest.mark.parametrize("Hq,Hkv,G", [(8, 2, 32), (32, 8, 32), (16, 4, 64), (8, 2, 128), (8, 8, 32),
                                      (16, 8, 64), (16, 2, 128)])
def test_integer_path(Hq, Hkv, G):
    H.log(f"case integer path Hq={Hq} Hkv={Hkv} G={G}")
    _int_case(Hq, Hkv, G, 4, 64, [0, 3, 7, 8, 9, 40, 67, 68, 69, 300, 1000, 2500], seed=110 + Hq + G)


def test_integer_path_edges_rotation_layers():
    for S, R in ((0, 0), (0, 8), (16, 3), (4, 128)):
        H.log(f"case integer path edges S={S} R={R}")
        _int_case(8, 2, 32, S, R, list(range(0, 40, 3)) + [S + R, S + R + 1, 600], seed=120 + S + R)
    H.log("case integer path, rotated keys, GQA 4 (matrix core)")
    _int_case(8, 2, 32, 4, 64, [0, 40, 67, 300, 1000, 2500], seed=131, rotate=True)
    _int_case(16, 4, 128, 16, 8, [3, 200, 1500], seed=136, rotate=True)
    H.log("case integer path, rotated keys, GQA 2 and 8 (matrix core)")
    _int_case(8, 4, 32, 4, 64, [0, 67, 1000], seed=134, rotate=True)
    _int_case(16, 2, 64, 4, 64, [5, 300], seed=135, rotate=True)
    H.log("case integer path, 3 layers, layer 1, waves 7")
    _int_case(8, 2, 32, 4, 32, [33, 150, 401, 1200], seed=132, layers=3, layer=1, waves=7)
    H.log("case integer path, 32q/8kv long")
    _int_case(32, 8, 32, 4, 128, [9000, 17, 4000], seed=133)
    H.log("case integer path, queries x30 (peaked softmax, vanishing blocks), GQA 4 and 2")
    _int_case(8, 2, 32, 4, 64, [300, 1000, 2500], seed=138, qscale=30.0)
    _int_case(8, 4, 32, 4, 64, [300, 1000, 2500], seed=139, qscale=30.0)
    H.log("case integer path, dynamic pool of 16 chunks, 64 waves")
    _int_case(8, 2, 32, 4, 64, [1000, 2500, 40, 3000], seed=137, waves=64, pool_chunks=16)


# ---------------------------------------------------------------------------
# Keys stored in the rotated basis (KV4-RL Section 5.1, Appendix A.3): the
# append rotates k before both quantizers, the decode rotates q; bytes are
# compared with the oracle's quantization of wht(k), outputs with its fp64
# attention of wht(q) over that cache.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv,G", [(8, 2, 32), (8, 2, 128), (16, 4, 64), (4, 4, 32), (16, 2, 32),
                                      (32, 8, 32)])
def test_rotated_keys(Hq, Hkv, G):
    H.log(f"case rotated keys Hq={Hq} Hkv={Hkv} G={G}")
    _run_case(Hq, Hkv, G, 4, 64, [0, 3, 40, 67, 68, 69, 300, 1000, 2500], seed=Hq + 3 * G + Hkv,
              rotate=True)


def test_rotated_keys_edges_and_layers():
    for S, R in ((0, 0), (0, 8), (16, 3), (4, 128)):
        H.log(f"case rotated keys edges S={S} R={R}")
        _run_case(8, 2, 32, S, R, list(range(0, 40, 3)) + [S + R, S + R + 1, 600], seed=71 + S + R,
                  rotate=True)
    H.log("case rotated keys, 3 layers, layer 1, waves 7")
    _run_case(8, 2, 32, 4, 32, [33, 150, 401, 1200], seed=72, layers=3, layer=1, waves=7, rotate=True)

