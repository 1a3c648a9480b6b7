"""The documented decode partition (static shares plus a pool of chunks), written
out on the host in plain Python integers, for the layout tests.  It mirrors the
closed forms that kv4_decode_partials documents; nothing here runs on the GPU."""

MIN_UNITS = 20
POOL_MIN = 8
POOL_SIXTEENTHS = 3


def prot_units(S, R):
    return 3 * -(-(S + R) // 32) if S + R > 0 else 0


def plan(T4, P, U8, waves, pool_chunks):
    """Share boundaries of one launch: a list sbeg with share s covering tiles
    [sbeg[s], sbeg[s + 1]), plus the quantities the closed forms use."""
    weight = T4 + U8 * P
    W = min(waves, max(1, -(-weight // MIN_UNITS)))
    tp = T4 * POOL_SIXTEENTHS // 16
    cd = pool_chunks
    if cd > 0 and 2 * cd > tp:
        cd = 1 << ((tp // 2).bit_length() - 1) if tp >= 2 else 0
    if cd < POOL_MIN:
        cd = 0
    A = tp - cd if cd else 0
    Ts = T4 - (tp if cd else 0)
    balanced = (Ts + U8 * P) // W >= U8 * (-(-P // W)) + 1
    Wt = max(1, min(W, Ts))
    S0 = W if balanced else Wt

    def tbeg(w):
        return w * (Ts + U8 * P) // W - U8 * (w * P // W) if balanced else min(w, Wt) * Ts // Wt

    def cbeg(c):
        return Ts + c + A - (A * (cd - c) ** 2) // (cd * cd) if cd else Ts

    sbeg = [tbeg(s) for s in range(S0 + 1)] + [cbeg(c) for c in range(1, cd + 1)]
    return dict(W=W, S0=S0, Cd=cd, Ts=Ts, Tp=tp if cd else 0, balanced=balanced, sbeg=sbeg,
                pbeg=[w * P // W for w in range(W + 1)])


def seq_units(n, S, R, mixed=True):
    """Per sequence: INT4 (or BF16) tile count and whether it has a protected part."""
    tiles, prot = [], []
    for nb in (int(x) for x in n):
        if mixed:
            rec = max(S, nb - R)
            tiles.append(-(-rec // 32) - S // 32 if rec > S else 0)
            prot.append(1 if min(S, nb) + max(nb - rec, 0) > 0 else 0)
        else:
            tiles.append(-(-nb // 32) if nb > 0 else 0)
            prot.append(0)
    return tiles, prot


def header(n, S, R, Hkv, waves, pool_chunks, mixed=True):
    """(first, last) share of every (b, h) with tiles, the tile and protected
    counts per sequence, and the plan."""
    tiles, prot = seq_units(n, S, R, mixed)
    U8 = prot_units(int(S), int(R)) if mixed else 0
    pl = plan(sum(tiles) * Hkv, sum(prot) * Hkv, U8, waves, pool_chunks)
    sb = pl["sbeg"]

    def share_of(x):
        s = max(s for s in range(len(sb) - 1) if sb[s] <= x)
        assert sb[s] < sb[s + 1]          # the share holding x runs it
        return s

    out, x = {}, 0
    for b in range(len(n)):
        for h in range(Hkv):
            if tiles[b]:
                out[(b, h)] = (share_of(x), share_of(x + tiles[b] - 1))
            x += tiles[b]
    return out, tiles, prot, pl


def walk_share(tiles, Hkv, x, xe, touch):
    """The tile walk of one share [x, xe) as the decode kernels run it: locate
    the sequence holding tile x, then cut the share into maximal runs of one
    (b, h).  Calls touch(b) for every sequence index read and returns the runs
    (b, h, first tile, end tile).  An empty share reads nothing."""
    runs = []
    if x >= xe:
        return runs
    B = len(tiles)
    C, b = 0, 0
    while True:                                   # locate: first b whose count passes x
        touch(b)
        if C + Hkv * tiles[b] > x:
            break
        C += Hkv * tiles[b]
        b += 1
    while x < xe:
        touch(b)
        nt = tiles[b]
        r = x - C
        h, t0 = r // nt, r % nt
        base = C + h * nt
        t1 = min(nt, xe - base)
        runs.append((b, h, t0, t1))
        x = base + t1
        if x < xe and x >= C + Hkv * nt:          # next sequence with tiles
            C += Hkv * nt
            while True:
                b += 1
                if b >= B:
                    return runs
                touch(b)
                if tiles[b]:
                    break
    return runs
