"""The decode partition's tile walk on the host (tests/partition.py mirrors
the kernels' closed forms and walk): every share reads only sequence indices
inside the batch -- also when no sequence has INT4 tiles, where every share is
empty -- and the runs of all shares cover every (sequence, kv head, tile)
exactly once."""
import numpy as np
import pytest

from tests import partition as PT


def _check(n, S, R, Hkv, waves, pool):
    tiles, prot = PT.seq_units(n, S, R)
    pl = PT.plan(sum(tiles) * Hkv, sum(prot) * Hkv, PT.prot_units(S, R), waves, pool)
    sb = pl["sbeg"]
    B = len(n)
    seen = []

    def touch(b):
        assert 0 <= b < B, f"sequence index {b} outside batch {B}"
        seen.append(b)

    cover = {}
    for s in range(len(sb) - 1):
        for b, h, t0, t1 in PT.walk_share(tiles, Hkv, sb[s], sb[s + 1], touch):
            assert 0 <= h < Hkv and 0 <= t0 < t1 <= tiles[b]
            for t in range(t0, t1):
                key = (b, h, t)
                assert key not in cover, key
                cover[key] = s
    assert len(cover) == sum(tiles) * Hkv
    return pl


@pytest.mark.parametrize("S,R", [(4, 128), (0, 64), (16, 3), (4, 0)])
def test_all_protected_batches_read_inside_the_batch(S, R):
    rng = np.random.default_rng(S * 7 + R)
    for B in (1, 2, 5, 64):
        n = rng.integers(1, max(2, S + R + 1), size=B)
        n = np.minimum(n, max(1, S + R))           # every position protected: no INT4 tile
        for waves in (1, 7, 4096):
            pl = _check(n, S, R, 8, waves, 0)
            if S + R > 0:
                assert pl["Ts"] == 0


@pytest.mark.parametrize("waves,pool", [(1, 0), (7, 0), (64, 16), (4096, 0), (5000, 0), (256, 4096)])
def test_walk_covers_every_tile_once(waves, pool):
    rng = np.random.default_rng(waves + pool)
    for _ in range(6):
        B = int(rng.integers(1, 40))
        n = rng.integers(1, 3000, size=B)
        n[rng.integers(B)] = 1                     # a one-token sequence
        _check(n, 4, 128, 8, waves, pool)
        _check(n, 0, 0, 2, waves, pool)
