"""Pins of the oracle's attention and region rule.

KV4-RL: protected positions (the first s and the w most recent, Section 5.2)
are read from the INT8 side copy and all others from INT4, as disjoint
regions (Section 5.3); attention is exact softmax over the dequantized cache
(the regional merge, eq. A1 of Appendix A.3, reaches the same result).

Pins (none re-derives the oracle's own loop):
  * region rule: closed-form counts and the disjoint-union property for the
    boundary cases n <= S, n = S+R, n = S+R+1, R = 0, S = 0;
  * region membership of *every* position, read back through attention with
    hand-built inconsistent copies (INT8 copy = e_p, INT4 copy = 3 e_p);
  * q = 0 (or sm_scale = 0): output = mean of the dequantized values;
  * n = 1: output = the only value; n = 2: logistic closed form;
  * one dominant key: output -> that key's value;
  * GQA grouping: q head j reads kv head j // (Hq/Hkv);
  * invariances: (a*q, sm_scale/a) gives the same output; permuting INT4
    positions leaves the output unchanged;
  * dense (BF16 comparator) attention: the same closed forms.
"""
import math

import numpy as np
import pytest

import oracle


def _bf16(a):
    from int8_mixed_precision_amd.workloads import to_bf16_values
    return to_bf16_values(np.asarray(a, dtype=np.float32))


def _count_protected(n, S, R):
    return min(S, n) + min(R, max(n - S, 0))


@pytest.mark.parametrize("S", [0, 1, 4, 16])
@pytest.mark.parametrize("R", [0, 1, 3, 8, 64])
def test_region_rule_counts(S, R):
    for n in range(1, 100):
        prot = [oracle.is_protected(p, n, S, R) for p in range(n)]
        assert sum(prot) == _count_protected(n, S, R)
        # the first min(S, n) are protected
        assert all(prot[:min(S, n)])
        # the last min(R, n - S) are protected; everything between is INT4
        k = min(R, max(n - S, 0))
        assert all(prot[n - k:])
        assert not any(prot[min(S, n):n - k])
    # S = R = 0 -> pure INT4; S + R >= n -> pure INT8
    assert not any(oracle.is_protected(p, 50, 0, 0) for p in range(50))
    assert all(oracle.is_protected(p, 50, 20, 30) for p in range(50))


def _raw_cache(n, Hkv, d, G, rng):
    """Random representation arrays for one sequence of n positions."""
    ng = d // G
    k4 = rng.integers(0, 16, size=(n, Hkv, d)).astype(np.uint8)
    v4 = rng.integers(0, 16, size=(n, Hkv, d)).astype(np.uint8)
    f16 = lambda a: np.asarray(a, np.float16).view(np.uint16)
    k4d = f16(rng.uniform(0.05, 0.3, size=(n, Hkv, ng)))
    v4d = f16(rng.uniform(0.05, 0.3, size=(n, Hkv, ng)))
    k4m = f16(rng.uniform(-2, -0.5, size=(n, Hkv, ng)))
    v4m = f16(rng.uniform(-2, -0.5, size=(n, Hkv, ng)))
    k8 = rng.integers(-127, 128, size=(n, Hkv, d)).astype(np.int8)
    v8 = rng.integers(-127, 128, size=(n, Hkv, d)).astype(np.int8)
    k8s = f16(rng.uniform(0.005, 0.02, size=(n, Hkv)))
    v8s = f16(rng.uniform(0.005, 0.02, size=(n, Hkv)))
    return [k4, k4d, k4m, v4, v4d, v4m, k8, k8s, v8, v8s]


def _dequant_seq(arrs, n, S, R, G):
    """Dequantized K and V per the region rule (binary64)."""
    k4, k4d, k4m, v4, v4d, v4m, k8, k8s, v8, v8s = arrs
    K4 = oracle.dequant_int4(k4, k4d, k4m, G)
    V4 = oracle.dequant_int4(v4, v4d, v4m, G)
    K8 = oracle.dequant_int8(k8, k8s)
    V8 = oracle.dequant_int8(v8, v8s)
    prot = np.array([oracle.is_protected(p, n, S, R) for p in range(n)])[:, None, None]
    return np.where(prot, K8, K4), np.where(prot, V8, V4)


@pytest.mark.parametrize("S,R", [(0, 0), (4, 64), (16, 3), (1, 0), (0, 5), (50, 50)])
def test_region_membership_every_position(S, R):
    d, Hkv, G = 128, 1, 32
    for n in (1, 3, 4, 5, 10, 67, 68, 69, 100, 127):
        arrs = [np.zeros((n, Hkv, d), np.uint8), np.zeros((n, Hkv, 4), np.uint16),
                np.zeros((n, Hkv, 4), np.uint16), np.zeros((n, Hkv, d), np.uint8),
                np.full((n, Hkv, 4), 0x3C00, np.uint16), np.zeros((n, Hkv, 4), np.uint16),
                np.zeros((n, Hkv, d), np.int8), np.zeros((n, Hkv), np.uint16),
                np.zeros((n, Hkv, d), np.int8), np.full((n, Hkv), 0x3C00, np.uint16)]
        # INT8 copy of position p: scale 1, code +1 at channel p % d (value 1);
        # INT4 copy: Delta 1, offset 0, code 3 at channel p % d (value 3).
        v4, v8 = arrs[3], arrs[8]
        for p in range(n):
            v8[p, 0, p % d] = 1
            v4[p, 0, p % d] = 3
        q = np.zeros((1, 1, d), np.float32)
        out = oracle.attend_mixed_raw(q, [n], [0], Hkv, G, S, R, 0.1, *arrs)[0, 0]
        # each position contributes 1/n * (1 if protected else 3) at channel p%d
        want = np.zeros(d)
        for p in range(n):
            want[p % d] += (1.0 if oracle.is_protected(p, n, S, R) else 3.0) / n
        assert np.allclose(out, want, rtol=0, atol=1e-14), (n, S, R)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_uniform_query_gives_mean_value(G):
    rng = np.random.default_rng(1)
    n, Hq, Hkv, d, S, R = 77, 8, 2, 128, 4, 16
    arrs = _raw_cache(n, Hkv, d, G, rng)
    K, V = _dequant_seq(arrs, n, S, R, G)
    q = np.zeros((1, Hq, d), np.float32)
    out = oracle.attend_mixed_raw(q, [n], [0], Hkv, G, S, R, 0.088, *arrs)
    for j in range(Hq):
        assert np.allclose(out[0, j], V[:, j // (Hq // Hkv)].mean(0), rtol=0, atol=1e-13)
    # sm_scale = 0 with a nonzero query also gives the mean
    q2 = _bf16(rng.standard_normal((1, Hq, d)))
    out2 = oracle.attend_mixed_raw(q2, [n], [0], Hkv, G, S, R, 0.0, *arrs)
    assert np.allclose(out2, out, rtol=0, atol=1e-13)
    # GQA grouping: the two kv heads have different means, heads 0-3 read kv 0
    assert not np.allclose(V[:, 0].mean(0), V[:, 1].mean(0))


def test_single_and_two_positions_closed_form():
    rng = np.random.default_rng(4)
    Hq, Hkv, d, G = 4, 1, 128, 32
    for S, R in ((0, 0), (1, 0), (0, 1), (4, 128)):
        arrs = _raw_cache(1, Hkv, d, G, rng)
        K, V = _dequant_seq(arrs, 1, S, R, G)
        q = _bf16(rng.standard_normal((1, Hq, d)))
        out = oracle.attend_mixed_raw(q, [1], [0], Hkv, G, S, R, 0.2, *arrs)
        assert np.allclose(out[0], np.broadcast_to(V[0, 0], (Hq, d)), rtol=0, atol=1e-14)
        arrs = _raw_cache(2, Hkv, d, G, rng)
        K, V = _dequant_seq(arrs, 2, S, R, G)
        sm = 0.1
        out = oracle.attend_mixed_raw(q, [2], [0], Hkv, G, S, R, sm, *arrs)
        for j in range(Hq):
            s0 = sm * float(np.dot(q[0, j].astype(np.float64), K[0, 0]))
            s1 = sm * float(np.dot(q[0, j].astype(np.float64), K[1, 0]))
            w1 = 1.0 / (1.0 + math.exp(s0 - s1))                  # logistic
            want = (1 - w1) * V[0, 0] + w1 * V[1, 0]
            assert np.allclose(out[0, j], want, rtol=0, atol=1e-12)


def test_dominant_key():
    rng = np.random.default_rng(6)
    n, Hq, Hkv, d, G, S, R = 60, 4, 1, 128, 32, 4, 8
    for star in (2, 30, 57):                       # sink, INT4 and recent positions
        arrs = _raw_cache(n, Hkv, d, G, rng)
        k4, k4d, k4m, v4, v4d, v4m, k8, k8s, v8, v8s = arrs
        q = np.zeros((1, Hq, d), np.float32)
        q[0, :, 0] = 64.0
        # make key 'star' large on channel 0 in whichever copy it is read from
        # channel 0 of every other key: code 0 (INT4: value m < 0; INT8: value 0)
        k4[:, 0, 0] = 0
        k8[:, 0, 0] = 0
        if oracle.is_protected(star, n, S, R):
            k8[star, 0, 0] = 127
        else:
            k4[star, 0, 0] = 15
            k4d[star, 0, 0] = np.float16(0.3).view(np.uint16)
            k4m[star, 0, 0] = 0
        K, V = _dequant_seq(arrs, n, S, R, G)
        assert np.argmax(K[:, 0, 0]) == star
        gap = 64.0 * (K[star, 0, 0] - np.sort(K[:, 0, 0])[-2])
        sm = 50.0 / gap                              # score gap of 50 nats
        out = oracle.attend_mixed_raw(q, [n], [0], Hkv, G, S, R, sm, *arrs)
        bound = n * math.exp(-50.0) * np.abs(V).max() * 2
        assert np.abs(out[0] - V[star, 0]).max() <= bound + 1e-15


def test_scale_invariance_and_permutation():
    rng = np.random.default_rng(8)
    n, Hq, Hkv, d, G, S, R = 90, 8, 2, 128, 32, 4, 16
    arrs = _raw_cache(n, Hkv, d, G, rng)
    q = _bf16(rng.standard_normal((1, Hq, d)))
    a = 4.0                                          # power of two keeps q bf16-exact
    o1 = oracle.attend_mixed_raw(q, [n], [0], Hkv, G, S, R, 0.125, *arrs)
    o2 = oracle.attend_mixed_raw((q * a).astype(np.float32), [n], [0], Hkv, G, S, R,
                                 0.125 / a, *arrs)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)
    # permute the INT4 positions [S, n - R)
    perm = np.arange(n)
    mid = perm[S:n - R].copy()
    rng.shuffle(mid)
    perm[S:n - R] = mid
    arrs_p = [a_[perm] for a_ in arrs]
    o3 = oracle.attend_mixed_raw(q, [n], [0], Hkv, G, S, R, 0.125, *arrs_p)
    assert np.allclose(o1, o3, rtol=0, atol=1e-12)
    # swapping a protected and an INT4 position's data changes the result
    arrs_s = [a_.copy() for a_ in arrs]
    for a_ in arrs_s:
        a_[[1, 40]] = a_[[40, 1]]
    o4 = oracle.attend_mixed_raw(q, [n], [0], Hkv, G, S, R, 0.125, *arrs_s)
    assert not np.allclose(o1, o4, rtol=0, atol=1e-6)


def test_batch_rows_are_independent():
    rng = np.random.default_rng(12)
    Hq, Hkv, d, G, S, R = 8, 2, 128, 32, 4, 8
    lens = [5, 40, 17]
    per = [_raw_cache(n, Hkv, d, G, rng) for n in lens]
    q = _bf16(rng.standard_normal((3, Hq, d)))
    cat = [np.concatenate([p[i] for p in per], 0) for i in range(10)]
    off = np.array([0, 5, 45])
    out = oracle.attend_mixed_raw(q, lens, off, Hkv, G, S, R, 0.09, *cat)
    for b, n in enumerate(lens):
        ob = oracle.attend_mixed_raw(q[b:b + 1], [n], [0], Hkv, G, S, R, 0.09, *per[b])
        assert np.array_equal(out[b], ob[0])


def test_mixed_cache_from_sources():
    """End to end through MixedCache: all-protected equals attention over INT8
    reconstructions, S=R=0 equals attention over INT4 reconstructions."""
    rng = np.random.default_rng(13)
    n, Hq, Hkv, d, G = 50, 4, 1, 128, 32
    k = _bf16(rng.standard_normal((n, Hkv, d)))
    v = _bf16(rng.standard_normal((n, Hkv, d)))
    q = _bf16(rng.standard_normal((1, Hq, d)))
    c = oracle.MixedCache([k], [v], G)
    sm = 1 / math.sqrt(d)
    o8 = oracle.attend_mixed(q, c, S=20, R=40, sm_scale=sm)
    K8 = oracle.dequant_int8(c.k8, c.k8s)
    V8 = oracle.dequant_int8(c.v8, c.v8s)
    o8d = oracle.attend_dense(q, [K8.astype(np.float32)], [V8.astype(np.float32)], sm)
    # the dense routine takes float32 inputs; the int8 reconstructions are
    # exact in float32 (8-bit code times an fp16 scale)
    assert np.allclose(o8, o8d, rtol=0, atol=1e-12)
    o4 = oracle.attend_mixed(q, c, S=0, R=0, sm_scale=sm)
    K4 = oracle.dequant_int4(c.k4, c.k4d, c.k4m, G)
    V4 = oracle.dequant_int4(c.v4, c.v4d, c.v4m, G)
    assert np.array_equal(K4.astype(np.float32).astype(np.float64), K4)
    o4d = oracle.attend_dense(q, [K4.astype(np.float32)], [V4.astype(np.float32)], sm)
    assert np.allclose(o4, o4d, rtol=0, atol=1e-12)
    # quantized output stays close to the unquantized one (sanity, loose)
    od = oracle.attend_dense(q, [k], [v], sm)
    assert np.abs(o4 - od).max() < 0.2


def test_dense_closed_forms():
    rng = np.random.default_rng(14)
    n, Hq, Hkv, d = 33, 8, 2, 128
    k = _bf16(rng.standard_normal((n, Hkv, d)))
    v = _bf16(rng.standard_normal((n, Hkv, d)))
    q = np.zeros((1, Hq, d), np.float32)
    out = oracle.attend_dense(q, [k], [v], 0.3)
    for j in range(Hq):
        assert np.allclose(out[0, j], v[:, j // 4].astype(np.float64).mean(0), rtol=0, atol=1e-13)
    q = _bf16(rng.standard_normal((1, Hq, d)))
    out = oracle.attend_dense(q, [k[:2]], [v[:2]], 0.05)
    for j in range(Hq):
        h = j // 4
        s0 = 0.05 * float(np.dot(q[0, j].astype(np.float64), k[0, h].astype(np.float64)))
        s1 = 0.05 * float(np.dot(q[0, j].astype(np.float64), k[1, h].astype(np.float64)))
        w1 = 1 / (1 + math.exp(s0 - s1))
        want = (1 - w1) * v[0, h].astype(np.float64) + w1 * v[1, h].astype(np.float64)
        assert np.allclose(out[0, j], want, rtol=0, atol=1e-12)
