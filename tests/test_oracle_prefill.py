"""Pins of the oracle's prefill attention (KV4-RL Appendix A.3: prefill and
carried-prefix reconstruction run BF16 attention over the new K/V; reading P-1
in oracle/kv4_oracle.c).

Independent routes used here:
  * the first position of a sequence attends to itself only: its output is its
    own value vector (closed form);
  * identical keys: position i's output is the mean of the values [0, i]
    (closed form);
  * each position equals the separately written (and separately pinned) dense
    decode attention of its query over its prefix;
  * causality: changing later positions' keys and values leaves earlier rows
    unchanged; packing: a batch equals its sequences run alone.
"""
import math

import numpy as np

import oracle

SCALE = 1 / math.sqrt(128)


def _bf16(a):
    from int8_mixed_precision_amd.workloads import to_bf16_values
    return to_bf16_values(np.asarray(a, dtype=np.float32))


def _case(rng, lens, Hq=8, Hkv=2, d=128):
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = _bf16(rng.standard_normal((T, Hq, d)) * 2)
    k = _bf16(rng.standard_normal((T, Hkv, d)))
    v = _bf16(rng.standard_normal((T, Hkv, d)))
    return q, k, v, cu


def test_first_position_and_identical_keys():
    rng = np.random.default_rng(70)
    q, k, v, cu = _case(rng, [1, 9, 40])
    out = oracle.prefill_attn(q, k, v, cu, SCALE)
    for b in range(3):
        t0 = cu[b]
        for j in range(8):
            assert np.array_equal(out[t0, j], v[t0, j // 4].astype(np.float64))
    k[:] = k[0:1]                                         # every key the same
    out = oracle.prefill_attn(q, k, v, cu, SCALE)
    for b in range(3):
        for t in range(cu[b], cu[b + 1]):
            mean = v[cu[b]:t + 1].astype(np.float64).mean(0)      # [Hkv, d]
            for j in range(8):
                assert np.allclose(out[t, j], mean[j // 4], rtol=0, atol=1e-12)


def test_rows_equal_dense_decode_attention_of_the_prefix():
    rng = np.random.default_rng(71)
    lens = [5, 33, 70]
    q, k, v, cu = _case(rng, lens)
    out = oracle.prefill_attn(q, k, v, cu, SCALE)
    for b in range(3):
        for t in list(range(cu[b], cu[b + 1], 7)) + [cu[b + 1] - 1]:
            want = oracle.attend_dense(q[t][None], [k[cu[b]:t + 1]], [v[cu[b]:t + 1]], SCALE)[0]
            assert np.allclose(out[t], want, rtol=0, atol=1e-13)


def test_causality_and_packing():
    rng = np.random.default_rng(72)
    lens = [17, 50]
    q, k, v, cu = _case(rng, lens)
    out = oracle.prefill_attn(q, k, v, cu, SCALE)
    k2, v2 = k.copy(), v.copy()
    k2[cu[0] + 10:cu[1]] = _bf16(rng.standard_normal(k2[cu[0] + 10:cu[1]].shape))
    v2[cu[0] + 10:cu[1]] = _bf16(rng.standard_normal(v2[cu[0] + 10:cu[1]].shape))
    out2 = oracle.prefill_attn(q, k2, v2, cu, SCALE)
    assert np.array_equal(out[:cu[0] + 10], out2[:cu[0] + 10])
    assert not np.array_equal(out[cu[0] + 10:cu[1]], out2[cu[0] + 10:cu[1]])
    for b in range(2):
        sl = slice(cu[b], cu[b + 1])
        alone = oracle.prefill_attn(q[sl], k[sl], v[sl], np.array([0, lens[b]], np.int32), SCALE)
        assert np.array_equal(alone, out[sl])
