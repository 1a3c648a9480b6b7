"""GPU parity of the prefill attention (kv4_prefill_attn; KV4-RL Appendix A.3:
BF16 attention over the newly computed K/V in prefill and carried-prefix
reconstruction) against the oracle's causal fp64 attention, through the C ABI,
at the decode's bar: max |o - o*| <= 1e-3 and row-relative 2e-3.  Packed
sequences span single positions, exact and ragged 16- and 32-position tiles and
long prompts."""
import math

import numpy as np
import pytest
import torch

import oracle
from int8_mixed_precision_amd import kv4
from int8_mixed_precision_amd import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-3, 2e-3


def _case(Hq, Hkv, lens, seed, out_dtype=kv4.KV4_OUT_F32, sm_scale=1 / math.sqrt(128)):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = W.to_bf16_values(rng.standard_normal((T, Hq, 128)).astype(np.float32) * 2)
    k = W.to_bf16_values(rng.standard_normal((T, Hkv, 128)).astype(np.float32))
    v = W.to_bf16_values(rng.standard_normal((T, Hkv, 128)).astype(np.float32))
    built = H.make_cache(Hq, Hkv, 32, 4, 16, [16], seed=seed)
    dev = torch.device("cuda")
    out = torch.empty((T, Hq, 128), dtype=torch.float32 if out_dtype == kv4.KV4_OUT_F32 else torch.bfloat16,
                      device=dev)
    kv4.kv4_prefill_attn(built.cache.handle, H.to_dev_bf16(q), H.to_dev_bf16(k), H.to_dev_bf16(v),
                         torch.from_numpy(cu).to(dev), len(lens), int(max(lens)), sm_scale,
                         out, out_dtype)
    torch.cuda.synchronize()
    want = oracle.prefill_attn(q, k, v, cu, sm_scale)
    return out.float().cpu().numpy(), want


# q head counts that are multiples of 8 take the XCD-grouped head order (at
# 32/8, 64/8 and 40/8 each XCD holds whole kv-head groups); 12/3 keeps the
# launch order; ratios 3, 5 and 16 as well as powers of two
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 8), (8, 8), (16, 2), (12, 3), (64, 8), (40, 8), (64, 4)])
def test_prefill_matches_oracle(Hq, Hkv):
    lens = [1, 15, 16, 17, 31, 32, 33, 100, 257, 600]
    H.log(f"case prefill Hq={Hq} Hkv={Hkv} lens={lens}")
    out, want = _case(Hq, Hkv, lens, seed=200 + Hq + Hkv)
    err = H.check_output(out, want, ATOL, RTOL)
    H.log(f"  max abs {err[0]:.2e} row rel {err[1]:.2e}")


def test_prefill_scales():
    """A negative, a large, a small and a zero softmax scale (the kernel takes
    the scale's sign into the query operand and compares raw scores; a zero
    scale is the uniform average of every prefix)."""
    for sc in (-1 / math.sqrt(128), 4 / math.sqrt(128), 1e-3, 0.0):
        H.log(f"case prefill sm_scale {sc:.4g}")
        out, want = _case(8, 2, [1, 33, 200, 700], seed=230, sm_scale=sc)
        err = H.check_output(out, want, ATOL, RTOL)
        H.log(f"  max abs {err[0]:.2e} row rel {err[1]:.2e}")


def test_prefill_long_prompt_and_bf16_output():
    H.log("case prefill long prompt 2048 + 5, bf16 output")
    out32, want = _case(32, 8, [2048, 5], seed=210)
    H.check_output(out32, want, ATOL, RTOL)
    outb, _ = _case(32, 8, [2048, 5], seed=210, out_dtype=kv4.KV4_OUT_BF16)
    ref = torch.from_numpy(out32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(outb, ref)


@pytest.mark.timeout(600)
def test_prefill_16k_prompt_sampled_rows():
    """Prompts as long as the benchmark's (16,384 tokens, packed with a 3,000-
    and a 7-token one): sampled rows -- the first and last of each prompt, tile
    and block boundaries, random ones -- against the oracle's fp64 dense
    attention of that row's query over its prefix [0, t] (row t of a causal
    prefill is exactly that)."""
    Hq, Hkv = 32, 8
    lens = [16384, 3000, 7]
    H.log(f"case prefill 16k prompt: lens {lens}, sampled rows")
    rng = np.random.default_rng(220)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = W.to_bf16_values(rng.standard_normal((T, Hq, 128)).astype(np.float32) * 2)
    k = W.to_bf16_values(rng.standard_normal((T, Hkv, 128)).astype(np.float32))
    v = W.to_bf16_values(rng.standard_normal((T, Hkv, 128)).astype(np.float32))
    built = H.make_cache(Hq, Hkv, 32, 4, 16, [16], seed=220)
    dev = torch.device("cuda")
    out = torch.empty((T, Hq, 128), dtype=torch.float32, device=dev)
    kv4.kv4_prefill_attn(built.cache.handle, H.to_dev_bf16(q), H.to_dev_bf16(k), H.to_dev_bf16(v),
                         torch.from_numpy(cu).to(dev), len(lens), int(max(lens)), 1 / math.sqrt(128),
                         out, kv4.KV4_OUT_F32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    rows = []
    for b, n in enumerate(lens):
        fixed = [0, 1, 15, 16, 31, 32, 127, 128, 129, 4095, 4096, 8191, 12000, n - 2, n - 1]
        picks = set(t for t in fixed if 0 <= t < n)
        picks |= set(int(t) for t in rng.integers(0, n, size=12 if n > 100 else n))
        rows += [(b, t) for t in sorted(picks)]
    for i in range(0, len(rows), 16):
        chunk = rows[i:i + 16]
        idx = [int(cu[b]) + t for b, t in chunk]
        ks = [k[cu[b]:cu[b] + t + 1] for b, t in chunk]
        vs = [v[cu[b]:cu[b] + t + 1] for b, t in chunk]
        want = oracle.attend_dense(q[idx], ks, vs, 1 / math.sqrt(128))
        err = H.check_output(got[idx], want, ATOL, RTOL)
    H.log(f"  {len(rows)} sampled rows within the bar (last chunk max abs {err[0]:.2e})")
