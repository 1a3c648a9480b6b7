"""fp64 CPU oracle for the KV4 decode step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it, and
it shares no code with the HIP kernels.  It wraps ``kv4_oracle.c`` (plain C,
fp64, OpenMP over independent output rows) through ctypes.

Method: KV4-RL (arXiv 2610.14448) -- affine INT4 x^ = Delta*c + m (Section 3,
eq. 3.3) with FP16 Delta and m per channel group (Section 5.1; Appendix A.3;
Appendix D.4, Fig. A4b); symmetric per-token-head INT8 side copies of the sink
and recent positions (Section 5.2; Appendix A.3); exact softmax attention over
the dequantized cache (the merge of eq. A1 reaches the same result).

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, exact rational brute force, numpy's own binary16 conversion and
invariants; see the test docstrings for which pin covers which function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kv4_oracle.c")
_LIB = os.path.join(_HERE, "libkv4_oracle.so")
# a separately built oracle library to load instead (for example the
# sanitizer build of tests/sanitize_cpu.py); it is then not rebuilt here
_LIB_OVERRIDE = os.environ.get("KV4_ORACLE_LIB", "")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-shared", "-fPIC", "-Wall", "-Wno-unknown-pragmas"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build(force=False)                  # (re)builds when missing or older than the source
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = dbl
        L.orc_f32_to_f16_array.argtypes = [P, P, i64]
        L.orc_f16_to_f64_array.argtypes = [P, P, i64]
        L.orc_quant_int4.argtypes = [P, i64, i32, i32, P, P, P]
        L.orc_quant_int8.argtypes = [P, i64, i32, P, P]
        L.orc_wht_f32.argtypes = [P, i64, i32, P]
        L.orc_wht_scale.argtypes = [i32]
        L.orc_wht_scale.restype = ctypes.c_float
        L.orc_is_protected.argtypes = [i64, i64, i32, i32]
        L.orc_is_protected.restype = i32
        L.orc_attend_mixed.argtypes = [i32, P, P, i32, i32, i32, i32, i32, i32, dbl, P,
                                       P, P, P, P, P, P, P, P, P, P, P]
        L.orc_attend_dense.argtypes = [i32, P, P, i32, i32, i32, dbl, P, P, P, P]
        L.orc_prefill_attn.argtypes = [i32, P, i32, i32, i32, dbl, P, P, P, P]
        L.orc_attend_int.argtypes = [i32, P, P, i32, i32, i32, i32, i32, i32, dbl, P,
                                     P, P, P, P, P, P, P, P, P, P, dbl, P, P]
        L.orc_num_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().orc_num_threads())


# --------------------------------------------------------------------------
# binary16
# --------------------------------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    """Round binary32 values to binary16 (nearest, ties to even); bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_f64(h) -> np.ndarray:
    """Exact binary64 values of binary16 bit patterns."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.float64)
    lib().orc_f16_to_f64_array(_ptr(h), _ptr(out), h.size)
    return out


# --------------------------------------------------------------------------
# quantizers (Q-1 .. Q-4)
# --------------------------------------------------------------------------

def quant_int4(x, G: int):
    """INT4 of vectors x[..., d] (float32 holding bf16 values).

    Returns (codes uint8 [..., d], delta uint16 [..., d/G], offs uint16 [..., d/G])
    where delta/offs are binary16 bit patterns of Delta and m (eq. 3.3).
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    d = x.shape[-1]
    assert d % G == 0
    nvec = x.size // d
    codes = np.empty(x.shape, dtype=np.uint8)
    delta = np.empty(x.shape[:-1] + (d // G,), dtype=np.uint16)
    offs = np.empty_like(delta)
    lib().orc_quant_int4(_ptr(x), nvec, d, G, _ptr(codes), _ptr(delta), _ptr(offs))
    return codes, delta, offs


def quant_int8(x):
    """Symmetric INT8 of vectors x[..., d]; returns (codes int8, scale uint16 [...])."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    d = x.shape[-1]
    nvec = x.size // d
    codes = np.empty(x.shape, dtype=np.int8)
    scale = np.empty(x.shape[:-1], dtype=np.uint16)
    lib().orc_quant_int8(_ptr(x), nvec, d, _ptr(codes), _ptr(scale))
    return codes, scale


def dequant_int4(codes, delta, offs, G: int) -> np.ndarray:
    """x^ = Delta*c + m in binary64 (eq. 3.3)."""
    D = np.repeat(f16_bits_to_f64(delta), G, axis=-1)
    M = np.repeat(f16_bits_to_f64(offs), G, axis=-1)
    return D * codes.astype(np.float64) + M


def dequant_int8(codes, scale) -> np.ndarray:
    return f16_bits_to_f64(scale)[..., None] * codes.astype(np.float64)


def wht(x) -> np.ndarray:
    """The fixed normalized Hadamard transform y = x H / sqrt(d) of vectors
    x[..., d] (KV4-RL Section 5.1; Appendix A.3), in binary32 in the order of
    reading R-10: butterfly stages of span 1, 2, ..., d/2, then one product
    with the binary32 value nearest 1/sqrt(d)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    d = x.shape[-1]
    assert d & (d - 1) == 0 and d <= 1024
    y = np.empty_like(x)
    lib().orc_wht_f32(_ptr(x), x.size // d, d, _ptr(y))
    return y


def wht_scale(d: int) -> float:
    return float(lib().orc_wht_scale(d))


def is_protected(p: int, n: int, S: int, R: int) -> bool:
    return bool(lib().orc_is_protected(p, n, S, R))


# --------------------------------------------------------------------------
# cache state and attention (Q-5, Q-6)
# --------------------------------------------------------------------------

class MixedCache:
    """Dense per-position quantized state of a batch of sequences.

    ``k_src[b]``/``v_src[b]`` are float32 arrays [n_b, Hkv, d] of bf16 source
    values (post-RoPE keys, values).  Every position gets its INT4 encoding
    and its INT8 encoding, both from the source vector; which one attention
    reads is decided by the position's region at attention time.
    """

    def __init__(self, k_src, v_src, G: int, protect=None, rotate: bool = False):
        """``protect=(S, R)`` computes the INT8 copies only of positions that
        are protected at the stored length (others stay zero); the default
        computes them for every position, so any prefix can be attended.
        ``rotate`` stores the keys in the rotated basis (R-10): both the INT4
        and the INT8 copy are computed from wht(k); values stay as they are."""
        self.G = G
        self.seq_lens = np.array([k.shape[0] for k in k_src], dtype=np.int32)
        self.pos_off = np.zeros(len(k_src), dtype=np.int64)
        if len(k_src) > 1:
            self.pos_off[1:] = np.cumsum(self.seq_lens[:-1])
        K = np.ascontiguousarray(np.concatenate([np.asarray(k, np.float32) for k in k_src], 0))
        V = np.ascontiguousarray(np.concatenate([np.asarray(v, np.float32) for v in v_src], 0))
        self.Hkv, self.d = K.shape[1], K.shape[2]
        self.rotate = rotate
        if rotate:
            K = wht(K)
        self.k4, self.k4d, self.k4m = quant_int4(K, G)
        self.v4, self.v4d, self.v4m = quant_int4(V, G)
        if protect is None:
            self.k8, self.k8s = quant_int8(K)
            self.v8, self.v8s = quant_int8(V)
        else:
            S, R = protect
            rows = np.concatenate([
                o + np.nonzero([is_protected(p, n, S, R) for p in range(n)])[0]
                for o, n in zip(self.pos_off, self.seq_lens)]).astype(np.int64)
            self.k8 = np.zeros(K.shape, np.int8)
            self.v8 = np.zeros(V.shape, np.int8)
            self.k8s = np.zeros(K.shape[:2], np.uint16)
            self.v8s = np.zeros(V.shape[:2], np.uint16)
            if rows.size:
                self.k8[rows], self.k8s[rows] = quant_int8(K[rows])
                self.v8[rows], self.v8s[rows] = quant_int8(V[rows])

    def seq(self, b: int):
        """Row slice of sequence b."""
        o = int(self.pos_off[b])
        return slice(o, o + int(self.seq_lens[b]))


def attend_mixed(q, cache: MixedCache, S: int, R: int, sm_scale: float,
                 seq_lens=None) -> np.ndarray:
    """fp64 softmax attention of q [B, Hq, d] over the mixed cache.

    ``seq_lens`` (default: the cache's lengths) may be shorter than the stored
    rows to attend over a prefix of each sequence.
    """
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    B, Hq, d = q.shape
    sl = cache.seq_lens if seq_lens is None else np.ascontiguousarray(np.asarray(seq_lens, np.int32))
    assert np.all(sl <= cache.seq_lens)
    out = np.empty((B, Hq, d), dtype=np.float64)
    c = cache
    lib().orc_attend_mixed(B, _ptr(sl), _ptr(c.pos_off), Hq, c.Hkv, d, c.G, S, R,
                           float(sm_scale), _ptr(q),
                           _ptr(c.k4), _ptr(c.k4d), _ptr(c.k4m),
                           _ptr(c.v4), _ptr(c.v4d), _ptr(c.v4m),
                           _ptr(c.k8), _ptr(c.k8s), _ptr(c.v8), _ptr(c.v8s),
                           _ptr(out))
    return out


def attend_int(q, cache: MixedCache, S: int, R: int, sm_scale: float, eps: float = 2.0 ** -6,
               seq_lens=None):
    """The integer decode path (KV4-RL Appendix A.3; readings I-1 .. I-6 in
    kv4_oracle.c): INT8 q per (sequence, q head), integer QK with the affine
    fold, binary64 softmax, an 8-bit probability operand per (8-position block,
    value group, q head) for the INT4 values, full-precision PV for the
    protected ones.  Returns (out, bound), both float64 [B, Hq, d]; bound is the
    largest change of out if every code within eps of a rounding tie moved by
    one.  q must already be in the keys' basis when the cache is rotated."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    B, Hq, d = q.shape
    sl = cache.seq_lens if seq_lens is None else np.ascontiguousarray(np.asarray(seq_lens, np.int32))
    assert np.all(sl <= cache.seq_lens)
    out = np.empty((B, Hq, d), dtype=np.float64)
    bound = np.empty((B, Hq, d), dtype=np.float64)
    c = cache
    lib().orc_attend_int(B, _ptr(sl), _ptr(c.pos_off), Hq, c.Hkv, d, c.G, S, R,
                         float(sm_scale), _ptr(q),
                         _ptr(c.k4), _ptr(c.k4d), _ptr(c.k4m),
                         _ptr(c.v4), _ptr(c.v4d), _ptr(c.v4m),
                         _ptr(c.k8), _ptr(c.k8s), _ptr(c.v8), _ptr(c.v8s),
                         float(eps), _ptr(out), _ptr(bound))
    return out, bound


def prefill_attn(q, k, v, cu, sm_scale: float) -> np.ndarray:
    """Causal fp64 attention of every packed position over its sequence's
    prefix (reading P-1 in kv4_oracle.c): q [T, Hq, d], k, v [T, Hkv, d] (bf16
    values in float32), cu [B + 1] row offsets.  Returns float64 [T, Hq, d]."""
    q = np.ascontiguousarray(np.asarray(q, np.float32))
    k = np.ascontiguousarray(np.asarray(k, np.float32))
    v = np.ascontiguousarray(np.asarray(v, np.float32))
    cu = np.ascontiguousarray(np.asarray(cu, np.int32))
    T, Hq, d = q.shape
    assert int(cu[-1]) == T and k.shape == v.shape and k.shape[0] == T
    out = np.empty((T, Hq, d), dtype=np.float64)
    lib().orc_prefill_attn(len(cu) - 1, _ptr(cu), Hq, k.shape[1], d, float(sm_scale),
                           _ptr(q), _ptr(k), _ptr(v), _ptr(out))
    return out


def attend_mixed_raw(q, seq_lens, pos_off, Hkv, G, S, R, sm_scale,
                     k4, k4d, k4m, v4, v4d, v4m, k8, k8s, v8, v8s) -> np.ndarray:
    """Same as :func:`attend_mixed` on explicitly given representation arrays
    (used by tests that hand-build inconsistent INT4/INT8 copies)."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    B, Hq, d = q.shape
    arrs = [np.ascontiguousarray(a) for a in (k4, k4d, k4m, v4, v4d, v4m, k8, k8s, v8, v8s)]
    sl = np.ascontiguousarray(np.asarray(seq_lens, np.int32))
    po = np.ascontiguousarray(np.asarray(pos_off, np.int64))
    out = np.empty((B, Hq, d), dtype=np.float64)
    lib().orc_attend_mixed(B, _ptr(sl), _ptr(po), Hq, Hkv, d, G, S, R, float(sm_scale),
                           _ptr(q), *[_ptr(a) for a in arrs], _ptr(out))
    return out


def attend_dense(q, k_src, v_src, sm_scale: float) -> np.ndarray:
    """fp64 softmax attention over unquantized (bf16) keys and values."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    B, Hq, d = q.shape
    sl = np.array([k.shape[0] for k in k_src], dtype=np.int32)
    po = np.zeros(B, dtype=np.int64)
    if B > 1:
        po[1:] = np.cumsum(sl[:-1])
    K = np.ascontiguousarray(np.concatenate([np.asarray(k, np.float32) for k in k_src], 0))
    V = np.ascontiguousarray(np.concatenate([np.asarray(v, np.float32) for v in v_src], 0))
    out = np.empty((B, Hq, d), dtype=np.float64)
    lib().orc_attend_dense(B, _ptr(sl), _ptr(po), Hq, K.shape[1], d, float(sm_scale),
                           _ptr(q), _ptr(K), _ptr(V), _ptr(out))
    return out
