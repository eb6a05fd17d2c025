"""fp8 (OCP E4M3) quantised KV cache: plain fp64 CPU reference.

TEST INFRASTRUCTURE ONLY (see ``oracle/paged_attention.py``).

The pages only name the feature: ember, "Deliberately out of scope (for now)",
lists paged KV quantisation (fp8/int8) as a next step.  Everything below is
a reading of that one line (format, scales, rounding):

* format: OCP 8-bit floating point, E4M3 with the "fn" encoding (1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
  NaN; largest finite magnitude 448; subnormals m/8 * 2^-6);
* one fp32 scale per KV head and per pool (``k_scale[h]``, ``v_scale[h]``):
  an element x of KV head h is stored as ``encode(fp32(x / scale[h]))`` and
  read back as ``decode(code) * scale[h]``;
* ``fp32(x / s)`` is the correctly rounded fp32 quotient (IEEE division of
  the fp32 values);
* encode rounds to nearest, ties to even, and saturates: a finite magnitude
  above 448 (and infinity) becomes +-448; NaN becomes the NaN code 0x7F.

Attention over an fp8 pool is attention over the dequantised pool, computed
in fp64 by ``ref_decode``/``ref_prefill`` (they accept fp64 pools).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import widen

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "ref_quantize", "ref_dequantize",
           "ref_reshape_and_cache_fp8"]

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 codes (uint8)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


def _round_half_even(x: np.ndarray) -> np.ndarray:
    """Nearest integer, ties to the even one (x >= 0, exact in fp64)."""
    f = np.floor(x)
    d = x - f
    up = (d > 0.5) | ((d == 0.5) & (np.mod(f, 2.0) == 1.0))
    return f + up


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes (uint8) of fp64 values: round to nearest even, saturate at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    out = np.zeros(x.shape, dtype=np.int64)
    nan = np.isnan(x)
    big = ~nan & (a > E4M3_MAX)
    sub = ~nan & ~big & (a < 2.0 ** -6)
    nrm = ~nan & ~big & ~sub
    # subnormal grid: multiples of 2^-9 (m = 8 is the smallest normal, code 0x08)
    out[sub] = _round_half_even(a[sub] * 2.0 ** 9).astype(np.int64)
    # normal: a = 2^e (1 + f), 3 fraction bits
    mant, exp = np.frexp(a[nrm])           # a = mant * 2^exp, mant in [0.5, 1)
    e = exp.astype(np.int64) - 1
    frac = mant * 2.0 - 1.0                # in [0, 1)
    r = _round_half_even(frac * 8.0).astype(np.int64)
    carry = r == 8
    r[carry] = 0
    e[carry] += 1
    code = ((e + 7) << 3) | r
    out[nrm] = np.minimum(code, 0x7E)      # 480 would be the NaN pattern: saturate
    out[big] = 0x7E
    out = out | sign
    out[nan] = 0x7F
    return out.astype(np.uint8)


def ref_quantize(x, scale) -> np.ndarray:
    """Codes of ``x [..., H_kv, D]`` (bf16 bits or fp32) with per-head ``scale [H_kv]``."""
    xv = widen(x).astype(np.float32)
    s = np.asarray(scale, dtype=np.float32)
    assert s.shape == (xv.shape[-2],) and np.all(s > 0)
    q = (xv.astype(np.float64) / s.astype(np.float64)[:, None]).astype(np.float32)
    return e4m3_encode(q.astype(np.float64))


def ref_dequantize(codes, scale) -> np.ndarray:
    """fp64 values of an fp8 pool or token block ``[..., H_kv, D]``."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return e4m3_decode(codes) * s[:, None]


def ref_reshape_and_cache_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Quantise this step's keys/values and scatter the codes into copies of the
    uint8 pools ``[N, P, H_kv, D]`` (same slot rules as ``ref_reshape_and_cache``:
    negative slots are skipped, slots must be unique)."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    kc = np.array(k_cache, dtype=np.uint8, copy=True)
    vc = np.array(v_cache, dtype=np.uint8, copy=True)
    N, P, H, D = kc.shape
    keep = slots >= 0
    used = slots[keep]
    assert np.all(used < N * P), "oracle: slot outside the pool"
    assert len(np.unique(used)) == len(used), "oracle: duplicate slots in one call"
    kq = ref_quantize(k, k_scale)
    vq = ref_quantize(v, v_scale)
    kc.reshape(N * P, H, D)[used] = kq[keep]
    vc.reshape(N * P, H, D)[used] = vq[keep]
    return kc, vc
