"""Independent brute-force attention for tiny inputs, used to pin the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/paged_attention.py``).

It never touches a block pool, a block table or a slot.  It builds weft's
*contiguous* layout ("Cache layouts": per-layer view ``[B, H_kv, S_max, D]``,
request ``b`` owns row ``b``, written at a cursor) straight from each request's
token stream in logical order, then evaluates attention with explicit Python
loops and ``math.exp``: no reshape, no fancy indexing, no matrix products.  The
paged oracle must agree with it, which pins slot math, scatter, gather, the GQA
head map, masking and the softmax together.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["bf16_value", "scalar_value", "contiguous_cache", "brute_decode", "brute_prefill"]


def bf16_value(bits: int) -> float:
    """Value of one bfloat16 bit pattern, decoded field by field.

    bfloat16 keeps binary32's layout with the low 16 fraction bits dropped: one
    sign bit, 8 exponent bits with bias 127 and 7 fraction bits.  Exponent 0
    holds zero and the subnormals ``f / 2^7 * 2^-126``; exponent 255 holds the
    infinities (``f = 0``) and NaN (``f != 0``); every other exponent ``e`` holds
    ``(1 + f / 2^7) * 2^(e - 127)``.  This decoder is written from that
    definition on its own and does not use the oracle's conversion, so that the
    two can pin each other.
    """
    b = int(bits) & 0xFFFF
    sign = -1.0 if b >> 15 else 1.0
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if e == 0xFF:
        return math.nan if f else sign * math.inf
    if e == 0:
        return sign * math.ldexp(float(f), -126 - 7)
    return sign * math.ldexp(float(128 + f), e - 127 - 7)


def scalar_value(x) -> float:
    """One element as a Python float: uint16 elements are bfloat16 bit patterns
    (decoded by ``bf16_value``); float32 and float64 elements convert exactly."""
    if isinstance(x, np.uint16):
        return bf16_value(int(x))
    if isinstance(x, (np.float32, np.float64, float)):
        return float(x)
    raise TypeError(f"brute force: unsupported element type {type(x)}")


def contiguous_cache(tok, cu_ctx, H_kv, D):
    """``cache[b][g][s][d]`` (nested lists of floats) from a packed token stream
    ``tok[cu_ctx[b] + s, g, d]`` (weft "Cache layouts", contiguous column: slice
    assignment at a cursor)."""
    x = np.asarray(tok)
    B = len(cu_ctx) - 1
    cache = []
    for b in range(B):
        rows = []
        for g in range(H_kv):
            seq = []
            for s in range(int(cu_ctx[b]), int(cu_ctx[b + 1])):
                seq.append([scalar_value(x[s, g, d]) for d in range(D)])
            rows.append(seq)
        cache.append(rows)
    return cache


def _one_row(qv, Krows, Vrows, count, scale):
    D = len(qv)
    if count == 0:
        return [0.0] * D
    scores = []
    for j in range(count):
        acc = 0.0
        for d in range(D):
            acc += qv[d] * Krows[j][d]
        scores.append(acc * scale)
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = sum(weights)
    out = []
    for d in range(D):
        acc = 0.0
        for j in range(count):
            acc += weights[j] * Vrows[j][d]
        out.append(acc / total)
    return out


def brute_decode(q, k_tok, v_tok, cu_ctx, H_kv, scale):
    """Decode: query head ``h`` of request ``b`` attends, unmasked, to all of the
    request's tokens (tiny-vllm-py "KV Cache").  Returns nested lists
    ``[B][H_q][D]``."""
    qd = np.asarray(q)
    B, Hq, D = qd.shape
    G = Hq // H_kv
    Kc = contiguous_cache(k_tok, cu_ctx, H_kv, D)
    Vc = contiguous_cache(v_tok, cu_ctx, H_kv, D)
    out = []
    for b in range(B):
        L = int(cu_ctx[b + 1] - cu_ctx[b])
        heads = []
        for h in range(Hq):
            g = h // G
            qv = [scalar_value(qd[b, h, d]) for d in range(D)]
            heads.append(_one_row(qv, Kc[b][g], Vc[b][g], L, scale))
        out.append(heads)
    return out


def brute_prefill(q, cu_q, k_tok, v_tok, cu_ctx, H_kv, scale):
    """Chunked prefill: the last ``T_b`` tokens of request ``b`` are the chunk;
    chunk row ``i`` sits at position ``L_b - T_b + i`` and sees keys up to and
    including itself (tiny-vllm-py "KV Cache" and "Mistakes I made").
    Returns nested lists ``[T_total][H_q][D]``."""
    qd = np.asarray(q)
    T_total, Hq, D = qd.shape
    G = Hq // H_kv
    Kc = contiguous_cache(k_tok, cu_ctx, H_kv, D)
    Vc = contiguous_cache(v_tok, cu_ctx, H_kv, D)
    out = []
    for b in range(len(cu_q) - 1):
        L = int(cu_ctx[b + 1] - cu_ctx[b])
        T = int(cu_q[b + 1] - cu_q[b])
        for i in range(T):
            r = int(cu_q[b]) + i
            visible = L - T + i + 1
            heads = []
            for h in range(Hq):
                g = h // G
                qv = [scalar_value(qd[r, h, d]) for d in range(D)]
                heads.append(_one_row(qv, Kc[b][g], Vc[b][g], visible, scale))
            out.append(heads)
    return out
