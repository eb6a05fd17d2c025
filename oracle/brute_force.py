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

from .paged_attention import widen

__all__ = ["contiguous_cache", "brute_decode", "brute_prefill"]


def contiguous_cache(tok, cu_ctx, H_kv, D):
    """``cache[b][g][s][d]`` (nested lists of floats) from a packed token stream
    ``tok[cu_ctx[b] + s, g, d]`` (weft "Cache layouts", contiguous column: slice
    assignment at a cursor)."""
    x = widen(tok)
    B = len(cu_ctx) - 1
    cache = []
    for b in range(B):
        rows = []
        for g in range(H_kv):
            seq = []
            for s in range(int(cu_ctx[b]), int(cu_ctx[b + 1])):
                seq.append([float(x[s, g, d]) for d in range(D)])
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
    qd = widen(q)
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
            qv = [float(qd[b, h, d]) for d in range(D)]
            heads.append(_one_row(qv, Kc[b][g], Vc[b][g], L, scale))
        out.append(heads)
    return out


def brute_prefill(q, cu_q, k_tok, v_tok, cu_ctx, H_kv, scale):
    """Chunked prefill: the last ``T_b`` tokens of request ``b`` are the chunk;
    chunk row ``i`` sits at position ``L_b - T_b + i`` and sees keys up to and
    including itself (tiny-vllm-py "KV Cache" and "Mistakes I made").
    Returns nested lists ``[T_total][H_q][D]``."""
    qd = widen(q)
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
                qv = [float(qd[r, h, d]) for d in range(D)]
                heads.append(_one_row(qv, Kc[b][g], Vc[b][g], visible, scale))
            out.append(heads)
    return out
