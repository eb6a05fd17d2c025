"""Plain fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library and does not
import the product package.

What it computes, and where that comes from (page title, then section):

* weft, "Shapes and symbols" / "Cache layouts": the paged per-layer cache view is
  ``[N, P, H_kv, D]``; writes scatter through ``slot_mapping``; reads gather
  through ``block_table``.
* ember, "The core idea, in one picture": logical position ``p`` of a sequence
  lives at block ``block_table[p // P]``, offset ``p % P``.
* tiny-vllm-py, "KV Cache" / "Mental Model" and "Design Choices": the cache holds
  keys after RoPE and plain values; at time ``t`` a query may attend to every
  earlier token and to ``t`` itself; a token's position is the cache length
  before its own K/V is appended; prefill is causal, decode is not masked.
* tiny-vllm-py, "Paged KV Cache / Paged Attention", "Mental Model": a request's
  logical prefix is still the contiguous token sequence ``0..L-1``; paging only
  changes where each entry physically lives.  So the oracle gathers each
  request's keys/values into a dense buffer and evaluates
  ``softmax(scale * q K^T) V`` directly, in fp64.
* weft, "Shapes and symbols": ``H_q / H_kv`` is the GQA group size ``G``.

Readings of points the pages leave open:

* slot encoding: ``slot = physical_block * P + offset`` indexes the flattened
  ``[N * P]`` token rows of the pool;
* a negative slot marks a padding token that is skipped; duplicate slots in one
  call are a caller error (asserted here);
* ``context_lens[b]`` counts every cached token of request ``b`` *including*
  this step's new tokens (the scatter runs before attention);
* query head ``h`` reads KV head ``h // G`` (contiguous groups);
* a chunk of ``T`` new tokens over a cached prefix is causal by absolute
  position: its row ``i`` sits at position ``L - T + i`` and sees keys
  ``0 .. L - T + i``;
* ``context_lens[b] == 0`` yields an all-zero output row.

Host conventions: bfloat16 data is carried as ``uint16`` bit patterns and
widened exactly; fp32 data as ``float32``.  Index arrays may be any integer
dtype.  Every result is fp64.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "widen",
    "ref_slot_mapping",
    "ref_reshape_and_cache",
    "ref_copy_blocks",
    "ref_gather",
    "ref_decode",
    "ref_prefill",
]


def widen(x) -> np.ndarray:
    """Exact conversion of a host array to fp64.

    ``uint16`` arrays hold bfloat16 bit patterns: a bfloat16 is the upper half
    of an IEEE binary32, so shifting the bits left by 16 and reading them as
    float32 is exact; float32 -> float64 is exact as well.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.float32 or x.dtype == np.float64:
        return x.astype(np.float64)
    raise TypeError(f"oracle: unsupported element dtype {x.dtype}")


def _bits(x: np.ndarray) -> np.ndarray:
    """Raw-bit view so copies never touch floating-point values (NaN payloads survive)."""
    if x.dtype == np.uint16 or x.dtype == np.uint8:
        return x
    if x.dtype == np.float32:
        return x.view(np.uint32)
    raise TypeError(f"oracle: unsupported cache dtype {x.dtype}")


def ref_slot_mapping(block_table, cu_seqlens, context_lens, block_size) -> np.ndarray:
    """Slot of every new token (weft "Cache layouts"; ember "The core idea").

    Request ``b`` contributes ``T_b = cu_seqlens[b+1] - cu_seqlens[b]`` new
    tokens.  Its cache already holds ``context_lens[b] - T_b`` tokens, so new
    token ``i`` takes position ``p = context_lens[b] - T_b + i`` (tiny-vllm-py,
    "Design Choices": the position is the cache length before the append), and
    lives at block ``block_table[b][p // P]``, offset ``p % P``.
    Returns int64 ``[T_total]``.
    """
    bt = np.asarray(block_table, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.asarray(context_lens, dtype=np.int64)
    P = int(block_size)
    pieces = []
    for b in range(len(lens)):
        T = int(cu[b + 1] - cu[b])
        assert 0 <= T <= lens[b], "oracle: a request has more new tokens than context"
        pos = np.arange(lens[b] - T, lens[b], dtype=np.int64)
        pieces.append(bt[b, pos // P] * P + pos % P)
    if not pieces:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(pieces)


def ref_reshape_and_cache(k, v, slot_mapping, k_cache, v_cache):
    """Scatter new keys/values into copies of the pool (weft "Cache layouts": write
    = scatter via slot_mapping; tiny-vllm-py "Mental Model": append into the tail
    block).  Token ``t`` is copied bit for bit to flattened row ``slot_mapping[t]``
    of the ``[N*P, H_kv, D]`` view.  Negative slots are skipped.  Returns
    ``(new_k_cache, new_v_cache)``; the inputs are not modified.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    N, P, H, D = kc.shape
    assert np.asarray(k).shape == (len(slots), H, D)
    assert np.asarray(v).shape == (len(slots), H, D)
    keep = slots >= 0
    used = slots[keep]
    assert np.all(used < N * P), "oracle: slot outside the pool"
    assert len(np.unique(used)) == len(used), "oracle: duplicate slots in one call"
    kflat = _bits(kc).reshape(N * P, H, D)
    vflat = _bits(vc).reshape(N * P, H, D)
    kflat[used] = _bits(np.asarray(k, dtype=kc.dtype))[keep]
    vflat[used] = _bits(np.asarray(v, dtype=vc.dtype))[keep]
    return kc, vc


def ref_copy_blocks(k_cache, v_cache, block_mapping):
    """Copy whole blocks for copy-on-write (tiny-vllm-py, "Prefix Sharing": requests
    with a common prefix point their block tables at the same physical blocks,
    and a shared partial tail block is copied before a request appends to it;
    ember, "Deliberately out of scope": copy-on-write block tables).  For each
    pair ``(src, dst)`` of ``block_mapping`` (``[n, 2]``), block ``dst`` of both
    pools becomes a bit-for-bit copy of block ``src``.  Pairs with a negative
    entry are skipped.  Destinations must be distinct and no destination may be
    a source (so the order of the pairs does not matter).  Returns
    ``(new_k_cache, new_v_cache)``; the inputs are not modified.
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    N = kc.shape[0]
    keep = (pairs[:, 0] >= 0) & (pairs[:, 1] >= 0)
    src, dst = pairs[keep, 0], pairs[keep, 1]
    assert np.all(src < N) and np.all(dst < N), "oracle: block outside the pool"
    assert len(np.unique(dst)) == len(dst), "oracle: a block is copied into twice"
    assert not np.any(np.isin(dst, src)), "oracle: a destination is also a source"
    kb, vb = _bits(kc), _bits(vc)
    kb[dst] = _bits(np.asarray(k_cache))[src]
    vb[dst] = _bits(np.asarray(v_cache))[src]
    return kc, vc


def ref_gather(cache, block_table_row, length, block_size) -> np.ndarray:
    """Dense fp64 ``[length, H_kv, D]`` copy of one request's logical prefix
    (weft "Cache layouts": read = gather by block_table; ember "The core idea")."""
    N, P, H, D = cache.shape
    assert P == block_size
    pos = np.arange(int(length), dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[pos // P]
    assert np.all((blocks >= 0) & (blocks < N)), "oracle: block id outside the pool"
    rows = blocks * P + pos % P
    return widen(cache.reshape(N * P, H, D)[rows])


def _attend(qrow: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """``softmax(scale * K q) V`` for one query row over the visible keys, fp64.
    The max is subtracted before ``exp`` only to avoid overflow; the result is the
    same function."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = (K @ qrow) * scale
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def ref_decode(q, k_cache, v_cache, block_table, context_lens, scale, select=None):
    """Decode attention (tiny-vllm-py "KV Cache": the new token attends to every
    cached token including itself, no causal mask; weft "Shapes and symbols": GQA
    with group size ``G = H_q / H_kv``).

    ``q``: ``[B, H_q, D]``.  ``context_lens[b]`` tokens of request ``b`` are
    visible.  Returns fp64 ``[B, H_q, D]``; with ``select`` (an iterable of
    request indices) only those rows are computed and the others are NaN.
    """
    qd = widen(q)
    B, Hq, D = qd.shape
    N, P, Hkv, D2 = k_cache.shape
    assert D2 == D and Hq % Hkv == 0
    G = Hq // Hkv
    out = np.full((B, Hq, D), np.nan)
    for b in (range(B) if select is None else select):
        L = int(context_lens[b])
        K = ref_gather(k_cache, block_table[b], L, P)
        V = ref_gather(v_cache, block_table[b], L, P)
        for h in range(Hq):
            g = h // G
            out[b, h] = _attend(qd[b, h], K[:, g, :], V[:, g, :], scale)
    return out


def ref_prefill(q, k_cache, v_cache, cu_seqlens, block_table, context_lens, scale, rows=None):
    """Varlen / chunked prefill attention over the paged cache (tiny-vllm-py
    "Mistakes I made": prefill is causal; "KV Cache": a token sees itself;
    ember "What's implemented" and weft "Shapes and symbols" for ragged
    ``T_total`` packing).

    ``q``: ``[T_total, H_q, D]`` packed by request through ``cu_seqlens``.  The
    chunk's keys/values are already in the pool.  Packed row ``cu[b] + i`` sits at
    absolute position ``L_b - T_b + i`` and sees keys ``0 .. L_b - T_b + i``.
    Returns fp64 ``[T_total, H_q, D]``; with ``rows`` (packed row indices) only
    those rows are computed and the others are NaN.
    """
    qd = widen(q)
    T_total, Hq, D = qd.shape
    N, P, Hkv, _ = k_cache.shape
    G = Hq // Hkv
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.full((T_total, Hq, D), np.nan)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(len(cu) - 1):
        T = int(cu[b + 1] - cu[b])
        L = int(context_lens[b])
        assert 0 <= T <= L, "oracle: chunk longer than the request's context"
        mine = [r for r in range(int(cu[b]), int(cu[b + 1])) if wanted is None or r in wanted]
        if not mine:
            continue
        K = ref_gather(k_cache, block_table[b], L, P)
        V = ref_gather(v_cache, block_table[b], L, P)
        for r in mine:
            pos = L - T + (r - int(cu[b]))
            for h in range(Hq):
                g = h // G
                out[r, h] = _attend(qd[r, h], K[: pos + 1, g, :], V[: pos + 1, g, :], scale)
    return out
