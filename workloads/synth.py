"""Seeded synthetic inputs for attention over a paged KV cache.

This module is shared by the tests, ``bench.py`` and the oracle's checks, so it
holds none of the method's arithmetic: it draws context lengths, deals out
physical blocks and draws values.  It never computes a slot, gathers a key or
evaluates a score; each side does that with its own code.

Recipe (the five workloads, all seeded with numpy PCG64):

* ``tiny``: B=4, H_q=H_kv=12, D=64, P=16, N=64, fp32, context ~ U[1,200], one
  new token per request.
* ``gpt2_124m``: 12 layers, H_q=H_kv=12, D=64, P=16, B=64, bf16,
  context ~ U[32,1024], N=4096.
* ``llama32_1b``: 16 layers, H_q=32, H_kv=8, D=64, P=16, B=128, bf16,
  context ~ U[128,4096], pool sized for 90% occupancy.
* ``llama3_8b``: 32 layers, H_q=32, H_kv=8, D=128, P=16, B=256, bf16, context
  log-normal with median 1024 and sigma 1 (``rint(exp(N(ln 1024, 1)))``),
  clipped to [16, 8192], pool sized for 90% occupancy.
* ``mixed``: H_q=32, H_kv=8, D=128, bf16, 64 requests: 16 prefill chunks of
  T ~ U[128,2048] new tokens over cached prefixes ~ U[0,4096], then 48 decodes
  with context ~ U[256,8192]; block size 1, 16 or 64; 90% occupancy.

Values are N(0,1) drawn in fp32 and, for bf16 workloads, rounded to the nearest
bfloat16 (ties to even); bf16 data travels as ``uint16`` bit patterns.  The
block table gives request ``b`` exactly ``ceil(L_b / P)`` blocks (so at most one
partly used block per request), taken in turn from a random permutation of the
pool, so requests' blocks are randomly interleaved.  Table entries past a
request's last block hold ``filler_block``, a block that no request owns.

Streams: lengths come from ``default_rng([seed, 1])``, the block permutation
from ``default_rng([seed, 2, P])`` and the values of layer ``l`` from
``default_rng([seed, 3, l])``.  Values therefore do not depend on the block
size, and every layer shares the same lengths and block table, as the layers
of one model do.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

__all__ = [
    "CONFIGS",
    "Case",
    "to_bf16_bits",
    "draw_values",
    "make_case",
    "config_case",
    "nan_pool",
    "SharedPrefixCase",
    "shared_prefix_case",
]

NAN_BITS = {"bf16": 0x7FC0, "f32": 0x7FC00000}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite normals, so no NaN/inf handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) values: float32 for ``f32``, bfloat16 bits (uint16) for ``bf16``."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def nan_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: str) -> np.ndarray:
    """A pool whose every entry is a quiet NaN, as host bits/values."""
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    if dtype == "bf16":
        return np.full(shape, NAN_BITS["bf16"], dtype=np.uint16)
    return np.full(shape, NAN_BITS["f32"], dtype=np.uint32).view(np.float32)


@dataclass
class Case:
    """One step's inputs.  Shapes: ``k_tok``/``v_tok`` ``[sum L, H_kv, D]`` hold each
    request's whole token stream in logical order (request ``b`` at rows
    ``cu_ctx[b] .. cu_ctx[b+1]-1``); ``q`` ``[T_total, H_q, D]`` holds the new
    tokens' queries packed by request through ``cu_seqlens``."""

    name: str
    dtype: str
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    context_lens: np.ndarray  # int32 [B]
    query_lens: np.ndarray  # int32 [B], new tokens this step
    block_table: np.ndarray  # int32 [B, M]
    filler_block: int
    num_layers: int = 1
    layer: int = 0
    seed: int = 0
    k_tok: Optional[np.ndarray] = field(default=None, repr=False)
    v_tok: Optional[np.ndarray] = field(default=None, repr=False)
    q: Optional[np.ndarray] = field(default=None, repr=False)

    @property
    def B(self) -> int:
        return int(len(self.context_lens))

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.query_lens, dtype=np.int64)]).astype(np.int32)

    @property
    def cu_ctx(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.context_lens, dtype=np.int64)])

    @property
    def T_total(self) -> int:
        return int(self.query_lens.sum())

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.query_lens == 1))

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    def new_kv(self):
        """Keys/values of this step's new tokens, packed like ``q``: the last
        ``query_lens[b]`` rows of each request's stream."""
        cu = self.cu_ctx
        idx = np.concatenate(
            [np.arange(cu[b + 1] - self.query_lens[b], cu[b + 1]) for b in range(self.B)]
            or [np.zeros(0, dtype=np.int64)]
        ).astype(np.int64)
        return self.k_tok[idx], self.v_tok[idx]

    def prefix(self):
        """``(k, v, cu_seqlens, context_lens)`` of the tokens cached before this
        step: the first ``context_lens[b] - query_lens[b]`` rows of each stream,
        written as one earlier step whose new tokens are the whole prefix."""
        cu = self.cu_ctx
        lens = (self.context_lens - self.query_lens).astype(np.int32)
        idx = np.concatenate(
            [np.arange(cu[b], cu[b] + lens[b]) for b in range(self.B)] or [np.zeros(0, dtype=np.int64)]
        ).astype(np.int64)
        cu_pre = np.concatenate([[0], np.cumsum(lens, dtype=np.int64)]).astype(np.int32)
        return self.k_tok[idx], self.v_tok[idx], cu_pre, lens

    def with_values(self, layer: Optional[int] = None) -> "Case":
        """Same layout with values drawn for ``layer`` (default: this case's layer)."""
        layer = self.layer if layer is None else layer
        rng = np.random.default_rng([self.seed, 3, layer])
        S = int(self.context_lens.sum())
        shp = (S, self.num_kv_heads, self.head_dim)
        k = draw_values(rng, shp, self.dtype)
        v = draw_values(rng, shp, self.dtype)
        q = draw_values(rng, (self.T_total, self.num_q_heads, self.head_dim), self.dtype)
        return replace(self, layer=layer, k_tok=k, v_tok=v, q=q)


def _deal_blocks(context_lens, block_size, num_blocks, max_blocks, rng):
    need = [(int(L) + block_size - 1) // block_size for L in context_lens]
    total = sum(need)
    if total >= num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {total} blocks plus a filler block")
    perm = rng.permutation(num_blocks).astype(np.int32)
    filler = int(perm[total])
    table = np.full((len(need), max_blocks), filler, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        if n > max_blocks:
            raise ValueError("a request needs more blocks than max_blocks")
        table[b, :n] = perm[off : off + n]
        off += n
    return table, filler


def make_case(
    *,
    name: str = "custom",
    dtype: str,
    block_size: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    context_lens,
    query_lens=None,
    seed: int = 0,
    num_blocks: Optional[int] = None,
    occupancy: float = 0.9,
    max_blocks_per_seq: Optional[int] = None,
    num_layers: int = 1,
    layer: int = 0,
    values: bool = True,
) -> Case:
    """Build a case from explicit lengths.  ``query_lens`` defaults to one new
    token per request (decode).  ``num_blocks`` defaults to the smallest pool at
    or below ``occupancy`` (plus room for the filler block)."""
    lens = np.asarray(context_lens, dtype=np.int32)
    qlens = np.ones_like(lens) if query_lens is None else np.asarray(query_lens, dtype=np.int32)
    assert lens.shape == qlens.shape and np.all(qlens <= lens) and np.all(qlens >= 0)
    P = int(block_size)
    need = int(sum((int(L) + P - 1) // P for L in lens))
    if num_blocks is None:
        num_blocks = max(need + 1, int(math.ceil(need / occupancy)))
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, max((int(L) + P - 1) // P for L in lens) if len(lens) else 1)
    table, filler = _deal_blocks(lens, P, num_blocks, max_blocks_per_seq, np.random.default_rng([seed, 2, P]))
    case = Case(
        name=name,
        dtype=dtype,
        block_size=P,
        num_blocks=int(num_blocks),
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        scale=1.0 / math.sqrt(head_dim),
        context_lens=lens,
        query_lens=qlens,
        block_table=table,
        filler_block=filler,
        num_layers=num_layers,
        layer=layer,
        seed=seed,
    )
    return case.with_values() if values else case


# name, layers, dtype, H_q, H_kv, D, default P, fixed N (None = 90% occupancy), longest context
CONFIGS = [
    dict(name="tiny", layers=1, dtype="f32", H_q=12, H_kv=12, D=64, P=16, N=64, max_ctx=200),
    dict(name="gpt2_124m", layers=12, dtype="bf16", H_q=12, H_kv=12, D=64, P=16, N=4096, max_ctx=1024),
    dict(name="llama32_1b", layers=16, dtype="bf16", H_q=32, H_kv=8, D=64, P=16, N=None, max_ctx=4096),
    dict(name="llama3_8b", layers=32, dtype="bf16", H_q=32, H_kv=8, D=128, P=16, N=None, max_ctx=8192),
    dict(name="mixed", layers=1, dtype="bf16", H_q=32, H_kv=8, D=128, P=16, N=None, max_ctx=8192),
]


def _draw_lengths(idx: int, rng: np.random.Generator):
    """Context and new-token lengths for workload ``idx`` (see the module docstring)."""
    if idx == 0:
        lens = rng.integers(1, 200, size=4, endpoint=True)
        return lens, np.ones_like(lens)
    if idx == 1:
        lens = rng.integers(32, 1024, size=64, endpoint=True)
        return lens, np.ones_like(lens)
    if idx == 2:
        lens = rng.integers(128, 4096, size=128, endpoint=True)
        return lens, np.ones_like(lens)
    if idx == 3:
        z = rng.standard_normal(size=256)
        lens = np.clip(np.rint(np.exp(math.log(1024.0) + z)), 16, 8192).astype(np.int64)
        return lens, np.ones_like(lens)
    if idx == 4:
        T = rng.integers(128, 2048, size=16, endpoint=True)
        prefix = rng.integers(0, 4096, size=16, endpoint=True)
        dec = rng.integers(256, 8192, size=48, endpoint=True)
        lens = np.concatenate([prefix + T, dec])
        qlens = np.concatenate([T, np.ones(48, dtype=np.int64)])
        return lens, qlens
    raise IndexError(idx)


def config_case(idx: int, seed: Optional[int] = None, block_size: Optional[int] = None,
                layer: int = 0, values: bool = True) -> Case:
    """Workload ``idx`` (0..4, in the order of the module docstring)."""
    cfg = CONFIGS[idx]
    seed = idx if seed is None else seed
    lens, qlens = _draw_lengths(idx, np.random.default_rng([seed, 1]))
    P = cfg["P"] if block_size is None else int(block_size)
    M = (cfg["max_ctx"] + P - 1) // P
    return make_case(
        name=cfg["name"],
        dtype=cfg["dtype"],
        block_size=P,
        num_q_heads=cfg["H_q"],
        num_kv_heads=cfg["H_kv"],
        head_dim=cfg["D"],
        context_lens=lens,
        query_lens=qlens,
        seed=seed,
        num_blocks=cfg["N"] if block_size is None or cfg["N"] is None else None,
        max_blocks_per_seq=M,
        num_layers=cfg["layers"],
        layer=layer,
        values=values,
    )


# ---------------------------------------------------------------------------
# Prefix sharing: several requests whose streams start with the same tokens.
# ---------------------------------------------------------------------------

@dataclass
class SharedPrefixCase:
    """Requests ``b < B`` share their first ``prefix_len`` tokens (identical K/V
    rows) and then continue with ``tail_lens[b]`` tokens of their own.

    ``shared_blocks`` hold the prefix once: ``ceil(prefix_len / P)`` physical
    blocks, the last one partly used when ``prefix_len % P != 0``.
    ``cow_blocks[b]`` (``-1`` for request 0, and for every request when the
    prefix fills whole blocks) is a free block that receives a copy of that
    partly used block before request ``b`` appends to it.  ``block_table`` is
    the table after copy-on-write (request 0 keeps the shared partial block);
    ``naive_table`` points every request at the shared partial block instead.
    ``dup_table`` gives every request private copies of all prefix blocks
    (``dup_blocks[b]``, one per prefix block; request 0 keeps the originals).
    ``k_tok``/``v_tok`` are ``[sum L, H_kv, D]`` streams in request order
    (request ``b`` at rows ``cu_ctx[b] .. cu_ctx[b+1]-1``), ``q`` is
    ``[B, H_q, D]`` (one decode query per request)."""

    dtype: str
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    prefix_len: int
    tail_lens: np.ndarray
    context_lens: np.ndarray
    cu_ctx: np.ndarray
    shared_blocks: np.ndarray
    cow_blocks: np.ndarray
    dup_blocks: np.ndarray
    block_table: np.ndarray
    naive_table: np.ndarray
    dup_table: np.ndarray
    k_tok: np.ndarray
    v_tok: np.ndarray
    q: np.ndarray

    @property
    def B(self) -> int:
        return len(self.tail_lens)


def shared_prefix_case(*, dtype: str, block_size: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                       prefix_len: int, tail_lens, seed: int = 0) -> SharedPrefixCase:
    P = int(block_size)
    tails = np.asarray(tail_lens, dtype=np.int32)
    B = len(tails)
    S = int(prefix_len)
    lens = (S + tails).astype(np.int32)
    ns = (S + P - 1) // P              # prefix blocks
    partial = S % P != 0
    own = [(int(L) + P - 1) // P - ns for L in lens]  # blocks after the prefix blocks
    need = ns + sum(own) + (B - 1 if partial else 0) + ns * (B - 1) + 1
    N = need + 3
    rng = np.random.default_rng([seed, 4, P])
    perm = rng.permutation(N).astype(np.int32)
    it = iter(perm.tolist())
    shared = np.array([next(it) for _ in range(ns)], dtype=np.int32)
    cow = np.full(B, -1, dtype=np.int32)
    if partial:
        for b in range(1, B):
            cow[b] = next(it)
    dup = np.full((B, max(ns, 1)), -1, dtype=np.int32)
    for b in range(1, B):
        for i in range(ns):
            dup[b, i] = next(it)
    M = max(int(ns + o) for o in own)
    filler = None
    own_blocks = [[next(it) for _ in range(o)] for o in own]
    filler = next(it)
    table = np.full((B, M), filler, dtype=np.int32)
    naive = np.full((B, M), filler, dtype=np.int32)
    dupt = np.full((B, M), filler, dtype=np.int32)
    for b in range(B):
        row = list(shared) + own_blocks[b]
        naive[b, : len(row)] = row
        if partial and b > 0:
            row = list(shared[:-1]) + [int(cow[b])] + own_blocks[b]
        table[b, : len(row)] = row
        drow = (list(shared) if b == 0 else list(dup[b, :ns])) + own_blocks[b]
        dupt[b, : len(drow)] = drow
    vr = np.random.default_rng([seed, 5])
    pre_k = draw_values(vr, (S, num_kv_heads, head_dim), dtype)
    pre_v = draw_values(vr, (S, num_kv_heads, head_dim), dtype)
    ks, vs = [], []
    for b in range(B):
        ks += [pre_k, draw_values(vr, (int(tails[b]), num_kv_heads, head_dim), dtype)]
        vs += [pre_v, draw_values(vr, (int(tails[b]), num_kv_heads, head_dim), dtype)]
    q = draw_values(vr, (B, num_q_heads, head_dim), dtype)
    cu = np.concatenate([[0], np.cumsum(lens, dtype=np.int64)]).astype(np.int64)
    return SharedPrefixCase(dtype=dtype, block_size=P, num_blocks=N, num_q_heads=num_q_heads,
                            num_kv_heads=num_kv_heads, head_dim=head_dim, scale=1.0 / math.sqrt(head_dim),
                            prefix_len=S, tail_lens=tails, context_lens=lens, cu_ctx=cu, shared_blocks=shared,
                            cow_blocks=cow, dup_blocks=dup, block_table=table, naive_table=naive, dup_table=dupt,
                            k_tok=np.concatenate(ks), v_tok=np.concatenate(vs), q=q)
