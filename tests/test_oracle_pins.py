"""Pins for the CPU oracle: worked examples from the pages, closed forms, the
pages' invariances and an independent brute force.  CPU only."""

import json
import math
import os

import numpy as np
import pytest

from oracle import (
    brute_decode,
    brute_prefill,
    ref_decode,
    ref_prefill,
    ref_reshape_and_cache,
    ref_slot_mapping,
    widen,
)
from workloads import draw_values, make_case, nan_pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot_examples.json")


def _examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


# ----------------------------------------------------------------------------
# helpers: populate a NaN pool through the oracle's own scatter
# ----------------------------------------------------------------------------

def populate(case, include_new=True):
    """Oracle pool after writing the cached prefix and (optionally) this step's
    new tokens, each through ref_slot_mapping + ref_reshape_and_cache."""
    kc = nan_pool(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim, case.dtype)
    vc = kc.copy()
    kp, vp, cu_pre, lens_pre = case.prefix()
    slots = ref_slot_mapping(case.block_table, cu_pre, lens_pre, case.block_size)
    kc, vc = ref_reshape_and_cache(kp, vp, slots, kc, vc)
    if include_new:
        kn, vn = case.new_kv()
        slots = ref_slot_mapping(case.block_table, case.cu_seqlens, case.context_lens, case.block_size)
        kc, vc = ref_reshape_and_cache(kn, vn, slots, kc, vc)
    return kc, vc


def decode_oracle(case):
    kc, vc = populate(case)
    return ref_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale)


def tiny_case(G=2, H_kv=2, D=8, P=4, lens=(5, 1, 17, 9), seed=0, dtype="f32", qlens=None, **kw):
    return make_case(dtype=dtype, block_size=P, num_q_heads=G * H_kv, num_kv_heads=H_kv, head_dim=D,
                     context_lens=list(lens), query_lens=qlens, seed=seed, **kw)


# ----------------------------------------------------------------------------
# slot math: the pages' worked examples
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["source"][:40])
def test_slot_mapping_worked_examples(ex):
    P = ex["block_size"]
    n = len(ex["positions"])
    # the whole sequence written as one prefill step
    got = ref_slot_mapping([ex["block_table"]], [0, n], [n], P)
    assert got.tolist() == ex["slot"]
    assert [b * P + o for b, o in zip(ex["physical_block"], ex["offset"])] == ex["slot"]


@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["source"][:40])
def test_slot_mapping_decode_position_is_length_before_append(ex):
    # tiny-vllm-py "Design Choices": the new token's position is the cache length
    # before its K/V is appended; context_lens counts the new token too.
    P = ex["block_size"]
    for n in range(1, len(ex["positions"]) + 1):
        got = ref_slot_mapping([ex["block_table"]], [0, 1], [n], P)
        assert got.tolist() == [ex["slot"][n - 1]]


def test_slot_mapping_chunk_over_prefix():
    ex = _examples()[2]
    # 4 tokens cached, a chunk of 6 new tokens: positions 4..9
    got = ref_slot_mapping([ex["block_table"]], [0, 6], [10], 4)
    assert got.tolist() == ex["slot"][4:]


# ----------------------------------------------------------------------------
# bf16 -> fp64 conversion (the first step of every bf16 oracle result)
# ----------------------------------------------------------------------------

def _same_fp64(a, b):
    """Equal as values, NaN where either is NaN, and zeros with the same sign."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nan = np.isnan(a)
    return (np.array_equal(nan, np.isnan(b)) and np.array_equal(a[~nan], b[~nan])
            and np.array_equal(np.signbit(a[~nan]), np.signbit(b[~nan])))


ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_widen_matches_torch_on_every_bf16_pattern():
    import torch

    want = torch.from_numpy(ALL_BF16.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same_fp64(widen(ALL_BF16), want)


def test_widen_matches_field_decoder_on_every_bf16_pattern():
    from oracle.brute_force import bf16_value

    assert _same_fp64(widen(ALL_BF16), [bf16_value(int(b)) for b in ALL_BF16])


def test_widen_hand_constants():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x7F7F, 0x0080, 0x0001,
                     0x3EAB, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -126,
            2.0 ** -133, (1 + 0x2B / 128) * 2.0 ** -2, (1 + 0x49 / 128) * 2.0]
    assert _same_fp64(widen(bits), want)
    assert np.all(np.isnan(widen(np.array([0x7FC0, 0x7F81, 0xFFFF], dtype=np.uint16))))
    f = np.array([1.5, -0.0, 3.0e38, 1e-45], dtype=np.float32)
    assert _same_fp64(widen(f), [1.5, -0.0, float(np.float32(3.0e38)), float(np.float32(1e-45))])


def test_widen_pin_catches_a_wrong_width():
    # shifting the uint16 left by 16 without first widening wraps to zero
    wrong = (ALL_BF16 << np.uint16(16)).astype(np.uint32).view(np.float32).astype(np.float64)
    from oracle.brute_force import bf16_value

    assert not _same_fp64(wrong, [bf16_value(int(b)) for b in ALL_BF16])


# ----------------------------------------------------------------------------
# scatter
# ----------------------------------------------------------------------------

def test_reshape_and_cache_is_bit_exact_and_touches_only_its_slots():
    N, P, H, D = 6, 4, 2, 4
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00001, 0xFFBADBAD,
                        0x00000001, 0x807FFFFF], dtype=np.uint32)
    rng = np.random.default_rng(5)
    k = rng.choice(special, size=(5, H, D)).view(np.float32)
    v = rng.integers(0, 2**32, size=(5, H, D), dtype=np.uint64).astype(np.uint32).view(np.float32)
    kc = rng.integers(0, 2**32, size=(N, P, H, D), dtype=np.uint64).astype(np.uint32).view(np.float32)
    vc = kc.copy()
    slots = np.array([7, 0, 23, -1, 13])
    nk, nv = ref_reshape_and_cache(k, v, slots, kc, vc)
    fk = nk.view(np.uint32).reshape(N * P, H, D)
    fv = nv.view(np.uint32).reshape(N * P, H, D)
    ok = kc.view(np.uint32).reshape(N * P, H, D)
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(fk[s], k[t].view(np.uint32))
            assert np.array_equal(fv[s], v[t].view(np.uint32))
    untouched = np.setdiff1d(np.arange(N * P), slots[slots >= 0])
    assert np.array_equal(fk[untouched], ok[untouched])
    # inputs are not modified
    assert np.array_equal(kc.view(np.uint32).reshape(N * P, H, D), ok)


def test_reshape_and_cache_bf16_bits_and_duplicates_rejected():
    kc = nan_pool(3, 2, 1, 4, "bf16")
    k = np.array([[[0x0001, 0x8000, 0x7F80, 0x1234]]], dtype=np.uint16)
    nk, _ = ref_reshape_and_cache(k, k, [5], kc, kc)
    assert nk.reshape(6, 1, 4)[5].tolist() == k[0].tolist()
    with pytest.raises(AssertionError):
        ref_reshape_and_cache(np.concatenate([k, k]), np.concatenate([k, k]), [1, 1], kc, kc)


# ----------------------------------------------------------------------------
# decode: brute force and closed forms
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("G,H_kv,P", [(1, 3, 1), (2, 2, 3), (3, 1, 4), (4, 2, 7)])
def test_decode_matches_brute_force(G, H_kv, P):
    case = tiny_case(G=G, H_kv=H_kv, P=P, lens=(5, 1, 17, 9, 30), seed=G * 10 + P)
    ref = decode_oracle(case)
    bf = np.array(brute_decode(case.q, case.k_tok, case.v_tok, case.cu_ctx, case.num_kv_heads, case.scale))
    np.testing.assert_allclose(ref, bf, rtol=0, atol=1e-12)


def test_decode_matches_brute_force_bf16():
    case = tiny_case(G=4, H_kv=2, D=16, P=5, lens=(33, 2, 40), seed=3, dtype="bf16")
    ref = decode_oracle(case)
    bf = np.array(brute_decode(case.q, case.k_tok, case.v_tok, case.cu_ctx, case.num_kv_heads, case.scale))
    np.testing.assert_allclose(ref, bf, rtol=0, atol=1e-12)


def test_decode_single_token_returns_its_value_exactly():
    case = tiny_case(lens=(1, 1, 1), seed=11)
    out = decode_oracle(case)
    G = case.num_q_heads // case.num_kv_heads
    v = widen(case.v_tok)
    for b in range(case.B):
        for h in range(case.num_q_heads):
            assert np.array_equal(out[b, h], v[case.cu_ctx[b], h // G])


def test_decode_zero_query_is_mean_of_values():
    case = tiny_case(lens=(7, 12, 3), seed=12)
    case.q[:] = 0
    out = decode_oracle(case)
    v = widen(case.v_tok)
    G = case.num_q_heads // case.num_kv_heads
    for b in range(case.B):
        rows = v[case.cu_ctx[b]: case.cu_ctx[b + 1]]
        for h in range(case.num_q_heads):
            np.testing.assert_allclose(out[b, h], rows[:, h // G].mean(axis=0), rtol=0, atol=1e-14)


def test_decode_identical_values_return_that_value():
    case = tiny_case(lens=(9, 4), seed=13)
    case.v_tok[:] = case.v_tok[0]
    out = decode_oracle(case)
    v0 = widen(case.v_tok[0])
    G = case.num_q_heads // case.num_kv_heads
    for b in range(case.B):
        for h in range(case.num_q_heads):
            np.testing.assert_allclose(out[b, h], v0[h // G], rtol=1e-15, atol=1e-15)


def test_decode_dominant_key_and_two_key_logistic():
    # one key whose score is 60 above every other: output is that key's value to e^-60
    case = tiny_case(G=1, H_kv=1, D=4, lens=(6,), seed=14)
    case.q[:] = 0
    case.q[0, 0, 0] = 1.0
    case.k_tok[:] = 0
    j = 3
    case.k_tok[j, 0, 0] = 60.0 / case.scale
    out = decode_oracle(case)
    np.testing.assert_allclose(out[0, 0], widen(case.v_tok)[j, 0], rtol=0, atol=10 * math.exp(-60) * 6)
    # two keys: out = sigma(s0 - s1) v0 + sigma(s1 - s0) v1
    case = tiny_case(G=1, H_kv=1, D=4, lens=(2,), seed=15)
    q, k, v = widen(case.q)[0, 0], widen(case.k_tok)[:, 0], widen(case.v_tok)[:, 0]
    s0, s1 = case.scale * (q @ k[0]), case.scale * (q @ k[1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    expect = w0 * v[0] + (1.0 - w0) * v[1]
    np.testing.assert_allclose(decode_oracle(case)[0, 0], expect, rtol=0, atol=1e-14)


def test_decode_empty_context_gives_zeros():
    case = tiny_case(lens=(3, 0, 2), qlens=(1, 0, 1), seed=16)
    kc, vc = populate(case)
    out = ref_decode(case.q[[0, 0, 1]], kc, vc, case.block_table, case.context_lens, case.scale)
    assert np.all(out[1] == 0)


# ----------------------------------------------------------------------------
# decode: the pages' invariances (bitwise in the oracle)
# ----------------------------------------------------------------------------

def test_decode_block_size_invariance_bitwise():
    # ember "Correctness": identical output for block_size in {1,2,3,7,16,64}
    outs = [decode_oracle(tiny_case(G=2, H_kv=2, P=P, lens=(70, 5, 129, 1), seed=21)) for P in (1, 2, 3, 7, 16, 64)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_decode_block_permutation_invariance_bitwise():
    # tiny-vllm-py "Mental Model": only where the KV entries physically live changes
    a = tiny_case(P=4, lens=(13, 22, 9), seed=22)
    kc, vc = populate(a)
    ref = ref_decode(a.q, kc, vc, a.block_table, a.context_lens, a.scale)
    rng = np.random.default_rng(99)
    perm = rng.permutation(a.num_blocks)  # physical block i moves to perm[i]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = perm[a.block_table]
    out = ref_decode(a.q, kc2, vc2, bt2, a.context_lens, a.scale)
    assert np.array_equal(out, ref)


def test_decode_batch_invariance_bitwise():
    # ember "Correctness": a request alone == alongside others
    full = tiny_case(lens=(11, 40, 3, 25), seed=23)
    ref = decode_oracle(full)
    for b in range(full.B):
        alone = tiny_case(lens=(int(full.context_lens[b]),), seed=0)
        # carry request b's own values into the single-request case
        s, e = full.cu_ctx[b], full.cu_ctx[b + 1]
        alone.k_tok[:] = full.k_tok[s:e]
        alone.v_tok[:] = full.v_tok[s:e]
        alone.q[:] = full.q[b: b + 1]
        assert np.array_equal(decode_oracle(alone)[0], ref[b])


def test_gqa_equals_replicated_mha_bitwise():
    g = tiny_case(G=4, H_kv=2, lens=(10, 3), seed=24)
    ref = decode_oracle(g)
    G = 4
    m = tiny_case(G=1, H_kv=8, lens=(10, 3), seed=0)
    m.k_tok[:] = np.repeat(g.k_tok, G, axis=1)
    m.v_tok[:] = np.repeat(g.v_tok, G, axis=1)
    m.q[:] = g.q
    assert np.array_equal(decode_oracle(m), ref)


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

def prefill_oracle(case):
    kc, vc = populate(case)
    return ref_prefill(case.q, kc, vc, case.cu_seqlens, case.block_table, case.context_lens, case.scale)


@pytest.mark.parametrize("G,H_kv,P", [(1, 2, 1), (2, 2, 3), (4, 1, 16)])
def test_prefill_matches_brute_force(G, H_kv, P):
    case = tiny_case(G=G, H_kv=H_kv, P=P, lens=(9, 20, 4, 13), qlens=(9, 6, 1, 13), seed=30 + G)
    ref = prefill_oracle(case)
    bf = np.array(brute_prefill(case.q, case.cu_seqlens, case.k_tok, case.v_tok, case.cu_ctx,
                                case.num_kv_heads, case.scale))
    np.testing.assert_allclose(ref, bf, rtol=0, atol=1e-12)


def test_prefill_without_prefix_is_textbook_causal_attention():
    # tiny-vllm-py "Mistakes I made": prefill is causal (is_causal=True)
    case = tiny_case(G=2, H_kv=1, D=8, P=3, lens=(12,), qlens=(12,), seed=31)
    out = prefill_oracle(case)
    q = widen(case.q)[:, :, :]
    k = widen(case.k_tok)[:, 0]
    v = widen(case.v_tok)[:, 0]
    T = 12
    mask = np.triu(np.full((T, T), -np.inf), k=1)
    for h in range(2):
        S = case.scale * q[:, h] @ k.T + mask
        W = np.exp(S - S.max(axis=1, keepdims=True))
        W /= W.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(out[:, h], W @ v, rtol=0, atol=1e-13)


def test_prefill_single_new_token_equals_decode_bitwise():
    case = tiny_case(lens=(8, 19, 1), seed=32)
    kc, vc = populate(case)
    dec = ref_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale)
    pre = ref_prefill(case.q, kc, vc, case.cu_seqlens, case.block_table, case.context_lens, case.scale)
    assert np.array_equal(dec, pre)


def test_mixed_batch_equals_its_parts_bitwise():
    """A ragged batch of one-token chunks (decodes) and longer chunks (the
    single-launch mixed call's reading of a step): each request's rows are
    those of its chunk computed alone, and the one-token rows are decode."""
    case = tiny_case(lens=(8, 19, 1, 30, 6), qlens=(1, 7, 1, 30, 2), seed=36)
    kc, vc = populate(case)
    cu = case.cu_seqlens
    mixed = ref_prefill(case.q, kc, vc, cu, case.block_table, case.context_lens, case.scale)
    for b in range(case.B):
        s, e = int(cu[b]), int(cu[b + 1])
        alone = ref_prefill(case.q[s:e], kc, vc, [0, e - s], case.block_table[b:b + 1], case.context_lens[b:b + 1],
                            case.scale)
        assert np.array_equal(mixed[s:e], alone), b
        if e - s == 1:
            dec = ref_decode(case.q[s:e], kc, vc, case.block_table[b:b + 1], case.context_lens[b:b + 1], case.scale)
            assert np.array_equal(mixed[s:e], dec), b


def test_chunked_prefill_equals_one_shot_bitwise():
    one = tiny_case(G=2, H_kv=2, P=3, lens=(23,), qlens=(23,), seed=33)
    ref = prefill_oracle(one)
    # the same prompt in chunks of 5, 9, 1, 8: each chunk scatters, then attends
    kc = nan_pool(one.num_blocks, 3, 2, one.head_dim, one.dtype)
    vc = kc.copy()
    start = 0
    pieces = []
    for T in (5, 9, 1, 8):
        L = start + T
        slots = ref_slot_mapping(one.block_table, [0, T], [L], 3)
        kc, vc = ref_reshape_and_cache(one.k_tok[start:L], one.v_tok[start:L], slots, kc, vc)
        pieces.append(ref_prefill(one.q[start:L], kc, vc, [0, T], one.block_table, [L], one.scale))
        start = L
    assert np.array_equal(np.concatenate(pieces), ref)


def test_prefill_rows_subset_matches_full():
    case = tiny_case(lens=(9, 20), qlens=(4, 7), seed=34)
    kc, vc = populate(case)
    full = ref_prefill(case.q, kc, vc, case.cu_seqlens, case.block_table, case.context_lens, case.scale)
    part = ref_prefill(case.q, kc, vc, case.cu_seqlens, case.block_table, case.context_lens, case.scale,
                       rows=[1, 5, 10])
    for r in (1, 5, 10):
        assert np.array_equal(part[r], full[r])
    assert np.isnan(part[0]).all()


def test_unused_table_entries_are_never_read():
    # entries past ceil(L/P) may hold anything, even ids outside the pool
    case = tiny_case(P=4, lens=(5, 9), seed=35)
    kc, vc = populate(case)
    ref = ref_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale)
    bt = case.block_table.copy()
    for b in range(case.B):
        bt[b, (case.context_lens[b] + 3) // 4:] = case.num_blocks + 7
    assert np.array_equal(ref_decode(case.q, kc, vc, bt, case.context_lens, case.scale), ref)


# ----------------------------------------------------------------------------
# planted mistakes: each pin above must catch a plausible bug in the oracle
# ----------------------------------------------------------------------------

def test_pins_catch_planted_mistakes(monkeypatch):
    import oracle.paged_attention as pa

    case = tiny_case(G=2, H_kv=2, P=3, lens=(7, 12), seed=40)
    bf = np.array(brute_decode(case.q, case.k_tok, case.v_tok, case.cu_ctx, 2, case.scale))

    # 1. wrong GQA head map (h % H_kv instead of h // G)
    def bad_decode(q, k_cache, v_cache, block_table, context_lens, scale, select=None):
        qd = pa.widen(q)
        B, Hq, D = qd.shape
        Hkv = k_cache.shape[2]
        out = np.zeros((B, Hq, D))
        for b in range(B):
            K = pa.ref_gather(k_cache, block_table[b], context_lens[b], k_cache.shape[1])
            V = pa.ref_gather(v_cache, block_table[b], context_lens[b], k_cache.shape[1])
            for h in range(Hq):
                out[b, h] = pa._attend(qd[b, h], K[:, h % Hkv], V[:, h % Hkv], scale)
        return out

    kc, vc = populate(case)
    assert not np.allclose(bad_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale), bf)

    # 2. slot offset taken from the wrong term (p // P instead of p % P)
    ex = _examples()[2]
    bt = np.asarray([ex["block_table"]])
    pos = np.arange(10)
    wrong = bt[0, pos // 4] * 4 + pos // 4
    assert wrong.tolist() != ex["slot"]

    # 3. causal mask off by one (a row does not see itself)
    pcase = tiny_case(G=1, H_kv=1, P=3, lens=(6,), qlens=(6,), seed=41)
    kc, vc = populate(pcase)
    bfp = np.array(brute_prefill(pcase.q, pcase.cu_seqlens, pcase.k_tok, pcase.v_tok, pcase.cu_ctx, 1, pcase.scale))
    orig = pa._attend
    monkeypatch.setattr(pa, "_attend", lambda q, K, V, s: orig(q, K[:-1], V[:-1], s))
    bad = pa.ref_prefill(pcase.q, kc, vc, pcase.cu_seqlens, pcase.block_table, pcase.context_lens, pcase.scale)
    assert not np.allclose(bad[1:], bfp[1:])


# ----------------------------------------------------------------------------
# prefix sharing and copy-on-write (tiny-vllm-py, "Prefix Sharing")
# ----------------------------------------------------------------------------

from oracle import ref_copy_blocks  # noqa: E402
from workloads import shared_prefix_case  # noqa: E402


def prefix_pools(c, table, pairs, per_request=False):
    """Oracle pools of a shared-prefix case: the prefix written once through
    request 0's table, then the block copies, then every request's tail through
    ``table`` (one call, or one call per request)."""
    P, S = c.block_size, c.prefix_len
    kc = nan_pool(c.num_blocks, P, c.num_kv_heads, c.head_dim, c.dtype)
    vc = kc.copy()
    slots = ref_slot_mapping(table[:1], [0, S], [S], P)
    kc, vc = ref_reshape_and_cache(c.k_tok[:S], c.v_tok[:S], slots, kc, vc)
    if len(pairs):
        kc, vc = ref_copy_blocks(kc, vc, pairs)
    rows = [np.arange(c.cu_ctx[b] + S, c.cu_ctx[b + 1]) for b in range(c.B)]
    groups = [[b] for b in range(c.B)] if per_request else [list(range(c.B))]
    for grp in groups:
        idx = np.concatenate([rows[b] for b in grp]).astype(np.int64)
        cu = np.concatenate([[0], np.cumsum([len(rows[b]) for b in grp])])
        slots = ref_slot_mapping(table[grp], cu, c.context_lens[grp], P)
        kc, vc = ref_reshape_and_cache(c.k_tok[idx], c.v_tok[idx], slots, kc, vc)
    return kc, vc


def cow_pairs(c):
    return [(int(c.shared_blocks[-1]), int(c.cow_blocks[b])) for b in range(c.B) if c.cow_blocks[b] >= 0]


def dup_pairs(c):
    return [(int(c.shared_blocks[i]), int(c.dup_blocks[b, i])) for b in range(1, c.B)
            for i in range(len(c.shared_blocks))]


def test_copy_blocks_is_a_bit_copy_and_skips_negative_pairs():
    kc = np.arange(6 * 2 * 1 * 4, dtype=np.uint16).reshape(6, 2, 1, 4)
    kc[1, 0, 0, 0] = 0x7FC1  # a NaN payload survives
    vc = kc + np.uint16(1000)
    nk, nv = ref_copy_blocks(kc, vc, [[1, 4], [-1, 5], [2, -1], [0, 3]])
    assert np.array_equal(nk[4], kc[1]) and np.array_equal(nv[4], vc[1])
    assert np.array_equal(nk[3], kc[0]) and np.array_equal(nv[3], vc[0])
    for blk in (0, 1, 2, 5):
        assert np.array_equal(nk[blk], kc[blk]) and np.array_equal(nv[blk], vc[blk])
    assert np.array_equal(kc[4], np.arange(32, 40).reshape(2, 1, 4))  # input untouched
    with pytest.raises(AssertionError):
        ref_copy_blocks(kc, vc, [[1, 2], [2, 3]])  # a destination that is also a source
    with pytest.raises(AssertionError):
        ref_copy_blocks(kc, vc, [[1, 2], [0, 2]])  # two copies into one block


@pytest.mark.parametrize("S,P,tails", [(10, 4, (3, 0, 9)), (8, 4, (5, 1)), (13, 1, (2, 7, 4)), (21, 7, (6, 30))])
def test_prefix_sharing_with_copy_on_write_matches_brute_force(S, P, tails):
    c = shared_prefix_case(dtype="f32", block_size=P, num_q_heads=4, num_kv_heads=2, head_dim=8, prefix_len=S,
                           tail_lens=tails, seed=S + P)
    kc, vc = prefix_pools(c, c.block_table, cow_pairs(c))
    out = ref_decode(c.q, kc, vc, c.block_table, c.context_lens, c.scale)
    bf = np.array(brute_decode(c.q, c.k_tok, c.v_tok, c.cu_ctx, c.num_kv_heads, c.scale))
    np.testing.assert_allclose(out, bf, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,P,tails", [(10, 4, (3, 0, 9)), (16, 4, (5, 1, 2)), (13, 1, (2, 7, 4))])
def test_shared_blocks_equal_duplicated_blocks_bitwise(S, P, tails):
    c = shared_prefix_case(dtype="bf16", block_size=P, num_q_heads=8, num_kv_heads=2, head_dim=16, prefix_len=S,
                           tail_lens=tails, seed=3 * S + P)
    kc, vc = prefix_pools(c, c.block_table, cow_pairs(c))
    shared = ref_decode(c.q, kc, vc, c.block_table, c.context_lens, c.scale)
    kd, vd = prefix_pools(c, c.dup_table, dup_pairs(c))
    dup = ref_decode(c.q, kd, vd, c.dup_table, c.context_lens, c.scale)
    assert np.array_equal(shared, dup)


def test_appending_into_a_shared_partial_block_without_copy_corrupts_the_other_request():
    # planted mistake: no copy-on-write; request 0 then reads request 2's tail
    c = shared_prefix_case(dtype="f32", block_size=4, num_q_heads=4, num_kv_heads=2, head_dim=8, prefix_len=10,
                           tail_lens=(3, 0, 9), seed=14)
    kc, vc = prefix_pools(c, c.naive_table, [], per_request=True)
    out = ref_decode(c.q, kc, vc, c.naive_table, c.context_lens, c.scale)
    bf = np.array(brute_decode(c.q, c.k_tok, c.v_tok, c.cu_ctx, c.num_kv_heads, c.scale))
    assert not np.allclose(out[0], bf[0], atol=1e-6)
    np.testing.assert_allclose(out[2], bf[2], rtol=0, atol=1e-12)  # the last writer sees its own tail


# ----------------------------------------------------------------------------
# fp8 (OCP E4M3) KV: encode / decode against the format's definition and
# torch's float8_e4m3fn conversion (a library routine), then attention over
# the dequantised pool against the brute force
# ----------------------------------------------------------------------------

import torch  # noqa: E402

from oracle import (  # noqa: E402
    e4m3_decode,
    e4m3_encode,
    ref_dequantize,
    ref_quantize,
    ref_reshape_and_cache_fp8,
)


def _torch_e4m3(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_decode_table():
    codes = np.arange(256, dtype=np.uint8)
    d = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(np.isnan(d), np.isnan(ref))
    assert np.array_equal(d[~np.isnan(d)], ref[~np.isnan(ref)])
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0 and d[0x38] == 1.0
    assert d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6 and d[0x07] == 7 * 2.0 ** -9
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and d[0x80] == 0 and np.signbit(d[0x80])
    assert np.all(np.diff(d[:0x7F]) > 0)  # monotone over the finite positive codes


def test_e4m3_encode_round_trip_ties_and_saturation():
    codes = np.arange(256, dtype=np.uint8)
    d = e4m3_decode(codes)
    fin = ~np.isnan(d)
    assert np.array_equal(e4m3_encode(d[fin]), codes[fin])
    # exact midpoints between neighbouring positive codes go to the even code
    mids = (d[0:0x7E] + d[1:0x7F]) / 2.0
    want = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F)).astype(np.uint8)
    assert np.array_equal(e4m3_encode(mids), want)
    assert np.array_equal(e4m3_encode(-mids), want | 0x80)
    assert np.array_equal(_torch_e4m3(mids.astype(np.float32)), want)
    # saturation (torch turns these into NaN; this reading clamps to 448)
    big = np.array([448.5, 464.0, 479.0, 480.0, 1e4, np.inf])
    assert np.all(e4m3_encode(big) == 0x7E) and np.all(e4m3_encode(-big) == 0xFE)
    assert e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(-463.9, 463.9, 200000), rng.uniform(-0.03, 0.03, 100000),
                        rng.standard_normal(100000) * 4]).astype(np.float32)
    assert np.array_equal(e4m3_encode(x.astype(np.float64)), _torch_e4m3(x))


def test_quantize_is_scaled_rne_with_bounded_error():
    rng = np.random.default_rng(9)
    H, D = 4, 32
    x = draw_values(rng, (500, H, D), "bf16")
    s = np.array([0.01, 0.05, 0.3, 1.7], dtype=np.float32)
    codes = ref_quantize(x, s)
    # the quotient is fp32 division of the fp32 values (torch's CPU division is IEEE)
    xf = torch.from_numpy(widen(x).astype(np.float32))
    q = (xf / torch.from_numpy(s)[:, None]).numpy()
    assert np.all(np.abs(q) < 463)
    assert np.array_equal(codes, _torch_e4m3(q))
    back = ref_dequantize(codes, s)
    err = np.abs(back - widen(x))
    # half a step of the code grid, plus the fp32 rounding of the quotient
    # (which can land exactly on a tie, as 0.02490234375 / 1.7 does)
    bound = np.maximum(np.abs(widen(x)) * 2.0 ** -4, 2.0 ** -10 * s[:, None].astype(np.float64))
    assert np.all(err <= bound * (1 + 2.0 ** -16))


@pytest.mark.parametrize("G,H_kv,P", [(2, 2, 4), (4, 1, 3), (1, 3, 16)])
def test_fp8_decode_is_attention_over_dequantised_values(G, H_kv, P):
    case = tiny_case(G=G, H_kv=H_kv, D=16, P=P, lens=(5, 1, 30, 17), seed=40 + P, dtype="bf16")
    ks = np.linspace(0.005, 0.02, H_kv).astype(np.float32)
    vs = np.linspace(0.01, 0.03, H_kv).astype(np.float32)
    # pool: prefix and new tokens written through the fp8 scatter
    kc = np.zeros((case.num_blocks, P, H_kv, 16), dtype=np.uint8)
    vc = kc.copy()
    kp, vp, cu_pre, lens_pre = case.prefix()
    kc, vc = ref_reshape_and_cache_fp8(kp, vp, ref_slot_mapping(case.block_table, cu_pre, lens_pre, P), kc, vc,
                                       ks, vs)
    kn, vn = case.new_kv()
    kc, vc = ref_reshape_and_cache_fp8(
        kn, vn, ref_slot_mapping(case.block_table, case.cu_seqlens, case.context_lens, P), kc, vc, ks, vs)
    out = ref_decode(case.q, ref_dequantize(kc, ks), ref_dequantize(vc, vs), case.block_table, case.context_lens,
                     case.scale)
    # brute force on the dequantised token streams (contiguous layout, no pool)
    kq = ref_dequantize(ref_quantize(case.k_tok, ks), ks)
    vq = ref_dequantize(ref_quantize(case.v_tok, vs), vs)
    bf = np.array(brute_decode(case.q, kq, vq, case.cu_ctx, H_kv, case.scale))
    np.testing.assert_allclose(out, bf, rtol=0, atol=1e-12)
