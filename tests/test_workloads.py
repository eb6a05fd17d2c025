"""The seeded input generator: layout invariants and value rounding.  CPU only."""

import math

import numpy as np
import pytest

from workloads import CONFIGS, config_case, make_case, to_bf16_bits


def _check_tables(case):
    P = case.block_size
    owned = []
    for b in range(case.B):
        n = (int(case.context_lens[b]) + P - 1) // P
        row = case.block_table[b]
        owned.extend(row[:n].tolist())
        # ember "What's implemented": at most one partly used block per sequence
        assert n * P - case.context_lens[b] < P
        assert np.all(row[n:] == case.filler_block)
    assert len(set(owned)) == len(owned), "a physical block is owned twice"
    assert case.filler_block not in owned
    assert all(0 <= x < case.num_blocks for x in owned)


@pytest.mark.parametrize("idx", range(5))
def test_config_layouts(idx):
    case = config_case(idx, values=False)
    _check_tables(case)
    cfg = CONFIGS[idx]
    assert case.num_q_heads == cfg["H_q"] and case.num_kv_heads == cfg["H_kv"] and case.head_dim == cfg["D"]
    assert case.max_blocks_per_seq * case.block_size >= cfg["max_ctx"]
    if cfg["N"] is not None:
        assert case.num_blocks == cfg["N"]
    else:
        used = sum((int(L) + case.block_size - 1) // case.block_size for L in case.context_lens)
        assert used / case.num_blocks == pytest.approx(0.9, abs=0.01)


def test_config_length_ranges():
    assert config_case(0, values=False).context_lens.min() >= 1
    c = config_case(3, values=False)
    assert c.B == 256 and c.context_lens.min() >= 16 and c.context_lens.max() <= 8192
    assert 600 < np.median(c.context_lens) < 1700
    m = config_case(4, values=False)
    T = m.query_lens[:16]
    assert np.all((T >= 128) & (T <= 2048)) and np.all(m.query_lens[16:] == 1)
    pre = m.context_lens[:16] - T
    assert np.all((pre >= 0) & (pre <= 4096))
    assert np.all((m.context_lens[16:] >= 256) & (m.context_lens[16:] <= 8192))


@pytest.mark.parametrize("P", [1, 16, 64])
def test_mixed_block_size_variants_share_values(P):
    a = make_case(dtype="bf16", block_size=P, num_q_heads=4, num_kv_heads=2, head_dim=8,
                  context_lens=[40, 7], query_lens=[5, 1], seed=7)
    b = make_case(dtype="bf16", block_size=16, num_q_heads=4, num_kv_heads=2, head_dim=8,
                  context_lens=[40, 7], query_lens=[5, 1], seed=7)
    _check_tables(a)
    assert np.array_equal(a.k_tok, b.k_tok) and np.array_equal(a.q, b.q)


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000).astype(np.float32)
    bits = to_bf16_bits(x)
    for xi, bi in zip(x[:2000], bits[:2000]):
        # the two bf16 neighbours of xi, by truncation
        lo = int(np.float32(xi).view(np.uint32)) >> 16
        cands = [lo, lo + 1]
        vals = [np.uint32(c << 16).view(np.float32) for c in cands]
        d = [abs(float(v) - float(xi)) for v in vals]
        if d[0] < d[1]:
            want = cands[0]
        elif d[1] < d[0]:
            want = cands[1]
        else:
            want = cands[0] if cands[0] % 2 == 0 else cands[1]
        assert int(bi) == want
    # exact halfway cases
    half = np.array([0x3F808000, 0x3F818000], dtype=np.uint32).view(np.float32)
    assert to_bf16_bits(half).tolist() == [0x3F80, 0x3F82]


def test_case_new_and_prefix_split():
    c = make_case(dtype="f32", block_size=4, num_q_heads=2, num_kv_heads=1, head_dim=4,
                  context_lens=[6, 3], query_lens=[2, 3], seed=1)
    kn, _ = c.new_kv()
    kp, _, cu_pre, lens_pre = c.prefix()
    assert lens_pre.tolist() == [4, 0] and cu_pre.tolist() == [0, 4, 4]
    assert np.array_equal(kn, c.k_tok[[4, 5, 6, 7, 8]])
    assert np.array_equal(kp, c.k_tok[[0, 1, 2, 3]])
    assert c.scale == pytest.approx(1 / math.sqrt(4))
