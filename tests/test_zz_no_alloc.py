"""The allocation-free decode call (pa_paged_decode_attention_noalloc) against
the decode call with a caller workspace (pa_paged_decode_attention): the same
kernels, so the same bits, over consecutive calls that share the library's
static scratch array (each call leaves its contents for the next)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_48_amd as pa
from oracle import ref_decode
from workloads import config_case, make_case

from gpu_util import DevCase, assert_close, oracle_pool, to_host_bits

pytestmark = pytest.mark.gpu


def both_ways(d):
    c = d.case
    want = torch.empty_like(d.q)
    got = torch.full_like(d.q, float("nan"))
    pa.paged_decode_attention(d.q, d.kc, d.vc, d.bt, d.lens, c.scale, want)
    pa.paged_decode_attention_noalloc(d.q, d.kc, d.vc, d.bt, d.lens, c.scale, got)
    torch.cuda.synchronize()
    return want, got


def check(d, rows, what):
    c = d.case
    print(f"{what}: B={c.B} {c.dtype} H_q={c.num_q_heads} H_kv={c.num_kv_heads} D={c.head_dim}", flush=True)
    want, got = both_ways(d)
    assert np.array_equal(to_host_bits(got), to_host_bits(want)), f"{what}: outputs differ"
    kc, vc = oracle_pool(c)
    ref = ref_decode(c.q, kc, vc, c.block_table, c.context_lens, c.scale, select=rows)
    assert_close(got, ref, c.dtype, what, rows=rows)


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    # 1: the Llama-3-8B-shaped batch (B=256, contexts up to 8192): 132 MiB of scratch
    big = config_case(3)
    need = pa.decode_workspace_size(big.B, big.num_q_heads, big.head_dim, big.block_size, big.max_blocks_per_seq)
    assert need <= 160 << 20
    order = np.argsort(big.context_lens)
    check(DevCase(big), sorted({int(order[0]), int(order[-1]), 3, 100, 200}), "llama3_8b")
    # 2: a smaller call right after it, over the scratch the first one left
    check(DevCase(config_case(0)), [0, 1, 2, 3], "tiny fp32")
    # 3: above 1024 requests the work items are listed in the scratch by a plan kernel
    rng = np.random.default_rng(91)
    lens = rng.integers(1, 600, size=1100)
    lens[:4] = [1, 256, 257, 599]
    c3 = make_case(dtype="bf16", block_size=16, num_q_heads=8, num_kv_heads=2, head_dim=64,
                   context_lens=lens.tolist(), seed=91)
    check(DevCase(c3), [0, 1, 2, 3, 500, 1099], "1100 requests")


def test_noalloc_rejects_batches_beyond_the_scratch():
    c = config_case(0)
    d = DevCase(c)
    q = d.q.new_zeros((1024, 32, 128)).to(torch.bfloat16)
    pool = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16, device=q.device)
    bt = torch.zeros((1024, 512), dtype=torch.int32, device=q.device)
    lens = torch.ones(1024, dtype=torch.int32, device=q.device)
    with pytest.raises(ValueError, match="static scratch"):
        pa.paged_decode_attention_noalloc(q, pool, pool, bt, lens, 0.1, torch.empty_like(q))
