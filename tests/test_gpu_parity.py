"""GPU parity: the HIP path against the fp64 oracle on seeded inputs.

Scatter and slot math must be bit-exact; attention must be within 1e-4 (fp32
inputs) or 1e-2 + 2e-2 |ref| (bf16 inputs) element by element.  Every pool is
NaN-filled before it is written, so a kernel that lets a masked slot reach the
output fails.  All calls go through the C ABI (ctypes binding)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_48_amd as pa
from oracle import ref_copy_blocks, ref_decode, ref_prefill, ref_slot_mapping
from workloads import config_case, make_case, shared_prefix_case

from gpu_util import (DEV, DevCase, Fp8Case, assert_close, dev_nan_pool, fp8_scales, idx, oracle_pool, to_dev,
                      to_host_bits)

pytestmark = pytest.mark.gpu


def decode_ref(case, select=None, block_table=None):
    kc, vc = oracle_pool(case, block_table)
    bt = case.block_table if block_table is None else block_table
    return ref_decode(case.q, kc, vc, bt, case.context_lens, case.scale, select=select)


def small(dtype="bf16", P=16, Hq=32, Hkv=8, D=128, lens=(1, 16, 255, 256, 257, 511, 700), qlens=None, seed=0, **kw):
    return make_case(dtype=dtype, block_size=P, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                     context_lens=list(lens), query_lens=qlens, seed=seed, **kw)


# ----------------------------------------------------------------------------
# slot mapping and scatter: bit-exact
# ----------------------------------------------------------------------------

def test_slot_mapping_worked_examples_on_gpu():
    # ember "The core idea" (block table [2, 0, 5], P = 4) and tiny-vllm-py
    # "Mental Model" (blocks 17, 4, 23): whole sequence as one prefill step
    for table, n, want in (([2, 0, 5], 9, [8, 9, 10, 11, 0, 1, 2, 3, 20]),
                           ([17, 4, 23], 10, [68, 69, 70, 71, 16, 17, 18, 19, 92, 93])):
        got = pa.slot_mapping(idx([table]), idx([0, n]), idx([n]), 4, n)
        assert got.cpu().tolist() == want


@pytest.mark.parametrize("idx_cfg,P", [(0, None), (4, 1), (4, 16), (4, 64)])
def test_slot_mapping_matches_oracle(idx_cfg, P):
    c = config_case(idx_cfg, block_size=P, values=False)
    got = pa.slot_mapping(idx(c.block_table), idx(c.cu_seqlens), idx(c.context_lens), c.block_size, c.T_total)
    want = ref_slot_mapping(c.block_table, c.cu_seqlens, c.context_lens, c.block_size)
    assert np.array_equal(got.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reshape_and_cache_bit_exact_whole_pool(dtype):
    c = small(dtype=dtype, P=7, Hq=4, Hkv=2, D=64, lens=(3, 40, 9, 64), qlens=(3, 5, 1, 64), seed=3)
    # plant special values in the new tokens' K: +-0, +-inf, NaN payloads, denormals
    specials = {"f32": np.array([0x0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00123, 0xFFBADBAD, 0x1, 0x807FFFFF],
                                dtype=np.uint32).view(np.float32),
                "bf16": np.array([0x0, 0x8000, 0x7F80, 0xFF80, 0x7FC1, 0xFFAB, 0x1, 0x807F], dtype=np.uint16)}[dtype]
    flat = c.k_tok.reshape(-1)
    flat[-len(specials) * 50:] = np.tile(specials, 50)
    d = DevCase(c)
    kc, vc = oracle_pool(c)
    bits = np.uint16 if dtype == "bf16" else np.uint32
    assert np.array_equal(to_host_bits(d.kc).view(bits), kc.view(bits))
    assert np.array_equal(to_host_bits(d.vc).view(bits), vc.view(bits))


def test_reshape_and_cache_skips_negative_slots():
    c = small(dtype="bf16", P=4, Hq=2, Hkv=2, D=64, lens=(6,), qlens=(6,), seed=4)
    d = DevCase(c)
    before = to_host_bits(d.kc).copy()
    k = to_dev(c.k_tok[:3] ^ np.uint16(0x1234), "bf16")
    pa.reshape_and_cache(k, k, idx([-1, -5, -1]), d.kc, d.vc)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(d.kc), before)


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def test_decode_tiny_config():
    c = config_case(0)
    d = DevCase(c)
    assert_close(d.decode(), decode_ref(c), "f32", "tiny")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_decode_config_shapes_reduced(cfg):
    """The config's head shape and dtype with a hand-picked set of lengths that
    covers L = 1, one tile, exactly one partition, one partition + 1 token,
    several partitions and the longest context."""
    base = config_case(cfg, values=False)
    lens = [1, 15, 16, 17, 255, 256, 257, 769, int(base.context_lens.max())]
    c = small(dtype=base.dtype, P=base.block_size, Hq=base.num_q_heads, Hkv=base.num_kv_heads, D=base.head_dim,
              lens=lens, seed=10 + cfg)
    d = DevCase(c)
    assert_close(d.decode(), decode_ref(c), c.dtype, f"config {cfg} shape")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_decode_config_full_size(cfg):
    """The seeded batch of the GPT-2-124M (B=64), Llama-3.2-1B (B=128) and
    Llama-3-8B (B=256, 90% pool) workloads at full size, one layer (every layer
    has the same shape), in the launch configuration the benchmark times: every
    row of the decode call against the oracle, and decode with append equal bit
    for bit to the slot mapping, the scatter and the decode call, outputs and
    pools."""
    c = config_case(cfg)
    print(f"config {c.name}: B={c.B} N={c.num_blocks} sum L={int(c.context_lens.sum())}", flush=True)
    d = DevCase(c)
    out = d.decode()
    ref = decode_ref(c)
    assert_close(out, ref, c.dtype, f"{c.name} decode")
    del d
    kn, vn = (to_dev(x, c.dtype) for x in c.new_kv())
    q, bt, lens = to_dev(c.q, c.dtype), idx(c.block_table), idx(c.context_lens)
    (o1, k1, v1), (o2, k2, v2) = append_both_ways(c, q, kn, vn, bt, lens)
    assert same_bits(k1, k2) and same_bits(v1, v2), "pools differ"
    assert same_bits(o1, o2), "outputs differ"
    assert same_bits(o1, out), "decode of the same pools differs"
    assert_close(o2, ref, c.dtype, f"{c.name} decode with append")


@pytest.mark.parametrize("G,Hkv,D,dtype", [(1, 12, 64, "f32"), (1, 4, 128, "bf16"), (3, 2, 64, "bf16"),
                                           (4, 8, 128, "f32"), (8, 2, 128, "bf16"), (6, 1, 64, "bf16"),
                                           (2, 3, 128, "bf16"), (16, 1, 64, "bf16")])
def test_decode_head_layouts(G, Hkv, D, dtype):
    c = small(dtype=dtype, P=16, Hq=G * Hkv, Hkv=Hkv, D=D, lens=(1, 33, 300, 520), seed=G * 7 + D)
    d = DevCase(c)
    assert_close(d.decode(), decode_ref(c), dtype, f"G={G} D={D} {dtype}")


@pytest.mark.parametrize("kind,G,Hkv,D,P", [
    ("bf16", 8, 8, 128, 16), ("bf16", 16, 2, 128, 16), ("bf16", 12, 2, 64, 7), ("bf16", 7, 4, 64, 16),
    ("bf16", 32, 1, 128, 32), ("bf16", 20, 2, 64, 16), ("f32", 8, 2, 64, 16), ("f32", 16, 1, 128, 5),
    ("fp8", 8, 8, 128, 16), ("fp8", 16, 2, 128, 32), ("fp8", 6, 2, 64, 16), ("fp8", 12, 2, 64, 16)])
def test_decode_wide_query_groups(kind, G, Hkv, D, P):
    """GQA groups of 5 to 32 query heads: a work item takes up to 16 of them (8
    per head of a pair), so each KV slice is read once per 16 query heads.
    Against the oracle, and (bf16 queries) bit for bit against the mixed call,
    whose decode rows read one KV head at a time."""
    c = small(dtype="f32" if kind == "f32" else "bf16", P=P, Hq=G * Hkv, Hkv=Hkv, D=D,
              lens=(1, 16, 255, 256, 257, 700, 1500), seed=110 + G * D + P)
    print(f"wide group {kind} G={G} Hkv={Hkv} D={D} P={P}", flush=True)
    if kind == "fp8":
        d = Fp8Case(c, fp8_scales(Hkv, 111), fp8_scales(Hkv, 112))
        scales, ref = (d.dks, d.dvs), d.reference()
    else:
        d = DevCase(c)
        scales, ref = (None, None), decode_ref(c)
    got = d.decode()
    assert_close(got, ref, "bf16" if kind == "fp8" else c.dtype, f"{kind} G={G} Hkv={Hkv} D={D} P={P}")
    if kind != "f32":
        one = torch.empty_like(d.q)
        pa.paged_mixed_attention(d.q, d.kc, d.vc, idx(np.arange(c.B + 1)), d.bt, d.lens, c.scale, one, *scales)
        assert np.array_equal(to_host_bits(got), to_host_bits(one)), "decode differs from the mixed call"


@pytest.mark.parametrize("kind,G,Hkv,D", [("bf16", 8, 8, 128), ("bf16", 16, 2, 64), ("bf16", 8, 2, 64),
                                          ("fp8", 8, 8, 128), ("fp8", 16, 1, 128)])
def test_decode_group_width_does_not_change_bits(kind, G, Hkv, D):
    """A query head's output does not depend on which other query heads share
    its work item: the call with G query heads per KV head equals, bit for bit,
    G / 4 calls of 4 heads per KV head (each taking every KV head's heads
    4i .. 4i+3), whose items hold 4 heads each."""
    c = small(P=16, Hq=G * Hkv, Hkv=Hkv, D=D, lens=(1, 40, 256, 257, 700, 1500, 3000), seed=120 + G + D)
    print(f"group split {kind} G={G} Hkv={Hkv} D={D}", flush=True)
    if kind == "fp8":
        d = Fp8Case(c, fp8_scales(Hkv, 121), fp8_scales(Hkv, 122))
        scales = (d.dks, d.dvs)
    else:
        d = DevCase(c)
        scales = (None, None)

    def decode(q):
        out = torch.empty_like(q)
        pa.paged_decode_attention(q, d.kc, d.vc, d.bt, d.lens, c.scale, out, *scales)
        return to_host_bits(out)

    whole = decode(d.q).reshape(c.B, Hkv, G, D)
    for i in range(G // 4):
        q4 = d.q.view(c.B, Hkv, G, D)[:, :, 4 * i:4 * i + 4].contiguous().view(c.B, Hkv * 4, D)
        part = decode(q4).reshape(c.B, Hkv, 4, D)
        assert np.array_equal(part, whole[:, :, 4 * i:4 * i + 4]), f"heads {4 * i}..{4 * i + 3} differ"


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("G,Hkv,P", [(1, 2, 16), (4, 2, 16), (6, 4, 7), (8, 8, 1), (1, 16, 64), (5, 2, 3)])
def test_decode_paired_64_dim_heads(kind, G, Hkv, P):
    """bf16 and fp8 pools with 64-dim heads and an even number of KV heads are
    read two adjacent heads at a time, as one 128-dim row per token; each query
    head must still attend to its own KV head only (fp8: with its own head's
    scales).  Checked against the oracle, and bit for bit against the mixed
    call, whose decode rows (one-token chunks) read one KV head at a time."""
    c = small(P=P, Hq=G * Hkv, Hkv=Hkv, D=64, lens=(1, 40, 256, 257, 700, 1500), seed=31 + G * Hkv + P)
    if kind == "fp8":
        d = Fp8Case(c, fp8_scales(Hkv, 63 + P), fp8_scales(Hkv, 64 + P))
        scales, ref = (d.dks, d.dvs), d.reference()
    else:
        d = DevCase(c)
        scales, ref = (None, None), decode_ref(c)
    got = d.decode()
    assert_close(got, ref, "bf16", f"paired heads {kind} G={G} Hkv={Hkv} P={P}")
    one = torch.empty_like(d.q)
    pa.paged_mixed_attention(d.q, d.kc, d.vc, idx(np.arange(c.B + 1)), d.bt, d.lens, c.scale, one, *scales)
    assert np.array_equal(to_host_bits(got), to_host_bits(one)), "paired read differs from the single-head read"


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_decode_paired_heads_keep_a_non_finite_key_to_its_own_head(kind):
    """An infinite (bf16) or NaN-coded (fp8) key element in one KV head of a
    pair changes no output of the other head's query heads: the two heads'
    score products are accumulated apart."""
    G, Hkv = 4, 2
    c = small(P=16, Hq=G * Hkv, Hkv=Hkv, D=64, lens=(300, 40, 700), seed=41)
    if kind == "fp8":
        d = Fp8Case(c, fp8_scales(Hkv, 65), fp8_scales(Hkv, 66))
        bad = 0x7F
    else:
        d = DevCase(c)
        bad = float("inf")
    ref = to_host_bits(d.decode())
    blk = int(c.block_table[0][3])  # tokens 48 .. 63 of request 0
    d.kc[blk, 5, 1, 7] = bad
    got = to_host_bits(d.decode())
    assert np.array_equal(got[:, :G], ref[:, :G]), "KV head 0's query heads changed"
    assert np.array_equal(got[1:], ref[1:]), "other requests changed"


def test_decode_block_size_invariance():
    """ember "Correctness": block_size in {1,2,3,7,16,64}.  Each matches the
    oracle; the kernel tiles by token position only, so results are bitwise
    identical across block sizes."""
    outs = []
    for P in (1, 2, 3, 7, 16, 64):
        c = small(P=P, lens=(5, 130, 257, 600), seed=21)
        d = DevCase(c)
        o = d.decode()
        assert_close(o, decode_ref(c), "bf16", f"P={P}")
        outs.append(to_host_bits(o))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_decode_block_permutation_invariance_bitwise():
    c = small(P=16, lens=(40, 300, 513), seed=22)
    d = DevCase(c)
    ref = to_host_bits(d.decode())
    perm = np.random.default_rng(5).permutation(c.num_blocks).astype(np.int64)
    kc2 = torch.empty_like(d.kc)
    vc2 = torch.empty_like(d.vc)
    p = torch.as_tensor(perm, device=DEV)
    kc2[p] = d.kc
    vc2[p] = d.vc
    bt2 = idx(perm[c.block_table])
    out = torch.empty_like(d.q)
    pa.paged_decode_attention(d.q, kc2, vc2, bt2, d.lens, c.scale, out)
    assert np.array_equal(to_host_bits(out), ref)


def test_decode_batch_invariance_bitwise():
    c = small(P=16, lens=(12, 700, 256, 33, 1025), seed=23)
    d = DevCase(c)
    full = to_host_bits(d.decode())
    for b in range(c.B):
        out = torch.empty_like(d.q[b:b + 1])
        pa.paged_decode_attention(d.q[b:b + 1].contiguous(), d.kc, d.vc, d.bt[b:b + 1].contiguous(),
                                  d.lens[b:b + 1].contiguous(), c.scale, out)
        assert np.array_equal(to_host_bits(out)[0], full[b]), b


def test_decode_empty_context_gives_zeros_and_repeat_is_deterministic():
    c = small(P=16, Hq=8, Hkv=2, lens=(300, 5, 1), seed=24)
    d = DevCase(c)
    lens = d.lens.clone()
    lens[1] = 0
    out = torch.full_like(d.q, 7.0)
    pa.paged_decode_attention(d.q, d.kc, d.vc, d.bt, lens, c.scale, out)
    o = to_host_bits(out)
    assert np.all(o[1] == 0)
    ref = decode_ref(c)
    assert_close(out, ref, "bf16", "len0 batch", rows=[0, 2])
    out2 = torch.empty_like(d.q)
    pa.paged_decode_attention(d.q, d.kc, d.vc, d.bt, lens, c.scale, out2)
    assert np.array_equal(to_host_bits(out2), o)


def _decode_with_workspace(d, ws):
    """pa_paged_decode_attention through the C ABI with a caller-supplied workspace."""
    c = d.case
    lib = pa.load_library()
    out = torch.empty_like(d.q)
    N, P, Hkv, D = d.kc.shape
    code = 1 if c.dtype == "bf16" else 0
    st = lib.pa_paged_decode_attention(d.q.data_ptr(), d.kc.data_ptr(), d.vc.data_ptr(), d.bt.data_ptr(),
                                       d.lens.data_ptr(), float(c.scale), out.data_ptr(), c.B, d.q.shape[1], Hkv,
                                       D, P, N, d.bt.shape[1], code, ws.data_ptr(), ws.numel(),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    return out


def test_decode_any_workspace_contents():
    """The work queues reset themselves in every launch: a workspace holding
    random bytes, all ones, or another call's state gives the same bits."""
    c = small(P=16, lens=(1, 40, 256, 257, 700, 1500, 3000, 90), seed=26)
    d = DevCase(c)
    ref = to_host_bits(d.decode())
    assert_close(d.decode(), decode_ref(c), "bf16", "workspace")
    need = pa.decode_workspace_size(c.B, c.num_q_heads, c.head_dim, c.block_size, c.max_blocks_per_seq)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    for fill in ("random", "ones", "reuse", "reuse"):
        if fill == "random":
            ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=gen)
        elif fill == "ones":
            ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)
        out = _decode_with_workspace(d, ws)
        assert np.array_equal(to_host_bits(out), ref), fill


def test_decode_large_batch_plan_kernel_path_bitwise():
    """Above 1024 requests a plan kernel lists the items; below, the
    workgroups do.  Both must give each request the same bits (the split
    depends on its length only), and match the oracle."""
    rng = np.random.default_rng(27)
    lens = rng.integers(1, 800, size=1100)
    lens[:6] = [1, 16, 255, 256, 257, 799]
    c = small(P=16, Hq=8, Hkv=2, D=64, lens=tuple(int(x) for x in lens), seed=27)
    d = DevCase(c)
    full = to_host_bits(d.decode())
    pick = [0, 1, 2, 3, 4, 5, 517, 1023, 1024, 1099]
    assert_close(d.decode(), decode_ref(c, select=pick), "bf16", "B=1100", rows=pick)
    for lo, hi in ((0, 300), (1000, 1100)):
        out = torch.empty_like(d.q[lo:hi])
        pa.paged_decode_attention(d.q[lo:hi].contiguous(), d.kc, d.vc, d.bt[lo:hi].contiguous(),
                                  d.lens[lo:hi].contiguous(), c.scale, out)
        assert np.array_equal(to_host_bits(out), full[lo:hi]), (lo, hi)


def test_decode_graph_replays_match_eager():
    """Captured in a HIP graph, every replay gets a new dispatch id and so
    resets the queues again: each replay equals the eager result, with other
    eager decode calls and synchronisations in between."""
    c = small(P=16, lens=(5, 300, 1025, 4000, 77, 512), seed=28)
    d = DevCase(c)
    c2 = small(P=16, lens=(900, 3, 2048), seed=29)
    d2 = DevCase(c2)
    ref = to_host_bits(d.decode())
    ref2 = to_host_bits(d2.decode())
    out = torch.empty_like(d.q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pa.paged_decode_attention(d.q, d.kc, d.vc, d.bt, d.lens, c.scale, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.paged_decode_attention(d.q, d.kc, d.vc, d.bt, d.lens, c.scale, out)
    for rep in range(4):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(out), ref), rep
        assert np.array_equal(to_host_bits(d2.decode()), ref2), rep


def test_graphs_of_two_sizes_on_one_pool_replay_correctly():
    """Two graphs captured on one memory pool, the small batch first: the
    larger batch's capture replaces the cached workspace, and the smaller
    graph's workspace must stay allocated, so that a third capture on the same
    pool cannot take its memory.  Replays of all three, interleaved, keep
    both outputs equal to the eager results and the third graph's tensor
    intact."""
    ca = small(P=16, lens=(5, 300, 77), seed=30)
    cb = small(P=16, lens=tuple(range(200, 8200, 50)), seed=31)
    da, db = DevCase(ca), DevCase(cb)
    ref_a, ref_b = to_host_bits(da.decode()), to_host_bits(db.decode())
    out_a, out_b = torch.empty_like(da.q), torch.empty_like(db.q)
    need_a = pa.decode_workspace_size(ca.B, ca.num_q_heads, ca.head_dim, 16, ca.max_blocks_per_seq)
    need_b = pa.decode_workspace_size(cb.B, cb.num_q_heads, cb.head_dim, 16, cb.max_blocks_per_seq)
    assert need_b > 2 * need_a
    torch.cuda.synchronize()
    pool = torch.cuda.graph_pool_handle()
    ga, gb, gc = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga, pool=pool):
        pa.paged_decode_attention(da.q, da.kc, da.vc, da.bt, da.lens, ca.scale, out_a)
    with torch.cuda.graph(gb, pool=pool):
        pa.paged_decode_attention(db.q, db.kc, db.vc, db.bt, db.lens, cb.scale, out_b)
    with torch.cuda.graph(gc, pool=pool):
        x = torch.full((need_a,), 7, dtype=torch.uint8, device=DEV)
    for rep in range(3):
        out_a.fill_(0)
        out_b.fill_(0)
        gc.replay()
        ga.replay()
        gb.replay()
        ga.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(out_a), ref_a), rep
        assert np.array_equal(to_host_bits(out_b), ref_b), rep
        assert bool((x == 7).all()), rep
        assert np.array_equal(to_host_bits(da.decode()), ref_a), rep


def _scale_bf16(bits: np.ndarray, pow2: int) -> np.ndarray:
    """bf16 bits times 2**pow2 (exact while in range)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** pow2)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_decode_values_beyond_fp16_range():
    """bf16 values far above 65504 (up to ~2^24 here), with the magnitude
    changing from partition to partition inside a request: the partial results
    of several-partition requests must neither overflow nor be weighted wrongly.
    Attention is homogeneous in V, so each request is compared at the usual bf16
    tolerance after dividing both sides by its largest power-of-two factor."""
    lens = (300, 1025, 700, 40, 512)
    pow2 = ([22, 22], [20, 17, 20, 0, 16], [0, 0, 0], [24], [17, 16])  # per 256-token partition
    c = small(P=16, Hq=8, Hkv=2, lens=lens, seed=25)
    row = 0
    for L, ps in zip(lens, pow2):
        for j, e in enumerate(ps):
            lo, hi = row + 256 * j, row + min(L, 256 * (j + 1))
            c.v_tok[lo:hi] = _scale_bf16(c.v_tok[lo:hi], e)
        row += L
    d = DevCase(c)
    out = d.decode()
    ref = decode_ref(c)
    assert np.all(np.isfinite(ref)) and np.abs(ref).max() > 1e5
    S = np.array([2.0 ** max(ps) for ps in pow2])
    got = out.float() / torch.as_tensor(S, dtype=torch.float32, device=DEV)[:, None, None]
    assert_close(got, ref / S[:, None, None], "bf16", "large values")


# ----------------------------------------------------------------------------
# copy-on-write block copies and prefix sharing
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,P,H,D", [("bf16", 16, 8, 128), ("f32", 7, 2, 64), ("bf16", 1, 4, 64)])
def test_copy_blocks_bit_exact(dtype, P, H, D):
    N = 97
    rng = np.random.default_rng(P * 31 + D)
    bits = np.uint16 if dtype == "bf16" else np.uint32
    kc = rng.integers(0, np.iinfo(bits).max, size=(N, P, H, D), dtype=bits, endpoint=True)
    vc = rng.integers(0, np.iinfo(bits).max, size=(N, P, H, D), dtype=bits, endpoint=True)
    perm = rng.permutation(N)
    pairs = np.stack([perm[:30], perm[30:60]], axis=1).astype(np.int32)  # distinct, no dst is a src
    pairs[3] = (-1, perm[70])
    pairs[7] = (perm[71], -5)
    if dtype == "f32":
        kc, vc = kc.view(np.float32), vc.view(np.float32)
    want_k, want_v = ref_copy_blocks(kc, vc, pairs)
    dk, dv = to_dev(kc, dtype), to_dev(vc, dtype)
    # out-of-range pairs are skipped, never followed
    gpu_pairs = np.concatenate([pairs, [[N, perm[72]], [perm[73], N + 3]]]).astype(np.int32)
    pa.copy_blocks(dk, dv, idx(gpu_pairs))
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(dk).view(bits), want_k.view(bits))
    assert np.array_equal(to_host_bits(dv).view(bits), want_v.view(bits))


def _prefix_case(P, S, tails, dtype="bf16", Hq=32, Hkv=8, D=128, seed=0):
    return shared_prefix_case(dtype=dtype, block_size=P, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              prefix_len=S, tail_lens=tails, seed=seed)


def _pairs(c, dup):
    if dup:
        return [(int(c.shared_blocks[i]), int(c.dup_blocks[b, i])) for b in range(1, c.B)
                for i in range(len(c.shared_blocks))]
    return [(int(c.shared_blocks[-1]), int(c.cow_blocks[b])) for b in range(c.B) if c.cow_blocks[b] >= 0]


def _oracle_prefix(c, table, pairs):
    from oracle import ref_reshape_and_cache
    from workloads import nan_pool
    P, S = c.block_size, c.prefix_len
    kc = nan_pool(c.num_blocks, P, c.num_kv_heads, c.head_dim, c.dtype)
    vc = kc.copy()
    kc, vc = ref_reshape_and_cache(c.k_tok[:S], c.v_tok[:S], ref_slot_mapping(table[:1], [0, S], [S], P), kc, vc)
    if pairs:
        kc, vc = ref_copy_blocks(kc, vc, pairs)
    rows = np.concatenate([np.arange(c.cu_ctx[b] + S, c.cu_ctx[b + 1]) for b in range(c.B)]).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(c.tail_lens)])
    kc, vc = ref_reshape_and_cache(c.k_tok[rows], c.v_tok[rows], ref_slot_mapping(table, cu, c.context_lens, P),
                                   kc, vc)
    return kc, vc


def _gpu_prefix(c, table, pairs):
    P, S = c.block_size, c.prefix_len
    kc, vc = dev_nan_pool(c), dev_nan_pool(c)
    bt = idx(table)
    slots = pa.slot_mapping(bt[:1].contiguous(), idx([0, S]), idx([S]), P, S)
    pa.reshape_and_cache(to_dev(c.k_tok[:S], c.dtype), to_dev(c.v_tok[:S], c.dtype), slots, kc, vc)
    if pairs:
        pa.copy_blocks(kc, vc, idx(np.array(pairs, dtype=np.int32)))
    rows = np.concatenate([np.arange(c.cu_ctx[b] + S, c.cu_ctx[b + 1]) for b in range(c.B)]).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(c.tail_lens)])
    slots = pa.slot_mapping(bt, idx(cu), idx(c.context_lens), P, len(rows))
    pa.reshape_and_cache(to_dev(c.k_tok[rows], c.dtype), to_dev(c.v_tok[rows], c.dtype), slots, kc, vc)
    q = to_dev(c.q, c.dtype)
    out = torch.empty_like(q)
    pa.paged_decode_attention(q, kc, vc, bt, idx(c.context_lens), c.scale, out)
    return kc, vc, out


@pytest.mark.parametrize("P,S,tails", [(16, 300, (50, 0, 700, 9)), (16, 512, (1, 300)), (7, 100, (20, 257, 3))])
def test_prefix_sharing_copy_on_write(P, S, tails):
    """Requests share a prefix's blocks; the partly filled one is copied before
    the others append.  The pools match the oracle's bit for bit, the outputs
    match the oracle, and sharing gives the same bits as private copies."""
    c = _prefix_case(P, S, tails, seed=P + S)
    kc, vc, out = _gpu_prefix(c, c.block_table, _pairs(c, False))
    ok, ov = _oracle_prefix(c, c.block_table, _pairs(c, False))
    assert np.array_equal(to_host_bits(kc), ok) and np.array_equal(to_host_bits(vc), ov)
    assert_close(out, ref_decode(c.q, ok, ov, c.block_table, c.context_lens, c.scale), c.dtype, "shared prefix")
    _, _, dup = _gpu_prefix(c, c.dup_table, _pairs(c, True))
    assert np.array_equal(to_host_bits(dup), to_host_bits(out))


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("G,Hkv,D,P", [(4, 2, 128, 16), (1, 3, 64, 16), (2, 2, 128, 7), (8, 1, 64, 1),
                                       (3, 2, 128, 64), (4, 8, 64, 16)])
def test_prefill_matches_oracle(G, Hkv, D, P):
    # chunks: whole prompt; chunk over a prefix; T not a multiple of the q tile;
    # a single new token; a long chunk over a long prefix
    lens = (70, 300, 45, 9, 620)
    qlens = (70, 100, 33, 1, 300)
    c = small(P=P, Hq=G * Hkv, Hkv=Hkv, D=D, lens=lens, qlens=qlens, seed=30 + G * D)
    d = DevCase(c)
    kc, vc = oracle_pool(c)
    ref = ref_prefill(c.q, kc, vc, c.cu_seqlens, c.block_table, c.context_lens, c.scale)
    assert_close(d.prefill(), ref, "bf16", f"prefill G={G} D={D} P={P}")


def test_prefill_largest_group_and_longest_table():
    """The limits of the prefill call: a GQA group of 64 (an item is 4 tokens
    x 64 heads) and a request whose block table has the largest supported
    length (16384 entries at P = 1, all staged on chip)."""
    c = small(P=16, Hq=64, Hkv=1, D=64, lens=(300, 1), qlens=(37, 1), seed=42)
    d = DevCase(c)
    kc, vc = oracle_pool(c)
    ref = ref_prefill(c.q, kc, vc, c.cu_seqlens, c.block_table, c.context_lens, c.scale)
    assert_close(d.prefill(), ref, "bf16", "G=64")
    c = small(P=1, Hq=4, Hkv=1, D=64, lens=(16384,), qlens=(40,), seed=43)
    assert c.max_blocks_per_seq == 16384
    d = DevCase(c)
    rows = [0, 17, 39]
    kc, vc = oracle_pool(c)
    ref = ref_prefill(c.q, kc, vc, c.cu_seqlens, c.block_table, c.context_lens, c.scale, rows=rows)
    assert_close(d.prefill(), ref, "bf16", "16384 blocks", rows=rows)


def test_prefill_single_token_matches_decode():
    c = small(P=16, lens=(77, 400, 1), seed=40)
    d = DevCase(c)
    dec = d.decode()
    pre = d.prefill()
    ref = decode_ref(c)
    assert_close(pre, ref, "bf16", "prefill T=1")
    assert_close(dec, ref, "bf16", "decode")


def test_prefill_chunked_matches_one_shot():
    """The same prompt prefilled in chunks (scatter each chunk, then attend)
    gives the rows of a one-shot prefill, within tolerance of the oracle."""
    one = small(P=16, Hq=8, Hkv=2, lens=(390,), qlens=(390,), seed=41)
    d = DevCase(one)
    whole = d.prefill()
    kc, vc = oracle_pool(one)
    ref = ref_prefill(one.q, kc, vc, one.cu_seqlens, one.block_table, one.context_lens, one.scale)
    assert_close(whole, ref, "bf16", "one shot")
    kpool = torch.full_like(d.kc, float("nan"))
    vpool = torch.full_like(d.vc, float("nan"))
    start = 0
    pieces = []
    k_all = to_dev(one.k_tok, "bf16")
    v_all = to_dev(one.v_tok, "bf16")
    for T in (100, 1, 130, 159):
        L = start + T
        slots = pa.slot_mapping(d.bt, idx([0, T]), idx([L]), 16, T)
        pa.reshape_and_cache(k_all[start:L].contiguous(), v_all[start:L].contiguous(), slots, kpool, vpool)
        out = torch.empty_like(d.q[start:L])
        pa.paged_prefill_attention(d.q[start:L].contiguous(), kpool, vpool, idx([0, T]), d.bt, idx([L]),
                                   one.scale, out)
        pieces.append(out)
        start = L
    assert_close(torch.cat(pieces), ref, "bf16", "chunked")


def mixed_step(c):
    """One mixed step: scatter every new token, prefill the first 16 requests'
    chunks, decode the other 48 (the workload's order)."""
    d = DevCase(c)
    npf = 16
    cu = c.cu_seqlens
    qp = d.q[: cu[npf]].contiguous()
    outp = torch.empty_like(qp)
    pa.paged_prefill_attention(qp, d.kc, d.vc, d.cu[: npf + 1].contiguous(), d.bt[:npf].contiguous(),
                               d.lens[:npf].contiguous(), c.scale, outp)
    qd = d.q[cu[npf]:].contiguous()
    outd = torch.empty_like(qd)
    pa.paged_decode_attention(qd, d.kc, d.vc, d.bt[npf:].contiguous(), d.lens[npf:].contiguous(), c.scale, outd)
    return d, outp, outd


@pytest.mark.parametrize("P", [1, 16, 64])
def test_mixed_step_full_size_sampled(P):
    """The mixed chunked-prefill + decode workload at full size, block sizes
    1, 16, 64; the oracle checks sampled prefill rows and decode requests."""
    c = config_case(4, block_size=P)
    d, outp, outd = mixed_step(c)
    kc, vc = oracle_pool(c)
    cu = c.cu_seqlens
    rng = np.random.default_rng(7)
    rows = []
    for b in range(16):  # first, last and two random rows of each chunk
        s, e = int(cu[b]), int(cu[b + 1])
        rows += [s, e - 1] + rng.integers(s, e, 2).tolist()
    rows = sorted(set(rows))
    refp = ref_prefill(c.q, kc, vc, cu, c.block_table, c.context_lens, c.scale, rows=rows)
    assert_close(outp, refp[: cu[16]], "bf16", f"mixed prefill P={P}", rows=rows)
    pick = sorted(set([0, 1, 47] + rng.integers(0, 48, 5).tolist()))
    qdec = c.q[cu[16:64]]
    refd = ref_decode(qdec, kc, vc, c.block_table[16:], c.context_lens[16:], c.scale, select=pick)
    assert_close(outd, refd, "bf16", f"mixed decode P={P}", rows=pick)


# ----------------------------------------------------------------------------
# fp8 (OCP E4M3) pools
# ----------------------------------------------------------------------------

from oracle import ref_dequantize, ref_reshape_and_cache_fp8  # noqa: E402


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_reshape_and_cache_fp8_bit_exact(src):
    N, P, H, D = 40, 7, 4, 64
    rng = np.random.default_rng(50)
    T = 150
    x = rng.standard_normal((T, H, D)).astype(np.float32) * np.float32(3.0) ** rng.integers(-9, 9, (T, H, D))
    x[0, 0, :8] = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e30, -1e30, 2.0 ** -20]
    if src == "bf16":
        from workloads import to_bf16_bits
        xb = to_bf16_bits(np.nan_to_num(x, nan=0.0, posinf=3e38, neginf=-3e38))
        xb[0, 0, :8] = [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC1, 0x7149, 0xF149, 0x3580]
        k = xb
        v = xb[::-1].copy()
    else:
        k, v = x, x[::-1].copy()
    ks, vs = fp8_scales(H, 51, 0.01, 2.0), fp8_scales(H, 52, 0.01, 2.0)
    slots = rng.permutation(N * P)[:T].astype(np.int32)
    slots[5] = -1
    kc0 = rng.integers(0, 256, (N, P, H, D), dtype=np.uint8)
    vc0 = rng.integers(0, 256, (N, P, H, D), dtype=np.uint8)
    want_k, want_v = ref_reshape_and_cache_fp8(k, v, slots, kc0, vc0, ks, vs)
    dk = torch.from_numpy(kc0).to(DEV)
    dv = torch.from_numpy(vc0).to(DEV)
    pa.reshape_and_cache(to_dev(k, src), to_dev(v, src), idx(slots), dk, dv, torch.from_numpy(ks).to(DEV),
                         torch.from_numpy(vs).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), want_k)
    assert np.array_equal(dv.cpu().numpy(), want_v)


@pytest.mark.parametrize("G,Hkv,D,P", [(4, 8, 128, 16), (1, 4, 64, 16), (8, 2, 128, 7), (3, 2, 64, 1),
                                       (16, 1, 128, 64), (4, 2, 128, 48), (2, 2, 64, 32)])
def test_decode_fp8_matches_oracle(G, Hkv, D, P):
    # fp8 tiles hold 32 tokens: P = 16 splits each tile over two blocks, P = 48
    # puts tiles at block offsets 0, 32 and 16 (some straddling), P = 32 and 64
    # hold whole tiles
    c = small(P=P, Hq=G * Hkv, Hkv=Hkv, D=D, lens=(1, 16, 255, 256, 257, 700, 1500), seed=60 + G * D + P)
    f = Fp8Case(c, fp8_scales(Hkv, 61), fp8_scales(Hkv, 62))
    # the pools hold exactly the oracle's codes
    kc0 = np.full((c.num_blocks, P, Hkv, D), 0x7E, dtype=np.uint8)
    kp, vp, cu_pre, lens_pre = c.prefix()
    ok, ov = ref_reshape_and_cache_fp8(kp, vp, ref_slot_mapping(c.block_table, cu_pre, lens_pre, P), kc0, kc0,
                                       f.ks, f.vs)
    kn, vn = c.new_kv()
    ok, ov = ref_reshape_and_cache_fp8(kn, vn, ref_slot_mapping(c.block_table, c.cu_seqlens, c.context_lens, P),
                                       ok, ov, f.ks, f.vs)
    assert np.array_equal(f.kc.cpu().numpy(), ok) and np.array_equal(f.vc.cpu().numpy(), ov)
    assert_close(f.decode(), f.reference(), "bf16", f"fp8 G={G} D={D} P={P}")


def test_decode_fp8_llama3_8b_full_size_sampled():
    """The full Llama-3-8B-shaped batch with fp8 pools (quantised through the
    HIP scatter), in the launch configuration the fp8 benchmark times; the
    oracle checks 12 requests on the dequantised pools."""
    c = config_case(3)
    f = Fp8Case(c, fp8_scales(8, 97), fp8_scales(8, 98))
    out = f.decode()
    order = np.argsort(c.context_lens)
    rng = np.random.default_rng(124)
    pick = sorted(set([int(order[0]), int(order[1]), int(order[-1]), int(order[-2])]
                      + rng.choice(c.B, 8, replace=False).tolist()))
    assert_close(out, f.reference(select=pick), "bf16", "fp8 llama3_8b", rows=pick)


def test_decode_fp8_long_contexts_and_batch_invariance_bitwise():
    c = small(P=16, Hq=32, Hkv=8, D=128, lens=(8192, 3000, 17, 4097, 256), seed=63)
    f = Fp8Case(c, fp8_scales(8, 64), fp8_scales(8, 65))
    full = f.decode()
    assert_close(full, f.reference(), "bf16", "fp8 long contexts")
    fb = to_host_bits(full)
    for b in range(c.B):
        one = f.decode(f.q[b:b + 1].contiguous(), f.bt[b:b + 1].contiguous(), f.lens[b:b + 1].contiguous())
        assert np.array_equal(to_host_bits(one)[0], fb[b]), b


def test_copy_blocks_fp8_pools():
    N, P, H, D = 50, 16, 8, 128
    rng = np.random.default_rng(66)
    kc = rng.integers(0, 256, (N, P, H, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (N, P, H, D), dtype=np.uint8)
    pairs = np.array([[3, 40], [7, 41], [-1, 42]], dtype=np.int32)
    wk, wv = ref_copy_blocks(kc, vc, pairs)
    dk, dv = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    pa.copy_blocks(dk, dv, idx(pairs))
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), wk) and np.array_equal(dv.cpu().numpy(), wv)


@pytest.mark.parametrize("G,Hkv,D,P", [(4, 2, 128, 16), (1, 3, 64, 16), (2, 2, 128, 7), (8, 1, 64, 1)])
def test_prefill_fp8_matches_oracle(G, Hkv, D, P):
    lens = (70, 300, 45, 9, 620)
    qlens = (70, 100, 33, 1, 300)
    c = small(P=P, Hq=G * Hkv, Hkv=Hkv, D=D, lens=lens, qlens=qlens, seed=70 + G * D + P)
    f = Fp8Case(c, fp8_scales(Hkv, 71), fp8_scales(Hkv, 72))
    out = torch.empty_like(f.q)
    pa.paged_prefill_attention(f.q, f.kc, f.vc, idx(c.cu_seqlens), f.bt, f.lens, c.scale, out, f.dks, f.dvs)
    kc, vc = f.kc.cpu().numpy(), f.vc.cpu().numpy()
    ref = ref_prefill(c.q, ref_dequantize(kc, f.ks), ref_dequantize(vc, f.vs), c.cu_seqlens, c.block_table,
                      c.context_lens, c.scale)
    assert_close(out, ref, "bf16", f"fp8 prefill G={G} D={D} P={P}")


def test_check_metadata_flags_each_rule():
    c = small(P=16, Hq=8, Hkv=2, lens=(40, 300, 17), qlens=(5, 300, 1), seed=80)
    bt, lens, cu = idx(c.block_table), idx(c.context_lens), idx(c.cu_seqlens)
    N, P, T = c.num_blocks, c.block_size, c.T_total
    slots = pa.slot_mapping(bt, cu, lens, P, T)
    assert pa.check_metadata(bt, lens, N, P, cu, slots) == (0, 0)
    bad = lens.clone()
    bad[1] = c.max_blocks_per_seq * P + 1
    assert pa.check_metadata(bt, bad, N, P)[0] == 1
    bt2 = bt.clone()
    bt2[0, 1] = N
    bt2[2, 0] = -3
    assert pa.check_metadata(bt2, lens, N, P) == (2, 2)
    bt3 = bt.clone()
    bt3[0, c.max_blocks_per_seq - 1] = -1  # past the request's blocks: never read, not an error
    assert pa.check_metadata(bt3, lens, N, P) == (0, 0)
    cu2 = cu.clone()
    cu2[2] = cu2[1] - 1
    assert pa.check_metadata(bt, lens, N, P, cu2, slots)[0] & 4
    long_chunk = lens.clone()
    long_chunk[0] = 3  # 5 new tokens over a context of 3
    assert pa.check_metadata(bt, long_chunk, N, P, cu, slots)[0] & 8
    s2 = slots.clone()
    s2[3] = N * P
    s2[4] = -1  # padding is fine
    assert pa.check_metadata(bt, lens, N, P, cu, s2) == (16, 1)


# ----------------------------------------------------------------------------
# decode with append: the step's scatter and decode in one call
# ----------------------------------------------------------------------------

def prefix_pools(c, scales=(None, None)):
    """Pools holding only the cached prefix (positions < L - 1) of a decode case."""
    if scales[0] is not None:
        shape = (c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
        kc = torch.full(shape, 0x7E, dtype=torch.uint8, device=DEV)
        vc = torch.full(shape, 0x7E, dtype=torch.uint8, device=DEV)
    else:
        kc, vc = dev_nan_pool(c), dev_nan_pool(c)
    kp, vp, cu_pre, lens_pre = c.prefix()
    if len(kp):
        slots = pa.slot_mapping(idx(c.block_table), idx(cu_pre), idx(lens_pre), c.block_size, len(kp))
        pa.reshape_and_cache(to_dev(kp, c.dtype), to_dev(vp, c.dtype), slots, kc, vc, *scales)
    return kc, vc


def append_both_ways(c, q, kn, vn, bt, lens, scales=(None, None)):
    """(out, k pool, v pool) of the slot mapping + scatter + decode calls, and
    of one decode-with-append call, from the same prefix pools."""
    k1, v1 = prefix_pools(c, scales)
    slots = pa.slot_mapping(bt, idx(np.arange(c.B + 1)), lens, c.block_size, c.B)
    pa.reshape_and_cache(kn, vn, slots, k1, v1, *scales)
    o1 = torch.empty_like(q)
    pa.paged_decode_attention(q, k1, v1, bt, lens, c.scale, o1, *scales)
    k2, v2 = prefix_pools(c, scales)
    o2 = torch.empty_like(q)
    pa.paged_decode_append(q, kn, vn, k2, v2, bt, lens, c.scale, o2, *scales)
    torch.cuda.synchronize()
    return (o1, k1, v1), (o2, k2, v2)


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("kind,G,Hkv,D,P", [("bf16", 4, 8, 128, 16), ("f32", 1, 4, 64, 7), ("bf16", 4, 2, 64, 1),
                                            ("bf16", 8, 2, 128, 48), ("bf16", 3, 3, 64, 5), ("fp8", 4, 8, 128, 16),
                                            ("fp8-f32", 2, 2, 64, 3), ("fp8", 5, 3, 64, 32), ("fp8", 8, 1, 128, 48),
                                            ("bf16", 16, 1, 64, 16), ("bf16", 32, 1, 128, 16), ("fp8", 12, 2, 64, 7),
                                            ("fp8", 7, 4, 64, 16)])
def test_decode_append_equals_scatter_then_decode(kind, G, Hkv, D, P):
    """pa_paged_decode_append writes each request's new token at position L - 1
    and attends to it in one call: bit for bit the outputs and the pools of the
    slot mapping, the scatter and the decode call (tiles of the new token that
    straddle blocks, query-head groups past the first (G=32: two groups of
    16), groups of 8 and 16 heads, paired heads, fp8 codes quantised from bf16
    or fp32 rows), and the oracle."""
    fp8 = kind.startswith("fp8")
    c = small(dtype="f32" if kind == "f32" else "bf16", P=P, Hq=G * Hkv, Hkv=Hkv, D=D,
              lens=(1, 2, 16, 17, 31, 33, 255, 256, 257, 700, 1500), seed=70 + G * D + P)
    q, bt, lens = to_dev(c.q, c.dtype), idx(c.block_table), idx(c.context_lens)
    kn, vn = (to_dev(x, c.dtype) for x in c.new_kv())
    if kind == "fp8-f32":  # fp32 rows that bf16 cannot hold
        gen = torch.Generator(device=DEV)
        gen.manual_seed(7)
        kn = torch.randn(kn.shape, generator=gen, device=DEV, dtype=torch.float32)
        vn = torch.randn(vn.shape, generator=gen, device=DEV, dtype=torch.float32)
    ks, vs = fp8_scales(Hkv, 71), fp8_scales(Hkv, 72)
    scales = (torch.from_numpy(ks).to(DEV), torch.from_numpy(vs).to(DEV)) if fp8 else (None, None)
    (o1, k1, v1), (o2, k2, v2) = append_both_ways(c, q, kn, vn, bt, lens, scales)
    assert same_bits(k1, k2) and same_bits(v1, v2), "pools differ"
    assert same_bits(o1, o2), "outputs differ"
    if fp8:
        ref = ref_decode(c.q, ref_dequantize(k2.cpu().numpy(), ks), ref_dequantize(v2.cpu().numpy(), vs),
                         c.block_table, c.context_lens, c.scale)
        assert_close(o2, ref, "bf16", f"append {kind} G={G} D={D} P={P}")
    elif kind != "fp8-f32":
        assert_close(o2, decode_ref(c), c.dtype, f"append {kind} G={G} D={D} P={P}")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_decode_append_edge_metadata(kind):
    """A request with no context appends nothing and gives a zero row; a new
    token whose block id is out of range is not written (as the scatter skips
    its slot) and is masked; a length beyond the block table appends nothing.
    Both ways agree bit for bit on outputs and pools."""
    fp8 = kind == "fp8"
    c = small(P=16, Hq=8, Hkv=2, D=128, lens=(40, 300, 33, 700, 64), seed=77)
    q, bt_np, lens_np = to_dev(c.q, c.dtype), c.block_table.copy(), c.context_lens.copy()
    lens_np[0] = 0                         # no context
    bt_np[2, (33 - 1) // 16] = -1          # the new token's block id is invalid
    bt_np[4, (64 - 1) // 16] = c.num_blocks + 3
    lens_np[3] = bt_np.shape[1] * 16 + 5   # beyond the block table
    kn, vn = (to_dev(x, c.dtype) for x in c.new_kv())
    scales = ((torch.from_numpy(fp8_scales(2, 73)).to(DEV), torch.from_numpy(fp8_scales(2, 74)).to(DEV))
              if fp8 else (None, None))
    (o1, k1, v1), (o2, k2, v2) = append_both_ways(c, q, kn, vn, idx(bt_np), idx(lens_np), scales)
    assert same_bits(k1, k2) and same_bits(v1, v2), "pools differ"
    assert same_bits(o1, o2), "outputs differ"
    assert not o2[0].float().abs().sum().item()


@pytest.mark.parametrize("bad", [1 << 28, -(1 << 28), (1 << 31) - 1, -(1 << 31)])
def test_slot_mapping_huge_block_ids_store_nothing(bad):
    """A block id far outside the pool (whose slot would wrap in int32) gives a
    slot the scatter skips, so the new token lands in no block: the separate
    calls and decode with append leave the same pools, and both equal the
    prefix pools with only the valid requests' tokens written."""
    c = small(P=16, Hq=8, Hkv=2, D=128, lens=(40, 300, 33, 17), seed=82)
    bt_np = c.block_table.copy()
    for b in (1, 3):
        bt_np[b, (int(c.context_lens[b]) - 1) // 16] = bad
    bt, lens = idx(bt_np), idx(c.context_lens)
    slots = pa.slot_mapping(bt, idx(np.arange(c.B + 1)), lens, 16, c.B).cpu().numpy().astype(np.int64)
    N = c.num_blocks
    for b in (1, 3):
        assert slots[b] < 0 or slots[b] >= N * 16, (b, slots[b])
    q = to_dev(c.q, c.dtype)
    kn, vn = (to_dev(x, c.dtype) for x in c.new_kv())
    (o1, k1, v1), (o2, k2, v2) = append_both_ways(c, q, kn, vn, bt, lens)
    assert same_bits(k1, k2) and same_bits(v1, v2), "pools differ"
    assert same_bits(o1, o2), "outputs differ"
    k3, v3 = prefix_pools(c)
    good = ref_slot_mapping(c.block_table, np.arange(c.B + 1), c.context_lens, 16)
    good[[1, 3]] = -1
    pa.reshape_and_cache(kn, vn, idx(good), k3, v3)
    torch.cuda.synchronize()
    assert same_bits(k1, k3) and same_bits(v1, v3), "a token with an invalid block id was stored"


def test_decode_append_graph_replays():
    """Captured in a HIP graph, every replay of the append call writes the new
    tokens again and gives the eager result of the separate calls, with the
    pools reset to the prefix and other eager calls between replays."""
    c = small(P=16, lens=(5, 300, 1025, 77, 4000), seed=78)
    q, bt, lens = to_dev(c.q, c.dtype), idx(c.block_table), idx(c.context_lens)
    kn, vn = (to_dev(x, c.dtype) for x in c.new_kv())
    (o1, k1, v1), _ = append_both_ways(c, q, kn, vn, bt, lens)
    k0, v0 = prefix_pools(c)
    k2, v2 = k0.clone(), v0.clone()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pa.paged_decode_append(q, kn, vn, k2, v2, bt, lens, c.scale, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.paged_decode_append(q, kn, vn, k2, v2, bt, lens, c.scale, out)
    for rep in range(3):
        out.fill_(0)
        k2.copy_(k0)
        v2.copy_(v0)
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(out, o1) and same_bits(k2, k1) and same_bits(v2, v1), rep
        other = torch.empty_like(q)
        pa.paged_decode_attention(q, k1, v1, bt, lens, c.scale, other)
        torch.cuda.synchronize()
        assert same_bits(other, o1), rep


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_decode_append_large_batch_plan_kernel_path(kind):
    """Above 1024 requests the items come from the plan kernel: decode with
    append still equals the separate calls bit for bit (64-dim heads, read in
    pairs)."""
    rng = np.random.default_rng(79)
    lens = rng.integers(1, 700, size=1100)
    lens[:5] = [1, 16, 256, 257, 699]
    c = small(P=16, Hq=8, Hkv=2, D=64, lens=tuple(int(x) for x in lens), seed=79)
    q, bt, lens_d = to_dev(c.q, c.dtype), idx(c.block_table), idx(c.context_lens)
    kn, vn = (to_dev(x, c.dtype) for x in c.new_kv())
    scales = ((torch.from_numpy(fp8_scales(2, 80)).to(DEV), torch.from_numpy(fp8_scales(2, 81)).to(DEV))
              if kind == "fp8" else (None, None))
    (o1, k1, v1), (o2, k2, v2) = append_both_ways(c, q, kn, vn, bt, lens_d, scales)
    assert same_bits(k1, k2) and same_bits(v1, v2), "pools differ"
    assert same_bits(o1, o2), "outputs differ"


@pytest.mark.parametrize("append", [False, True])
def test_decode_one_and_two_tiles_in_flight_agree_bitwise(append):
    """bf16 batches whose shapes bound the work at 8192 items or fewer run with
    two tiles in flight per wave, larger ones with one; the items and their
    arithmetic are the same, so the bits are.  The same requests with a block
    table of 64 entries (40 x 4 partitions x 8 KV heads = 1280 items) and of
    512 entries (10240) take the two paths and must give identical outputs
    and pools, against the oracle too."""
    lens = [1, 15, 16, 17, 255, 256, 257, 300, 511, 512, 513, 700, 1000, 1024] + list(range(33, 1024, 39))
    c = small(P=16, Hq=32, Hkv=8, D=128, lens=tuple(lens), seed=95)
    assert c.max_blocks_per_seq <= 64
    outs = []
    for M in (64, 512):
        bt_np = np.full((c.B, M), c.filler_block, dtype=np.int32)
        bt_np[:, :c.max_blocks_per_seq] = c.block_table
        bt, lens_d = idx(bt_np), idx(c.context_lens)
        q = to_dev(c.q, c.dtype)
        out = torch.empty_like(q)
        if append:
            kc, vc = prefix_pools(c)
            kn, vn = (to_dev(x, c.dtype) for x in c.new_kv())
            pa.paged_decode_append(q, kn, vn, kc, vc, bt, lens_d, c.scale, out)
        else:
            d = DevCase(c)
            kc, vc = d.kc, d.vc
            pa.paged_decode_attention(q, kc, vc, bt, lens_d, c.scale, out)
        torch.cuda.synchronize()
        outs.append((out, kc, vc))
    (o1, k1, v1), (o2, k2, v2) = outs
    assert same_bits(o1, o2), "one and two tiles in flight differ"
    assert same_bits(k1, k2) and same_bits(v1, v2)
    assert_close(o1, decode_ref(c), c.dtype, f"decode append={append}")
