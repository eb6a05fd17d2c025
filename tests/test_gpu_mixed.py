"""GPU parity of the single-launch mixed batch (``paged_mixed_attention``):
decode requests (one-token chunks) and prefill chunks of one step in one
persistent launch.  It must compute what the varlen prefill call computes on
the same ragged batch: checked against the fp64 oracle (``ref_prefill``) within
the bf16 tolerance, and bit for bit against the separate calls whose work it
takes over (the prefill call for chunks of two or more tokens, the decode call
for one-token chunks).  All calls go through the C ABI (ctypes binding)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_48_amd as pa
from oracle import ref_dequantize, ref_prefill
from workloads import config_case, make_case

from gpu_util import DEV, DevCase, Fp8Case, assert_close, fp8_scales, idx, oracle_pool, to_host_bits

pytestmark = pytest.mark.gpu


def case(P=16, Hq=32, Hkv=8, D=128, lens=(), qlens=(), seed=0, **kw):
    return make_case(dtype="bf16", block_size=P, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                     context_lens=list(lens), query_lens=list(qlens), seed=seed, **kw)


def mixed(d, q=None, cu=None, bt=None, lens=None, out=None, scales=None):
    c = d.case
    q = d.q if q is None else q
    out = torch.empty_like(q) if out is None else out
    ks, vs = (None, None) if scales is None else scales
    pa.paged_mixed_attention(q, d.kc, d.vc, d.cu if cu is None else cu, d.bt if bt is None else bt,
                             d.lens if lens is None else lens, c.scale, out, ks, vs)
    return out


def separate(d, scales=None):
    """The rows of the separate calls: prefill for chunks of two or more tokens,
    decode (on the one-token requests alone) for the others."""
    c = d.case
    ks, vs = (None, None) if scales is None else scales
    out = torch.empty_like(d.q)
    pa.paged_prefill_attention(d.q, d.kc, d.vc, d.cu, d.bt, d.lens, c.scale, out, ks, vs)
    qlens = np.diff(c.cu_seqlens)
    one = np.flatnonzero(qlens == 1)
    if len(one):
        rows = idx(c.cu_seqlens[one])
        qd = d.q.index_select(0, rows.long()).contiguous()
        od = torch.empty_like(qd)
        pa.paged_decode_attention(qd, d.kc, d.vc, d.bt.index_select(0, idx(one).long()).contiguous(),
                                  d.lens.index_select(0, idx(one).long()).contiguous(), c.scale, od, ks, vs)
        out.index_copy_(0, rows.long(), od)
    return out


def oracle(c, rows=None):
    kc, vc = oracle_pool(c)
    return ref_prefill(c.q, kc, vc, c.cu_seqlens, c.block_table, c.context_lens, c.scale, rows=rows)


# decodes with one and several partitions (256 tokens each, a ragged tail),
# whole prompts, chunks over a prefix, a chunk of two tokens, a chunk not a
# multiple of the q tile, long chunks over long prefixes
LENS = (1, 70, 300, 45, 9, 620, 257, 1500, 256, 2, 3000, 800)
QLENS = (1, 70, 1, 33, 1, 300, 1, 1, 2, 2, 1, 130)


@pytest.mark.parametrize("G,Hkv,D,P", [(4, 8, 128, 16), (4, 2, 128, 16), (1, 3, 64, 16), (2, 2, 128, 7),
                                       (8, 1, 64, 1), (3, 2, 128, 64), (8, 4, 128, 16), (16, 2, 64, 16)])
def test_mixed_matches_oracle_and_separate_calls(G, Hkv, D, P):
    c = case(P=P, Hq=G * Hkv, Hkv=Hkv, D=D, lens=LENS, qlens=QLENS, seed=80 + G * D + P)
    d = DevCase(c)
    got = mixed(d)
    assert_close(got, oracle(c), "bf16", f"mixed G={G} D={D} P={P}")
    assert np.array_equal(to_host_bits(got), to_host_bits(separate(d))), "mixed differs from the separate calls"


def test_mixed_largest_group():
    """A GQA group of 64: decode items take the heads in 4 groups of 16, prefill
    items are 4 tokens x 64 heads."""
    c = case(Hq=64, Hkv=1, D=64, lens=(300, 1, 700, 257), qlens=(37, 1, 1, 2), seed=97)
    d = DevCase(c)
    got = mixed(d)
    assert_close(got, oracle(c), "bf16", "G=64")
    assert np.array_equal(to_host_bits(got), to_host_bits(separate(d)))


def test_mixed_all_decode_and_all_prefill_batches():
    lens = (1, 256, 257, 900, 4000, 33)
    for qlens, what in (((1,) * 6, "all decode"), ((1, 200, 2, 900, 64, 33), "all prefill but one"),
                        ((1, 2, 2, 2, 2, 2), "short chunks")):
        c = case(lens=lens, qlens=qlens, seed=90)
        d = DevCase(c)
        got = mixed(d)
        assert_close(got, oracle(c), "bf16", what)
        assert np.array_equal(to_host_bits(got), to_host_bits(separate(d))), what


def test_mixed_leaves_empty_and_invalid_chunks_untouched():
    """Chunks of zero tokens have no rows; a chunk longer than its context
    (T > L) is skipped, as by the prefill call: its rows keep what out held."""
    c = case(lens=(300, 50, 700, 1, 40), qlens=(1, 0, 20, 1, 5), seed=91)
    d = DevCase(c)
    lens = d.lens.clone()
    lens[4] = 3  # T = 5 > L = 3
    out = torch.full_like(d.q, 7.0)
    mixed(d, lens=lens, out=out)
    cu = c.cu_seqlens
    got = to_host_bits(out)
    seven = to_host_bits(torch.full_like(d.q[:1], 7.0))[0]
    for r in range(cu[4], cu[5]):
        assert np.array_equal(got[r], seven), r
    valid = list(range(0, cu[4]))
    assert_close(out, oracle(c, rows=valid), "bf16", "valid rows", rows=valid)


def test_mixed_any_workspace_contents_and_replays():
    """Queue counters carry a per-launch tag: a workspace of random bytes, all
    ones or another call's state gives the same bits, and so does every replay
    of a captured graph."""
    c = case(lens=LENS, qlens=QLENS, seed=92)
    d = DevCase(c)
    ref = to_host_bits(mixed(d))
    lib = pa.load_library()
    N, P, Hkv, D = d.kc.shape
    need = pa.mixed_workspace_size(c.B, c.num_q_heads, D, P, d.bt.shape[1])
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    for fill in ("random", "ones", "reuse", "reuse"):
        if fill == "random":
            ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=gen)
        elif fill == "ones":
            ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)
        out = torch.empty_like(d.q)
        st = lib.pa_paged_mixed_attention(d.q.data_ptr(), d.kc.data_ptr(), d.vc.data_ptr(), d.cu.data_ptr(),
                                          d.bt.data_ptr(), d.lens.data_ptr(), float(c.scale), out.data_ptr(), c.B,
                                          c.T_total, c.num_q_heads, Hkv, D, P, N, d.bt.shape[1], 1, ws.data_ptr(),
                                          ws.numel(), torch.cuda.current_stream().cuda_stream)
        assert st == 0, (st, lib.pa_last_error())
        assert np.array_equal(to_host_bits(out), ref), fill
    out = torch.empty_like(d.q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mixed(d, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mixed(d, out=out)
    for rep in range(3):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(out), ref), rep
        assert np.array_equal(to_host_bits(separate(d)), ref), rep


@pytest.mark.parametrize("P", [1, 16, 64])
def test_mixed_workload_full_size(P):
    """The mixed chunked-prefill + decode workload (16 chunks of 128-2048
    tokens over prefixes of up to 4096, 48 decodes of 256-8192) at full size:
    bit for bit the separate calls, and the oracle on sampled rows."""
    c = config_case(4, block_size=P)
    d = DevCase(c)
    got = mixed(d)
    assert np.array_equal(to_host_bits(got), to_host_bits(separate(d))), f"P={P}"
    cu = c.cu_seqlens
    rng = np.random.default_rng(8)
    rows = []
    for b in range(c.B):  # each chunk's first and last row and one random row
        s, e = int(cu[b]), int(cu[b + 1])
        rows += [s, e - 1, int(rng.integers(s, e))]
    rows = sorted(set(rows))
    assert_close(got, oracle(c, rows=rows), "bf16", f"mixed workload P={P}", rows=rows)


def test_mixed_large_batch():
    """1000 requests (the in-LDS plans handle up to 1024): mostly decodes of
    1 .. 600 tokens, every tenth a chunk of 2 .. 100 tokens over its prefix."""
    rng = np.random.default_rng(96)
    B = 1000
    lens = rng.integers(1, 600, size=B)
    qlens = np.ones(B, dtype=np.int64)
    pf = np.arange(0, B, 10)
    qlens[pf] = rng.integers(2, 100, size=len(pf))
    lens = np.maximum(lens, qlens)
    c = case(Hq=8, Hkv=2, D=64, lens=tuple(int(x) for x in lens), qlens=tuple(int(x) for x in qlens), seed=96)
    d = DevCase(c)
    got = mixed(d)
    assert np.array_equal(to_host_bits(got), to_host_bits(separate(d)))
    cu = c.cu_seqlens
    rows = sorted(set([0, 1, int(cu[-1]) - 1] + [int(cu[b]) for b in (5, 10, 500, 990, 999)]
                      + [int(cu[b + 1]) - 1 for b in (10, 990)]))
    assert_close(got, oracle(c, rows=rows), "bf16", "B=1000", rows=rows)


def test_mixed_fp8_pools():
    for G, Hkv, D, P in ((4, 8, 128, 16), (2, 2, 64, 7)):
        c = case(P=P, Hq=G * Hkv, Hkv=Hkv, D=D, lens=LENS, qlens=QLENS, seed=93 + D + P)
        f = Fp8Case(c, fp8_scales(Hkv, 94), fp8_scales(Hkv, 95))
        got = mixed(f, scales=(f.dks, f.dvs))
        kc, vc = f.kc.cpu().numpy(), f.vc.cpu().numpy()
        ref = ref_prefill(c.q, ref_dequantize(kc, f.ks), ref_dequantize(vc, f.vs), c.cu_seqlens, c.block_table,
                          c.context_lens, c.scale)
        assert_close(got, ref, "bf16", f"fp8 mixed G={G} D={D} P={P}")
        assert np.array_equal(to_host_bits(got), to_host_bits(separate(f, scales=(f.dks, f.dvs))))


def test_queue_giveup_is_reported(monkeypatch):
    """A wave that gives up waiting on a work queue leaves that queue's items
    uncomputed; the workspace's status word must say so.  PA_TEST_QUEUE_GIVEUP=1
    forces every claim to give up at once (every kernel still exits): the
    decode call reports bit 1 (with one and with two tiles in flight per wave:
    block tables of 512 and of 256 entries), the mixed call bits 1 and 2, the
    allocation-free call bit 1 in the static scratch.  Batches whose items are
    all dealt statically make no claim and lose nothing.  Normal calls leave
    the word clear and compute the right rows again."""
    c = case(lens=(5, 300, 1025, 4000, 77, 512, 2048, 700), qlens=(1, 1, 1, 300, 1, 100, 1, 1), seed=93)
    d = DevCase(c)
    ref = to_host_bits(separate(d))
    B, Hq, D, P, M = c.B, c.num_q_heads, c.head_dim, c.block_size, c.max_blocks_per_seq
    wsm = torch.empty(pa.mixed_workspace_size(B, Hq, D, P, M), dtype=torch.uint8, device=DEV)
    # 40 requests of 4000 tokens: 5000 items, more than the waves, so the queues are used
    dd = DevCase(case(lens=(4000,) * 40, qlens=(1,) * 40, seed=94, max_blocks_per_seq=512))
    cd = dd.case
    bt256 = dd.bt[:, :256].contiguous()
    outs = {w: torch.empty_like(dd.q) for w in (256, 512)}
    ws = {w: torch.empty(pa.decode_workspace_size(cd.B, Hq, D, P, w), dtype=torch.uint8, device=DEV)
          for w in (256, 512)}
    outm = torch.empty_like(d.q)
    tiny = DevCase(case(lens=(5, 300, 1025), qlens=(1, 1, 1), seed=96))
    wst = torch.empty(pa.decode_workspace_size(3, Hq, D, P, tiny.case.max_blocks_per_seq), dtype=torch.uint8,
                      device=DEV)
    outt = torch.empty_like(tiny.q)

    def run():
        for w, bt in ((256, bt256), (512, dd.bt)):
            pa.paged_decode_attention(dd.q, dd.kc, dd.vc, bt, dd.lens, cd.scale, outs[w], workspace=ws[w])
        pa.paged_decode_attention(tiny.q, tiny.kc, tiny.vc, tiny.bt, tiny.lens, tiny.case.scale, outt, workspace=wst)
        pa.paged_mixed_attention(d.q, d.kc, d.vc, d.cu, d.bt, d.lens, c.scale, outm, workspace=wsm)
        pa.paged_decode_attention_noalloc(dd.q, dd.kc, dd.vc, dd.bt, dd.lens, cd.scale, outs[512])

    def status():
        return (pa.workspace_status(ws[256]), pa.workspace_status(ws[512]), pa.workspace_status(wst),
                pa.workspace_status(wsm), pa.workspace_status(noalloc=True))

    status()  # a new workspace holds arbitrary bits: the first query clears them
    run()
    assert status() == (0, 0, 0, 0, 0)
    monkeypatch.setenv("PA_TEST_QUEUE_GIVEUP", "1")
    run()
    monkeypatch.delenv("PA_TEST_QUEUE_GIVEUP")
    assert status() == (1, 1, 0, 3, 1)
    run()
    assert status() == (0, 0, 0, 0, 0)
    assert np.array_equal(to_host_bits(outm), ref)
    assert np.array_equal(to_host_bits(outs[256]), to_host_bits(outs[512]))
