#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Headline workload: Llama-3-8B-shaped decode at large batch (32 layers, H_q=32,
H_kv=8, D=128, block size 16, B=256, log-normal context lengths with median
1024 and sigma 1, clipped to [16, 8192], pool at 90% occupancy), bf16.

One step = one decode step of the whole model's attention: for each of the 32
layers, one decode-with-append call, which writes the 256 new tokens' K/V to
the layer's pool and computes decode attention over it (bit for bit the
scatter followed by the decode call).  Every layer owns its pool, queries and
outputs, so no layer's data is still in the 256 MB Infinity Cache when it is
read.  The same run also times the step as separate calls (slot mapping, then
per layer reshape_and_cache and paged_decode_attention) and attention alone.

Prints ONE JSON line.  ``value`` is the algorithmic HBM bytes of the step
(KV read by decode + q/out + block table + lengths + the new rows) divided by
the step time, in GB/s.  ``roofline`` reports the decode partition kernel alone
(its average duration from HIP events recorded around it inside the timed
region).  ``cpu_baseline`` times the fp64 oracle on a bounded sample.

The default run (``--workload all``) also measures every other seeded workload
and adds them under ``workloads``: tiny (fp32), GPT-2-124M, Llama-3.2-1B, the
Llama-3-8B batch with fp8 pools, and the mixed chunked-prefill + decode step
(as prefill and decode calls, and as one mixed call).  Each entry gives KV
GB/s, us per layer-step (p10/p50/p90), decode tokens/s, the roofline fraction
of its dominant kernel and the oracle's time on the host cores.
"""

from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, AMD published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["all", "llama3_8b", "llama3_8b_fp8", "llama3_8b_g8", "tiny", "gpt2_124m",
                                           "llama32_1b", "mixed", "mixed_fp8", "mixed_single", "mixed_single_fp8",
                                           "cow", "copy"],
                    default="all")
    ap.add_argument("--layers", type=int, default=None, help="profile runs only: fewer layers")
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="no GPU run: turn the rocprofv3 CSVs under DIR into the summaries in profiles/")
    return ap.parse_args()


def decode_bytes(lens, P, Hq, Hkv, D, s, s_kv=None):
    """Algorithmic bytes one decode launch must move: every cached K and V row
    of every request (``s_kv`` bytes per element; 1 for fp8 pools), q and out
    (``s``), the used block-table entries and the lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    s_kv = s if s_kv is None else s_kv
    return int(lens.sum() * Hkv * D * 2 * s_kv + 2 * len(lens) * Hq * D * s
               + 4 * ((lens + P - 1) // P).sum() + 4 * len(lens))


def scatter_bytes(T, Hkv, D, s, s_kv=None):
    """New K and V rows read (``s``) and written (``s_kv``), plus the slots."""
    s_kv = s if s_kv is None else s_kv
    return int(2 * T * Hkv * D * (s + s_kv) + 4 * T)


def append_bytes(B, Hkv, D, s, s_kv=None):
    """The new K and V rows a decode-with-append launch reads (``s``) and writes (``s_kv``)."""
    s_kv = s if s_kv is None else s_kv
    return int(2 * B * Hkv * D * (s + s_kv))


def sources_sha(files) -> str:
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "paged_kv_cache_48_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profiles(files, key: str):
    """Measured HBM bytes per launch from profiles/traffic.json, if it was taken
    for the current sources of the kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(key)
    if not rec:
        return None
    if rec.get("source_sha256") != sources_sha(files):
        return None
    return rec.get("bytes_per_launch")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def host_line() -> str:
    return (f"host has {os.cpu_count()} logical CPUs, {len(os.sched_getaffinity(0))} allowed to this process, "
            f"BLAS threads {blas_threads()}")


def cpu_baseline_decode(case, budget_s, fp8=False):
    """The oracle (fp64 numpy) on a sample of the workload's requests, taken in a
    fixed random order until the time budget is spent; GB/s of algorithmic
    decode bytes, and the whole batch's layer-step time at that rate.  The
    sample's pool is built beforehand (untimed); fp8 pools are quantised with
    the oracle's encoder and dequantised once, also untimed, so the timed work
    is attention over the dequantised values."""
    from oracle import ref_decode, ref_dequantize, ref_reshape_and_cache, ref_slot_mapping
    from workloads import draw_values, make_case, nan_pool

    threads = blas_threads()
    order = np.random.default_rng(0).permutation(case.B)[:16 if fp8 else 64]
    sub = make_case(name="cpu_sample", dtype=case.dtype, block_size=case.block_size,
                    num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                    context_lens=case.context_lens[order], seed=0, values=not fp8)
    if fp8:  # random finite E4M3 codes, as the GPU benchmark's pools hold
        rng = np.random.default_rng(7)
        q = draw_values(rng, (sub.B, sub.num_q_heads, sub.head_dim), "bf16")
        shape = (sub.num_blocks, sub.block_size, sub.num_kv_heads, sub.head_dim)
        sc = np.full(sub.num_kv_heads, 0.02, dtype=np.float32)
        pools = []
        for _ in range(2):
            codes = rng.integers(0, 256, size=shape, dtype=np.uint8)
            codes[(codes & 0x7F) == 0x7F] -= 1
            pools.append(ref_dequantize(codes, sc))
        kc, vc = pools
    else:
        q = sub.q
        slots = ref_slot_mapping(sub.block_table, sub.cu_ctx, sub.context_lens, sub.block_size)
        kc = nan_pool(sub.num_blocks, sub.block_size, sub.num_kv_heads, sub.head_dim, sub.dtype)
        vc = kc.copy()
        kc, vc = ref_reshape_and_cache(sub.k_tok, sub.v_tok, slots, kc, vc)
    done = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:  # repeat passes over the sample until the budget is spent
        for i in range(sub.B):
            ref_decode(q, kc, vc, sub.block_table, sub.context_lens, sub.scale, select=[i])
            done.append(i)
    dt = time.perf_counter() - t0
    s_kv = 1 if fp8 else 2
    lens_done = sub.context_lens[done]
    nbytes = decode_bytes(lens_done, case.block_size, case.num_q_heads, case.num_kv_heads, case.head_dim, 2, s_kv)
    full = decode_bytes(case.context_lens, case.block_size, case.num_q_heads, case.num_kv_heads, case.head_dim, 2,
                        s_kv)
    rate = nbytes / dt
    return {
        "value": round(rate / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "us_per_layer_step": round(full / rate * 1e6, 1),
        "sample": f"{sub.B} requests drawn from the workload's {case.B} ({int(sub.context_lens.sum())} cached tokens, "
                  f"one layer{', fp8 pools dequantised beforehand' if fp8 else ''}), {len(done) / sub.B:.1f} passes "
                  f"of fp64 numpy decode in {dt:.1f} s; the whole batch's layer-step time is extrapolated at that "
                  f"rate; {host_line()}",
    }


def cpu_baseline_config(idx, repeats=3):
    """The oracle (fp64 numpy ``ref_decode``) on one whole layer-step of seeded
    workload ``idx`` (every layer has the same shape), median of ``repeats``;
    the pool is written beforehand by the oracle's own slot math and scatter
    (untimed)."""
    from oracle import ref_decode, ref_reshape_and_cache, ref_slot_mapping
    from workloads import config_case, nan_pool

    case = config_case(idx)
    kc = nan_pool(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim, case.dtype)
    vc = kc.copy()
    kp, vp, cu_pre, lens_pre = case.prefix()
    if len(kp):
        kc, vc = ref_reshape_and_cache(kp, vp, ref_slot_mapping(case.block_table, cu_pre, lens_pre,
                                                                 case.block_size), kc, vc)
    kn, vn = case.new_kv()
    kc, vc = ref_reshape_and_cache(kn, vn, ref_slot_mapping(case.block_table, case.cu_seqlens, case.context_lens,
                                                             case.block_size), kc, vc)
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        ref_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"us_per_layer_step": round(t * 1e6, 1), "cores": blas_threads(), "kind": "oracle",
            "sample": f"the whole batch ({case.B} requests, one layer), median of {repeats} runs of fp64 numpy "
                      f"decode ({', '.join(f'{x:.3f}' for x in times)} s); {host_line()}"}


def cpu_baseline_mixed(case, budget_s, npf=16):
    """The oracle (fp64 numpy ``ref_prefill``) on a sample of the mixed step: two
    of its prefill chunks and six of its decodes, rebuilt with values (untimed),
    then timed on random rows until the budget is spent.  The whole step's time
    is extrapolated from the sampled rows' share of the step's (row, visible
    key) pairs, which the oracle's work is proportional to."""
    from oracle import ref_prefill, ref_reshape_and_cache, ref_slot_mapping
    from workloads import make_case, nan_pool

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    pick = np.concatenate([rng.permutation(npf)[:2], npf + rng.permutation(case.B - npf)[:6]])
    sub = make_case(name="cpu_sample", dtype=case.dtype, block_size=case.block_size,
                    num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                    context_lens=case.context_lens[pick], query_lens=case.query_lens[pick], seed=0)
    kc = nan_pool(sub.num_blocks, sub.block_size, sub.num_kv_heads, sub.head_dim, sub.dtype)
    vc = kc.copy()
    kp, vp, cu_pre, lens_pre = sub.prefix()
    if len(kp):
        kc, vc = ref_reshape_and_cache(kp, vp, ref_slot_mapping(sub.block_table, cu_pre, lens_pre, sub.block_size),
                                       kc, vc)
    kn, vn = sub.new_kv()
    kc, vc = ref_reshape_and_cache(kn, vn, ref_slot_mapping(sub.block_table, sub.cu_seqlens, sub.context_lens,
                                                            sub.block_size), kc, vc)

    def visible(cu, lens):  # visible keys of every packed row
        T = np.diff(cu)
        return np.concatenate([lens[b] - T[b] + 1 + np.arange(T[b]) for b in range(len(T))])

    vis_sub = visible(sub.cu_seqlens, sub.context_lens.astype(np.int64))
    vis_full = visible(case.cu_seqlens, case.context_lens.astype(np.int64))
    decode_rows = sub.cu_seqlens[2:8].tolist()
    keys_done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        rows = sorted(set(rng.integers(0, int(sub.cu_seqlens[2]), 32).tolist() + decode_rows))
        ref_prefill(sub.q, kc, vc, sub.cu_seqlens, sub.block_table, sub.context_lens, sub.scale, rows=rows)
        keys_done += int(vis_sub[rows].sum())
    dt = time.perf_counter() - t0
    est_ms = dt / keys_done * float(vis_full.sum()) * 1e3
    return {
        "value": round(est_ms, 1),
        "unit": "ms/step",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"2 of the 16 prefill chunks and 6 of the 48 decodes, random rows for {dt:.1f} s "
                  f"({keys_done} (row, key) pairs of the step's {int(vis_full.sum())}), extrapolated to the "
                  f"whole step; host has {os.cpu_count()} logical CPUs",
    }


def hbm_read_ceiling(pa, dev, reps=10, nbytes=4 << 30):
    """Practical HBM read ceiling: the library's read-only streaming kernel
    over a 4 GiB buffer (16x the 256 MB Infinity Cache), best of a sweep of
    grid sizes, each timed with events over `reps` back-to-back launches."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = (0.0, 0)
    for wg in (256, 384, 512, 640, 768, 1024, 2048):
        pa.hbm_read(buf, sink, wg)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            pa.hbm_read(buf, sink, wg)
        t1.record()
        torch.cuda.synchronize()
        gbs = nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
        log(f"HBM read stream, {wg} workgroups: {gbs:.0f} GB/s")
        best = max(best, (gbs, wg))
    del buf
    torch.cuda.empty_cache()
    return {"kernel": "hbm_read_kernel (read-only stream, 16-byte nontemporal loads)", "gbs": round(best[0], 1),
            "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4), "bytes": nbytes, "workgroups": best[1]}


def graph_step_ms(step, reps, per_graph=1):
    """Per-step times (ms) from HIP-graph replays of ``per_graph`` consecutive
    steps, with an event between consecutive replays: the host launches one
    graph per replay, so short steps are not stretched by per-call host work."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            step()
    for _ in range(3):
        g.replay()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for k in range(reps):
        g.replay()
        marks[k + 1].record()
    torch.cuda.synchronize()
    return np.array([marks[k].elapsed_time(marks[k + 1]) / per_graph for k in range(reps)])


def eager_step_ms(step, reps):
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for k in range(reps):
        step()
        marks[k + 1].record()
    torch.cuda.synchronize()
    return np.array([marks[k].elapsed_time(marks[k + 1]) for k in range(reps)])


def guarded_kernel_ms(pa, call, reps, dev):
    """Average duration (ms) of the partition kernel of ``call(layer)``, from the
    events the library records around it.  Each call follows a read-only stream
    over 1 GiB (about 150 us of GPU work, which also evicts the Infinity
    Cache), so that the host has enqueued the call before the GPU reaches it;
    on an idle stream the start event would also count the host's launch time."""
    gbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for k in range(reps):
        pa.hbm_read(gbuf, sink, 512)
        with pa.kernel_timer(*evs[k]):
            call(k)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


SMALL_DECODE = {"tiny": 0, "gpt2_124m": 1, "llama32_1b": 2}
# A GQA group of 8: the Llama-3-8B batch, pool and lengths with 64 query
# heads over its 8 KV heads (the head layout of the 70B and 405B models), one
# layer.  Each KV slice is read once for all 8 query heads it serves.
WIDE_GROUP = {"llama3_8b_g8": dict(idx=3, Hq=64, layers=1)}


def bench_decode_small(args, name):
    """Decode step of a smaller seeded workload (tiny, GPT-2-124M, Llama-3.2-1B,
    or one layer of the GQA-8 batch): per layer one decode-with-append call,
    every layer with its own pool.  Steps take tens of microseconds per layer,
    less than the host needs to issue a call from Python, so the step is timed
    as HIP-graph replays (the eager time is reported beside it).  The partition
    kernel's own duration comes from the guarded event loop."""
    import paged_kv_cache_48_amd as pa
    from workloads import config_case

    wide = WIDE_GROUP.get(name)
    idx = wide["idx"] if wide else SMALL_DECODE[name]
    case = config_case(idx, values=False)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D, P, N = case.B, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size, case.num_blocks
    L = case.num_layers
    if wide:
        Hq, L = wide["Hq"], wide["layers"]
    tdt = torch.float32 if case.dtype == "f32" else torch.bfloat16
    s = 4 if case.dtype == "f32" else 2
    gen = torch.Generator(device=dev)
    bt = torch.as_tensor(case.block_table, device=dev)
    lens = torch.as_tensor(case.context_lens, device=dev)
    layers = []
    for layer in range(L):
        gen.manual_seed(2000 + 100 * idx + layer)
        kc = torch.randn((N, P, Hkv, D), generator=gen, device=dev, dtype=tdt)
        vc = torch.randn((N, P, Hkv, D), generator=gen, device=dev, dtype=tdt)
        q = torch.randn((B, Hq, D), generator=gen, device=dev, dtype=tdt)
        kn = torch.randn((B, Hkv, D), generator=gen, device=dev, dtype=tdt)
        vn = torch.randn((B, Hkv, D), generator=gen, device=dev, dtype=tdt)
        layers.append((kc, vc, q, kn, vn, torch.empty_like(q)))
    scale = case.scale

    def call(i):
        kc, vc, q, kn, vn, out = layers[i % L]
        pa.paged_decode_append(q, kn, vn, kc, vc, bt, lens, scale, out)

    def step():
        for i in range(L):
            call(i)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per_graph = max(1, 12 // L)  # at least 12 layer-calls per replay
    g_ms = graph_step_ms(step, args.steps, per_graph)
    e_ms = eager_step_ms(step, args.steps)
    kern_ms = guarded_kernel_ms(pa, call, max(args.steps, 2 * L), dev)
    dec_b = decode_bytes(case.context_lens, P, Hq, Hkv, D, s)
    step_bytes = L * (dec_b + scatter_bytes(B, Hkv, D, s))
    kern_b = dec_b + append_bytes(B, Hkv, D, s)
    ms = float(np.median(g_ms))
    achieved = kern_b / (kern_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(DECODE_SOURCES, f"decode_{name}") if wide else None
    log(f"{name}: {1e3 * ms / L:.2f} us/layer-step (graph), {1e3 * float(np.median(e_ms)) / L:.2f} (eager), "
        f"partition kernel {kern_ms * 1e3:.2f} us")
    return {
        "config": f"{name}: {L} layer(s) x paged decode with append, B={B}, H_q={Hq}, H_kv={Hkv}, D={D}, P={P}, "
                  f"N={N} blocks/layer, {case.dtype}, sum L = {int(case.context_lens.sum())}",
        "layers": L,
        "dtype": case.dtype,
        "timing": f"HIP-graph replays of {per_graph} step(s), {args.steps} replays",
        "kv_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "us_per_layer_step_p10_p50_p90": [round(float(x), 2) for x in np.percentile(1e3 * g_ms / L, [10, 50, 90])],
        "eager_us_per_layer_step_p50": round(1e3 * float(np.median(e_ms)) / L, 2),
        "decode_tokens_per_s": round(B / (ms * 1e-3), 1),
        "roofline_tokens_per_s": round(B / (step_bytes / (HBM_PEAK_GBS * 1e9)), 1),
        "roofline": {"kernel": f"decode_partition_kernel<{case.dtype},{D}> (decode with append)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": kern_b, "avg_launch_us": round(kern_ms * 1e3, 2),
                     "timing": "library events around the kernel, each launch after a 1 GiB read-only stream"},
    }


def bench_decode(args, ceiling_run=True):
    import paged_kv_cache_48_amd as pa
    from workloads import config_case

    case = config_case(3, block_size=args.block_size, values=False)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D, P, N, M = (case.B, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size,
                              case.num_blocks, case.max_blocks_per_seq)
    L = case.num_layers if args.layers is None else args.layers
    s = 2
    fp8 = args.workload == "llama3_8b_fp8"
    s_kv = 1 if fp8 else 2
    gen = torch.Generator(device=dev)
    bt = torch.as_tensor(case.block_table, device=dev)
    lens = torch.as_tensor(case.context_lens, device=dev)
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    layers = []
    for layer in range(L):
        gen.manual_seed(1000 + layer)
        if fp8:  # random finite E4M3 codes (the two NaN codes replaced by +-448)
            kc = torch.randint(0, 256, (N, P, Hkv, D), generator=gen, device=dev, dtype=torch.uint8)
            vc = torch.randint(0, 256, (N, P, Hkv, D), generator=gen, device=dev, dtype=torch.uint8)
            for t in (kc, vc):
                t[(t & 0x7F) == 0x7F] -= 1
        else:
            kc = torch.randn((N, P, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
            vc = torch.randn((N, P, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
        q = torch.randn((B, Hq, D), generator=gen, device=dev, dtype=torch.bfloat16)
        kn = torch.randn((B, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
        vn = torch.randn((B, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
        layers.append((kc, vc, q, kn, vn, torch.empty_like(q)))
    slots = torch.empty(B, dtype=torch.int32, device=dev)
    scale = case.scale
    # fp8 pools: per-KV-head scales (values of this size keep N(0,1) data in range)
    ks = torch.full((Hkv,), 0.02, dtype=torch.float32, device=dev) if fp8 else None
    vs = torch.full((Hkv,), 0.02, dtype=torch.float32, device=dev) if fp8 else None
    log(f"llama3_8b: {L} layer pools of {N} blocks ready ({'fp8 e4m3' if fp8 else 'bf16'})")

    # One decode step: per layer, the new tokens' K/V are written to the pool
    # and attended to in one call (paged_decode_append, bit for bit the scatter
    # followed by the decode call).
    def step(ev=None, timed_layer=-1):
        for i, (kc, vc, q, kn, vn, out) in enumerate(layers):
            if i != timed_layer:
                pa.paged_decode_append(q, kn, vn, kc, vc, bt, lens, scale, out, ks, vs)
            else:
                with pa.kernel_timer(*ev):
                    pa.paged_decode_append(q, kn, vn, kc, vc, bt, lens, scale, out, ks, vs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The decode partition kernel is timed by a pair of events that the library
    # records around it; one layer per step (a different one each step), so the
    # event records barely perturb the timed region.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    # one event between consecutive steps: the timed region is bracketed by
    # the first and the last, and each step's own time is the gap between two
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for k in range(args.steps):
        step(evs[k], k % L)
        marks[k + 1].record()
    torch.cuda.synchronize()
    ms_total = marks[0].elapsed_time(marks[-1])
    ms_step = ms_total / args.steps
    step_ms = np.array([marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps)])
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_avg_ms = float(np.mean(kern_ms))
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step, decode kernel {kern_avg_ms * 1e3:.1f} us avg")

    # attention only: each layer's decode call over pools that already hold
    # the new tokens (no append)
    def attn_only():
        for kc, vc, q, kn, vn, out in layers:
            pa.paged_decode_attention(q, kc, vc, bt, lens, scale, out, ks, vs)

    attn_only()
    amarks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    amarks[0].record()
    for k in range(args.steps):
        attn_only()
        amarks[k + 1].record()
    torch.cuda.synchronize()
    attn_ms = np.array([amarks[k].elapsed_time(amarks[k + 1]) for k in range(args.steps)])

    # the same step as separate calls: slot mapping, then per layer the
    # scatter (reshape_and_cache) and the decode call
    def separate_step():
        pa.slot_mapping(bt, cu, lens, P, B, out=slots)
        for kc, vc, q, kn, vn, out in layers:
            pa.reshape_and_cache(kn, vn, slots, kc, vc, ks, vs)
            pa.paged_decode_attention(q, kc, vc, bt, lens, scale, out, ks, vs)

    separate_step()
    smarks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    smarks[0].record()
    for k in range(args.steps):
        separate_step()
        smarks[k + 1].record()
    torch.cuda.synchronize()
    sep_ms = np.array([smarks[k].elapsed_time(smarks[k + 1]) for k in range(args.steps)])
    log(f"as separate calls: {float(np.mean(sep_ms)):.3f} ms/step")

    ceiling = hbm_read_ceiling(pa, dev) if ceiling_run else None
    if ceiling:
        log(f"HBM read ceiling: {ceiling['gbs']} GB/s ({ceiling['workgroups']} workgroups)")

    dec_b = decode_bytes(case.context_lens, P, Hq, Hkv, D, s, s_kv)
    sc_b = scatter_bytes(B, Hkv, D, s, s_kv)
    step_bytes = L * (dec_b + sc_b)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    kern_b = dec_b + append_bytes(B, Hkv, D, s, s_kv)  # the launch also reads and writes the new rows
    achieved = kern_b / (kern_avg_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(DECODE_SOURCES, "decode_llama3_8b_fp8" if fp8 else "decode_llama3_8b")
    res = {
        "metric": ("paged decode attn (fp8 e4m3 KV) KV GB/s (% HBM peak) + us/layer-step + tokens/s, Llama-3-8B shape"
                   if fp8 else "paged decode attn KV GB/s (% HBM peak) + us/layer-step, Llama-3-8B shape"),
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 KV, bf16 q/out" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"llama3_8b{'_fp8' if fp8 else ''} decode step: {L} layers x paged decode with append "
                        f"(the new token's K/V written and attended to in one call), B={B}, "
                        f"H_q={Hq}, H_kv={Hkv}, D={D}, P={P}, N={N} blocks/layer, context log-normal "
                        f"(median 1024, sigma 1) clipped to [16, 8192], sum L = {int(case.context_lens.sum())}",
            "global_batch": B,
            "layers": L,
            "block_size": P,
            "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "us_per_layer_step": round(1e3 * ms_step / L, 2),
        "us_per_layer_step_p10_p50_p90": [round(float(x), 2) for x in np.percentile(1e3 * step_ms / L, [10, 50, 90])],
        "attention_only_us_per_layer_step_p10_p50_p90": [round(float(x), 2)
                                                         for x in np.percentile(1e3 * attn_ms / L, [10, 50, 90])],
        "separate_calls_us_per_layer_step_p10_p50_p90": [round(float(x), 2)
                                                          for x in np.percentile(1e3 * sep_ms / L, [10, 50, 90])],
        "decode_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "roofline_tokens_per_s": round(B / (step_bytes / (HBM_PEAK_GBS * 1e9)), 1),
        "roofline": {
            "kernel": ("decode_partition_kernel<fp8_e4m3,128> (decode with append)" if fp8
                       else "decode_partition_kernel<bf16,128> (decode with append)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kern_b,
            "avg_launch_us": round(kern_avg_ms * 1e3, 2),
        },
    }
    if ceiling:
        res["hbm_read_ceiling"] = dict(ceiling, decode_frac_of_ceiling=round(achieved / ceiling["gbs"], 4))
    return res, case


def bench_mixed(args):
    """Mixed chunked-prefill + decode step (one layer): scatter, then prefill of
    16 chunks and decode of 48 requests, as two calls (``mixed``) or as one
    single-launch mixed call over the whole ragged batch (``mixed_single``).
    Roofline: the prefill (or mixed) kernel vs bf16 MFMA, counting the prefill
    flops only."""
    import paged_kv_cache_48_amd as pa
    from workloads import config_case

    P = args.block_size or 16
    case = config_case(4, block_size=P, values=False)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D, N = case.B, case.num_q_heads, case.num_kv_heads, case.head_dim, case.num_blocks
    T = case.T_total
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    fp8 = args.workload.endswith("_fp8")
    single = args.workload.startswith("mixed_single")
    if fp8:  # random finite E4M3 codes; per-KV-head scales
        kc = torch.randint(0, 256, (N, P, Hkv, D), generator=gen, device=dev, dtype=torch.uint8)
        vc = torch.randint(0, 256, (N, P, Hkv, D), generator=gen, device=dev, dtype=torch.uint8)
        for t in (kc, vc):
            t[(t & 0x7F) == 0x7F] -= 1
        ks = torch.full((Hkv,), 0.02, dtype=torch.float32, device=dev)
        vs = torch.full((Hkv,), 0.02, dtype=torch.float32, device=dev)
    else:
        kc = torch.randn((N, P, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
        vc = torch.randn((N, P, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
        ks = vs = None
    q = torch.randn((T, Hq, D), generator=gen, device=dev, dtype=torch.bfloat16)
    kn = torch.randn((T, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
    vn = torch.randn((T, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
    bt = torch.as_tensor(case.block_table, device=dev)
    lens = torch.as_tensor(case.context_lens, device=dev)
    cu = torch.as_tensor(case.cu_seqlens, device=dev)
    npf = 16
    cu_np = case.cu_seqlens
    qp, qd = q[: cu_np[npf]], q[cu_np[npf]:]
    outp, outd = torch.empty_like(qp), torch.empty_like(qd)
    cup, btp, lp = cu[: npf + 1].contiguous(), bt[:npf].contiguous(), lens[:npf].contiguous()
    btd, ld = bt[npf:].contiguous(), lens[npf:].contiguous()
    slots = torch.empty(T, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)

    def step(ev=None):
        pa.slot_mapping(bt, cu, lens, P, T, out=slots)
        pa.reshape_and_cache(kn, vn, slots, kc, vc, ks, vs)
        if single:
            with pa.kernel_timer(*ev) if ev is not None else contextlib.nullcontext():
                pa.paged_mixed_attention(q, kc, vc, cu, bt, lens, case.scale, out, ks, vs)
            return
        if ev is None:
            pa.paged_prefill_attention(qp, kc, vc, cup, btp, lp, case.scale, outp, ks, vs)
        else:
            with pa.kernel_timer(*ev):
                pa.paged_prefill_attention(qp, kc, vc, cup, btp, lp, case.scale, outp, ks, vs)
        pa.paged_decode_attention(qd, kc, vc, btd, ld, case.scale, outd, ks, vs)

    for _ in range(args.warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for k in range(args.steps):
        step(evs[k])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    Tb = case.query_lens[:npf].astype(np.int64)
    Lb = case.context_lens[:npf].astype(np.int64)
    flops = int(np.sum(4 * D * Hq * (Tb * (Lb - Tb) + Tb * (Tb + 1) // 2)))
    tflops = flops / (kern_ms * 1e-3) / 1e12
    Ld = case.context_lens[npf:].astype(np.int64)
    dec_bytes = decode_bytes(Ld, P, Hq, Hkv, D, 2, 1 if fp8 else 2)
    kname = ("mixed_kernel" if single else "prefill_kernel") + ("<128, fp8>" if fp8 else "<128>")
    res = {
        "metric": ("single-launch " if single else "") + "mixed chunked-prefill + decode step time "
                  "(prefill MFMA utilisation)" + (", fp8 e4m3 KV" if fp8 else ""),
        "value": round(ms_step, 4),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 KV, bf16 q/out" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} step: 16 prefill chunks (sum T = {int(Tb.sum())}) + 48 decodes, "
                               f"H_q={Hq}, H_kv={Hkv}, D={D}, P={P}"
                               + (", one mixed call" if single else ", prefill and decode calls"),
                   "global_batch": B, "block_size": P},
        "roofline": {
            "kernel": kname,
            "bound": "mfma",
            "achieved": round(tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(kern_ms * 1e3, 2),
        },
    }
    if single:
        # the mixed kernel also reads the decodes' KV: its lower bound is the
        # larger of the two roofline times (the resources could overlap fully)
        roof_us = max(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), dec_bytes / (HBM_PEAK_GBS * 1e9)) * 1e6
        res["roofline"].update({"decode_bytes_per_launch": int(dec_bytes), "roofline_time_us": round(roof_us, 1),
                                "time_frac": round(roof_us / (kern_ms * 1e3), 4)})
    return res, case


def bench_cow(args):
    """Copy-on-write block copies (pa_copy_blocks) in a Llama-3-8B layer pool:
    4096 (src, dst) pairs of 32 KiB blocks (P=16, H_kv=8, D=128, bf16) per pool,
    K and V.  Roofline: HBM, each byte read once and written once."""
    import paged_kv_cache_48_amd as pa

    dev = torch.device("cuda:0")
    N, P, Hkv, D, pairs_n = 30438, 16, 8, 128, 4096
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    kc = torch.randn((N, P, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
    vc = torch.randn((N, P, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
    perm = np.random.default_rng(6).permutation(N)
    pairs = torch.as_tensor(np.stack([perm[:pairs_n], perm[pairs_n:2 * pairs_n]], axis=1).astype(np.int32),
                            device=dev)
    for _ in range(args.warmup):
        pa.copy_blocks(kc, vc, pairs)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for k in range(args.steps):
        evs[k][0].record()
        pa.copy_blocks(kc, vc, pairs)
        evs[k][1].record()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    moved = 2 * 2 * pairs_n * P * Hkv * D * 2  # K and V, read and written
    achieved = moved / (kern_ms * 1e-3) / 1e9
    return {"metric": "copy-on-write block copies GB/s (read + write)", "value": round(moved / (ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"pa_copy_blocks: {pairs_n} random (src, dst) pairs of 32 KiB blocks per pool "
                                   f"(P={P}, H_kv={Hkv}, D={D}, bf16), K and V, pool of {N} blocks"},
            "roofline": {"kernel": "copy_blocks_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": None, "algorithmic_bytes_per_launch": moved,
                         "avg_launch_us": round(kern_ms * 1e3, 2)},
            "cpu_baseline": None}


def bench_copy(args):
    """A plain device copy of 1 GiB, the calibration run for HBM byte counters
    (FETCH_SIZE / WRITE_SIZE per dispatch divided by 1 GiB)."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    return {"metric": "device copy of 1 GiB (read + write)", "value": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "torch copy_ of 1 GiB", "bytes": n}, "cpu_baseline": None}


# ---------------------------------------------------------------------------
# Profile summaries.  Each GPU run below writes CSVs under DIR (run from the
# repository root); ``--summarize-profiles DIR`` turns them into profiles/.
B_CMD = "python3 bench.py --no-cpu-baseline --workload "
# kernel statistics: key -> (workload, steps, description)
TRACES = {
    "decode_llama3_8b": ("llama3_8b", 10, "Llama-3-8B-shaped decode step: 32 layers x paged decode with append "
                         "(partition kernel with in-kernel plan and the new token's write, then the merge), B=256, "
                         "H_q=32, H_kv=8, D=128, P=16, bf16; the same run times the step as separate calls (slot "
                         "mapping, reshape_and_cache, decode without append) and attention alone."),
    "decode_llama3_8b_fp8": ("llama3_8b_fp8", 10, "The same Llama-3-8B-shaped decode step over fp8 (OCP E4M3) pools "
                             "with per-KV-head scales; adjacent KV heads read in pairs."),
    "decode_gpt2_124m": ("gpt2_124m", 20, "GPT-2-124M-shaped decode step: 12 layers x paged decode with append, "
                         "B=64, H_q=H_kv=12, D=64 (KV heads read in pairs), P=16, N=4096, bf16; graph replays, eager "
                         "steps, then the guarded per-kernel loop."),
    "decode_llama32_1b": ("llama32_1b", 20, "Llama-3.2-1B-shaped decode step: 16 layers x paged decode with append, "
                          "B=128, H_q=32, H_kv=8, D=64 (KV heads read in pairs), P=16, bf16; graph replays, eager "
                          "steps, then the guarded per-kernel loop."),
    "decode_tiny": ("tiny", 20, "Tiny decode step: 1 layer, paged decode with append, B=4, H_q=H_kv=12, D=64, P=16, "
                    "N=64, fp32 (launch-latency bound)."),
    "decode_llama3_8b_g8": ("llama3_8b_g8", 5, "GQA group of 8: one layer of the Llama-3-8B batch (B=256, 90% pool, "
                            "H_kv=8, D=128, P=16, bf16) with 64 query heads, paged decode with append; graph replays, "
                            "eager steps, then the guarded per-kernel loop."),
    "prefill_mixed": ("mixed", 10, "Mixed chunked-prefill + decode step as two calls: 16 prefill chunks over cached "
                      "prefixes (paged_prefill_attention) and 48 decodes (paged_decode_attention), after the slot "
                      "mapping and the scatter of all new tokens; Llama-3-8B heads, P=16, bf16."),
    "mixed_single_launch": ("mixed_single", 10, "The same mixed step as one single-launch mixed call over the whole "
                            "ragged batch (64 requests: 16 prefill chunks + 48 one-token decodes), then the merge of "
                            "the decodes' partitions."),
    "copy_blocks_cow": ("cow", 20, "Copy-on-write block copies: pa_copy_blocks with 4096 (src, dst) pairs of 32 KiB "
                        "blocks per pool (P=16, H_kv=8, D=128, bf16), K and V: 512 MiB moved per launch."),
}
# HBM traffic (FETCH_SIZE, WRITE_SIZE per dispatch): key -> (workload, kernel name pattern)
TRAFFIC = {
    "decode_llama3_8b": ("llama3_8b", "decode_partition_kernel<unsigned short, 128, false, true, 1, 1, true>"),
    "decode_llama3_8b_fp8": ("llama3_8b_fp8", "fp8_e4m3, 256, false, true, 1, 2, true"),
    "decode_llama3_8b_g8": ("llama3_8b_g8", "decode_partition_kernel<unsigned short, 128, false, true, 1, 1, true>"),
}
# prefill counters, two passes (each within one pass's counter limits)
PREFILL_PMC = {
    "a": "MfmaUtil VALUBusy LdsBankConflict SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES SQ_WAVE_CYCLES",
    "b": "SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_ANY SQ_INSTS_LDS "
         "SQ_INSTS_VALU SQ_INSTS_MFMA",
}
PREFILL_SOURCES = ("prefill.hip", "prefill_dev.h", "common.h")
# sources the decode partition kernel is compiled from
DECODE_SOURCES = ("decode.hip", "decode_dev.h", "common.h")


def profile_commands():
    cmds = {}
    for key, (wl, steps, _) in TRACES.items():
        cmds[f"trace_{key}"] = (f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace_{key} -o {key} -- "
                                f"{B_CMD}{wl} --steps {steps} --warmup 2")
    for key, (wl, _) in TRAFFIC.items():
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            tag = c.split("_")[0].lower()
            cmds[f"{tag}_{key}"] = (f"rocprofv3 --pmc {c} --output-format csv -d DIR/{tag}_{key} -o {tag}_{key} -- "
                                    f"{B_CMD}{wl} --layers 2 --steps 2 --warmup 1")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        tag = c.split("_")[0].lower()
        cmds[f"{tag}_copy"] = (f"rocprofv3 --pmc {c} --output-format csv -d DIR/{tag}_copy -o {tag}_copy -- "
                               f"{B_CMD}copy --steps 3 --warmup 1")
    for p, ctr in PREFILL_PMC.items():
        cmds[f"pmc_prefill_{p}"] = (f"rocprofv3 --pmc {ctr} --output-format csv -d DIR/pmc_prefill_{p} -o "
                                    f"pmc_prefill_{p} -- {B_CMD}mixed --steps 2 --warmup 1")
    return cmds


def _short_kernel(name):
    name = name.replace("(anonymous namespace)::", "").replace("pa::", "")
    return name if len(name) < 110 else name[:107] + "..."


def _stats_table(path, top=8):
    import csv

    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"{'kernel':<110} {'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'% time':>7}"]
    for r in rows[:top]:
        out.append(f"{_short_kernel(r['Name']):<110} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                   f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>7.2f}")
    return out, rows


def _counter_means(path, kernel_substr):
    """Mean over dispatches of every counter for the kernels whose name contains
    kernel_substr: {counter: (mean, dispatches)}."""
    import collections
    import csv

    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if kernel_substr in r["Kernel_Name"].replace("pa::", ""):
            vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def _sha_line(files):
    return f"kernel sources ({', '.join(files)}) sha256: {sources_sha(files)}"


def summarize_profiles(d):
    import glob

    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    cmds = profile_commands()
    one = lambda pat: (glob.glob(os.path.join(d, pat)) or [None])[0]  # noqa: E731
    for key, (wl, _, desc) in TRACES.items():
        stats = one(f"trace_{key}/*kernel_stats.csv")
        if not stats:
            continue
        table, _ = _stats_table(stats)
        srcs = PREFILL_SOURCES if key == "prefill_mixed" else DECODE_SOURCES
        with open(os.path.join(prof, f"{key}_kernel_stats.txt"), "w") as f:
            f.write(desc + "\nrocprofv3 kernel statistics.\n")
            f.write("command (run from the repository root, DIR = an output folder):\n  " + cmds[f"trace_{key}"] + "\n")
            f.write(_sha_line(srcs) + "\n\n")
            f.write("\n".join(table) + "\n")
        log(f"profiles/{key}_kernel_stats.txt written")

    # prefill counters
    pa_csv, pb_csv = one("pmc_prefill_a/*counter_collection.csv"), one("pmc_prefill_b/*counter_collection.csv")
    if pa_csv and pb_csv:
        a = _counter_means(pa_csv, "prefill_kernel")
        b = _counter_means(pb_csv, "prefill_kernel")
        from workloads import config_case

        case = config_case(4, values=False)
        Tb = case.query_lens[:16].astype(np.int64)
        Lb = case.context_lens[:16].astype(np.int64)
        D, Hq = case.head_dim, case.num_q_heads
        alg = int(np.sum(4 * D * Hq * (Tb * (Lb - Tb) + Tb * (Tb + 1) // 2)))
        g = lambda m, k: m[k][0] if k in m else float("nan")  # noqa: E731
        mops = g(a, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
        wave = g(a, "SQ_WAVE_CYCLES")
        lines = [
            "Counters of prefill_kernel<128> on the mixed step's 16 prefill chunks (sum T = "
            f"{int(Tb.sum())}, Llama-3-8B heads, P=16, bf16), mean per dispatch.",
            "commands (run from the repository root, DIR = an output folder):",
            "  " + cmds["pmc_prefill_a"], "  " + cmds["pmc_prefill_b"],
            _sha_line(PREFILL_SOURCES), "",
            f"MfmaUtil        {g(a, 'MfmaUtil'):8.2f} %   MFMA busy cycles / (GPU active cycles x 1024 SIMDs)",
            f"VALUBusy        {g(a, 'VALUBusy'):8.2f} %   VALU instruction cycles / (GPU active cycles x 256 CUs)",
            f"LdsBankConflict {g(a, 'LdsBankConflict'):8.4f}     bank-conflict cycles per LDS access cycle",
            f"bf16 MFMA flops executed {mops:.4e} (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) against {alg:.4e} algorithmic "
            f"(causal half only): {mops / alg:.3f}x",
            "",
            "fractions of wave-resident cycles (SQ_WAVE_CYCLES):",
        ]
        for k in ("SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS"):
            lines.append(f"  {k:<22} {g(b, k) / wave:8.4f}")
        lines.append("instructions per dispatch:")
        for k in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS"):
            lines.append(f"  {k:<22} {g(b, k):.4e}")
        lines.append("raw means: " + ", ".join(f"{k}={v[0]:.6g}" for k, v in sorted({**a, **b}.items())))
        with open(os.path.join(prof, "prefill_mixed_counters.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        log("profiles/prefill_mixed_counters.txt written")

    # HBM traffic of the decode partition kernels
    cf, cw = one("fetch_copy/*counter_collection.csv"), one("write_copy/*counter_collection.csv")
    if not (cf and cw):
        log("copy calibration CSVs missing; traffic summaries not written")
        return
    cf_kib = _counter_means(cf, "copyBuffer").get("FETCH_SIZE", (None, 0))[0]
    cw_kib = _counter_means(cw, "copyBuffer").get("WRITE_SIZE", (None, 0))[0]
    gib = float(1 << 30)
    kf, kw = gib / (cf_kib * 1024), gib / (cw_kib * 1024)  # true bytes per counted byte
    from workloads import config_case

    case = config_case(3, values=False)
    path = os.path.join(prof, "traffic.json")
    rec_all = json.load(open(path)) if os.path.exists(path) else {}
    for key, (wl, pat) in TRAFFIC.items():
        fe, wr = one(f"fetch_{key}/*counter_collection.csv"), one(f"write_{key}/*counter_collection.csv")
        if not (fe and wr):
            continue
        fetch_kib, nf = _counter_means(fe, pat).get("FETCH_SIZE", (None, 0))
        write_kib, nw = _counter_means(wr, pat).get("WRITE_SIZE", (None, 0))
        if fetch_kib is None or write_kib is None:
            log(f"{key}: no dispatch of a kernel matching {pat!r}")
            continue
        s_kv = 1 if wl.endswith("fp8") else 2
        Hq = WIDE_GROUP[wl]["Hq"] if wl in WIDE_GROUP else case.num_q_heads
        alg = (decode_bytes(case.context_lens, case.block_size, Hq, case.num_kv_heads, case.head_dim,
                            2, s_kv) + append_bytes(case.B, case.num_kv_heads, case.head_dim, 2, s_kv))
        fetch_b, write_b = fetch_kib * 1024 * kf, write_kib * 1024 * kw
        lines = [
            f"HBM traffic of the decode partition kernel with append ({pat}) on the Llama-3-8B-shaped batch",
            f"({'fp8 e4m3' if s_kv == 1 else 'bf16'} pools; one launch = one layer, the new token's K/V written in "
            f"the same launch: B=256, sum of context lengths {int(case.context_lens.sum())}, H_q={Hq}, H_kv=8, "
            f"D=128, P=16).",
            "commands (run from the repository root, DIR = an output folder):",
            "  " + cmds[f"fetch_{key}"], "  " + cmds[f"write_{key}"], "  " + cmds["fetch_copy"],
            "  " + cmds["write_copy"], _sha_line(DECODE_SOURCES), "",
            f"calibration: torch copy_ of 1 GiB reads FETCH_SIZE {cf_kib:.0f} KiB and WRITE_SIZE {cw_kib:.0f} KiB "
            f"per dispatch -> scale {kf:.4f} (fetch), {kw:.4f} (write)",
            f"FETCH_SIZE {fetch_kib:.0f} KiB, WRITE_SIZE {write_kib:.0f} KiB per dispatch (mean of {nf} and {nw} "
            f"dispatches)",
            f"  -> fetched {fetch_b / 1e9:.4f} GB + written {write_b / 1e9:.4f} GB = {(fetch_b + write_b) / 1e9:.4f} "
            f"GB per launch",
            f"algorithmic bytes per launch: {alg / 1e9:.4f} GB (KV rows + q/out + block table + lengths + new rows); "
            f"measured / algorithmic = {(fetch_b + write_b) / alg:.3f}",
        ]
        with open(os.path.join(prof, f"{key}_hbm_traffic.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        rec_all[key] = {"source_sha256": sources_sha(DECODE_SOURCES), "bytes_per_launch": int(fetch_b + write_b),
                        "fetch_bytes": int(fetch_b), "write_bytes": int(write_b), "fetch_scale": kf,
                        "write_scale": kw}
        log(f"profiles/{key}_hbm_traffic.txt written")
    rec_all.pop("decode_partition_llama3_8b", None)
    with open(path, "w") as f:
        json.dump(rec_all, f, indent=1)


def decode_summary(res):
    """The ``workloads`` entry of a Llama-3-8B-shaped decode result."""
    keys = ("pct_hbm_peak", "us_per_layer_step_p10_p50_p90", "attention_only_us_per_layer_step_p10_p50_p90",
            "separate_calls_us_per_layer_step_p10_p50_p90", "decode_tokens_per_s", "roofline_tokens_per_s",
            "roofline", "cpu_baseline")
    out = {"config": res["config"]["workload"], "layers": res["config"]["layers"], "dtype": res["dtype"],
           "timing": f"eager calls, {res['steps']} steps", "kv_gbs": res["value"]}
    out.update({k: res[k] for k in keys if k in res})
    return out


def mixed_summary(res):
    out = {"config": res["config"]["workload"], "ms_per_step": res["value"], "roofline": res["roofline"],
           "cpu_baseline": res.get("cpu_baseline")}
    if res.get("cpu_baseline"):
        out["oracle_ms_per_step"] = res["cpu_baseline"]["value"]
    return out


def with_oracle_speedup(entry):
    cb = entry.get("cpu_baseline") or {}
    if "us_per_layer_step" in cb and "us_per_layer_step_p10_p50_p90" in entry:
        entry["oracle_us_per_layer_step"] = cb["us_per_layer_step"]
        entry["gpu_speedup_vs_oracle"] = round(cb["us_per_layer_step"] / entry["us_per_layer_step_p10_p50_p90"][1], 1)
    return entry


def free_gpu():
    import gc

    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def run_all(args):
    """The headline decode step, then every other seeded workload as extra keys."""
    sub = lambda **kw: argparse.Namespace(**dict(vars(args), **kw))  # noqa: E731
    res, case = bench_decode(sub(workload="llama3_8b"))
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_decode(case, args.cpu_seconds)
    free_gpu()
    wl = {"llama3_8b": with_oracle_speedup(decode_summary(res))}
    for name in SMALL_DECODE:
        entry = bench_decode_small(args, name)
        free_gpu()
        if not args.no_cpu_baseline:
            log(f"timing the oracle on {name}")
            entry["cpu_baseline"] = cpu_baseline_config(SMALL_DECODE[name])
        wl[name] = with_oracle_speedup(entry)
    for name in WIDE_GROUP:
        wl[name] = bench_decode_small(args, name)
        free_gpu()
    r8, c8 = bench_decode(sub(workload="llama3_8b_fp8"), ceiling_run=False)
    free_gpu()
    if not args.no_cpu_baseline:
        log("timing the oracle on the fp8 batch")
        r8["cpu_baseline"] = cpu_baseline_decode(c8, args.cpu_seconds / 2, fp8=True)
    wl["llama3_8b_fp8"] = with_oracle_speedup(decode_summary(r8))
    rm, _ = bench_mixed(sub(workload="mixed", block_size=16))
    free_gpu()
    wl["mixed"] = mixed_summary(rm)
    rs, cs = bench_mixed(sub(workload="mixed_single", block_size=16))
    free_gpu()
    if not args.no_cpu_baseline:
        log("timing the oracle on the mixed step")
        rs["cpu_baseline"] = cpu_baseline_mixed(cs, args.cpu_seconds / 2)
    wl["mixed_single"] = mixed_summary(rs)
    res["workloads"] = wl
    return res


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import paged_kv_cache_48_amd as pa

    pa.load_library()
    if args.workload == "all":
        res = run_all(args)
    elif args.workload == "copy":
        res = bench_copy(args)
    elif args.workload == "cow":
        res = bench_cow(args)
    elif args.workload in SMALL_DECODE or args.workload in WIDE_GROUP:
        res = bench_decode_small(args, args.workload)
        if not args.no_cpu_baseline and args.workload in SMALL_DECODE:
            res["cpu_baseline"] = cpu_baseline_config(SMALL_DECODE[args.workload])
    elif args.workload.startswith("mixed"):
        res, case = bench_mixed(args)
        if args.no_cpu_baseline or args.workload != "mixed_single":
            res["cpu_baseline"] = None
        else:
            log("timing the oracle on the host")
            res["cpu_baseline"] = cpu_baseline_mixed(case, args.cpu_seconds)
    else:
        res, case = bench_decode(args)
        if args.no_cpu_baseline:
            res["cpu_baseline"] = None
        else:
            log("timing the oracle on the host")
            res["cpu_baseline"] = cpu_baseline_decode(case, args.cpu_seconds, fp8=args.workload.endswith("_fp8"))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
