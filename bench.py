"""Decode-step benchmark: kv_append + paged decode attention on one MI355X.

One step is the whole hot path over one synthetic batch: every layer's kv_append (each sequence's
new K/V row into its page), then every layer's paged decode attention (plus the partition merge
when the context is split).  Inputs are generated on the host with the seeded generators and are
resident in HBM before timing starts.  The default workload is 256 sequences at context 2048
(32768 pages, 1 GiB of BF16 K+V).

Prints ONE JSON line.  ``value`` is algorithmic GB/s of the whole step (bytes / wall time per
step, with nothing but the step's launches in the timed region); ``roofline`` reports the fused
decode kernel against the 8 TB/s HBM peak using the HIP events that bracket the timed steps on
the stream the kernel runs on (one launch per layer); ``prefill`` adds the paged prefill
kernels on a second workload; ``cpu_baseline`` times the FP64 CPU oracle on the host cores.  The
pages report no throughput or hardware numbers for this kernel, so ``vs_baseline`` is null.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "paged decode attention GB/s and % of HBM peak; seq-tokens attended/sec"
ATTN_SOURCE = os.path.join(ROOT, "paged_kv_cache_pages_amd", "csrc", "paged_attention.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "paged_decode_{config}_traffic.md")
PREFILL_SOURCE = os.path.join(ROOT, "paged_kv_cache_pages_amd", "csrc", "prefill.hip")
PREFILL_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "paged_prefill_16x512_traffic.md")

WORKLOAD_TEXT = {
    "tiny": "1 sequence, context 37 (3 pages, last partial), 8-page pool",
    "long": "1 sequence, context 2048 (128 pages), 512-page pool, split context + merge",
    "mixed": "16 sequences, context uniform in [1,2048], 2048-page pool",
    "model16": "16 layers, 128 MiB pool (4096 pages), FIFO-admitted batch, geometric contexts (mean 256)",
    "bw256": "256 sequences x context 2048, 32768 pages (1 GiB BF16 K+V), random page order",
    "bw256tp8": "one GPU's share of bw256 under 8-way KV-head tensor parallelism: 256 sequences x context 2048, "
                "1 KV head (4 query heads), 32768 pages (128 MiB BF16 K+V), random page order",
}


# ---------------------------------------------------------------------------------------------
# byte accounting (algorithmic bytes: what the step must move at least once)
# ---------------------------------------------------------------------------------------------

def attention_bytes(w) -> int:
    """Q + every referenced K/V page (whole pages) + referenced table entries + BF16 output."""
    hq, d, hkv = w.num_q_heads, w.head_dim, w.num_kv_heads
    pages = int(np.sum((w.context_lens.astype(np.int64) + 15) // 16))
    page_bytes = 2 * hkv * 16 * d * 2  # K and V of one page, all KV heads
    per_layer = w.batch * (hq * d * 2) * 2 + pages * page_bytes + pages * 4
    return per_layer * w.layers


def attention_bytes_token_exact(w) -> int:
    """As attention_bytes, with K/V counted per attended token (L x 2 KiB) instead of whole pages."""
    hq, d, hkv = w.num_q_heads, w.head_dim, w.num_kv_heads
    pages = int(np.sum((w.context_lens.astype(np.int64) + 15) // 16))
    per_layer = w.batch * (hq * d * 2) * 2 + int(w.context_lens.sum()) * (2 * hkv * d * 2) + pages * 4
    return per_layer * w.layers


def append_bytes(w) -> int:
    """k_new + v_new read, the same rows written, one position and one table entry per row."""
    row = w.num_kv_heads * w.head_dim * 2
    return w.layers * w.batch * (2 * row + 2 * row + 4 + 4)


def seq_tokens(w) -> int:
    return int(w.context_lens.sum()) * w.layers


# ---------------------------------------------------------------------------------------------
# HBM traffic measured with rocprofv3 counters (taken offline, recorded under profiles/)
# ---------------------------------------------------------------------------------------------

def kernel_source_digest(path: str = ATTN_SOURCE) -> str:
    """Hash of a kernel source's code with comments and whitespace removed, so the recorded
    counters stay valid across comment-only edits and lapse on any code change."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def recorded_traffic(tag: str, profile: str, source: str = ATTN_SOURCE):
    """Traffic per launch of the ``tag`` kernel from a committed counter summary, or None when the
    summary is missing or the kernel source has changed since the counters were taken."""
    if not os.path.exists(profile):
        return None
    text = open(profile).read()
    m_src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch\[" + tag + r"\]:\s*([0-9.eE+]+)", text)
    if not (m_src and m_val) or m_src.group(1) != kernel_source_digest(source):
        return None
    return float(m_val.group(1))


# ---------------------------------------------------------------------------------------------
# CPU baseline: the FP64 oracle as it stands, on the host
# ---------------------------------------------------------------------------------------------

def cpu_baseline(w, min_seconds: float, max_seconds: float):
    """Time the oracle's append + attention on the same workload, on one host core.

    Whole passes over the batch (append of every layer, then attention of every sequence and
    layer) are repeated until ``min_seconds`` have elapsed; a pass is cut short at sequence
    granularity when ``max_seconds`` is reached, so the sample stays bounded for large
    workloads.  The rate is in the same GB/s units as ``value``: algorithmic bytes of the
    sequences processed divided by the elapsed time.  BLAS is pinned to one thread.
    """
    import oracle
    from threadpoolctl import threadpool_limits

    bytes_per_seq = (attention_bytes(w) + append_bytes(w)) / w.batch
    seqs = 0
    tokens = 0
    passes = 0
    chunk = 8
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            for layer in range(w.layers):
                k, v = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[layer], w.positions, w.k_new[layer],
                                        w.v_new[layer])
            b = 0
            while b < w.batch and (time.perf_counter() - t0) < max_seconds:
                rows = list(range(b, min(w.batch, b + chunk)))
                for layer in range(w.layers):
                    oracle.paged_decode_attention(w.q[layer], k, v, w.block_tables[layer], w.context_lens, 0.125,
                                                  sequences=rows)
                seqs += len(rows)
                tokens += int(w.context_lens[rows].sum()) * w.layers
                b += len(rows)
            passes += 1 if b >= w.batch else 0
            elapsed = time.perf_counter() - t0
            if b < w.batch or elapsed >= min_seconds:
                break
        secs = time.perf_counter() - t0
    return {
        "value": round(bytes_per_seq * seqs / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{seqs} sequence-passes ({passes} full pass(es) over the {w.batch} sequences x {w.layers} layer(s) "
                  f"of the same workload; FP64 numpy append of the whole pool + attention) in {secs:.2f} s",
        "seconds": round(secs, 3),
        "seq_tokens_per_s": round(tokens / secs, 1),
    }


_POOL_STATE = {}


def _oracle_rows(rows):
    """Worker: the oracle's attention for some sequences of every layer (state inherited by fork)."""
    import oracle

    w, pools = _POOL_STATE["w"], _POOL_STATE["pools"]
    for layer in range(w.layers):
        k, v = pools[layer]
        oracle.paged_decode_attention(w.q[layer], k, v, w.block_tables[layer], w.context_lens, 0.125, sequences=rows)
    return len(rows), int(w.context_lens[rows].sum()) * w.layers


def cpu_baseline_all_cores(w, min_seconds: float, max_seconds: float, max_workers: int = 16):
    """The oracle as it stands on every host core of this process (at most ``max_workers``): the
    append of every layer runs once in the parent (it copies the pool), then sequences are spread
    over a fork pool with BLAS pinned to one thread per worker, in rounds until ``min_seconds``
    (cap ``max_seconds``).  Must run before the GPU is initialised (workers are forked)."""
    import multiprocessing as mp

    import oracle
    from threadpoolctl import threadpool_limits

    cores = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    bytes_per_seq = (attention_bytes(w) + append_bytes(w)) / w.batch
    chunk = 4
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        pools = [oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[layer], w.positions, w.k_new[layer],
                                  w.v_new[layer]) for layer in range(w.layers)]
        t_append = time.perf_counter() - t0
        _POOL_STATE.update(w=w, pools=pools)
        seqs = tokens = 0
        rounds = 0
        with mp.get_context("fork").Pool(cores) as pool:
            t1 = time.perf_counter()
            order = [list(range(b, min(w.batch, b + chunk))) for b in range(0, w.batch, chunk)]
            i = 0
            while True:
                batch = [order[(i + k) % len(order)] for k in range(cores * 2)]
                i += len(batch)
                for n_seq, n_tok in pool.map(_oracle_rows, batch, chunksize=1):
                    seqs += n_seq
                    tokens += n_tok
                rounds += 1
                elapsed = time.perf_counter() - t1
                if elapsed >= min_seconds or elapsed >= max_seconds:
                    break
            t_attn = time.perf_counter() - t1
        _POOL_STATE.clear()
    secs = t_attn + t_append * seqs / w.batch  # the append is charged per pass over the batch
    return {
        "value": round(bytes_per_seq * seqs / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{seqs} sequence-passes of the same workload ({rounds} rounds of {cores * 2} tasks of {chunk} "
                  f"sequences x {w.layers} layer(s)) on {cores} worker processes in {t_attn:.2f} s, plus the FP64 "
                  f"numpy append of the whole pool once per layer ({t_append:.2f} s, charged per pass)",
        "seconds": round(secs, 3),
        "seq_tokens_per_s": round(tokens / secs, 1),
    }


# ---------------------------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------------------------

def run(args):
    import torch

    import paged_kv_cache_pages_amd as pkv
    from workloads import make_config

    t_gen = time.perf_counter()
    w = make_config(args.config)
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] workload {args.config}: B={w.batch} layers={w.layers} pages={w.num_pages} "
          f"(generated in {gen_s:.1f} s)", file=sys.stderr, flush=True)
    cpu = cpu_1 = None
    if not args.no_cpu_baseline:  # before the GPU is touched: the all-cores leg forks workers
        cpu = cpu_baseline_all_cores(w, args.cpu_min_seconds, args.cpu_max_seconds)
        print(f"[bench] CPU oracle on {cpu['cores']} cores: {cpu['value']} GB/s", file=sys.stderr, flush=True)
        cpu_1 = cpu_baseline(w, min(5.0, args.cpu_min_seconds), min(10.0, args.cpu_max_seconds))
        print(f"[bench] CPU oracle on 1 core: {cpu_1['value']} GB/s", file=sys.stderr, flush=True)

    pkv.require_library()
    torch.cuda.set_device(0)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    def dev_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    kp, vp = dev_bf16(w.k_pool), dev_bf16(w.v_pool)
    pos, lens = dev_i32(w.positions), dev_i32(w.context_lens)
    layers = []
    for layer in range(w.layers):
        layers.append({
            "bt": dev_i32(w.block_tables[layer]),
            "q": dev_bf16(w.q[layer]),
            "k_new": dev_bf16(w.k_new[layer]),
            "v_new": dev_bf16(w.v_new[layer]),
            "out": torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda"),
        })
    # The scheduler knows every context length on the host, so the plan gets the longest one.
    pp = args.partition_pages if args.partition_pages > 0 else pkv.plan_partition_pages(
        w.batch, w.num_kv_heads, w.max_blocks, max_context=int(np.max(w.context_lens)) if w.batch else None)
    ws_bytes = pkv.decode_workspace_bytes(w.batch, w.num_q_heads, w.max_blocks, pp)
    workspace = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def append_all():
        for t in layers:
            pkv.kv_append(kp, vp, t["bt"], pos, t["k_new"], t["v_new"])

    def attend_all():
        for t in layers:
            pkv.paged_decode_attention(t["q"], kp, vp, t["bt"], lens, t["out"], partition_pages=pp,
                                       workspace=workspace)

    # The fused step goes through PreparedDecodeStep: the same pkv_decode_step launch with its
    # arguments checked once, so an eager loop is not bound by Python argument handling.
    prepared = [pkv.PreparedDecodeStep(t["q"], kp, vp, t["bt"], pos, t["k_new"], t["v_new"], t["out"],
                                       partition_pages=pp, workspace=workspace) for t in layers]

    def fused_all():
        for step in prepared:
            step()

    K = args.steps
    samples = []
    regions = []

    def timed(phases):
        """Run K steps made of ``phases`` (callables, run in order) by wall clock with nothing else
        in the timed region, then K more with HIP events on the launch stream around every phase.
        Returns (wall seconds for the first K steps, per-phase mean ms from the second K)."""
        for _ in range(args.warmup):
            for f in phases:
                f()
        torch.cuda.synchronize()
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        r0.record()
        for _ in range(K):
            for f in phases:
                f()
        r1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        regions.append(r0.elapsed_time(r1) / K)  # GPU ms per step over the timed region
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            for j, f in enumerate(phases):
                ev[i][j].record()
                f()
            ev[i][len(phases)].record()
        torch.cuda.synchronize()
        per = [[e[j].elapsed_time(e[j + 1]) for e in ev] for j in range(len(phases))]
        samples.append(per)
        return wall, [float(np.mean(x)) for x in per]

    def capture(*phases):
        """The phases captured once as a HIP graph (after one eager run on a side stream)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for f in phases:
                f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for f in phases:
                f()
        return graph

    def graph_wall(phases):
        """The whole step captured once as a HIP graph and replayed K times: same kernels and
        bytes, no per-launch host work."""
        graph = capture(*phases)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # Both forms of the step do the same work: every layer's append, then its attention over the
    # context including the appended token.  "two-call" uses pkv_kv_append + pkv_paged_decode_
    # attention; "fused" uses pkv_decode_step, one launch per layer that also writes the new rows.
    two_wall, (append_ms, attn_ms) = timed([append_all, attend_all])
    fused_wall, (fused_ms,) = timed([fused_all])
    attn_samples, fused_samples = samples[0][1], samples[1][0]

    def stats_us(ms_list, per):
        a = np.asarray(ms_list) * 1e3 / per
        return {"median": round(float(np.median(a)), 3), "min": round(float(a.min()), 3),
                "p90": round(float(np.percentile(a, 90)), 3)}

    # Cold timing: before each of `reps` single steps, read a 512 MiB scratch tensor.  Reading
    # (not writing) evicts the XCD L2s and the 256 MiB Infinity Cache without leaving dirty lines
    # whose write-back would compete with the step.
    evict = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    evict.sum()
    torch.cuda.synchronize()

    def cold_us(fn, reps=10):
        # The step is captured once as a HIP graph and each replay is enqueued behind the eviction
        # read (~90 us of GPU work) with no host sync in between, so the GPU reaches the first
        # event with the whole step already queued: the interval is the kernels on cold caches,
        # not the host's launch latency (a 16-layer step takes the host longer to launch eagerly
        # than the eviction read lasts).
        graph = capture(fn)
        times = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            evict.sum()
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        return round(float(np.median(times)), 3)

    cold_fused_us = cold_us(fused_all) if not args.no_cold else None
    cold_attn_us = cold_us(attend_all) if not args.no_cold else None
    del evict
    if args.graph:
        two_wall = graph_wall([append_all, attend_all])
        fused_wall = graph_wall([fused_all])

    # plain device-to-device copy of 1 GiB (2 GiB moved) as an achievable-bandwidth reference
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * src.numel() * 2 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    a_bytes, p_bytes = attention_bytes(w), append_bytes(w)
    step_bytes = a_bytes + p_bytes
    gbps = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    two_ms = two_wall * 1e3 / K
    fused_msps = fused_wall * 1e3 / K
    fused_mode = args.step == "fused"
    ms_per_step = fused_msps if fused_mode else two_ms
    value = gbps(step_bytes, ms_per_step)
    # One "launch" = one layer.  Dominant kernel: the fused decode kernel (attention + append
    # bytes) or, for the two-call step, the attention kernel (attention bytes).
    # The library's kernel choice: the matrix-core flavour for every split launch and for batches
    # with fewer (sequence, KV head) pairs than compute units, else the vector-ALU flavour.
    split = pp < min(w.max_blocks, 256)
    mfma = split or w.batch * w.num_kv_heads < pkv.cu_count()
    kernel = "paged_decode_mfma_kernel" if mfma else "paged_decode_kernel"
    if fused_mode:
        # the fused step is one launch per layer: the events bracketing the timed region give the
        # launches' average duration with nothing else between them
        launch_ms = regions[1] / w.layers
        launch_bytes = step_bytes // w.layers
        kernel += " (fused append)"
    else:
        launch_ms = attn_ms / w.layers
        launch_bytes = a_bytes // w.layers
    if split:
        kernel += ", split context merged in the launch"

    def graph_launch_ms(phase, reps):
        """Mean ms per step of `reps` steps of `phase` captured in one HIP graph and replayed between
        two events on the launch stream: the GPU never waits for the host, so this is the kernels'
        own duration plus the gaps between graph nodes."""
        graph = capture(*([phase] * reps))
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) / reps

    # The roofline uses the events bracketing the timed region (fused step) or the per-launch
    # events (attention of the two-call step).  Back-to-back launches replayed from one graph are
    # reported beside it: they remove host launch gaps (which matter for short kernels) but add
    # the graph's node-to-node gap.
    reps = max(10, min(K, 100))
    launch_ms_graph = graph_launch_ms(fused_all if fused_mode else attend_all, reps) / w.layers
    achieved = gbps(launch_bytes, launch_ms)
    # counters are recorded for the partition plan the bench uses by default
    traffic = recorded_traffic("fused" if fused_mode else "attention", TRAFFIC_PROFILE.format(config=args.config)) \
        if args.partition_pages <= 0 else None

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "compute": "bf16 inputs, f32 accumulate and softmax",
        "step": "fused: pkv_decode_step (PreparedDecodeStep), one launch per layer" if fused_mode
                else "two-call: pkv_kv_append + pkv_paged_decode_attention per layer",
        "launch": "hip graph replay of the whole step" if args.graph else "eager launches through the C ABI",
        "data": "synthetic (seeded N(0,1) BF16; no dataset)",
        "config": {
            "workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}",
            "batch": w.batch,
            "layers": w.layers,
            "context_tokens": seq_tokens(w),
            "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": 16,
            "pool_pages": w.num_pages,
            "partition_pages": pp,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "seq_tokens_per_s": round(seq_tokens(w) / (ms_per_step * 1e-3), 1),
        "bytes_per_step": step_bytes,
        "fused": {"ms_per_step": round(fused_msps, 5), "us_per_launch": round(fused_ms / w.layers * 1e3, 3),
                  "us_per_launch_stats": stats_us(fused_samples, w.layers),
                  "value": round(gbps(step_bytes, fused_msps), 2)},
        "two_call": {"ms_per_step": round(two_ms, 5), "attention_us_per_launch": round(attn_ms / w.layers * 1e3, 3),
                     "append_us_per_step": round(append_ms * 1e3, 3), "value": round(gbps(step_bytes, two_ms), 2),
                     "attention_gbps": round(gbps(a_bytes / w.layers, attn_ms / w.layers), 2),
                     "attention_us_per_launch_stats": stats_us(attn_samples, w.layers)},
        "cold": {"fused_us_per_step": cold_fused_us, "attention_us_per_step": cold_attn_us,
                 "fused_gbps": round(gbps(step_bytes, cold_fused_us / 1e3), 2) if cold_fused_us else None,
                 "protocol": "median of 10 single steps, each a graph replay enqueued behind a read of a 512 MiB scratch tensor "
                             "(L2 and Infinity Cache evicted, no dirty lines)"},
        "algorithmic_bytes_token_exact": attention_bytes_token_exact(w) + p_bytes,
        "copy_d2d_gbps": round(copy_gbps, 1),
        "pct_of_copy": round(100.0 * achieved / copy_gbps, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "algorithmic_bytes_per_launch": launch_bytes,
            "us_per_launch": round(launch_ms * 1e3, 3),
            "timing": ("HIP events bracketing the K timed steps on the launch stream, per layer launch"
                       if fused_mode else "mean of HIP events around each launch, on the launch stream"),
            "us_per_launch_events": round((fused_ms if fused_mode else attn_ms) / w.layers * 1e3, 3),
            "us_per_launch_graph": round(launch_ms_graph * 1e3, 3),
        },
        "note": "The reference pages report no throughput or hardware numbers for this kernel; "
                "figures are this build's measurements on one MI355X.",
    }

    if not args.no_prefill:
        result["prefill"] = prefill_leg(args, torch, pkv)
    if cpu is not None:
        result["cpu_baseline"] = cpu
        result["cpu_baseline_1core"] = cpu_1
    print(json.dumps(result), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_leg(args, torch, pkv):
    """The second workload: paged prefill (prompt K/V append, then causal attention over the
    pages) on ``--prefill-config``.  Reported beside the decode step, never as ``value``.
    Algorithmic flops: every visible (query, key) pair costs 2*64 for q.k and 2*64 for p*v, per
    query head."""
    from workloads import make_prefill_config

    w = make_prefill_config(args.prefill_config)
    dev_bf16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    dev_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    kp, vp = dev_bf16(w.k_pool), dev_bf16(w.v_pool)
    bt, cu, sp = dev_i32(w.block_tables), dev_i32(w.cu_seqlens), dev_i32(w.start_pos)
    q, kn, vn = dev_bf16(w.q), dev_bf16(w.k_new), dev_bf16(w.v_new)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    mpl = int(w.prompt_lens.max())
    append = lambda: pkv.prefill_kv_append(kp, vp, bt, cu, sp, kn, vn, max_prompt_len=mpl)
    attend = lambda: pkv.paged_prefill_attention(q, kp, vp, bt, cu, sp, out, max_prompt_len=mpl)
    for _ in range(args.warmup):
        append()
        attend()
    torch.cuda.synchronize()
    K = args.steps

    def back_to_back(fn):
        """Mean ms per launch of K launches captured in one HIP graph and replayed between two
        events: the GPU never waits for the host, so this is the kernel's own duration plus the
        gap between graph nodes (the append alone is shorter than a Python-side launch)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(K):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    t0 = time.perf_counter()
    for _ in range(K):
        append()
        attend()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / K
    app_ms = back_to_back(append)  # the append rewrites the same rows: repeatable
    att_ms = back_to_back(attend)
    pairs = int(w.meta["causal_pairs"])
    flops = pairs * w.q.shape[1] * 4 * w.q.shape[2]
    tflops = flops / (att_ms * 1e-3) / 1e12
    return {
        "workload": f"{args.prefill_config}: {w.batch} prompts, {w.tokens} query rows, start {int(w.start_pos.max())}",
        "ms_per_step": round(wall_ms, 5),
        "append_us": round(app_ms * 1e3, 3),
        "attention_us": round(att_ms * 1e3, 3),
        "tokens_per_s": round(w.tokens / (wall_ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill_attention", PREFILL_TRAFFIC_PROFILE, PREFILL_SOURCE)
                     if args.prefill_config == "prefill16x512" else None,
                     # the launch picks 32-key steps (prefill_attention_kernel_k32) from four
                     # workgroups per compute unit, as at 16 x 512, else prefill_attention_kernel
                     "kernel": "prefill attention (prefill_attention_kernel[_k32])",
                     "algorithmic_flops_per_launch": flops},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="bw256", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--partition-pages", type=int, default=0, help="<= 0: library plan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="time the step as one captured HIP graph")
    ap.add_argument("--step", choices=["fused", "two-call"], default="fused",
                    help="which form of the step gives value/roofline (both are timed and reported)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the paged prefill measurement")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing (profiler runs: keeps the per-kernel averages warm)")
    ap.add_argument("--prefill-config", default="prefill16x512",
                    choices=["prefill_tiny", "prefill512", "prefill_chunked", "prefill16x512"])
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0, help="repeat CPU oracle passes at least this long")
    ap.add_argument("--cpu-max-seconds", type=float, default=30.0, help="hard bound on the CPU oracle timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (this path has no "
              "multi-GPU mode).", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
