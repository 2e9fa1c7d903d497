#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the whole path over one batch: the slot write of the step's new
K/V and varlen paged attention over the updated pools, issued as one
paged_attention_varlen_with_write call (the same result as paged_kv_write followed by
paged_attention_varlen; that two-call step is timed too and reported beside it).

Default workload (the one the headline metric is quoted on): Llama-3.2-1B-shaped
single-layer decode in bf16, 32 sequences, 32 query / 8 KV heads, head_dim 64,
16-token blocks, contexts uniform in [128, 2048], a pool of 8,192 blocks.

Timing
  * Inputs are resident in HBM before timing starts.  R device copies of the batch
    (separate pools, tables, queries) are used round-robin, with R chosen so that R
    working sets exceed 1 GiB, four times the 256 MB MALL: each step's K/V comes from
    HBM, not from the last-level cache.
  * W eager warm-up steps run first.  Then exactly K steps are captured into one HIP
    graph; after one untimed warm replay, the timed replay is bracketed by
    torch.cuda.synchronize() on both sides (one process, one GPU: no barrier needed).
  * `roofline.achieved` uses the decode launch's average duration from HIP events
    recorded on the replay stream around the timed graph (one launch per step at this
    shape: the decode kernel, which also performs the slot write), i.e. back-to-back
    launches including their dispatch gaps.  The eager call (HIP events around each
    call, queued behind a spin kernel) is reported beside it.
  * value = algorithmic bytes of one step / ms_per_step (GB/s).  Algorithmic bytes
    count every logical KV token of a sequence once (shared-prefix blocks once per
    physical block), plus q, out, table entries, lengths, and the write's new K/V
    read and stored, and its slot indices.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                       [--only-main] [--only-chunk] [--only-scaling] [--only-long]
                       [--only-achievable] [--only-mixed] [--only-chunk-sweep]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "paged-attn decode KV GB/s (% of HBM peak); prefill-chunk TFLOP/s (% MFMA)"
MAIN = "llama32_1b_decode"
ROTATE_BYTES = 1 << 30


# ---------------------------------------------------------------------------
# algorithmic work of one step (counts only; no attention arithmetic)
# ---------------------------------------------------------------------------

def kv_token_slots(b) -> int:
    """Distinct pool slots the attention reads (shared blocks count once)."""
    import numpy as np

    seen = {}
    for s in range(b.num_seqs):
        c = int(b.context_lens[s])
        nb = (c + 15) // 16
        for lb in range(nb):
            pb = int(b.block_tables[s, lb])
            used = min(16, c - lb * 16)
            seen[pb] = max(seen.get(pb, 0), used)
    del np
    return sum(seen.values())


def attention_bytes(b, unique=True) -> int:
    e = b.elem_bytes
    toks = kv_token_slots(b) if unique else int(b.context_lens.sum())
    kv = toks * b.num_kv_heads * b.head_dim * e * 2
    qo = 2 * b.total_q * b.num_q_heads * b.head_dim * e
    meta = int(((b.context_lens.astype("int64") + 15) // 16).sum()) * 4
    meta += 4 * b.num_seqs + 4 * (b.num_seqs + 1)
    return kv + qo + meta


def write_bytes(b) -> int:
    return 2 * 2 * b.total_q * b.num_kv_heads * b.head_dim * b.elem_bytes + 4 * b.total_q


def chunk_flops(b) -> int:
    """4 * D * Hq per attended (query, key) pair of the rows with q_len > 1."""
    pairs = 0
    for s in range(b.num_seqs):
        q = int(b.query_lens[s])
        if q > 1:
            c = int(b.context_lens[s])
            pairs += sum(c - q + i + 1 for i in range(q))
    return 4 * b.head_dim * b.num_q_heads * pairs


# ---------------------------------------------------------------------------
# device side
# ---------------------------------------------------------------------------

_FIELDS = ("k_pool", "v_pool", "q", "k_new", "v_new", "block_tables", "context_lens",
           "query_start_loc", "slot_mapping")


def device_copy(b):
    """The batch's arrays as device tensors (bf16 bit patterns viewed as bfloat16)."""
    import types

    import numpy as np
    import torch

    d = types.SimpleNamespace(b=b)
    for f in _FIELDS:
        a = np.ascontiguousarray(getattr(b, f))
        if f in ("block_tables", "context_lens", "query_start_loc", "slot_mapping"):
            t = torch.from_numpy(a.astype(np.int32))
        elif b.dtype == "bf16":
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a.astype(np.float32))
        setattr(d, f, t.to("cuda"))
    return d


class Runner:
    """R device copies of one batch and the step on copy i % R."""

    def __init__(self, b, rotate: int):
        import torch
        import paged_kv_cache_290_amd as pkv

        self.b, self.pkv, self.torch = b, pkv, torch
        base = device_copy(b)
        self.sets = [base]
        for _ in range(rotate - 1):
            c = type(base)(b=b)
            for f in _FIELDS:
                setattr(c, f, getattr(base, f).clone())
            self.sets.append(c)
        for s in self.sets:
            s.out = torch.empty_like(s.q)
        nbytes = pkv.workspace_size(b.num_seqs, b.total_q, b.num_q_heads, b.num_kv_heads,
                                    b.head_dim, b.max_context_len, base.q.dtype)
        self.shared = int(b.meta.get("shared_prefix_blocks", 0))
        if self.shared:
            nbytes = max(nbytes, pkv.shared_prefix_workspace_size(
                b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, b.max_context_len,
                self.shared, base.q.dtype))
        self.ws = [torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
                   for _ in self.sets]

    def write(self, i):
        s = self.sets[i % len(self.sets)]
        self.pkv.kv_write(s.k_new, s.v_new, s.k_pool, s.v_pool, s.slot_mapping)

    def attend(self, i):
        s = self.sets[i % len(self.sets)]
        b = self.b
        self.pkv.attention(s.q, s.k_pool, s.v_pool, s.block_tables, s.context_lens,
                           s.query_start_loc, scale=b.scale,
                           max_context_len=b.max_context_len,
                           max_query_len=b.max_query_len, out=s.out,
                           workspace=self.ws[i % len(self.sets)])

    def fused(self, i):
        s = self.sets[i % len(self.sets)]
        b = self.b
        self.pkv.attention_with_write(s.q, s.k_new, s.v_new, s.k_pool, s.v_pool,
                                      s.slot_mapping, s.block_tables, s.context_lens,
                                      s.query_start_loc, scale=b.scale,
                                      max_context_len=b.max_context_len,
                                      max_query_len=b.max_query_len, out=s.out,
                                      workspace=self.ws[i % len(self.sets)])

    def cascade(self, i):
        """The fused step through the shared-prefix entry point (the shared blocks read
        once for all rows)."""
        s = self.sets[i % len(self.sets)]
        b = self.b
        self.pkv.attention_shared_prefix(s.q, s.k_pool, s.v_pool, s.block_tables,
                                         s.context_lens, s.query_start_loc,
                                         shared_blocks=self.shared, scale=b.scale,
                                         max_context_len=b.max_context_len, k_new=s.k_new,
                                         v_new=s.v_new, slot_mapping=s.slot_mapping,
                                         out=s.out, workspace=self.ws[i % len(self.sets)])

    def step(self, i):
        self.fused(i)

    def step_two_calls(self, i):
        self.write(i)
        self.attend(i)


def time_graph(r: Runner, steps: int, warmup: int, fn=None, events: dict | None = None) -> float:
    """ms per step from one HIP graph of exactly `steps` calls of fn (default r.step).
    If `events` is given, it receives `event_ms`: the timed replay's duration from HIP
    events recorded on the replay stream around it, divided by `steps`."""
    torch = r.torch
    fn = fn or r.step
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()                         # untimed warm replay
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    if events is not None:
        events["event_ms"] = ev0.elapsed_time(ev1) / steps
    return ms


def time_calls(r: Runner, calls: int, fn=None, dist: dict | None = None) -> float:
    """Average duration (ms) of one call of fn (default r.step), from HIP events
    recorded on the stream the kernels are launched on.  If `dist` is given, it
    receives the 10th, 50th and 90th percentiles of the per-call durations."""
    torch = r.torch
    fn = fn or r.step
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for i in range(2):
        fn(i)
    torch.cuda.synchronize()
    # queue everything behind a spin kernel so the calls run back to back on the GPU
    torch.cuda._sleep(int(2e8))
    for i in range(calls):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    if dist is not None:
        for q in (10, 50, 90):
            dist[f"p{q}_ms"] = round(ts[min(len(ts) - 1, (len(ts) * q) // 100)], 5)
    return sum(ts) / calls


class DeviceRunner(Runner):
    """A Runner over batches built directly on the device (one `sets` entry per copy)."""

    def __init__(self, b, sets):
        import torch
        import paged_kv_cache_290_amd as pkv

        self.b, self.pkv, self.torch, self.sets = b, pkv, torch, sets
        for s in sets:
            s.out = torch.empty_like(s.q)
        nbytes = pkv.workspace_size(b.num_seqs, b.total_q, b.num_q_heads, b.num_kv_heads,
                                    b.head_dim, b.max_context_len, sets[0].q.dtype)
        self.ws = [torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
                   for _ in sets]


def _device_decode_case(ctx, steps: int, warmup: int, seed: int) -> dict:
    """One fused decode step over Llama-3.2-1B heads (32q/8kv, d=64, bf16) with the
    context lengths `ctx` (a CPU int tensor), drawn on the device with a torch
    generator seeded by `seed` (no oracle is involved: these are the kernels the
    parity tests cover).  Same protocol as the headline: fused steps in one HIP graph
    over rotating copies (>= 1 GiB in total)."""
    import types

    import torch

    hq, hkv, d = 32, 8, 64
    batch = int(ctx.numel())
    g = torch.Generator().manual_seed(seed)
    nblk = (ctx + 15) // 16
    mb = int(nblk.max())
    nb = max(8192, batch * mb)
    tbl = torch.randperm(nb, generator=g)[: batch * mb].view(batch, mb).to(torch.int32)
    tbl[torch.arange(mb).view(1, -1) >= nblk.view(-1, 1)] = -1
    last = ctx - 1
    slot = tbl[torch.arange(batch), last // 16].long() * 16 + last % 16
    b = types.SimpleNamespace(
        num_seqs=batch, total_q=batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        max_context_len=int(ctx.max()), max_query_len=1, scale=d ** -0.5)
    kv = int(ctx.sum()) * hkv * d * 2 * 2
    per = (kv + 2 * batch * hq * d * 2 + int(nblk.sum()) * 4 + 8 * batch + 4 +
           2 * 2 * batch * hkv * d * 2 + 4 * batch)
    rot = max(2, min(32, math.ceil(ROTATE_BYTES / per)))
    sets = []
    for _ in range(rot):
        s = types.SimpleNamespace()
        s.k_pool = torch.randn(nb, hkv, 16, d, device="cuda").to(torch.bfloat16)
        s.v_pool = torch.randn(nb, hkv, 16, d, device="cuda").to(torch.bfloat16)
        s.q = torch.randn(batch, hq, d, device="cuda").to(torch.bfloat16)
        s.k_new = torch.randn(batch, hkv, d, device="cuda").to(torch.bfloat16)
        s.v_new = torch.randn(batch, hkv, d, device="cuda").to(torch.bfloat16)
        s.block_tables = tbl.cuda()
        s.context_lens = ctx.to(torch.int32).cuda()
        s.query_start_loc = torch.arange(batch + 1, dtype=torch.int32, device="cuda")
        s.slot_mapping = slot.to(torch.int32).cuda()
        sets.append(s)
    r = DeviceRunner(b, sets)
    ms = time_graph(r, steps, warmup)
    ws = r.pkv.workspace_size(batch, batch, hq, hkv, d, int(ctx.max()), torch.bfloat16)
    gbs = per / (ms * 1e-3) / 1e9
    res = {"bytes_per_step": per, "rotating_copies": rot, "ms_per_step": round(ms, 5),
           "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "key_ranges": ws > 0}
    del r, sets
    torch.cuda.empty_cache()
    return res


def measure_batch_scaling(steps: int, warmup: int) -> dict:
    """Context for the headline: the same decode shape (Llama-3.2-1B heads, 32q/8kv,
    d=64, contexts U[128, 2048], bf16) at batches 32, 128 and 512.  A call has fixed
    costs — the launch, the table walk before the first K/V bytes arrive, the
    segments' unequal lengths — that weigh less as the bytes per step grow."""
    import torch

    res = {}
    for batch in (32, 128, 512):
        g = torch.Generator().manual_seed(batch)
        ctx = torch.randint(128, 2049, (batch,), generator=g)
        res[f"batch_{batch}"] = _device_decode_case(ctx, steps, warmup, batch)
    return res


def measure_long_context(steps: int, warmup: int) -> dict:
    """Context: decode over long contexts with the same heads (Llama-3.2-1B, bf16), where
    each (sequence, kv head) segment is cut into key ranges whose partial results the
    merge kernel combines: 4 sequences of 32,768 tokens and 1 of 131,072 (~268 MB of
    K/V per step each), beside 64 sequences of 2,048 (the same bytes, no key ranges)."""
    import torch

    res = {}
    for batch, c in ((4, 32768), (1, 131072), (64, 2048)):
        ctx = torch.full((batch,), c, dtype=torch.int64)
        res[f"{batch}x{c}"] = _device_decode_case(ctx, steps, warmup, 7 * batch + 1)
    return res


def _time_fn(fn, calls: int) -> float:
    """Average ms of fn() from HIP events on the current stream, the calls queued
    behind a spin kernel so that they run back to back."""
    import torch

    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / calls


def measure_achievable(calls: int) -> dict:
    """Measured ceilings to read the rooflines against (the published peaks stay the
    `peak` of the roofline objects):
      * HBM read rate of this library's read-only probe (pkv_read_probe): a contiguous
        1 GiB stream in 4 KiB tiles (the waves sweeping it side by side); scattered
        2 KiB tiles (the K or V tile of one (block, kv head) at d=64 bf16), a random
        permutation of a 1 GiB pool, 512 MiB per call; and the same scattered pattern
        at the headline decode step's K/V bytes, i.e. a pure-read floor for that step
        (one launch, no metadata walk).  Consecutive calls read disjoint tile sets, so
        the 256 MB MALL does not serve them.  The best of grids of 2, 4 and 8
        workgroups per CU is reported.
      * bf16 GEMM rate of torch.matmul (hipBLASLt) at 8192^3, a measuring stick only.
    """
    import torch

    import paged_kv_cache_290_amd as pkv
    from workloads import make_config

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator().manual_seed(0)
    pool = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    pool.random_(0, 255)
    sink = torch.empty(8 * cus * 4, dtype=torch.int32, device="cuda")
    res = {}

    def best(lists, tile_bytes, order=None):
        """Best rate over the grids; calls cycle through `lists` (disjoint tile sets,
        together larger than the MALL, so a call does not read what the previous
        calls left in it)."""
        nbytes = lists[0].numel() * tile_bytes
        out = {}
        for per_cu in (2, 4, 8):
            grid = per_cu * cus
            src = [order(t, grid * 4) if order else t for t in lists]
            k = [0]

            def call():
                pkv.read_probe(pool, src[k[0] % len(src)], tile_bytes, sink, grid)
                k[0] += 1

            ms = _time_fn(call, calls)
            out[per_cu] = nbytes / (ms * 1e-3) / 1e9
        k = max(out, key=out.get)
        return {"GBs": round(out[k], 1), "frac_of_peak": round(out[k] / HBM_PEAK_GBS, 4),
                "bytes": nbytes, "wgs_per_cu": k, "tile_sets": len(lists)}

    def sweep(t, waves):
        # wave w's contiguous share of the list holds tiles w, w + waves, ...: the
        # waves read neighbouring tiles at the same time (a sweeping front)
        n = t.numel() // waves * waves
        return t[:n].view(-1, waves).t().contiguous().view(-1)

    ntiles = (1 << 30) // 2048
    seq = torch.arange((1 << 30) // 4096, dtype=torch.int32, device="cuda")
    res["read_contiguous_1GiB"] = best([seq], 4096, order=sweep)
    perm = torch.randperm(ntiles, generator=g).to(torch.int32).cuda()
    half = ntiles // 2
    res["read_scattered_2KiB_512MiB"] = best([perm[:half], perm[half:]], 2048)
    b = make_config(MAIN, 0)
    kv_tiles = int(((b.context_lens.astype("int64") + 15) // 16).sum()) * b.num_kv_heads * 2
    nsets = ntiles // kv_tiles
    res["read_scattered_2KiB_headline_step"] = best(
        [perm[i * kv_tiles:(i + 1) * kv_tiles] for i in range(nsets)], 2048)
    res["read_scattered_2KiB_headline_step"]["note"] = (
        "as many 2 KiB tiles as the headline step's K and V tiles, one launch per call")
    del pool, seq, perm
    torch.cuda.empty_cache()

    n = 8192
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    ms = _time_fn(lambda: torch.matmul(x, y), max(5, calls // 4))
    tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
    res["bf16_gemm_8192"] = {"TFLOPs": round(tf, 1),
                             "frac_of_peak": round(tf / BF16_MFMA_PEAK_TFS, 4),
                             "via": "torch.matmul (hipBLASLt)"}
    del x, y
    torch.cuda.empty_cache()
    return res


def rotation_for(b) -> int:
    per = attention_bytes(b) + write_bytes(b)
    return max(2, min(32, math.ceil(ROTATE_BYTES / per)))


# ---------------------------------------------------------------------------
# oracle timing (CPU baseline leg)
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    """The host CPU's model name (lscpu's "Model name"; /proc/cpuinfo if lscpu is
    missing)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(b, budget_s: float = 10.0) -> dict:
    """The CPU oracle (as is) on the main workload: slot write + paged attention,
    repeated whole steps until about `budget_s` seconds have run."""
    from threadpoolctl import threadpool_info
    import oracle.pagedkv_oracle as O

    reps, t0 = 0, time.perf_counter()
    while True:
        O.step(b)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    per_step = el / reps
    gbs = (attention_bytes(b) + write_bytes(b)) / per_step / 1e9
    # the same with BLAS limited to one thread (a third of the budget)
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        reps1, t1 = 0, time.perf_counter()
        while True:
            O.step(b)
            reps1 += 1
            el1 = time.perf_counter() - t1
            if el1 >= budget_s / 3 or reps1 >= 20:
                break
    per1 = el1 / reps1
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{reps} whole steps of {b.name} (seed 0), fp64 NumPy, "
                      f"{per_step * 1e3:.1f} ms per step",
            "host_cpus": os.cpu_count(),
            "one_thread": {"value": round((attention_bytes(b) + write_bytes(b)) / per1 / 1e9, 4),
                           "unit": "GB/s", "cores": 1,
                           "sample": f"{reps1} whole steps, {per1 * 1e3:.1f} ms per step"}}


# ---------------------------------------------------------------------------
# counters taken offline (profiles/traffic.json), valid only for unchanged kernels
# ---------------------------------------------------------------------------

# The sources that define the decode call whose HBM traffic the counters measure.
TRAFFIC_SOURCES = ("api.hip", "decode.hip", "decode_body.h", "pkv_device.h", "pkv_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_290_amd", "csrc")
    for n in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(n.encode() + f.read())
    return h.hexdigest()


def traffic_for(workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != kernel_source_hash():
        return None
    ent = t.get("workloads", {}).get(workload)
    return None if ent is None else ent.get("bytes_per_call")


def write_traffic(out_dir: str, workload: str = MAIN) -> dict:
    """Build profiles/traffic.json from rocprofv3 --pmc runs of this script: FETCH_SIZE
    and WRITE_SIZE of `bench.py --only-main` (one pass each) and of
    `bench.py --copy-calibration` (5 plain 256 MiB copies), in `out_dir`/pmc_bench_<C>
    and `out_dir`/pmc_copy_<C>.  Counts are KiB per dispatch; each counter is scaled
    by copy bytes / what it reads for the copies.  bytes_per_call covers the kernels
    of one fused step call (the library's kernels other than kv_write_kernel, which
    only the two-call comparison launches)."""
    import collections
    import csv
    import glob

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        for f in files:
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] != counter:
                    continue
                acc[row["Kernel_Name"]][row["Dispatch_Id"]] += float(row["Counter_Value"])
        return acc

    res = {"workloads": {}}
    copy_bytes = 256 << 20
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = per_kernel(os.path.join(out_dir, f"pmc_copy_{c}"), c)
        vals = [v for k, ds in cp.items() if "copy" in k.lower() or "elementwise" in k
                for v in ds.values() if v > 100000]
        kib = sorted(vals)[len(vals) // 2]
        scale[c] = copy_bytes / (kib * 1024.0)
        res.setdefault("calibration", {})[c.lower() + "_kib"] = kib
    res["calibration"]["copy_bytes"] = copy_bytes
    res["calibration"]["fetch_scale"] = round(scale["FETCH_SIZE"], 4)
    res["calibration"]["write_scale"] = round(scale["WRITE_SIZE"], 4)
    kernels = {}
    total = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        pk = per_kernel(os.path.join(out_dir, f"pmc_bench_{c}"), c)
        tot = 0.0
        for k, ds in pk.items():
            if "pkv::" not in k:
                continue
            short = k.split("<")[0].replace("void ", "").replace("pkv::", "")
            med = sorted(ds.values())[len(ds) // 2]
            kernels.setdefault(short, {})[c] = med
            kernels[short]["dispatches"] = len(ds)
            if short != "kv_write_kernel":  # the two-call comparison only
                tot += med
        total[c] = tot * 1024.0 * scale[c]
    from workloads import make_config
    b = make_config(workload, 0)
    res["workloads"][workload] = {
        "bytes_per_call": int(total["FETCH_SIZE"] + total["WRITE_SIZE"]),
        "fetch_bytes": int(total["FETCH_SIZE"]), "write_bytes": int(total["WRITE_SIZE"]),
        "algorithmic_bytes": attention_bytes(b) + write_bytes(b),
        "per_kernel_kib_raw": kernels}
    res["about"] = ("HBM traffic per step call of the headline workload, from rocprofv3 "
                    "FETCH_SIZE/WRITE_SIZE scaled by a 256 MiB copy calibration; valid "
                    "only while the kernel sources hash to source_sha256")
    res["source_sha256"] = kernel_source_hash()
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(res, f, indent=1)
    return res


def measure_chunk_sweep(calls: int) -> dict:
    """Context: the chunk kernel at step budgets of 512, 1,024, 2,048 and 3,500 rows,
    each the last rows of a 3,500-token prompt (positions 3,500 - q .. 3,499, the
    earlier ones cached), Qwen3-1.7B heads (16q/8kv, d=128, bf16), one sequence, so
    only the chunk kernel launches; HIP events per call.  Pools of 1,024 shuffled
    blocks drawn with the seeded generator (the kernel is MFMA-bound; its K/V traffic
    is ~30 MB per call)."""
    import numpy as np
    import torch

    from workloads import make_batch

    res = {}
    for q in (512, 1024, 2048, 3500):
        rng = np.random.Generator(np.random.PCG64(q))
        b = make_batch(rng, name=f"chunk_{q}", dtype="bf16", num_q_heads=16,
                       num_kv_heads=8, head_dim=128, num_blocks=1024, context_lens=[3500],
                       query_lens=[q])
        r = Runner(b, 4)
        r.write(0)
        ms = time_calls(r, calls, fn=r.attend)
        fl = chunk_flops(b)
        tfs = fl / (ms * 1e-3) / 1e12
        res[f"rows_{q}"] = {"avg_ms": round(ms, 5), "TFLOPs": round(tfs, 1),
                            "frac": round(tfs / BF16_MFMA_PEAK_TFS, 4), "flops": fl}
        del r
        torch.cuda.empty_cache()
    return res


def measure_cascade(r: Runner, steps: int, warmup: int) -> dict:
    """The shared-prefix workload through paged_attention_varlen_shared_prefix (slot
    write + private tails by the decode kernel, the 187 shared blocks once by the chunk
    kernel, merge): graph-timed step and event-timed call, GB/s on unique bytes."""
    b = r.b
    ms = time_graph(r, steps, warmup, fn=r.cascade)
    call_ms = time_calls(r, steps, fn=r.cascade)
    nbytes = attention_bytes(b) + write_bytes(b)
    return {"ms_per_step": round(ms, 5), "call_ms": round(call_ms, 5),
            "step_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "call_GBs": round(nbytes / (call_ms * 1e-3) / 1e9, 1),
            "call_hbm_frac": round(nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "calls": "paged_attention_varlen_shared_prefix (decode_kernel on the "
                     "private blocks, prefill_mfma_kernel on the shared run, "
                     "cascade_merge_kernel)"}


def measure_chunk(bx, calls: int) -> dict:
    """The 2,017-row prefill chunk of the mixed step alone (sequence 0 only): the
    attention call launches prefill_mfma_kernel only.  The launch's average comes from
    HIP events around a HIP graph of `calls` back-to-back calls (as for the decode
    headline); the eager call, timed with HIP events per call, is context."""
    import copy

    import torch

    bc = copy.copy(bx)
    bc.block_tables = bx.block_tables[:1]
    bc.context_lens = bx.context_lens[:1]
    q0 = int(bx.query_start_loc[1])
    bc.query_start_loc = bx.query_start_loc[:2]
    bc.q, bc.k_new, bc.v_new = bx.q[:q0], bx.k_new[:q0], bx.v_new[:q0]
    bc.slot_mapping = bx.slot_mapping[:q0]
    rc = Runner(bc, 4)
    for i in range(4):
        rc.write(i)
    ev = {}
    time_graph(rc, calls, 2, fn=rc.attend, events=ev)
    gms = ev["event_ms"]
    cms = time_calls(rc, calls, fn=rc.attend)
    cfl = chunk_flops(bc)
    tfs = cfl / (gms * 1e-3) / 1e12
    del rc
    torch.cuda.empty_cache()
    return {"workload": "chunked_prefill_mixed: the 2,017-row chunk alone",
            "bound": "mfma", "achieved": round(tfs, 2), "peak": BF16_MFMA_PEAK_TFS,
            "unit": "TFLOP/s", "frac": round(tfs / BF16_MFMA_PEAK_TFS, 4), "flops": cfl,
            "avg_ms": round(gms, 5),
            "avg_ms_source": "HIP events on the replay stream around a graph of back-to-back "
                             "calls, divided by their number",
            "eager_call_ms": round(cms, 5), "kernel": "prefill_mfma_kernel"}


def measure_block_copy(calls: int, pairs: int = 1024) -> dict:
    """Copy-on-write block copies (paged_kv_copy_blocks) on a Qwen3-1.7B-shaped pool
    (8 kv heads, d=128, bf16: 32 KiB per block and pool): `pairs` random (source,
    destination) pairs per call, both pools.  Algorithmic bytes per call = every
    copied byte read once and written once.  Four pools are rotated (over 1 GiB in
    total) so the copies come from HBM."""
    import numpy as np
    import torch

    import paged_kv_cache_290_amd as pkv

    hkv, d, nb = 8, 128, 4 * pairs
    rng = np.random.Generator(np.random.PCG64(0))
    sets = []
    for _ in range(4):
        k = torch.empty((nb, hkv, 16, d), dtype=torch.bfloat16, device="cuda").normal_()
        v = torch.empty_like(k).normal_()
        perm = rng.permutation(nb)[:2 * pairs].reshape(pairs, 2)
        sets.append((k, v, torch.from_numpy(perm.astype(np.int32)).cuda()))
    stream = torch.cuda.current_stream()
    for k, v, c in sets:
        pkv.copy_blocks(k, v, c)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    torch.cuda._sleep(int(2e8))
    for i in range(calls):
        k, v, c = sets[i % 4]
        evs[i][0].record(stream)
        pkv.copy_blocks(k, v, c)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = sum(a.elapsed_time(b) for a, b in evs) / calls
    # The launch's average, as for the other kernels: HIP events on the replay stream
    # around a graph of `calls` back-to-back copies (the same four rotating pools),
    # divided by their number.
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(calls):
                k, v, c = sets[i % 4]
                pkv.copy_blocks(k, v, c)
    stream.wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e8))
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    del g
    nbytes = pairs * 2 * (hkv * 16 * d * 2) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    # Context: a plain contiguous device copy of the same bytes (torch's copy_), timed
    # the same way over four rotating buffer pairs.
    half = nbytes // 2
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda").fill_(1),
             torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(4)]
    for a_, b_ in bufs:
        b_.copy_(a_)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    for i in range(calls):
        a_, b_ = bufs[i % 4]
        evs[i][0].record(stream)
        b_.copy_(a_)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms_plain = sum(a.elapsed_time(b) for a, b in evs) / calls
    del sets, bufs
    torch.cuda.empty_cache()
    return {"workload": f"{pairs} copy-on-write block copies, 8 kv heads x 16 x 128 bf16 "
                        "blocks, both pools", "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "avg_ms": round(ms, 5),
            "avg_ms_source": "HIP events on the replay stream around a graph of back-to-back "
                             "calls, divided by their number",
            "eager_call_ms": round(call_ms, 5),
            "kernel": "copy_blocks_kernel",
            "plain_contiguous_copy_GBs": round(nbytes / (ms_plain * 1e-3) / 1e9, 1),
            "vs_plain_contiguous_copy": round(ms_plain / call_ms, 4),
            "vs_plain_contiguous_copy_note": "both timed per eager call"}



def measure_planned_prefill(reps: int = 3) -> dict:
    """Chunked prefill driven by the library's planner: an 8,192-token prompt arrives
    while 31 requests decode (contexts U[300, 4096], Qwen3-1.7B heads 16q/8kv, d=128,
    bf16) under a 2,048-token step budget.  Each step is planned on the host
    (pkv_plan_step, pkv_build_step through the binding), its metadata goes to the
    device in one pinned host-to-device copy, the fused write + attention call runs,
    and the host waits for the step (the next step's plan needs its result).  Reports
    the host planning time per step, the GPU time per step (HIP events around the
    step's calls), and the wall time of the whole prefill with its tokens/s.  The
    per-step q, k_new and v_new come from buffers filled before timing."""
    import numpy as np
    import torch

    import paged_kv_cache_290_amd as pkv

    hq, hkv, d, nb, budget, plen = 16, 8, 128, 8192, 2048, 8192
    rng = np.random.Generator(np.random.PCG64(0))
    dec_ctx = [int(c) for c in rng.integers(300, 4096, size=31, endpoint=True)]
    max_blocks = plen // 16 + 1
    nreq = len(dec_ctx) + 1

    def fresh():
        alloc = pkv.BlockAllocator(nb)
        tables = np.full((nreq, max_blocks), -1, dtype=np.int32)
        for r, c in enumerate(dec_ctx):
            t = []
            alloc.append(t, 0, c - 1)
            tables[r, :len(t)] = t
        prompt = np.array([c - 1 for c in dec_ctx] + [plen], dtype=np.int32)
        done = prompt.copy()
        done[-1] = 0
        return alloc, tables, prompt, done

    def advance(done, q):
        done += np.asarray(q, dtype=np.int32)

    # host planning alone
    plan_s, nplan = 0.0, 0
    for _ in range(20):
        alloc, tables, prompt, done = fresh()
        while done[-1] < prompt[-1]:
            t0 = time.perf_counter()
            q = pkv.plan_step(prompt, done, budget)
            alloc.build_step(tables, done, q, max_blocks)
            plan_s += time.perf_counter() - t0
            nplan += 1
            advance(done, q)
        alloc.close()

    kp = torch.empty((nb, hkv, 16, d), dtype=torch.bfloat16, device="cuda").normal_()
    vp = torch.empty_like(kp).normal_()
    qb = torch.empty((budget, hq, d), dtype=torch.bfloat16, device="cuda").normal_()
    knb = torch.empty((budget, hkv, d), dtype=torch.bfloat16, device="cuda").normal_()
    vnb = torch.empty_like(knb).normal_()
    out = torch.empty_like(qb)
    ws = torch.empty(pkv.workspace_size(nreq, budget, hq, hkv, d, plen + 1, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    o_bt, o_ctx = 0, nreq * max_blocks
    o_qsl, o_sl = o_ctx + nreq, o_ctx + 2 * nreq + 1
    o_cp, total_i32 = o_sl + budget, o_sl + budget + 2 * nreq
    host = torch.empty(total_i32, dtype=torch.int32, pin_memory=True)
    hv = host.numpy()
    dev = torch.empty(total_i32, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def gpu_step(sb, evs=None):
        ns, tq, nc = len(sb.seq_request), int(sb.query_start_loc[-1]), len(sb.copies)
        hv[o_bt:o_bt + ns * max_blocks] = sb.block_tables.reshape(-1)
        hv[o_ctx:o_ctx + ns] = sb.context_lens
        hv[o_qsl:o_qsl + ns + 1] = sb.query_start_loc
        hv[o_sl:o_sl + tq] = sb.slot_mapping
        hv[o_cp:o_cp + 2 * nc] = sb.copies.reshape(-1)
        dev.copy_(host, non_blocking=True)
        if evs:
            evs[0].record(stream)
        if nc:
            pkv.copy_blocks(kp, vp, dev[o_cp:o_cp + 2 * nc].view(nc, 2))
        pkv.attention_with_write(
            qb[:tq], knb[:tq], vnb[:tq], kp, vp, dev[o_sl:o_sl + tq],
            dev[o_bt:o_bt + ns * max_blocks].view(ns, max_blocks), dev[o_ctx:o_ctx + ns],
            dev[o_qsl:o_qsl + ns + 1], scale=1.0 / math.sqrt(d),
            max_context_len=int(sb.context_lens.max()),
            max_query_len=int(np.diff(sb.query_start_loc).max()), out=out[:tq],
            workspace=ws)
        if evs:
            evs[1].record(stream)
        torch.cuda.synchronize()

    walls, gpu_ms, steps, tokens = [], [], 0, 0
    for rep in range(reps + 1):               # the first run warms up
        alloc, tables, prompt, done = fresh()
        n_steps = n_tok = 0
        step_ms = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while done[-1] < prompt[-1]:
            q = pkv.plan_step(prompt, done, budget)
            sb = alloc.build_step(tables, done, q, max_blocks)
            evs = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            gpu_step(sb, evs)
            step_ms.append(evs[0].elapsed_time(evs[1]))
            n_steps += 1
            n_tok += int(sum(q))
            advance(done, q)
        wall = time.perf_counter() - t0
        alloc.close()
        if rep:
            walls.append(wall)
            gpu_ms.append(sum(step_ms) / len(step_ms))
            steps, tokens = n_steps, n_tok
    wall = min(walls)
    del kp, vp, qb, knb, vnb, out, ws, dev
    torch.cuda.empty_cache()
    return {"workload": "8,192-token prompt prefilled under a 2,048-token step budget "
                        "beside 31 decoding requests (contexts U[300,4096]), 16q/8kv "
                        "heads, d=128, bf16, planned by pkv_plan_step/pkv_build_step",
            "steps": steps, "tokens": tokens,
            "host_plan_us_per_step": round(plan_s / nplan * 1e6, 1),
            "gpu_ms_per_step": round(min(gpu_ms), 5),
            "wall_ms_per_step": round(wall / steps * 1e3, 5),
            "wall_ms_total": round(wall * 1e3, 4),
            "prefill_tokens_per_s": round(plen / wall, 1),
            "step_tokens_per_s": round(tokens / wall, 1),
            "wall_includes": "planning, one pinned H2D copy of the step metadata, the "
                             "fused call, and a host wait per step"}


def measure_prefix_cache(calls: int = 20) -> dict:
    """Prefix caching on the serving-engine page's measurement shape: a 3,000-token
    common prefix plus a 32-token tail per request (Qwen3-1.7B heads 16q/8kv, d=128,
    bf16).  Host: the block keys of one 3,032-token prompt (pkv_block_keys, SHA-256)
    and the cache lookup of a later request (pkv_prefix_match, 187 blocks found).
    GPU: the attention prefill of the whole prompt (the first request) against that of
    the 40 tokens a later request still computes (HIP events per call, calls queued
    behind a spin kernel)."""
    import numpy as np
    import torch

    import paged_kv_cache_290_amd as pkv

    hq, hkv, d, nb, mb = 16, 8, 128, 1024, 256
    rng = np.random.Generator(np.random.PCG64(0))
    prefix = rng.integers(0, 151_936, 3000).astype(np.int32)
    prompts = [np.concatenate([prefix, rng.integers(0, 151_936, 32).astype(np.int32)])
               for _ in range(8)]

    t0 = time.perf_counter()
    for p in prompts:
        pkv.block_keys(p)
    key_us = (time.perf_counter() - t0) / len(prompts) * 1e6
    alloc = pkv.BlockAllocator(nb)
    alloc.enable_prefix_cache()
    first = []
    alloc.append(first, 0, len(prompts[0]))
    alloc.prefix_register(first, pkv.block_keys(prompts[0]))
    match_us, tables, hits = 0.0, [], 0
    for p in prompts[1:]:
        keys = pkv.block_keys(p)
        t0 = time.perf_counter()
        t = alloc.prefix_match(keys)
        match_us += time.perf_counter() - t0
        hits = len(t)
        alloc.append(t, 16 * len(t), len(p) - 16 * len(t))
        tables.append(t)
    match_us = match_us / (len(prompts) - 1) * 1e6

    kp = torch.empty((nb, hkv, 16, d), dtype=torch.bfloat16, device="cuda").normal_()
    vp = torch.empty_like(kp).normal_()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa
    stream = torch.cuda.current_stream()

    def timed(table, ctx, n):
        q = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda").normal_()
        kn = torch.empty((n, hkv, d), dtype=torch.bfloat16, device="cuda").normal_()
        vn = torch.empty_like(kn).normal_()
        slots = i32([table[p // 16] * 16 + p % 16 for p in range(ctx - n, ctx)])
        bt = np.full((1, mb), -1, np.int32)
        bt[0, :len(table)] = table
        bt, cl, qsl = i32(bt), i32([ctx]), i32([0, n])
        ws = torch.empty(pkv.workspace_size(1, n, hq, hkv, d, ctx, torch.bfloat16) or 1,
                         dtype=torch.uint8, device="cuda")
        out = torch.empty_like(q)

        def call():
            pkv.attention_with_write(q, kn, vn, kp, vp, slots, bt, cl, qsl,
                                     scale=1.0 / math.sqrt(d), max_context_len=ctx,
                                     max_query_len=n, out=out, workspace=ws)
        call()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(calls)]
        torch.cuda._sleep(int(1e8))
        for a, b in evs:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / calls

    ctx = len(prompts[0])
    full_ms = timed(first, ctx, ctx)
    tail_ms = timed(tables[0], ctx, ctx - 16 * hits)
    del kp, vp
    torch.cuda.empty_cache()
    return {"workload": "3,000-token common prefix + 32-token tail per request, 16q/8kv "
                        "heads, d=128, bf16",
            "host_block_keys_us_per_prompt": round(key_us, 1),
            "host_hash_MBps": round((ctx // 16) * (32 + 64 + 4) / key_us, 1),
            "host_keys_via": "binding, int32 token array in",
            "host_match_us": round(match_us, 2), "blocks_found": hits,
            "tokens_prefilled_first": ctx, "tokens_prefilled_later": ctx - 16 * hits,
            "gpu_prefill_first_ms": round(full_ms, 5),
            "gpu_prefill_later_ms": round(tail_ms, 5),
            "prefill_speedup": round(full_ms / tail_ms, 2)}


def measure_swap(calls: int = 10, n: int = 1024) -> dict:
    """KV swap of n Qwen3-1.7B-shaped blocks (8 kv heads x 16 x 128 bf16: 32 KiB per
    block and pool, 64 MiB for n = 1,024) to pinned host memory and back, each call
    timed with HIP events; beside them, plain pinned copies of the same size in each
    direction (the host link's practical limit on this machine)."""
    import numpy as np
    import torch

    import paged_kv_cache_290_amd as pkv

    hkv, d, nb = 8, 128, 4 * n
    rng = np.random.Generator(np.random.PCG64(0))
    kp = torch.empty((nb, hkv, 16, d), dtype=torch.bfloat16, device="cuda").normal_()
    vp = torch.empty_like(kp).normal_()
    blocks = torch.from_numpy(rng.permutation(nb)[:n].astype(np.int32)).cuda()
    nbytes = pkv.swap_bytes(kp, n)
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    staging = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(calls)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / calls

    out_ms = timed(lambda: pkv.swap_out(kp, vp, blocks, staging, host))
    in_ms = timed(lambda: pkv.swap_in(kp, vp, blocks, staging, host))
    d2h_ms = timed(lambda: host.copy_(dev, non_blocking=True))
    h2d_ms = timed(lambda: dev.copy_(host, non_blocking=True))
    gb = nbytes / 1e9
    del kp, vp, staging, dev
    torch.cuda.empty_cache()
    return {"workload": f"{n} blocks of 8 kv heads x 16 x 128 bf16, both pools "
                        f"({nbytes / 2**20:.0f} MiB), pinned host memory",
            "swap_out_ms": round(out_ms, 4), "swap_in_ms": round(in_ms, 4),
            "swap_out_GBs": round(gb / (out_ms * 1e-3), 2),
            "swap_in_GBs": round(gb / (in_ms * 1e-3), 2),
            "plain_d2h_GBs": round(gb / (d2h_ms * 1e-3), 2),
            "plain_h2d_GBs": round(gb / (h2d_ms * 1e-3), 2),
            "swap_out_frac_of_link": round(d2h_ms / out_ms, 3),
            "swap_in_frac_of_link": round(h2d_ms / in_ms, 3)}

# ---------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-main", action="store_true",
                    help="skip the other four workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain 256 MiB device copies (counter calibration)")
    ap.add_argument("--only-chunk-sweep", action="store_true",
                    help="only the chunk kernel at 512/1,024/2,048/3,500-row budgets")
    ap.add_argument("--only-mixed", action="store_true",
                    help="only the mixed chunked-prefill step (chunk + 31 decodes)")
    ap.add_argument("--only-achievable", action="store_true",
                    help="only the measured HBM read and bf16 GEMM ceilings")
    ap.add_argument("--only-scaling", action="store_true",
                    help="only the headline decode shape at batches 32, 128 and 512")
    ap.add_argument("--only-long", action="store_true",
                    help="only the long-context decode leg (key ranges + merge)")
    ap.add_argument("--only-shared", action="store_true",
                    help="only the shared-prefix workload, plain and cascade (profiling)")
    ap.add_argument("--only-chunk", action="store_true",
                    help="only time the prefill chunk of the mixed step (profiling)")
    ap.add_argument("--only-copy", action="store_true",
                    help="only time the copy-on-write block copies (profiling)")
    ap.add_argument("--only-swap", action="store_true",
                    help="only time the KV swap to host memory and back")
    ap.add_argument("--only-prefix", action="store_true",
                    help="only time prefix caching (host keys and lookup, GPU prefill)")
    ap.add_argument("--only-planned", action="store_true",
                    help="only time the planner-driven chunked prefill (profiling)")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="(host only) summarise rocprofv3 --pmc runs found in DIR into "
                         "profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.write_traffic:
        print(json.dumps(write_traffic(args.write_traffic), indent=1))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library and this benchmark run on exactly one GPU; there is "
              "no multi-GPU path (decode would shard by sequence or by kv head, with no "
              "exchange between GPUs)", file=sys.stderr)
        return 2

    import torch
    from workloads import make_config

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": src.numel()}))
        return 0

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.only_copy:
        print(json.dumps({"block_copy": measure_block_copy(args.steps)}))
        return 0
    if args.only_planned:
        print(json.dumps({"planned_prefill": measure_planned_prefill()}))
        return 0
    if args.only_prefix:
        print(json.dumps({"prefix_cache": measure_prefix_cache()}))
        return 0
    if args.only_swap:
        print(json.dumps({"swap": measure_swap()}))
        return 0
    if args.only_chunk_sweep:
        print(json.dumps({"chunk_budget_sweep": measure_chunk_sweep(args.steps)}))
        return 0

    if args.only_mixed:
        bx = make_config("chunked_prefill_mixed", 0)
        rx = Runner(bx, rotation_for(bx))
        msx = time_graph(rx, args.steps, args.warmup)
        ax = time_calls(rx, args.steps)
        ab, wb = attention_bytes(bx), write_bytes(bx)
        print(json.dumps({"chunked_prefill_mixed": {
            "ms_per_step": round(msx, 5), "call_ms": round(ax, 5),
            "step_GBs": round((ab + wb) / (msx * 1e-3) / 1e9, 1),
            "step_TFLOPs": round(chunk_flops(bx) / (msx * 1e-3) / 1e12, 2)}}))
        return 0

    if args.only_shared:
        bx = make_config("shared_prefix_decode", 0)
        rx = Runner(bx, rotation_for(bx))
        ab, wb = attention_bytes(bx), write_bytes(bx)
        ax = time_calls(rx, args.steps)
        print(json.dumps({"shared_prefix_decode": {
            "plain_call_ms": round(ax, 5),
            "plain_call_GBs": round((ab + wb) / (ax * 1e-3) / 1e9, 1),
            "shared_prefix_cascade": measure_cascade(rx, args.steps, args.warmup)}}))
        return 0

    if args.only_achievable:
        print(json.dumps({"achievable": measure_achievable(args.steps)}))
        return 0

    if args.only_long:
        print(json.dumps({"decode_long_context": measure_long_context(args.steps,
                                                                      args.warmup)}))
        return 0

    if args.only_scaling:
        print(json.dumps({"decode_batch_scaling": measure_batch_scaling(args.steps,
                                                                        args.warmup)}))
        return 0

    if args.only_chunk:
        print(json.dumps({"prefill_chunk": measure_chunk(make_config("chunked_prefill_mixed",
                                                                     0), args.steps)}))
        return 0

    # ---- the headline workload ----
    log(f"generating {MAIN}")
    b = make_config(MAIN, 0)
    rot = rotation_for(b)
    r = Runner(b, rot)
    log(f"timing {args.steps} graph-captured steps over {rot} rotating copies")
    ev = {}
    ms = time_graph(r, args.steps, args.warmup, events=ev)
    ms_two = time_graph(r, args.steps, args.warmup, fn=r.step_two_calls)
    call_dist = {}
    call_ms = time_calls(r, args.steps, dist=call_dist)
    abytes, wbytes = attention_bytes(b), write_bytes(b)
    value = (abytes + wbytes) / (ms * 1e-3) / 1e9
    # One launch per step at this shape (no key ranges, so no merge launch): the
    # launch's average duration is the timed region's HIP-event time over its K steps.
    assert r.pkv.workspace_size(b.num_seqs, b.total_q, b.num_q_heads, b.num_kv_heads,
                                b.head_dim, b.max_context_len, torch.bfloat16) == 0
    launch_ms = ev["event_ms"]
    achieved = (abytes + wbytes) / (launch_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(MAIN),
            "kernel": "paged_attention_varlen_with_write: decode_kernel (with the slot "
                      "write; one launch per step, no key ranges to merge at this shape)",
            "algorithmic_bytes": abytes + wbytes, "avg_ms": round(launch_ms, 5),
            "avg_ms_source": "HIP events on the replay stream around the timed graph of "
                             "K steps, divided by K (back-to-back launches)",
            "eager_call_ms": round(call_ms, 5), "eager_call_percentiles": call_dist}
    del r
    torch.cuda.empty_cache()
    # warm: the same copy every step, so K/V may come from the 256 MB MALL (context)
    rw = Runner(b, 1)
    ms_warm = time_graph(rw, args.steps, args.warmup)
    warm = {"ms_per_step": round(ms_warm, 5),
            "GBs": round((abytes + wbytes) / (ms_warm * 1e-3) / 1e9, 1),
            "note": "one copy reused every step (unflushed caches); context only"}
    del rw
    torch.cuda.empty_cache()

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": MAIN, "batch": 32, "num_q_heads": 32, "num_kv_heads": 8,
                   "head_dim": 64, "block_size": 16, "context_lens": "U[128,2048]",
                   "pool_blocks": 8192, "seed": 0, "rotating_copies": rot,
                   "timed_region": "HIP graph of the K steps"},
        "roofline": roof,
        "warm_step": warm,
        "two_call_step": {"ms_per_step": round(ms_two, 5),
                          "GBs": round((abytes + wbytes) / (ms_two * 1e-3) / 1e9, 1),
                          "calls": "paged_kv_write then paged_attention_varlen"},
    }

    # ---- the other workloads (context lines, same protocol) ----
    if not args.only_main:
        extra = {}
        for name in ("qwen3_1p7b_decode_640", "shared_prefix_decode",
                     "chunked_prefill_mixed", "tiny_f32_decode"):
            log(f"generating {name}")
            bx = make_config(name, 0)
            rx = Runner(bx, rotation_for(bx))
            msx = time_graph(rx, args.steps, args.warmup)
            ax = time_calls(rx, args.steps)
            ab, wb = attention_bytes(bx), write_bytes(bx)
            ent = {"ms_per_step": round(msx, 5), "call_ms": round(ax, 5),
                   "step_GBs": round((ab + wb) / (msx * 1e-3) / 1e9, 1),
                   "call_GBs": round((ab + wb) / (ax * 1e-3) / 1e9, 1),
                   "call_hbm_frac": round((ab + wb) / (ax * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if name == "shared_prefix_decode":
                lb = attention_bytes(bx, unique=False)
                ent["call_logical_GBs"] = round((lb + wb) / (ax * 1e-3) / 1e9, 1)
                ent["shared_prefix_cascade"] = measure_cascade(rx, args.steps, args.warmup)
            if name == "chunked_prefill_mixed":
                fl = chunk_flops(bx)
                ent["step_TFLOPs"] = round(fl / (msx * 1e-3) / 1e12, 2)
                del rx
                torch.cuda.empty_cache()
                result["prefill_chunk"] = measure_chunk(bx, args.steps)
            else:
                del rx
            torch.cuda.empty_cache()
            extra[name] = ent
        result["workloads"] = extra
        log("timing the headline decode shape at larger batches")
        result["decode_batch_scaling"] = measure_batch_scaling(args.steps, args.warmup)
        log("timing long-context decode (key ranges + merge)")
        result["decode_long_context"] = measure_long_context(args.steps, args.warmup)
        log("timing the chunk kernel at several step budgets")
        result["chunk_budget_sweep"] = measure_chunk_sweep(args.steps)
        log("measuring achievable HBM read and bf16 GEMM rates")
        ach = measure_achievable(args.steps)
        ach["headline_call_vs_scattered_read"] = round(
            roof["achieved"] / ach["read_scattered_2KiB_512MiB"]["GBs"], 4)
        ach["headline_call_vs_step_sized_read"] = round(
            roof["achieved"] / ach["read_scattered_2KiB_headline_step"]["GBs"], 4)
        if "prefill_chunk" in result:
            ach["chunk_vs_gemm"] = round(
                result["prefill_chunk"]["achieved"] / ach["bf16_gemm_8192"]["TFLOPs"], 4)
        result["achievable"] = ach
        log("timing copy-on-write block copies")
        result["block_copy"] = measure_block_copy(args.steps)
        log("timing the planner-driven chunked prefill")
        result["planned_prefill"] = measure_planned_prefill()
        log("timing prefix caching")
        result["prefix_cache"] = measure_prefix_cache()
        log("timing KV swap")
        result["swap"] = measure_swap()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
