#!/usr/bin/env python3
"""Decode-step benchmark for paged decode attention on one MI355X.

One step = one new token for every sequence, through every layer: kv_append of
the token's K/V row into the page its block table names, then paged decode
attention (split kernel + log-sum-exp merge) over all of the sequence's pages.
The default workload is the Llama-3-70B-shaped full cache: 80 layers, 32
sequences of 8,192 tokens, 64 query / 8 KV heads, head_dim 128, pages of 16
tokens, bfloat16 K/V (85,899,345,920 bytes, "Understanding KV-Cache
Optimization in Modern LLM Serving", section "Concrete Example"), every page
resident in HBM when the timed region starts.

Prints ONE JSON line on stdout (progress goes to stderr):
  value       KV-read GB/s: algorithmic bytes of a step / wall time of a step
  roofline    the split kernel's algorithmic bytes per launch / its mean
              duration from HIP events inside the timed region, against 8 TB/s
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same data
  parity      sampled outputs of the timed step against the oracle

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
    python bench.py --copy-calibration   # plain copy kernel for counter scaling
    python bench.py --probe-calibration  # streaming-read probe (non-temporal loads), same
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD's published figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")
# sources that decide the split kernel's code and launch shape
KERNEL_SOURCES = ("paged_kv_cache_465_amd/csrc/decode.hip",
                  "paged_kv_cache_465_amd/csrc/decode_kernels.h",
                  *(f"paged_kv_cache_465_amd/csrc/decode_{f}_{p}.hip"
                    for f in ("bf16", "int8", "int4", "fp8") for p in ("split", "sched")),
                  "paged_kv_cache_465_amd/csrc/device_common.h",
                  "paged_kv_cache_465_amd/csrc/pool.cpp")
# sources that decide the multi-query (chunked prefill, verification) kernel
PREFILL_SOURCES = ("paged_kv_cache_465_amd/csrc/prefill.hip",
                   "paged_kv_cache_465_amd/csrc/prefill_kernels.h",
                   *(f"paged_kv_cache_465_amd/csrc/prefill_{f}.hip"
                     for f in ("bf16", "int8", "int4", "fp8")),
                   "paged_kv_cache_465_amd/csrc/device_common.h")
MALL_FLUSH_BYTES = 1 << 30      # > 256 MB Infinity Cache


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warmup steps (default: at least 5 and at least half a second "
                        "of steps, so that the clocks have settled before the timed steps)")
    p.add_argument("--config", default="llama3_70b_full_cache")
    p.add_argument("--splits", type=int, default=0, help="forced split count (0 = planner)")
    p.add_argument("--plan", choices=("auto", "uniform", "balanced"), default="auto",
                   help="decode work plan: the uniform split plan, a balanced schedule built "
                        "from the host lengths, or auto (balanced when the lengths differ)")
    p.add_argument("--bins", type=int, default=0,
                   help="most bins of the balanced schedule (0 = the library's choice: "
                        "four per compute unit, eight for quantized pools)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--no-parity", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of known size (for counter scaling)")
    p.add_argument("--probe-calibration", action="store_true",
                   help="only run the streaming-read probe (2 GiB of non-temporal chunk reads "
                        "per launch: counter scaling for the decode kernels' loads)")
    return p.parse_args(argv)


# ---- algorithmic bytes -----------------------------------------------------------
def is_chunked(cfg) -> bool:
    return cfg.q_len > 1 or cfg.q_len_hi > 1


def step_flops(cfg, ctx: np.ndarray, q_start: np.ndarray) -> int:
    """Multiply-adds x 2 of q.K^T and P.V over every (query row, position it
    attends to), all layers: 4 * D * H_q per (row, position)."""
    total = 0
    for b in range(len(ctx)):
        n, L = int(ctx[b]), int(q_start[b + 1] - q_start[b])
        if cfg.window_tokens > 0:
            n_att = min(n, cfg.sink_tokens + cfg.window_tokens)
            total += L * n_att
        else:
            pos = n - L + np.arange(L)
            total += int(np.maximum(pos + 1, 0).sum())
    return 4 * cfg.head_dim * cfg.num_q_heads * total * cfg.layers


def step_bytes(cfg, ctx: np.ndarray, n_rows: int = None) -> dict:
    """Bytes a step must move at minimum, per term, summed over sequences and layers.

    Per sequence of n tokens and per layer: K and V rows n*H_kv*D elements each
    (plus one float16 (scale, zero) pair per row for the quantized formats:
    INT8 and FP8 one byte per element, INT4 half a byte), the query and output
    rows H_q*D bfloat16 each, the used block-table entries and the context
    length (int32), and the appended row (read once, written once, K and V).
    """
    eb = {"bf16": 2, "int8": 1, "fp8": 1, "int4": 0.5}[cfg.kv_dtype]
    quant = cfg.kv_dtype != "bf16"
    n = ctx.astype(np.int64)
    if cfg.window_tokens > 0:
        # tokens attended with sinks + a recent window
        n = np.minimum(n, cfg.sink_tokens + cfg.window_tokens)
    Hkv, Hq, D, P, L = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.page_size, cfg.layers
    kv = int((n * Hkv * 2 * D * eb).sum())
    if quant:
        kv += int((n * Hkv * 2 * 4).sum())
    B = int(n.shape[0])
    N = B if n_rows is None else int(n_rows)     # query rows (new tokens) in a step
    q_out = N * Hq * D * 2 * 2
    table = int((-(-n // P) * 4).sum()) + B * 4
    append = N * Hkv * D * 2 * 2 * (1 + eb / 2) + (N * Hkv * 2 * 4 if quant else 0)
    return {"kv": kv * L, "q_out": q_out * L, "table": table * L, "append": int(append) * L,
            "split_kernel_per_launch": kv + N * Hq * D * 2 + table}


# ---- device setup ------------------------------------------------------------------
class Layer:
    __slots__ = ("k", "v", "km", "vm", "q", "nk", "nv", "out")


def setup_device(kvp, cfg, case, dev):
    import torch
    from workloads import history_rows_device

    desc = kvp.make_desc(case.num_pages, cfg.page_size, cfg.num_kv_heads, cfg.head_dim,
                         cfg.kv_dtype)
    pool = kvp.kvp_pool_create(desc)
    kv_bytes, meta_bytes = kvp.kvp_pool_bytes(desc)
    quant = cfg.kv_dtype != "bf16"
    bt = torch.from_numpy(case.block_tables).to(dev)
    ctx = torch.from_numpy(case.ctx).to(dev)
    seq_idx = torch.from_numpy(case.new_seq.astype(np.int32)).to(dev)
    new_pos = torch.from_numpy(case.new_pos.astype(np.int32)).to(dev)
    layers = []
    t0 = time.perf_counter()
    for l in range(cfg.layers):
        L = Layer()
        if quant:
            L.k = torch.empty(kv_bytes, dtype=torch.int8, device=dev)
            L.v = torch.empty(kv_bytes, dtype=torch.int8, device=dev)
            L.km = torch.empty(meta_bytes // 2, dtype=torch.int16, device=dev)
            L.vm = torch.empty(meta_bytes // 2, dtype=torch.int16, device=dev)
        else:
            L.k = torch.empty(kv_bytes // 2, dtype=torch.int16, device=dev)
            L.v = torch.empty(kv_bytes // 2, dtype=torch.int16, device=dev)
            L.km = L.vm = None
        if cfg.device_data:
            q, hk, hv, hs, hp, nk, nv, _ = history_rows_device(cfg, case, l, dev)
            q, hk, hv = q.view(torch.int16), hk.view(torch.int16), hv.view(torch.int16)
            nk, nv = nk.view(torch.int16), nv.view(torch.int16)
        else:
            def up(a):
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
            q, hk, hv, nk, nv = up(case.q), up(case.hist_k), up(case.hist_v), up(case.new_k), \
                up(case.new_v)
            hs = torch.from_numpy(case.hist_seq).to(dev)
            hp = torch.from_numpy(case.hist_pos).to(dev)
        kvp.kvp_kv_append(pool, L.k, L.v, L.km, L.vm, hk, hv, hs, hp, bt)
        del hk, hv, hs, hp
        L.q, L.nk, L.nv = q, nk, nv
        L.out = torch.empty_like(q)
        layers.append(L)
        if l % 10 == 9 or l == cfg.layers - 1:
            torch.cuda.synchronize()
            log(f"[setup] layer {l + 1}/{cfg.layers} filled ({time.perf_counter() - t0:.1f} s)")
    torch.cuda.synchronize()
    return pool, layers, bt, ctx, seq_idx, new_pos


def run_gpu(args, kvp, cfg, case):
    import torch
    dev = torch.device("cuda:0")
    pool, layers, bt, ctx, seq_idx, new_pos = setup_device(kvp, cfg, case, dev)
    B, Hq, D = case.B, cfg.num_q_heads, cfg.head_dim
    max_ctx = int(case.ctx.max())
    plan_ctx = max_ctx
    if cfg.window_tokens > 0:
        P = cfg.page_size
        plan_ctx = min(max_ctx, (-(-cfg.sink_tokens // P) + -(-cfg.window_tokens // P) + 1) * P)
    S, pbytes = kvp.kvp_decode_partials_bytes(pool, B, Hq, plan_ctx, args.splits)
    plan = kvp.kvp_decode_plan(pool.desc, B, Hq, plan_ctx, args.splits,
                               torch.cuda.get_device_properties(0).multi_processor_count)
    partials = torch.empty(max(pbytes, 4) // 4, dtype=torch.float32, device=dev) if S > 1 else None
    scale = float(case.scale)
    log(f"[plan] {plan}")

    windowed = cfg.window_tokens > 0
    chunked = is_chunked(cfg)
    balanced = not chunked and args.splits == 0 and (
        args.plan == "balanced" or (args.plan == "auto" and int(np.ptp(case.ctx)) > 0))
    sched = sched_dev = sched_ws = None
    if balanced:
        # one schedule serves every layer (they share lengths and tables); the
        # bench's lengths are the same every step, so it is built once here
        cus = args.bins or kvp.kvp_decode_schedule_bins(pool, Hq)
        t0 = time.perf_counter()
        reps = 20
        for _ in range(reps):
            sched = kvp.kvp_decode_schedule(pool, case.ctx, Hq, int(case.block_tables.shape[1]),
                                            cus, cfg.sink_tokens, cfg.window_tokens)
        sched_host_us = (time.perf_counter() - t0) / reps * 1e6
        sched_dev = torch.from_numpy(sched.used.copy()).to(dev)
        wsb = sched.info.workspace_bytes
        sched_ws = torch.empty(max(wsb, 4) // 4, dtype=torch.float32, device=dev) if wsb else None
        i = sched.info
        plan = {"balanced": True, "num_bins": i.num_bins, "num_items": i.num_items,
                "num_merge": i.num_merge, "num_slots": i.num_slots,
                "waves_per_group": plan["waves_per_group"], "use_mfma": plan["use_mfma"],
                "workspace_bytes": int(wsb), "schedule_bytes": int(i.sched_words) * 4,
                "schedule_host_us": round(sched_host_us, 1)}
        log(f"[plan] balanced schedule {plan}")
    q_start = torch.from_numpy(case.q_start.astype(np.int32)).to(dev)
    max_q_len = int(np.diff(case.q_start).max())
    prefill_order = None
    prefill_plan = {"plan": "grid order"}
    if chunked and args.plan != "uniform":
        # longest-first workgroup order for the multi-query call, built once
        # from the host lengths (the same every step)
        t0 = time.perf_counter()
        reps = 20
        for _ in range(reps):
            order = kvp.kvp_prefill_schedule(pool, case.q_start, case.ctx, Hq,
                                             int(case.block_tables.shape[1]), max_q_len, max_ctx)
        sched_host_us = (time.perf_counter() - t0) / reps * 1e6
        prefill_order = torch.from_numpy(order).to(dev)
        prefill_plan = {"plan": "longest-first", "order_entries": int(order.size),
                        "order_padding": int(np.count_nonzero(order < 0)),
                        "schedule_host_us": round(sched_host_us, 1)}
        log(f"[plan] multi-query order {prefill_plan}")
    if windowed:
        wsb = kvp.kvp_decode_window_workspace_bytes(pool, B, Hq, max_ctx, cfg.sink_tokens,
                                                    cfg.window_tokens, args.splits)
        wspace = torch.empty(max(wsb, 4) // 4, dtype=torch.float32, device=dev) if wsb else None

    def one_step(probe=None):
        """All layers once.  probe = (layer, start event, end event): that
        layer's split kernel (with a window: the whole decode call) is
        bracketed by the two events."""
        for i, L in enumerate(layers):
            kvp.kvp_kv_append(pool, L.k, L.v, L.km, L.vm, L.nk, L.nv, seq_idx, new_pos, bt)
            timed = probe is not None and probe[0] == i
            if timed:
                probe[1].record()
            if chunked and prefill_order is not None:
                kvp.kvp_paged_attention_prefill_scheduled(pool, L.q, q_start, L.k, L.v, L.km,
                                                          L.vm, bt, ctx, max_q_len, max_ctx,
                                                          scale, prefill_order, L.out)
                if timed:
                    probe[2].record()
            elif chunked:
                kvp.kvp_paged_attention_prefill(pool, L.q, q_start, L.k, L.v, L.km, L.vm, bt, ctx,
                                                max_q_len, max_ctx, scale, L.out)
                if timed:
                    probe[2].record()
            elif balanced:
                kvp.kvp_paged_attention_decode_scheduled(pool, L.q, L.k, L.v, L.km, L.vm, bt, ctx,
                                                         max_ctx, scale, sched_dev, sched, L.out,
                                                         sched_ws)
                if timed:
                    probe[2].record()
            elif windowed:
                kvp.kvp_paged_attention_decode_window(
                    pool, L.q, L.k, L.v, L.km, L.vm, bt, ctx, max_ctx, scale, cfg.sink_tokens,
                    cfg.window_tokens, L.out, args.splits, wspace)
                if timed:
                    probe[2].record()
            elif S > 1:
                kvp.kvp_paged_attention_decode_partials(pool, L.q, L.k, L.v, L.km, L.vm, bt, ctx,
                                                        max_ctx, scale, partials, args.splits)
                if timed:
                    probe[2].record()
                kvp.kvp_lse_merge(partials, B * Hq, S, D, L.out)
            else:
                kvp.kvp_paged_attention_decode(pool, L.q, L.k, L.v, L.km, L.vm, bt, ctx, max_ctx,
                                               scale, L.out, args.splits)
                if timed:
                    probe[2].record()

    flush = None
    if cfg.layers == 1:
        flush = torch.empty(MALL_FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    if args.warmup is None:
        # short steps: a few of them leave the device below its working clock,
        # so warm up for at least half a second (and at least five steps)
        n, t0 = 0, time.perf_counter()
        while n < 5 or (time.perf_counter() - t0 < 0.5 and n < 20000):
            if flush is not None:
                flush.fill_(float(n))
            one_step()
            n += 1
            if n >= 5:
                torch.cuda.synchronize()
        args.warmup = n
    else:
        for _ in range(args.warmup):
            one_step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # one layer per step (rotating) has its split kernel bracketed by events:
    # an event pair costs a few microseconds of queue time, so bracketing
    # every layer would inflate the step it is meant to measure
    probes = [((k * 37) % len(layers), ev(), ev()) for k in range(args.steps)]
    step_evs = [(ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = 0.0
    if flush is None:
        t0 = time.perf_counter()
        for k in range(args.steps):
            step_evs[k][0].record()
            one_step(probes[k])
            step_evs[k][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # caches smaller than the Infinity Cache: evict it between steps, outside
        # the event pair that times each step
        for k in range(args.steps):
            flush.fill_(float(k))
            step_evs[k][0].record()
            one_step(probes[k])
            step_evs[k][1].record()
        torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in step_evs])
    kern_ms = np.array([a.elapsed_time(b) for _, a, b in probes])
    ms_per_step = wall * 1e3 / args.steps if flush is None else float(step_ms.mean())
    log(f"[bench] ms/step wall={wall * 1e3 / max(args.steps, 1):.3f} events "
        f"mean={step_ms.mean():.3f} min={step_ms.min():.3f}; split kernel mean "
        f"{kern_ms.mean() * 1e3:.1f} us min {kern_ms.min() * 1e3:.1f} us")
    res = {"ms_per_step": ms_per_step, "step_ms_events": step_ms, "kernel_ms": kern_ms,
           "plan": plan, "prefill_plan": prefill_plan, "num_splits": S, "balanced": balanced,
           "merge_launched": bool(balanced and sched.info.num_merge > 0)}
    return res, (pool, layers, bt, ctx)


def kernel_source_digest(chunked: bool = False) -> str:
    """sha256 over the measured kernel's sources (counter readings are tied to
    it): the decode kernels', or the multi-query kernel's for chunked
    workloads."""
    import hashlib
    h = hashlib.sha256()
    for rel in (PREFILL_SOURCES if chunked else KERNEL_SOURCES):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str, chunked: bool = False):
    """HBM bytes per launch of the split kernel from the committed counter
    readings (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads
    for a plain copy of known size), or None when there are none for this
    workload or the kernel's sources changed after they were taken."""
    path = os.path.join(PROFILES, f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest(chunked):
        return None
    return rec


def copy_probe(dev, nbytes=1 << 32, reps=5):
    """A plain device copy of known size: its rate, and the kernel whose
    hardware counters scale FETCH_SIZE/WRITE_SIZE readings."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us": ms * 1e3,
            "GBps_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e9}


def stream_read_probe(kvp, dev, num_cus, pool_bytes=1 << 30, reps=5):
    """The rate the decode kernels' access pattern allows with no arithmetic:
    kvp_probe_read_chunks over two 1 GiB buffers (a K-like and a V-like pool)
    in shuffled 4 KiB chunks (one (page, KV head) tile of 16 tokens x 128
    bfloat16 channels), non-temporal 16-byte loads.  Measured with the decode
    kernel's own shape (two chunks in flight per wavefront, one wavefront per
    SIMD) and with a few others; the best shuffled rate is the ceiling.  For
    context, the same buffers read in order in 8 KiB chunks."""
    import torch
    a = torch.ones(pool_bytes // 4, dtype=torch.int32, device=dev)
    b = torch.ones_like(a)
    g = torch.Generator(device=dev)
    g.manual_seed(465)
    ids = {4096: torch.randperm(pool_bytes // 4096, generator=g, device=dev).to(torch.int32),
           8192: torch.arange(pool_bytes // 8192, dtype=torch.int32, device=dev)}
    runs = [("decode_shape", 4096, 2, 4), ("shuffled_d1_w8", 4096, 1, 8),
            ("shuffled_d2_w8", 4096, 2, 8), ("shuffled_d4_w4", 4096, 4, 4),
            ("linear_8k_d1_w4", 8192, 1, 4)]
    res = {}
    for name, chunk, depth, per_cu in runs:
        waves = per_cu * num_cus
        sink = torch.empty(waves * 64, dtype=torch.int32, device=dev)
        kvp.kvp_probe_read_chunks(a, b, ids[chunk], chunk, waves, sink, depth)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            kvp.kvp_probe_read_chunks(a, b, ids[chunk], chunk, waves, sink, depth)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[name] = {"chunk_bytes": chunk, "chunks_in_flight": depth, "wavefronts": waves,
                     "us": round(us, 2), "GBps": round(2 * pool_bytes / (us * 1e-6) / 1e9, 1)}
    del a, b
    best = max((v["GBps"] for k, v in res.items() if k != "linear_8k_d1_w4"))
    return {"pattern": "two 1 GiB buffers, shuffled 4 KiB chunks, non-temporal 16-byte loads "
                       "(kvp_probe_read_chunks); GBps = best of the shuffled shapes",
            "bytes_per_launch": 2 * pool_bytes, "GBps": best,
            "frac_of_peak": round(best / HBM_PEAK_GBPS, 4), "runs": res}


# ---- CPU oracle leg ------------------------------------------------------------------
def host_layer(cfg, case, dev, layer=0):
    """One layer's inputs on the host, drawn exactly as the device setup draws them."""
    if not cfg.device_data:
        return case
    import copy
    from workloads import history_rows_device
    q, hk, hv, hs, hp, nk, nv, npos = history_rows_device(cfg, case, layer, dev)
    c = copy.copy(case)
    h = lambda t: t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)  # noqa: E731
    c.q, c.hist_k, c.hist_v, c.new_k, c.new_v = h(q), h(hk), h(hv), h(nk), h(nv)
    c.hist_seq, c.hist_pos = hs.cpu().numpy(), hp.cpu().numpy()
    c.new_pos = npos.cpu().numpy()
    c.new_seq = np.arange(c.B, dtype=np.int32)
    return c


def oracle_layer(cfg, hc, seqs):
    """Oracle pools holding the rows of ``seqs`` (bfloat16 or INT8 per the config)."""
    import oracle
    from workloads import POISON_BF16, POISON_F16, POISON_I8
    lay = oracle.PoolLayout(hc.num_pages, cfg.page_size, cfg.num_kv_heads, cfg.head_dim,
                            cfg.kv_dtype)
    k, v, km, vm = lay.empty_pools(POISON_BF16 if cfg.kv_dtype == "bf16" else POISON_I8,
                                   POISON_F16)
    need = set(int(s) for s in seqs) | ({0} if cfg.shared_prefix else set())
    sel = np.isin(hc.hist_seq, list(need))
    oracle.append(lay, k, v, km, vm, hc.hist_k[sel], hc.hist_v[sel], hc.hist_seq[sel],
                  hc.hist_pos[sel], hc.block_tables)
    nsel = np.isin(hc.new_seq, list(need))
    oracle.append(lay, k, v, km, vm, hc.new_k[nsel], hc.new_v[nsel], hc.new_seq[nsel],
                  hc.new_pos[nsel], hc.block_tables)
    return lay, (k, v, km, vm)


def oracle_decode(cfg, lay, hc, pools, seqs):
    """The oracle's output for ``seqs`` (sinks + window when the config has one)."""
    import oracle
    if is_chunked(cfg):
        return oracle.paged_prefill(lay, hc.q, hc.q_start, *pools, hc.block_tables, hc.ctx,
                                    hc.scale, seqs=seqs)
    if cfg.window_tokens > 0:
        return oracle.paged_decode_window(lay, hc.q, *pools, hc.block_tables, hc.ctx, hc.scale,
                                          cfg.sink_tokens, cfg.window_tokens, seqs=seqs)
    return oracle.paged_decode(lay, hc.q, *pools, hc.block_tables, hc.ctx, hc.scale, seqs=seqs)


def cpu_baseline(cfg, hc, target_s: float):
    import oracle
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    except Exception:
        threads = 1
    order = list(range(hc.B))
    # one sequence first to size the sample, then enough for ~target_s of work
    lay, pools = oracle_layer(cfg, hc, order[:1])
    t0 = time.perf_counter()
    oracle_decode(cfg, lay, hc, pools, order[:1])
    t1 = time.perf_counter() - t0
    n = int(min(hc.B, max(1, round(target_s / max(t1, 1e-6)))))
    seqs = order[:n]
    lay, pools = oracle_layer(cfg, hc, seqs)
    # whole passes over the sample until about target_s of CPU time is spent
    passes, dt = 0, 0.0
    while passes == 0 or dt < target_s:
        t0 = time.perf_counter()
        oracle_decode(cfg, lay, hc, pools, seqs)
        dt += time.perf_counter() - t0
        passes += 1
    # bytes of the sample: one layer of the sampled sequences (same terms as the GPU)
    n_rows = int(sum(hc.q_start[b + 1] - hc.q_start[b] for b in seqs))
    sb = step_bytes(dataclasses.replace(cfg, layers=1, batch=n), hc.ctx[seqs], n_rows)
    sample_bytes = (sb["kv"] + sb["q_out"] + sb["table"]) * passes
    gbps = sample_bytes / dt / 1e9
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"value": gbps, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "blas_threads": int(threads), "os_cpu_count": os.cpu_count(),
            "affinity_cpus": affinity,
            "sample": f"layer 0, sequences 0..{n - 1} of {hc.B}, {passes} passes (float64 numpy "
                      f"gather + attention, {dt:.1f} s); GB/s of the same algorithmic bytes",
            "seconds": dt, "tokens_per_s_equiv": n * passes / dt / cfg.layers,
            "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, family, model and
    stepping (a virtualised host may report a short model name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v
            elif fields:
                break
    except OSError:
        pass
    if not fields:
        return "unknown"
    return (f"{fields.get('model name', 'unknown')} (family {fields.get('cpu family', '?')}, "
            f"model {fields.get('model', '?')}, stepping {fields.get('stepping', '?')})")


def prefix_cache_bench(kvp, dev, n_req=100, prefix=2000, suffix=512, P=16, copies=4096):
    """Host prefix-cache calls for the shared-prefix workload ("Prefix
    Caching": 100 requests sharing a 2000-token prefix): per request one match,
    one grow and one insert; then the device page copy (copy-on-write) over
    ``copies`` pages of a Llama-3-8B-shaped layer (8 KV heads, D = 128)."""
    import torch
    rng = np.random.default_rng(465009)
    desc = kvp.make_desc(16384, P, 8, 128, "bf16")
    pool = kvp.kvp_pool_create(desc)
    cache = kvp.kvp_prefix_cache_create(pool)
    shared = rng.integers(0, 128000, prefix).tolist()
    reqs = [shared + rng.integers(0, 128000, suffix).tolist() for _ in range(n_req)]
    rows = []
    t0 = time.perf_counter()
    matched = 0
    for toks in reqs:
        got = kvp.kvp_prefix_match(cache, toks)
        row = np.full(-(-len(toks) // P), -1, dtype=np.int32)
        row[:got.size] = got
        kvp.kvp_seq_grow(pool, row, got.size * P, len(toks))
        kvp.kvp_prefix_insert(cache, toks, row)
        rows.append(row)
        matched += got.size
    host_s = time.perf_counter() - t0
    unique = n_req * (prefix + suffix) // P - matched
    # device copy-on-write throughput
    kv_bytes, _ = kvp.kvp_pool_bytes(desc)
    k = torch.zeros(kv_bytes // 2, dtype=torch.int16, device=dev)
    v = torch.zeros_like(k)
    perm = rng.permutation(16384).astype(np.int32)
    pairs = torch.from_numpy(np.stack([perm[:copies], perm[copies:2 * copies]], 1).copy()).to(dev)
    kvp.kvp_copy_pages(pool, k, v, None, None, pairs)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        kvp.kvp_copy_pages(pool, k, v, None, None, pairs)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / 10
    page_bytes = 2 * 8 * P * 128 * 2
    moved = 2 * copies * page_bytes   # read + write, K and V
    cache.close()
    pool.close()
    return {"metric": "prefix cache: host us per request; page copy GB/s", "data": "synthetic",
            "config": {"workload": "prefix_cache", "requests": n_req, "shared_tokens": prefix,
                       "own_tokens": suffix, "page_size": P},
            "host_us_per_request": round(host_s * 1e6 / n_req, 2),
            "pages_matched": int(matched), "pages_unique": int(unique),
            "copy_pages": copies, "copy_us": round(us, 2),
            "copy_GBps_read_plus_write": round(moved / (us * 1e-6) / 1e9, 1)}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path "
              "has no multi-GPU mode (the way it would shard across GPUs is documented with the "
              "design).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        r = copy_probe(dev, nbytes=1 << 30, reps=3)
        print(json.dumps({"copy_calibration": r}))
        return
    import paged_kv_cache_465_amd as kvp
    if args.probe_calibration:
        r = stream_read_probe(kvp, dev, torch.cuda.get_device_properties(0).multi_processor_count)
        print(json.dumps({"probe_calibration": r}))
        return
    if args.config == "prefix_cache":
        print(json.dumps(prefix_cache_bench(kvp, dev)), flush=True)
        return
    from workloads import CONFIGS, EXTRA_CONFIGS, make_case
    cfg = {**CONFIGS, **EXTRA_CONFIGS}[args.config]
    case = make_case(cfg, with_data=not cfg.device_data)
    log(f"[config] {cfg.name}: layers={cfg.layers} B={case.B} Hq={cfg.num_q_heads} "
        f"Hkv={cfg.num_kv_heads} D={cfg.head_dim} P={cfg.page_size} {cfg.kv_dtype} "
        f"ctx[min,max]=[{int(case.ctx.min())},{int(case.ctx.max())}] pages={case.num_pages}")
    n_rows = int(case.q_start[-1])
    sb = step_bytes(cfg, case.ctx, n_rows)
    total = sb["kv"] + sb["q_out"] + sb["table"] + sb["append"]
    flops = step_flops(cfg, case.ctx, case.q_start)
    res, state = run_gpu(args, kvp, cfg, case)
    ms = res["ms_per_step"]
    kern_us = float(res["kernel_ms"].mean() * 1e3)
    achieved = sb["split_kernel_per_launch"] / (kern_us * 1e-6) / 1e9
    # the bound: arithmetic intensity of a launch against the bf16 matrix-core
    # ridge (2.5 PFLOP/s dense / 8 TB/s)
    flops_launch = flops / cfg.layers
    intensity = flops_launch / sb["split_kernel_per_launch"]
    mfma_bound = intensity > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if is_chunked(cfg):
        # bfloat16 pools with more than 32 rows per (sequence, KV head): the
        # LDS-staged kernel; otherwise the register-streaming one
        rows = int(np.diff(case.q_start).max()) * (cfg.num_q_heads // cfg.num_kv_heads)
        kernel_name = ("prefill_fa_kernel" if cfg.kv_dtype == "bf16" and rows > 32
                       else "prefill_mfma_kernel")
    elif res["plan"]["use_mfma"]:
        kernel_name = "decode_mfma_stream_kernel" if res["balanced"] else "decode_mfma_kernel"
    else:
        kernel_name = "decode_valu_kernel"
    if mfma_bound:
        tflops = flops_launch / (kern_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    out = {
        "metric": "paged decode attn: KV-read GB/s (% of HBM peak) + decode tokens/s, 1xMI355X",
        "value": round(total / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.kv_dtype + " KV, f32 accumulate",
        "data": "synthetic (seeded N(0,1), bf16-rounded; pages shuffled)",
        "config": {"workload": cfg.name, "layers": cfg.layers, "batch": case.B,
                   "context": int(case.ctx.max()) if cfg.ctx_fixed else
                   [int(case.ctx.min()), int(case.ctx.max())],
                   "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "page_size": cfg.page_size,
                   "kv_dtype": cfg.kv_dtype,
                   **({"plan": res["prefill_plan"]["plan"],
                       "order_entries": res["prefill_plan"].get("order_entries")}
                      if is_chunked(cfg) else
                      {"plan": "balanced", "num_bins": res["plan"]["num_bins"],
                       "num_merge": res["plan"]["num_merge"]} if res["balanced"]
                      else {"plan": "uniform", "num_splits": res["num_splits"]}),
                   **({"sink_tokens": cfg.sink_tokens, "window_tokens": cfg.window_tokens}
                      if cfg.window_tokens > 0 else {}),
                   "waves_per_group": res["plan"]["waves_per_group"]},
        "tokens_per_s": round(n_rows / (ms * 1e-3), 1),
        "flops_per_step": int(flops),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "hbm_frac": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "bytes_per_step": {k: int(v) for k, v in sb.items()},
        "roofline": {**roof, "traffic": None, "kernel": kernel_name,
                     "kernel_us_mean": round(kern_us, 2),
                     "timed": ("multi-query call (one kernel)" if is_chunked(cfg) else
                               "decode call (split kernel + merge kernel)"
                               if res["merge_launched"] else
                               "window decode call (split kernel, + merge when split)"
                               if cfg.window_tokens > 0 and not res["balanced"]
                               else "split kernel"),
                     "bytes_per_launch": int(sb["split_kernel_per_launch"]),
                     "flops_per_launch": int(flops_launch),
                     "intensity_flop_per_byte": round(intensity, 2),
                     "hbm_GBps": round(achieved, 1)},
    }
    rec = recorded_traffic(cfg.name, is_chunked(cfg))
    if rec is not None:
        out["roofline"]["traffic"] = rec["traffic_bytes_per_launch"]
        out["roofline"]["traffic_over_algorithmic"] = round(
            rec["traffic_bytes_per_launch"] / sb["split_kernel_per_launch"], 4)
        # the same record's cache and ALU counters for this kernel, when taken
        counters = {k: rec[k] for k in ("l2_hit_rate", "valu_busy_pct", "mfma_util_pct")
                    if k in rec}
        if counters:
            out["roofline"]["counters"] = counters
    out["copy_probe"] = copy_probe(dev)
    ceiling = stream_read_probe(kvp, dev, torch.cuda.get_device_properties(0).multi_processor_count)
    out["stream_read_ceiling"] = ceiling
    if roof["unit"] == "GB/s":
        out["roofline"]["frac_of_stream_ceiling"] = round(roof["achieved"] / ceiling["GBps"], 4)
    hc = None
    if not (args.no_parity and args.no_cpu_baseline):
        hc = host_layer(cfg, case, dev, 0)
    if not args.no_parity:
        # the first and the last layer of the timed run (inputs of a layer are
        # drawn from its own seed, so each is checked against its own oracle)
        checks = [parity_sample(cfg, hc, state, 0)]
        if cfg.layers > 1:
            checks.append(parity_sample(cfg, host_layer(cfg, case, dev, cfg.layers - 1), state,
                                        cfg.layers - 1))
        out["parity"] = {"layers": [c["layer"] for c in checks], "seqs": checks[0]["seqs"],
                         "max_abs": max(c["max_abs"] for c in checks),
                         "rel_l2": max(c["rel_l2"] for c in checks),
                         "ok": all(c["ok"] for c in checks), "per_layer": checks}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, hc, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def parity_sample(cfg, hc, state, layer=0, seqs=(0, 13, 31)):
    """One layer's output rows of the timed run for a few sequences against the oracle."""
    pool, layers, bt, ctx = state
    seqs = [s for s in seqs if s < hc.B]
    lay, pools = oracle_layer(cfg, hc, seqs)
    ref = oracle_decode(cfg, lay, hc, pools, seqs)
    got_bits = layers[layer].out.cpu().numpy().view(np.uint16)
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rows = np.concatenate([np.arange(hc.q_start[b], hc.q_start[b + 1]) for b in seqs])
    d = np.abs(got[rows] - ref[rows])
    rel = float(np.linalg.norm(got[rows] - ref[rows]) / np.linalg.norm(ref[rows]))
    r = {"layer": layer, "seqs": seqs, "max_abs": float(d.max()), "rel_l2": rel,
         "ok": bool(d.max() <= 1e-2 and rel <= 5e-3)}
    log(f"[parity] {r}")
    return r


if __name__ == "__main__":
    main()
