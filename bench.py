"""Paged decode attention benchmark on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama7b]

A step is one decode step of the whole batch on the device, inputs resident in
HBM: the copy-on-write block copies the step raised (prefix_sharing only), the
newest tokens' K/V stored into their slots, and decode attention over the block
tables (with context partitions and their log-sum-exp merge when the workload uses
them).  Where the attention launch can store the newest K/V (every kernel form but
the vector kernel's balanced split), the store rides in it (pa_decode_append /
pa_decode_fp8_append); otherwise (--unfused, or that balanced split) it is its own
launch (pa_reshape_and_cache).  Steps rotate over R replicas of
the batch in separate allocations, so no step finds the previous one's K/V in the
last-level cache.

Printed: one JSON line.  value = effective KV GB/s of the whole step
(sum_s ctx_s * 2 * H_kv * d * esz / step time), timed over K steps with nothing
but one event on each side; then the same K steps run again with events around
each step's parts for the decode call alone and its roofline against 8 TB/s.
Also: decode seqs/s, the same kernels on an identity (physically contiguous)
layout, the host allocator's cost per step, and the oracle's CPU time on the same
inputs.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # dense, MI355X
REPLICAS = 3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# Sources the vector decode kernels are built from (their counters go stale when these change).
DECODE_SOURCES = {
    "f16": ["decode_valu.h", "balanced.h", "kernel_common.h", "internal.h", "decode_valu_f16.hip"],
    "bf16": ["decode_valu.h", "balanced.h", "kernel_common.h", "internal.h", "decode_valu_bf16.hip"],
    "f32": ["decode_valu.h", "balanced.h", "kernel_common.h", "internal.h", "decode_valu_f32.hip"],
    "fp8": ["decode_valu.h", "balanced.h", "kernel_common.h", "internal.h", "decode_valu_fp8_f16.hip",
            "decode_valu_fp8_bf16.hip"],
    "mfma": ["decode_mfma.h", "balanced.h", "kernel_common.h", "internal.h", "decode_mfma_f16.hip",
             "decode_mfma_bf16.hip"],
}


def kernel_sources_digest(files) -> str:
    """sha256 over the named libpa sources (names and contents, in the given order)."""
    import hashlib
    d = os.path.join(ROOT, "paged_kv_cache_308_amd", "csrc")
    h = hashlib.sha256()
    for name in files:
        h.update(name.encode())
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or None
    when the kernels have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != kernel_sources_digest(rec.get("sources", [])):
        return None
    return rec["bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 100 untimed steps by default: after the GPU has been idle, the matrix-core-heavy
    # multi-query kernel runs up to 40% slower for about its first hundred calls while the
    # clocks settle (the decode kernels are steady from their first calls)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="llama7b")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--no-identity", action="store_true")
    ap.add_argument("--layout", choices=("paged", "identity"), default="paged",
                    help="physical placement of the timed batch: the allocator's seeded random free order "
                         "(paged), or every sequence on consecutive blocks (identity; for profiling the "
                         "contiguous comparison point)")
    ap.add_argument("--unfused", action="store_true",
                    help="store the newest tokens with their own launch even where the attention "
                         "launch can do it")
    ap.add_argument("--no-grouped", action="store_true",
                    help="batches of forked sequences: attend per sequence (pa_decode_append) instead of "
                         "reading each shared partition once per group (pa_decode_grouped)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the read-bandwidth probes (pa_stream_read over 4 GiB, pa_gather_read over the step's tiles)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--swap", type=int, default=0, metavar="N",
                    help="instead of decode: move N sequences' blocks to pinned host memory and "
                         "back (pa_swap_blocks) and report both directions' GB/s")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    return args


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, ctx: np.ndarray, unique_tokens: int = None) -> dict:
    """Bytes one decode call must move: K/V of every cached token, q in, out, the
    table entries it reads and the lengths (E4M3 pools: also the K and V scale of every
    (block, KV head) it reads).  kv / total count every sequence's tokens (the metric's
    effective bytes); *_unique count a block shared by several sequences once, the
    bytes that must come from HBM (the roofline's)."""
    per_tok = 2 * w.num_kv_heads * w.head_dim * w.kv_elem_bytes
    kv = int(ctx.astype(np.int64).sum()) * per_tok
    qo = 2 * w.num_seqs * w.num_q_heads * w.head_dim * w.elem_bytes
    blocks = int(np.sum((ctx.astype(np.int64) + w.block_size - 1) // w.block_size))
    tbl = 4 * blocks + 4 * w.num_seqs
    if w.kv == "fp8":
        tbl += 8 * blocks * w.num_kv_heads
    kv_u = kv if unique_tokens is None else unique_tokens * per_tok
    return {"kv": kv, "total": kv + qo + tbl, "kv_unique": kv_u, "total_unique": kv_u + qo + tbl}


def build_replicas(args, w, batch, identity: bool):
    import torch
    from paged_kv_cache_308_amd.replay import replay
    import workloads as W
    b = batch
    if identity:
        b = W.Batch(batch.workload, batch.lengths, np.arange(w.num_blocks, dtype=np.int32),
                    batch.script, batch.q, batch.append_k, batch.append_v)
    reps = []
    for r in range(REPLICAS):
        db = replay(b, poison=False)
        ws = db.cache.workspace(w.num_seqs, w.num_q_heads, db.max_context_len, args.P)
        src = torch.from_numpy(db.cow_src).cuda()
        dst = torch.from_numpy(db.cow_dst).cuda()
        out = torch.empty_like(db.query)
        if args.grouped:
            ws = db.grouped_workspace(args.P)
            db.group_args = db.groups(args.P)
        reps.append((db, ws, src, dst, out))
    torch.cuda.synchronize()
    return reps


def run_steps(args, reps, n_steps: int, record: bool, attend_only: bool = False, rewarm: int = 0):
    """Returns (total ms, per-step decode ms list, per-step pre-decode ms list).
    With record=False nothing but the two bracketing events touches the stream, so the
    total is the whole job's time; record=True adds events around each step's parts
    (for the decode-only figures), which themselves cost a few microseconds a step.
    attend_only: the decode calls alone, back to back (no copies, no separate scatter;
    both are idempotent here, so the pools hold the same data either way).
    rewarm: untimed steps of the same kind enqueued right before the first event, with no
    wait between them, so that the timed steps start in the state a steady run is in
    rather than after the host's pause."""
    import torch
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)] if record else None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for k in range(-rewarm, n_steps):
        if k == 0:
            t0.record(st)
        db, ws, src, dst, out = reps[k % len(reps)]
        if record and k >= 0:
            evs[k][0].record(st)
        if src.numel() and not attend_only:
            db.cache.copy(src, dst, st)
        if not args.fused and not attend_only:
            db.cache.write(db.new_key, db.new_value, db.slot_mapping, st)
        if record and k >= 0:
            evs[k][1].record(st)
        if args.grouped:  # shared partitions once per group, the newest tokens stored
            db.step_grouped(args.P, db.group_args, out=out, workspace=ws, stream=st, variant=args.variant)
        elif args.fused:  # the newest tokens' store rides in the attention launch
            db.step(args.P, args.variant, out=out, workspace=ws, stream=st)
        else:
            db.attend(args.P, args.variant, out=out, workspace=ws, stream=st)
        if record and k >= 0:
            evs[k][2].record(st)
    t1.record(st)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    if not record:
        return total, [], []
    dec = [a[1].elapsed_time(a[2]) for a in evs]
    pre = [a[0].elapsed_time(a[1]) for a in evs]
    return total, dec, pre


def host_alloc_cost(w, batch, steps: int = 50) -> float:
    """Microseconds per step for the host allocator to reserve every sequence's
    next slot (pa_alloc_append_slots over the batch): the median over `steps` steps, so
    that a pause of the host process does not count."""
    import paged_kv_cache_308_amd as pa
    a = pa.Allocator(w.num_blocks, w.block_size)
    a.set_free_order(batch.free_order)
    ids = {}
    for op in batch.script:
        if op.kind == "new":
            ids[op.seq] = a.new_seq()
        elif op.kind == "fork":
            ids[op.arg] = a.fork(ids[op.seq])
        else:
            a.append_slots([ids[op.seq]] * op.arg)
    seqs = [ids[s] for s in range(w.num_seqs)]
    times = []
    for _ in range(steps):
        t = time.perf_counter()
        a.append_slots(seqs)
        times.append(time.perf_counter() - t)
    return float(np.median(times)) * 1e6


def upload_cost(w, db, steps: int = 50) -> dict:
    """Host -> device upload of a step's index data (slots, block tables, context
    lengths) through engine.StepUploader: pinned staging, one asynchronous copy on the
    stream.  Microseconds from the host arrays to the data on the device (the call plus a
    stream synchronisation, PCIe included), median over `steps` uploads."""
    import torch
    from paged_kv_cache_308_amd.engine import StepUploader
    tb, cl = db.host_tables, db.host_context_lens
    sl = db.slot_mapping.cpu().numpy()
    up = StepUploader(tb.shape[0], tb.shape[1])
    st = torch.cuda.current_stream()
    times = []
    for k in range(steps + 3):
        torch.cuda.synchronize()
        t = time.perf_counter()
        up.upload(sl, tb, cl, st)
        st.synchronize()
        if k >= 3:
            times.append(time.perf_counter() - t)
    return {"us": round(float(np.median(times)) * 1e6, 2), "bytes": int(4 * (2 * tb.shape[0] + tb.size))}


def cpu_baseline(args, w, batch, kv_bytes: int) -> dict:
    """The oracle (binary64, one thread) on the same step, timed on this host."""
    from oracle import place
    import oracle
    p = place.place(batch, poison=False)
    o = oracle.default()
    p.write(p.new_key, p.new_value, p.slot_mapping, w.dtype)
    t = time.perf_counter()
    if w.kv == "fp8":
        o.decode_fp8(batch.q, p.key_cache, p.value_cache, p.k_scales, p.v_scales, p.block_tables,
                     p.context_lens, w.scale, w.dtype)
    else:
        o.decode(batch.q, p.key_cache, p.value_cache, p.block_tables, p.context_lens, w.scale,
                 w.dtype)
    dt = time.perf_counter() - t
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole {w.name} decode step ({w.num_seqs} sequences, all heads), "
                      f"oracle decode call only, {dt:.2f} s on one thread of {cpu}",
            "seconds": round(dt, 3), "seqs_per_s": round(w.num_seqs / dt, 3),
            "threads": cpu_baseline_threads(w, batch, p, o, kv_bytes)}


def cpu_baseline_threads(w, batch, p, o, kv_bytes: int) -> dict:
    """The same oracle call split over sequences on the host's cores (threads: the oracle
    is C behind ctypes, which releases the GIL; its decode keeps no shared state).
    Contiguous sequence ranges of about equal token counts, one per thread."""
    import concurrent.futures as cf
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    n = max(1, min(n, 16, w.num_seqs))
    ctx = np.maximum(np.asarray(p.context_lens, np.int64), 1)
    cuts = np.searchsorted(np.cumsum(ctx), np.arange(1, n) * ctx.sum() / n)
    bounds = [0, *[int(c) + 1 for c in cuts], w.num_seqs]
    ranges = [(a, b) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]

    def run(r):
        a, b = r
        if w.kv == "fp8":
            o.decode_fp8(batch.q[a:b], p.key_cache, p.value_cache, p.k_scales, p.v_scales,
                         p.block_tables[a:b], p.context_lens[a:b], w.scale, w.dtype)
        else:
            o.decode(batch.q[a:b], p.key_cache, p.value_cache, p.block_tables[a:b],
                     p.context_lens[a:b], w.scale, w.dtype)

    with cf.ThreadPoolExecutor(len(ranges)) as ex:
        t = time.perf_counter()
        list(ex.map(run, ranges))
        dt = time.perf_counter() - t
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": len(ranges),
            "seconds": round(dt, 3)}


def stream_read_gbs(nbytes: int = 4 << 30, reps: int = 5) -> float:
    """Achievable HBM read bandwidth: pa_stream_read over a buffer far beyond the caches,
    timed with events on the launch stream."""
    import torch
    from paged_kv_cache_308_amd import pa_stream_read
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    for _ in range(2):
        pa_stream_read(buf, sink, st)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(reps):
        pa_stream_read(buf, sink, st)
    b.record(st)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del buf, sink
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def gather_read_gbs(w, reps, n_runs: int = 5) -> dict:
    """Achievable read rate for the step's own access pattern: pa_gather_read over the
    (physical block, KV head) tiles of both pools that each replica's tables reach (a
    block shared by several sequences once; tiles above 4 KiB as 4 KiB pieces), the
    replicas in turn as the decode steps take them, timed with events on the launch
    stream."""
    import torch
    from paged_kv_cache_308_amd import pa_gather_read
    tile = w.block_size * w.head_dim * w.kv_elem_bytes
    piece = min(tile, 4096)
    lists, nbytes = [], []
    for db, *_ in reps:
        ctx = db.host_context_lens.astype(np.int64)
        used = [db.host_tables[s, :(int(c) + w.block_size - 1) // w.block_size] for s, c in enumerate(ctx)]
        ids = np.concatenate(used) if used else np.zeros(0, np.int32)
        _, first = np.unique(ids, return_index=True)
        blocks = ids[np.sort(first)].astype(np.int64)
        kc, vc = db.cache.key_cache, db.cache.value_cache
        off = ((blocks[:, None] * w.num_kv_heads + np.arange(w.num_kv_heads)[None, :]) * tile).reshape(-1)
        off = (off[:, None] + np.arange(0, tile, piece)[None, :]).reshape(-1)
        addrs = np.stack([kc.data_ptr() + off, vc.data_ptr() + off], axis=1).reshape(-1)
        assert off.max() + piece <= kc.numel() * kc.element_size()
        lists.append(torch.from_numpy(addrs.astype(np.int64)).cuda())
        nbytes.append(len(addrs) * piece)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    for i in range(2 * len(lists)):
        pa_gather_read(lists[i % len(lists)], piece, sink, st)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(st)
    for i in range(n_runs * len(lists)):
        pa_gather_read(lists[i % len(lists)], piece, sink, st)
    b.record(st)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (n_runs * len(lists))
    return {"gbs": float(np.mean(nbytes)) / (ms * 1e-3) / 1e9, "bytes": int(np.mean(nbytes)), "piece": piece,
            "us": ms * 1e3}


def swap_bench(args, w, batch) -> dict:
    """Block swap (preemption data mover): N sequences out to pinned host memory and back."""
    import torch
    from paged_kv_cache_308_amd import pa_swap_blocks
    from paged_kv_cache_308_amd.engine import HostKVPool
    from paged_kv_cache_308_amd.replay import replay
    db = replay(batch, poison=False)
    cache = db.cache
    n = min(args.swap, w.num_seqs)
    tables = [cache.alloc.block_table(db.seq_ids[s])[0] for s in range(n)]
    src = np.concatenate([np.asarray(t, np.int32) for t in tables])
    nblk = len(src)
    host = HostKVPool(nblk, w.num_kv_heads, w.head_dim, w.block_size, cache.dtype)
    dev_ids = torch.from_numpy(src).cuda()
    host_ids = torch.arange(nblk, dtype=torch.int32, device="cuda")
    nbytes = 2 * nblk * w.num_kv_heads * w.block_size * w.head_dim * w.kv_elem_bytes
    st = torch.cuda.current_stream()
    res = {}
    for name, (a, b, s_, d_) in {
            "out": ((cache.key_cache, cache.value_cache), (host.key_cache, host.value_cache), dev_ids, host_ids),
            "in": ((host.key_cache, host.value_cache), (cache.key_cache, cache.value_cache), host_ids, dev_ids)}.items():
        for _ in range(2):
            pa_swap_blocks(a[0], a[1], b[0], b[1], s_, d_, st)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(args.steps):
            pa_swap_blocks(a[0], a[1], b[0], b[1], s_, d_, st)
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        res[name] = {"ms": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 2)}
    return {"metric": "block swap GB/s (device <-> pinned host, pa_swap_blocks)",
            "value": res["out"]["GBps"], "unit": "GB/s", "higher_is_better": True,
            "n_gpus": 1, "steps": args.steps, "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": w.name, "sequences": n, "blocks": nblk, "bytes": nbytes},
            "swap_out": res["out"], "swap_in": res["in"]}


def mq_bench(args, w, batch) -> dict:
    """Chunked prefill: each sequence's last query_len tokens are written into the cache
    (pa_reshape_and_cache) and attend causally (pa_multi_query).  The roofline is the
    matrix cores': 4 * d * H_q flops per (query token, visible key)."""
    import torch
    import paged_kv_cache_308_amd as pa
    import workloads as W
    from paged_kv_cache_308_amd.engine import to_torch
    from paged_kv_cache_308_amd.replay import replay
    ctx = batch.lengths.context_lens.astype(np.int64)
    nq = np.minimum(ctx, w.query_len)
    qstart = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    T = int(qstart[-1])
    keys_seen = int(sum(int(((c - n + 1) + c) * n // 2) for c, n in zip(ctx, nq)))  # sum of pos + 1
    flops = 4 * w.head_dim * w.num_q_heads * keys_seen
    kv_bytes = int(ctx.sum()) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    reps = []
    for r in range(REPLICAS):
        db = replay(batch, poison=False)
        q = torch.cat([to_torch(W.chunk_queries(w, s, int(n)), w.dtype) for s, n in enumerate(nq)]).cuda()
        slots, ks, vs = [], [], []
        bt = db.host_tables
        appends = [op for op in batch.script if op.kind == "append"]
        for s, (c, n) in enumerate(zip(ctx, nq)):
            for p in range(int(c - n), int(c)):
                slots.append(int(bt[s, p // w.block_size]) * w.block_size + p % w.block_size)
            ks.append(batch.append_k[s][int(c - n):])
            vs.append(batch.append_v[s][int(c - n):])
        assert len(appends) == w.num_seqs
        reps.append((db, q, torch.empty_like(q), torch.tensor(slots, dtype=torch.int32, device="cuda"),
                     to_torch(np.concatenate(ks), w.dtype).cuda(), to_torch(np.concatenate(vs), w.dtype).cuda(),
                     torch.from_numpy(qstart).cuda()))
    st = torch.cuda.current_stream()

    def steps(n, record, attend_only=False, rewarm=0):
        """record=False: only the bracketing events (whole-job time); True: events
        around each step's scatter and attention as well.  attend_only: the attention
        calls alone, back to back (the scatter writes the same tokens every step).
        rewarm: untimed steps of the same kind enqueued right before the first event, with
        no wait between them (after an idle stretch the kernel needs about a hundred calls
        before its clocks settle)."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)] if record else None
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        for k in range(-rewarm, n):
            if k == 0:
                t0.record(st)
            db, q, out, sl, kk, vv, qs = reps[k % len(reps)]
            if record and k >= 0:
                evs[k][0].record(st)
            if not attend_only:
                pa.pa_reshape_and_cache(kk, vv, db.cache.key_cache, db.cache.value_cache, sl, st)
            if record and k >= 0:
                evs[k][1].record(st)
            pa.pa_multi_query(out, q, db.cache.key_cache, db.cache.value_cache, db.block_tables,
                              db.context_lens, qs, w.scale, w.query_len, st)
            if record and k >= 0:
                evs[k][2].record(st)
        t1.record(st)
        torch.cuda.synchronize()
        if not record:
            return t0.elapsed_time(t1), [], []
        return (t0.elapsed_time(t1), [e[1].elapsed_time(e[2]) for e in evs],
                [e[0].elapsed_time(e[1]) for e in evs])

    steps(args.warmup, False)
    total, _, _ = steps(args.steps, False)
    # the attention calls alone, K back to back between two events: the call's duration
    # free of the markers the per-part events put between launches
    att_total, _, _ = steps(args.steps, False, attend_only=True, rewarm=args.warmup)
    _, att, pre = steps(args.steps, True, rewarm=args.warmup)
    ms_step = total / args.steps
    att_ms = att_total / args.steps
    cpu = None
    if not args.no_cpu:
        # the oracle on one sequence's first 64 chunk rows' worth of work: the last 64
        # positions of sequence 0, all heads
        from oracle import place
        import oracle
        sub = W.make_batch(w, seqs=[0])
        p = place.place(sub, poison=False)
        p.write(p.new_key, p.new_value, p.slot_mapping, w.dtype)
        n0 = 64
        q0 = W.chunk_queries(w, 0, int(nq[0]))[-n0:]
        c0 = int(ctx[0])
        t = time.perf_counter()
        oracle.default().multi_query(q0, p.key_cache, p.value_cache, p.block_tables, p.context_lens,
                                     np.array([0, n0], np.int32), w.scale, w.dtype)
        dt = time.perf_counter() - t
        f0 = 4 * w.head_dim * w.num_q_heads * int((2 * c0 - n0 + 1) * n0 // 2)
        cpu = {"value": round(f0 / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
               "sample": f"sequence 0's last {n0} query tokens (context {c0}, all {w.num_q_heads} heads), "
                         f"oracle multi_query call, {dt:.2f} s on one thread"}
    tflops = flops / (att_ms * 1e-3) / 1e12
    return {"metric": "chunked prefill paged attention TFLOP/s (pa_multi_query)",
            "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic",
            "config": {"workload": w.name, "num_seqs": w.num_seqs, "query_tokens": T,
                       "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                       "head_dim": w.head_dim, "block_size": w.block_size,
                       "sum_context_lens": int(ctx.sum()), "flops_per_step": flops,
                       "kv_bytes_per_step": kv_bytes, "replicas": REPLICAS},
            "attention_us": round(att_ms * 1e3, 2),
            "attention_us_between_events": round(float(np.mean(att)) * 1e3, 2),
            "scatter_us": round(float(np.mean(pre)) * 1e3, 2),
            "kv_gbs": round(kv_bytes / (att_ms * 1e-3) / 1e9, 2),
            "roofline": {"bound": "mfma", "kernel": "multi_query_kernel", "achieved": round(tflops, 2),
                         "peak": MFMA_PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_PEAK_TFLOPS[w.dtype], 4), "flops_per_launch": flops,
                         "duration_us": round(att_ms * 1e3, 2),
                         "timing": "K attention calls back to back between two events (the scatter left out)",
                         "traffic": measured_traffic(w.name)},
            "cpu_baseline": cpu}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(sequences, KV heads and context partitions shard without communication; "
              "run one process per GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return
    import workloads as W
    import paged_kv_cache_308_amd as pa  # noqa: F401  (fails loudly without libpa.so)
    pa._lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = W.WORKLOADS[args.workload]
    args.P = w.partition_size if args.partition_size is None else args.partition_size
    # batches of forked sequences (shared prompts) take the grouped path by default
    args.grouped = (w.lengths == "prefix" and not args.no_grouped and args.P > 0 and w.kv != "fp8"
                    and w.num_q_heads == w.num_kv_heads and w.dtype in ("f16", "bf16"))
    log(args, f"[bench] {w.name}: generating inputs")
    batch = W.make_batch(w)
    ctx = batch.lengths.context_lens
    ab = algorithmic_bytes(w, ctx)
    if args.swap:
        print(json.dumps(swap_bench(args, w, batch)), flush=True)
        return
    if w.query_len:
        print(json.dumps(mq_bench(args, w, batch)), flush=True)
        return
    log(args, f"[bench] placing {REPLICAS} replicas")
    reps = build_replicas(args, w, batch, identity=args.layout == "identity")
    # tokens held in the pool (a block shared by several sequences counts once)
    ab = algorithmic_bytes(w, ctx, reps[0][0].cache.alloc.stats()["stored_tokens"])
    args.fused = args.grouped or (not args.unfused and
                                  reps[0][0].cache.fused_step_ok(w.num_q_heads, args.P, args.variant))
    if args.fused:  # the attention launch also stores the newest K/V into the pool
        newest = 2 * w.num_seqs * w.num_kv_heads * w.head_dim * w.kv_elem_bytes
        ab["total"] += newest
        ab["total_unique"] += newest

    log(args, f"[bench] warmup {args.warmup}")
    run_steps(args, reps, args.warmup, record=False)
    log(args, f"[bench] timing {args.steps} steps")
    total_ms, _, _ = run_steps(args, reps, args.steps, record=False)
    # the decode calls alone, K of them back to back between two events: the call's duration
    # free of the markers the per-part events put between launches
    att_ms, _, _ = run_steps(args, reps, args.steps, record=False, attend_only=True, rewarm=args.warmup)
    # the same steps again with events around each part: decode-only and scatter times
    _, dec_ms, pre_ms = run_steps(args, reps, args.steps, record=True, rewarm=args.warmup)
    ms_step = total_ms / args.steps
    dec_avg = float(np.mean(dec_ms))
    dec_time = att_ms / args.steps
    log(args, f"[bench] {ms_step * 1e3:.1f} us/step, decode {dec_avg * 1e3:.1f} us")
    gather = None if args.no_stream else gather_read_gbs(w, reps)
    upload = upload_cost(w, reps[0][0])

    ident = ident_gather = None
    if not args.no_identity and args.layout == "paged":
        del reps
        torch.cuda.empty_cache()
        reps_i = build_replicas(args, w, batch, identity=True)
        _, dec_i, _ = run_steps(args, reps_i, args.steps, record=True, rewarm=args.warmup)
        ident = float(np.mean(dec_i))
        # the same read probe over the identity layout's tiles: separates the memory
        # system's response to the address pattern from the kernel's
        ident_gather = None if args.no_stream else gather_read_gbs(w, reps_i)
        del reps_i
        torch.cuda.empty_cache()
        log(args, f"[bench] identity layout decode {ident * 1e3:.1f} us")

    alloc_us = host_alloc_cost(w, batch)
    stream = None if args.no_stream else stream_read_gbs()
    cpu = None if args.no_cpu else cpu_baseline(args, w, batch, ab["kv"])

    gbs = ab["kv"] / (ms_step * 1e-3) / 1e9
    achieved = ab["total_unique"] / (dec_time * 1e-3) / 1e9
    g = w.num_q_heads // w.num_kv_heads
    mfma = w.kv != "fp8" and (args.variant == 2 or (args.variant == 0 and g >= 2 and w.dtype != "f32"))
    if args.grouped:
        kernels = "decode_mfma_grouped_kernel (with the plan) + decode_valu_kernel"
    elif args.P < 0:
        kernels = ("decode_mfma_balanced_kernel" if mfma else "decode_balanced_kernel") + " + balanced_merge_kernel"
    else:
        kernels = ("decode_mfma_kernel" if mfma else "decode_valu_kernel") + (" + lse_merge_kernel" if args.P else "")
    line = {
        "metric": "paged decode attn: effective KV HBM GB/s (% of peak) and decode seqs/sec",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if w.kv == "fp8" else w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "kv_dtype": w.kv, "query_dtype": w.dtype,
                   "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "sum_context_lens": int(ctx.sum()), "max_context_len": int(ctx.max()),
                   "partition_size": args.P, "variant": args.variant, "layout": args.layout,
                   "kv_bytes_per_step": ab["kv"], "replicas": REPLICAS},
        # against the nominal peak on the bytes HBM must deliver: a block shared by several
        # sequences counts once (equal to value's bytes when nothing is shared)
        "pct_of_peak": round(100 * ab["kv_unique"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "pct_of_peak_bytes": "unique KV bytes per step" if ab["kv_unique"] != ab["kv"] else "KV bytes per step",
        "seqs_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "decode_us": round(dec_avg * 1e3, 2),
        "decode_us_p10_median_p90": [round(float(np.percentile(dec_ms, x)) * 1e3, 2) for x in (10, 50, 90)],
        "stream_read_gbs": None if stream is None else round(stream, 1),
        # the same unique bytes as pct_of_peak, against the measured streaming read
        "pct_of_stream_read": None if stream is None else round(
            100 * ab["kv_unique"] / (ms_step * 1e-3) / 1e9 / stream, 2),
        "gather_read_gbs": None if gather is None else round(gather["gbs"], 1),
        "gather_read": None if gather is None else {
            "bytes": gather["bytes"], "piece_bytes": gather["piece"], "us": round(gather["us"], 2),
            "what": "pa_gather_read over the (block, KV head) tiles of both pools the step's tables reach"},
        "pct_of_gather_read": None if gather is None else round(100 * achieved / gather["gbs"], 2),
        "mfma_util": round(4.0 * float(ctx.sum()) * w.num_q_heads * w.head_dim / (dec_avg * 1e-3) / 1e12 /
                           MFMA_PEAK_TFLOPS[w.dtype], 4) if mfma else None,
        "fused_store": args.fused,
        "grouped": args.grouped,
        "pre_decode_us": round(float(np.mean(pre_ms)) * 1e3, 2),
        "decode_kv_gbs": round(ab["kv"] / (dec_avg * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": kernels, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": ab["total_unique"],
                     "duration_us": round(dec_time * 1e3, 2),
                     "timing": "K decode calls back to back between two events (the step's copies and "
                               "separate scatter left out)",
                     "traffic": measured_traffic(w.name + ("_grouped" if args.grouped else ""))},
        "identity_decode_us": None if ident is None else round(ident * 1e3, 2),
        "paged_vs_identity": None if ident is None else round(ident / dec_avg, 4),
        "identity_gather_read_gbs": None if ident_gather is None else round(ident_gather["gbs"], 1),
        # physically consecutive blocks read the same bytes (counters) but more slowly, the
        # read probe as much as the kernel: the contiguous layout concentrates the concurrent
        # workgroups' reads on neighbouring addresses; against its own probe the kernel is as
        # close on either layout
        "identity_pct_of_gather_read": None if ident is None or ident_gather is None else
        round(100 * ab["total_unique"] / (ident * 1e-3) / 1e9 / ident_gather["gbs"], 2),
        "host_alloc_us_per_step": round(alloc_us, 2),
        "upload_us": upload["us"],
        "upload_bytes": upload["bytes"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
