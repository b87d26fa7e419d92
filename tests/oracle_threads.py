"""The oracle's decode and multi-query calls split over host threads (TEST INFRASTRUCTURE).

Sequences are independent in attention, so cutting a batch into sequence ranges, or a
sequence's query rows into row ranges, and calling the oracle on each piece changes no
arithmetic; the oracle is C behind ctypes, which releases the GIL.  Used by the
full-size parity tests, whose batches take the single-threaded oracle minutes.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
from typing import List, Tuple

import numpy as np

import oracle
import workloads as W
from oracle import place


def host_threads(cap: int = 16) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, cap))


def _ranges(weights: np.ndarray, n: int) -> List[Tuple[int, int]]:
    """Contiguous index ranges of about equal total weight, at most n of them."""
    w = np.maximum(np.asarray(weights, np.float64), 1.0)
    cuts = np.searchsorted(np.cumsum(w), np.arange(1, n) * w.sum() / n)
    bounds = sorted({0, *[int(c) + 1 for c in cuts], len(w)})
    return [(a, b) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]


def decode(q, p: place.Placed, w: W.Workload) -> np.ndarray:
    """oracle decode (or decode_fp8) of every sequence of a placed batch, float64."""
    o = oracle.default()
    S = q.shape[0]
    ranges = _ranges(p.context_lens, host_threads())

    def run(r):
        a, b = r
        if p.k_scales is not None:
            return o.decode_fp8(q[a:b], p.key_cache, p.value_cache, p.k_scales, p.v_scales,
                                p.block_tables[a:b], p.context_lens[a:b], w.scale, w.dtype)
        return o.decode(q[a:b], p.key_cache, p.value_cache, p.block_tables[a:b], p.context_lens[a:b],
                        w.scale, w.dtype)

    with cf.ThreadPoolExecutor(len(ranges)) as ex:
        parts = list(ex.map(run, ranges))
    out = np.concatenate(parts) if parts else np.zeros((0,) + q.shape[1:])
    assert out.shape[0] == S
    return out


def compact_place(batch: W.Batch, seed: int = 7) -> place.Placed:
    """The oracle's own placement of a whole batch in a pool just large enough for it
    (sum over sequences of ceil(ctx / B) blocks plus one, handed out in a seeded random
    order), with every token but the newest ones placed.  Attention does not depend on
    where blocks sit, so the oracle need not mirror the device pool's 40,000-block size.
    E4M3 pools: each compact block takes the scale of the block that holds the same
    tokens in the workload's own pool (found by the model allocator's replay of the
    full batch)."""
    w = batch.workload
    ctx = batch.lengths.context_lens.astype(np.int64)
    nb = int(((ctx + w.block_size - 1) // w.block_size).sum()) + 1
    wc = dataclasses.replace(w, num_blocks=nb)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    b2 = W.Batch(wc, batch.lengths, order, batch.script, batch.q, batch.append_k, batch.append_v)
    scales = None
    if w.kv == "fp8":
        ks_full, vs_full = W.fp8_scales(w)
        a_full, sids, _, _ = place.replay(batch)
        a_c, sids_c, _, _ = place.replay(b2)
        ks = np.ones((nb, w.num_kv_heads), np.float32)
        vs = np.ones_like(ks)
        for s in range(w.num_seqs):
            full_t, _ = a_full.block_table(sids[s])
            c_t, _ = a_c.block_table(sids_c[s])
            for fb, cb in zip(full_t, c_t):
                ks[cb] = ks_full[fb]
                vs[cb] = vs_full[fb]
        scales = (ks, vs)
    return place.place(b2, poison=True, fp8_scales=scales)


def decode_step(batch: W.Batch) -> np.ndarray:
    """The oracle's decode step of a whole batch (newest tokens stored, then attention
    over every sequence) in its compact pool, on host threads."""
    p = compact_place(batch)
    p.write(p.new_key, p.new_value, p.slot_mapping, batch.workload.dtype)
    return decode(batch.q, p, batch.workload)


@dataclasses.dataclass
class RowPick:
    """Query rows of one sequence to check: row indices (into its n rows) in order."""
    seq: int
    rows: np.ndarray


def multi_query_rows(picks: List[RowPick], query_rows: List[np.ndarray], p: place.Placed,
                     w: W.Workload, n_rows: np.ndarray) -> List[np.ndarray]:
    """oracle multi_query for chosen query rows: row i of sequence s (n_s rows, context
    ctx_s) sits at position ctx_s - n_s + i and attends to t <= that position.  Runs of
    consecutive rows go to the oracle as one piece (a context cut just after the run's
    last row, the run as its query rows); pieces are spread over host threads.  Returns
    float64 [len(rows)][H_q][d] per pick."""
    o = oracle.default()
    pieces = []  # (pick index, first row, last row + 1)
    for k, pk in enumerate(picks):
        r = np.asarray(pk.rows, np.int64)
        if len(r) == 0:
            continue
        brk = np.nonzero(np.diff(r) != 1)[0] + 1
        for run in np.split(r, brk):
            pieces.append((k, int(run[0]), int(run[-1]) + 1))
    # cut long runs (32 rows at most) so the work spreads over the threads
    nthr = host_threads()
    out_pieces = []
    for k, a, b in pieces:
        for x in range(a, b, 32):
            out_pieces.append((k, x, min(b, x + 32)))
    ctx = p.context_lens.astype(np.int64)

    def cost(pc):
        k, a, b = pc
        s = picks[k].seq
        return (b - a) * (ctx[s] - n_rows[s] + b)

    order = sorted(range(len(out_pieces)), key=lambda i: -cost(out_pieces[i]))

    def run(i):
        k, a, b = out_pieces[i]
        s = picks[k].seq
        c = int(ctx[s] - n_rows[s] + b)  # the context ends with the run's last row
        q = np.ascontiguousarray(query_rows[s][a:b])
        return o.multi_query(q, p.key_cache, p.value_cache, p.block_tables[s:s + 1],
                             np.array([c], np.int32), np.array([0, b - a], np.int32), w.scale, w.dtype)

    with cf.ThreadPoolExecutor(nthr) as ex:
        res = dict(zip(order, ex.map(run, order)))
    outs = [[] for _ in picks]
    for i, (k, a, b) in enumerate(out_pieces):
        outs[k].append(res[i])
    return [np.concatenate(x) if x else np.zeros((0, w.num_q_heads, w.head_dim)) for x in outs]
