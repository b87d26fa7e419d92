"""Full-size workloads on the GPU in the benchmark's launch setup, against the oracle.

Every sequence of every full-size decode batch is compared with the oracle (in its own
compact pool: attention does not depend on where blocks sit), at each kernel form the
batch can take: the benchmark's own setting first.  The chunked-prefill batch compares
all 512 query rows of its 4 longest sequences and 16 rows of every other sequence.
Bars: max-abs 2e-2 for f16 / bf16 output (E4M3 pools included), the oracle in binary64.
Each check's largest error is listed at the end of the run.
"""
import sys

import numpy as np
import pytest
import torch

import oracle_threads as OT
import paged_kv_cache_308_amd as pa
import workloads as W
from paged_kv_cache_308_amd.engine import to_torch
from paged_kv_cache_308_amd.replay import replay

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
AUTO = pa.PA_VARIANT_AUTO
BAL = pa.PA_PARTITION_BALANCED


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


# partition settings per workload: the benchmark's first, then the other kernel forms
FULL_SIZE = {
    "llama7b": [0, 512, BAL],
    "llama13b_long": [512, BAL, 0],
    "llama70b_gqa": [BAL, 0, 512],
    "prefix_sharing": [512, 0],
    "llama7b_fp8": [0, 512, BAL],
}


@pytest.mark.parametrize("name", list(FULL_SIZE))
def test_full_size_every_sequence(name, margin):
    """The whole batch on the GPU (newest tokens stored, then attention: one launch where
    the kernel form allows) against the oracle's decode step of the same batch, every
    sequence and head."""
    w = W.WORKLOADS[name]
    say(f"[gpu] full-size {name}: generating")
    batch = W.make_batch(w)
    say(f"[gpu] full-size {name}: oracle on {OT.host_threads()} threads")
    want = OT.decode_step(batch)
    db = replay(batch)
    if w.lengths == "prefix":
        assert len(db.cow_src) == 64
    for P in FULL_SIZE[name]:
        say(f"[gpu] full-size {name}: step P={P}")
        got = f64(db.step(partition_size=P, variant=AUTO))
        torch.cuda.synchronize()
        assert got.shape == want.shape and np.all(np.isfinite(got)), (name, P)
        err = float(np.max(np.abs(got - want)))
        worst = int(np.argmax(np.max(np.abs(got - want), axis=(1, 2))))
        margin(f"{name} P={P} all {w.num_seqs} seqs", err, TOL[w.dtype])
        assert err <= TOL[w.dtype], (name, P, err, worst)


def test_full_size_prefix_sharing_grouped(margin):
    """The prefix-sharing workload through pa_decode_grouped, as the benchmark runs it:
    16 groups of 5 forks, each sharing its prompt's two whole 512-token partitions;
    all 80 sequences against the oracle."""
    w = W.WORKLOADS["prefix_sharing"]
    say("[gpu] full-size prefix_sharing grouped: generating")
    batch = W.make_batch(w)
    want = OT.decode_step(batch)
    db = replay(batch)
    groups = db.groups(w.partition_size)
    gs, gp, gmax, pmax = groups
    assert gs.tolist() == list(range(0, 81, 5)) and gp.tolist() == [2] * 16 and gmax == 5 and pmax == 2
    say("[gpu] full-size prefix_sharing grouped: step")
    got = f64(db.step_grouped(w.partition_size, groups, workspace=db.grouped_workspace(w.partition_size)))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    margin("prefix_sharing grouped all 80 seqs", err, TOL[w.dtype])
    assert err <= TOL[w.dtype]


def test_full_size_chunked_prefill(margin):
    """The chunked-prefill batch as the benchmark runs it (16 sequences, contexts 1,406 to
    3,047, each ending in a 512-token chunk: the chunk's K/V scattered, then
    pa_multi_query over the whole batch).  Oracle: every row of the 4 longest sequences
    (2,048 rows) and, of each other sequence, its first 4 and last 4 rows and 8 seeded
    rows between."""
    w = W.WORKLOADS["chunked_prefill"]
    say("[gpu] full-size chunked_prefill: generating")
    batch = W.make_batch(w)
    ctx = batch.lengths.context_lens.astype(np.int64)
    nq = np.minimum(ctx, w.query_len)
    qstart = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qrows = [W.chunk_queries(w, s, int(n)) for s, n in enumerate(nq)]

    # the GPU side, as the benchmark: replay, scatter the chunks, attend
    db = replay(batch)
    slots, ks, vs = [], [], []
    bt = db.host_tables
    for s, (c, n) in enumerate(zip(ctx, nq)):
        for p in range(int(c - n), int(c)):
            slots.append(int(bt[s, p // w.block_size]) * w.block_size + p % w.block_size)
        ks.append(batch.append_k[s][int(c - n):])
        vs.append(batch.append_v[s][int(c - n):])
    q = torch.cat([to_torch(x, w.dtype) for x in qrows]).cuda()
    out = torch.empty_like(q)
    pa.pa_reshape_and_cache(to_torch(np.concatenate(ks), w.dtype).cuda(),
                            to_torch(np.concatenate(vs), w.dtype).cuda(), db.cache.key_cache,
                            db.cache.value_cache, torch.tensor(slots, dtype=torch.int32, device="cuda"))
    say("[gpu] full-size chunked_prefill: pa_multi_query")
    pa.pa_multi_query(out, q, db.cache.key_cache, db.cache.value_cache, db.block_tables, db.context_lens,
                      torch.from_numpy(qstart).cuda(), w.scale, w.query_len)
    torch.cuda.synchronize()
    got = f64(out)
    assert np.all(np.isfinite(got))

    # the oracle: its own placement of every token (the chunks included)
    p = OT.compact_place(batch)
    p.write(p.new_key, p.new_value, p.slot_mapping, w.dtype)
    longest = set(np.argsort(-ctx, kind="stable")[:4].tolist())
    rng = np.random.default_rng(2024)
    picks = []
    for s in range(w.num_seqs):
        n = int(nq[s])
        if s in longest:
            rows = np.arange(n)
        else:
            mid = rng.choice(np.arange(4, n - 4), size=8, replace=False)
            rows = np.unique(np.concatenate([np.arange(4), np.arange(n - 4, n), mid]))
        picks.append(OT.RowPick(s, rows))
    say(f"[gpu] full-size chunked_prefill: oracle on {sum(len(x.rows) for x in picks)} rows, "
        f"{OT.host_threads()} threads")
    wants = OT.multi_query_rows(picks, qrows, p, w, nq)
    err = 0.0
    for pk, want in zip(picks, wants):
        g = got[qstart[pk.seq] + pk.rows]
        err = max(err, float(np.max(np.abs(g - want))))
    margin(f"chunked_prefill {sum(len(x.rows) for x in picks)} rows", err, TOL[w.dtype])
    assert err <= TOL[w.dtype]
