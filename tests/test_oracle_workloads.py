"""Oracle-side construction of workload batches (allocator replay, scatter, copies)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import place


def _logical(batch):
    """Per sequence: all its tokens' K and V in order (prompt, private, current)."""
    w = batch.workload
    ks = {s: [] for s in range(w.num_seqs)}
    vs = {s: [] for s in range(w.num_seqs)}
    appends = [op for op in batch.script if op.kind == "append"]
    group_prompt = {}
    for i, op in enumerate(appends):
        if w.lengths == "prefix" and op.seq % w.samples == 0 and op.seq not in group_prompt:
            group_prompt[op.seq] = i
            continue
        ks[op.seq].append(batch.append_k[i])
        vs[op.seq].append(batch.append_v[i])
    if w.lengths == "prefix":
        for s in range(w.num_seqs):
            i = group_prompt[(s // w.samples) * w.samples]
            ks[s].insert(0, batch.append_k[i])
            vs[s].insert(0, batch.append_v[i])
    return ({s: np.concatenate(v) for s, v in ks.items()},
            {s: np.concatenate(v) for s, v in vs.items()})


def _f64(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double()
    return torch.from_numpy(a.astype(np.float64))


def _sdpa(batch):
    w = batch.workload
    K, V = _logical(batch)
    out = np.zeros((w.num_seqs, w.num_q_heads, w.head_dim))
    for s in range(w.num_seqs):
        q = _f64(batch.q[s], w.dtype)[None, :, None, :]
        k = _f64(K[s], w.dtype).permute(1, 0, 2)[None].contiguous()
        v = _f64(V[s], w.dtype).permute(1, 0, 2)[None].contiguous()
        out[s] = F.scaled_dot_product_attention(
            q, k, v, scale=w.scale, enable_gqa=w.num_q_heads != w.num_kv_heads)[0, :, 0].numpy()
    return out


SMALL = {
    "tiny_fp32": W.WORKLOADS["tiny_fp32"],
    "prefix_small": W.scaled(W.WORKLOADS["prefix_sharing"], num_seqs=6, groups=2, samples=3,
                             prefix_base=20, private_max=6, block_size=4, num_blocks=64,
                             num_q_heads=4, num_kv_heads=2, head_dim=8),
    "gqa_small": W.scaled(W.WORKLOADS["llama70b_gqa"], num_seqs=3, low=100, high=300,
                          num_blocks=64, block_size=16, num_q_heads=16, num_kv_heads=2,
                          head_dim=16),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_step_equals_attention_over_logical_tokens(name):
    batch = W.make_batch(SMALL[name])
    out, p = place.decode_step(batch)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - _sdpa(batch))) <= 1e-12
    assert np.array_equal(p.context_lens, batch.lengths.context_lens)


def test_prefix_construction_raises_one_copy_per_extra_sample():
    w = SMALL["prefix_small"]
    batch = W.make_batch(w)
    p = place.place(batch)
    assert len(p.cow_src) == w.groups * (w.samples - 1)
    # every copy's source is its group's partly filled last prompt block
    for j in range(w.groups):
        srcs = set(p.cow_src[j * (w.samples - 1):(j + 1) * (w.samples - 1)].tolist())
        assert len(srcs) == 1
    st = p.alloc.stats()
    assert st["shared_blocks"] == w.groups * (int(batch.lengths.prefix_lens[0]) // w.block_size)


def test_identity_layout_gives_consecutive_blocks():
    w = W.WORKLOADS["tiny_fp32"]
    p = place.place(W.make_batch(w, identity=True))
    flat = [b for row in p.block_tables for b in row if b >= 0]
    assert flat == list(range(len(flat)))


def test_full_size_lengths_match_the_recipe():
    """The seeded draws of every workload (only the length step)."""
    sums = {n: int(W.draw_lengths(w)[0].context_lens.sum()) for n, w in W.WORKLOADS.items()}
    assert sums == {"tiny_fp32": 134, "llama7b": 46958, "llama13b_long": 95677,
                    "prefix_sharing": 93983, "llama70b_gqa": 191507, "llama7b_fp8": 46958,
                    "chunked_prefill": 34069}


def test_fp8_prefix_step_equals_attention_over_dequantised_tokens():
    """E4M3 pools with per-(block, head) scales, copy-on-write included: each token of
    each sequence stands for torch's E4M3 rounding of x / s times s, s the final scale
    of the block holding it (a copied block carries its source's scale)."""
    from oracle_pins import torch_fp8_encode, torch_fp8_values
    w = W.scaled(SMALL["prefix_small"], kv_dtype="fp8", dtype="f16")
    batch = W.make_batch(w)
    out, p = place.decode_step(batch)
    assert len(p.cow_src) > 0 and np.all(np.isfinite(out))
    vals = torch_fp8_values()
    K, V = _logical(batch)
    ref = np.zeros_like(out)
    g = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        n = int(p.context_lens[s])
        blocks = p.block_tables[s, np.arange(n) // w.block_size]
        kq = np.empty((n, w.num_kv_heads, w.head_dim))
        vq = np.empty_like(kq)
        for t in range(n):
            ks = p.k_scales[blocks[t]][:, None]
            vs = p.v_scales[blocks[t]][:, None]
            kx = (torch.from_numpy(K[s][t].astype(np.float32)) / torch.from_numpy(ks)).numpy()
            vx = (torch.from_numpy(V[s][t].astype(np.float32)) / torch.from_numpy(vs)).numpy()
            kq[t] = vals[torch_fp8_encode(kx)] * ks.astype(np.float64)
            vq[t] = vals[torch_fp8_encode(vx)] * vs.astype(np.float64)
        q = _f64(batch.q[s], w.dtype)[None, :, None, :]
        ref[s] = F.scaled_dot_product_attention(
            q, torch.from_numpy(kq).permute(1, 0, 2)[None].contiguous(),
            torch.from_numpy(vq).permute(1, 0, 2)[None].contiguous(), scale=w.scale,
            enable_gqa=g > 1)[0, :, 0].numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


# ------------------------------------------- the full-size tests' threaded oracle


@pytest.mark.parametrize("name,changes", [
    ("llama7b_fp8", dict(num_seqs=9, num_q_heads=8, num_kv_heads=8, num_blocks=1500)),
    ("prefix_sharing", dict(num_seqs=10, groups=2, samples=5, num_q_heads=4, num_kv_heads=4,
                            prefix_base=40, private_max=30, num_blocks=200)),
    ("llama70b_gqa", dict(num_seqs=5, num_q_heads=16, num_kv_heads=2, low=100, high=600,
                          block_size=16, num_blocks=300)),
])
def test_threaded_oracle_equals_plain_oracle(name, changes):
    """The full-size tests' oracle (its own compact pool, sequences split over threads)
    gives exactly the plain oracle step in the workload's own pool: the split changes no
    arithmetic and attention does not depend on where blocks sit (E4M3 scales travel
    with their tokens)."""
    import oracle_threads as OT
    w = W.scaled(W.WORKLOADS[name], **changes)
    batch = W.make_batch(w)
    want, _ = place.decode_step(batch)
    got = OT.decode_step(batch)
    assert np.array_equal(got, want)


def test_threaded_multi_query_rows_equal_the_whole_call():
    """Rows picked from a chunked-prefill batch through the threaded helper (runs cut into
    pieces whose context ends at the piece's last row) equal the same rows of one oracle
    call over the whole batch, bit for bit."""
    import oracle
    import oracle_threads as OT
    w = W.scaled(W.WORKLOADS["chunked_prefill"], num_seqs=3, num_q_heads=4, num_kv_heads=2,
                 low=80, high=200, query_len=70, num_blocks=64)
    batch = W.make_batch(w)
    ctx = batch.lengths.context_lens.astype(np.int64)
    nq = np.minimum(ctx, w.query_len)
    qstart = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qrows = [W.chunk_queries(w, s, int(n)) for s, n in enumerate(nq)]
    p = OT.compact_place(batch)
    p.write(p.new_key, p.new_value, p.slot_mapping, w.dtype)
    whole = oracle.default().multi_query(np.concatenate(qrows), p.key_cache, p.value_cache, p.block_tables,
                                         p.context_lens, qstart, w.scale, w.dtype)
    picks = [OT.RowPick(0, np.arange(int(nq[0]))), OT.RowPick(1, np.array([0, 1, 5, 6, 7, 40, int(nq[1]) - 1])),
             OT.RowPick(2, np.array([3]))]
    got = OT.multi_query_rows(picks, qrows, p, w, nq)
    for pk, g in zip(picks, got):
        assert np.array_equal(g, whole[qstart[pk.seq] + pk.rows])
