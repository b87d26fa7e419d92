"""Several causal query tokens per sequence (pa_multi_query) against the oracle on the GPU.

Bar: max-abs 2e-2 (f16 / bf16 output, oracle in binary64), as for decode.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_308_amd as pa
from oracle_pins import MQCase
from paged_kv_cache_308_amd.engine import to_torch

pytestmark = pytest.mark.gpu
TOL = 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_mq(c: MQCase, max_query_len=None, tables=None, ctx=None, qstart=None):
    q = to_torch(c.mq, c.dtype).cuda()
    kc, vc = to_torch(c.kc, c.dtype).cuda(), to_torch(c.vc, c.dtype).cuda()
    bt = torch.from_numpy(c.tables if tables is None else tables).cuda()
    cl = torch.from_numpy(c.ctx if ctx is None else ctx).cuda()
    qs = torch.from_numpy(c.qstart if qstart is None else qstart).cuda()
    out = torch.full_like(q, 7.0)  # rows the call must not touch keep 7
    mql = max(c.qlens) if max_query_len is None else max_query_len
    pa.pa_multi_query(out, q, kc, vc, bt, cl, qs, c.scale, max(mql, 1))
    torch.cuda.synchronize()
    return out


SHAPES = [
    # lens, qlens, Hq, Hkv, d, B, dtype
    ([100, 37, 513, 16, 1, 300], [100, 5, 200, 16, 1, 33], 4, 4, 128, 16, "f16"),
    ([70, 300], [64, 17], 8, 2, 64, 32, "bf16"),
    ([129, 64, 1000], [40, 64, 3], 8, 1, 128, 16, "f16"),
    ([257, 90], [100, 90], 16, 2, 128, 128, "bf16"),
    ([600, 33], [31, 33], 32, 2, 64, 64, "f16"),
    ([45, 45, 200], [0, 45, 7], 16, 16, 128, 16, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"g{s[2] // s[3]}-d{s[4]}-B{s[5]}-{s[6]}")
def test_multi_query_matches_oracle(shape):
    lens, qlens, Hq, Hkv, d, B, dt = shape
    c = MQCase(np.random.default_rng(40), lens, qlens, Hq, Hkv, d, B, dt)
    want = c.run_mq(oracle.default())
    say(f"[gpu] multi_query {shape}")
    got = run_mq(c)
    err = float(np.max(np.abs(got.float().cpu().numpy().astype(np.float64) - want)))
    assert err <= TOL, (shape, err)
    # a chunk that starts the context: its first row sees only token 0
    g = Hq // Hkv
    for s, (n, nq) in enumerate(zip(c.lens, c.qlens)):
        if nq == n and nq > 0:
            row0 = got[int(c.qstart[s])].cpu()
            v0 = to_torch(c.v[s], dt)[0].repeat_interleave(g, dim=0)
            assert torch.equal(row0, v0)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_multi_query_rescales_when_a_row_max_grows(dt):
    """Scores with a wide spread (scale 8 / sqrt(d)): a row's running max keeps growing
    past the 2^8 margin of the kernel's reference max over later key tiles, so the
    rescaling of the accumulators runs mid-sequence, not only on the first tile."""
    lens, qlens = [1000, 700, 130], [300, 64, 130]
    c = MQCase(np.random.default_rng(45), lens, qlens, 8, 2, 128, 16, dt)
    c.scale = 8.0 / np.sqrt(128)
    want = c.run_mq(oracle.default())
    say(f"[gpu] multi_query wide scores {dt}")
    got = run_mq(c).float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL, err


def test_multi_query_with_one_token_per_sequence_is_decode():
    """n_s = 1 is a decode step: same result as pa_decode within the bar of each."""
    lens = [40, 513, 17, 1]
    c = MQCase(np.random.default_rng(41), lens, [1] * 4, 8, 2, 128, 16, "f16")
    got = run_mq(c).float().cpu().numpy()
    q = to_torch(c.mq, "f16").cuda()
    out = torch.empty_like(q)
    pa.pa_decode(out, q, to_torch(c.kc, "f16").cuda(), to_torch(c.vc, "f16").cuda(),
                 torch.from_numpy(c.tables).cuda(), torch.from_numpy(c.ctx).cuda(), c.scale)
    torch.cuda.synchronize()
    assert np.max(np.abs(got - out.float().cpu().numpy())) <= 2 * TOL
    want = c.run_mq(oracle.default())
    assert np.max(np.abs(got - want)) <= TOL


def test_multi_query_bad_inputs_give_nan_rows_of_that_sequence_only():
    lens, qlens = [60, 80, 50], [10, 20, 5]
    c = MQCase(np.random.default_rng(42), lens, qlens, 4, 4, 128, 16, "bf16")
    clean = run_mq(c)
    rows = [slice(int(c.qstart[s]), int(c.qstart[s + 1])) for s in range(3)]
    # a table entry outside the pool for a token the chunk sees
    t = c.tables.copy()
    t[1, 2] = c.num_blocks
    say("[gpu] multi_query bad entry")
    got = run_mq(c, tables=t)
    assert torch.isnan(got[rows[1]]).all()
    assert torch.equal(got[rows[0]], clean[rows[0]]) and torch.equal(got[rows[2]], clean[rows[2]])
    # more query tokens than context
    cl = c.ctx.copy()
    cl[2] = 3
    say("[gpu] multi_query n > ctx")
    got = run_mq(c, ctx=cl)
    assert torch.isnan(got[rows[2]]).all()
    assert torch.equal(got[rows[0]], clean[rows[0]]) and torch.equal(got[rows[1]], clean[rows[1]])


def test_multi_query_never_writes_outside_its_rows():
    """query_start past the output rows: those rows are skipped, the rest untouched."""
    lens, qlens = [30, 30], [8, 8]
    c = MQCase(np.random.default_rng(43), lens, qlens, 4, 4, 64, 16, "f16")
    qs = c.qstart.copy()
    qs[1] = 12  # sequence 0 claims rows 0..11 but only rows 0..15 exist; sequence 1 rows 12..15
    qs[2] = 20  # past T = 16
    say("[gpu] multi_query rows past T")
    got = run_mq(c, qstart=qs, max_query_len=12)
    assert got.shape[0] == 16 and not torch.isnan(got[:12]).any()


def test_chunked_prefill_step_through_the_cache():
    """A chunk's K/V go into the cache with pa_reshape_and_cache, then pa_multi_query
    reads them: the result equals the oracle on the same placement."""
    lens, qlens = [500, 260, 33], [128, 260, 16]
    c = MQCase(np.random.default_rng(44), lens, qlens, 8, 8, 128, 16, "f16")
    kc, vc = to_torch(c.kc, "f16").cuda(), to_torch(c.vc, "f16").cuda()
    # wipe the chunk tokens' slots, then write them back through the scatter
    slots, keys, vals = [], [], []
    for s, (n, nq) in enumerate(zip(lens, qlens)):
        for p in range(n - nq, n):
            slots.append(int(c.tables[s, p // c.B]) * c.B + p % c.B)
            keys.append(c.k[s][p])
            vals.append(c.v[s][p])
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    kv_flat = kc.view(-1, c.Hkv, c.B, c.d)
    for x in (kc, vc):
        x.view(c.num_blocks, c.Hkv, c.B, c.d)[sl // c.B, :, sl % c.B, :] = float("nan")
    pa.pa_reshape_and_cache(to_torch(np.stack(keys), "f16").cuda(), to_torch(np.stack(vals), "f16").cuda(),
                            kc, vc, sl)
    assert kv_flat.shape[0] == c.num_blocks
    q = to_torch(c.mq, "f16").cuda()
    out = torch.empty_like(q)
    say("[gpu] chunked prefill step")
    pa.pa_multi_query(out, q, kc, vc, torch.from_numpy(c.tables).cuda(), torch.from_numpy(c.ctx).cuda(),
                      torch.from_numpy(c.qstart).cuda(), c.scale, max(qlens))
    torch.cuda.synchronize()
    want = c.run_mq(oracle.default())
    assert np.max(np.abs(out.float().cpu().numpy() - want)) <= TOL


def test_multi_query_identity_and_relabelled_tables_are_bit_identical():
    """Where the blocks sit changes nothing ("PagedAttention" concept report §5): the same
    cache laid out in table order and under a random relabelling of the physical blocks
    gives bit-identical multi-query output (1 and 4 query heads per KV head)."""
    for Hq, Hkv, d, dt in ((4, 4, 128, "f16"), (8, 2, 64, "bf16")):
        c = MQCase(np.random.default_rng(71), [300, 37, 513, 16, 1], [300, 5, 200, 16, 1], Hq, Hkv, d, 16, dt)
        used = []
        for b in c.tables.reshape(-1):
            if b >= 0 and int(b) not in used:
                used.append(int(b))
        ident = np.full(c.num_blocks, -1, np.int64)
        ident[used] = np.arange(len(used))
        ident[ident < 0] = np.arange(len(used), c.num_blocks)
        outs = []
        for name, perm in (("paged", None), ("table order", ident),
                           ("relabelled", np.random.default_rng(72).permutation(c.num_blocks))):
            cc = c
            if perm is not None:
                cc = MQCase.__new__(MQCase)
                cc.__dict__.update(c.__dict__)
                t = c.tables.copy()
                t[t >= 0] = perm[t[t >= 0]]
                cc.tables = t
                for nm in ("kc", "vc"):
                    a = getattr(c, nm)
                    m = np.empty_like(a)
                    m[perm] = a
                    setattr(cc, nm, m)
            say(f"[gpu] multi_query layout {name} g={Hq // Hkv} d={d}")
            outs.append(run_mq(cc).cpu().contiguous().view(torch.uint8).numpy().tobytes())
        assert outs[0] == outs[1] == outs[2], (Hq, Hkv, d)


@pytest.mark.parametrize("S", [65, 100, 257, 300])
def test_multi_query_large_batches_around_the_sort_limits(S):
    """Batches past one wave's sort (64 sequences: the workgroup sorts through LDS) and
    past the workgroup's (256: sequences in index order), with 8 KV heads (each XCD's
    range of workgroups takes one head's sequences longest first) and 2 heads."""
    rng = np.random.default_rng(80 + S)
    lens = rng.integers(1, 60, S).tolist()
    qlens = [int(rng.integers(0, n + 1)) for n in lens]
    for Hq, Hkv in ((8, 8), (4, 2)):
        c = MQCase(rng, lens, qlens, Hq, Hkv, 64, 16, "f16")
        say(f"[gpu] multi_query S={S} Hq={Hq} Hkv={Hkv}")
        got = run_mq(c).double().cpu().numpy()
        want = c.run_mq(oracle.default())
        assert np.max(np.abs(got - want)) <= TOL, (S, Hq, Hkv)
