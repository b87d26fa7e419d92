"""HIP path against the oracle on the GPU (through the C ABI).

Bars: bitwise for the block operations and the pools they write; max-abs 1e-5 for
fp32 attention and 2e-2 for fp16 / bf16 attention (output rounded to the storage
type, oracle in binary64, unrounded).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_308_amd as pa
import workloads as W
from oracle import place
from oracle_pins import Case, Fp8Case, torch_fp8_values
from paged_kv_cache_308_amd.engine import TORCH_DTYPE, to_torch
from paged_kv_cache_308_amd.replay import replay

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
VALU, MFMA, AUTO = pa.PA_VARIANT_VALU, pa.PA_VARIANT_MFMA, pa.PA_VARIANT_AUTO
BAL = pa.PA_PARTITION_BALANCED


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> bytes:
    return t.cpu().contiguous().view(torch.uint8).numpy().tobytes()


def np_bits(a: np.ndarray) -> bytes:
    return np.ascontiguousarray(a).tobytes()


HAVE_MFMA = True


def variants(Hq, Hkv, dtype, P=0):
    vs = [VALU]
    if HAVE_MFMA and Hq // Hkv >= 2 and dtype != "f32":
        vs.append(MFMA)
    return vs


def variants_for(w, P=0):
    if w.kv == "fp8":  # E4M3 pools run on the vector kernel
        return [VALU, AUTO]
    return variants(w.num_q_heads, w.num_kv_heads, w.dtype, P)


# ----------------------------------------------------------- small workloads

SMALL = {
    "tiny_fp32": W.WORKLOADS["tiny_fp32"],
    "mha_f16": W.scaled(W.WORKLOADS["llama7b"], num_seqs=8, num_q_heads=8, num_kv_heads=8,
                        num_blocks=1200, partition_size=128),
    "long_bf16": W.scaled(W.WORKLOADS["llama13b_long"], num_seqs=4, num_q_heads=8, num_kv_heads=8,
                          low=600, high=1100, num_blocks=400, partition_size=256),
    "prefix_f16": W.scaled(W.WORKLOADS["prefix_sharing"], num_seqs=10, groups=2, samples=5,
                           num_q_heads=8, num_kv_heads=8, prefix_base=64, private_max=40,
                           num_blocks=256, partition_size=64),
    "gqa_bf16": W.scaled(W.WORKLOADS["llama70b_gqa"], num_seqs=3, num_q_heads=16, num_kv_heads=2,
                         low=300, high=700, num_blocks=64, partition_size=256),
    "gqa_f16_b16": W.scaled(W.WORKLOADS["llama70b_gqa"], num_seqs=3, num_q_heads=8,
                            num_kv_heads=2, low=100, high=300, num_blocks=128, block_size=16,
                            dtype="f16", partition_size=64),
    "f16_d64_b32": W.scaled(W.WORKLOADS["llama7b"], num_seqs=5, num_q_heads=4, num_kv_heads=4,
                            head_dim=64, block_size=32, num_blocks=300, partition_size=64),
    "f32_d128_b64_g4": W.scaled(W.WORKLOADS["llama70b_gqa"], num_seqs=3, num_q_heads=8,
                                num_kv_heads=2, low=50, high=200, num_blocks=32, block_size=64,
                                dtype="f32", partition_size=128),
    "bf16_d64_b128_g16": W.scaled(W.WORKLOADS["llama70b_gqa"], num_seqs=2, num_q_heads=16,
                                  num_kv_heads=1, head_dim=64, low=200, high=400, num_blocks=16,
                                  partition_size=256),
    # E4M3 pools with per-(block, KV head) scales
    "fp8_mha_f16": W.scaled(W.WORKLOADS["llama7b_fp8"], num_seqs=8, num_q_heads=8, num_kv_heads=8,
                            num_blocks=1200, partition_size=128),
    "fp8_prefix_bf16": W.scaled(W.WORKLOADS["prefix_sharing"], num_seqs=10, groups=2, samples=5,
                                num_q_heads=8, num_kv_heads=8, prefix_base=64, private_max=40,
                                num_blocks=256, partition_size=64, dtype="bf16", kv_dtype="fp8"),
    "fp8_gqa4_bf16": W.scaled(W.WORKLOADS["llama70b_gqa"], num_seqs=3, num_q_heads=16,
                              num_kv_heads=4, low=300, high=700, num_blocks=96, block_size=16,
                              partition_size=256, kv_dtype="fp8"),
    "fp8_d64_g8_f16": W.scaled(W.WORKLOADS["llama70b_gqa"], num_seqs=3, num_q_heads=16,
                               num_kv_heads=2, head_dim=64, low=100, high=300, num_blocks=64,
                               block_size=32, dtype="f16", partition_size=64, kv_dtype="fp8"),
    "fp8_d64_g2_f16": W.scaled(W.WORKLOADS["llama7b_fp8"], num_seqs=5, num_q_heads=8,
                               num_kv_heads=4, head_dim=64, num_blocks=300, partition_size=64),
}


@pytest.fixture(scope="module")
def oracle_steps():
    cache = {}

    def get(name):
        if name not in cache:
            batch = W.make_batch(SMALL[name])
            out, p = place.decode_step(batch)
            cache[name] = (batch, out, p)
        return cache[name]
    return get


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_workload(name, oracle_steps):
    w = SMALL[name]
    batch, want, placed = oracle_steps(name)
    for P in sorted({0, w.partition_size, BAL}):
        for v in variants_for(w, P):
            say(f"[gpu] small {name} P={P} variant={v}")
            db = replay(batch)
            assert np.array_equal(db.host_tables, placed.block_tables)
            assert np.array_equal(db.cow_src, placed.cow_src)
            assert np.array_equal(db.cow_dst, placed.cow_dst)
            got = db.step(partition_size=P, variant=v)
            torch.cuda.synchronize()
            err = np.max(np.abs(f64(got) - want))
            assert err <= TOL[w.dtype], (name, P, v, err)
            # the pools after the step: bit for bit what the oracle's scatter/copy wrote
            assert bits(db.cache.key_cache) == np_bits(placed.key_cache)
            assert bits(db.cache.value_cache) == np_bits(placed.value_cache)
            if w.kv == "fp8":  # copied blocks took their scales along
                assert bits(db.cache.k_scales) == np_bits(placed.k_scales)
                assert bits(db.cache.v_scales) == np_bits(placed.v_scales)


@pytest.mark.parametrize("name", ["mha_f16", "long_bf16", "prefix_f16", "tiny_fp32", "gqa_f16_b16",
                                  "gqa_bf16", "bf16_d64_b128_g16", "fp8_mha_f16", "fp8_gqa4_bf16",
                                  "fp8_d64_g8_f16"])
def test_fused_step_matches_scatter_then_decode(name, oracle_steps):
    """The newest-token store inside the attention launch: the pools afterwards are
    bit-identical to the separate scatter's, the output matches the oracle."""
    w = SMALL[name]
    batch, want, placed = oracle_steps(name)
    mfma = w.kv != "fp8" and w.dtype != "f32" and w.num_q_heads > w.num_kv_heads
    runs = [(P, VALU) for P in sorted({0, w.partition_size})]
    if mfma:  # the matrix-core kernels: one pass, partitions, balanced split
        runs += [(P, MFMA) for P in sorted({0, w.partition_size, BAL})]
    for P, v in runs:
        say(f"[gpu] fused step {name} P={P} variant={v}")
        db = replay(batch)
        got = db.step(partition_size=P, variant=v, fused=True)
        torch.cuda.synchronize()
        assert np.max(np.abs(f64(got) - want)) <= TOL[w.dtype], (name, P, v)
        assert bits(db.cache.key_cache) == np_bits(placed.key_cache)
        assert bits(db.cache.value_cache) == np_bits(placed.value_cache)
        ref = replay(batch)
        two = ref.step(partition_size=P, variant=v, fused=False)
        torch.cuda.synchronize()
        assert np.max(np.abs(f64(got) - f64(two))) <= TOL[w.dtype]


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_fused_step_edge_lengths(kernel):
    """Contexts of 1 (the newest token alone), partition starts and ends, block edges."""
    rng = np.random.default_rng(31)
    lens = [1, 2, 16, 17, 31, 32, 33, 64, 65, 128, 129, 511, 512, 513]
    Hq, Hkv, v, Ps = (4, 4, VALU, (0, 64)) if kernel == "valu" else (8, 2, MFMA, (0, 64, BAL))
    c = Case(rng, lens, Hq, Hkv, 128, 16, "f16")
    want = c.run(oracle.default())
    q, kc, vc, bt, cl = _upload_case(c)
    # the newest token of each sequence, taken from the placed pools, then poisoned there
    S = len(lens)
    nk = torch.empty((S, c.Hkv, c.d), dtype=kc.dtype, device="cuda")
    nv = torch.empty_like(nk)
    for s_, n in enumerate(lens):
        b, o = int(c.tables[s_, (n - 1) // c.B]), (n - 1) % c.B
        nk[s_] = kc[b, :, o, :]
        nv[s_] = vc[b, :, o, :]
        kc[b, :, o, :] = float("nan")
        vc[b, :, o, :] = float("nan")
    for P in Ps:
        out = torch.empty_like(q)
        ws = None
        if P:
            ws = torch.empty(pa.pa_decode_workspace_bytes(S, Hq, Hkv, 128, max(lens), P), dtype=torch.uint8,
                             device="cuda")
        say(f"[gpu] fused edge {kernel} P={P}")
        pa.pa_decode_append(out, q, nk, nv, kc, vc, bt, cl, c.scale, max_context_len=max(lens),
                            partition_size=P, variant=v, workspace=ws)
        torch.cuda.synchronize()
        assert np.max(np.abs(f64(out) - want)) <= TOL["f16"], P
        assert bits(kc) == np_bits(c.kc) and bits(vc) == np_bits(c.vc)
        # one token: exactly its V
        g = Hq // Hkv
        assert bits(out[0]) == bits(nv[0].repeat_interleave(g, dim=0))


# ----------------------------------------------------------------- edge cases


def _upload_case(c: Case):
    dt = TORCH_DTYPE[c.dtype]
    dev = lambda a: to_torch(a, c.dtype).cuda()
    q = dev(c.q)
    kc, vc = dev(c.kc), dev(c.vc)
    bt = torch.from_numpy(c.tables).cuda()
    cl = torch.from_numpy(c.ctx).cuda()
    assert kc.dtype == dt
    return q, kc, vc, bt, cl


def _run_case(c: Case, P, variant, max_ctx=None, tables=None):
    q, kc, vc, bt, cl = _upload_case(c)
    if tables is not None:
        bt = torch.from_numpy(tables).cuda()
    out = torch.empty_like(q)
    mc = int(c.ctx.max()) if max_ctx is None else max_ctx
    ws = None
    if P:
        n = pa.pa_decode_workspace_bytes(q.shape[0], q.shape[1], c.Hkv, c.d, mc, P)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    pa.pa_decode(out, q, kc, vc, bt, cl, c.scale, max_context_len=mc, partition_size=P,
                 variant=variant, workspace=ws)
    torch.cuda.synchronize()
    return out


EDGE_LENS = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1000]

EDGE_SHAPES = [
    # Hq, Hkv, d, B, dtype
    (4, 4, 128, 16, "f16"),
    (4, 4, 64, 16, "f32"),
    (8, 1, 128, 16, "bf16"),
    (8, 2, 64, 32, "f16"),
    (16, 16, 128, 128, "bf16"),
    (32, 2, 128, 64, "bf16"),
    (4, 2, 128, 16, "f32"),
]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_edge_lengths(shape):
    Hq, Hkv, d, B, dt = shape
    rng = np.random.default_rng(7)
    c = Case(rng, EDGE_LENS, Hq, Hkv, d, B, dt)
    want = c.run(oracle.default())
    for P in (0, 64, 512, BAL) if B <= 64 else (0, 128, 512, BAL):
        for v in variants(Hq, Hkv, dt, P):
            say(f"[gpu] edge {shape} P={P} variant={v}")
            got = _run_case(c, P, v)
            err = np.max(np.abs(f64(got) - want))
            assert err <= TOL[dt], (shape, P, v, err)
            assert torch.all(got[0] == 0)  # empty context
            # one token: exactly that token's V
            g = Hq // Hkv
            v1 = to_torch(c.v[1], dt)[0]  # [Hkv][d]
            assert bits(got[1]) == bits(v1.repeat_interleave(g, dim=0))


def _relabel(tables, pools, perm):
    """The same cache with physical block b moved to perm[b]: pools (and per-block
    arrays) permuted along their first axis, table entries mapped (padding kept)."""
    t = tables.copy()
    t[t >= 0] = perm[t[t >= 0]]
    moved = []
    for a in pools:
        m = np.empty_like(a)
        m[perm] = a
        moved.append(m)
    return t, moved


def _identity_perm(tables, num_blocks):
    """A relabelling that makes the tables physically consecutive (block ids in table
    order: the contiguous layout); blocks no table uses go after them."""
    used = [int(b) for b in tables.reshape(-1) if b >= 0]
    perm = np.full(num_blocks, -1, np.int64)
    nxt = 0
    for b in used:
        if perm[b] < 0:
            perm[b] = nxt
            nxt += 1
    for b in range(num_blocks):
        if perm[b] < 0:
            perm[b] = nxt
            nxt += 1
    return perm


@pytest.mark.parametrize("dt,Hq,Hkv,v", [("f32", 8, 2, VALU), ("f16", 8, 2, VALU), ("bf16", 8, 2, VALU),
                                         ("bf16", 64, 8, MFMA), ("f16", 16, 2, MFMA), ("bf16", 32, 32, VALU)])
def test_identity_and_permuted_tables_are_bit_identical(dt, Hq, Hkv, v):
    """Where the blocks sit changes nothing ("PagedAttention" concept report §5: the
    table maps logical blocks to any physical ones): the same cache laid out
    contiguously (identity tables) and under a random relabelling of the physical blocks
    gives bit-identical output on every kernel form (one pass, partitions, balanced
    split), the matrix-core kernel with 8 query heads per KV head included."""
    lens = [100, 37, 513, 16, 1, 700, 129]
    c = Case(np.random.default_rng(11), lens, Hq, Hkv, 128, 16, dt)
    perm_id = _identity_perm(c.tables, c.num_blocks)
    perm_rand = np.random.default_rng(12).permutation(c.num_blocks)
    outs = {}
    for lay, perm in (("paged", None), ("identity", perm_id), ("relabelled", perm_rand)):
        t, kc, vc = c.tables, c.kc, c.vc
        if perm is not None:
            t, (kc, vc) = _relabel(c.tables, (c.kc, c.vc), perm)
        if lay == "identity":  # physically consecutive
            nb = [-(-n // c.B) for n in lens]
            assert [t[s, :nb[s]].tolist() for s in range(len(lens))] == \
                [list(range(sum(nb[:s]), sum(nb[:s + 1]))) for s in range(len(lens))]
        c2 = Case.__new__(Case)
        c2.__dict__.update(c.__dict__)
        c2.tables, c2.kc, c2.vc = t, kc, vc
        for P in (0, 64, BAL):
            say(f"[gpu] layout {lay} {dt} g={Hq // Hkv} variant={v} P={P}")
            outs[(lay, P)] = bits(_run_case(c2, P, v))
    for P in (0, 64, BAL):
        assert outs[("paged", P)] == outs[("identity", P)] == outs[("relabelled", P)], P


def test_fp8_identity_and_permuted_tables_are_bit_identical():
    """E4M3 pools: moving every block together with its scales leaves the output
    bit-identical (one pass, partitions, balanced split; 1 and 4 query heads per KV head)."""
    for Hq, Hkv in ((8, 8), (16, 4)):
        c = Fp8Case(np.random.default_rng(13), [100, 37, 513, 16, 1, 300], Hq, Hkv, 128, 16, "bf16")
        perm_id = _identity_perm(c.tables, c.num_blocks)
        perm_rand = np.random.default_rng(14).permutation(c.num_blocks)
        res = {}
        for lay, perm in (("paged", None), ("identity", perm_id), ("relabelled", perm_rand)):
            arrays = (c.kc, c.vc, c.ks, c.vs)
            t = c.tables
            if perm is not None:
                t, arrays = _relabel(c.tables, arrays, perm)
            kc, vc, ks, vs = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays)
            q = to_torch(c.q, "bf16").cuda()
            bt, cl = torch.from_numpy(t).cuda(), torch.from_numpy(c.ctx).cuda()
            for P in (0, 64, BAL):
                out = torch.empty_like(q)
                ws = None
                if P:
                    ws = torch.empty(pa.pa_decode_workspace_bytes(q.shape[0], Hq, Hkv, 128, int(c.ctx.max()), P),
                                     dtype=torch.uint8, device="cuda")
                say(f"[gpu] fp8 layout {lay} g={Hq // Hkv} P={P}")
                pa.pa_decode_fp8(out, q, kc, vc, ks, vs, bt, cl, c.scale, max_context_len=int(c.ctx.max()),
                                 partition_size=P, workspace=ws)
                torch.cuda.synchronize()
                res[(lay, P)] = bits(out)
        for P in (0, 64, BAL):
            assert res[("paged", P)] == res[("identity", P)] == res[("relabelled", P)], (Hq, Hkv, P)


def test_grouped_decode_identity_and_permuted_layouts_are_bit_identical():
    """pa_decode_grouped over the same forked batch placed by the allocator from a
    permuted free list and from the identity free list: bit-identical outputs."""
    w = SMALL["prefix_f16"]
    outs = []
    for identity in (False, True):
        batch = W.make_batch(w, identity=identity)
        db = replay(batch)
        groups = db.groups(w.partition_size)
        assert groups[1].max() >= 1  # some partitions are shared
        say(f"[gpu] grouped layout identity={identity}")
        outs.append(bits(db.step_grouped(w.partition_size, groups, workspace=db.grouped_workspace(w.partition_size))))
        torch.cuda.synchronize()
    assert outs[0] == outs[1]


def test_shared_kv_hint_changes_nothing_but_the_cache_policy():
    """PA_DECODE_SHARED_KV selects cacheable loads; the result is bit-identical."""
    batch = W.make_batch(SMALL["prefix_f16"])
    for v in (VALU, AUTO):
        outs = []
        for hint in (0, pa.PA_DECODE_SHARED_KV):
            db = replay(batch)
            db.shared = False
            say(f"[gpu] shared-kv hint={hint} variant={v}")
            outs.append(bits(db.step(partition_size=64, variant=v | hint)))
        assert outs[0] == outs[1]
    g = W.make_batch(SMALL["gqa_bf16"])
    outs = []
    for hint in (0, pa.PA_DECODE_SHARED_KV):
        db = replay(g)
        say(f"[gpu] shared-kv hint={hint} mfma")
        outs.append(bits(db.step(partition_size=0, variant=MFMA | hint)))
    assert outs[0] == outs[1]


@pytest.mark.parametrize("P", [0, 64, BAL])
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_bad_table_entry_gives_nan_for_that_sequence_only(P, kernel):
    rng = np.random.default_rng(12)
    Hq, Hkv, v = (4, 4, VALU) if kernel == "valu" else (8, 2, MFMA)
    c = Case(rng, [40, 50, 60], Hq, Hkv, 128, 16, "f16")
    clean = _run_case(c, P, v)
    for bad in (-1, c.num_blocks, 1 << 30):
        t = c.tables.copy()
        t[1, 2] = bad
        say(f"[gpu] bad entry {bad} P={P} {kernel}")
        got = _run_case(c, P, v, tables=t)
        assert torch.isnan(got[1]).all()
        assert bits(got[0]) == bits(clean[0]) and bits(got[2]) == bits(clean[2])


@pytest.mark.parametrize("S", [1, 2, 63, 64, 65, 256, 257, 300, 512, 513, 700])
def test_one_pass_batch_sizes_and_longest_first_order(S):
    """The one-pass vector kernel runs sequences longest first (a sort of the lengths
    inside every workgroup: one wave up to 64 sequences, the whole 4-wave workgroup up
    to 256, index order beyond; f32 pools too).  Outputs must not depend on it: every row against the oracle,
    many equal lengths (ties), and a negative length (NaN for that sequence only)."""
    rng = np.random.default_rng(100 + S)
    lens = rng.integers(0, 49, S)
    lens[rng.integers(0, S)] = 48
    for dt, v in (("f16", VALU), ("f32", VALU)):
        c = Case(rng, lens, 2, 2, 64, 16, dt)
        want = c.run(oracle.default())
        say(f"[gpu] one pass S={S} {dt}")
        got = _run_case(c, 0, v)
        err = np.max(np.abs(f64(got) - want))
        assert err <= TOL[dt], (S, dt, err)
        assert torch.all(got[torch.from_numpy(lens == 0).cuda()] == 0)
        if S >= 2:
            bad = int(rng.integers(0, S))
            q, kc, vc, bt, cl = _upload_case(c)
            cl[bad] = -1
            out = torch.empty_like(q)
            pa.pa_decode(out, q, kc, vc, bt, cl, c.scale, max_context_len=int(c.ctx.max()),
                         partition_size=0, variant=v)
            torch.cuda.synchronize()
            assert torch.isnan(out[bad]).all()
            keep = torch.arange(S, device="cuda") != bad
            assert bits(out[keep]) == bits(got[keep])


def test_context_longer_than_max_context_len_gives_nan():
    rng = np.random.default_rng(13)
    c = Case(rng, [100, 300], 4, 4, 128, 16, "bf16")
    say("[gpu] ctx > max_context_len")
    got = _run_case(c, 64, VALU, max_ctx=128)
    assert torch.isnan(got[1]).all() and not torch.isnan(got[0]).any()


def test_reshape_and_cache_bitwise():
    rng = np.random.default_rng(14)
    for dt, nb, H, B, d in (("f16", 40, 8, 16, 128), ("f32", 9, 2, 64, 64), ("bf16", 7, 16, 128, 128)):
        N = nb * B // 3
        slots = rng.choice(nb * B, size=N, replace=False).astype(np.int32)
        slots[::7] = -1
        slots[3] = nb * B + 5  # past the pool: skipped
        key = W.round_to(rng.standard_normal((N, H, d), dtype=np.float32), dt)
        val = W.round_to(rng.standard_normal((N, H, d), dtype=np.float32), dt)
        kc = W.round_to(rng.standard_normal((nb, H, B, d), dtype=np.float32), dt)
        vc = W.round_to(rng.standard_normal((nb, H, B, d), dtype=np.float32), dt)
        gk, gv = to_torch(kc, dt).cuda(), to_torch(vc, dt).cuda()
        say(f"[gpu] reshape_and_cache {dt} N={N}")
        pa.pa_reshape_and_cache(to_torch(key, dt).cuda(), to_torch(val, dt).cuda(), gk, gv,
                                torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        ok = slots.copy()
        ok[3] = -1
        oracle.default().reshape_and_cache(key, val, kc, vc, ok, dt)
        assert bits(gk) == np_bits(kc) and bits(gv) == np_bits(vc)


def test_copy_blocks_bitwise():
    rng = np.random.default_rng(15)
    for dt, nb, H, B, d in (("f16", 64, 32, 16, 128), ("f32", 20, 4, 32, 64), ("bf16", 30, 8, 128, 128)):
        kc = W.round_to(rng.standard_normal((nb, H, B, d), dtype=np.float32), dt)
        vc = W.round_to(rng.standard_normal((nb, H, B, d), dtype=np.float32), dt)
        ids = rng.permutation(nb).astype(np.int32)
        n = nb // 3
        src, dst = ids[:n].copy(), ids[n:2 * n].copy()
        gk, gv = to_torch(kc, dt).cuda(), to_torch(vc, dt).cuda()
        s_dev = torch.from_numpy(np.append(src, nb + 3).astype(np.int32)).cuda()  # last pair skipped
        d_dev = torch.from_numpy(np.append(dst, 0).astype(np.int32)).cuda()
        say(f"[gpu] copy_blocks {dt} pairs={n}")
        pa.pa_copy_blocks(gk, gv, s_dev, d_dev)
        torch.cuda.synchronize()
        oracle.default().copy_blocks(kc, vc, src, dst, dt)
        assert bits(gk) == np_bits(kc) and bits(gv) == np_bits(vc)


def test_swap_out_and_in_round_trip():
    """Three sequences (two of them sharing prompt blocks) go to pinned host memory, their
    device blocks are reused and overwritten, and they come back: the host copy equals the
    oracle's move bit for bit, and attention afterwards is bit-identical to before."""
    from paged_kv_cache_308_amd.engine import HostKVPool, swap_in, swap_out
    w = SMALL["prefix_f16"]
    batch = W.make_batch(w)
    db = replay(batch)
    before = bits(db.step(partition_size=0, variant=VALU, fused=False))
    cache = db.cache
    host = HostKVPool(300, w.num_kv_heads, w.head_dim, w.block_size, TORCH_DTYPE[w.dtype])
    host.key_cache.fill_(0.0)
    host.value_cache.fill_(0.0)
    moved = [1, 3, 6]
    kc0 = cache.key_cache.cpu().numpy().view(np.uint16)
    vc0 = cache.value_cache.cpu().numpy().view(np.uint16)
    want_k = host.key_cache.numpy().view(np.uint16).copy()
    want_v = host.value_cache.numpy().view(np.uint16).copy()
    hseqs = []
    for s_ in moved:
        table, _ = cache.alloc.block_table(db.seq_ids[s_])
        say(f"[gpu] swap out seq {s_} ({len(table)} blocks)")
        h = swap_out(cache, host, db.seq_ids[s_])
        htable, _ = host.alloc.block_table(h)
        oracle.default().swap_blocks(kc0, vc0, want_k, want_v, np.asarray(table, np.int32),
                                     np.asarray(htable, np.int32), w.dtype)
        hseqs.append(h)
    torch.cuda.synchronize()
    assert host.key_cache.numpy().view(np.uint16).tobytes() == want_k.tobytes()
    assert host.value_cache.numpy().view(np.uint16).tobytes() == want_v.tobytes()
    # reuse the released device blocks for junk
    junk = cache.new_seq()
    n_free = cache.alloc.stats()["free_blocks"]
    slots, _, _ = cache.reserve([junk] * (n_free * w.block_size))
    rnd = torch.randn(len(slots), w.num_kv_heads, w.head_dim, device="cuda").to(TORCH_DTYPE[w.dtype])
    cache.write(rnd, rnd, slots)
    cache.free_seq(junk)
    for s_, h in zip(moved, hseqs):
        say(f"[gpu] swap in seq {s_}")
        db.seq_ids[s_] = swap_in(cache, host, h)
    bt, cl = cache.tables(db.seq_ids, db.host_tables.shape[1])
    assert np.array_equal(cl, db.host_context_lens)
    db.block_tables = torch.from_numpy(bt).cuda()
    db.shared = False
    after = bits(db.attend(partition_size=0, variant=VALU))
    torch.cuda.synchronize()
    assert after == before


# ------------------------------------------------------------------ E4M3 pools


def _run_fp8_case(c: Fp8Case, P, variant=VALU, tables=None):
    q = to_torch(c.q, c.qdtype).cuda()
    kc = torch.from_numpy(c.kc).cuda()
    vc = torch.from_numpy(c.vc).cuda()
    ks = torch.from_numpy(c.ks).cuda()
    vs = torch.from_numpy(c.vs).cuda()
    bt = torch.from_numpy(c.tables if tables is None else tables).cuda()
    cl = torch.from_numpy(c.ctx).cuda()
    out = torch.empty_like(q)
    mc = int(c.ctx.max())
    ws = None
    if P:
        n = pa.pa_decode_workspace_bytes(q.shape[0], q.shape[1], c.Hkv, c.d, mc, P)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    pa.pa_decode_fp8(out, q, kc, vc, ks, vs, bt, cl, c.scale, max_context_len=mc, partition_size=P,
                     variant=variant, workspace=ws)
    torch.cuda.synchronize()
    return out


FP8_EDGE_SHAPES = [
    # Hq, Hkv, d, B, query dtype: groups 1, 2 (16-code slices) and 4, 8 (8-code slices)
    (4, 4, 128, 16, "f16"),
    (4, 2, 64, 16, "bf16"),
    (8, 2, 128, 32, "f16"),
    (8, 1, 64, 16, "bf16"),
    (16, 2, 128, 64, "bf16"),
]


@pytest.mark.parametrize("shape", FP8_EDGE_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_fp8_edge_lengths(shape):
    Hq, Hkv, d, B, qdt = shape
    rng = np.random.default_rng(21)
    c = Fp8Case(rng, EDGE_LENS, Hq, Hkv, d, B, qdt)
    want = c.run(oracle.default())
    g = Hq // Hkv
    for P in (0, 64, 512, BAL) if B <= 64 else (0, 128, 512, BAL):
        say(f"[gpu] fp8 edge {shape} P={P}")
        got = _run_fp8_case(c, P)
        err = np.max(np.abs(f64(got) - want))
        assert err <= TOL[qdt], (shape, P, err)
        assert torch.all(got[0] == 0)  # empty context
        # one token: its dequantised V (code value times the block's scale), rounded
        b = int(c.tables[1, 0])
        v1 = torch.from_numpy(torch_fp8_values()[c.vc[b, :, 0, :]] *
                              c.vs[b][:, None].astype(np.float64))
        assert torch.equal(got[1].cpu(), v1.to(got.dtype).repeat_interleave(g, dim=0))


@pytest.mark.parametrize("P", [0, 64, BAL])
def test_fp8_bad_table_entry_gives_nan_for_that_sequence_only(P):
    rng = np.random.default_rng(22)
    c = Fp8Case(rng, [40, 50, 60], 4, 4, 128, 16, "f16")
    clean = _run_fp8_case(c, P)
    t = c.tables.copy()
    t[1, 2] = c.num_blocks
    say(f"[gpu] fp8 bad entry P={P}")
    got = _run_fp8_case(c, P, tables=t)
    assert torch.isnan(got[1]).all()
    assert bits(got[0]) == bits(clean[0]) and bits(got[2]) == bits(clean[2])


@pytest.mark.parametrize("S", [1, 64, 65, 256, 257, 300])
def test_fp8_one_pass_batch_sizes_and_longest_first_order(S):
    """The E4M3 one-pass kernel (4-wave workgroups) sorts up to 256 sequences longest
    first and keeps index order beyond; outputs against the oracle either way, ties
    included."""
    rng = np.random.default_rng(200 + S)
    lens = rng.integers(0, 40, S)
    lens[rng.integers(0, S)] = 40
    c = Fp8Case(rng, lens, 2, 2, 128, 16, "f16")
    want = c.run(oracle.default())
    say(f"[gpu] E4M3 one pass S={S}")
    got = _run_fp8_case(c, 0)
    err = np.max(np.abs(f64(got) - want))
    assert err <= TOL["f16"], (S, err)
    assert torch.all(got[torch.from_numpy(lens == 0).cuda()] == 0)


def _fp8_special_values(rng, n):
    """Every E4M3 value and every midpoint between neighbours (ties), both signs, the
    saturation edge, zeros, infinities, NaN, then random numbers over many magnitudes."""
    vals = torch_fp8_values()
    finite = vals[:0x7F]
    mids = (finite[:-1] + finite[1:]) / 2
    special = np.concatenate([finite, mids, -finite, -mids,
                              [447.0, 448.0, 455.0, 456.0, 463.0, 464.0, 500.0, 1e4, -1e4, np.inf,
                               -np.inf, np.nan, 0.0, -0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11]])
    rest = rng.standard_normal(max(0, n - len(special))) * np.exp2(rng.uniform(-12, 10, max(0, n - len(special))))
    return np.concatenate([special, rest])[:n].astype(np.float32)


def test_reshape_and_cache_fp8_bitwise():
    """E4M3 scatter against the oracle's brute-force nearest-code search: exact values,
    ties, saturation, NaN / inf, with power-of-two scales (x / s exact) and random ones."""
    rng = np.random.default_rng(23)
    for dt, nb, H, B, d in (("f32", 12, 2, 16, 64), ("f16", 40, 8, 16, 128), ("bf16", 7, 4, 128, 128)):
        N = nb * B // 2
        slots = rng.choice(nb * B, size=N, replace=False).astype(np.int32)
        slots[::7] = -1
        slots[3] = nb * B + 5  # past the pool: skipped
        vals = _fp8_special_values(rng, N * H * d).reshape(N, H, d)
        key = W.round_to(vals, dt)
        val = W.round_to(rng.permutation(vals.ravel()).reshape(N, H, d), dt)
        ks = np.where(rng.random((nb, H)) < 0.5, np.exp2(rng.integers(-8, 3, (nb, H))),
                      np.exp2(rng.uniform(-8, 2, (nb, H)))).astype(np.float32)
        vs = np.exp2(rng.uniform(-8, 2, (nb, H))).astype(np.float32)
        kc = rng.integers(0, 256, (nb, H, B, d)).astype(np.uint8)
        vc = rng.integers(0, 256, (nb, H, B, d)).astype(np.uint8)
        gk, gv = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
        say(f"[gpu] reshape_and_cache_fp8 {dt} N={N}")
        pa.pa_reshape_and_cache_fp8(to_torch(key, dt).cuda(), to_torch(val, dt).cuda(), gk, gv,
                                    torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda(),
                                    torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        ok = slots.copy()
        ok[3] = -1
        oracle.default().reshape_and_cache_fp8(key, val, kc, vc, ks, vs, ok, dt)
        assert bits(gk) == np_bits(kc) and bits(gv) == np_bits(vc)


def test_fp8_blocks_and_scales_copy_and_swap_bitwise():
    """E4M3 pools move with pa_copy_blocks / pa_swap_blocks, and so do their scale arrays,
    as pools of one float32 per (block, KV head): 4-byte words when H_kv * 4 is not a
    multiple of 16."""
    rng = np.random.default_rng(24)
    for H in (2, 8):
        nb, B, d = 30, 16, 128
        kc = rng.integers(0, 256, (nb, H, B, d)).astype(np.uint8)
        vc = rng.integers(0, 256, (nb, H, B, d)).astype(np.uint8)
        ks = rng.random((nb, H, 1, 1)).astype(np.float32)
        vs = rng.random((nb, H, 1, 1)).astype(np.float32)
        ids = rng.permutation(nb).astype(np.int32)
        src, dst = ids[:9].copy(), ids[9:18].copy()
        g = [torch.from_numpy(a).cuda() for a in (kc, vc, ks, vs)]
        sd, dd = torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda()
        say(f"[gpu] fp8 copy H={H}")
        pa.pa_copy_blocks(g[0], g[1], sd, dd)
        pa.pa_copy_blocks(g[2], g[3], sd, dd)
        torch.cuda.synchronize()
        o = oracle.default()
        o.copy_blocks(kc, vc, src, dst, "fp8")
        o.copy_blocks(ks, vs, src, dst, "f32")
        for t, a in zip(g, (kc, vc, ks, vs)):
            assert bits(t) == np_bits(a)
        # device -> pinned host
        hk = torch.zeros((12, H, B, d), dtype=torch.uint8, pin_memory=True)
        hv = torch.zeros_like(hk).pin_memory()
        hks = torch.zeros((12, H, 1, 1), dtype=torch.float32, pin_memory=True)
        hvs = torch.zeros_like(hks).pin_memory()
        hs, hd = src[:5].copy(), rng.choice(12, 5, replace=False).astype(np.int32)
        say(f"[gpu] fp8 swap H={H}")
        pa.pa_swap_blocks(g[0], g[1], hk, hv, torch.from_numpy(hs).cuda(), torch.from_numpy(hd).cuda())
        pa.pa_swap_blocks(g[2], g[3], hks, hvs, torch.from_numpy(hs).cuda(), torch.from_numpy(hd).cuda())
        torch.cuda.synchronize()
        wk, wv = np.zeros((12, H, B, d), np.uint8), np.zeros((12, H, B, d), np.uint8)
        wks, wvs = np.zeros((12, H, 1, 1), np.float32), np.zeros((12, H, 1, 1), np.float32)
        o.swap_blocks(kc, vc, wk, wv, hs, hd, "fp8")
        o.swap_blocks(ks, vs, wks, wvs, hs, hd, "f32")
        for t, a in zip((hk, hv, hks, hvs), (wk, wv, wks, wvs)):
            assert t.numpy().tobytes() == a.tobytes()


def test_fp8_swap_out_and_in_round_trip():
    """E4M3 pools swap with their block scales: out to pinned host memory, device blocks
    reused, back in; attention afterwards is bit-identical to before."""
    from paged_kv_cache_308_amd.engine import HostKVPool, swap_in, swap_out
    w = SMALL["fp8_prefix_bf16"]
    batch = W.make_batch(w)
    db = replay(batch)
    before = bits(db.step(partition_size=0, variant=VALU, fused=False))
    cache = db.cache
    host = HostKVPool(300, w.num_kv_heads, w.head_dim, w.block_size, torch.uint8)
    moved = [0, 4, 7]
    hseqs = []
    for s_ in moved:
        say(f"[gpu] fp8 swap out seq {s_}")
        hseqs.append(swap_out(cache, host, db.seq_ids[s_]))
    torch.cuda.synchronize()
    # overwrite the released blocks and their scales
    junk = cache.new_seq()
    n_free = cache.alloc.stats()["free_blocks"]
    slots, _, _ = cache.reserve([junk] * (n_free * w.block_size))
    cache.k_scales.fill_(0.5)
    cache.v_scales.fill_(0.25)
    rnd = torch.randn(len(slots), w.num_kv_heads, w.head_dim, device="cuda").to(TORCH_DTYPE[w.dtype])
    cache.write(rnd, rnd, slots)
    cache.free_seq(junk)
    for s_, h in zip(moved, hseqs):
        say(f"[gpu] fp8 swap in seq {s_}")
        db.seq_ids[s_] = swap_in(cache, host, h)
    # the scale fill above also hit the kept sequences' blocks: restore theirs
    ref = replay(batch)
    keep = [s_ for s_ in range(w.num_seqs) if s_ not in moved]
    for s_ in keep:
        t, _ = cache.alloc.block_table(db.seq_ids[s_])
        idx = torch.tensor(t, dtype=torch.long, device="cuda")
        cache.k_scales[idx] = ref.cache.k_scales[idx]
        cache.v_scales[idx] = ref.cache.v_scales[idx]
    bt, cl = cache.tables(db.seq_ids, db.host_tables.shape[1])
    assert np.array_equal(cl, db.host_context_lens)
    db.block_tables = torch.from_numpy(bt).cuda()
    db.shared = False
    after = bits(db.attend(partition_size=0, variant=VALU))
    torch.cuda.synchronize()
    # the moved sequences are bit-identical (their blocks and scales came back)
    g = bits_rows(after, moved, w)
    assert g == bits_rows(before, moved, w)


def bits_rows(b: bytes, rows, w) -> bytes:
    per = w.num_q_heads * w.head_dim * 2
    return b"".join(b[r * per:(r + 1) * per] for r in rows)


@pytest.mark.parametrize("tile", [1024, 2048, 4096, 8192])
def test_gather_read_probe_reads_without_writing(tile):
    """pa_gather_read reads the listed tiles (addresses inside one zero buffer, in random
    order, an odd count) and leaves the sink alone (all-zero data folds to 0)."""
    ntiles = 37
    buf = torch.zeros(ntiles * tile, dtype=torch.uint8, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    order = np.random.default_rng(tile).permutation(ntiles).astype(np.int64)
    addrs = torch.from_numpy(buf.data_ptr() + order * tile).cuda()
    say(f"[gpu] gather read {ntiles} tiles of {tile} bytes")
    pa.pa_gather_read(addrs, tile, sink)
    pa.pa_gather_read(addrs[:1], tile, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]


def test_stream_read_probe_reads_without_writing():
    """pa_stream_read (the read-bandwidth probe) runs over a buffer and leaves the sink
    alone unless the folded value hits its constant (an all-zero buffer folds to 0)."""
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    say("[gpu] stream read 1 MiB")
    pa.pa_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]
    small = torch.zeros(48, dtype=torch.uint8, device="cuda")  # fewer words than one workgroup
    pa.pa_stream_read(small, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]


def test_step_upload_equals_host_arrays():
    """A step's slots, tables and lengths, packed into pinned staging and copied on the
    stream (engine.StepUploader), arrive equal to the host arrays; with two stagings the
    views of the previous upload stay intact while the next one is packed and copied."""
    from paged_kv_cache_308_amd.engine import StepUploader
    rng = np.random.default_rng(77)
    up = StepUploader(64, 300)
    prev = None
    for k in range(8):
        S, mb = int(rng.integers(1, 65)), int(rng.integers(1, 301))
        tb = rng.integers(-1, 40000, (S, mb)).astype(np.int32)
        sl = rng.integers(-1, 1 << 20, S).astype(np.int32)
        cl = rng.integers(0, 4097, S).astype(np.int32)
        say(f"[gpu] step upload {k}: S={S} max_blocks={mb}")
        got = up.upload(sl, tb, cl)
        torch.cuda.synchronize()
        for g, want in zip(got, (sl, tb, cl)):
            assert g.is_contiguous() and np.array_equal(g.cpu().numpy(), want)
        if prev is not None:  # the previous upload's views are still intact
            for g, want in zip(*prev):
                assert np.array_equal(g.cpu().numpy(), want)
        prev = (got, (sl, tb, cl))
    with pytest.raises(ValueError):
        up.upload(np.zeros(65, np.int32), np.zeros((65, 1), np.int32), np.zeros(65, np.int32))


def test_step_upload_drives_decode():
    """The allocator's step (slots, tables, lengths) through the pinned upload feeds the
    decode launch: the result is bit-identical to the same step with the tables uploaded
    by a plain synchronous copy."""
    from paged_kv_cache_308_amd.engine import StepUploader
    w = SMALL["mha_f16"]
    batch = W.make_batch(w)
    db = replay(batch)
    ref = bits(db.step(partition_size=0, variant=VALU))
    up = StepUploader(w.num_seqs, db.host_tables.shape[1])
    slots = db.slot_mapping.cpu().numpy()
    sl, bt, cl = up.upload(slots, db.host_tables, db.host_context_lens)
    db2 = replay(batch)
    db2.slot_mapping, db2.block_tables, db2.context_lens = sl, bt, cl
    say("[gpu] decode through uploaded step data")
    assert bits(db2.step(partition_size=0, variant=VALU)) == ref
