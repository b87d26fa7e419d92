"""Pins that tie the oracle to facts it does not define itself.

Each pin takes an oracle instance so the same checks can be run against copies
of the oracle with a planted mistake (see test_oracle_pins.py).  The facts used:

  library    torch's scaled_dot_product_attention in float64 on the CPU, fed the
             tokens in logical order (the contiguous layout the block table hides:
             "PagedAttention 深度解析" (5ulink) §二 item 3); numpy fancy indexing for
             the scatter and the block copy; numpy / torch for f16 / bf16 decoding.
  closed     a context of one token returns that token's V exactly; equal keys give
  forms      the mean of the values; a key whose score leads by >= 800 returns its
             V exactly (every other weight underflows to zero in binary64).
  invariants relabelling physical blocks leaves the output bit-identical; shared
             prefix blocks equal duplicated blocks; NaN in slots past the context
             never reaches the output.
  pages      the 100-token / 7-block request with physical blocks 5,2,7,0,12,3,9
             (5ulink §二), computed through its table, equals attention over the
             same 100 tokens laid out contiguously.
  brute      pure-Python loops through the table on tiny inputs.
  E4M3       torch's float8_e4m3fn for the value of every code and for rounding
             (clamped to +-448 first: the saturating reading), every midpoint
             between neighbouring codes (ties to even), the round trip of every
             finite code, and torch SDPA over dequantised tokens for the decode.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import workloads as W
from oracle import OracleError
from oracle.alloc_model import ModelAllocator

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# independent construction of paged inputs (numpy reshapes, no oracle code)


class Case:
    """Per-sequence logical K/V, a random placement into pools, and tables."""

    def __init__(self, rng, lens, Hq, Hkv, d, B, dtype, num_blocks=None, identity=False,
                 scale=None, poison=True):
        self.lens = [int(x) for x in lens]
        self.Hq, self.Hkv, self.d, self.B, self.dtype = Hq, Hkv, d, B, dtype
        nblk = [max(0, -(-n // B)) for n in self.lens]
        need = sum(nblk)
        self.num_blocks = num_blocks or max(need + 3, 1)
        self.scale = float(np.float32(scale if scale is not None else 1.0 / math.sqrt(d)))
        npd = W.storage_np_dtype(dtype)
        S = len(self.lens)
        self.q = W.round_to(rng.standard_normal((S, Hq, d), dtype=np.float32), dtype)
        self.k = [W.round_to(rng.standard_normal((n, Hkv, d), dtype=np.float32), dtype)
                  for n in self.lens]
        self.v = [W.round_to(rng.standard_normal((n, Hkv, d), dtype=np.float32), dtype)
                  for n in self.lens]
        ids = np.arange(self.num_blocks) if identity else rng.permutation(self.num_blocks)
        self.max_blocks = max(1, max(nblk) if nblk else 1)
        self.tables = np.full((S, self.max_blocks), -1, np.int32)
        pos = 0
        for s, nb in enumerate(nblk):
            self.tables[s, :nb] = ids[pos:pos + nb]
            pos += nb
        fill = W.nan_bits(dtype) if poison else npd(0)
        shape = (self.num_blocks, Hkv, B, d)
        self.kc = np.full(shape, fill, npd)
        self.vc = np.full(shape, fill, npd)
        for s in range(S):
            self._put(s, self.kc, self.k[s])
            self._put(s, self.vc, self.v[s])
        self.ctx = np.asarray(self.lens, np.int32)

    def _put(self, s, pool, x):
        n = x.shape[0]
        nb = -(-n // self.B)
        if nb == 0:
            return
        pad = np.zeros((nb * self.B, self.Hkv, self.d), x.dtype)
        pad[:n] = x
        tiles = pad.reshape(nb, self.B, self.Hkv, self.d).transpose(0, 2, 1, 3)
        ids = self.tables[s, :nb]
        for j in range(nb):
            valid = min(self.B, n - j * self.B)
            pool[ids[j], :, :valid, :] = tiles[j, :, :valid, :]

    def f64(self, a):
        if self.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double().numpy()
        return a.astype(np.float64)

    def run(self, o):
        return o.decode(self.q, self.kc, self.vc, self.tables, self.ctx, self.scale, self.dtype)

    def sdpa(self):
        """torch SDPA (float64, CPU) over the logical tokens of each sequence."""
        S = len(self.lens)
        out = np.zeros((S, self.Hq, self.d))
        for s in range(S):
            n = self.lens[s]
            if n == 0:
                continue
            q = torch.from_numpy(self.f64(self.q[s]))[None, :, None, :]
            k = torch.from_numpy(self.f64(self.k[s])).permute(1, 0, 2)[None].contiguous()
            v = torch.from_numpy(self.f64(self.v[s])).permute(1, 0, 2)[None].contiguous()
            o = F.scaled_dot_product_attention(q, k, v, scale=self.scale,
                                               enable_gqa=self.Hq != self.Hkv)
            out[s] = o[0, :, 0, :].numpy()
        return out


SHAPES = [
    # lens, Hq, Hkv, d, B, dtype
    ([1, 2, 3, 7, 16, 17, 40], 2, 2, 8, 4, "f32"),
    ([5, 33], 4, 2, 8, 16, "f16"),
    ([9, 1, 24], 4, 1, 2, 1, "bf16"),
    ([31, 8], 8, 2, 16, 2, "f32"),
    ([100, 17, 16, 1], 4, 4, 64, 16, "f32"),
    ([65, 129], 16, 2, 128, 32, "bf16"),
]


def pin_sdpa(o):
    """Decode through random tables equals torch SDPA over the logical tokens."""
    rng = np.random.default_rng(100)
    for lens, Hq, Hkv, d, B, dt in SHAPES:
        for identity in (True, False):
            c = Case(rng, lens, Hq, Hkv, d, B, dt, identity=identity)
            got, want = c.run(o), c.sdpa()
            err = np.max(np.abs(got - want))
            assert err <= 1e-12, (lens, Hq, Hkv, d, B, dt, identity, err)


def pin_brute(o):
    """Pure-Python loops through the table (math.fsum / math.exp)."""
    rng = np.random.default_rng(101)
    c = Case(rng, [3, 6, 1], 4, 2, 3, 2, "f16")
    got = c.run(o)
    g = c.Hq // c.Hkv
    kc, vc = c.f64(c.kc), c.f64(c.vc)
    qf = c.f64(c.q)
    for s, n in enumerate(c.lens):
        for h in range(c.Hq):
            kh = h // g
            xs = []
            for t in range(n):
                b = c.tables[s, t // c.B]
                xs.append(c.scale * math.fsum(qf[s, h, j] * kc[b, kh, t % c.B, j] for j in range(c.d)))
            m = max(xs)
            ps = [math.exp(x - m) for x in xs]
            Z = math.fsum(ps)
            for j in range(c.d):
                ref = math.fsum(ps[t] * vc[c.tables[s, t // c.B], kh, t % c.B, j] for t in range(n)) / Z
                assert abs(got[s, h, j] - ref) <= 1e-12, (s, h, j, got[s, h, j], ref)


def pin_permutation(o):
    """Relabelling the physical blocks leaves the result bit-identical."""
    rng = np.random.default_rng(102)
    for lens, Hq, Hkv, d, B, dt in SHAPES[:4]:
        c = Case(rng, lens, Hq, Hkv, d, B, dt)
        a = c.run(o)
        pi = rng.permutation(c.num_blocks)
        kc2 = np.empty_like(c.kc)
        vc2 = np.empty_like(c.vc)
        kc2[pi] = c.kc
        vc2[pi] = c.vc
        t2 = np.where(c.tables >= 0, pi[np.maximum(c.tables, 0)], -1).astype(np.int32)
        b = o.decode(c.q, kc2, vc2, t2, c.ctx, c.scale, c.dtype)
        assert np.array_equal(a, b)


def pin_ctx1(o):
    """One cached token: the output is that token's V exactly (per KV head)."""
    rng = np.random.default_rng(103)
    for Hq, Hkv, dt in ((4, 4, "f32"), (8, 2, "bf16"), (6, 3, "f16")):
        c = Case(rng, [1, 1, 1], Hq, Hkv, 8, 4, dt)
        out = c.run(o)
        g = Hq // Hkv
        for s in range(3):
            for h in range(Hq):
                assert np.array_equal(out[s, h], c.f64(c.v[s][0, h // g])), (dt, s, h)


def pin_equal_keys(o):
    """All keys equal: uniform weights, the output is the mean of the values."""
    rng = np.random.default_rng(104)
    c = Case(rng, [7, 20], 2, 2, 8, 4, "f32")
    for s in range(2):
        c.k[s][:] = c.k[s][0]
        c._put(s, c.kc, c.k[s])
    out = c.run(o)
    for s, n in enumerate(c.lens):
        for h in range(2):
            for j in range(8):
                mean = math.fsum(float(c.v[s][t, h, j]) for t in range(n)) / n
                assert abs(out[s, h, j] - mean) <= 1e-14 * max(1.0, abs(mean)) + 1e-15


def pin_dominant(o):
    """A key whose score leads by >= 800 takes all the weight: output == its V."""
    rng = np.random.default_rng(105)
    c = Case(rng, [5], 1, 1, 4, 2, "f32", scale=1.0)
    c.q[0, 0] = [40.0, 0.0, 0.0, 0.0]
    c.k[0][:] = 0.0
    c.k[0][3, 0] = [40.0, 0.0, 0.0, 0.0]  # score 1600, the others 0
    c._put(0, c.kc, c.k[0])
    out = c.run(o)
    assert np.array_equal(out[0, 0], c.v[0][3, 0].astype(np.float64))


def pin_shared_prefix(o):
    """Tables that share prefix blocks give what duplicated copies give."""
    rng = np.random.default_rng(106)
    B, H, d = 4, 2, 8
    c = Case(rng, [10, 10, 10], H, H, d, B, "bf16", poison=True)
    # make sequences 1 and 2 share sequence 0's first two (full) blocks
    shared = c.tables[0, :2].copy()
    dup = c.tables.copy()
    for s in (1, 2):
        c.kc[c.tables[s, :2]] = c.kc[shared]
        c.vc[c.tables[s, :2]] = c.vc[shared]
        dup[s, :2] = c.tables[s, :2]
    sharing = c.tables.copy()
    sharing[1:, :2] = shared
    a = o.decode(c.q, c.kc, c.vc, sharing, c.ctx, c.scale, "bf16")
    b = o.decode(c.q, c.kc, c.vc, dup, c.ctx, c.scale, "bf16")
    assert np.array_equal(a, b)


def pin_nan_poison(o):
    """NaN in unused slots and blocks never reaches the result."""
    rng = np.random.default_rng(107)
    c = Case(rng, [5, 17, 3], 2, 2, 8, 8, "f16", poison=True)
    a = c.run(o)
    rng = np.random.default_rng(107)
    z = Case(rng, [5, 17, 3], 2, 2, 8, 8, "f16", poison=False)
    b = z.run(o)
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)


def pin_empty(o):
    """A context of length 0 gives zeros; the other sequences are unaffected."""
    rng = np.random.default_rng(108)
    c = Case(rng, [0, 9], 2, 2, 8, 4, "f32")
    out = c.run(o)
    assert np.all(out[0] == 0.0)
    assert np.max(np.abs(out[1] - c.sdpa()[1])) <= 1e-12


def pin_bad_index(o):
    """A table entry needed for t < ctx outside [0, num_blocks) is rejected."""
    rng = np.random.default_rng(109)
    c = Case(rng, [9], 1, 1, 4, 4, "f32")
    for bad in (-1, c.num_blocks):
        t = c.tables.copy()
        t[0, 2] = bad  # token 8 lives in logical block 2
        try:
            o.decode(c.q, c.kc, c.vc, t, c.ctx, c.scale, "f32")
        except OracleError:
            continue
        raise AssertionError(f"entry {bad} accepted")
    t = np.concatenate([c.tables, np.full((1, 2), -1, np.int32)], axis=1)
    o.decode(c.q, c.kc, c.vc, t, c.ctx, c.scale, "f32")  # padding past ctx is fine


def pin_reshape(o):
    """The slot scatter equals numpy fancy indexing over [blocks*B] slots."""
    rng = np.random.default_rng(110)
    for dt, nb, H, B, d in (("f16", 6, 2, 4, 8), ("f32", 3, 3, 16, 4), ("bf16", 5, 1, 2, 16)):
        npd = W.storage_np_dtype(dt)
        N = nb * B // 2
        slots = rng.choice(nb * B, size=N, replace=False).astype(np.int32)
        slots[::5] = -1
        key = W.round_to(rng.standard_normal((N, H, d), dtype=np.float32), dt)
        val = W.round_to(rng.standard_normal((N, H, d), dtype=np.float32), dt)
        kc = W.round_to(rng.standard_normal((nb, H, B, d), dtype=np.float32), dt)
        vc = W.round_to(rng.standard_normal((nb, H, B, d), dtype=np.float32), dt)
        want_k, want_v = kc.copy(), vc.copy()
        keep = slots >= 0
        for want, x in ((want_k, key), (want_v, val)):
            flat = want.transpose(0, 2, 1, 3).reshape(nb * B, H, d).copy()
            flat[slots[keep]] = x[keep]
            want[...] = flat.reshape(nb, B, H, d).transpose(0, 2, 1, 3)
        o.reshape_and_cache(key, val, kc, vc, slots, dt)
        assert kc.tobytes() == want_k.tobytes() and vc.tobytes() == want_v.tobytes(), dt
        assert npd is not None


def pin_copy(o):
    """Whole-block copies equal numpy pool[dst] = pool[src] on both pools."""
    rng = np.random.default_rng(111)
    for dt in ("f32", "f16", "bf16"):
        nb, H, B, d = 12, 2, 4, 8
        kc = W.round_to(rng.standard_normal((nb, H, B, d), dtype=np.float32), dt)
        vc = W.round_to(rng.standard_normal((nb, H, B, d), dtype=np.float32), dt)
        ids = rng.permutation(nb)
        src, dst = ids[:4].astype(np.int32), ids[4:8].astype(np.int32)
        wk, wv = kc.copy(), vc.copy()
        wk[dst] = wk[src]
        wv[dst] = wv[src]
        o.copy_blocks(kc, vc, src, dst, dt)
        assert kc.tobytes() == wk.tobytes() and vc.tobytes() == wv.tobytes()


def pin_swap(o):
    """Moves between two pools equal numpy dst[dst_ids] = src[src_ids], bitwise; the
    source pools are untouched."""
    rng = np.random.default_rng(114)
    for dt in ("f32", "f16", "bf16"):
        H, B, d = 2, 4, 8
        sk = W.round_to(rng.standard_normal((10, H, B, d), dtype=np.float32), dt)
        sv = W.round_to(rng.standard_normal((10, H, B, d), dtype=np.float32), dt)
        dk = W.round_to(rng.standard_normal((7, H, B, d), dtype=np.float32), dt)
        dv = W.round_to(rng.standard_normal((7, H, B, d), dtype=np.float32), dt)
        src = rng.choice(10, 5, replace=False).astype(np.int32)
        dst = rng.choice(7, 5, replace=False).astype(np.int32)
        wk, wv = dk.copy(), dv.copy()
        wk[dst] = sk[src]
        wv[dst] = sv[src]
        sk0, sv0 = sk.copy(), sv.copy()
        o.swap_blocks(sk, sv, dk, dv, src, dst, dt)
        assert dk.tobytes() == wk.tobytes() and dv.tobytes() == wv.tobytes()
        assert sk.tobytes() == sk0.tobytes() and sv.tobytes() == sv0.tobytes()


def pin_page3_request(o):
    """The 100-token request of 5ulink §二 through its table [5,2,7,0,12,3,9]
    equals attention over its 100 tokens laid out contiguously."""
    g = golden("page3_100_token_request.json")
    B, n = g["block_size"], g["tokens"]
    a = ModelAllocator(16, B)
    rest = [i for i in range(16) if i not in g["physical_blocks"]]
    a.set_free_order(g["physical_blocks"] + rest)
    sid = a.new_seq()
    slots = np.array([a.append_slot(sid)[0] for _ in range(n)], np.int32)
    table, ctx = a.block_table(sid)
    assert table == g["physical_blocks"] and len(table) == g["num_logical_blocks"] and ctx == n
    rng = np.random.default_rng(112)
    H, d = 2, 16
    key = rng.standard_normal((n, H, d), dtype=np.float32)
    val = rng.standard_normal((n, H, d), dtype=np.float32)
    q = rng.standard_normal((1, H, d), dtype=np.float32)
    kc = np.full((16, H, B, d), np.nan, np.float32)
    vc = np.full((16, H, B, d), np.nan, np.float32)
    o.reshape_and_cache(key, val, kc, vc, slots, "f32")
    bt = np.array([table], np.int32)
    out = o.decode(q, kc, vc, bt, np.array([n], np.int32), 0.25, "f32")
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q[0].astype(np.float64))[None, :, None, :],
        torch.from_numpy(key.astype(np.float64)).permute(1, 0, 2)[None].contiguous(),
        torch.from_numpy(val.astype(np.float64)).permute(1, 0, 2)[None].contiguous(),
        scale=0.25)[0, :, 0, :].numpy()
    assert np.max(np.abs(out[0] - ref)) <= 1e-12


def pin_dtype_decode(o):
    """Stored f16 / bf16 / f32 values decode to binary64 exactly (all bit patterns)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.load(bits.view(np.float16), "f16")
    want = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(got, want, equal_nan=True)
    got = o.load(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want, equal_nan=True)
    x = np.random.default_rng(113).standard_normal(1000).astype(np.float32)
    x[:4] = [0.0, -0.0, np.float32(1e-45), np.float32(3.4e38)]
    assert np.array_equal(o.load(x, "f32"), x.astype(np.float64))


# ---------------------------------------------------------------------------
# E4M3 pools with a scale per (physical block, KV head)


def torch_fp8_values() -> np.ndarray:
    """float64 value of each of the 256 E4M3 codes, decoded by torch."""
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def torch_fp8_encode(y) -> np.ndarray:
    """Codes for float32 numbers: torch's round-to-nearest-even cast after clamping to
    +-448 (NaN stays NaN and becomes 0x7F)."""
    t = torch.from_numpy(np.ascontiguousarray(y, np.float32))
    codes = t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    codes[np.isnan(np.asarray(y))] = 0x7F
    return codes


def pin_fp8_codes(o):
    """Every E4M3 code decodes to torch's value (NaN at 0x7F / 0xFF only), with the
    format's landmarks: 1.0 = 0x38, 448 = 0x7E, 2^-6 = 0x08, 2^-9 = 0x01."""
    c = np.arange(256, dtype=np.uint8)
    got = o.fp8_value(c)
    assert np.array_equal(got, torch_fp8_values(), equal_nan=True)
    assert [i for i in range(256) if np.isnan(got[i])] == [0x7F, 0xFF]
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0xBC] == -1.5 and np.signbit(got[0x80]) and got[0x80] == 0.0


def pin_fp8_encode(o):
    """Rounding to E4M3 equals torch's cast after clamping to +-448: random numbers over
    many magnitudes, every midpoint between neighbouring codes (ties go to the even
    code), the saturation edge, zeros, infinities and NaN; finite codes round-trip."""
    vals = torch_fp8_values()
    finite = [c for c in range(0x7F)]  # 0x00..0x7E
    mids = [(vals[c] + vals[c + 1]) / 2 for c in finite[:-1]]
    rng = np.random.default_rng(120)
    ys = np.concatenate([
        np.asarray(mids, np.float32), -np.asarray(mids, np.float32),
        (rng.standard_normal(4000) * np.exp2(rng.uniform(-14, 10, 4000))).astype(np.float32),
        np.array([447.9, 448.0, 455.9, 456.0, 463.99, 464.0, 500.0, 1e30, np.inf, -np.inf, -464.0,
                  0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, 3 * 2.0 ** -11, np.nan], np.float32)])
    got = o.fp8_encode(ys)
    want = torch_fp8_encode(ys)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(ys[i]), int(got[i]), int(want[i])) for i in bad[:5]]
    # midpoint ties land on the even neighbour
    for c, m in zip(finite[:-1], mids):
        assert int(o.fp8_encode(np.float32(m))) % 2 == 0, (c, m)
    codes = np.array(finite + [0x80 + c for c in finite], np.uint8)
    assert np.array_equal(o.fp8_encode(vals[codes].astype(np.float32)), codes)


class Fp8Case:
    """E4M3 pools with random per-(block, KV head) scales, placed through a random
    permutation of blocks; slots past each context hold the NaN code.  Tokens are
    standard normal numbers x stored as torch's E4M3 rounding of x / s (s the scale of
    the block and head holding them), so dequantised values are O(1)."""

    def __init__(self, rng, lens, Hq, Hkv, d, B, qdtype):
        self.lens = [int(x) for x in lens]
        self.Hq, self.Hkv, self.d, self.B, self.qdtype = Hq, Hkv, d, B, qdtype
        self.dtype = qdtype  # of the query (Case.f64 reads it)
        nblk = [-(-n // B) for n in self.lens]
        self.num_blocks = sum(nblk) + 3
        self.scale = float(np.float32(1.0 / math.sqrt(d)))
        S = len(self.lens)
        self.q = W.round_to(rng.standard_normal((S, Hq, d), dtype=np.float32), qdtype)
        self.ks = np.exp2(rng.uniform(-7, -4, (self.num_blocks, Hkv))).astype(np.float32)
        self.vs = np.exp2(rng.uniform(-7, -4, (self.num_blocks, Hkv))).astype(np.float32)
        ids = rng.permutation(self.num_blocks)
        self.max_blocks = max(1, max(nblk))
        self.tables = np.full((S, self.max_blocks), -1, np.int32)
        pos = 0
        for s, nb in enumerate(nblk):
            self.tables[s, :nb] = ids[pos:pos + nb]
            pos += nb
        shape = (self.num_blocks, Hkv, B, d)
        self.kc = np.full(shape, 0x7F, np.uint8)
        self.vc = np.full(shape, 0x7F, np.uint8)
        vals = torch_fp8_values()
        self.kf, self.vf = [], []  # dequantised tokens [n][H_kv][d] in logical order
        for s, n in enumerate(self.lens):
            kx = rng.standard_normal((n, Hkv, d), dtype=np.float32)
            vx = rng.standard_normal((n, Hkv, d), dtype=np.float32)
            kf = np.empty((n, Hkv, d))
            vf = np.empty((n, Hkv, d))
            for t in range(n):
                b = self.tables[s, t // B]
                ks, vs = self.ks[b][:, None], self.vs[b][:, None]
                kcode = torch_fp8_encode((torch.from_numpy(kx[t]) / torch.from_numpy(ks)).numpy())
                vcode = torch_fp8_encode((torch.from_numpy(vx[t]) / torch.from_numpy(vs)).numpy())
                self.kc[b, :, t % B, :] = kcode
                self.vc[b, :, t % B, :] = vcode
                kf[t] = vals[kcode] * ks.astype(np.float64)
                vf[t] = vals[vcode] * vs.astype(np.float64)
            self.kf.append(kf)
            self.vf.append(vf)
        self.ctx = np.asarray(self.lens, np.int32)

    def run(self, o):
        return o.decode_fp8(self.q, self.kc, self.vc, self.ks, self.vs, self.tables, self.ctx,
                            self.scale, self.qdtype)

    def sdpa(self):
        out = np.zeros((len(self.lens), self.Hq, self.d))
        qf = Case.f64(self, self.q)
        for s, n in enumerate(self.lens):
            if n == 0:
                continue
            q = torch.from_numpy(qf[s])[None, :, None, :]
            k = torch.from_numpy(self.kf[s]).permute(1, 0, 2)[None].contiguous()
            v = torch.from_numpy(self.vf[s]).permute(1, 0, 2)[None].contiguous()
            out[s] = F.scaled_dot_product_attention(q, k, v, scale=self.scale,
                                                    enable_gqa=self.Hq != self.Hkv)[0, :, 0, :].numpy()
        return out


def pin_fp8_sdpa(o):
    """Decode over E4M3 pools equals torch SDPA over the dequantised tokens (code value
    times the scale of the block and head holding it), in logical order."""
    rng = np.random.default_rng(121)
    for lens, Hq, Hkv, d, B, qdt in (([1, 5, 16, 33], 2, 2, 8, 4, "f16"),
                                     ([40, 7], 8, 2, 16, 8, "bf16"),
                                     ([0, 70], 4, 1, 32, 16, "f16")):
        c = Fp8Case(rng, lens, Hq, Hkv, d, B, qdt)
        got, want = c.run(o), c.sdpa()
        assert np.max(np.abs(got - want)) <= 1e-12, (lens, Hq, Hkv, d, B, qdt)


def pin_fp8_reshape(o):
    """The E4M3 scatter equals numpy fancy indexing of torch's clamped cast of
    x / scale (one float32 division) into the slots; untouched slots keep their bytes."""
    rng = np.random.default_rng(122)
    for dt, nb, H, B, d in (("f16", 6, 2, 4, 8), ("bf16", 5, 3, 8, 16), ("f32", 4, 1, 2, 4)):
        N = nb * B // 2
        slots = rng.choice(nb * B, size=N, replace=False).astype(np.int32)
        slots[::5] = -1
        key = W.round_to(rng.standard_normal((N, H, d), dtype=np.float32) * 8, dt)
        val = W.round_to(rng.standard_normal((N, H, d), dtype=np.float32) * 8, dt)
        key.reshape(-1)[:3] = W.round_to(np.array([1e4, -1e4, 0.0], np.float32), dt)
        ks = np.exp2(rng.uniform(-6, -2, (nb, H))).astype(np.float32)
        vs = np.exp2(rng.uniform(-6, -2, (nb, H))).astype(np.float32)
        kc = rng.integers(0, 256, (nb, H, B, d)).astype(np.uint8)
        vc = rng.integers(0, 256, (nb, H, B, d)).astype(np.uint8)
        wk, wv = kc.copy(), vc.copy()
        keep = slots >= 0
        tmp = Case.__new__(Case)
        tmp.dtype = dt
        for want, x, sc in ((wk, key, ks), (wv, val, vs)):
            xf = tmp.f64(x).astype(np.float32)  # exact: every source value fits
            for i in np.nonzero(keep)[0]:
                b, off = divmod(int(slots[i]), B)
                y = (torch.from_numpy(xf[i]) / torch.from_numpy(sc[b])[:, None]).numpy()
                want[b, :, off, :] = torch_fp8_encode(y)
        o.reshape_and_cache_fp8(key, val, kc, vc, ks, vs, slots, dt)
        assert kc.tobytes() == wk.tobytes() and vc.tobytes() == wv.tobytes(), dt


# ---------------------------------------------------------------------------
# several causal query tokens per sequence


class MQCase(Case):
    """A Case whose sequences also carry n_s query tokens (the last n_s positions)."""

    def __init__(self, rng, lens, qlens, Hq, Hkv, d, B, dtype, **kw):
        super().__init__(rng, lens, Hq, Hkv, d, B, dtype, **kw)
        self.qlens = [int(x) for x in qlens]
        assert all(0 <= a <= b for a, b in zip(self.qlens, self.lens))
        self.qstart = np.concatenate([[0], np.cumsum(self.qlens)]).astype(np.int32)
        T = int(self.qstart[-1])
        self.mq = W.round_to(rng.standard_normal((T, Hq, d), dtype=np.float32), dtype)

    def run_mq(self, o):
        return o.multi_query(self.mq, self.kc, self.vc, self.tables, self.ctx, self.qstart,
                             self.scale, self.dtype)

    def sdpa_mq(self):
        """torch SDPA (float64) with the causal mask t <= ctx - n_s + i, per sequence."""
        out = np.zeros((int(self.qstart[-1]), self.Hq, self.d))
        for s, (n, nq) in enumerate(zip(self.lens, self.qlens)):
            if nq == 0:
                continue
            a, b = int(self.qstart[s]), int(self.qstart[s + 1])
            q = torch.from_numpy(self.f64(self.mq[a:b])).permute(1, 0, 2)[None].contiguous()
            k = torch.from_numpy(self.f64(self.k[s])).permute(1, 0, 2)[None].contiguous()
            v = torch.from_numpy(self.f64(self.v[s])).permute(1, 0, 2)[None].contiguous()
            pos = torch.arange(n - nq, n)[:, None]
            mask = torch.arange(n)[None, :] <= pos
            o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=self.scale,
                                               enable_gqa=self.Hq != self.Hkv)
            out[a:b] = o[0].permute(1, 0, 2).numpy()
        return out


def pin_mq_sdpa(o):
    """Several query tokens per sequence equal torch SDPA with the causal mask over the
    logical tokens (query i of n sits at position ctx - n + i)."""
    rng = np.random.default_rng(130)
    for lens, qlens, Hq, Hkv, d, B, dt in (([1, 5, 17, 40], [1, 5, 3, 17], 2, 2, 8, 4, "f32"),
                                           ([33, 20], [33, 1], 8, 2, 16, 16, "bf16"),
                                           ([70, 9, 0], [24, 9, 0], 4, 1, 32, 8, "f16")):
        c = MQCase(rng, lens, qlens, Hq, Hkv, d, B, dt)
        got, want = c.run_mq(o), c.sdpa_mq()
        assert np.max(np.abs(got - want)) <= 1e-12, (lens, qlens, dt)


def pin_mq_causal(o):
    """A query token never sees later tokens: changing K and V after its position leaves
    its output bit-identical; a chunk covering the whole context starts with V(0)."""
    rng = np.random.default_rng(131)
    c = MQCase(rng, [30], [30], 2, 2, 8, 4, "f32")
    a = c.run_mq(o)
    assert np.array_equal(a[0], c.v[0][0].astype(np.float64))
    for cut in (5, 17):
        c.k[0][cut + 1:] = rng.standard_normal(c.k[0][cut + 1:].shape, dtype=np.float32)
        c.v[0][cut + 1:] = rng.standard_normal(c.v[0][cut + 1:].shape, dtype=np.float32)
        c._put(0, c.kc, c.k[0])
        c._put(0, c.vc, c.v[0])
        b = c.run_mq(o)
        assert np.array_equal(a[:cut + 1], b[:cut + 1]) and not np.array_equal(a[cut + 1:], b[cut + 1:])
        a = b


ORACLE_PINS = [pin_sdpa, pin_brute, pin_permutation, pin_ctx1, pin_equal_keys, pin_dominant,
               pin_shared_prefix, pin_nan_poison, pin_empty, pin_bad_index, pin_reshape, pin_copy,
               pin_swap,
               pin_page3_request, pin_dtype_decode, pin_fp8_codes, pin_fp8_encode, pin_fp8_sdpa,
               pin_fp8_reshape, pin_mq_sdpa, pin_mq_causal]
