"""Seeded synthetic inputs for paged decode attention.

This module is shared by the HIP path's tests and benchmark and by the oracle's
tests.  It holds none of the method's arithmetic: it draws context lengths, the
order in which physical blocks are handed out, the sequence of allocator
operations, and the query/key/value numbers of every token in logical (token)
order.  Where those tokens land in the block pools, which slots they get and how
attention is computed is left to each side (the HIP library with its allocator,
or the oracle with its model allocator).

Workloads (shapes and length mixes of the serving examples on the pages):
  - tiny_fp32       4 seqs, context lengths {1, 16, 17, 100}, 4 heads, d=64, B=16,
                    32-block pool.  The 100-token case is the worked example of
                    "PagedAttention 深度解析" (5ulink) §二 (7 blocks of 16).
  - llama7b         LLaMA-7B-shaped decode layer: 64 seqs, 32 heads MHA, d=128,
                    B=16, fp16, 40,000-block pool, lengths lognormal around 600.
  - llama13b_long   LLaMA-13B-shaped long context: 32 seqs, 40 heads, d=128, B=16,
                    bf16, 16,384 blocks, lengths uniform in [2048, 4096], 512-token
                    context partitions.
  - prefix_sharing  16 prompts x 5 samples: each group shares a 1024+r token prompt
                    (the last prompt block partly filled), then 0..256 private tokens
                    and the current one; 32 heads, d=128, B=16, fp16, 8,192 blocks.
  - llama70b_gqa    70B-shaped GQA: 32 seqs, 64 query / 8 KV heads, d=128, B=128,
                    bf16, 4,096 blocks, lengths uniform in [4096, 8192], balanced split
                    (partition_size -1).
  - llama7b_fp8     llama7b (same seed, lengths and numbers) with the pools held as
                    OCP E4M3 codes and one fp32 scale per (block, KV head) for K and
                    for V; query, new K/V and output stay fp16.
  - chunked_prefill LLaMA-7B-shaped chunked prefill: 16 seqs, 32 heads MHA, d=128,
                    B=16, fp16, 8,192 blocks; contexts uniform in [1024, 3072] whose
                    last 512 tokens are the chunk being prefilled (512 causal query
                    tokens per sequence over the cached prefix and the chunk).

Draw recipe (numpy PCG64):
  base stream  default_rng(seed): (1) length parameters, (2) free order =
               permutation(num_blocks) (arange for the identity layout).
  per sequence default_rng(SeedSequence([seed, 1, s])): q[H_q][d], then K of its
               tokens [n][H_kv][d], then V [n][H_kv][d] (prefix_sharing: the
               private tokens and the current one).
  per group    default_rng(SeedSequence([seed, 2, j])): K then V of the shared
               prompt (prefix_sharing only).
  values       standard_normal(float32) rounded to the storage type with
               round-to-nearest-even; bf16 is returned as raw uint16 bits.
  chunk query  default_rng(SeedSequence([seed, 4, s])): the query rows
               [query_len][H_q][d] of sequence s (chunked_prefill).
  E4M3 scales  default_rng(SeedSequence([seed, 3])): K scales then V scales,
               [num_blocks][H_kv] float32, each 2^u with u uniform in [-7, -5]
               (448 * scale spans 3.5 to 14 standard deviations of the values).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Tuple

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str
    partition_size: int  # 0: one pass over the whole context; -1: balanced split
    lengths: str  # "fixed" | "lognormal" | "uniform" | "prefix"
    fixed_lengths: Tuple[int, ...] = ()
    low: int = 0  # uniform: inclusive bounds
    high: int = 0
    groups: int = 0  # prefix: number of prompts
    samples: int = 0  # prefix: samples per prompt
    prefix_base: int = 0  # prefix: shared prompt = prefix_base + U{1..block_size-1}
    private_max: int = 0  # prefix: private tokens U{0..private_max}
    kv_dtype: str = ""  # pool storage type; "" = the query's type, "fp8" = E4M3 codes
    query_len: int = 0  # > 0: that many causal query tokens per sequence (chunked prefill)

    @property
    def scale(self) -> float:
        """1/sqrt(head_dim), as the fp32 value every side receives."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def kv(self) -> str:
        """Storage type of the K/V pools."""
        return self.kv_dtype or self.dtype

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.kv == "fp8" else self.elem_bytes


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", 1, 4, 4, 4, 64, 16, 32, "f32", 0, "fixed",
                          fixed_lengths=(1, 16, 17, 100)),
    "llama7b": Workload("llama7b", 2, 64, 32, 32, 128, 16, 40000, "f16", 0, "lognormal"),
    "llama13b_long": Workload("llama13b_long", 3, 32, 40, 40, 128, 16, 16384, "bf16", 512,
                              "uniform", low=2048, high=4096),
    "prefix_sharing": Workload("prefix_sharing", 4, 80, 32, 32, 128, 16, 8192, "f16", 512,
                               "prefix", groups=16, samples=5, prefix_base=1024,
                               private_max=256),
    "llama70b_gqa": Workload("llama70b_gqa", 5, 32, 64, 8, 128, 128, 4096, "bf16", -1,
                             "uniform", low=4096, high=8192),
    "llama7b_fp8": Workload("llama7b_fp8", 2, 64, 32, 32, 128, 16, 40000, "f16", 0, "lognormal",
                            kv_dtype="fp8"),
    "chunked_prefill": Workload("chunked_prefill", 6, 16, 32, 32, 128, 16, 8192, "f16", 0, "uniform",
                                low=1024, high=3072, query_len=512),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of `w` with some fields changed (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


# ---------------------------------------------------------------------------
# storage types


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 numbers to the storage type (RNE). bf16 -> uint16 bits."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return rounded.astype(np.uint16)
    raise ValueError(dtype)


def nan_bits(dtype: str):
    """A quiet NaN in the storage representation (for poisoning unused slots)."""
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0),
            "fp8": np.uint8(0x7F)}[dtype]


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}[dtype]


def fp8_scales(w: Workload):
    """K and V scales [num_blocks][H_kv] float32 of an E4M3 workload."""
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 3]))
    shape = (w.num_blocks, w.num_kv_heads)
    ks = np.exp2(rng.uniform(-7.0, -5.0, shape)).astype(np.float32)
    vs = np.exp2(rng.uniform(-7.0, -5.0, shape)).astype(np.float32)
    return ks, vs


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return round_to(rng.standard_normal(shape, dtype=np.float32), dtype)


# ---------------------------------------------------------------------------
# lengths, free order and the allocator script


@dataclasses.dataclass
class Lengths:
    context_lens: np.ndarray  # int32 [S], including the current token
    prefix_lens: np.ndarray  # int32 [groups] (prefix workloads), else empty
    private_lens: np.ndarray  # int32 [S] private tokens before the current one


def draw_lengths(w: Workload) -> Tuple[Lengths, np.random.Generator]:
    rng = np.random.default_rng(w.seed)
    empty = np.zeros(0, np.int32)
    if w.lengths == "fixed":
        ctx = np.asarray(w.fixed_lengths, np.int32)
        return Lengths(ctx, empty, np.zeros(len(ctx), np.int32)), rng
    if w.lengths == "lognormal":
        raw = rng.lognormal(mean=math.log(600.0), sigma=0.6, size=w.num_seqs)
        ctx = np.clip(np.rint(raw), 32, 2048).astype(np.int32)
        return Lengths(ctx, empty, np.zeros(w.num_seqs, np.int32)), rng
    if w.lengths == "uniform":
        ctx = rng.integers(w.low, w.high + 1, size=w.num_seqs).astype(np.int32)
        return Lengths(ctx, empty, np.zeros(w.num_seqs, np.int32)), rng
    if w.lengths == "prefix":
        r = rng.integers(1, w.block_size, size=w.groups)
        p = rng.integers(0, w.private_max + 1, size=w.groups * w.samples)
        prefix = (w.prefix_base + r).astype(np.int32)
        ctx = (np.repeat(prefix, w.samples) + p + 1).astype(np.int32)
        return Lengths(ctx, prefix, p.astype(np.int32)), rng
    raise ValueError(w.lengths)


def free_order(w: Workload, rng: np.random.Generator, identity: bool = False) -> np.ndarray:
    """Order in which the allocator hands out physical blocks."""
    perm = rng.permutation(w.num_blocks).astype(np.int32)
    if identity:
        return np.arange(w.num_blocks, dtype=np.int32)
    return perm


@dataclasses.dataclass
class Op:
    """One allocator operation: ('new', seq) | ('append', seq, n) | ('fork', parent, seq)."""
    kind: str
    seq: int
    arg: int = 0


def alloc_script(w: Workload, lengths: Lengths) -> List[Op]:
    """Operations that build the batch; `seq` numbers are 0..S-1 in batch order.

    Plain workloads: every sequence is created and its tokens appended one by one.
    prefix_sharing: per group, the first sample is created and the prompt appended,
    it is forked samples-1 times, then each sample (in order) appends its private
    tokens and its current token.
    """
    ops: List[Op] = []
    if w.lengths != "prefix":
        for s, n in enumerate(lengths.context_lens.tolist()):
            ops.append(Op("new", s))
            ops.append(Op("append", s, n))
        return ops
    for j in range(w.groups):
        first = j * w.samples
        ops.append(Op("new", first))
        ops.append(Op("append", first, int(lengths.prefix_lens[j])))
        for c in range(1, w.samples):
            ops.append(Op("fork", first, first + c))
        for c in range(w.samples):
            s = first + c
            ops.append(Op("append", s, int(lengths.private_lens[s]) + 1))
    return ops


# ---------------------------------------------------------------------------
# values


def seq_values(w: Workload, s: int, n_tokens: int):
    """q [H_q][d] and K, V [n_tokens][H_kv][d] of sequence s (storage type).

    For prefix_sharing, n_tokens counts the private tokens plus the current one.
    """
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 1, s]))
    q = _normal(rng, (w.num_q_heads, w.head_dim), w.dtype)
    k = _normal(rng, (n_tokens, w.num_kv_heads, w.head_dim), w.dtype)
    v = _normal(rng, (n_tokens, w.num_kv_heads, w.head_dim), w.dtype)
    return q, k, v


def group_prefix_values(w: Workload, j: int, n_tokens: int):
    """K, V [n_tokens][H_kv][d] of the shared prompt of group j."""
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 2, j]))
    k = _normal(rng, (n_tokens, w.num_kv_heads, w.head_dim), w.dtype)
    v = _normal(rng, (n_tokens, w.num_kv_heads, w.head_dim), w.dtype)
    return k, v


def chunk_queries(w: Workload, s: int, n: int) -> np.ndarray:
    """Query rows [n][H_q][d] of sequence s's chunk (storage type)."""
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 4, s]))
    return _normal(rng, (n, w.num_q_heads, w.head_dim), w.dtype)


@dataclasses.dataclass
class Batch:
    """All numbers of one workload, in logical order (no placement)."""
    workload: Workload
    lengths: Lengths
    free_order: np.ndarray
    script: List[Op]
    q: np.ndarray  # [S][H_q][d]
    # token values in the order the script appends them: one entry per append op,
    # each [n][H_kv][d]
    append_k: List[np.ndarray]
    append_v: List[np.ndarray]

    @property
    def fp8_scales(self):
        """K and V block scales of an E4M3 workload."""
        return fp8_scales(self.workload)


def make_batch(w: Workload, identity: bool = False, seqs=None) -> Batch:
    """Draw a whole batch.  `seqs` (plain workloads only) keeps just those
    sequences (their lengths and values are the same as in the full batch)."""
    lengths, rng = draw_lengths(w)
    order = free_order(w, rng, identity)
    if seqs is not None:
        if w.lengths == "prefix":
            raise ValueError("sub-batches are for plain workloads")
        seqs = [int(s) for s in seqs]
        lengths = Lengths(lengths.context_lens[seqs].copy(), lengths.prefix_lens,
                          lengths.private_lens[seqs].copy())
    else:
        seqs = list(range(len(lengths.context_lens)))
    sub = dataclasses.replace(w, num_seqs=len(seqs))
    script = alloc_script(sub, lengths)
    q = np.zeros((len(seqs), w.num_q_heads, w.head_dim), storage_np_dtype(w.dtype))
    ak: List[np.ndarray] = []
    av: List[np.ndarray] = []
    if w.lengths != "prefix":
        for i, s in enumerate(seqs):
            q[i], k, v = seq_values(w, s, int(lengths.context_lens[i]))
            ak.append(k)
            av.append(v)
    else:
        # per sequence: the first append of a group's first sample is the shared
        # prompt; every other append is a sample's private tokens + current token
        seen = set()
        for op in script:
            if op.kind != "append":
                continue
            j, c = divmod(op.seq, w.samples)
            if c == 0 and op.seq not in seen:
                k, v = group_prefix_values(w, j, op.arg)
            else:
                q[op.seq], k, v = seq_values(w, op.seq, op.arg)
            seen.add(op.seq)
            ak.append(k)
            av.append(v)
    return Batch(sub, lengths, order, script, q, ak, av)
