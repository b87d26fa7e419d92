"""Build pools and tables for a workload batch on the oracle side (TEST INFRASTRUCTURE).

Replays the batch's allocator script on the model allocator, scatters every
token with the oracle's reshape_and_cache (reshape_and_cache_fp8 for E4M3 pools),
applies the copy-on-write pairs with the oracle's copy_blocks (E4M3 blocks take
their scales along), and returns everything the oracle's decode needs.
Step order (the decode step of the KV-cache/paging tutorial (wmrh.cn): only the
newest token's K/V are written, then attention runs over all cached tokens):
  1. earlier tokens of every sequence are placed (prompt, then private tokens,
     after the copy-on-write copies they triggered);
  2. the decode step: copy-on-write copies, then the newest token's K/V, then
     attention.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

import workloads as W
from . import default as _default_oracle
from .alloc_model import ModelAllocator


@dataclasses.dataclass
class Placed:
    key_cache: np.ndarray
    value_cache: np.ndarray
    block_tables: np.ndarray  # int32 [S][max_blocks], padded with -1
    context_lens: np.ndarray  # int32 [S]
    slot_mapping: np.ndarray  # int32 [S]: slot of each sequence's newest token
    new_key: np.ndarray  # [S][H_kv][d]
    new_value: np.ndarray
    cow_src: np.ndarray  # int32: copy-on-write pairs in the order they arose
    cow_dst: np.ndarray
    alloc: ModelAllocator
    k_scales: Optional[np.ndarray] = None  # E4M3 pools: float32 [num_blocks][H_kv]
    v_scales: Optional[np.ndarray] = None

    def write(self, key, value, slots, src_dtype: str) -> None:
        """Scatter tokens (src_dtype) into the pools with the oracle's scatter."""
        o = _default_oracle()
        if self.k_scales is None:
            o.reshape_and_cache(key, value, self.key_cache, self.value_cache, slots, src_dtype)
        else:
            o.reshape_and_cache_fp8(key, value, self.key_cache, self.value_cache, self.k_scales,
                                    self.v_scales, slots, src_dtype)

    def copy(self, src, dst, kv_dtype: str) -> None:
        """Whole-block copies; E4M3 blocks take their scales along."""
        o = _default_oracle()
        o.copy_blocks(self.key_cache, self.value_cache, src, dst, kv_dtype)
        if self.k_scales is not None:
            nb, H = self.k_scales.shape
            o.copy_blocks(self.k_scales.reshape(nb, H, 1, 1), self.v_scales.reshape(nb, H, 1, 1),
                          src, dst, "f32")


def replay(batch: W.Batch):
    """Run the allocator script.
    Returns (allocator, batch seq -> allocator id, per-append slot arrays, cow pairs)."""
    w = batch.workload
    a = ModelAllocator(w.num_blocks, w.block_size)
    a.set_free_order(batch.free_order)
    sids = {}
    slots: List[np.ndarray] = []
    cow: List[tuple] = []
    for op in batch.script:
        if op.kind == "new":
            sids[op.seq] = a.new_seq()
        elif op.kind == "fork":
            sids[op.arg] = a.fork(sids[op.seq])
        else:
            s = np.empty(op.arg, np.int32)
            for i in range(op.arg):
                slot, c = a.append_slot(sids[op.seq])
                s[i] = slot
                if c is not None:
                    cow.append(c)
            slots.append(s)
    return a, sids, slots, cow


def place(batch: W.Batch, poison: bool = True, fp8_scales=None) -> Placed:
    """Pools with every token placed except each sequence's newest one.  E4M3 pools take
    the workload's block scales unless `fp8_scales` = (k, v) [num_blocks][H_kv] is given."""
    w = batch.workload
    a, sids, slots, cow = replay(batch)
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    npd = W.storage_np_dtype(w.kv)
    fill = W.nan_bits(w.kv) if poison else npd(0)
    S = w.num_seqs
    if cow:
        src = np.array([c[0] for c in cow], np.int32)
        dst = np.array([c[1] for c in cow], np.int32)
    else:
        src = np.zeros(0, np.int32)
        dst = np.zeros(0, np.int32)
    qnp = W.storage_np_dtype(w.dtype)
    newest_slot = np.full(S, -1, np.int32)
    newest_k = np.zeros((S, w.num_kv_heads, w.head_dim), qnp)
    newest_v = np.zeros_like(newest_k)
    p = Placed(np.full(shape, fill, dtype=npd), np.full(shape, fill, dtype=npd), None, None,
               newest_slot, newest_k, newest_v, src, dst, a)
    if w.kv == "fp8":
        ks, vs = fp8_scales if fp8_scales is not None else W.fp8_scales(w)
        p.k_scales = np.array(ks, np.float32)
        p.v_scales = np.array(vs, np.float32)
    appends = [op for op in batch.script if op.kind == "append"]
    # prompts first; then the copy-on-write copies; then each sequence's private
    # tokens (all of its last append but the newest token)
    last_append_of = {}
    for i, op in enumerate(appends):
        last_append_of[op.seq] = i
    prompt_like = [i for i, op in enumerate(appends) if last_append_of[op.seq] != i]
    for i in prompt_like:
        p.write(batch.append_k[i], batch.append_v[i], slots[i], w.dtype)
    p.copy(src, dst, w.kv)
    for seq, i in last_append_of.items():
        n = appends[i].arg
        if n > 1:
            p.write(batch.append_k[i][:-1], batch.append_v[i][:-1], slots[i][:-1], w.dtype)
        newest_slot[seq] = slots[i][-1]
        newest_k[seq] = batch.append_k[i][-1]
        newest_v[seq] = batch.append_v[i][-1]
    max_blocks = max(1, max(len(a.block_table(sids[s])[0]) for s in range(S))) if S else 1
    bt = np.full((S, max_blocks), -1, np.int32)
    cl = np.zeros(S, np.int32)
    for s in range(S):
        t, n = a.block_table(sids[s])
        bt[s, :len(t)] = t
        cl[s] = n
    p.block_tables, p.context_lens = bt, cl
    return p


def decode_step(batch: W.Batch, placed: Optional[Placed] = None, poison: bool = True,
                fp8_scales=None):
    """The oracle's decode step: scatter the newest tokens, then attention.
    Returns (out float64 [S][H_q][d], placed)."""
    o = _default_oracle()
    w = batch.workload
    p = placed or place(batch, poison, fp8_scales)
    p.write(p.new_key, p.new_value, p.slot_mapping, w.dtype)
    if p.k_scales is None:
        out = o.decode(batch.q, p.key_cache, p.value_cache, p.block_tables, p.context_lens,
                       w.scale, w.dtype)
    else:
        out = o.decode_fp8(batch.q, p.key_cache, p.value_cache, p.k_scales, p.v_scales,
                           p.block_tables, p.context_lens, w.scale, w.dtype)
    return out, p
