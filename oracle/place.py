"""Build pools and tables for a workload batch on the oracle side (TEST INFRASTRUCTURE).

Replays the batch's allocator script on the model allocator, scatters every
token with the oracle's reshape_and_cache, applies the copy-on-write pairs with
the oracle's copy_blocks, and returns everything the oracle's decode needs.
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


def place(batch: W.Batch, poison: bool = True) -> Placed:
    """Pools with every token placed except each sequence's newest one."""
    o = _default_oracle()
    w = batch.workload
    a, sids, slots, cow = replay(batch)
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    npd = W.storage_np_dtype(w.dtype)
    fill = W.nan_bits(w.dtype) if poison else npd(0)
    kc = np.full(shape, fill, dtype=npd)
    vc = np.full(shape, fill, dtype=npd)
    S = w.num_seqs
    newest_slot = np.full(S, -1, np.int32)
    newest_k = np.zeros((S, w.num_kv_heads, w.head_dim), npd)
    newest_v = np.zeros_like(newest_k)
    appends = [op for op in batch.script if op.kind == "append"]
    # prompts first; then the copy-on-write copies; then each sequence's private
    # tokens (all of its last append but the newest token)
    last_append_of = {}
    for i, op in enumerate(appends):
        last_append_of[op.seq] = i
    prompt_like = [i for i, op in enumerate(appends) if last_append_of[op.seq] != i]
    for i in prompt_like:
        o.reshape_and_cache(batch.append_k[i], batch.append_v[i], kc, vc, slots[i], w.dtype)
    if cow:
        src = np.array([c[0] for c in cow], np.int32)
        dst = np.array([c[1] for c in cow], np.int32)
    else:
        src = np.zeros(0, np.int32)
        dst = np.zeros(0, np.int32)
    o.copy_blocks(kc, vc, src, dst, w.dtype)
    for seq, i in last_append_of.items():
        n = appends[i].arg
        if n > 1:
            o.reshape_and_cache(batch.append_k[i][:-1], batch.append_v[i][:-1], kc, vc,
                                slots[i][:-1], w.dtype)
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
    return Placed(kc, vc, bt, cl, newest_slot, newest_k, newest_v, src, dst, a)


def decode_step(batch: W.Batch, placed: Optional[Placed] = None, poison: bool = True):
    """The oracle's decode step: scatter the newest tokens, then attention.
    Returns (out float64 [S][H_q][d], placed)."""
    o = _default_oracle()
    w = batch.workload
    p = placed or place(batch, poison)
    o.reshape_and_cache(p.new_key, p.new_value, p.key_cache, p.value_cache, p.slot_mapping, w.dtype)
    out = o.decode(batch.q, p.key_cache, p.value_cache, p.block_tables, p.context_lens,
                   w.scale, w.dtype)
    return out, p
