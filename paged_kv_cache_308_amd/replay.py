"""Build a decode batch on the device by replaying an allocator script.

The script is a list of operations ('new', seq) / ('fork', parent, child) /
('append', seq, n) and every append carries the K/V of its n tokens.  Placement
order: prompts; then the copy-on-write copies the appends raised; then every
sequence's later tokens except its newest one.  The newest tokens are what a
decode step writes (DeviceBatch.step).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

from . import PA_DECODE_SHARED_KV, PA_VARIANT_AUTO, pa_decode_grouped, pa_decode_grouped_workspace_bytes
from .engine import TORCH_DTYPE, PagedKVCache, prefix_groups, to_torch


@dataclasses.dataclass
class DeviceBatch:
    cache: PagedKVCache
    query: torch.Tensor  # [S][H_q][d]
    new_key: torch.Tensor  # [S][H_kv][d]
    new_value: torch.Tensor
    slot_mapping: torch.Tensor  # int32 [S]: newest token of each sequence
    block_tables: torch.Tensor  # int32 [S][max_blocks]
    context_lens: torch.Tensor  # int32 [S]
    cow_src: np.ndarray
    cow_dst: np.ndarray
    host_tables: np.ndarray
    host_context_lens: np.ndarray
    max_context_len: int
    scale: float
    shared: bool = False  # tables share physical blocks: pass the cache hint
    seq_ids: Optional[List[int]] = None  # allocator id of each batch sequence

    def step(self, partition_size: int = 0, variant: int = PA_VARIANT_AUTO, out=None,
             workspace=None, stream=None, fused: bool = True) -> torch.Tensor:
        """The decode step: newest K/V into their slots, then attention (one launch when
        the vector kernel serves it and `fused`)."""
        if self.shared:
            variant |= PA_DECODE_SHARED_KV
        if fused:
            return self.cache.step(self.query, self.new_key, self.new_value, self.slot_mapping,
                                   self.block_tables, self.context_lens, self.scale, out=out,
                                   partition_size=partition_size,
                                   max_context_len=self.max_context_len, variant=variant,
                                   workspace=workspace, stream=stream)
        self.cache.write(self.new_key, self.new_value, self.slot_mapping, stream)
        return self.attend(partition_size, variant & ~PA_DECODE_SHARED_KV, out, workspace, stream)

    def groups(self, partition_size: int):
        """Shared-prefix groups of the batch (host tables) as device arrays, with the
        largest group and the most shared partitions, for step_grouped."""
        gs, gp, gmax, pmax = prefix_groups(self.host_tables, self.host_context_lens, self.cache.block_size,
                                           partition_size)
        dev = self.block_tables.device
        return torch.from_numpy(gs).to(dev), torch.from_numpy(gp).to(dev), gmax, pmax

    def grouped_workspace(self, partition_size: int) -> torch.Tensor:
        n = pa_decode_grouped_workspace_bytes(self.query.shape[0], self.query.shape[1], self.cache.num_kv_heads,
                                              self.cache.head_dim, self.max_context_len, partition_size)
        return torch.empty(n, dtype=torch.uint8, device=self.block_tables.device)

    def step_grouped(self, partition_size: int, groups, out=None, workspace=None, stream=None,
                     variant: int = PA_VARIANT_AUTO) -> torch.Tensor:
        """The decode step over shared-prefix groups (pa_decode_grouped): the newest
        K/V stored, shared partitions read once per group."""
        gs, gp, gmax, pmax = groups
        out = torch.empty_like(self.query) if out is None else out
        return pa_decode_grouped(out, self.query, self.cache.key_cache, self.cache.value_cache, self.block_tables,
                                 self.context_lens, self.scale, gs, gp, gmax, pmax, self.max_context_len,
                                 partition_size, new_key=self.new_key, new_value=self.new_value,
                                 variant=variant, workspace=workspace, stream=stream)

    def attend(self, partition_size: int = 0, variant: int = PA_VARIANT_AUTO, out=None,
               workspace=None, stream=None) -> torch.Tensor:
        if self.shared:
            variant |= PA_DECODE_SHARED_KV
        return self.cache.attend(self.query, self.block_tables, self.context_lens, self.scale,
                                 out=out, partition_size=partition_size,
                                 max_context_len=self.max_context_len, variant=variant,
                                 workspace=workspace, stream=stream)


def replay(batch, poison: bool = True, device="cuda",
           num_blocks: Optional[int] = None) -> DeviceBatch:
    """`batch` carries .workload (sizes), .free_order, .script, .q, .append_k, .append_v
    (and .fp8_scales, the K and V block scales, when the workload's pools are E4M3)."""
    w = batch.workload
    kv = getattr(w, "kv", w.dtype)
    cache = PagedKVCache(num_blocks or w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                         TORCH_DTYPE[kv], device, fill=float("nan") if poison else 0.0)
    if kv == "fp8":
        ks, vs = batch.fp8_scales
        cache.k_scales.copy_(torch.from_numpy(ks[:cache.num_blocks]))
        cache.v_scales.copy_(torch.from_numpy(vs[:cache.num_blocks]))
    cache.set_free_order(batch.free_order)
    ids = {}
    slots: List[np.ndarray] = []
    src, dst = [], []
    for op in batch.script:
        if op.kind == "new":
            ids[op.seq] = cache.new_seq()
        elif op.kind == "fork":
            ids[op.arg] = cache.fork(ids[op.seq])
        else:
            s, cs, cd = cache.reserve([ids[op.seq]] * op.arg)
            slots.append(s)
            src += cs.tolist()
            dst += cd.tolist()
    appends = [op for op in batch.script if op.kind == "append"]
    last = {}
    for i, op in enumerate(appends):
        last[op.seq] = i

    def dev(a):
        return to_torch(a, w.dtype).to(device)

    for i, op in enumerate(appends):
        if last[op.seq] != i:
            cache.write(dev(batch.append_k[i]), dev(batch.append_v[i]), slots[i])
    cow_src = np.asarray(src, np.int32)
    cow_dst = np.asarray(dst, np.int32)
    cache.copy(cow_src, cow_dst)
    S = w.num_seqs
    newest = np.empty(S, np.int32)
    nk = np.empty((S, w.num_kv_heads, w.head_dim), batch.append_k[0].dtype)
    nv = np.empty_like(nk)
    for seq, i in last.items():
        if appends[i].arg > 1:
            cache.write(dev(batch.append_k[i][:-1]), dev(batch.append_v[i][:-1]), slots[i][:-1])
        newest[seq] = slots[i][-1]
        nk[seq] = batch.append_k[i][-1]
        nv[seq] = batch.append_v[i][-1]
    seq_ids = [ids[s] for s in range(S)]
    bt, cl = cache.tables(seq_ids)
    return DeviceBatch(cache, dev(batch.q), dev(nk), dev(nv), cache.upload(newest),
                       cache.upload(bt), cache.upload(cl), cow_src, cow_dst, bt, cl,
                       int(cl.max()) if S else 0, w.scale,
                       cache.alloc.stats()["shared_blocks"] > 0, seq_ids)
