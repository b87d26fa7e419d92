"""Paged KV cache: device block pools plus the host allocator, driving libpa.

One decode step, in stream order ("vLLM PagedAttention 技术深度解析" (kwkr.cn)
§1.2.2 allocation flow; "PagedAttention" concept report (compassingai.com) §6
copy-on-write, §8 attention over the block table; the KV-cache tutorial
(wmrh.cn): only the newest token's K/V are computed at a step):
  1. host: reserve a slot for every sequence's new token (a new block when the
     last one is full, a copy-on-write pair when it is shared);
  2. host -> device: the step's slots, tables and lengths;
  3. device: pa_copy_blocks for the pairs, pa_reshape_and_cache for the new K/V,
     pa_decode over the tables.
Python only marshals arguments and keeps host bookkeeping; all device work runs in
libpa's kernels on the caller's stream.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import (PA_VARIANT_AUTO, PA_VARIANT_MFMA, PA_VARIANT_VALU, Allocator, pa_copy_blocks,
               pa_decode, pa_decode_append, pa_decode_fp8, pa_decode_workspace_bytes,
               pa_reshape_and_cache, pa_reshape_and_cache_fp8, pa_swap_blocks)

FP8_NAN_CODE = 0x7F


def _scale_pools(k_scales: torch.Tensor, v_scales: torch.Tensor):
    """[num_blocks][H_kv] scale arrays viewed as pools of 1x1 float32 blocks, so the block
    copy and swap calls move a block's scales with it."""
    nb, h = k_scales.shape
    return k_scales.view(nb, h, 1, 1), v_scales.view(nb, h, 1, 1)


def prefix_groups(host_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                  partition_size: int, max_group_size: int = 16):
    """Shared-prefix groups for pa_decode_grouped, from the step's host tables: runs of
    consecutive sequences whose tables start with the same block ids ("PagedAttention"
    concept report (compassingai.com) §6: forked sequences hold their prompt's blocks).
    A sequence joins the current group when it shares at least one whole partition with
    the group's first sequence; the group's shared partitions are the fewest any member
    has (shared leading blocks, ending before each member's newest token).  Returns
    (group_start int32 [G + 1], group_parts int32 [G], largest group size, largest
    group_parts).  Host bookkeeping only: the device re-checks every member."""
    S = len(context_lens)
    bpp = partition_size // block_size
    ctx = np.asarray(context_lens, np.int64)

    def own_parts(s):  # partitions wholly before the newest token
        return max(0, int(ctx[s] - 1)) // partition_size

    def common_parts(a, b):
        n = min(own_parts(a), own_parts(b)) * bpp
        if n == 0:
            return 0
        eq = host_tables[a, :n] == host_tables[b, :n]
        k = n if eq.all() else int(np.argmin(eq))
        return k // bpp

    starts, parts = [0], []
    i = 0
    while i < S:
        g = own_parts(i)
        j = i + 1
        while j < S and j - i < max_group_size:
            c = common_parts(i, j)
            if c < 1:
                break
            g = min(g, c)
            j += 1
        if j - i == 1:
            g = 0
        parts.append(g)
        starts.append(j)
        i = j
    start = np.asarray(starts, np.int32)
    gp = np.asarray(parts, np.int32)
    return start, gp, int(np.max(np.diff(start))) if S else 1, int(gp.max()) if len(gp) else 0


class StepUploader:
    """Host -> device upload of a decode step's index data: the newest tokens' slots
    (int32 [S]), the block tables (int32 [S][max_blocks]) and the context lengths
    (int32 [S]) ("PagedAttention" concept report (compassingai.com) §5: the tables are
    plain integer arrays handed to the kernel).

    The arrays are packed into one pinned host staging buffer and copied into one device
    buffer with a single asynchronous copy on the caller's stream, so the step's kernels,
    queued after it on that stream, see them without a host synchronisation.  `depth`
    stagings (pinned and device) are used in turn; before a staging is packed again the
    host waits for the event recorded after its previous copy, so a copy still in flight
    never reads a half-written staging, and the device views a call returned stay valid
    until `depth` - 1 further uploads have been made.  Buffers are allocated once, for
    up to max_seqs sequences of max_blocks_per_seq table entries."""

    def __init__(self, max_seqs: int, max_blocks_per_seq: int, device="cuda", depth: int = 2):
        import torch as _t
        self.max_seqs, self.max_blocks = int(max_seqs), int(max_blocks_per_seq)
        n = 2 * self.max_seqs + self.max_seqs * self.max_blocks
        self._host = [_t.empty(n, dtype=_t.int32, pin_memory=True) for _ in range(depth)]
        self._dev = [_t.empty(n, dtype=_t.int32, device=device) for _ in range(depth)]
        self._done = [None] * depth
        self._next = 0

    def upload(self, slots, block_tables, context_lens, stream=None):
        """Returns device int32 views (slots [S], block_tables [S][mb], context_lens [S])
        whose contents arrive in stream order."""
        import torch as _t
        tb = np.asarray(block_tables, np.int32)
        S, mb = tb.shape
        if S > self.max_seqs or mb > self.max_blocks:
            raise ValueError(f"{S} sequences of {mb} blocks exceed the uploader's {self.max_seqs} x {self.max_blocks}")
        st = stream if stream is not None else _t.cuda.current_stream()
        i = self._next
        self._next = (i + 1) % len(self._host)
        if self._done[i] is not None:
            self._done[i].synchronize()  # the staging's previous copy has read it
        h = self._host[i].numpy()
        n = 2 * S + S * mb
        h[:S] = np.asarray(slots, np.int32)
        h[S:2 * S] = np.asarray(context_lens, np.int32)
        h[2 * S:n] = tb.reshape(-1)
        d = self._dev[i]
        with _t.cuda.stream(st):
            d[:n].copy_(self._host[i][:n], non_blocking=True)
            ev = _t.cuda.Event()
            ev.record(st)
        self._done[i] = ev
        return d[:S], d[2 * S:n].view(S, mb), d[S:2 * S]


class PagedKVCache:
    """Device K/V pools of one layer and the host allocator.  dtype=torch.uint8 holds
    E4M3 codes, with k_scales / v_scales float32 [num_blocks][H_kv] (one per block and
    KV head, set by the owner before a block's first write; default 1)."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                 dtype: torch.dtype, device="cuda", fill: Optional[float] = None):
        self.num_blocks, self.num_kv_heads = num_blocks, num_kv_heads
        self.head_dim, self.block_size, self.dtype = head_dim, block_size, dtype
        self.fp8 = dtype == torch.uint8
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.key_cache = torch.empty(shape, dtype=dtype, device=device)
        self.value_cache = torch.empty(shape, dtype=dtype, device=device)
        if fill is not None:
            if self.fp8:  # NaN poison is the NaN code; any other fill is zero
                fill = FP8_NAN_CODE if fill != fill else 0
            self.key_cache.fill_(fill)
            self.value_cache.fill_(fill)
        self.k_scales = self.v_scales = None
        if self.fp8:
            self.k_scales = torch.ones((num_blocks, num_kv_heads), dtype=torch.float32, device=device)
            self.v_scales = torch.ones_like(self.k_scales)
        self.alloc = Allocator(num_blocks, block_size)
        self.device = torch.device(device)

    # host allocator -------------------------------------------------------
    def set_free_order(self, ids: Sequence[int]) -> None:
        self.alloc.set_free_order(ids)

    def new_seq(self) -> int:
        return self.alloc.new_seq()

    def fork(self, parent: int) -> int:
        return self.alloc.fork(parent)

    def free_seq(self, seq: int) -> None:
        self.alloc.free_seq(seq)

    def reserve(self, seqs: Sequence[int]):
        """One new token per entry of `seqs` (in order).
        Returns (slots, cow_src, cow_dst) as int32 numpy arrays."""
        return self.alloc.append_slots(seqs)

    def tables(self, seqs: Sequence[int], max_blocks_per_seq: Optional[int] = None):
        if max_blocks_per_seq is None:
            max_blocks_per_seq = max(1, max(len(self.alloc.block_table(s)[0]) for s in seqs))
        return self.alloc.block_tables(seqs, max_blocks_per_seq)

    # device ----------------------------------------------------------------
    def upload(self, a: np.ndarray) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.device, non_blocking=False)

    def copy(self, cow_src, cow_dst, stream=None) -> None:
        if len(cow_src):
            src, dst = _as_dev(cow_src, self.device), _as_dev(cow_dst, self.device)
            pa_copy_blocks(self.key_cache, self.value_cache, src, dst, stream)
            if self.fp8:
                pa_copy_blocks(*_scale_pools(self.k_scales, self.v_scales), src, dst, stream)

    def write(self, key: torch.Tensor, value: torch.Tensor, slots, stream=None) -> None:
        if self.fp8:
            pa_reshape_and_cache_fp8(key, value, self.key_cache, self.value_cache, self.k_scales,
                                     self.v_scales, _as_dev(slots, self.device), stream)
        else:
            pa_reshape_and_cache(key, value, self.key_cache, self.value_cache,
                                 _as_dev(slots, self.device), stream)

    def workspace(self, num_seqs: int, num_q_heads: int, max_context_len: int,
                  partition_size: int) -> Optional[torch.Tensor]:
        n = pa_decode_workspace_bytes(num_seqs, num_q_heads, self.num_kv_heads, self.head_dim,
                                      max_context_len, partition_size)
        return torch.empty(n, dtype=torch.uint8, device=self.device) if n else None

    def attend(self, query, block_tables, context_lens, scale: float, out=None,
               partition_size: int = 0, max_context_len: int = 0, variant: int = PA_VARIANT_AUTO,
               workspace=None, stream=None) -> torch.Tensor:
        out = torch.empty_like(query) if out is None else out
        if partition_size and workspace is None:
            workspace = self.workspace(query.shape[0], query.shape[1], max_context_len,
                                       partition_size)
        if self.fp8:
            pa_decode_fp8(out, query, self.key_cache, self.value_cache, self.k_scales,
                          self.v_scales, block_tables, context_lens, scale,
                          max_context_len=max_context_len, partition_size=partition_size,
                          variant=variant, workspace=workspace, stream=stream)
        else:
            pa_decode(out, query, self.key_cache, self.value_cache, block_tables, context_lens,
                      scale, max_context_len=max_context_len, partition_size=partition_size,
                      variant=variant, workspace=workspace, stream=stream)
        return out


    def fused_step_ok(self, num_q_heads: int, partition_size: int, variant: int) -> bool:
        """Whether the newest-token store can ride in the attention launch: every kernel
        form but the vector kernel's balanced split (the matrix-core kernels serve 16-bit
        grouped heads under AUTO, or PA_VARIANT_MFMA)."""
        choice = variant & 15
        mfma = choice == PA_VARIANT_MFMA or (
            choice == PA_VARIANT_AUTO and not self.fp8 and self.dtype != torch.float32
            and num_q_heads > self.num_kv_heads)
        return partition_size >= 0 or mfma

    def step(self, query, new_key, new_value, slots, block_tables, context_lens, scale: float,
             out=None, partition_size: int = 0, max_context_len: int = 0,
             variant: int = PA_VARIANT_AUTO, workspace=None, stream=None) -> torch.Tensor:
        """The decode step: the newest K/V into their slots (position ctx - 1 of each
        table, `slots` as int32), then attention over the tables.  One launch
        (pa_decode_append) unless the vector kernel's balanced split serves the step; then
        the scatter and the attention launch."""
        if not self.fused_step_ok(query.shape[1], partition_size, variant):
            self.write(new_key, new_value, slots, stream)
            return self.attend(query, block_tables, context_lens, scale, out=out,
                               partition_size=partition_size, max_context_len=max_context_len,
                               variant=variant, workspace=workspace, stream=stream)
        out = torch.empty_like(query) if out is None else out
        if partition_size and workspace is None:
            workspace = self.workspace(query.shape[0], query.shape[1], max_context_len,
                                       partition_size)
        pa_decode_append(out, query, new_key, new_value, self.key_cache, self.value_cache,
                         block_tables, context_lens, scale, max_context_len=max_context_len,
                         partition_size=partition_size, variant=variant, workspace=workspace,
                         stream=stream, k_scales=self.k_scales, v_scales=self.v_scales)
        return out


class HostKVPool:
    """Swap space: a block pool of the same shape in pinned host memory (the device
    reads and writes it directly) with its own allocator ("PagedAttention" concept
    report §6 and §11: under memory pressure a request's blocks move to CPU memory and
    come back when it is rescheduled)."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                 dtype: torch.dtype):
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.key_cache = torch.empty(shape, dtype=dtype, pin_memory=True)
        self.value_cache = torch.empty(shape, dtype=dtype, pin_memory=True)
        self.k_scales = self.v_scales = None
        if dtype == torch.uint8:  # E4M3 codes: the blocks' scales travel with them
            self.k_scales = torch.ones((num_blocks, num_kv_heads), dtype=torch.float32,
                                       pin_memory=True)
            self.v_scales = torch.ones_like(self.k_scales).pin_memory()
        self.alloc = Allocator(num_blocks, block_size)
        self.num_blocks, self.block_size = num_blocks, block_size


def swap_out(cache: PagedKVCache, host: HostKVPool, seq: int, stream=None) -> int:
    """Move `seq`'s blocks to host memory and release them on the device; returns the
    sequence's id in the host pool.  Stream order keeps the freed device blocks from
    being overwritten before the copy has read them."""
    table, ctx = cache.alloc.block_table(seq)
    hseq, hids = host.alloc.adopt(ctx)
    if len(table):
        src = _as_dev(np.asarray(table, np.int32), cache.device)
        dst = _as_dev(hids, cache.device)
        pa_swap_blocks(cache.key_cache, cache.value_cache, host.key_cache, host.value_cache, src,
                       dst, stream)
        if cache.fp8:
            pa_swap_blocks(*_scale_pools(cache.k_scales, cache.v_scales),
                           *_scale_pools(host.k_scales, host.v_scales), src, dst, stream)
    cache.free_seq(seq)
    return hseq


def swap_in(cache: PagedKVCache, host: HostKVPool, hseq: int, stream=None) -> int:
    """Move a swapped-out sequence back onto fresh device blocks; returns its new id."""
    table, ctx = host.alloc.block_table(hseq)
    seq, ids = cache.alloc.adopt(ctx)
    if len(table):
        src = _as_dev(np.asarray(table, np.int32), cache.device)
        dst = _as_dev(ids, cache.device)
        pa_swap_blocks(host.key_cache, host.value_cache, cache.key_cache, cache.value_cache, src,
                       dst, stream)
        if cache.fp8:
            pa_swap_blocks(*_scale_pools(host.k_scales, host.v_scales),
                           *_scale_pools(cache.k_scales, cache.v_scales), src, dst, stream)
    host.alloc.free_seq(hseq)
    return seq


def _as_dev(a, device) -> torch.Tensor:
    if isinstance(a, torch.Tensor):
        return a if a.device.type != "cpu" else a.to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def to_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage numpy array (f32 / f16 / bf16 bits as uint16 / E4M3 codes) -> CPU tensor."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


TORCH_DTYPE: Dict[str, torch.dtype] = {"f32": torch.float32, "f16": torch.float16,
                                       "bf16": torch.bfloat16, "fp8": torch.uint8}
