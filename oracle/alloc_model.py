"""Model block allocator in plain Python (TEST INFRASTRUCTURE ONLY).

What the pages fix:
  - "vLLM PagedAttention 技术深度解析" (kwkr.cn) §1.2.2: a new sequence starts with
    an empty block table; when its current block is full a block is taken from
    the pool; when it finishes its blocks are released and reference counts
    updated.  §1.3.2: shared prefixes, copy-on-write, reference counts, release
    deferred until nobody holds the block.
  - "PagedAttention" concept report (compassingai.com) §6: sharing raises a
    block's count; before a write into a block whose count exceeds one, a new
    block is allocated and the content copied.  §11: the free blocks are kept in
    a global free list.  §13: when no block is left the allocator reports an
    explicit out-of-memory error instead of failing the running requests.
  - KV-cache/paging tutorial (wmrh.cn), "paged attention" part: forked requests
    point at the same physical blocks with count 2 (three beams: count 3).
  - "PagedAttention" concept report §6 and §11: under memory pressure a request's
    blocks move to CPU memory and back; `adopt` is the receiving end of such a move
    (a sequence of n tokens on fresh blocks).

Readings (pages silent): the free list is a LIFO stack whose pops initially return
0, 1, 2, ... (or a given order); blocks released by free_seq are pushed in table
order; copy-on-write copies the whole block and moves the writer to the copy; the
last holder writes in place; an out-of-memory append changes nothing, and a batch of
appends that runs out part-way changes nothing either (append_slots).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple


class OutOfBlocks(Exception):
    pass


class InvalidOp(Exception):
    pass


class ModelAllocator:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidOp("sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: List[int] = list(range(num_blocks - 1, -1, -1))  # pop() -> 0, 1, ...
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.ctx: Dict[int, int] = {}
        self.next_id = 0

    def set_free_order(self, ids) -> None:
        ids = [int(i) for i in ids]
        if any(self.ref):
            raise InvalidOp("blocks in use")
        if sorted(ids) != list(range(self.num_blocks)):
            raise InvalidOp("not a permutation of all blocks")
        self.free = list(reversed(ids))

    def new_seq(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.ctx[sid] = 0
        return sid

    def _seq(self, sid: int) -> List[int]:
        if sid not in self.tables:
            raise InvalidOp(f"unknown sequence {sid}")
        return self.tables[sid]

    def append_slot(self, sid: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Slot for the next token of `sid`, and the (src, dst) copy if one is due."""
        table = self._seq(sid)
        n = self.ctx[sid]
        B = self.block_size
        if n % B == 0:  # no block yet, or the last one is full
            if not self.free:
                raise OutOfBlocks()
            b = self.free.pop()
            self.ref[b] = 1
            table.append(b)
            self.ctx[sid] = n + 1
            return b * B, None
        last = table[-1]
        if self.ref[last] > 1:  # shared and about to be written: copy first
            if not self.free:
                raise OutOfBlocks()
            b = self.free.pop()
            self.ref[b] = 1
            self.ref[last] -= 1
            table[-1] = b
            self.ctx[sid] = n + 1
            return b * B + n % B, (last, b)
        self.ctx[sid] = n + 1
        return last * B + n % B, None

    def append_slots(self, sids) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Appends in order, all or nothing: if one runs out of blocks (or names an
        unknown sequence) the allocator is restored to its state before the call, free
        list order included, and the error is raised."""
        saved = (list(self.free), list(self.ref), {k: list(v) for k, v in self.tables.items()},
                 dict(self.ctx))
        slots, cow = [], []
        try:
            for sid in sids:
                slot, c = self.append_slot(sid)
                slots.append(slot)
                if c is not None:
                    cow.append(c)
        except (OutOfBlocks, InvalidOp):
            self.free, self.ref, self.tables, self.ctx = saved
            raise
        return slots, cow

    def adopt(self, num_tokens: int):
        """A sequence of num_tokens tokens on fresh blocks (the receiving end of a swap)."""
        n = -(-num_tokens // self.block_size)
        if n > len(self.free):
            raise OutOfBlocks()
        sid = self.new_seq()
        for _ in range(n):
            b = self.free.pop()
            self.ref[b] = 1
            self.tables[sid].append(b)
        self.ctx[sid] = num_tokens
        return sid, list(self.tables[sid])

    def fork(self, parent: int) -> int:
        table = self._seq(parent)
        child = self.new_seq()
        self.tables[child] = list(table)
        self.ctx[child] = self.ctx[parent]
        for b in table:
            self.ref[b] += 1
        return child

    def free_seq(self, sid: int) -> None:
        table = self._seq(sid)
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[sid]
        del self.ctx[sid]

    def block_table(self, sid: int) -> Tuple[List[int], int]:
        return list(self._seq(sid)), self.ctx[sid]

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            raise InvalidOp("block out of range")
        return self.ref[block]

    def stats(self) -> dict:
        """Monitoring figures (kwkr.cn §1.4.1; compassingai.com §7)."""
        used = sum(1 for r in self.ref if r > 0)
        shared = sum(1 for r in self.ref if r > 1)
        fill = [0] * self.num_blocks  # tokens held by each block (max over holders)
        B = self.block_size
        for sid, table in self.tables.items():
            n = self.ctx[sid]
            for j, b in enumerate(table):
                fill[b] = max(fill[b], min(B, n - j * B))
        stored = sum(fill)
        wasted = used * B - stored
        return {
            "total_blocks": self.num_blocks,
            "used_blocks": used,
            "free_blocks": len(self.free),
            "shared_blocks": shared,
            "num_seqs": len(self.tables),
            "logical_tokens": sum(self.ctx.values()),
            "stored_tokens": stored,
            "wasted_slots": wasted,
            # kwkr.cn §1.4.1: blocks in use / all blocks; shared blocks / all blocks;
            # free-but-unusable memory / all memory (in a paged pool every free block is
            # usable, so the unusable part is the allocated slots no token fills)
            "block_utilisation": used / self.num_blocks,
            "sharing_rate": shared / self.num_blocks,
            "fragmentation_rate": wasted / (self.num_blocks * B),
            # compassingai.com §7: KV the requests need / KV allocated to them
            "emu": stored / (used * B) if used else 0.0,
        }
