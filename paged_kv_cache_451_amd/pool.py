"""Host-side KV block pool: the allocator that produces block tables and slots.

What the pages describe, restated:

* The KV cache lives in a shared pool of fixed-size blocks of ``block_size``
  tokens (16 by default); a sequence's block table maps its logical blocks to
  arbitrary physical blocks of that pool.  ("49 vLLM / PagedAttention",
  section "Идея и механизм"; "PagedAttention：KV cache 即虚拟内存", section
  "直接答案".)
* Free blocks sit in ``free_block_queue``, a doubly linked list kept in
  eviction order: allocation pops the head, release pushes to the tail, both
  in O(1).  Each block carries ``ref_cnt``; a finished request decrements it
  and the block returns to the free queue when it reaches zero.  Requests own
  per-request block lists drawn from the shared pool.  ("PagedAttention：KV
  cache 即虚拟内存", section "深入原理", bullets on the V1 structure and the
  block lifecycle; "vLLM innenfra", paragraph on the KV-cache manager.)
* Growth is on demand: a new block is taken only when the last one is full,
  so the waste per sequence is at most one partly filled block.  ("49 vLLM /
  PagedAttention", listing "Таблица блоков"; "PagedAttention：KV cache 即虚拟
  内存", sections "直接答案" and "深入原理".)
* Sequences with a common prefix point at the same physical blocks;
  ``touch()`` raises the reference count of a block another request already
  holds.  ("PagedAttention：KV cache 即虚拟内存", section "深入原理", bullet on
  sharing / prefix caching.)

Readings taken where the pages leave a step open:

* ``req.len`` in the allocate-on-growth test is the number of tokens already
  stored; a new block is needed exactly when that count is a multiple of
  ``block_size``; the write offset inside the last block is ``len % block_size``.
* Admission is first-come-first-served and stops at the first request that
  does not fit (the scheduler queues once the pool is full).  With this rule
  the pages' capacity example gives 13 paged sequences; admitting later,
  smaller requests past a miss gives 14.
* A finished sequence returns its blocks in table order.
* Appending into a block with ``ref_cnt > 1`` would need copy-on-write, which
  this harness does not implement: it raises instead.

Pure host logic (Python, no GPU): it builds the int32 ``block_tables``,
``seq_lens`` and ``slot_mapping`` arrays the device entry points consume.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np


class KVCacheBlock:
    """One physical block of the pool (``block_id`` indexes the pool tensors)."""

    __slots__ = ("block_id", "ref_cnt", "prev", "next", "in_free_queue")

    def __init__(self, block_id: int):
        self.block_id = block_id
        self.ref_cnt = 0
        self.prev: Optional[KVCacheBlock] = None
        self.next: Optional[KVCacheBlock] = None
        self.in_free_queue = False

    def __repr__(self) -> str:  # pragma: no cover - debugging aid
        return f"KVCacheBlock(id={self.block_id}, ref_cnt={self.ref_cnt})"


class FreeBlockQueue:
    """Intrusive doubly linked list of free blocks with O(1) pop-head,
    push-tail and remove (the last is what ``touch`` of a free block needs)."""

    def __init__(self, blocks: Iterable[KVCacheBlock] = ()):
        self._head = KVCacheBlock(-1)  # sentinels
        self._tail = KVCacheBlock(-2)
        self._head.next = self._tail
        self._tail.prev = self._head
        self._len = 0
        for b in blocks:
            self.append(b)

    def __len__(self) -> int:
        return self._len

    def append(self, block: KVCacheBlock) -> None:
        if block.in_free_queue:
            raise ValueError(f"block {block.block_id} is already free")
        last = self._tail.prev
        last.next = block
        block.prev = last
        block.next = self._tail
        self._tail.prev = block
        block.in_free_queue = True
        self._len += 1

    def popleft(self) -> Optional[KVCacheBlock]:
        if self._len == 0:
            return None
        block = self._head.next
        self.remove(block)
        return block

    def remove(self, block: KVCacheBlock) -> None:
        if not block.in_free_queue:
            raise ValueError(f"block {block.block_id} is not in the free queue")
        block.prev.next = block.next
        block.next.prev = block.prev
        block.prev = block.next = None
        block.in_free_queue = False
        self._len -= 1

    def ids(self) -> List[int]:
        out, b = [], self._head.next
        while b is not self._tail:
            out.append(b.block_id)
            b = b.next
        return out


class BlockPool:
    """Owns every ``KVCacheBlock``; hands them out from the free queue.

    ``order`` is the initial free-queue order (a permutation of block ids);
    a seeded random permutation gives shuffled physical blocks.
    """

    def __init__(self, num_blocks: int, order: Optional[Sequence[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = num_blocks
        self.blocks = [KVCacheBlock(i) for i in range(num_blocks)]
        if order is None:
            order = range(num_blocks)
        order = [int(i) for i in order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self.free_block_queue = FreeBlockQueue(self.blocks[i] for i in order)

    @property
    def num_free(self) -> int:
        return len(self.free_block_queue)

    def alloc(self) -> Optional[KVCacheBlock]:
        """Pop the head of the free queue (None when the pool is exhausted)."""
        block = self.free_block_queue.popleft()
        if block is None:
            return None
        assert block.ref_cnt == 0
        block.ref_cnt = 1
        return block

    def touch(self, block: KVCacheBlock) -> None:
        """Another request starts sharing ``block``."""
        if block.ref_cnt == 0 and block.in_free_queue:
            self.free_block_queue.remove(block)
        block.ref_cnt += 1

    def free(self, block: KVCacheBlock) -> None:
        """Drop one reference; at zero the block goes to the free-queue tail."""
        if block.ref_cnt <= 0:
            raise ValueError(f"ref_cnt underflow on block {block.block_id}")
        block.ref_cnt -= 1
        if block.ref_cnt == 0:
            self.free_block_queue.append(block)


@dataclass
class SeqState:
    seq_id: int
    num_tokens: int = 0  # tokens already stored in the cache
    blocks: List[KVCacheBlock] = field(default_factory=list)


class KVCacheManager:
    """Per-request block lists (``req_to_blocks``) drawn from a shared pool."""

    def __init__(self, pool: BlockPool, block_size: int = 16):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.pool = pool
        self.block_size = block_size
        self.req_to_blocks: Dict[int, SeqState] = {}

    # -- admission -----------------------------------------------------------
    def blocks_needed(self, num_tokens: int) -> int:
        return -(-num_tokens // self.block_size)

    def can_admit(self, num_tokens: int) -> bool:
        return self.blocks_needed(num_tokens) <= self.pool.num_free

    def admit(self, seq_id: int, num_tokens: int,
              shared_prefix: Sequence[KVCacheBlock] = ()) -> bool:
        """Reserve blocks for ``num_tokens`` already-computed tokens.

        ``shared_prefix`` are full blocks owned by another request: they are
        touched (ref_cnt + 1) instead of allocated.  Returns False, leaving the
        pool unchanged, when the fresh blocks do not fit.
        """
        if seq_id in self.req_to_blocks:
            raise ValueError(f"sequence {seq_id} already admitted")
        n_shared = len(shared_prefix)
        if n_shared * self.block_size > num_tokens:
            raise ValueError("shared prefix longer than the sequence")
        fresh = self.blocks_needed(num_tokens) - n_shared
        if fresh > self.pool.num_free:
            return False
        state = SeqState(seq_id)
        for blk in shared_prefix:
            self.pool.touch(blk)
            state.blocks.append(blk)
        for _ in range(fresh):
            state.blocks.append(self.pool.alloc())
        state.num_tokens = num_tokens
        self.req_to_blocks[seq_id] = state
        return True

    def admit_fcfs(self, lengths: Sequence[int]) -> int:
        """Admit requests in arrival order; stop at the first that does not fit."""
        admitted = 0
        for i, n in enumerate(lengths):
            if not self.admit(len(self.req_to_blocks), int(n)):
                break
            admitted += 1
        return admitted

    # -- growth --------------------------------------------------------------
    def append_slot(self, seq_id: int) -> int:
        """Reserve the slot of one new token (allocate-on-growth).

        A block is popped only when every slot of the existing blocks is used.
        Returns the flat slot ``phys * block_size + offset``; raises when the
        pool is exhausted or the target block is shared.
        """
        st = self.req_to_blocks[seq_id]
        if len(st.blocks) * self.block_size <= st.num_tokens:
            blk = self.pool.alloc()
            if blk is None:
                raise MemoryError("KV block pool exhausted")
            st.blocks.append(blk)
        last = st.blocks[st.num_tokens // self.block_size]
        if last.ref_cnt > 1:
            raise RuntimeError("append into a shared block needs copy-on-write")
        slot = last.block_id * self.block_size + st.num_tokens % self.block_size
        st.num_tokens += 1
        return slot

    def free_seq(self, seq_id: int) -> None:
        st = self.req_to_blocks.pop(seq_id)
        for blk in st.blocks:
            self.pool.free(blk)

    # -- views ---------------------------------------------------------------
    def block_ids(self, seq_id: int) -> List[int]:
        return [b.block_id for b in self.req_to_blocks[seq_id].blocks]

    def wasted_slots(self, seq_id: int) -> int:
        st = self.req_to_blocks[seq_id]
        return len(st.blocks) * self.block_size - st.num_tokens

    def tables(self, seq_ids: Sequence[int], pad: int = -1,
               width: Optional[int] = None):
        """int32 ``block_tables`` [B, width] (padded with ``pad``) and
        ``seq_lens`` [B] for ``seq_ids`` in that order."""
        rows = [self.block_ids(s) for s in seq_ids]
        w = max((len(r) for r in rows), default=0) if width is None else width
        w = max(w, 1)
        table = np.full((len(rows), w), pad, dtype=np.int32)
        for i, r in enumerate(rows):
            if len(r) > w:
                raise ValueError("table width too small")
            table[i, :len(r)] = r
        lens = np.array([self.req_to_blocks[s].num_tokens for s in seq_ids],
                        dtype=np.int32)
        return table, lens
