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
* Prefix caching: a full block is keyed by a hash of its tokens and of its
  parent block's hash, kept in ``cached_block_hash_to_block``; a request
  whose leading full blocks hash to cached blocks points at them instead of
  recomputing them.  Only full blocks are cached, so identical prefixes give
  byte-identical KV and unchanged output; when sequences diverge inside a
  shared block, that block is copied first (copy-on-write).  (Same bullet;
  "49 vLLM / PagedAttention", sections "Почему это важно" and "Вопросы
  пытливого ума".)

Readings taken where the pages leave a step open:

* ``req.len`` in the allocate-on-growth test is the number of tokens already
  stored; a new block is needed exactly when that count is a multiple of
  ``block_size``; the write offset inside the last block is ``len % block_size``.
* Admission is first-come-first-served and stops at the first request that
  does not fit (the scheduler queues once the pool is full).  With this rule
  the pages' capacity example gives 13 paged sequences; admitting later,
  smaller requests past a miss gives 14.
* A finished sequence returns its blocks in table order.  A freed block
  keeps its hash and stays findable until allocation pops it from the free
  queue (the queue is in eviction order), which evicts it from the cache.
* The block hash is the first 8 bytes of SHA-256 over the parent's hash
  and the block's token ids (both as little-endian 64-bit integers); the
  first block's parent hash is 0.  Lookups stop at the first miss.
* Copy-on-write: appending into a block with ``ref_cnt > 1`` takes a fresh
  block, records the (source, destination) pair for the device copy
  (``pa_copy_blocks``), drops one reference to the source and continues in
  the copy.

Pure host logic (Python, no GPU): it builds the int32 ``block_tables``,
``seq_lens`` and ``slot_mapping`` arrays the device entry points consume.
"""
from __future__ import annotations

import hashlib
import struct
from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class KVCacheBlock:
    """One physical block of the pool (``block_id`` indexes the pool tensors)."""

    __slots__ = ("block_id", "ref_cnt", "prev", "next", "in_free_queue",
                 "block_hash")

    def __init__(self, block_id: int):
        self.block_id = block_id
        self.ref_cnt = 0
        self.prev: Optional[KVCacheBlock] = None
        self.next: Optional[KVCacheBlock] = None
        self.in_free_queue = False
        self.block_hash: Optional[int] = None

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


_KEY_LAYOUT: Dict[int, struct.Struct] = {}


def hash_block_tokens(parent_hash: int, token_ids: Sequence[int]) -> int:
    """Key of a full block: its token ids chained to its parent's key (the
    first 8 bytes of the SHA-256 of the parent key, as a little-endian
    uint64, followed by the ids as little-endian int64)."""
    n = len(token_ids)
    layout = _KEY_LAYOUT.get(n)
    if layout is None:
        layout = _KEY_LAYOUT[n] = struct.Struct(f"<Q{n}q")
    digest = hashlib.sha256(
        layout.pack(parent_hash & (2**64 - 1), *token_ids)).digest()
    return int.from_bytes(digest[:8], "little")


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
        self.cached_block_hash_to_block: Dict[int, KVCacheBlock] = {}

    @property
    def num_free(self) -> int:
        return len(self.free_block_queue)

    def alloc(self) -> Optional[KVCacheBlock]:
        """Pop the head of the free queue (None when the pool is exhausted).
        A popped block that was still cached is evicted from the cache."""
        block = self.free_block_queue.popleft()
        if block is None:
            return None
        assert block.ref_cnt == 0
        if block.block_hash is not None:
            if self.cached_block_hash_to_block.get(block.block_hash) is block:
                del self.cached_block_hash_to_block[block.block_hash]
            block.block_hash = None
        block.ref_cnt = 1
        return block

    def lookup(self, block_hash: int) -> Optional[KVCacheBlock]:
        return self.cached_block_hash_to_block.get(block_hash)

    def cache(self, block: KVCacheBlock, block_hash: int) -> None:
        """Register a full block under its key (first one wins)."""
        if block.block_hash is None and \
                block_hash not in self.cached_block_hash_to_block:
            block.block_hash = block_hash
            self.cached_block_hash_to_block[block_hash] = block

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
    token_ids: Optional[List[int]] = None  # kept when prefix caching is used
    # (block index, key) of fresh full blocks admitted without registering
    # them, in order; cache_written registers them once their KV is stored
    pending_keys: List[Tuple[int, int]] = field(default_factory=list)
    # int32 ids of ``blocks``, rebuilt after the list changes (None then)
    ids: Optional[np.ndarray] = field(default=None, repr=False,
                                      compare=False)


class KVCacheManager:
    """Per-request block lists (``req_to_blocks``) drawn from a shared pool."""

    def __init__(self, pool: BlockPool, block_size: int = 16):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.pool = pool
        self.block_size = block_size
        self.req_to_blocks: Dict[int, SeqState] = {}
        # (source, destination) block pairs the device must copy before the
        # next append (copy-on-write); drained by take_copies()
        self.pending_copies: List[Tuple[int, int]] = []

    @property
    def num_free(self) -> int:
        return self.pool.num_free

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

    def prefix_keys(self, token_ids: Sequence[int]) -> List[int]:
        """Keys of the full blocks of ``token_ids``, in order (each chained
        to the one before); a caller that prices and admits the same tokens
        more than once can compute them once and pass them in."""
        bs = self.block_size
        toks = [int(t) for t in token_ids]
        keys, parent = [], 0
        for i in range(len(toks) // bs):
            parent = hash_block_tokens(parent, toks[i * bs:(i + 1) * bs])
            keys.append(parent)
        return keys

    def _cached_prefix(self, toks: Sequence[int],
                       keys: Optional[List[int]] = None):
        """Keys of the full blocks of ``toks`` and the cached blocks of its
        longest cached prefix (lookups stop at the first miss)."""
        hashes = self.prefix_keys(toks) if keys is None else keys
        if len(hashes) != len(toks) // self.block_size:
            raise ValueError("keys do not match the tokens' full blocks")
        hits: List[KVCacheBlock] = []
        for h in hashes:
            blk = self.pool.lookup(h)
            if blk is None:
                break
            hits.append(blk)
        return hashes, hits

    def blocks_to_admit(self, token_ids: Sequence[int],
                        keys: Optional[List[int]] = None) -> int:
        """Free-queue blocks ``admit_cached(token_ids)`` would take: its
        fresh blocks plus the cached hits that sit in the free queue (a
        touch takes them out of it).  Reserves nothing.  ``keys``, if
        given, are ``prefix_keys(token_ids)``."""
        _, hits = self._cached_prefix(token_ids, keys)
        fresh = self.blocks_needed(len(token_ids)) - len(hits)
        return fresh + sum(1 for b in hits if b.ref_cnt == 0)

    def admit_cached(self, seq_id: int, token_ids: Sequence[int],
                     register: bool = True,
                     keys: Optional[List[int]] = None) -> Tuple[bool, int]:
        """Admit a request whose tokens are known, reusing cached full
        blocks of an identical prefix.  Returns (admitted, cached blocks
        reused); the reused blocks' KV is already in the pool, only the rest
        must be written.  Fresh full blocks are registered in the cache at
        once, so the caller must write their KV before the next admission
        can find them (a caller that may undo an admission checks
        ``blocks_to_admit`` first instead of undoing it).  With
        ``register=False`` they are registered only by ``cache_written``,
        for a caller that writes a prompt over several steps and may free
        the request before all of it is written.  ``keys``, if given, are
        ``prefix_keys(token_ids)``."""
        if seq_id in self.req_to_blocks:
            raise ValueError(f"sequence {seq_id} already admitted")
        toks = [int(t) for t in token_ids]
        nfull = len(toks) // self.block_size
        hashes, hits = self._cached_prefix(toks, keys)
        # a hit that sits in the free queue still counts as free until
        # touched: it must not be allocated for this request's fresh blocks
        fresh = self.blocks_needed(len(toks)) - len(hits)
        free_hits = sum(1 for b in hits if b.ref_cnt == 0)
        if fresh > self.pool.num_free - free_hits:
            return False, 0
        state = SeqState(seq_id, token_ids=list(toks))
        for blk in hits:
            self.pool.touch(blk)
            state.blocks.append(blk)
        for i in range(fresh):
            blk = self.pool.alloc()
            state.blocks.append(blk)
            j = len(hits) + i
            if j < nfull:
                if register:
                    self.pool.cache(blk, hashes[j])
                else:
                    state.pending_keys.append((j, hashes[j]))
        state.num_tokens = len(toks)
        self.req_to_blocks[seq_id] = state
        return True, len(hits)

    def cache_written(self, seq_id: int, num_tokens: int) -> None:
        """Registers the pending full blocks that lie within the first
        ``num_tokens`` tokens of the sequence, whose KV is now stored."""
        st = self.req_to_blocks[seq_id]
        done = num_tokens // self.block_size
        k = 0
        while k < len(st.pending_keys) and st.pending_keys[k][0] < done:
            idx, key = st.pending_keys[k]
            self.pool.cache(st.blocks[idx], key)
            k += 1
        del st.pending_keys[:k]

    def fork(self, src_id: int, new_id: int) -> None:
        """A new sequence continuing src's context: it shares every block
        (parallel sampling, beam search); divergence is copy-on-write."""
        if new_id in self.req_to_blocks:
            raise ValueError(f"sequence {new_id} already admitted")
        src = self.req_to_blocks[src_id]
        for blk in src.blocks:
            self.pool.touch(blk)
        self.req_to_blocks[new_id] = SeqState(
            new_id, src.num_tokens, list(src.blocks),
            None if src.token_ids is None else list(src.token_ids))

    def take_copies(self) -> List[Tuple[int, int]]:
        out, self.pending_copies = self.pending_copies, []
        return out

    def admit_fcfs(self, lengths: Sequence[int]) -> int:
        """Admit requests in arrival order; stop at the first that does not fit."""
        admitted = 0
        for i, n in enumerate(lengths):
            if not self.admit(len(self.req_to_blocks), int(n)):
                break
            admitted += 1
        return admitted

    # -- growth --------------------------------------------------------------
    def append_slot(self, seq_id: int, token_id: Optional[int] = None) -> int:
        """Reserve the slot of one new token (allocate-on-growth).

        A block is popped only when every slot of the existing blocks is used.
        If the target block is shared, it is copied first (copy-on-write: the
        pair is queued in ``pending_copies``).  Returns the flat slot
        ``phys * block_size + offset``; raises MemoryError when the pool is
        exhausted.  With prefix caching (token ids known), a block that the
        token fills up is registered in the cache.
        """
        st = self.req_to_blocks[seq_id]
        bs = self.block_size
        if len(st.blocks) * bs <= st.num_tokens:
            blk = self.pool.alloc()
            if blk is None:
                raise MemoryError("KV block pool exhausted")
            st.blocks.append(blk)
            st.ids = None
        idx = st.num_tokens // bs
        last = st.blocks[idx]
        if last.ref_cnt > 1:
            copy = self.pool.alloc()
            if copy is None:
                raise MemoryError("KV block pool exhausted (copy-on-write)")
            self.pending_copies.append((last.block_id, copy.block_id))
            self.pool.free(last)
            st.blocks[idx] = copy
            st.ids = None
            last = copy
        slot = last.block_id * bs + st.num_tokens % bs
        st.num_tokens += 1
        if st.token_ids is not None:
            st.token_ids.append(-1 if token_id is None else int(token_id))
            if st.num_tokens % bs == 0:
                parent = 0 if idx == 0 else st.blocks[idx - 1].block_hash
                if parent is not None:
                    self.pool.cache(last, hash_block_tokens(
                        parent, st.token_ids[idx * bs:(idx + 1) * bs]))
        return slot

    def append_slots(self, seq_ids: Sequence[int],
                     token_ids: Optional[Sequence[int]] = None) -> np.ndarray:
        """``append_slot`` for each sequence in order: their int32 slots."""
        if token_ids is None:
            token_ids = [None] * len(seq_ids)
        return np.asarray([self.append_slot(s, t)
                           for s, t in zip(seq_ids, token_ids)],
                          dtype=np.int32)

    def free_seq(self, seq_id: int) -> None:
        st = self.req_to_blocks.pop(seq_id)
        for blk in st.blocks:
            self.pool.free(blk)

    # -- views ---------------------------------------------------------------
    def num_tokens(self, seq_id: int) -> int:
        return self.req_to_blocks[seq_id].num_tokens

    def block_ids(self, seq_id: int) -> List[int]:
        return [b.block_id for b in self.req_to_blocks[seq_id].blocks]

    def wasted_slots(self, seq_id: int) -> int:
        st = self.req_to_blocks[seq_id]
        return len(st.blocks) * self.block_size - st.num_tokens

    def tables(self, seq_ids: Sequence[int], pad: int = -1,
               width: Optional[int] = None):
        """int32 ``block_tables`` [B, width] (padded with ``pad``) and
        ``seq_lens`` [B] for ``seq_ids`` in that order."""
        states = [self.req_to_blocks[s] for s in seq_ids]
        rows = []
        for st in states:
            if st.ids is None:
                st.ids = np.fromiter((b.block_id for b in st.blocks),
                                     dtype=np.int32, count=len(st.blocks))
            rows.append(st.ids)
        n = np.fromiter((len(r) for r in rows), dtype=np.int64,
                        count=len(rows))
        w = int(n.max(initial=0)) if width is None else width
        w = max(w, 1)
        if len(rows) and int(n.max()) > w:
            raise ValueError("table width too small")
        table = np.full((len(rows), w), pad, dtype=np.int32)
        if len(rows):
            # row-major order of the mask is the order of the rows' ids
            table[np.arange(w) < n[:, None]] = np.concatenate(rows)
        lens = np.fromiter((st.num_tokens for st in states), dtype=np.int32,
                           count=len(states))
        return table, lens
