"""A synthetic continuous-batching engine loop over the paged KV cache.

The pages describe the serving loop around the paged cache ("vLLM innenfra",
the ``step()`` paragraphs; "PagedAttention：KV cache 即虚拟内存（block manager
& 碎片）", section "深入原理", lifecycle bullet):

* each ``step()`` schedules work, runs the forward pass and post-processes:
  finished requests hand their blocks back to the free-block queue;
* new requests join between steps (continuous batching), first come first
  served; when the pool is full the scheduler queues them;
* a request's prompt takes its blocks on admission, decoding takes one more
  block whenever the last one is full;
* under pool pressure a running request is preempted (evicted and later
  recomputed, like a page-out) so that the others can keep growing.

There is no model here: random K/V stand in for the projections of each
token and random queries for the attention input, so the loop exercises the
block manager and the device path (``pa_kv_append`` for prompt tokens,
``pa_decode_append`` for one new token per running request) at the scale of
a serving batch.  Optionally (``max_prefill_tokens``) a step takes at most
that many prompt tokens, so a long prompt is cut into chunks spread over
several steps and mixed with the decode work of the others ("vLLM innenfra",
continuous-batching paragraph: chunked prefill), and (``prefill_attention``)
each step's chunks are attended with ``pa_prefill``, the compute-bound side
of the loop.  ``contiguous_capacity`` gives the number of requests a
cache that reserves ``max_len`` tokens per request would hold in the same
pool, for comparison with the concurrency the paged cache reaches.

Readings where the pages leave a step open:

* a preempted request is the most recently admitted running one; its blocks
  are freed and it goes back to the front of the waiting queue; on
  re-admission its prompt and the tokens generated so far are written again
  (recompute);
* admission is first come first served and stops at the first waiting
  request whose tokens do not fit next to the blocks the running requests
  need for this step's new tokens;
* every running request decodes one token per step; a request finishes
  after ``max_new_tokens`` decoded tokens and frees its blocks in the same
  step;
* with chunked prefill, a request takes all its blocks on admission (so
  admission is priced as before), its prompt tokens are written and attended
  chunk by chunk in admission order, and it decodes from the step that
  writes its last prompt token on (that step included, as a whole-prompt
  admission decodes in its admission step).
"""
from __future__ import annotations

import math
from collections import deque
from dataclasses import dataclass, field
from typing import Deque, Dict, List, Optional

import numpy as np

from .pool import BlockPool, KVCacheManager

BLOCK_SIZE = 16


@dataclass
class Request:
    req_id: int
    prompt_ids: List[int]
    max_new_tokens: int
    output_ids: List[int] = field(default_factory=list)
    admitted_step: int = -1
    finished_step: int = -1
    preemptions: int = 0
    written: int = 0       # tokens of this admission whose K/V are stored
    # (token count, prefix-cache keys of its full blocks), computed once
    # for the tokens a waiting request is priced and admitted with
    keys: Optional[tuple] = field(default=None, repr=False, compare=False)
    # prompt plus output tokens, kept up to date by add_output
    num_tokens: int = field(default=0, init=False, compare=False)

    def __post_init__(self):
        self.num_tokens = len(self.prompt_ids) + len(self.output_ids)

    def add_output(self, token: int) -> None:
        self.output_ids.append(token)
        self.num_tokens += 1

    @property
    def done(self) -> bool:
        return len(self.output_ids) >= self.max_new_tokens


@dataclass
class StepStats:
    step: int
    running: int                 # requests that decoded a token this step
    waiting: int
    admitted: int
    preempted: int
    finished: int
    prefill_tokens: int          # prompt tokens written this step
    prefill_chunks: int          # requests whose prompt tokens were written
    cached_prefix_tokens: int    # prompt tokens found in the prefix cache
    blocks_used: int
    slots_used: int              # tokens stored in the cache


def contiguous_capacity(num_blocks: int, max_len: int,
                        block: int = BLOCK_SIZE) -> int:
    """Requests a cache reserving max_len tokens per request can hold."""
    return num_blocks // math.ceil(max_len / block)


class Engine:
    """Continuous batching over a paged KV pool on one GPU.

    ``device=None`` runs the scheduler and block manager only (no kernels),
    for host-side tests.  ``native_pool=True`` keeps the blocks in the
    native block manager (``native_pool.py``, the same rules and keys in C++,
    one library call per step for the decode's slots and tables) instead of
    ``pool.py``'s; ``self.pool`` is then None.  ``mirror=True`` records, for the last step, the
    host copies of every K/V row written with its slots (``last_writes``,
    in the order the device writes them) and the step's queries, tables and
    lengths, so that a test can rebuild the pools and check each decode
    with its own reference.
    """

    def __init__(self, num_blocks: int, num_q_heads: int, num_kv_heads: int,
                 head_size: int, *, device=None, seed: int = 0,
                 max_running: Optional[int] = None,
                 prefix_caching: bool = True, mirror: bool = False,
                 max_prefill_tokens: Optional[int] = None,
                 prefill_attention: bool = False, native_pool: bool = False):
        self.num_blocks = num_blocks
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_size
        rng = np.random.default_rng(seed)
        self.rng = rng
        order = rng.permutation(num_blocks)
        if native_pool:
            from .native_pool import NativeKVCacheManager
            self.pool = None
            self.mgr = NativeKVCacheManager(num_blocks, BLOCK_SIZE, order)
        else:
            self.pool = BlockPool(num_blocks, order=order)
            self.mgr = KVCacheManager(self.pool, BLOCK_SIZE)
        self.max_running = max_running
        self.prefix_caching = prefix_caching
        if max_prefill_tokens is not None and max_prefill_tokens < 1:
            raise ValueError("max_prefill_tokens must be at least 1")
        self.max_prefill_tokens = max_prefill_tokens
        self.prefill_attention = prefill_attention
        # the last step's prefill attention, with a mirror: queries (bf16
        # bits), q_start, tables, lengths, and the device output
        self.last_prefill = None
        self.waiting: Deque[Request] = deque()
        self.running: List[Request] = []        # in admission order
        # running requests whose prompt is not all written, in order
        self._prefilling: List[Request] = []
        self.finished: List[Request] = []
        self.step_no = 0
        self.device = device
        self.mirror = mirror
        self.scale = float(np.float32(1.0 / math.sqrt(head_size)))
        self.last_out = None
        self.last_batch: List[int] = []
        self._dev_rand: Dict[str, object] = {}
        # pinned staging buffers of the host-to-device uploads, used in
        # turn, each with the event recorded after the copy that last read
        # it, so that the host never waits for the device's queued work
        self._staging: List[Optional[tuple]] = [None] * 3
        self._staging_next = 0
        # (start event, end event, KV bytes) of each decode, when timed
        self.time_decode = False
        self.decode_events: List[tuple] = []
        # (start event, end event, algorithmic flops) of each prefill
        # attention launch, when timed (with time_decode)
        self.prefill_events: List[tuple] = []
        if device is not None:
            import torch
            self.torch = torch
            self.k_pool = torch.zeros(num_blocks, num_kv_heads, BLOCK_SIZE,
                                      head_size, dtype=torch.bfloat16,
                                      device=device)
            self.v_pool = torch.zeros(num_blocks, num_kv_heads, head_size,
                                      BLOCK_SIZE, dtype=torch.bfloat16,
                                      device=device)
        # (k rows, v rows, slots) written in the last step, with a mirror:
        # raw bf16 bits [n, Hkv, D] and int32 slots [n]
        self.last_writes: List[tuple] = []
        self.last_q = None

    # -- requests ------------------------------------------------------------
    def add_request(self, req: Request) -> None:
        self.waiting.append(req)

    def has_work(self) -> bool:
        return bool(self.waiting or self.running)

    # -- scheduling ------------------------------------------------------------
    def _preempt_last(self) -> Request:
        victim = self.running.pop()
        # the prompts being written are a subsequence of the running list
        if self._prefilling and self._prefilling[-1] is victim:
            self._prefilling.pop()
        self.mgr.free_seq(victim.req_id)
        victim.preemptions += 1
        self.waiting.appendleft(victim)
        return victim

    def _growth_need(self) -> int:
        """Blocks the running requests take for this step's new tokens."""
        # a running request's stored tokens are its prompt and outputs
        return sum(1 for r in self.running if r.num_tokens % BLOCK_SIZE == 0)

    def _ensure_growth(self) -> tuple:
        """Every running request needs a slot for its next token; preempt
        from the back until the blocks needed fit in the pool.  Returns the
        preemptions and the blocks the remaining requests need."""
        preempted = 0
        need = self._growth_need()
        while self.running and need > self.mgr.num_free:
            self._preempt_last()
            preempted += 1
            need = self._growth_need()
        return preempted, need

    def _admit(self, need: int) -> List[tuple]:
        """FCFS admission next to the running requests' growth ``need``;
        returns (request, cached prompt tokens) pairs."""
        admitted = []
        while self.waiting:
            if self.max_running is not None and \
                    len(self.running) >= self.max_running:
                break
            req = self.waiting[0]
            ids = req.prompt_ids + req.output_ids
            # Everything is priced before anything is reserved: the blocks
            # the admission takes, the blocks the running requests need for
            # this step's tokens, and one for the request's own first
            # decoded token when its blocks are full.  A request that does
            # not fit leaves the pool and the prefix cache untouched (an
            # admission that registered its fresh blocks in the cache and
            # was then undone would leave keys to blocks that never
            # received their KV).
            keys = None
            if self.prefix_caching:
                if req.keys is None or req.keys[0] != len(ids):
                    req.keys = (len(ids), self.mgr.prefix_keys(ids))
                keys = req.keys[1]
            take = (self.mgr.blocks_to_admit(ids, keys) if self.prefix_caching
                    else self.mgr.blocks_needed(len(ids)))
            grow = 1 if len(ids) % BLOCK_SIZE == 0 else 0
            if take + need + grow > self.mgr.num_free:
                break
            if self.prefix_caching:
                # a prompt written over several steps registers its blocks
                # in the prefix cache as their KV is written, so that a
                # later admission (its own after a preemption included)
                # never finds a block that holds no KV yet
                ok, hits = self.mgr.admit_cached(
                    req.req_id, ids,
                    register=self.max_prefill_tokens is None, keys=keys)
            else:
                ok, hits = self.mgr.admit(req.req_id, len(ids)), 0
            assert ok, "an admission that was priced to fit must succeed"
            self.running.append(req)
            self.waiting.popleft()
            req.written = hits * BLOCK_SIZE
            if req.written < req.num_tokens:
                self._prefilling.append(req)
            if req.admitted_step < 0:
                req.admitted_step = self.step_no
            admitted.append((req, hits * BLOCK_SIZE))
            need += grow
        return admitted

    # -- device work -------------------------------------------------------------
    def _random_rows(self, n: int):
        """n random K and V rows (bf16).  With a mirror they are drawn on the
        host, seeded; otherwise they are slices of a random device buffer
        (their values do not matter to the loop)."""
        import torch
        if not self.mirror and self.device is not None:
            return self._device_rows(n, "kv")
        g = torch.Generator().manual_seed(int(self.rng.integers(1 << 62)))
        k = torch.randn(n, self.hkv, self.d, generator=g).to(torch.bfloat16)
        v = torch.randn(n, self.hkv, self.d, generator=g).to(torch.bfloat16)
        return k, v

    def _device_rows(self, n: int, what: str):
        import torch
        heads = self.hq if what == "q" else self.hkv
        buf = self._dev_rand.get(what)
        if buf is None or buf.shape[0] < 2 * n:
            rows = max(2 * n, 4096)
            buf = torch.randn(rows, heads, self.d, device=self.device).to(
                torch.bfloat16)
            self._dev_rand[what] = buf
        if what == "q":
            return buf[:n]
        return buf[:n], buf[n:2 * n]

    def _prefill_chunks(self) -> List[tuple]:
        """This step's prompt chunks, (request, first token, end), in
        admission order, within the prompt-token budget."""
        budget = self.max_prefill_tokens
        chunks = []
        for r in self._prefilling:
            n = r.num_tokens - r.written
            if budget is not None:
                if budget == 0:
                    break
                n = min(n, budget)
                budget -= n
            chunks.append((r, r.written, r.written + n))
        return chunks

    def _write_prompts(self, chunks) -> int:
        """Writes the chunks' K/V (one append) and, with prefill attention,
        attends each chunk's tokens to everything stored before them."""
        parts = []
        for req, lo, hi in chunks:
            blocks = np.asarray(self.mgr.block_ids(req.req_id), dtype=np.int64)
            t = np.arange(lo, hi)
            parts.append(blocks[t // BLOCK_SIZE] * BLOCK_SIZE + t % BLOCK_SIZE)
        for req, lo, hi in chunks:
            req.written = hi
            if self.prefix_caching and self.max_prefill_tokens is not None:
                self.mgr.cache_written(req.req_id, hi)
        n = sum(len(x) for x in parts)
        if n == 0:
            return 0
        if self.device is None and not self.mirror:
            return n
        k, v = self._random_rows(n)
        slots_np = np.concatenate(parts).astype(np.int32)
        if self.mirror:
            self._record_write(k, v, slots_np)
        if self.device is not None:
            from . import _lib
            ints = [slots_np]
            if self.prefill_attention:
                ids = [r.req_id for r, _, _ in chunks]
                tables, _ = self.mgr.tables(ids)
                lens = np.asarray([hi for _, _, hi in chunks], dtype=np.int32)
                q_start = np.concatenate(
                    [[0], np.cumsum([hi - lo for _, lo, hi in chunks])]
                ).astype(np.int32)
                ints += [tables, lens, q_start]
            dev_ints = self._upload(*ints)
            _lib.pa_kv_append(k.to(self.device), v.to(self.device),
                              dev_ints[0], self.k_pool, self.v_pool)
            if self.prefill_attention:
                self._prefill(n, ints[1:], dev_ints[1:])
        return n

    def _upload(self, *arrays):
        """One host-to-device copy of several int32 arrays; returns their
        device views in order, each starting on a 64-byte boundary.  On a
        GPU the copy is asynchronous, from a pinned staging buffer, so the
        host goes on scheduling while the device works through the steps
        already queued (a copy from pageable memory would wait for them)."""
        torch = self.torch
        sizes = [a.size for a in arrays]
        offs = np.cumsum([0] + [-(-n // 16) * 16 for n in sizes])
        total = int(offs[-1])
        if torch.device(self.device).type != "cuda":
            flat = np.zeros(total, dtype=np.int32)
            for a, o in zip(arrays, offs):
                flat[o:o + a.size] = a.ravel()
            buf = torch.from_numpy(flat).to(self.device)
        else:
            k = self._staging_next
            self._staging_next = (k + 1) % len(self._staging)
            held = self._staging[k]
            if held is not None:
                held[1].synchronize()     # its last copy has been read
            if held is None or held[0].numel() < total:
                host = torch.empty(max(total, 1 << 16), dtype=torch.int32,
                                   pin_memory=True)
            else:
                host = held[0]
            flat = host.numpy()
            flat[:total] = 0
            for a, o in zip(arrays, offs):
                flat[o:o + a.size] = a.ravel()
            buf = torch.empty(total, dtype=torch.int32, device=self.device)
            buf.copy_(host[:total], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            self._staging[k] = (host, ev)
        return [buf[o:o + a.size].view(a.shape) for a, o in zip(arrays, offs)]

    def _prefill(self, n, host, dev_ints) -> None:
        """pa_prefill over the step's chunks: ``host`` holds their tables,
        lengths and query starts, ``dev_ints`` the same on the device."""
        import torch
        from . import _lib
        tables, lens, q_start = host
        if self.mirror:
            g = torch.Generator().manual_seed(int(self.rng.integers(1 << 62)))
            q = torch.randn(n, self.hq, self.d, generator=g).to(
                torch.bfloat16)
        else:
            q = self._device_rows(n, "q")
        dev = self.device
        out = torch.empty(n, self.hq, self.d, dtype=torch.bfloat16,
                          device=dev)
        if self.time_decode:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        _lib.pa_prefill(q.to(dev), self.k_pool, self.v_pool, *dev_ints,
                        self.scale, out)
        if self.time_decode:
            e1.record()
            # 4 D flops per (query token, attended key) pair and query head;
            # token i of a chunk attends keys 0..i
            lo = lens - np.diff(q_start)
            pairs = int(((lens.astype(np.int64) * (lens + 1) -
                          lo.astype(np.int64) * (lo + 1)) // 2).sum())
            self.prefill_events.append(
                (e0, e1, 4 * self.d * self.hq * pairs))
        if self.mirror:
            self.last_prefill = (q, q_start, tables, lens, out)

    def step(self) -> StepStats:
        self.last_writes = []
        self.last_prefill = None
        preempted, need = self._ensure_growth()
        admitted = self._admit(need)
        if not self.running and self.waiting:
            req = self.waiting[0]
            raise MemoryError(
                f"request {req.req_id} ({req.num_tokens} tokens) does not fit "
                f"in an empty pool of {self.num_blocks} blocks")
        chunks = self._prefill_chunks()
        prefill = self._write_prompts(chunks)
        if chunks:
            self._prefilling = [r for r in self._prefilling
                                if r.written < r.num_tokens]
        cached = sum(c for _, c in admitted)
        # requests whose tokens are all stored decode this step
        batch = [r for r in self.running if r.written >= r.num_tokens] \
            if self._prefilling else list(self.running)
        finished = 0
        if batch:
            tokens = self.rng.integers(1 << 17, size=len(batch)).tolist()
            slots = self.mgr.append_slots([r.req_id for r in batch], tokens)
            copies = self.mgr.take_copies()
            assert not copies, "running requests never share a partial block"
            self._decode(batch, slots)
            # the sampled token (kept as the request's output when the
            # manager keeps token ids, for the prefix cache)
            keep = self.prefix_caching
            done = []
            for r, t in zip(batch, tokens):
                r.output_ids.append(t if keep else 0)
                r.num_tokens += 1
                r.written += 1
                if len(r.output_ids) >= r.max_new_tokens:
                    done.append(r)
            # only requests that decoded can finish; they leave in running
            # order (the order their blocks return to the free queue)
            for r in done:
                self.mgr.free_seq(r.req_id)
                r.finished_step = self.step_no
                self.finished.append(r)
            finished = len(done)
            if done:
                self.running = [r for r in self.running if not r.done]
        st = StepStats(
            step=self.step_no, running=len(batch), waiting=len(self.waiting),
            admitted=len(admitted), preempted=preempted, finished=finished,
            prefill_tokens=prefill, prefill_chunks=len(chunks),
            cached_prefix_tokens=cached,
            blocks_used=self.num_blocks - self.mgr.num_free,
            slots_used=sum(r.num_tokens for r in self.running))
        self.step_no += 1
        return st

    def _decode(self, batch, slots) -> None:
        self.last_batch = [r.req_id for r in batch]
        if self.device is None and not self.mirror:
            return
        import torch
        ids = [r.req_id for r in batch]
        tables, lens = self.mgr.tables(ids)
        n = len(batch)
        if self.mirror or self.device is None:
            g = torch.Generator().manual_seed(int(self.rng.integers(1 << 62)))
            q = torch.randn(n, self.hq, self.d, generator=g).to(
                torch.bfloat16)
        else:
            q = self._device_rows(n, "q")
        kn, vn = self._random_rows(n)
        if self.mirror:
            self._record_write(kn, vn, np.asarray(slots, dtype=np.int32))
            self.last_q = q
            self.last_tables, self.last_lens = tables, lens
        if self.device is None:
            return
        from . import _lib
        dev = self.device
        out = torch.empty(n, self.hq, self.d, dtype=torch.bfloat16,
                          device=dev)
        d_tables, d_lens, d_slots = self._upload(
            tables, lens.astype(np.int32), np.asarray(slots, dtype=np.int32))
        args = (q.to(dev), self.k_pool, self.v_pool, d_tables, d_lens,
                self.scale, out, kn.to(dev), vn.to(dev), d_slots)
        desc = _lib.decode_desc(args[0], self.k_pool, args[3],
                                max_seq_len=int(lens.max()),
                                total_blocks_hint=int(((lens + 15) // 16)
                                                      .sum()))
        ws = _lib.alloc_workspace(desc, dev, fused=True)
        if self.time_decode:
            # the events bracket the two kernels only (inputs are on the
            # device already)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        _lib.pa_decode_append(*args, max_seq_len=int(lens.max()),
                              workspace=ws, desc=desc)
        if self.time_decode:
            e1.record()
            self.decode_events.append(
                (e0, e1, int(lens.sum()) * self.hkv * self.d * 2 * 2))
        self.last_out = out

    def _record_write(self, k, v, slots) -> None:
        import torch
        self.last_writes.append((k.view(torch.uint16).numpy().copy(),
                                 v.view(torch.uint16).numpy().copy(),
                                 np.array(slots, dtype=np.int32)))
