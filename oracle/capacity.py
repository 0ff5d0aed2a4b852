"""Block/byte arithmetic and the contiguous-vs-paged capacity example.

* Bytes of one block: 2 (K and V) x block_size x KV heads x head size x bytes
  per element ("vLLM innenfra", KV-cache-manager paragraph).
* Elements of one request's cache: 2 x layers x heads x head dim x tokens
  ("49 vLLM / PagedAttention", section "Пейджинг для KV-кэша").
* Capacity example ("PagedAttention：KV cache 即虚拟内存", section "代码"): a
  contiguous cache reserves ceil(MAX_LEN / BLOCK) blocks per sequence, so a
  pool holds POOL // that many; a paged cache takes ceil(len / BLOCK) blocks
  per sequence.  Two admission rules are written out: first-come-first-served
  that stops at the first request that does not fit, and skip-and-continue,
  which admits any later request that still fits.
"""
import bisect
import itertools
import math


def block_bytes(block_size, num_kv_heads, head_size, dtype_bytes):
    return 2 * block_size * num_kv_heads * head_size * dtype_bytes


def request_kv_elements(num_layers, num_heads, head_dim, num_tokens):
    return 2 * num_layers * num_heads * head_dim * num_tokens


def contiguous_capacity(pool_blocks, block, max_len):
    return pool_blocks // math.ceil(max_len / block)


def _block_needs(block, lens):
    """Blocks each request takes under paging: ceil(len / block)."""
    return [-(-int(n) // block) for n in lens]


def paged_capacity_fcfs(pool_blocks, block, lens):
    """First come first served: requests are admitted in order while the
    running total of their block needs fits in the pool; the first request
    that would overflow it stops admission.  Returns (admitted, blocks)."""
    totals = list(itertools.accumulate(_block_needs(block, lens)))
    admitted = bisect.bisect_right(totals, pool_blocks)
    return admitted, (totals[admitted - 1] if admitted else 0)


def paged_capacity_skip(pool_blocks, block, lens):
    """Skip-and-continue: a request that does not fit in the blocks still
    free is passed over and later, smaller requests may still be admitted.
    Returns (admitted, blocks)."""
    free, admitted = pool_blocks, []
    for i, need in enumerate(_block_needs(block, lens)):
        admitted.append(need <= free)
        free -= need if admitted[-1] else 0
    return sum(admitted), pool_blocks - free
