"""KV append: write each new token's K and V into its pool slot, bytewise.

The pages' append step takes a fresh block only when the last one is full and
then writes the token's KV into the sequence's last block ("49 vLLM /
PagedAttention", listing "Таблица блоков"); the slot the harness computes is
``phys * 16 + offset``.  Here: for token ``i`` with ``slot = slot_mapping[i]``,
``k_pool[slot // 16, :, slot % 16, :] = k_new[i]`` and
``v_pool[slot // 16, :, :, slot % 16] = v_new[i]`` (layouts [NB, Hkv, 16, D]
and [NB, Hkv, D, 16]).  Negative slots, and slots past the pool, are skipped.
The arrays are raw storage bits, so the copy is exact.

``copy_blocks`` is the copy-on-write step: a sequence that appends into a
block other sequences still share gets its own copy first ("49 vLLM /
PagedAttention", section "Почему это важно"): whole K and V blocks, byte for
byte, skipping pairs with an id outside the pool.
"""
import numpy as np

BLOCK_SIZE = 16


def kv_append(k_pool, v_pool, k_new, v_new, slot_mapping):
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    nslots = k.shape[0] * BLOCK_SIZE
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0 or slot >= nslots:
            continue
        phys, off = divmod(slot, BLOCK_SIZE)
        k[phys, :, off, :] = k_new[i]
        v[phys, :, :, off] = v_new[i]
    return k, v


def copy_blocks(k_pool, v_pool, src, dst):
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    nb = k.shape[0]
    for s, t in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        if 0 <= s < nb and 0 <= t < nb:
            k[t] = k_pool[s]
            v[t] = v_pool[s]
    return k, v
