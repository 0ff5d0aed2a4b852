"""Paged chunked-prefill attention, float64.

Prefill runs the prompt's tokens through the model, and a scheduler may cut
a long prompt into chunks mixed with decode work ("vLLM innenfra", step()
loop and continuous-batching paragraphs: chunked prefill); prefill is
usually compute-bound.  Attention of a chunk reads the same paged pool as
decode: the chunk's own K/V are appended first, then every query token of
the chunk attends to all cached tokens before it and to the chunk's tokens
up to itself (causal).  As for decode, paging changes nothing in the result
("PagedAttention：KV cache 即虚拟内存", section "直接答案").

So for sequence b with L_b cached tokens (the chunk included) and a chunk of
C_b query tokens, query token i (0 <= i < C_b) sits at position
p = L_b - C_b + i and

    out[i, h] = sum_{t <= p} softmax_t(scale * <q[i, h], K_t>) V_t

with K_t, V_t of KV head h // (Hq / Hkv), gathered through the block table
exactly as in ``decode.gather_sequence``.  Queries are packed over the
batch: rows q_start[b] .. q_start[b+1] of q belong to sequence b.
Test infrastructure, not product code.
"""
import numpy as np

from .decode import _kv_head_of, gather_sequence
from .numerics import widen


def paged_prefill(q, k_raw, v_raw, block_tables, seq_lens, q_start, scale, *,
                  q_dtype, kv_dtype, k_scale=1.0, v_scale=1.0, seqs=None):
    """Chunked-prefill attention output, float64 [T, Hq, D] (rows of
    sequences outside ``seqs`` are left NaN)."""
    t_all, hq, d = q.shape
    hkv = k_raw.shape[1]
    sc = np.float64(np.float32(scale))
    out = np.full((t_all, hq, d), np.nan)
    q_start = np.asarray(q_start)
    for b in (range(len(seq_lens)) if seqs is None else seqs):
        lo, hi = int(q_start[b]), int(q_start[b + 1])
        c, n = hi - lo, int(seq_lens[b])
        if c <= 0:
            continue
        if c > n:
            raise ValueError("a chunk longer than its sequence")
        k, v = gather_sequence(k_raw, v_raw, block_tables[b], n, kv_dtype,
                               k_scale, v_scale)
        qf = widen(q[lo:hi], q_dtype)            # [C, Hq, D]
        for i in range(c):
            p = n - c + i
            for h in range(hq):
                g = _kv_head_of(h, hq, hkv)
                s = sc * (k[:p + 1, g, :] @ qf[i, h])
                e = np.exp(s - s.max())
                out[lo + i, h] = (e / e.sum()) @ v[:p + 1, g, :]
    return out


def prefill_flops(seq_lens, q_start, num_q_heads, head_size) -> int:
    """Multiply-adds x 2 of the causal QK^T and PV products actually needed:
    4 * D * Hq per (query, attended key) pair."""
    total = 0
    q_start = np.asarray(q_start)
    for b, n in enumerate(np.asarray(seq_lens).tolist()):
        c = int(q_start[b + 1] - q_start[b])
        # keys attended by query i: n - c + i + 1, for i in [0, c)
        total += c * (n - c + 1) + c * (c - 1) // 2
    return 4 * head_size * num_q_heads * total
