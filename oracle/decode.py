"""Paged single-token decode attention, float64.

What is computed (restated from the pages):

* A sequence's K/V are stored in fixed 16-token blocks anywhere in a shared
  pool; its block table maps logical block ``t // 16`` to a physical block,
  and token ``t`` sits at offset ``t % 16`` inside it ("49 vLLM /
  PagedAttention", section "Идея и механизм"; "PagedAttention：KV cache 即虚拟
  内存", section "直接答案").
* Paging changes neither the result nor the arithmetic: the kernel computes
  the same attention as over a contiguous cache ("PagedAttention：KV cache 即
  虚拟内存", sections "直接答案" and "面试官追问").

So the oracle first gathers each sequence's blocks into a contiguous
[L, Hkv, D] buffer, then evaluates ordinary attention of the one new query
token over all L cached tokens (no mask: decode attends to the whole
context), in float64:

    s_t = scale * <q_h, K_t>,  w = softmax(s),  out_h = sum_t w_t V_t

Readings where the pages are silent:

* storage layout: ``k_pool`` [NB, Hkv, 16, D], ``v_pool`` [NB, Hkv, D, 16];
* grouped-query attention: query head ``h`` reads KV head ``h // (Hq/Hkv)``;
* ``scale`` is the float32 value the caller passes, widened exactly;
* fp8 pools hold ``K / k_scale`` and ``V / v_scale``; the oracle multiplies
  the decoded values back by the per-tensor scales;
* ``seq_len == 0`` gives an all-zero output row.
"""
import numpy as np

from .numerics import widen

BLOCK_SIZE = 16


def _kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    return h // (num_q_heads // num_kv_heads)


def gather_sequence(k_raw, v_raw, table_row, seq_len, kv_dtype,
                    k_scale=1.0, v_scale=1.0):
    """Contiguous float64 K and V, each [seq_len, Hkv, D], of one sequence."""
    nblk = -(-int(seq_len) // BLOCK_SIZE)
    phys = np.asarray(table_row[:nblk], dtype=np.int64)
    kb = k_raw[phys]                    # [nblk, Hkv, 16, D]
    vb = v_raw[phys]                    # [nblk, Hkv, D, 16]
    kc = kb.transpose(0, 2, 1, 3)       # [nblk, 16, Hkv, D]
    vc = vb.transpose(0, 3, 1, 2)       # [nblk, 16, Hkv, D]
    hkv, d = kc.shape[2], kc.shape[3]
    kc = kc.reshape(nblk * BLOCK_SIZE, hkv, d)[:seq_len]
    vc = vc.reshape(nblk * BLOCK_SIZE, hkv, d)[:seq_len]
    k = widen(kc, kv_dtype) * np.float64(k_scale)
    v = widen(vc, kv_dtype) * np.float64(v_scale)
    return k, v


def attention_weights(q, k_raw, v_raw, block_tables, seq_lens, scale, *,
                      q_dtype, kv_dtype, k_scale=1.0, v_scale=1.0, seq=0):
    """Softmax weights [Hq, L] of one sequence (for the sum-to-one check)."""
    qf = widen(q[seq], q_dtype)
    hq = qf.shape[0]
    k, _ = gather_sequence(k_raw, v_raw, block_tables[seq], seq_lens[seq],
                           kv_dtype, k_scale, v_scale)
    hkv = k.shape[1]
    sc = np.float64(np.float32(scale))
    w = np.empty((hq, k.shape[0]))
    for h in range(hq):
        g = _kv_head_of(h, hq, hkv)
        s = sc * (k[:, g, :] @ qf[h])
        e = np.exp(s - s.max())
        w[h] = e / e.sum()
    return w


def paged_decode(q, k_raw, v_raw, block_tables, seq_lens, scale, *,
                 q_dtype, kv_dtype, k_scale=1.0, v_scale=1.0, seqs=None):
    """Decode attention output, float64 [B, Hq, D] (rows outside ``seqs`` are
    left NaN when only a sample of sequences is requested)."""
    b, hq, d = q.shape
    hkv = k_raw.shape[1]
    sc = np.float64(np.float32(scale))
    out = np.full((b, hq, d), np.nan)
    for i in (range(b) if seqs is None else seqs):
        n = int(seq_lens[i])
        if n <= 0:
            out[i] = 0.0
            continue
        qf = widen(q[i], q_dtype)
        k, v = gather_sequence(k_raw, v_raw, block_tables[i], n, kv_dtype,
                               k_scale, v_scale)
        for h in range(hq):
            g = _kv_head_of(h, hq, hkv)
            s = sc * (k[:, g, :] @ qf[h])
            e = np.exp(s - s.max())
            w = e / e.sum()
            out[i, h] = w @ v[:, g, :]
    return out
