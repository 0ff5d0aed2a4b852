"""Glue from generated cases (torch CPU tensors) to the oracle's arguments.

The oracle reads raw storage bits; these helpers take the bytes of a tensor
as a numpy array (float32, or uint16 for bf16, or uint8 for fp8 e4m3fn) and
apply the oracle's own append to a case's pools.
"""
import numpy as np
import torch

from .append import kv_append

_RAW_VIEW = {
    torch.float32: (torch.float32, "f32"),
    torch.bfloat16: (torch.uint16, "bf16"),
    torch.float8_e4m3fn: (torch.uint8, "fp8_e4m3fn"),
}


def raw(t: torch.Tensor):
    """Host numpy array of a tensor's storage bits plus its dtype name."""
    view, name = _RAW_VIEW[t.dtype]
    return t.detach().cpu().contiguous().view(view).numpy(), name


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """Bytes of a tensor as uint8 (for bit-exact comparisons)."""
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def oracle_args(case, k_pool=None, v_pool=None):
    """Keyword arguments of ``paged_decode`` for a generated decode case."""
    q, q_dtype = raw(case.q)
    k, kv_dtype = raw(case.k_pool if k_pool is None else k_pool)
    v, _ = raw(case.v_pool if v_pool is None else v_pool)
    return dict(q=q, k_raw=k, v_raw=v,
                block_tables=case.block_tables.numpy(),
                seq_lens=case.seq_lens.numpy(), scale=case.scale,
                q_dtype=q_dtype, kv_dtype=kv_dtype,
                k_scale=case.k_scale, v_scale=case.v_scale)


def appended_pools(case):
    """Raw K/V pools after the oracle's append of the case's new tokens."""
    k, _ = raw(case.k_pool)
    v, _ = raw(case.v_pool)
    kn, _ = raw(case.k_new)
    vn, _ = raw(case.v_new)
    return kv_append(k, v, kn, vn, case.slot_mapping.numpy())


def prefill_args(case, seqs=None):
    """Keyword arguments of ``paged_prefill`` for a generated prefill case."""
    q, q_dtype = raw(case.q)
    k, kv_dtype = raw(case.k_pool)
    v, _ = raw(case.v_pool)
    return dict(q=q, k_raw=k, v_raw=v,
                block_tables=case.block_tables.numpy(),
                seq_lens=case.seq_lens.numpy(),
                q_start=case.q_start.numpy(), scale=case.scale,
                q_dtype=q_dtype, kv_dtype=kv_dtype,
                k_scale=getattr(case, "k_scale", 1.0),
                v_scale=getattr(case, "v_scale", 1.0), seqs=seqs)
