"""ctypes binding of libpa.so (argument marshalling only).

Every entry point takes torch tensors that already live on the GPU, passes
their device pointers and the current HIP stream to the C ABI declared in
``include/pa.h``, and raises ``RuntimeError`` on a non-zero status.  The work
itself runs in the library's HIP kernels; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32, PA_BF16, PA_FP8_E4M3FN = 0, 1, 2
_DTYPE = {
    torch.float32: PA_F32,
    torch.bfloat16: PA_BF16,
    torch.float8_e4m3fn: PA_FP8_E4M3FN,
}

# names every build of the library exports (checked by the tests)
EXPORTS = ("pa_decode", "pa_decode_workspace_size", "pa_decode_append",
           "pa_decode_append_workspace_size", "pa_decode_append_shared",
           "pa_decode_append_shared_workspace_size", "pa_kv_append",
           "pa_kv_append_quant", "pa_copy_blocks", "pa_prefill",
           "pa_status_string", "pa_abi_version", "pa_decode_append_noalloc")


class DecodeDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("q_dtype", ctypes.c_int),
        ("kv_dtype", ctypes.c_int),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("total_blocks_hint", ctypes.c_int64),
        ("num_waves", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("profile_events", ctypes.c_void_p * 2),
    ]


class AppendDesc(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int),
    ]


class CopyDesc(ctypes.Structure):
    _fields_ = [
        ("num_pairs", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int),
    ]


class PrefillDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_query_tokens", ctypes.c_int32),
        ("q_dtype", ctypes.c_int),
        ("kv_dtype", ctypes.c_int),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpa.so (built by ``python -m paged_kv_cache_451_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m paged_kv_cache_451_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.pa_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeDesc)]
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_decode.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp,
                              ctypes.POINTER(DecodeDesc), vp, sz, vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_append_workspace_size.argtypes = [
        ctypes.POINTER(DecodeDesc)]
    lib.pa_decode_append_workspace_size.restype = sz
    lib.pa_decode_append.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                     vp, vp, vp, ctypes.POINTER(DecodeDesc),
                                     vp, sz, vp]
    lib.pa_decode_append.restype = ctypes.c_int
    lib.pa_decode_append_noalloc.argtypes = [
        vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp,
        ctypes.POINTER(DecodeDesc), vp]
    lib.pa_decode_append_noalloc.restype = ctypes.c_int
    lib.pa_decode_append_shared_workspace_size.argtypes = [
        ctypes.POINTER(DecodeDesc)]
    lib.pa_decode_append_shared_workspace_size.restype = sz
    lib.pa_decode_append_shared.argtypes = [
        vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp,
        ctypes.c_int32, ctypes.POINTER(DecodeDesc), vp, sz, vp]
    lib.pa_decode_append_shared.restype = ctypes.c_int
    lib.pa_kv_append.argtypes = [vp, vp, vp, vp, vp,
                                 ctypes.POINTER(AppendDesc), vp]
    lib.pa_kv_append.restype = ctypes.c_int
    lib.pa_kv_append_quant.argtypes = [vp, vp, vp, vp, vp,
                                       ctypes.POINTER(AppendDesc),
                                       ctypes.c_float, ctypes.c_float, vp]
    lib.pa_kv_append_quant.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, vp, ctypes.POINTER(CopyDesc),
                                   vp]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_prefill.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                               ctypes.POINTER(PrefillDesc), vp]
    lib.pa_prefill.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_abi_version.argtypes = []
    lib.pa_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load().pa_status_string(status).decode()
        raise RuntimeError(f"libpa error {status}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libpa takes GPU tensors only")
    if not t.is_contiguous():
        raise ValueError("libpa takes contiguous tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# -- argument checks (before any pointer is taken) ----------------------------
def _int32(name: str, t: Optional[torch.Tensor], n: Optional[int] = None,
           ndim: int = 1) -> None:
    """An index tensor must be int32 (the C ABI reads 32-bit entries; torch's
    default int64 would be read as pairs of words), with ``ndim`` dimensions
    and, when given, ``n`` entries along the first."""
    if t is None:
        return
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimension(s), "
                         f"got shape {tuple(t.shape)}")
    if n is not None and t.shape[0] != n:
        raise ValueError(f"{name} must have {n} entries along its first "
                         f"dimension, got {t.shape[0]}")


def _pools(k_pool: torch.Tensor, v_pool: torch.Tensor):
    """Pool shapes: K [NB, Hkv, 16, D] and V [NB, Hkv, D, 16], same dtype."""
    if k_pool.dim() != 4 or v_pool.dim() != 4:
        raise ValueError("k_pool and v_pool must be 4-dimensional")
    nb, hkv, bs, d = k_pool.shape
    if tuple(v_pool.shape) != (nb, hkv, d, bs):
        raise ValueError(f"v_pool must have shape {(nb, hkv, d, bs)} "
                         f"(K's tile transposed), got {tuple(v_pool.shape)}")
    if v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool must have the same dtype")
    if k_pool.dtype not in _DTYPE:
        raise ValueError(f"unsupported pool dtype {k_pool.dtype}")
    return nb, hkv, bs, d


def _rows(name: str, t: Optional[torch.Tensor], n: int, hkv: int, d: int,
          dtype: torch.dtype) -> None:
    """New-token rows: [n, Hkv, D] of ``dtype``."""
    if t is None:
        return
    if tuple(t.shape) != (n, hkv, d):
        raise ValueError(f"{name} must have shape {(n, hkv, d)}, got "
                         f"{tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _check_decode(q, k_pool, v_pool, block_tables, seq_lens, out,
                  k_new=None, v_new=None, slot_mapping=None) -> None:
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs, num_q_heads, head_size]")
    b, _, d = q.shape
    nb, hkv, _, d2 = _pools(k_pool, v_pool)
    if d2 != d:
        raise ValueError("head_size differs between q and the pools")
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported q dtype {q.dtype}")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    _int32("block_tables", block_tables, b, ndim=2)
    _int32("seq_lens", seq_lens, b)
    _int32("slot_mapping", slot_mapping, b)
    _rows("k_new", k_new, b, hkv, d, k_pool.dtype)
    _rows("v_new", v_new, b, hkv, d, k_pool.dtype)


def decode_desc(q: torch.Tensor, k_pool: torch.Tensor,
                block_tables: torch.Tensor, *, max_seq_len: int,
                k_scale: float = 1.0, v_scale: float = 1.0,
                total_blocks_hint: int = 0, num_waves: int = 0,
                events: Optional[Sequence] = None) -> DecodeDesc:
    b, hq, d = q.shape
    nb, hkv, bs, d2 = k_pool.shape
    if d2 != d:
        raise ValueError("head_size mismatch between q and k_pool")
    desc = DecodeDesc(
        num_seqs=b, num_q_heads=hq, num_kv_heads=hkv, head_size=d,
        block_size=bs, num_blocks=nb,
        max_blocks_per_seq=block_tables.shape[1], max_seq_len=max_seq_len,
        q_dtype=_DTYPE[q.dtype], kv_dtype=_DTYPE[k_pool.dtype],
        k_scale=k_scale, v_scale=v_scale,
        total_blocks_hint=total_blocks_hint, num_waves=num_waves,
        reserved=0)
    if events is not None:
        desc.profile_events[0] = events[0]
        desc.profile_events[1] = events[1]
    return desc


def workspace_size(desc: DecodeDesc, fused: bool = False,
                   shared: bool = False) -> int:
    lib = load()
    if shared:
        fn = lib.pa_decode_append_shared_workspace_size
    elif fused:
        fn = lib.pa_decode_append_workspace_size
    else:
        fn = lib.pa_decode_workspace_size
    return int(fn(ctypes.byref(desc)))


def alloc_workspace(desc: DecodeDesc, device=None, fused: bool = False,
                    shared: bool = False) -> torch.Tensor:
    n = max(workspace_size(desc, fused, shared), 256)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def pa_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out, *,
              max_seq_len: int, k_scale: float = 1.0, v_scale: float = 1.0,
              total_blocks_hint: int = 0, num_waves: int = 0,
              workspace: Optional[torch.Tensor] = None,
              events: Optional[Sequence] = None,
              desc: Optional[DecodeDesc] = None) -> torch.Tensor:
    """Paged decode attention into ``out`` (see ``include/pa.h``)."""
    _check_decode(q, k_pool, v_pool, block_tables, seq_lens, out)
    lib = load()
    if desc is None:
        desc = decode_desc(q, k_pool, block_tables, max_seq_len=max_seq_len,
                           k_scale=k_scale, v_scale=v_scale,
                           total_blocks_hint=total_blocks_hint,
                           num_waves=num_waves, events=events)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device)
    _check(lib.pa_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool),
                         _ptr(block_tables), _ptr(seq_lens),
                         ctypes.c_float(scale), _ptr(out), ctypes.byref(desc),
                         _ptr(workspace), workspace.numel(), _stream()))
    return out


def pa_decode_append(q, k_pool, v_pool, block_tables, seq_lens, scale, out,
                     k_new, v_new, slot_mapping, *, max_seq_len: int,
                     k_scale: float = 1.0, v_scale: float = 1.0,
                     total_blocks_hint: int = 0, num_waves: int = 0,
                     workspace: Optional[torch.Tensor] = None,
                     events: Optional[Sequence] = None,
                     desc: Optional[DecodeDesc] = None) -> torch.Tensor:
    """Append of each sequence's newest token fused with decode attention
    over the grown context (see ``include/pa.h``)."""
    _check_decode(q, k_pool, v_pool, block_tables, seq_lens, out, k_new,
                  v_new, slot_mapping)
    lib = load()
    if desc is None:
        desc = decode_desc(q, k_pool, block_tables, max_seq_len=max_seq_len,
                           k_scale=k_scale, v_scale=v_scale,
                           total_blocks_hint=total_blocks_hint,
                           num_waves=num_waves, events=events)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device, fused=True)
    _check(lib.pa_decode_append(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        _ptr(seq_lens), ctypes.c_float(scale), _ptr(out), _ptr(k_new),
        _ptr(v_new), _ptr(slot_mapping), ctypes.byref(desc), _ptr(workspace),
        workspace.numel(), _stream()))
    return out


def pa_decode_append_noalloc(q, k_pool, v_pool, block_tables, seq_lens,
                             scale, out, k_new, v_new, slot_mapping, *,
                             max_seq_len: int, k_scale: float = 1.0,
                             v_scale: float = 1.0, total_blocks_hint: int = 0,
                             num_waves: int = 0,
                             desc: Optional[DecodeDesc] = None
                             ) -> torch.Tensor:
    """pa_decode_append with the library's static scratch buffer instead of a
    workspace: allocates nothing (see ``include/pa.h``)."""
    _check_decode(q, k_pool, v_pool, block_tables, seq_lens, out, k_new,
                  v_new, slot_mapping)
    lib = load()
    if desc is None:
        desc = decode_desc(q, k_pool, block_tables, max_seq_len=max_seq_len,
                           k_scale=k_scale, v_scale=v_scale,
                           total_blocks_hint=total_blocks_hint,
                           num_waves=num_waves)
    _check(lib.pa_decode_append_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        _ptr(seq_lens), ctypes.c_float(scale), _ptr(out), _ptr(k_new),
        _ptr(v_new), _ptr(slot_mapping), ctypes.byref(desc), _stream()))
    return out


def pa_decode_append_shared(q, k_pool, v_pool, block_tables, seq_lens, scale,
                            out, k_new, v_new, slot_mapping, group_start,
                            group_prefix_blocks, *, max_seq_len: int,
                            k_scale: float = 1.0, v_scale: float = 1.0,
                            total_blocks_hint: int = 0, num_waves: int = 0,
                            workspace: Optional[torch.Tensor] = None,
                            events: Optional[Sequence] = None,
                            desc: Optional[DecodeDesc] = None
                            ) -> torch.Tensor:
    """Cascade form of the fused step: shared prompt prefixes read once per
    group of sequences (see ``include/pa.h``)."""
    _check_decode(q, k_pool, v_pool, block_tables, seq_lens, out, k_new,
                  v_new, slot_mapping)
    if (group_start is None) != (group_prefix_blocks is None):
        raise ValueError("group_start and group_prefix_blocks go together")
    if group_start is not None:
        _int32("group_start", group_start)
        _int32("group_prefix_blocks", group_prefix_blocks,
               group_start.numel() - 1)
    lib = load()
    if desc is None:
        desc = decode_desc(q, k_pool, block_tables, max_seq_len=max_seq_len,
                           k_scale=k_scale, v_scale=v_scale,
                           total_blocks_hint=total_blocks_hint,
                           num_waves=num_waves, events=events)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device, fused=True, shared=True)
    ng = 0 if group_start is None else group_start.numel() - 1
    _check(lib.pa_decode_append_shared(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        _ptr(seq_lens), ctypes.c_float(scale), _ptr(out), _ptr(k_new),
        _ptr(v_new), _ptr(slot_mapping), _ptr(group_start),
        _ptr(group_prefix_blocks), ng, ctypes.byref(desc), _ptr(workspace),
        workspace.numel(), _stream()))
    return out


def pa_kv_append(k_new, v_new, slot_mapping, k_pool, v_pool) -> None:
    """Write new tokens' K/V into their pool slots (see ``include/pa.h``)."""
    _, hkv, _, d = _pools(k_pool, v_pool)
    n = k_new.shape[0] if k_new.dim() == 3 else -1
    _rows("k_new", k_new, n, hkv, d, k_pool.dtype)
    _rows("v_new", v_new, n, hkv, d, k_pool.dtype)
    _int32("slot_mapping", slot_mapping, n)
    lib = load()
    desc = AppendDesc(num_tokens=n, num_kv_heads=hkv, head_size=d,
                      block_size=k_pool.shape[2], num_blocks=k_pool.shape[0],
                      kv_dtype=_DTYPE[k_pool.dtype])
    _check(lib.pa_kv_append(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                            _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc),
                            _stream()))


def pa_kv_append_quant(k_new, v_new, slot_mapping, k_pool, v_pool,
                       k_scale: float, v_scale: float) -> None:
    """Write bf16 rows into an fp8 e4m3fn pool as value / scale codes (see
    ``include/pa.h``)."""
    if k_pool.dtype != torch.float8_e4m3fn:
        raise ValueError("pa_kv_append_quant takes bf16 rows and fp8 pools")
    _, hkv, _, d = _pools(k_pool, v_pool)
    n = k_new.shape[0] if k_new.dim() == 3 else -1
    _rows("k_new", k_new, n, hkv, d, torch.bfloat16)
    _rows("v_new", v_new, n, hkv, d, torch.bfloat16)
    _int32("slot_mapping", slot_mapping, n)
    lib = load()
    desc = AppendDesc(num_tokens=n, num_kv_heads=hkv, head_size=d,
                      block_size=k_pool.shape[2], num_blocks=k_pool.shape[0],
                      kv_dtype=PA_FP8_E4M3FN)
    _check(lib.pa_kv_append_quant(
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_pool),
        _ptr(v_pool), ctypes.byref(desc), ctypes.c_float(k_scale),
        ctypes.c_float(v_scale), _stream()))


def pa_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks) -> None:
    """Copy whole K/V blocks src -> dst (copy-on-write; see
    ``include/pa.h``)."""
    nb, hkv, bs, d = _pools(k_pool, v_pool)
    _int32("src_blocks", src_blocks)
    _int32("dst_blocks", dst_blocks, src_blocks.numel())
    lib = load()
    desc = CopyDesc(num_pairs=src_blocks.numel(), num_kv_heads=hkv,
                    head_size=d, block_size=bs, num_blocks=nb,
                    kv_dtype=_DTYPE[k_pool.dtype])
    _check(lib.pa_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(src_blocks),
                              _ptr(dst_blocks), ctypes.byref(desc),
                              _stream()))


def prefill_desc(q, k_pool, block_tables, num_seqs: int, *,
                 k_scale: float = 1.0, v_scale: float = 1.0) -> PrefillDesc:
    t, hq, d = q.shape
    nb, hkv, bs, _ = k_pool.shape
    return PrefillDesc(num_seqs=num_seqs, num_q_heads=hq, num_kv_heads=hkv,
                       head_size=d, block_size=bs, num_blocks=nb,
                       max_blocks_per_seq=block_tables.shape[1],
                       num_query_tokens=t, q_dtype=_DTYPE[q.dtype],
                       kv_dtype=_DTYPE[k_pool.dtype], k_scale=k_scale,
                       v_scale=v_scale)


def pa_prefill(q, k_pool, v_pool, block_tables, seq_lens, q_start, scale,
               out, desc: Optional[PrefillDesc] = None, *,
               k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """Chunked-prefill attention into ``out`` (see ``include/pa.h``)."""
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must be [tokens, num_q_heads, head_size] "
                         "of one dtype")
    _pools(k_pool, v_pool)
    b = seq_lens.shape[0] if seq_lens.dim() == 1 else -1
    _int32("seq_lens", seq_lens, b)
    _int32("block_tables", block_tables, b, ndim=2)
    _int32("q_start", q_start, b + 1)
    lib = load()
    if desc is None:
        desc = prefill_desc(q, k_pool, block_tables, seq_lens.numel(),
                            k_scale=k_scale, v_scale=v_scale)
    _check(lib.pa_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool),
                          _ptr(block_tables), _ptr(seq_lens), _ptr(q_start),
                          ctypes.c_float(scale), _ptr(out),
                          ctypes.byref(desc), _stream()))
    return out


class PreparedStep:
    """A decode step (append, then decode; or both in ``pa_decode_append``
    when ``fused``) with its C arguments marshalled once, for replaying the
    same call many times (benchmarks, serving loops).  Holds references to
    every tensor it points at."""

    def __init__(self, q, k_pool, v_pool, block_tables, seq_lens, scale, out,
                 desc: DecodeDesc, workspace: torch.Tensor,
                 k_new=None, v_new=None, slot_mapping=None,
                 fused: bool = False, shared=None):
        _check_decode(q, k_pool, v_pool, block_tables, seq_lens, out,
                      k_new if (fused or shared is not None) else None,
                      v_new if (fused or shared is not None) else None,
                      slot_mapping if (fused or shared is not None) else None)
        if shared is not None:
            _int32("group_start", shared[0])
            _int32("group_prefix_blocks", shared[1], shared[0].numel() - 1)
        lib = load()
        self._keep = (q, k_pool, v_pool, block_tables, seq_lens, out,
                      workspace, k_new, v_new, slot_mapping, desc, shared)
        stream = _stream()
        self._append = None
        if shared is not None:  # (group_start, group_prefix_blocks)
            if k_new is None:
                raise ValueError("the cascade step needs k_new/v_new/slots")
            gs, gp = shared
            self._decode = lib.pa_decode_append_shared
            self._decode_args = (
                _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
                _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(gs),
                _ptr(gp), gs.numel() - 1, ctypes.byref(desc),
                _ptr(workspace), workspace.numel(), stream)
            return
        if fused:
            if k_new is None:
                raise ValueError("the fused step needs k_new/v_new/slots")
            self._decode = lib.pa_decode_append
            self._decode_args = (
                _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
                _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                ctypes.byref(desc), _ptr(workspace), workspace.numel(),
                stream)
            return
        self._decode = lib.pa_decode
        self._decode_args = (
            _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
            _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
            ctypes.byref(desc), _ptr(workspace), workspace.numel(), stream)
        if k_new is not None:
            n, hkv, d = k_new.shape
            self._adesc = AppendDesc(
                num_tokens=n, num_kv_heads=hkv, head_size=d,
                block_size=k_pool.shape[2], num_blocks=k_pool.shape[0],
                kv_dtype=_DTYPE[k_pool.dtype])
            self._append = lib.pa_kv_append
            self._append_args = (
                _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_pool),
                _ptr(v_pool), ctypes.byref(self._adesc), stream)

    def __call__(self) -> None:
        if self._append is not None:
            _check(self._append(*self._append_args))
        _check(self._decode(*self._decode_args))
