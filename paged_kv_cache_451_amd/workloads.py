"""Seeded synthetic decode workloads: block tables, lengths and q/K/V pools.

This module only *generates inputs*; it holds none of the attention or append
arithmetic.  Both the device path and the CPU oracle consume what it returns.

Storage layout of one decode step (the library boundary):

* ``q``            [B, Hq, D]               q dtype (fp32 or bf16)
* ``k_pool``       [NB, Hkv, 16, D]         one block = per KV head a 16 x D
                                            token-major tile
* ``v_pool``       [NB, Hkv, D, 16]         one block = per KV head a D x 16
                                            tile (tokens contiguous)
* ``block_tables`` int32 [B, max_blocks]    physical block ids, padded with -1
* ``seq_lens``     int32 [B]                tokens attended, including the one
                                            appended this step
* ``slot_mapping`` int32 [B]                flat slot ``phys*16 + offset`` of
                                            each sequence's new token
* ``k_new/v_new``  [B, Hkv, D]              the new token's K and V

The pages fix only the byte count of a block (2 x block_size x KV heads x
head size x dtype bytes; "vLLM innenfra", KV-cache-manager paragraph), not
the order of the axes inside it; the order above is this library's choice.

Recipe (one ``numpy.random.SeedSequence(seed)``, children drawn in a fixed
order: lengths, free-queue permutation, q, K pool, V pool, k_new, v_new;
an eighth child draws the token ids of the prefix case):

* lengths: integers, ``uniform[a, b]`` inclusive, or lognormal rounded and
  clipped, or the fixed list of the tiny case;
* the free queue starts as a random permutation of all physical blocks, so
  consecutive logical blocks land on unrelated physical blocks;
* every sequence is admitted with ``seq_len - 1`` cached tokens (the prefix
  case: ``2048 + suffix``, with a shared prompt's token ids, so that the
  block manager's hash-keyed prefix cache maps every later sequence's first
  128 blocks to the first sequence's), then one token is appended through
  the pool's allocate-on-growth rule, which yields ``slot_mapping``;
* q, K, V, k_new, v_new ~ N(0, 1) drawn in float32, then rounded to the
  storage dtype (bf16: round-to-nearest-even; fp8 e4m3fn: divided by a
  per-tensor scale ``amax/448``, clamped to +-448, rounded to nearest even);
* pool size: used blocks + 10 % (rounded up), except the tiny case (128);
* every slot no sequence has written (free blocks, the tail of each last
  block and the new token's slot before the append) holds NaN, so a read of
  a slot outside the context shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from .pool import BlockPool, KVCacheManager

BLOCK_SIZE = 16

_TORCH_DTYPES = {
    "f32": torch.float32,
    "bf16": torch.bfloat16,
    "fp8_e4m3fn": torch.float8_e4m3fn,
}
DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}
FP8_MAX = 448.0


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    q_dtype: str
    kv_dtype: str
    lens: str                      # "fixed", "uniform", "lognormal", "prefix"
    fixed_lens: tuple = ()
    lo: int = 0                    # uniform / clip bounds, prefix suffix bounds
    hi: int = 0
    median: float = 0.0            # lognormal
    sigma: float = 0.0
    prefix_len: int = 0            # tokens of the shared prefix
    num_blocks: int = 0            # 0 = used blocks + 10 %
    scale: Optional[float] = None  # None = float32(1/sqrt(head_size))
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: List[DecodeConfig] = [
    DecodeConfig(
        "tiny_fp32", 4, 2, 2, 64, "f32", "f32", "fixed",
        fixed_lens=(40, 128, 300, 64), num_blocks=128, scale=0.125,
        description="4 seqs, lens [40,128,300,64], 2 q heads = 2 KV heads, "
                    "D=64, fp32, 128-block pool"),
    DecodeConfig(
        "llama3_8b_bf16", 64, 32, 8, 128, "bf16", "bf16", "uniform",
        lo=128, hi=4096,
        description="batch 64, 32 q / 8 KV heads, D=128, bf16, "
                    "lens uniform[128,4096]"),
    DecodeConfig(
        "skewed_bf16", 256, 64, 8, 128, "bf16", "bf16", "lognormal",
        lo=16, hi=32768, median=512.0, sigma=1.5,
        description="batch 256, 64 q / 8 KV heads, D=128, bf16, lens "
                    "lognormal(median 512, sigma 1.5) clipped to [16,32768]"),
    DecodeConfig(
        "prefix_shared_bf16", 128, 32, 8, 128, "bf16", "bf16", "prefix",
        lo=64, hi=1024, prefix_len=2048,
        description="128 seqs sharing a 2048-token prefix + suffix "
                    "uniform[64,1024], one appended token each, 32/8 heads, "
                    "D=128, bf16"),
    DecodeConfig(
        "fp8_long", 32, 32, 8, 128, "bf16", "fp8_e4m3fn", "uniform",
        lo=8192, hi=32768,
        description="batch 32, 32/8 heads, D=128, bf16 q, fp8 e4m3fn K/V "
                    "with per-tensor scales, lens uniform[8192,32768]"),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}


@dataclass
class DecodeCase:
    config: DecodeConfig
    seed: int
    q: torch.Tensor
    k_pool: torch.Tensor          # before the append (new slots hold NaN)
    v_pool: torch.Tensor
    block_tables: torch.Tensor    # int32 [B, max_blocks]
    seq_lens: torch.Tensor        # int32 [B], after the append
    slot_mapping: torch.Tensor    # int32 [B]
    k_new: torch.Tensor
    v_new: torch.Tensor
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    ref_cnt: np.ndarray = field(default=None)  # per physical block after admission

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def total_blocks(self) -> int:
        """Sum over sequences of ceil(seq_len / 16) (block-table entries read)."""
        return int(((self.seq_lens.to(torch.int64) + BLOCK_SIZE - 1)
                    // BLOCK_SIZE).sum())

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.numel() else 0


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------
_CHUNK = 1 << 24


def _normal_f32(ss: np.random.SeedSequence, shape) -> np.ndarray:
    """N(0,1) float32 of ``shape``, drawn in fixed 16 Mi-element chunks, each
    from its own child generator (deterministic for any thread count)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // _CHUNK))
    kids = ss.spawn(nchunks)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        np.random.default_rng(kids[i]).standard_normal(
            hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(8, nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def draw_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    """Cached tokens per sequence *before* this step's append."""
    b = cfg.num_seqs
    if cfg.lens == "fixed":
        lens = np.asarray(cfg.fixed_lens[:b], dtype=np.int64)
        if len(lens) != b:
            raise ValueError("fixed_lens shorter than num_seqs")
        return lens - 1
    if cfg.lens == "uniform":
        return rng.integers(cfg.lo, cfg.hi, size=b, endpoint=True) - 1
    if cfg.lens == "lognormal":
        x = rng.lognormal(mean=math.log(cfg.median), sigma=cfg.sigma, size=b)
        return np.clip(np.rint(x), cfg.lo, cfg.hi).astype(np.int64) - 1
    if cfg.lens == "prefix":
        suffix = rng.integers(cfg.lo, cfg.hi, size=b, endpoint=True)
        return cfg.prefix_len + suffix
    raise ValueError(cfg.lens)


def _to_storage(x: np.ndarray, dtype: str, scale: float = 1.0) -> torch.Tensor:
    t = torch.from_numpy(x)
    if dtype == "fp8_e4m3fn":
        return (t / np.float32(scale)).clamp_(-FP8_MAX, FP8_MAX).to(
            torch.float8_e4m3fn)
    return t.to(_TORCH_DTYPES[dtype])


def _nan_of(dtype: str) -> torch.Tensor:
    if dtype == "fp8_e4m3fn":
        return torch.tensor([0x7F], dtype=torch.uint8).view(torch.float8_e4m3fn)
    return torch.tensor([float("nan")], dtype=_TORCH_DTYPES[dtype])


def build_case(cfg: DecodeConfig, seed: int = 0) -> DecodeCase:
    """Draw one decode step of ``cfg`` (see the module docstring)."""
    if cfg.num_q_heads % cfg.num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    kids = np.random.SeedSequence(seed).spawn(7)
    rng_len = np.random.default_rng(kids[0])
    rng_perm = np.random.default_rng(kids[1])

    existing = draw_lengths(cfg, rng_len)
    b, hkv, d = cfg.num_seqs, cfg.num_kv_heads, cfg.head_size
    final = existing + 1
    if cfg.lens == "prefix":
        prefix_blocks = cfg.prefix_len // BLOCK_SIZE
        used = prefix_blocks + int(sum(
            math.ceil(int(n) / BLOCK_SIZE) - prefix_blocks for n in final))
    else:
        used = int(sum(math.ceil(int(n) / BLOCK_SIZE) for n in final))
    nb = cfg.num_blocks or used + math.ceil(0.10 * used)
    if nb < used:
        raise ValueError(f"pool of {nb} blocks cannot hold {used}")

    pool = BlockPool(nb, order=rng_perm.permutation(nb))
    mgr = KVCacheManager(pool, BLOCK_SIZE)
    if cfg.lens == "prefix":
        if cfg.prefix_len % BLOCK_SIZE:
            raise ValueError("shared prefix must be whole blocks")
        # token ids: one shared prompt prefix, then per-sequence tokens; the
        # block manager's hash cache finds the prefix blocks for every
        # sequence after the first
        rng_tok = np.random.default_rng(
            np.random.SeedSequence(seed).spawn(8)[7])
        prefix_ids = rng_tok.integers(0, 1 << 17, size=cfg.prefix_len)
        for i in range(b):
            own = rng_tok.integers(0, 1 << 17,
                                   size=int(existing[i]) - cfg.prefix_len)
            ok, hits = mgr.admit_cached(i, np.concatenate([prefix_ids, own]))
            assert ok and hits == (0 if i == 0 else
                                   cfg.prefix_len // BLOCK_SIZE)
    else:
        for i in range(b):
            assert mgr.admit(i, int(existing[i]))
    ref_cnt = np.array([blk.ref_cnt for blk in pool.blocks], dtype=np.int32)
    slots = np.array([mgr.append_slot(i) for i in range(b)], dtype=np.int32)
    tables, lens = mgr.tables(range(b))
    assert np.array_equal(lens, final)

    q32 = _normal_f32(kids[2], (b, cfg.num_q_heads, d))
    k32 = _normal_f32(kids[3], (nb, hkv, BLOCK_SIZE, d))
    v32 = _normal_f32(kids[4], (nb, hkv, d, BLOCK_SIZE))
    kn32 = _normal_f32(kids[5], (b, hkv, d))
    vn32 = _normal_f32(kids[6], (b, hkv, d))

    k_scale = v_scale = 1.0
    if cfg.kv_dtype == "fp8_e4m3fn":
        k_scale = float(np.float32(max(np.abs(k32).max(), np.abs(kn32).max())
                                   / FP8_MAX))
        v_scale = float(np.float32(max(np.abs(v32).max(), np.abs(vn32).max())
                                   / FP8_MAX))
    q = _to_storage(q32, cfg.q_dtype)
    k_pool = _to_storage(k32, cfg.kv_dtype, k_scale)
    v_pool = _to_storage(v32, cfg.kv_dtype, v_scale)
    k_new = _to_storage(kn32, cfg.kv_dtype, k_scale)
    v_new = _to_storage(vn32, cfg.kv_dtype, v_scale)
    del q32, k32, v32, kn32, vn32

    # poison every slot that holds no cached token before the append
    written = np.zeros((nb, BLOCK_SIZE), dtype=bool)
    for i in range(b):
        n = int(existing[i])
        row = tables[i]
        nfull, rem = divmod(n, BLOCK_SIZE)
        written[row[:nfull]] = True
        if rem:
            written[row[nfull], :rem] = True
    free = torch.from_numpy(~written)
    nan = _nan_of(cfg.kv_dtype)
    blk_idx, tok_idx = torch.nonzero(free, as_tuple=True)
    k_pool[blk_idx, :, tok_idx, :] = nan
    v_pool[blk_idx, :, :, tok_idx] = nan

    scale = cfg.scale if cfg.scale is not None else float(
        np.float32(1.0 / math.sqrt(d)))
    return DecodeCase(
        config=cfg, seed=seed, q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=torch.from_numpy(tables),
        seq_lens=torch.from_numpy(lens.astype(np.int32)),
        slot_mapping=torch.from_numpy(slots), k_new=k_new, v_new=v_new,
        scale=scale, k_scale=k_scale, v_scale=v_scale, ref_cnt=ref_cnt)


def algorithmic_bytes(case: DecodeCase) -> dict:
    """Bytes the decode step must move at least once (no split-K partials):
    every cached token's K and V once per KV head, q in, out out, the block
    table entries read and the lengths; plus the append's read and write."""
    cfg = case.config
    lens = case.seq_lens.to(torch.int64)
    s_kv = DTYPE_BYTES[cfg.kv_dtype]
    s_q = DTYPE_BYTES[cfg.q_dtype]
    hkv, d, b = cfg.num_kv_heads, cfg.head_size, cfg.num_seqs
    kv = int(lens.sum()) * hkv * d * 2 * s_kv
    qo = b * cfg.num_q_heads * d * 2 * s_q
    tables = case.total_blocks * 4 + b * 4
    scales = 8 if cfg.kv_dtype == "fp8_e4m3fn" else 0
    append = 2 * (2 * b * hkv * d * s_kv) + 4 * b
    # unique KV bytes: each physical block a sequence reads counted once
    uniq_tokens = 0
    seen = set()
    tab = case.block_tables.numpy()
    for i in range(b):
        n = int(lens[i])
        for j in range(-(-n // BLOCK_SIZE)):
            p = int(tab[i, j])
            tok = min(BLOCK_SIZE, n - j * BLOCK_SIZE)
            if p in seen:
                continue
            seen.add(p)
            uniq_tokens += tok
    kv_unique = uniq_tokens * hkv * d * 2 * s_kv
    decode = kv + qo + tables + scales
    # the main pass of the fused step streams every cached token but the
    # newest (which the merge pass takes from k_new / v_new), reads q, the
    # table entries of those tokens and the lengths
    prev = (lens - 1).clamp(min=0)
    main_fused = (int(prev.sum()) * hkv * d * 2 * s_kv
                  + b * cfg.num_q_heads * d * s_q
                  + int(((prev + BLOCK_SIZE - 1) // BLOCK_SIZE).sum()) * 4
                  + b * 4 + scales)
    return {"kv": kv, "kv_unique": kv_unique, "decode": decode,
            "decode_unique": kv_unique + qo + tables + scales,
            "main_fused": main_fused,
            "append": append, "step": decode + append,
            "context_tokens": int(lens.sum())}


# --------------------------------------------------------------------------
# chunked prefill: a chunk of query tokens per sequence over the paged pool
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class PrefillConfig:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    chunk: int                     # query tokens per sequence
    prior_lo: int                  # cached tokens before the chunk:
    prior_hi: int                  #   uniform[prior_lo, prior_hi]
    description: str = ""
    kv_dtype: str = "bf16"         # or "fp8_e4m3fn" (per-tensor scales)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def replace(self, **kw) -> "PrefillConfig":
        return dataclasses.replace(self, **kw)


PREFILL_CONFIGS: List[PrefillConfig] = [
    PrefillConfig(
        "prefill_llama3_8b_bf16", 8, 32, 8, 128, chunk=512, prior_lo=0,
        prior_hi=3584,
        description="8 seqs, a 512-token chunk each after uniform[0,3584] "
                    "cached tokens, 32 q / 8 KV heads, D=128, bf16"),
    PrefillConfig(
        "prefill_llama3_8b_fp8", 8, 32, 8, 128, chunk=512, prior_lo=0,
        prior_hi=3584, kv_dtype="fp8_e4m3fn",
        description="the same chunks over an fp8 e4m3fn K/V pool "
                    "(per-tensor scales amax/448), bf16 q and output"),
]
PREFILL_BY_NAME = {c.name: c for c in PREFILL_CONFIGS}


@dataclass
class PrefillCase:
    config: PrefillConfig
    seed: int
    q: torch.Tensor               # [T, Hq, D] bf16, packed over sequences
    q_start: torch.Tensor         # int32 [B+1]
    k_pool: torch.Tensor          # chunk K/V already written
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor        # cached tokens including the chunk
    scale: float
    k_scale: float = 1.0          # fp8 pools: stored code * scale = value
    v_scale: float = 1.0

    @property
    def num_tokens(self) -> int:
        return int(self.q_start[-1])


def build_prefill_case(cfg: PrefillConfig, seed: int = 0,
                       chunks: Optional[Sequence[int]] = None) -> PrefillCase:
    """Seeded chunked-prefill input: lengths, a shuffled pool filled through
    the block manager (prior tokens + the chunk, all written), packed
    queries.  ``chunks`` overrides the per-sequence chunk lengths."""
    kids = np.random.SeedSequence(seed).spawn(6)
    rng_len = np.random.default_rng(kids[0])
    rng_perm = np.random.default_rng(kids[1])
    b, hkv, d = cfg.num_seqs, cfg.num_kv_heads, cfg.head_size
    prior = rng_len.integers(cfg.prior_lo, cfg.prior_hi, size=b,
                             endpoint=True)
    ch = np.full(b, cfg.chunk) if chunks is None else np.asarray(chunks)
    lens = prior + ch
    used = int(sum(-(-int(n) // BLOCK_SIZE) for n in lens))
    nb = used + -(-used // 10)
    pool = BlockPool(nb, order=rng_perm.permutation(nb))
    mgr = KVCacheManager(pool, BLOCK_SIZE)
    for i in range(b):
        assert mgr.admit(i, int(lens[i]))
    tables, seq_lens = mgr.tables(range(b))
    q_start = np.concatenate([[0], np.cumsum(ch)]).astype(np.int32)
    q32 = _normal_f32(kids[2], (int(q_start[-1]), cfg.num_q_heads, d))
    k32 = _normal_f32(kids[3], (nb, hkv, BLOCK_SIZE, d))
    v32 = _normal_f32(kids[4], (nb, hkv, d, BLOCK_SIZE))
    k_scale = v_scale = 1.0
    if cfg.kv_dtype == "fp8_e4m3fn":
        k_scale = float(np.float32(np.abs(k32).max() / FP8_MAX))
        v_scale = float(np.float32(np.abs(v32).max() / FP8_MAX))
    k_pool = _to_storage(k32, cfg.kv_dtype, k_scale)
    v_pool = _to_storage(v32, cfg.kv_dtype, v_scale)
    # slots past each sequence's length (and free blocks) hold NaN
    written = np.zeros((nb, BLOCK_SIZE), dtype=bool)
    for i in range(b):
        n = int(lens[i])
        nfull, rem = divmod(n, BLOCK_SIZE)
        written[tables[i, :nfull]] = True
        if rem:
            written[tables[i, nfull], :rem] = True
    blk_idx, tok_idx = torch.nonzero(torch.from_numpy(~written),
                                     as_tuple=True)
    nan = _nan_of(cfg.kv_dtype)
    if cfg.kv_dtype == "fp8_e4m3fn":  # index_put on the raw bytes
        k_pool.view(torch.uint8)[blk_idx, :, tok_idx, :] = nan.view(torch.uint8)
        v_pool.view(torch.uint8)[blk_idx, :, :, tok_idx] = nan.view(torch.uint8)
    else:
        k_pool[blk_idx, :, tok_idx, :] = nan
        v_pool[blk_idx, :, :, tok_idx] = nan
    return PrefillCase(
        config=cfg, seed=seed, q=_to_storage(q32, "bf16"),
        q_start=torch.from_numpy(q_start), k_pool=k_pool, v_pool=v_pool,
        block_tables=torch.from_numpy(tables),
        seq_lens=torch.from_numpy(seq_lens.astype(np.int32)),
        scale=float(np.float32(1.0 / math.sqrt(d))), k_scale=k_scale,
        v_scale=v_scale)


# --------------------------------------------------------------------------
# bulk appends and block copies (the append / copy-on-write benchmarks)
# --------------------------------------------------------------------------
def append_pool_blocks(tokens: int) -> int:
    """Pool size for a bulk append: the blocks the tokens fill, plus 10%."""
    need = -(-tokens // 16)
    return need + need // 10 + 1


def append_slots(tokens: int, num_blocks: int, pattern: str,
                 seed: int = 0) -> torch.Tensor:
    """Slots of a bulk append.  "runs": whole blocks of a shuffled pool
    filled in order, as a prefill chunk lands; "scattered": a seeded random
    set of distinct slots, as single-token decode appends land."""
    rng = np.random.default_rng(seed)
    if pattern == "runs":
        t = np.arange(tokens)
        s = rng.permutation(num_blocks)[t // 16] * 16 + t % 16
    elif pattern == "scattered":
        s = rng.permutation(num_blocks * 16)[:tokens]
    else:
        raise ValueError(pattern)
    return torch.from_numpy(s.astype(np.int32))


def copy_pairs(pairs: int, seed: int = 0):
    """Pool size and distinct (source, destination) block lists of a
    copy-on-write batch."""
    nb = 2 * pairs + 16
    perm = np.random.default_rng(seed).permutation(nb)
    return (nb, torch.from_numpy(perm[:pairs].astype(np.int32)),
            torch.from_numpy(perm[pairs:2 * pairs].astype(np.int32)))
