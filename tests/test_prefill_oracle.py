"""Pins of the chunked-prefill oracle.

* library routine: torch SDPA in float64 with grouped query heads and an
  explicit causal mask offset by the cached tokens, on contiguous K/V that
  the test scatters into a shuffled pool itself;
* reductions: a one-token chunk is decode (the decode oracle, pinned
  separately); the last token of a chunk sees the whole context; the first
  token of a whole-prompt chunk sees only itself;
* a planted off-by-one in the causal bound breaks the SDPA pin;
* the FLOP count against brute-force counting.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle import prefill as oprefill
from oracle import decode as odecode

from conftest import raw

BS = 16


def _case(seed, *, lens, chunks, hq, hkv, d, dtype="bf16"):
    g = torch.Generator().manual_seed(seed)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    need = sum(-(-n // BS) for n in lens)
    nb = need + 7
    perm = torch.randperm(nb, generator=g).tolist()
    kpool = torch.zeros(nb, hkv, BS, d).to(tdt)
    vpool = torch.zeros(nb, hkv, d, BS).to(tdt)
    width = max(-(-n // BS) for n in lens)
    tables = np.full((len(lens), width), -1, dtype=np.int32)
    kcs, vcs, nxt = [], [], 0
    for b, n in enumerate(lens):
        kc = torch.randn(n, hkv, d, generator=g).to(tdt)
        vc = torch.randn(n, hkv, d, generator=g).to(tdt)
        for j in range(-(-n // BS)):
            tables[b, j] = perm[nxt]
            nxt += 1
        for t in range(n):
            kpool[tables[b, t // BS], :, t % BS, :] = kc[t]
            vpool[tables[b, t // BS], :, :, t % BS] = vc[t]
        kcs.append(kc.to(torch.float64))
        vcs.append(vc.to(torch.float64))
    q_start = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = torch.randn(int(q_start[-1]), hq, d, generator=g).to(tdt)
    scale = float(np.float32(1 / math.sqrt(d)))
    args = dict(q=raw(q)[0], k_raw=raw(kpool)[0], v_raw=raw(vpool)[0],
                block_tables=tables, seq_lens=np.array(lens, np.int32),
                q_start=q_start, scale=scale, q_dtype=dtype, kv_dtype=dtype)
    return args, q.to(torch.float64), kcs, vcs


def _sdpa(args, q64, kcs, vcs, off_by_one=False):
    outs = []
    qs = args["q_start"]
    for b, (kc, vc) in enumerate(zip(kcs, vcs)):
        n, lo, hi = kc.shape[0], int(qs[b]), int(qs[b + 1])
        c = hi - lo
        pos = torch.arange(n - c, n)[:, None]
        mask = torch.arange(n)[None, :] <= pos          # [C, L]
        if off_by_one:
            mask = torch.arange(n)[None, :] < pos
            mask[:, 0] = True
        qq = q64[lo:hi].permute(1, 0, 2)[None]          # [1, Hq, C, D]
        kk = kc.permute(1, 0, 2)[None]
        vv = vc.permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=mask, enable_gqa=True,
            scale=float(np.float64(np.float32(args["scale"]))))
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.concatenate(outs)


CASES = [
    dict(lens=[40, 100, 300], chunks=[40, 17, 64], hq=8, hkv=2, d=64),
    dict(lens=[33, 16], chunks=[1, 16], hq=4, hkv=4, d=128, dtype="f32"),
    dict(lens=[257], chunks=[129], hq=16, hkv=2, d=128),
]


def test_prefill_equals_masked_sdpa():
    for i, spec in enumerate(CASES):
        args, q64, kcs, vcs = _case(i, **spec)
        ours = oprefill.paged_prefill(**args)
        ref = _sdpa(args, q64, kcs, vcs)
        assert np.abs(ours - ref).max() <= 1e-12, spec


def test_planted_causal_off_by_one_is_caught():
    args, q64, kcs, vcs = _case(0, **CASES[0])
    ours = oprefill.paged_prefill(**args)
    bad = _sdpa(args, q64, kcs, vcs, off_by_one=True)
    assert np.abs(ours - bad).max() > 1e-3


def test_one_token_chunk_is_decode():
    args, _, _, _ = _case(5, lens=[77, 31, 160], chunks=[1, 1, 1], hq=8,
                          hkv=2, d=64)
    ours = oprefill.paged_prefill(**args)
    dec = dict(args)
    dec.pop("q_start")
    ref = oracle.paged_decode(**dec)
    assert np.abs(ours - ref).max() <= 1e-12


def test_chunk_endpoints():
    args, q64, kcs, vcs = _case(6, lens=[50, 90], chunks=[50, 20], hq=4,
                                hkv=2, d=64)
    ours = oprefill.paged_prefill(**args)
    # a whole-prompt chunk: its first token attends to itself only
    v0 = vcs[0][0].numpy()                               # [Hkv, D]
    assert np.abs(ours[0] - np.repeat(v0, 2, axis=0)).max() <= 1e-12
    # the last token of a chunk sees the whole context: decode of it
    last = args["q_start"][1:] - 1
    dec = dict(args)
    dec.pop("q_start")
    dec["q"] = args["q"][last]
    ref = oracle.paged_decode(**dec)
    assert np.abs(ours[last] - ref).max() <= 1e-12


def test_flop_count_by_brute_force():
    lens, chunks = [40, 100, 7], [40, 17, 3]
    qs = np.concatenate([[0], np.cumsum(chunks)])
    pairs = 0
    for n, c in zip(lens, chunks):
        for i in range(c):
            for t in range(n):
                pairs += t <= n - c + i
    assert oprefill.prefill_flops(lens, qs, 8, 64) == 4 * 64 * 8 * pairs
