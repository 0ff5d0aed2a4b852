"""Seeded random shapes through the C ABI against the oracle.

Each case draws its own head counts, group size, head size, pool type,
batch, lengths (and, for prefill, chunk lengths; for the cascade step,
groups and shared prefixes) and range count, so that combinations the
hand-written cases do not name still meet the oracle at every output
element, and the pools written by the fused step equal the oracle's append
byte for byte.  Tolerances as everywhere: 1e-5 (fp32), 2e-2 (bf16), 6e-2
(fp8 KV) for decode; 2e-2 for prefill.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.adapters import appended_pools, oracle_args, prefill_args
from paged_kv_cache_451_amd.workloads import CONFIG_BY_NAME, \
    PREFILL_BY_NAME, build_case, build_prefill_case

from conftest import raw_bits

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8_e4m3fn": 6e-2}


def _decode_shape(seed, *, cascade=False):
    rng = np.random.default_rng(7000 + seed)
    kv = ["bf16", "fp8_e4m3fn"] if cascade else ["bf16", "fp8_e4m3fn", "f32"]
    kv = kv[rng.integers(len(kv))]
    hkv = int(rng.choice([1, 2, 4, 8]))
    gmax = 8 if kv == "f32" else 16
    g = int(rng.choice([x for x in (1, 2, 3, 4, 5, 8, 16) if x <= gmax]))
    d = int(rng.choice([64, 128] if cascade else [64, 128, 256]))
    b = int(rng.integers(1, 33))
    lens = rng.integers(1, 700, b)
    waves = int(rng.choice([0, 0, 1, 3, 64])) * hkv
    cfg = CONFIG_BY_NAME["llama3_8b_bf16"].replace(
        num_seqs=b, num_q_heads=hkv * g, num_kv_heads=hkv, head_size=d,
        q_dtype="f32" if kv == "f32" else "bf16", kv_dtype=kv, lens="fixed",
        fixed_lens=tuple(int(x) for x in lens))
    return build_case(cfg, seed), waves, rng


def _dev(case):
    return {k: getattr(case, k).cuda() for k in
            ("q", "k_pool", "v_pool", "block_tables", "seq_lens",
             "slot_mapping", "k_new", "v_new")}


def _oracle(case, tables=None):
    kp, vp = appended_pools(case)
    args = oracle_args(case)
    args.update(k_raw=kp, v_raw=vp)
    if tables is not None:
        args["block_tables"] = np.asarray(tables)
    return oracle.paged_decode(**args)


def _err(out, ref):
    g = out.detach().cpu().to(torch.float64).numpy()
    assert np.isfinite(g).all()
    return float(np.abs(g - ref).max())


def _pools_appended(case, dev):
    kp, vp = appended_pools(case)
    assert np.array_equal(raw_bits(dev["k_pool"]), kp.view(np.uint8))
    assert np.array_equal(raw_bits(dev["v_pool"]), vp.view(np.uint8))


def _shape_text(case, waves):
    c = case.config
    return (f"B={c.num_seqs} Hq={c.num_q_heads} Hkv={c.num_kv_heads} "
            f"D={c.head_size} kv={c.kv_dtype} waves={waves} "
            f"max_len={int(case.seq_lens.max())}")


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_step(gpu_lib, seed):
    """The fused step and append-then-decode on one random shape."""
    from paged_kv_cache_451_amd import _lib
    case, waves, _ = _decode_shape(seed)
    print(_shape_text(case, waves), flush=True)
    ref = _oracle(case)
    tol = TOL[case.config.kv_dtype]

    dev = _dev(case)
    out = torch.empty_like(dev["q"])
    _lib.pa_decode_append(
        dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
        dev["seq_lens"], case.scale, out, dev["k_new"], dev["v_new"],
        dev["slot_mapping"], max_seq_len=case.max_seq_len,
        k_scale=case.k_scale, v_scale=case.v_scale, num_waves=waves)
    torch.cuda.synchronize()
    assert _err(out, ref) <= tol
    _pools_appended(case, dev)

    dev = _dev(case)
    _lib.pa_kv_append(dev["k_new"], dev["v_new"], dev["slot_mapping"],
                      dev["k_pool"], dev["v_pool"])
    out = torch.empty_like(dev["q"])
    _lib.pa_decode(dev["q"], dev["k_pool"], dev["v_pool"],
                   dev["block_tables"], dev["seq_lens"], case.scale, out,
                   max_seq_len=case.max_seq_len, k_scale=case.k_scale,
                   v_scale=case.v_scale, num_waves=waves)
    torch.cuda.synchronize()
    assert _err(out, ref) <= tol
    _pools_appended(case, dev)


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill(gpu_lib, seed):
    from paged_kv_cache_451_amd import _lib
    rng = np.random.default_rng(8000 + seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8, 16]))
    while hkv * g > 32:
        hkv //= 2
    b = int(rng.integers(1, 7))
    cfg = PREFILL_BY_NAME["prefill_llama3_8b_bf16"].replace(
        num_seqs=b, num_q_heads=hkv * g, num_kv_heads=hkv,
        head_size=int(rng.choice([64, 128])),
        kv_dtype=["bf16", "fp8_e4m3fn"][rng.integers(2)],
        prior_lo=0, prior_hi=int(rng.integers(0, 600)))
    chunks = rng.integers(0, 61, b)
    case = build_prefill_case(cfg, seed=seed, chunks=chunks)
    print(f"B={b} Hq={cfg.num_q_heads} Hkv={hkv} D={cfg.head_size} "
          f"kv={cfg.kv_dtype} chunks={chunks.tolist()}", flush=True)
    dev = {k: getattr(case, k).cuda() for k in
           ("q", "k_pool", "v_pool", "block_tables", "seq_lens", "q_start")}
    out = torch.full_like(dev["q"], float("nan"))
    _lib.pa_prefill(dev["q"], dev["k_pool"], dev["v_pool"],
                    dev["block_tables"], dev["seq_lens"], dev["q_start"],
                    case.scale, out, k_scale=case.k_scale,
                    v_scale=case.v_scale)
    torch.cuda.synchronize()
    if case.num_tokens == 0:
        return
    ref = oracle.paged_prefill(**prefill_args(case))
    assert _err(out.cpu(), ref) <= 2e-2


@pytest.mark.parametrize("seed", range(8))
def test_random_cascade_step(gpu_lib, seed):
    """Random groups of consecutive sequences, each sharing its first
    member's leading table entries, and sequences outside every group."""
    from paged_kv_cache_451_amd import _lib
    case, waves, rng = _decode_shape(seed, cascade=True)
    b = case.config.num_seqs
    cuts = np.sort(rng.choice(np.arange(b + 1), size=min(b + 1, 4),
                              replace=False)).tolist()
    groups = cuts if len(cuts) >= 2 else [0, b]
    tab = case.block_tables.numpy().copy()
    lens = case.seq_lens.numpy()
    prefix = []
    for j in range(len(groups) - 1):
        first = groups[j]
        # every member keeps the block that holds its newest token
        pmax = min((int(lens[m]) - 1) // 16
                   for m in range(first, groups[j + 1]))
        p = int(rng.integers(0, pmax + 1))
        prefix.append(p)
        for m in range(first + 1, groups[j + 1]):
            tab[m, :p] = tab[first, :p]
    print(_shape_text(case, waves), "groups", groups, "prefix", prefix,
          flush=True)
    dev = _dev(case)
    dev["block_tables"] = torch.as_tensor(tab).cuda()
    out = torch.full_like(dev["q"], float("nan"))
    _lib.pa_decode_append_shared(
        dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
        dev["seq_lens"], case.scale, out, dev["k_new"], dev["v_new"],
        dev["slot_mapping"],
        torch.tensor(groups, dtype=torch.int32, device="cuda"),
        torch.tensor(prefix, dtype=torch.int32, device="cuda"),
        max_seq_len=case.max_seq_len, k_scale=case.k_scale,
        v_scale=case.v_scale, num_waves=waves)
    torch.cuda.synchronize()
    assert _err(out, _oracle(case, tables=tab)) <= TOL[case.config.kv_dtype]
    _pools_appended(case, dev)
