"""Device path (through the C ABI) against the CPU oracle.

Tolerances (max absolute error against the float64 oracle): 1e-5 for fp32,
2e-2 for bf16, 6e-2 for fp8 KV; the append is compared byte for byte over
the whole pools.  Reduced-size cases span many 16-token blocks, several
split ranges and ragged last blocks; full-size cases run in the launch
configuration the benchmark times and compare every output element.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_451_amd.workloads import CONFIG_BY_NAME, CONFIGS, \
    build_case

from conftest import appended_pools, oracle_args, raw, raw_bits

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8_e4m3fn": 6e-2}

# reduced sizes: the oracle finishes each in a few seconds
SMALL = {
    "tiny_fp32": {},
    "llama3_8b_bf16": dict(num_seqs=8, lo=100, hi=1500),
    "skewed_bf16": dict(num_seqs=16, hi=4000),
    "prefix_shared_bf16": dict(num_seqs=8, prefix_len=512, lo=1, hi=300),
    "fp8_long": dict(num_seqs=4, lo=1500, hi=5000),
}

_CACHE = {}


def small_case(name, seed=0):
    key = ("small", name, seed)
    if key not in _CACHE:
        _CACHE[key] = build_case(CONFIG_BY_NAME[name].replace(**SMALL[name]),
                                 seed)
    return _CACHE[key]


def full_case(name):
    key = ("full", name)
    if key not in _CACHE:
        _CACHE.clear() if len(_CACHE) > 8 else None
        idx = [c.name for c in CONFIGS].index(name)
        _CACHE[key] = build_case(CONFIG_BY_NAME[name], seed=idx)
    return _CACHE[key]


def to_dev(case):
    return {k: getattr(case, k).cuda() for k in
            ("q", "k_pool", "v_pool", "block_tables", "seq_lens",
             "slot_mapping", "k_new", "v_new")}


def run_step(lib, case, dev=None, *, num_waves=0, append=True):
    from paged_kv_cache_451_amd import _lib
    dev = dev or to_dev(case)
    if append:
        _lib.pa_kv_append(dev["k_new"], dev["v_new"], dev["slot_mapping"],
                          dev["k_pool"], dev["v_pool"])
    out = torch.empty_like(dev["q"])
    _lib.pa_decode(dev["q"], dev["k_pool"], dev["v_pool"],
                   dev["block_tables"], dev["seq_lens"], case.scale, out,
                   max_seq_len=case.max_seq_len, k_scale=case.k_scale,
                   v_scale=case.v_scale, total_blocks_hint=case.total_blocks,
                   num_waves=num_waves)
    torch.cuda.synchronize()
    return out, dev


def oracle_out(case, seqs=None):
    kp, vp = appended_pools(case)
    args = oracle_args(case)
    args.update(k_raw=kp, v_raw=vp)
    return oracle.paged_decode(**args, seqs=seqs)


def max_err(gpu_out, ref, seqs=None):
    g = gpu_out.detach().cpu().to(torch.float64).numpy()
    if seqs is not None:
        g, ref = g[seqs], ref[seqs]
    assert np.isfinite(g).all()
    return float(np.abs(g - ref).max())


# ---------------------------------------------------------------------------
# KV append: whole pools, byte for byte, at full size
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
def test_kv_append_bit_exact_full_size(gpu_lib, name):
    case = full_case(name)
    from paged_kv_cache_451_amd import _lib
    dev = to_dev(case)
    _lib.pa_kv_append(dev["k_new"], dev["v_new"], dev["slot_mapping"],
                      dev["k_pool"], dev["v_pool"])
    torch.cuda.synchronize()
    k1, v1 = appended_pools(case)
    assert np.array_equal(raw_bits(dev["k_pool"]).ravel(),
                          k1.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(dev["v_pool"]).ravel(),
                          v1.view(np.uint8).ravel())


def test_kv_append_skips_negative_and_out_of_range_slots(gpu_lib):
    from paged_kv_cache_451_amd import _lib
    case = small_case("llama3_8b_bf16")
    dev = to_dev(case)
    nb = case.num_blocks
    slots = case.slot_mapping.clone()
    slots[0] = -1
    slots[1] = nb * 16 + 3
    _lib.pa_kv_append(dev["k_new"], dev["v_new"], slots.cuda(),
                      dev["k_pool"], dev["v_pool"])
    torch.cuda.synchronize()
    k0, _ = raw(case.k_pool)
    v0, _ = raw(case.v_pool)
    kn, _ = raw(case.k_new)
    vn, _ = raw(case.v_new)
    k1, v1 = oracle.kv_append(k0, v0, kn, vn, slots.numpy())
    assert np.array_equal(raw_bits(dev["k_pool"]).ravel(),
                          k1.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(dev["v_pool"]).ravel(),
                          v1.view(np.uint8).ravel())


def _run_slots(nb, n_seqs, gen, max_len=70):
    """Prefill-shaped slots: each sequence writes a run of consecutive
    slots from a random offset of its first block through distinct random
    blocks; two slots are then made invalid."""
    blocks = torch.randperm(nb, generator=gen).tolist()
    out = []
    for _ in range(n_seqs):
        off = int(torch.randint(0, 16, (1,), generator=gen))
        length = int(torch.randint(1, max_len + 1, (1,), generator=gen))
        nblk = (off + length + 15) // 16
        mine, blocks = blocks[:nblk], blocks[nblk:]
        out += [mine[(off + j) // 16] * 16 + (off + j) % 16
                for j in range(length)]
    slots = torch.tensor(out, dtype=torch.int32)
    slots[len(out) // 3] = -1
    slots[len(out) // 2] = nb * 16 + 5
    return slots


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float8_e4m3fn,
                                   torch.float32])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_kv_append_slot_runs_bit_exact(gpu_lib, dtype, d):
    """Runs of consecutive slots (unaligned starts, token counts that are
    not multiples of 16, invalid slots) land byte for byte where the oracle
    puts them."""
    from paged_kv_cache_451_amd import _lib
    gen = torch.Generator().manual_seed(d)
    hkv, nb = 4, 96
    slots = _run_slots(nb, 7, gen)
    n = len(slots)
    size = 4 if dtype == torch.float32 else (1 if dtype == torch.float8_e4m3fn
                                              else 2)
    itype = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[size]

    def rand_bits(shape):
        b = torch.randint(0, 256, (*shape[:-1], shape[-1] * size),
                          generator=gen, dtype=torch.uint8)
        return b.view(itype).view(dtype)

    k_pool = rand_bits((nb, hkv, 16, d))
    v_pool = rand_bits((nb, hkv, d, 16))
    k_new = rand_bits((n, hkv, d))
    v_new = rand_bits((n, hkv, d))
    kp, vp = k_pool.cuda(), v_pool.cuda()
    _lib.pa_kv_append(k_new.cuda(), v_new.cuda(), slots.cuda(), kp, vp)
    torch.cuda.synchronize()
    k0 = raw(k_pool)[0]
    v0 = raw(v_pool)[0]
    k1, v1 = oracle.kv_append(k0, v0, raw(k_new)[0], raw(v_new)[0],
                              slots.numpy())
    assert np.array_equal(raw_bits(kp).ravel(), k1.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(vp).ravel(), v1.view(np.uint8).ravel())


def test_quantising_append_slot_runs(gpu_lib):
    gen = torch.Generator().manual_seed(29)
    hkv, d, nb = 8, 128, 96
    slots = _run_slots(nb, 9, gen)
    n = len(slots)
    k_new = torch.randn((n, hkv, d), generator=gen).to(torch.bfloat16)
    v_new = (torch.randn((n, hkv, d), generator=gen) * 5).to(torch.bfloat16)
    k_pool = torch.randint(0, 256, (nb, hkv, 16, d), generator=gen,
                           dtype=torch.uint8).view(torch.float8_e4m3fn)
    v_pool = torch.randint(0, 256, (nb, hkv, d, 16), generator=gen,
                           dtype=torch.uint8).view(torch.float8_e4m3fn)
    _quant_append_check(k_new, v_new, slots, k_pool, v_pool, 0.02, 0.03)


@pytest.mark.parametrize("quant, pattern", [(False, "runs"),
                                            (False, "scattered"),
                                            (True, "runs")])
def test_bulk_append_at_benchmark_size(gpu_lib, quant, pattern):
    """The append benchmark's workload (32768 tokens, 8 KV heads, D = 128,
    the same slots and scales), whole pools byte for byte."""
    from paged_kv_cache_451_amd import _lib
    from paged_kv_cache_451_amd.workloads import append_pool_blocks, \
        append_slots
    from oracle import quant as oquant
    n, hkv, d = 32768, 8, 128
    nb = append_pool_blocks(n)
    slots = append_slots(n, nb, pattern, 0)
    g = torch.Generator().manual_seed(0)
    k_new = torch.randn(n, hkv, d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(n, hkv, d, generator=g).to(torch.bfloat16)
    pdt = np.uint8 if quant else np.uint16
    kp_h = np.zeros((nb, hkv, 16, d), dtype=pdt)
    vp_h = np.zeros((nb, hkv, d, 16), dtype=pdt)
    tdt = torch.float8_e4m3fn if quant else torch.bfloat16
    kp = torch.from_numpy(kp_h.view(np.uint8)).view(tdt).cuda()
    vp = torch.from_numpy(vp_h.view(np.uint8)).view(tdt).cuda()
    ks = vs = float(np.float32(4.5 / 448))
    if quant:
        _lib.pa_kv_append_quant(k_new.cuda(), v_new.cuda(), slots.cuda(), kp,
                                vp, ks, vs)
    else:
        _lib.pa_kv_append(k_new.cuda(), v_new.cuda(), slots.cuda(), kp, vp)
    torch.cuda.synchronize()
    kn = k_new.view(torch.uint16).numpy()
    vn = v_new.view(torch.uint16).numpy()
    if quant:
        k1, v1 = oquant.kv_append_quant(kp_h, vp_h, kn, vn, slots.numpy(),
                                        ks, vs)
    else:
        k1, v1 = oracle.kv_append(kp_h, vp_h, kn, vn, slots.numpy())
    assert np.array_equal(raw_bits(kp).ravel(), k1.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(vp).ravel(), v1.view(np.uint8).ravel())


def test_copy_blocks_at_benchmark_size(gpu_lib):
    """The copy-on-write benchmark's batch (4096 pairs of 32 KiB blocks per
    pool), whole pools byte for byte."""
    from paged_kv_cache_451_amd import _lib
    from paged_kv_cache_451_amd.workloads import copy_pairs
    nb, src, dst = copy_pairs(4096, 0)
    g = torch.Generator().manual_seed(3)
    kp = torch.randint(0, 256, (nb, 8, 16, 256), generator=g,
                       dtype=torch.uint8)
    vp = torch.randint(0, 256, (nb, 8, 128, 32), generator=g,
                       dtype=torch.uint8)
    kd = kp.view(torch.bfloat16).cuda()
    vd = vp.view(torch.bfloat16).cuda()
    _lib.pa_copy_blocks(kd, vd, src.cuda(), dst.cuda())
    torch.cuda.synchronize()
    k1, v1 = oracle.append.copy_blocks(kp.numpy().reshape(nb, -1),
                                       vp.numpy().reshape(nb, -1),
                                       src.numpy(), dst.numpy())
    assert np.array_equal(raw_bits(kd).reshape(nb, -1), k1)
    assert np.array_equal(raw_bits(vd).reshape(nb, -1), v1)


# ---------------------------------------------------------------------------
# decode: reduced sizes, every element, several split schedules
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
@pytest.mark.parametrize("waves", ["auto", "one_range", "many"])
def test_decode_matches_oracle_small(gpu_lib, name, waves):
    case = small_case(name)
    hkv = case.config.num_kv_heads
    nw = {"auto": 0, "one_range": hkv, "many": hkv * 997}[waves]
    out, _ = run_step(gpu_lib, case, num_waves=nw)
    ref = oracle_out(case)
    err = max_err(out, ref)
    print(f"{name} waves={waves}: max abs err {err:.3e}")
    assert err <= TOL[case.config.kv_dtype]


@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
def test_decode_matches_oracle_full_size(gpu_lib, name):
    """Every (sequence, head, column) of each full-size workload, in the
    launch configuration the benchmark uses."""
    case = full_case(name)
    out, _ = run_step(gpu_lib, case)
    err = max_err(out, oracle_out(case))
    print(f"{name} full size, all {case.config.num_seqs} sequences: "
          f"max abs err {err:.3e}")
    assert err <= TOL[case.config.kv_dtype]


# ---------------------------------------------------------------------------
# which token was read: a dominant key at chosen positions
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["llama3_8b_bf16", "fp8_long", "tiny_fp32"])
def test_dominant_key_probe_reads_the_right_token(gpu_lib, name):
    """q = 1 everywhere; one token per sequence gets a large K along q, so its
    weight is ~1 and the output is that token's V row.  An off-by-one token,
    block or head mapping would return a different row (error ~1)."""
    case = small_case(name)
    case = build_case(case.config, seed=9)
    lens = case.seq_lens.numpy()
    tab = case.block_tables.numpy()
    qdt = case.q.dtype
    case.q = torch.ones_like(case.q, dtype=torch.float32).to(qdt)
    # a real K value of 4 along q: fp8 pools store value / k_scale
    hot_val = min(448.0, 4.0 / case.k_scale)
    hot = {}
    kp = case.k_pool.clone()
    picks = [0, 15, 16, 31, 32, 47]
    for i, n in enumerate(lens):
        t = picks[i % len(picks)] if i < len(picks) else int(n) - 2
        t = min(t, int(n) - 2)
        hot[i] = t
        kp[tab[i, t // 16], :, t % 16, :] = torch.tensor(hot_val).to(kp.dtype)
    case.k_pool = kp
    out, _ = run_step(gpu_lib, case)
    ref = oracle_out(case)
    err = max_err(out, ref)
    assert err <= TOL[case.config.kv_dtype]
    # the oracle agrees that the hot token dominates
    _, vp = appended_pools(case)
    vals = oracle.numerics.widen(vp, raw(case.v_pool)[1]) * case.v_scale
    g = case.config.group
    for i, t in hot.items():
        row = vals[tab[i, t // 16], :, :, t % 16]          # [Hkv, D]
        expect = np.repeat(row, g, axis=0)
        assert np.abs(ref[i] - expect).max() < 1e-3 * max(1, np.abs(row).max())


# ---------------------------------------------------------------------------
# invariants on the device: permutation and aliasing give identical bits
# ---------------------------------------------------------------------------
def test_block_permutation_is_bitwise_invariant_on_gpu(gpu_lib):
    case = small_case("skewed_bf16")
    out, _ = run_step(gpu_lib, case)
    rng = np.random.default_rng(5)
    pi = torch.from_numpy(rng.permutation(case.num_blocks))
    c2 = build_case(case.config, case.seed)
    kp, vp = torch.empty_like(c2.k_pool), torch.empty_like(c2.v_pool)
    kp[pi], vp[pi] = c2.k_pool, c2.v_pool
    tab = c2.block_tables
    c2.block_tables = torch.where(tab >= 0, pi[tab.clamp(min=0).long()]
                                  .to(torch.int32), tab)
    sl = c2.slot_mapping
    c2.slot_mapping = (pi[(sl // 16).long()] * 16 + sl % 16).to(torch.int32)
    c2.k_pool, c2.v_pool = kp, vp
    out2, _ = run_step(gpu_lib, c2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_prefix_aliasing_is_bitwise_invariant_on_gpu(gpu_lib):
    case = small_case("prefix_shared_bf16")
    out, _ = run_step(gpu_lib, case)
    npre = case.config.prefix_len // 16
    tab = case.block_tables.clone()
    shared = tab[0, :npre].clone()
    kparts, vparts, nxt = [case.k_pool], [case.v_pool], case.num_blocks
    for i in range(1, case.config.num_seqs):
        kparts.append(case.k_pool[shared.long()])
        vparts.append(case.v_pool[shared.long()])
        tab[i, :npre] = torch.arange(nxt, nxt + npre, dtype=torch.int32)
        nxt += npre
    c2 = build_case(case.config, case.seed)
    c2.k_pool, c2.v_pool = torch.cat(kparts), torch.cat(vparts)
    c2.block_tables = tab
    out2, _ = run_step(gpu_lib, c2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def _custom_case(lens, *, hq, hkv, d, q_dtype="bf16", kv_dtype="bf16",
                 seed=4):
    base = CONFIG_BY_NAME["llama3_8b_bf16"].replace(
        num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_size=d,
        q_dtype=q_dtype, kv_dtype=kv_dtype, lens="fixed",
        fixed_lens=tuple(max(1, n) for n in lens))
    return build_case(base, seed)


EDGE = [
    dict(lens=[1, 2, 15, 16, 17, 31, 32, 33, 48], hq=8, hkv=2, d=128),
    dict(lens=[1, 300, 7], hq=16, hkv=1, d=64),            # G = 16
    dict(lens=[64, 5, 129], hq=4, hkv=4, d=128),           # G = 1 on MFMA
    dict(lens=[200, 33], hq=6, hkv=2, d=256),              # D = 256, G = 3
    dict(lens=[100, 17], hq=4, hkv=2, d=64, kv_dtype="fp8_e4m3fn"),
    dict(lens=[90, 300], hq=8, hkv=2, d=256, kv_dtype="fp8_e4m3fn"),
    dict(lens=[33, 1, 250], hq=16, hkv=1, d=128,
         kv_dtype="fp8_e4m3fn"),                            # fp8, G = 16
    dict(lens=[1, 16, 77], hq=8, hkv=1, d=128, q_dtype="f32",
         kv_dtype="f32"),                                   # fp32, G = 8
    dict(lens=[1, 40], hq=2, hkv=2, d=256, q_dtype="f32", kv_dtype="f32"),
]


@pytest.mark.parametrize("spec", EDGE)
@pytest.mark.parametrize("waves", [0, 1, 4096])
def test_edge_shapes(gpu_lib, spec, waves):
    case = _custom_case(**spec)
    nw = waves * case.config.num_kv_heads if waves else 0
    out, _ = run_step(gpu_lib, case, num_waves=nw)
    err = max_err(out, oracle_out(case))
    assert err <= TOL[case.config.kv_dtype]


def test_zero_length_sequences_give_zero_rows(gpu_lib):
    from paged_kv_cache_451_amd import _lib
    case = small_case("llama3_8b_bf16")
    dev = to_dev(case)
    lens = dev["seq_lens"].clone()
    lens[1] = 0
    lens[5] = 0
    out = torch.full_like(dev["q"], float("nan"))
    _lib.pa_kv_append(dev["k_new"], dev["v_new"], dev["slot_mapping"],
                      dev["k_pool"], dev["v_pool"])
    _lib.pa_decode(dev["q"], dev["k_pool"], dev["v_pool"],
                   dev["block_tables"], lens, case.scale, out,
                   max_seq_len=case.max_seq_len,
                   total_blocks_hint=0)
    torch.cuda.synchronize()
    assert (out[1] == 0).all() and (out[5] == 0).all()
    args = oracle_args(case)
    kp, vp = appended_pools(case)
    args.update(k_raw=kp, v_raw=vp, seq_lens=lens.cpu().numpy())
    ref = oracle.paged_decode(**args)
    assert max_err(out, ref) <= TOL["bf16"]


def test_out_of_range_block_ids_are_not_dereferenced(gpu_lib):
    """An entry outside [0, num_blocks) contributes nothing: the result equals
    the oracle over the same context with that block's tokens removed."""
    case = small_case("llama3_8b_bf16")
    tab = case.block_tables.clone()
    tab[2, 1] = case.num_blocks + 1000
    tab[3, 0] = -7
    c2 = build_case(case.config, case.seed)
    c2.block_tables = tab
    out, _ = run_step(gpu_lib, c2)
    g = out.detach().cpu().to(torch.float64).numpy()
    assert np.isfinite(g).all()
    ref = oracle_out(case, seqs=[0, 1, 4])
    assert max_err(out, ref, [0, 1, 4]) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# the fused step: pa_decode_append == pa_kv_append then pa_decode
# ---------------------------------------------------------------------------
def run_fused(case, dev=None, *, num_waves=0, slots=None):
    from paged_kv_cache_451_amd import _lib
    dev = dev or to_dev(case)
    out = torch.empty_like(dev["q"])
    _lib.pa_decode_append(
        dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
        dev["seq_lens"], case.scale, out, dev["k_new"], dev["v_new"],
        dev["slot_mapping"] if slots is None else slots.cuda(),
        max_seq_len=case.max_seq_len, k_scale=case.k_scale,
        v_scale=case.v_scale, total_blocks_hint=case.total_blocks,
        num_waves=num_waves)
    torch.cuda.synchronize()
    return out, dev


def assert_pools_equal_oracle_append(case, dev, slots=None):
    k0, _ = raw(case.k_pool)
    v0, _ = raw(case.v_pool)
    kn, _ = raw(case.k_new)
    vn, _ = raw(case.v_new)
    sl = case.slot_mapping.numpy() if slots is None else slots.numpy()
    k1, v1 = oracle.kv_append(k0, v0, kn, vn, sl)
    assert np.array_equal(raw_bits(dev["k_pool"]).ravel(),
                          k1.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(dev["v_pool"]).ravel(),
                          v1.view(np.uint8).ravel())


@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
@pytest.mark.parametrize("waves", ["auto", "one_range", "many"])
def test_fused_step_matches_oracle_small(gpu_lib, name, waves):
    case = small_case(name)
    hkv = case.config.num_kv_heads
    nw = {"auto": 0, "one_range": hkv, "many": hkv * 997}[waves]
    out, dev = run_fused(case, num_waves=nw)
    assert_pools_equal_oracle_append(case, dev)
    err = max_err(out, oracle_out(case))
    print(f"fused {name} waves={waves}: max abs err {err:.3e}")
    assert err <= TOL[case.config.kv_dtype]


@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
def test_fused_step_matches_oracle_full_size(gpu_lib, name):
    """The benchmark's step (pa_decode_append) at full size: every output
    element against the oracle, and the whole pools byte for byte."""
    case = full_case(name)
    out, dev = run_fused(case)
    assert_pools_equal_oracle_append(case, dev)
    err = max_err(out, oracle_out(case))
    print(f"fused {name} full size, all {case.config.num_seqs} sequences: "
          f"max abs err {err:.3e}")
    assert err <= TOL[case.config.kv_dtype]


@pytest.mark.parametrize("spec", EDGE)
@pytest.mark.parametrize("waves", [0, 1, 4096])
def test_fused_step_edge_shapes(gpu_lib, spec, waves):
    case = _custom_case(**spec)
    nw = waves * case.config.num_kv_heads if waves else 0
    out, dev = run_fused(case, num_waves=nw)
    assert_pools_equal_oracle_append(case, dev)
    assert max_err(out, oracle_out(case)) <= TOL[case.config.kv_dtype]


# Batches with more (sequence, query head) pairs than the GPU holds merge
# workgroups at once (at most 32 per CU on 256 CUs = 8192) take the merge
# passes (fused and plain) with two query heads per workgroup.  These cases have at least 1.5x
# that many pairs of short sequences, so that path runs; they cover an odd
# head count, pairs whose halves belong to different KV heads, fp8, fp32
# and every head size.
MANY = [
    dict(hq=5, hkv=5, d=64),                               # odd Hq, G = 1
    dict(hq=6, hkv=2, d=128),                              # G = 3
    dict(hq=8, hkv=2, d=256, kv_dtype="fp8_e4m3fn"),       # fp8, D = 256
    dict(hq=2, hkv=2, d=64, q_dtype="f32", kv_dtype="f32"),
]


@pytest.mark.parametrize("spec", MANY)
@pytest.mark.parametrize("fused", [True, False])
def test_step_many_short_sequences(gpu_lib, spec, fused):
    n = -(-12288 // spec["hq"])
    lens = np.random.default_rng(11).integers(1, 49, n).tolist()
    case = _custom_case(lens, seed=12, **spec)
    if fused:
        out, dev = run_fused(case)
    else:
        out, dev = run_step(gpu_lib, case)
    assert_pools_equal_oracle_append(case, dev)
    err = max_err(out, oracle_out(case))
    print(f"{'fused' if fused else 'append + decode'}, {n} sequences x "
          f"{spec['hq']} heads: max abs err {err:.3e}")
    assert err <= TOL[case.config.kv_dtype]


@pytest.mark.parametrize("lens, kv_dtype", [([131072, 5], "bf16"),
                                             ([262144, 40], "fp8_e4m3fn")])
def test_one_very_long_sequence(gpu_lib, lens, kv_dtype):
    """A context far longer than the workloads' (128 k tokens in bf16, 256 k
    in fp8) next to a short one: the long sequence crosses every range of
    its heads, so the merge folds about 128 partials per head.  Both step
    forms, every output element, the pools byte for byte."""
    case = _custom_case(lens, hq=32, hkv=8, d=128, kv_dtype=kv_dtype,
                        seed=13)
    ref = oracle_out(case)
    out, dev = run_fused(case)
    assert_pools_equal_oracle_append(case, dev)
    err = max_err(out, ref)
    out2, dev2 = run_step(gpu_lib, case)
    assert_pools_equal_oracle_append(case, dev2)
    err2 = max_err(out2, ref)
    print(f"{lens[0]} tokens, {kv_dtype}: max abs err fused {err:.3e}, "
          f"append + decode {err2:.3e}")
    assert max(err, err2) <= TOL[kv_dtype]


def test_fused_step_dominant_new_token(gpu_lib):
    """The newest token carries a large key along q: its weight is ~1 and
    the output is its V row, which only k_new / v_new hold before the call
    (its pool slot holds NaN)."""
    case = build_case(small_case("llama3_8b_bf16").config, seed=11)
    case.q = torch.ones_like(case.q)
    case.k_new = torch.full_like(case.k_new, 4.0)
    out, dev = run_fused(case)
    ref = oracle_out(case)
    assert max_err(out, ref) <= TOL["bf16"]
    vn = case.v_new.to(torch.float64).numpy()          # [B, Hkv, D]
    expect = np.repeat(vn, case.config.group, axis=1)  # [B, Hq, D]
    assert np.abs(ref - expect).max() < 1e-3


def test_fused_step_negative_slot_skips_only_the_write(gpu_lib):
    case = small_case("llama3_8b_bf16")
    slots = case.slot_mapping.clone()
    slots[2] = -1
    out, dev = run_fused(case, slots=slots)
    assert_pools_equal_oracle_append(case, dev, slots=slots)
    # attention still includes token L-1 from k_new / v_new
    assert max_err(out, oracle_out(case)) <= TOL["bf16"]


def test_fused_step_single_token_sequences(gpu_lib):
    case = _custom_case([1, 1, 17, 2], hq=8, hkv=2, d=128)
    out, dev = run_fused(case)
    assert_pools_equal_oracle_append(case, dev)
    ref = oracle_out(case)
    assert max_err(out, ref) <= TOL["bf16"]
    vn = case.v_new.to(torch.float64).numpy()
    expect = np.repeat(vn, 4, axis=1)
    assert np.abs(out[:2].cpu().to(torch.float64).numpy() -
                  expect[:2]).max() <= TOL["bf16"]


# ---------------------------------------------------------------------------
# quantising append (bf16 rows into an fp8 e4m3fn pool): bit-exact
# ---------------------------------------------------------------------------
def _quant_append_check(k_new, v_new, slots, k_pool, v_pool, ks, vs):
    from oracle import quant
    from paged_kv_cache_451_amd import _lib
    kp, vp = k_pool.cuda(), v_pool.cuda()
    _lib.pa_kv_append_quant(k_new.cuda(), v_new.cuda(), slots.cuda(), kp, vp,
                            ks, vs)
    torch.cuda.synchronize()
    k1, v1 = quant.kv_append_quant(
        raw_bits(k_pool).reshape(k_pool.shape),
        raw_bits(v_pool).reshape(v_pool.shape),
        k_new.view(torch.uint16).numpy(), v_new.view(torch.uint16).numpy(),
        slots.numpy(), ks, vs)
    assert np.array_equal(raw_bits(kp).ravel(), k1.ravel())
    assert np.array_equal(raw_bits(vp).ravel(), v1.ravel())


_F32 = np.finfo(np.float32)


@pytest.mark.parametrize("ks, vs", [
    (1.0, 1.0), (0.0123, 1.0 / 448), (3.7, 0.5), (1.0 / 3, 0.1),
    (float(_F32.smallest_subnormal), float(_F32.max)),
    (float(_F32.tiny), float(np.nextafter(np.float32(2), np.float32(0))))])
def test_quantising_append_every_bf16_code(gpu_lib, ks, vs):
    """All 65536 bf16 codes (NaN, infinities, subnormals, every e4m3fn tie
    that bf16 can hold at scale 1) as K and, reversed, as V, at ordinary
    scales and at the float32 extremes (the kernel divides by multiplying
    with a float64 reciprocal)."""
    hkv, d, n, nb = 8, 128, 64, 80
    codes = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    k_new = codes.view(torch.bfloat16).reshape(n, hkv, d).contiguous()
    v_new = k_new.flip(0).contiguous()
    g = torch.Generator().manual_seed(17)
    k_pool = torch.randint(0, 256, (nb, hkv, 16, d), generator=g,
                           dtype=torch.uint8).view(torch.float8_e4m3fn)
    v_pool = torch.randint(0, 256, (nb, hkv, d, 16), generator=g,
                           dtype=torch.uint8).view(torch.float8_e4m3fn)
    slots = torch.randperm(nb * 16, generator=g)[:n].to(torch.int32)
    slots[3] = -1
    _quant_append_check(k_new, v_new, slots, k_pool, v_pool, ks, vs)


def test_quantising_append_full_fp8_workload(gpu_lib):
    case = full_case("fp8_long")
    g = torch.Generator().manual_seed(5)
    shape = tuple(case.k_new.shape)
    k_new = torch.randn(shape, generator=g).to(torch.bfloat16)
    v_new = (torch.randn(shape, generator=g) * 3).to(torch.bfloat16)
    _quant_append_check(k_new, v_new, case.slot_mapping, case.k_pool,
                        case.v_pool, case.k_scale, case.v_scale)


# ---------------------------------------------------------------------------
# copy-on-write: block copies, then a forked sequence diverging
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float8_e4m3fn,
                                   torch.float32])
def test_copy_blocks_bit_exact(gpu_lib, dtype):
    from paged_kv_cache_451_amd import _lib
    g = torch.Generator().manual_seed(23)
    nb, hkv, d = 97, 4, 128
    esize = torch.empty(0, dtype=dtype).element_size()
    kp = torch.randint(0, 256, (nb, hkv, 16, d * esize), generator=g,
                       dtype=torch.uint8).view(dtype)
    vp = torch.randint(0, 256, (nb, hkv, d * esize, 16), generator=g,
                       dtype=torch.uint8)
    vp = vp.reshape(nb, hkv, d, 16 * esize).view(dtype)
    perm = torch.randperm(nb, generator=g)
    src = perm[:30].to(torch.int32)
    dst = perm[30:60].to(torch.int32)
    src[4] = nb + 3          # skipped pair
    dst[7] = -1              # skipped pair
    kd, vd = kp.cuda(), vp.cuda()
    _lib.pa_copy_blocks(kd, vd, src.cuda(), dst.cuda())
    torch.cuda.synchronize()
    k1, v1 = oracle.append.copy_blocks(raw_bits(kp).reshape(nb, -1),
                                       raw_bits(vp).reshape(nb, -1),
                                       src.numpy(), dst.numpy())
    assert np.array_equal(raw_bits(kd).reshape(nb, -1), k1)
    assert np.array_equal(raw_bits(vd).reshape(nb, -1), v1)


def test_forked_sequence_diverges_by_copy_on_write(gpu_lib):
    """Sequence 1 forks sequence 0 (sharing its partly filled last block);
    both append a different token.  The block manager copies the shared
    block for the fork, the device copies it, then append and decode run;
    the result matches the oracle running the same steps."""
    from paged_kv_cache_451_amd import _lib
    from paged_kv_cache_451_amd.pool import BlockPool, KVCacheManager
    g = torch.Generator().manual_seed(31)
    nb, hq, hkv, d = 24, 8, 2, 128
    pool = BlockPool(nb, order=torch.randperm(nb, generator=g).tolist())
    mgr = KVCacheManager(pool, 16)
    assert mgr.admit(0, 37)
    mgr.fork(0, 1)
    slot1 = mgr.append_slot(1)            # the fork writes first: a copy
    slot0 = mgr.append_slot(0)
    copies = mgr.take_copies()
    assert len(copies) == 1
    tables, lens = mgr.tables([0, 1])
    assert tables[0, 2] != tables[1, 2] and (tables[0, :2] == tables[1, :2]).all()
    kp = torch.randn(nb, hkv, 16, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(nb, hkv, d, 16, generator=g).to(torch.bfloat16)
    kn = torch.randn(2, hkv, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(2, hkv, d, generator=g).to(torch.bfloat16)
    q = torch.randn(2, hq, d, generator=g).to(torch.bfloat16)
    slots = torch.tensor([slot0, slot1], dtype=torch.int32)
    src = torch.tensor([c[0] for c in copies], dtype=torch.int32)
    dst = torch.tensor([c[1] for c in copies], dtype=torch.int32)
    scale = float(np.float32(1 / np.sqrt(d)))

    kd, vd = kp.cuda(), vp.cuda()
    _lib.pa_copy_blocks(kd, vd, src.cuda(), dst.cuda())
    _lib.pa_kv_append(kn.cuda(), vn.cuda(), slots.cuda(), kd, vd)
    out = torch.empty(2, hq, d, dtype=torch.bfloat16, device="cuda")
    tab = torch.from_numpy(tables).cuda()
    ln = torch.from_numpy(lens.astype(np.int32)).cuda()
    _lib.pa_decode(q.cuda(), kd, vd, tab, ln, scale, out,
                   max_seq_len=int(lens.max()))
    torch.cuda.synchronize()

    k1, v1 = oracle.append.copy_blocks(raw(kp)[0], raw(vp)[0], src.numpy(),
                                       dst.numpy())
    k2, v2 = oracle.kv_append(k1, v1, raw(kn)[0], raw(vn)[0], slots.numpy())
    assert np.array_equal(raw_bits(kd).ravel(), k2.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(vd).ravel(), v2.view(np.uint8).ravel())
    ref = oracle.paged_decode(raw(q)[0], k2, v2, tables, lens, scale,
                              q_dtype="bf16", kv_dtype="bf16")
    assert max_err(out, ref) <= TOL["bf16"]
    # the two sequences share 36 tokens and differ in the last one
    assert np.abs(ref[0] - ref[1]).max() > 1e-3


# ---------------------------------------------------------------------------
# the continuous-batching loop on the device: every step against the oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("native", [False, True],
                         ids=["python block manager", "native block manager"])
def test_engine_steps_match_the_oracle(gpu_lib, native):
    """The loop's device pools and every decode against host pools that the
    test builds itself: each step's recorded K/V rows go through the
    oracle's append (in the order the device writes them: prompts, then
    the decoded tokens), and the oracle decodes the step's queries over
    the result.  Run on either block manager."""
    from paged_kv_cache_451_amd.engine import Engine, Request
    rng = np.random.default_rng(8)
    e = Engine(96, 8, 2, 128, device="cuda", seed=6, mirror=True,
               native_pool=native)
    for i in range(20):
        e.add_request(Request(i, rng.integers(0, 500, size=int(
            rng.integers(20, 200))).tolist(), int(rng.integers(5, 40))))
    k_host = np.zeros((96, 2, 16, 128), dtype=np.uint16)
    v_host = np.zeros((96, 2, 128, 16), dtype=np.uint16)
    checked = preempted = 0
    while e.has_work():
        st = e.step()
        preempted += st.preempted
        for k_rows, v_rows, slots in e.last_writes:
            k_host, v_host = oracle.kv_append(k_host, v_host, k_rows, v_rows,
                                              slots)
        if not st.running:
            continue
        torch.cuda.synchronize()
        ref = oracle.paged_decode(
            e.last_q.view(torch.uint16).numpy(), k_host, v_host,
            e.last_tables, e.last_lens, e.scale, q_dtype="bf16",
            kv_dtype="bf16")
        assert max_err(e.last_out, ref) <= TOL["bf16"], st.step
        checked += 1
    assert checked > 20 and preempted > 0
    assert np.array_equal(raw_bits(e.k_pool).ravel(),
                          k_host.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(e.v_pool).ravel(),
                          v_host.view(np.uint8).ravel())


@pytest.mark.parametrize("native", [False, True],
                         ids=["python block manager", "native block manager"])
def test_engine_chunked_prefill_matches_the_oracle(gpu_lib, native):
    """The loop with a prompt-token budget per step and prefill attention:
    each step's chunks are checked against the prefill oracle over host
    pools holding everything written before them (earlier steps and this
    step's chunks), each decode against the decode oracle after the step's
    token writes, and the device pools against the host pools at the end."""
    from paged_kv_cache_451_amd.engine import Engine, Request
    rng = np.random.default_rng(9)
    e = Engine(96, 8, 2, 128, device="cuda", seed=7, mirror=True,
               max_prefill_tokens=48, prefill_attention=True,
               native_pool=native)
    for i in range(16):
        e.add_request(Request(i, rng.integers(0, 500, size=int(
            rng.integers(20, 200))).tolist(), int(rng.integers(5, 30))))
    k_host = np.zeros((96, 2, 16, 128), dtype=np.uint16)
    v_host = np.zeros((96, 2, 128, 16), dtype=np.uint16)
    prefills = decodes = spread = 0
    while e.has_work():
        st = e.step()
        writes = list(e.last_writes)
        torch.cuda.synchronize()
        if st.prefill_tokens:
            k_rows, v_rows, slots = writes.pop(0)
            k_host, v_host = oracle.kv_append(k_host, v_host, k_rows, v_rows,
                                              slots)
            q, q_start, tables, lens, out = e.last_prefill
            ref = oracle.paged_prefill(
                q.view(torch.uint16).numpy(), k_host, v_host, tables, lens,
                q_start, e.scale, q_dtype="bf16", kv_dtype="bf16")
            assert max_err(out, ref) <= TOL["bf16"], st.step
            prefills += 1
            spread += st.running < len(e.running)
        for k_rows, v_rows, slots in writes:
            k_host, v_host = oracle.kv_append(k_host, v_host, k_rows, v_rows,
                                              slots)
        if st.running:
            ref = oracle.paged_decode(
                e.last_q.view(torch.uint16).numpy(), k_host, v_host,
                e.last_tables, e.last_lens, e.scale, q_dtype="bf16",
                kv_dtype="bf16")
            assert max_err(e.last_out, ref) <= TOL["bf16"], st.step
            decodes += 1
    assert prefills > 10 and decodes > 20 and spread > 0
    assert np.array_equal(raw_bits(e.k_pool).ravel(),
                          k_host.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(e.v_pool).ravel(),
                          v_host.view(np.uint8).ravel())


# ---------------------------------------------------------------------------
# fp8 widening, every code: a one-token context returns its V row exactly
# ---------------------------------------------------------------------------
def _every_code_pool(d=128):
    """Two one-block sequences whose single token's V row holds the 256
    e4m3fn codes (the two NaN codes replaced by 0): with one key its
    softmax weight is exactly 1, so the output is the widened V row."""
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    nb, hkv = 2, 1
    k = np.full((nb, hkv, 16, d), 0x7F, np.uint8)      # NaN past the token
    v = np.full((nb, hkv, d, 16), 0x7F, np.uint8)
    rng = np.random.default_rng(5)
    k[:, :, 0, :] = rng.integers(0, 0x7F, (nb, hkv, d))  # finite codes
    for b in range(nb):
        v[b, 0, :, 0] = codes[b * d:(b + 1) * d]
    as_fp8 = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn)
    expect = oracle.numerics.e4m3fn_bits_to_f64(
        np.stack([v[b, 0, :, 0] for b in range(nb)]))   # [B, D]
    return as_fp8(k), as_fp8(v), expect


def test_fp8_decode_widens_every_code_exactly(gpu_lib):
    from paged_kv_cache_451_amd import _lib
    kp, vp, expect = _every_code_pool()
    hq = 4
    q = torch.randn(2, hq, 128).to(torch.bfloat16).cuda()
    tables = torch.tensor([[0], [1]], dtype=torch.int32).cuda()
    lens = torch.tensor([1, 1], dtype=torch.int32).cuda()
    out = torch.full_like(q, float("nan"))
    _lib.pa_decode(q, kp.cuda(), vp.cuda(), tables, lens, 0.125, out,
                   max_seq_len=1, k_scale=1.0, v_scale=1.0)
    torch.cuda.synchronize()
    got = out.cpu().to(torch.float64).numpy()               # [B, Hq, D]
    assert np.array_equal(got, np.repeat(expect[:, None, :], hq, axis=1))
