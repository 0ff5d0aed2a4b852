"""Negative controls on the device path: planted mistakes must break parity.

Each test feeds the C-ABI path one of the mistakes that paging can make
(the pages name the block table and its indirect addressing as what a paged
kernel adds: "49 vLLM / PagedAttention", section "Вопросы пытливого ума";
"PagedAttention：KV cache 即虚拟内存", section "面试官追问", output equal to
dense attention): an off-by-one length, a block-table entry pointing at
another sequence's valid block, query heads moved to other KV groups, and
a dropped score scale.  Each is an ordinary, in-bounds input.  For the
plain step (append, then decode) the device output must still match the
oracle run on the same mistaken input - the kernel computed what it was
given - and for both step forms it must fail the tolerance against the
oracle on the correct input.  So the tolerance that every parity test uses
is shown to catch each of these mistakes.

The batch mixes very short sequences (where one token or one block is a
large share of the softmax) with long ones.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_451_amd.workloads import CONFIG_BY_NAME, build_case

from conftest import appended_pools, oracle_args

pytestmark = pytest.mark.gpu

TOL = 2e-2
LENS = (1, 2, 3, 17, 33, 150, 700, 1500)


def _case():
    cfg = CONFIG_BY_NAME["llama3_8b_bf16"].replace(
        num_seqs=len(LENS), lens="fixed", fixed_lens=LENS)
    return build_case(cfg, 21)


def _oracle(case, **override):
    kp, vp = appended_pools(case)
    args = oracle_args(case)
    args.update(k_raw=kp, v_raw=vp)
    args.update(override)
    return oracle.paged_decode(**args)


def _device(case, fused, *, q=None, tables=None, lens=None, scale=None):
    from paged_kv_cache_451_amd import _lib
    dev = {k: getattr(case, k).cuda() for k in
           ("q", "k_pool", "v_pool", "block_tables", "seq_lens",
            "slot_mapping", "k_new", "v_new")}
    if q is not None:
        dev["q"] = torch.from_numpy(q).view(torch.bfloat16).cuda()
    if tables is not None:
        dev["block_tables"] = torch.from_numpy(tables).cuda()
    if lens is not None:
        dev["seq_lens"] = torch.from_numpy(lens).cuda()
    sc = case.scale if scale is None else scale
    out = torch.empty_like(dev["q"])
    kw = dict(max_seq_len=case.max_seq_len,
              total_blocks_hint=case.total_blocks)
    if fused:
        _lib.pa_decode_append(dev["q"], dev["k_pool"], dev["v_pool"],
                              dev["block_tables"], dev["seq_lens"], sc, out,
                              dev["k_new"], dev["v_new"],
                              dev["slot_mapping"], **kw)
    else:
        _lib.pa_kv_append(dev["k_new"], dev["v_new"], dev["slot_mapping"],
                          dev["k_pool"], dev["v_pool"])
        _lib.pa_decode(dev["q"], dev["k_pool"], dev["v_pool"],
                       dev["block_tables"], dev["seq_lens"], sc, out, **kw)
    torch.cuda.synchronize()
    g = out.cpu().to(torch.float64).numpy()
    assert np.isfinite(g).all()
    return g


def _mistakes(case):
    """name -> (device keyword arguments, oracle overrides)."""
    args = oracle_args(case)
    lens = case.seq_lens.numpy()
    short_by_one = (lens - 1).astype(np.int32)
    tab = case.block_tables.numpy().copy()
    tab[4, 0] = tab[7, 5]          # 33-token sequence reads a foreign block
    tab[6, 3] = tab[7, 9]
    hq = case.config.num_q_heads
    g = case.config.group
    perm = np.array([(h + g) % hq for h in range(hq)])   # next KV group
    q_moved = np.ascontiguousarray(args["q"][:, perm])
    return {
        "length off by one": (dict(lens=short_by_one),
                              dict(seq_lens=short_by_one)),
        "foreign block in the table": (dict(tables=tab),
                                       dict(block_tables=tab)),
        "query heads in other KV groups": (dict(q=q_moved), dict(q=q_moved)),
        "scale dropped": (dict(scale=1.0), dict(scale=1.0)),
    }


@pytest.mark.parametrize("fused", [False, True], ids=["append+decode",
                                                       "fused"])
@pytest.mark.parametrize("mistake", ["length off by one",
                                     "foreign block in the table",
                                     "query heads in other KV groups",
                                     "scale dropped"])
def test_planted_mistake_breaks_parity(gpu_lib, mistake, fused):
    case = _case()
    ref = _oracle(case)
    ok = _device(case, fused)
    assert np.abs(ok - ref).max() <= TOL          # the control itself
    dev_kw, oracle_kw = _mistakes(case)[mistake]
    got = _device(case, fused, **dev_kw)
    err = float(np.abs(got - ref).max())
    print(f"{mistake} ({'fused' if fused else 'append+decode'}): max abs "
          f"err against the correct oracle {err:.3f}")
    assert err > 10 * TOL
    if not fused:
        # the device computed exactly the mistaken input
        assert np.abs(got - _oracle(case, **oracle_kw)).max() <= TOL


# -- chunked prefill ----------------------------------------------------------

def _prefill_case():
    from paged_kv_cache_451_amd.workloads import PREFILL_BY_NAME, \
        build_prefill_case
    cfg = PREFILL_BY_NAME["prefill_llama3_8b_bf16"].replace(
        num_seqs=4, prior_lo=0, prior_hi=60)
    return build_prefill_case(cfg, seed=27, chunks=[1, 5, 40, 100])


def _prefill_mistakes(case):
    """name -> inputs that differ from the case's (numpy arrays)."""
    lens = case.seq_lens.numpy()
    qs = case.q_start.numpy()
    tab = case.block_tables.numpy().copy()
    tab[2, 0] = tab[3, 1]             # a sequence reads a foreign block
    hq = case.q.shape[1]
    g = hq // case.k_pool.shape[1]
    perm = np.array([(h + g) % hq for h in range(hq)])
    q_bits = case.q.view(torch.int16).numpy()
    moved = qs.copy()
    moved[2] += 1                     # a token moved to the next chunk
    return {
        "length off by one": dict(seq_lens=(lens - 1).astype(np.int32)),
        "chunk boundary off by one": dict(q_start=moved),
        "foreign block in the table": dict(block_tables=tab),
        "query heads in other KV groups": dict(
            q=np.ascontiguousarray(q_bits[:, perm])),
        "scale dropped": dict(scale=1.0),
    }


def _prefill_oracle(case, change):
    from conftest import prefill_args
    args = prefill_args(case)
    for k, v in change.items():
        args[k] = v.view(np.uint16) if k == "q" else v
    return oracle.paged_prefill(**args)


def _prefill_device(case, change):
    from paged_kv_cache_451_amd import _lib
    dev = {k: getattr(case, k).cuda() for k in
           ("q", "k_pool", "v_pool", "block_tables", "seq_lens", "q_start")}
    for k, v in change.items():
        if k == "q":
            dev["q"] = torch.from_numpy(v).view(torch.bfloat16).cuda()
        elif k != "scale":
            dev[k] = torch.from_numpy(v).cuda()
    out = torch.full_like(dev["q"], float("nan"))
    _lib.pa_prefill(dev["q"], dev["k_pool"], dev["v_pool"],
                    dev["block_tables"], dev["seq_lens"], dev["q_start"],
                    change.get("scale", case.scale), out)
    torch.cuda.synchronize()
    g = out.cpu().to(torch.float64).numpy()
    assert np.isfinite(g).all()
    return g


@pytest.mark.parametrize("mistake", ["length off by one",
                                     "chunk boundary off by one",
                                     "foreign block in the table",
                                     "query heads in other KV groups",
                                     "scale dropped"])
def test_planted_prefill_mistake_breaks_parity(gpu_lib, mistake):
    """The same controls for chunked prefill (plus a query token moved
    across a chunk boundary): the device computes the mistaken input as
    given and misses the correct oracle by more than 10x the tolerance."""
    case = _prefill_case()
    ref = _prefill_oracle(case, {})
    assert np.abs(_prefill_device(case, {}) - ref).max() <= TOL
    change = _prefill_mistakes(case)[mistake]
    got = _prefill_device(case, change)
    err = float(np.abs(got - ref).max())
    print(f"prefill, {mistake}: max abs err against the correct oracle "
          f"{err:.3f}")
    assert err > 10 * TOL
    assert np.abs(got - _prefill_oracle(case, change)).max() <= TOL


# -- cascade step ---------------------------------------------------------------

def test_claimed_prefix_one_block_too_long_reads_the_first_members_block(
        gpu_lib):
    """A group whose claimed shared prefix runs one block past the blocks
    its members really share: the cascade step reads that block through the
    first member's table for every member (what the claim means), so it
    matches the oracle over tables in which each member's entry is the
    first member's, and misses the correct oracle by more than 10x the
    tolerance (short own contexts make one block a large share)."""
    from paged_kv_cache_451_amd import _lib
    cfg = CONFIG_BY_NAME["prefix_shared_bf16"].replace(
        num_seqs=6, prefix_len=64, lo=20, hi=40)
    case = build_case(cfg, 8)
    p = 64 // 16
    tab = case.block_tables.numpy()
    assert all(tab[m, p] != tab[0, p] for m in range(1, 6))

    def step(prefix_blocks):
        dev = {k: getattr(case, k).cuda() for k in
               ("q", "k_pool", "v_pool", "block_tables", "seq_lens",
                "slot_mapping", "k_new", "v_new")}
        out = torch.full_like(dev["q"], float("nan"))
        _lib.pa_decode_append_shared(
            dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
            dev["seq_lens"], case.scale, out, dev["k_new"], dev["v_new"],
            dev["slot_mapping"],
            torch.tensor([0, 6], dtype=torch.int32, device="cuda"),
            torch.tensor([prefix_blocks], dtype=torch.int32, device="cuda"),
            max_seq_len=case.max_seq_len)
        torch.cuda.synchronize()
        g = out.cpu().to(torch.float64).numpy()
        assert np.isfinite(g).all()
        return g

    ref = _oracle(case)
    assert np.abs(step(p) - ref).max() <= TOL
    got = step(p + 1)
    err = float(np.abs(got - ref).max())
    print(f"cascade, prefix claimed one block too long: max abs err "
          f"against the correct oracle {err:.3f}")
    assert err > 10 * TOL
    claimed = tab.copy()
    claimed[1:, p] = tab[0, p]
    assert np.abs(got - _oracle(case, block_tables=claimed)).max() <= TOL
