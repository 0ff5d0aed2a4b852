"""pa_decode_append_noalloc: the fused decode step without a workspace.

It runs the same kernels as pa_decode_append with the library's static
scratch buffer in place of the caller's workspace, so on the same input it
must give the same output bits and the same pools, and both must match the
oracle.  Two calls in a row, the second with a smaller input (another pool
type and batch), check that nothing the first call left in the shared
buffer leaks into the second.  A call whose scratch would not fit in the
buffer must be refused before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_451_amd.workloads import CONFIG_BY_NAME, build_case

from conftest import appended_pools, oracle_args, raw_bits

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp8_e4m3fn": 6e-2}
SCRATCH_BYTES = 32 << 20


def _dev(case):
    return {k: getattr(case, k).cuda() for k in
            ("q", "k_pool", "v_pool", "block_tables", "seq_lens",
             "slot_mapping", "k_new", "v_new")}


def _launch(case, dev, noalloc):
    from paged_kv_cache_451_amd import _lib
    out = torch.full_like(dev["q"], float("nan"))
    fn = _lib.pa_decode_append_noalloc if noalloc else _lib.pa_decode_append
    fn(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
       dev["seq_lens"], case.scale, out, dev["k_new"], dev["v_new"],
       dev["slot_mapping"], max_seq_len=case.max_seq_len,
       k_scale=case.k_scale, v_scale=case.v_scale,
       total_blocks_hint=case.total_blocks)
    return out


def _check_against_oracle(case, out, dev):
    kp, vp = appended_pools(case)
    assert np.array_equal(raw_bits(dev["k_pool"]).ravel(),
                          kp.view(np.uint8).ravel())
    assert np.array_equal(raw_bits(dev["v_pool"]).ravel(),
                          vp.view(np.uint8).ravel())
    args = oracle_args(case)
    args.update(k_raw=kp, v_raw=vp)
    ref = oracle.paged_decode(**args)
    g = out.cpu().to(torch.float64).numpy()
    assert np.isfinite(g).all()
    assert np.abs(g - ref).max() <= TOL[case.config.kv_dtype]


def test_noalloc_step_equals_the_workspace_step_twice_in_a_row(gpu_lib):
    from paged_kv_cache_451_amd import _lib
    big = build_case(CONFIG_BY_NAME["llama3_8b_bf16"], seed=1)
    small = build_case(CONFIG_BY_NAME["fp8_long"].replace(
        num_seqs=4, lo=1500, hi=5000), seed=0)
    for case in (big, small):
        desc = _lib.decode_desc(case.q, case.k_pool, case.block_tables,
                                max_seq_len=case.max_seq_len,
                                k_scale=case.k_scale, v_scale=case.v_scale,
                                total_blocks_hint=case.total_blocks)
        assert 0 < _lib.workspace_size(desc, fused=True) <= SCRATCH_BYTES
    # the two allocation-free calls back to back on one stream
    dev_a, dev_b = _dev(big), _dev(small)
    out_a = _launch(big, dev_a, noalloc=True)
    out_b = _launch(small, dev_b, noalloc=True)
    torch.cuda.synchronize()
    # the same steps with a caller-owned workspace
    ref_a_dev, ref_b_dev = _dev(big), _dev(small)
    ref_a = _launch(big, ref_a_dev, noalloc=False)
    ref_b = _launch(small, ref_b_dev, noalloc=False)
    torch.cuda.synchronize()
    for out, ref, dev, rdev, case in ((out_a, ref_a, dev_a, ref_a_dev, big),
                                      (out_b, ref_b, dev_b, ref_b_dev,
                                       small)):
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        for pool in ("k_pool", "v_pool"):
            assert np.array_equal(raw_bits(dev[pool]), raw_bits(rdev[pool]))
        _check_against_oracle(case, out, dev)


def test_noalloc_refuses_a_step_larger_than_its_scratch(gpu_lib):
    """2048 sequences x 32 query heads of size 128 need about 35 MB of
    partials: refused with PA_ERR_SCRATCH, nothing launched; the next call
    that fits runs normally."""
    from paged_kv_cache_451_amd import _lib
    b, hq, hkv, d, nb = 2048, 32, 8, 128, 64
    q = torch.zeros(b, hq, d, dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros(nb, hkv, 16, d, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros(nb, hkv, d, 16, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros(b, 1, dtype=torch.int32, device="cuda")
    lens = torch.ones(b, dtype=torch.int32, device="cuda")
    kn = torch.zeros(b, hkv, d, dtype=torch.bfloat16, device="cuda")
    slots = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    desc = _lib.decode_desc(q, kp, tables, max_seq_len=1,
                            total_blocks_hint=b)
    assert _lib.workspace_size(desc, fused=True) > SCRATCH_BYTES
    lib = _lib.load()
    st = lib.pa_decode_append_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kp.data_ptr()),
        ctypes.c_void_p(vp.data_ptr()), ctypes.c_void_p(tables.data_ptr()),
        ctypes.c_void_p(lens.data_ptr()), ctypes.c_float(0.1),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(kn.data_ptr()),
        ctypes.c_void_p(kn.data_ptr()), ctypes.c_void_p(slots.data_ptr()),
        ctypes.byref(desc),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -8
    assert lib.pa_status_string(st) == \
        b"call needs more than the library's static scratch buffer"
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    # a call that fits still works after the refusal
    case = build_case(CONFIG_BY_NAME["llama3_8b_bf16"].replace(
        num_seqs=8, lo=100, hi=1500), seed=3)
    dev = _dev(case)
    out = _launch(case, dev, noalloc=True)
    torch.cuda.synchronize()
    _check_against_oracle(case, out, dev)
