"""CPU check of the parity harness: the sliced, threaded oracle runs that the GPU
tests compare against equal the oracle run on the whole problem."""
import numpy as np
import torch

import oracle
import workloads as wl
from harness import block_errors, gpu_groups, host_f32, oracle_groups


def test_sliced_oracle_equals_whole_problem():
    case = wl.make_case("slices", [37, 130, 1, 77], head_num=6, kv_heads=2, head_dim=32, dtype=torch.bfloat16,
                        sparse_mode=3, alibi=True, sink=True, seed=21)
    a = (host_f32(case.q), host_f32(case.k), host_f32(case.v))
    kw = dict(sparse_mode=case.sparse_mode, alibi_slopes=case.alibi_slopes, sink=case.sink)
    args = (case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.scale)
    o, m, l = oracle.forward(*a, *args, **kw)
    dq, dk, dv, ds = oracle.backward(*a, host_f32(case.dy), *args, **kw)
    whole = gpu_groups(dict(out=o, m=m, l=l, dq=dq, dk=dk, dv=dv, dsink=ds), case, [1])
    parts = oracle_groups(case, [1], row_block=16, workers=3)
    for key in ("out", "m", "l", "dq", "dk", "dv", "dsink"):
        np.testing.assert_allclose(parts[key], whole[key], rtol=1e-12, atol=1e-13, err_msg=key)
    # the block view sees every (sequence, head) block of the group and no error
    errs = block_errors(whole["out"], parts["out"], case.cu_seqlens_q)
    assert len(errs) == 4 * 3 and max(e[0] for e in errs) < 1e-12


def test_sliced_oracle_modes_7_8():
    # the per-sequence modes (and mode 8's start indices) survive the slicing
    for mode, extra in ((7, {}), (8, dict(q_start_idx=30, kv_start_idx=0))):
        case = wl.make_case("slices78", [20, 9, 14], [50, 9, 14], head_num=4, kv_heads=2, head_dim=16,
                            dtype=torch.float32, sparse_mode=mode, pre_tokens=12, next_tokens=1,
                            alibi=mode == 8, sink=True, seed=23, **extra)
        a = (host_f32(case.q), host_f32(case.k), host_f32(case.v))
        kw = dict(sparse_mode=mode, pre_tokens=12, next_tokens=1, alibi_slopes=case.alibi_slopes, sink=case.sink,
                  q_start_idx=case.q_start_idx, kv_start_idx=case.kv_start_idx)
        args = (case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.scale)
        o, m, l = oracle.forward(*a, *args, **kw)
        dq, dk, dv, ds = oracle.backward(*a, host_f32(case.dy), *args, **kw)
        whole = gpu_groups(dict(out=o, m=m, l=l, dq=dq, dk=dk, dv=dv, dsink=ds), case, [0, 1])
        parts = oracle_groups(case, [0, 1], row_block=8, workers=2)
        for key in ("out", "m", "l", "dq", "dk", "dv", "dsink"):
            np.testing.assert_allclose(parts[key], whole[key], rtol=1e-12, atol=1e-13, err_msg=f"{mode} {key}")
