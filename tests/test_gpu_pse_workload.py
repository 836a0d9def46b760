"""Workload 4 (16 sequences x 2048, Nq = Nkv = 16, D = 128, causal, dropout 0.9, ALiBi) in fp32 with
its ALiBi bias handed over as an external pse tensor (pseType 0), full [1, N, S, S] or compressed to the
last 1024 rows, in the launch configuration `bench.py --workload 4 --dtype fp32 --pse full|compressed`
times (deterministic dQ): sampled (sequence, head) outputs against the fp64 oracle, and every output
against the same kernels run with the bias generated from the slopes (the same values)."""
import pytest
import torch

import attention_fa_fwd_amd as fa
import workloads as wl
from bench import alibi_pse
from harness import TOL, compare, device_inputs, kv_heads_complete, run_oracle, say

pytestmark = pytest.mark.gpu

F32 = torch.float32


@pytest.fixture(scope="module")
def w4():
    return wl.make_workload(4, F32)


def _run(case, pse):
    x = device_inputs(case)
    slopes = x["slopes"] if pse is None else None
    cfg = fa.Config(case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.head_dim,
                    case.dtype, case.scale, case.keep_prob, case.sparse_mode, case.pre_tokens, case.next_tokens,
                    True, **({} if pse is None else dict(pse=pse, pse_type=0)))
    out, m, l = fa.fa_fwd(cfg, x["q"], x["k"], x["v"], x["drop"], slopes, x["sink"])
    dq, dk, dv, ds = fa.fa_bwd(cfg, x["q"], x["k"], x["v"], x["dy"], out, m, l, x["drop"], slopes, x["sink"])
    torch.cuda.synchronize()
    res = dict(out=out, m=m, l=l, dq=dq, dk=dk, dv=dv)
    return {k: v.double().cpu().numpy() for k, v in res.items()}


@pytest.fixture(scope="module")
def generated(w4):
    say("workload 4 fp32, bias generated from the slopes")
    return _run(w4, None)


@pytest.mark.parametrize("form", ["full", "compressed"])
def test_workload4_fp32_external_pse(w4, generated, form):
    case = w4
    s_len = int(case.lens_q[0])
    pse = alibi_pse(torch.from_numpy(case.alibi_slopes).cuda(), s_len, s_len if form == "full" else 1024)
    assert pse.shape == (1, case.head_num, s_len if form == "full" else 1024, s_len)
    say(f"workload 4 fp32, external pse {form} {tuple(pse.shape)}")
    got = _run(case, pse)
    compare(got, generated, TOL[F32])
    batches, heads = [0, 15], [0, 9]
    say(f"  against the oracle: batches={batches} heads={heads}")
    ref = run_oracle(case, batches=batches, heads=heads)
    compare(got, ref, TOL[F32], keys=("out", "m", "l", "dq", "dk", "dv"),
            kv_select=kv_heads_complete(case, heads))
