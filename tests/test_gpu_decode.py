"""GPU parity of decode attention: libfa.so's fa_decode (through the C ABI) against
the fp64 decode oracle on the same seeded inputs.  Tolerances as for the
training path: max relative L2 error 2e-2 for bf16 and 5e-3 for fp16 inputs."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
import workloads as wl
from harness import TOL, rel_l2, say

pytestmark = pytest.mark.gpu

BF16, F16 = torch.bfloat16, torch.float16

# lengths span several 32-key steps, ragged tails, empty sequences, split sequences
# (more keys than one work item takes) and every group width the kernel has
DECODE_CASES = {
    "gqa8_bsnd_varlen": dict(lens=[1, 37, 300, 1025, 0, 64], s=1100, nq=16, nkv=2, d=128, layout="BSND"),
    "mha_bsh_d64": dict(lens=[129, 5, 640], s=700, nq=4, nkv=4, d=64, layout="BSH"),
    "mqa64_bnsd_mask": dict(lens=[500, 33, 2000], s=2048, nq=64, nkv=1, d=128, layout="BNSD", mask_p=0.3),
    "group48_d64_mask": dict(lens=[100, 1000, 0], s=1024, nq=48, nkv=1, d=64, layout="BSND", mask_p=0.5),
    "long_split": dict(lens=[16384, 7000, 31], s=16384, nq=8, nkv=8, d=128, layout="BSND"),
    "masked_rows_bnsd": dict(lens=[300, 77], s=320, nq=8, nkv=2, d=64, layout="BNSD", mask_p=0.2,
                             full_rows=[1]),
    # one long sequence over 4 kv heads: the split rule grows the chunk to 3072 keys (1024 per wave)
    "chunk_growth": dict(lens=[100000], s=100000, nq=16, nkv=4, d=128, layout="BSND"),
    # a large batch of short sequences (empty ones included), one item each
    "many_short": dict(lens=[int(x) for x in np.random.default_rng(7).integers(0, 41, 512)], s=40, nq=8, nkv=2,
                       d=64, layout="BSH"),
}


def _case(name, dtype, seed):
    kw = dict(DECODE_CASES[name])
    c = wl.make_decode_case(name, kw["lens"], kw["s"], num_heads=kw["nq"], num_kv_heads=kw["nkv"],
                            head_dim=kw["d"], dtype=dtype, layout=kw["layout"], seed=seed,
                            mask_p=kw.get("mask_p", 0.0))
    for b in kw.get("full_rows", []):
        c.atten_mask[b, :] = 1
    return c


def run_decode(c, batches=None):
    """fa_decode on cuda:0 over the listed sequences (all by default); returns out as fp64 numpy."""
    bl = list(range(c.batch)) if batches is None else list(batches)
    mask = None if c.atten_mask is None else torch.from_numpy(c.atten_mask[bl]).cuda()
    cfg = fa.DecodeConfig(len(bl), c.max_seq_len, c.num_heads, c.num_kv_heads, c.head_dim, c.dtype, c.scale,
                          c.layout, c.lens[bl], mask)
    q = c.q[bl].cuda()
    k, v = c.padded_cache("k", "cuda", bl), c.padded_cache("v", "cuda", bl)
    out = fa.fa_decode(cfg, q, k, v)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def run_oracle(c, batches=None):
    bl = list(range(c.batch)) if batches is None else list(batches)
    k = c.padded_cache("k", "cpu", bl).float().numpy()
    v = c.padded_cache("v", "cpu", bl).float().numpy()
    mask = None if c.atten_mask is None else c.atten_mask[bl]
    return oracle.decode(c.q[bl].float().numpy(), k, v, c.num_heads, c.num_kv_heads, c.scale, c.layout,
                         c.lens[bl], mask)


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_case(name, dtype):
    seed = 200 + list(DECODE_CASES).index(name)
    c = _case(name, dtype, seed)
    say(f"decode {name} dtype={dtype} seed={seed} lens={list(c.lens)}")
    got, ref = run_decode(c), run_oracle(c)
    empty = [b for b in range(c.batch) if c.lens[b] == 0]
    for b in empty:
        assert np.array_equal(got[b], np.zeros_like(got[b])), b
    err = rel_l2(got, ref)
    say(f"relL2 out={err:.2e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_decode_workload_sampled(dtype):
    # the timed decode workload, in the launch configuration the benchmark times (every
    # sequence in one call), checked on the shortest, a median and the longest sequence
    c = wl.make_decode_workload(dtype)
    order = np.argsort(c.lens)
    picks = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    say(f"decode workload dtype={dtype} sequences={picks} lens={[int(c.lens[b]) for b in picks]}")
    got = run_decode(c)
    ref = run_oracle(c, picks)
    err = rel_l2(got[picks], ref)
    say(f"relL2 out={err:.2e}")
    assert err <= TOL[dtype]
    assert np.all(np.isfinite(got))


def test_decode_is_deterministic():
    c = _case("long_split", BF16, 9)
    a, b = run_decode(c), run_decode(c)
    assert np.array_equal(a, b)
