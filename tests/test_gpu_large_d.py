"""Head dims above 128 (the grad page allows D up to 512, and qD == kD >= vD):
the materialised-score path against the fp64 oracle in bf16, fp16 and fp32, over
the mask family, dropout, ALiBi, the sink, GQA, cross attention, an empty key
range and a narrower value head dim; plus bitwise reproducibility."""
import numpy as np
import pytest
import torch

import workloads as wl
from harness import TOL, compare, device_inputs, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

BF16, F16, F32 = torch.bfloat16, torch.float16, torch.float32

LARGE_CASES = {
    "d192_causal_gqa_drop_alibi_sink": dict(lens_q=[150, 77, 300], head_num=4, kv_heads=2, head_dim=192,
                                            sparse_mode=3, keep_prob=0.9, alibi=True, sink=True),
    "d256_band_cross": dict(lens_q=[200, 129, 70], lens_kv=[300, 129, 64], head_num=4, kv_heads=1, head_dim=256,
                            sparse_mode=4, pre_tokens=64, next_tokens=16),
    "d512_nomask_sink": dict(lens_q=[130, 70], head_num=2, kv_heads=1, head_dim=512, sparse_mode=0, sink=True),
    "d256_v128_causal_drop": dict(lens_q=[190, 67, 129], head_num=4, kv_heads=2, head_dim=256, v_head_dim=128,
                                  sparse_mode=3, keep_prob=0.8),
    "d320_v192_mask_band_alibi": dict(lens_q=[150, 90], head_num=2, kv_heads=2, head_dim=320, v_head_dim=192,
                                      sparse_mode=4, pre_tokens=40, next_tokens=5, alibi=True, pse_type=3,
                                      mask=(0.3, [3])),
    "d256_prefix": dict(lens_q=[200, 77, 129, 5], lens_kv=[300, 40, 129, 64], head_num=2, kv_heads=1,
                        head_dim=256, sparse_mode=6, prefix=[150, 17, 64, 60]),
    "d256_mode8_split_alibi_sink": dict(lens_q=[150, 129, 64], lens_kv=[400, 129, 64], head_num=2, kv_heads=1,
                                        head_dim=256, sparse_mode=8, pre_tokens=180, next_tokens=0, alibi=True,
                                        sink=True, q_start_idx=250, kv_start_idx=0),
    "d256_empty_key_range": dict(lens_q=[50, 64, 0], lens_kv=[0, 64, 30], head_num=2, kv_heads=1, head_dim=256,
                                 sparse_mode=0, sink=True),
}


def _case(name, dtype, seed):
    kw = dict(LARGE_CASES[name])
    lq = kw.pop("lens_q")
    lkv = kw.pop("lens_kv", None)
    if "mask" in kw:
        p_masked, full_rows = kw.pop("mask")
        kw["atten_mask"] = wl.random_atten_mask(seed, max(lq), max(lkv or lq), p_masked, full_rows)
    return wl.make_case(name, lq, lkv, dtype=dtype, seed=seed, **kw)


@pytest.mark.parametrize("dtype", [BF16, F16, F32])
@pytest.mark.parametrize("name", list(LARGE_CASES))
def test_large_head_dim_against_oracle(name, dtype):
    seed = 500 + list(LARGE_CASES).index(name)
    case = _case(name, dtype, seed)
    say(f"large D {name} dtype={dtype} seed={seed} D={case.head_dim} vD={case.v.shape[2]} "
        f"lens={list(case.lens_q)}/{list(case.lens_kv)}")
    gpu = run_gpu(case, True)
    ref = run_oracle(case)
    compare(gpu, ref, TOL[dtype], case=case)


def test_large_head_dim_bitwise_reproducible():
    case = _case("d192_causal_gqa_drop_alibi_sink", BF16, 77)
    say("large D determinism")
    x = device_inputs(case)
    a = run_gpu(case, True, inputs=x)
    b = run_gpu(case, True, inputs=x)
    for key in ("out", "m", "l", "dq", "dk", "dv", "dsink"):
        assert np.array_equal(a[key], b[key]), key
