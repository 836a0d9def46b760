"""External pse with bf16 / fp16 inputs (the grad page's pseShiftOptional in FLOAT16 /
BFLOAT16; the ScoreV2 page's realShiftOptional): the library runs these calls on the
materialised-score path, since the fused 16-bit kernels have no external-pse
instances.  Checked against the fp64 oracle over the three tensor forms (full block,
one shared row, 1024-row compression), pseType 0 and 1, cross attention, GQA,
dropout, the sink, a padded head dim and a narrower value head dim; plus bitwise
reproducibility in both backward modes (both run the same deterministic passes)."""
import numpy as np
import pytest
import torch

import workloads as wl
from harness import TOL, compare, device_inputs, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

BF16, F16 = torch.bfloat16, torch.float16

PSE16_CASES = {
    "full_type1_cross_gqa": dict(lens_q=[180, 95, 129], lens_kv=[140, 260, 129], head_num=4, kv_heads=2,
                                 head_dim=128, sparse_mode=0, pse=("full", False), pse_type=1),
    "row_type0_causal_drop_sink": dict(lens_q=[170, 66], head_num=2, kv_heads=1, head_dim=64, sparse_mode=3,
                                       pse=("row", True), pse_type=0, keep_prob=0.8, sink=True),
    "compressed_causal": dict(lens_q=[1090, 260], head_num=2, kv_heads=2, head_dim=64, sparse_mode=3,
                              pse=("compressed", False), pse_type=1),
    "full_type0_band_d96": dict(lens_q=[210, 33, 129], head_num=4, kv_heads=1, head_dim=96, sparse_mode=4,
                                pre_tokens=50, next_tokens=9, pse=("full", True), pse_type=0),
    "full_type1_lucausal_v64": dict(lens_q=[150, 200], lens_kv=[220, 120], head_num=2, kv_heads=2, head_dim=128,
                                    v_head_dim=64, sparse_mode=2, pse=("full", False), pse_type=1, sink=True),
}


def _case(name, dtype, seed):
    kw = dict(PSE16_CASES[name])
    lq = kw.pop("lens_q")
    lkv = kw.pop("lens_kv", None)
    return wl.make_case("pse16 " + name, lq, lkv, dtype=dtype, seed=seed, **kw)


@pytest.mark.parametrize("deterministic", [True, False])
@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("name", list(PSE16_CASES))
def test_pse_16bit_against_oracle(name, dtype, deterministic):
    seed = 700 + list(PSE16_CASES).index(name)
    case = _case(name, dtype, seed)
    say(f"pse16 {name} dtype={dtype} det={deterministic} seed={seed} lens={list(case.lens_q)}/"
        f"{list(case.lens_kv)} pse={tuple(case.pse.shape)}")
    gpu = run_gpu(case, deterministic)
    ref = run_oracle(case)
    compare(gpu, ref, TOL[dtype], case=case)


def test_pse_16bit_bitwise_reproducible():
    case = _case("full_type1_cross_gqa", BF16, 71)
    say("pse16 determinism")
    x = device_inputs(case)
    a = run_gpu(case, True, inputs=x)
    b = run_gpu(case, False, inputs=x)
    for key in ("out", "m", "l", "dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key
