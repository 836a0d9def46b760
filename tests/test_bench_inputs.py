"""CPU checks of the benchmark's own input construction: the external-pse tensor that
`bench.py --pse full|compressed` builds from workload 4's slopes must be the bias the oracle
generates from the same slopes (pseType 2), in both forms, on the lower triangle the causal
mask keeps; and the option combinations the benchmark refuses exit with a message."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from bench import ROOT, alibi_pse

SLOPES = np.array([2.0 ** (-8.0 * (h + 1) / 4) for h in range(4)], dtype=np.float32)


@pytest.mark.parametrize("s_len, rows", [(64, 64), (1100, 1024), (2048, 1024)])
def test_external_pse_tensor_is_the_generated_bias(s_len, rows):
    pse = alibi_pse(torch.from_numpy(SLOPES), s_len, rows).numpy()
    assert pse.shape == (1, len(SLOPES), rows, s_len) and pse.dtype == np.float32
    low = np.tril(np.ones((s_len, s_len), dtype=bool))
    for h, slope in enumerate(SLOPES):
        want = oracle.alibi_pse(s_len, s_len, float(slope), 2)
        got = oracle.pse_block(pse, 0, h, s_len, s_len)
        sel = low & ~np.isnan(got)
        assert sel[low].all(), "the tensor leaves part of the lower triangle undefined"
        np.testing.assert_allclose(got[sel], want[sel], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("argv", [["--pse", "full"], ["--workload", "4", "--pse", "compressed", "--layout", "BSND"],
                                  ["--decode", "--dtype", "fp32"]])
def test_refused_option_combinations(argv):
    r = subprocess.run([sys.executable, "bench.py", "--no-cpu-baseline"] + argv, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "--pse" in r.stderr or "decode attention takes" in r.stderr


def test_kernel_source_groups_cover_every_source():
    # stored HBM counters are tied to a hash of their path's sources: every csrc file must
    # belong to exactly one group, so that no kernel change goes unnoticed
    import bench
    csrc = os.path.join(ROOT, "attention_fa_fwd_amd", "csrc")
    groups = [f for fs in bench.KERNEL_SOURCES.values() for f in fs] + list(bench.SHARED_SOURCES) + \
        list(bench.HOST_SOURCES)
    assert len(groups) == len(set(groups))
    assert set(groups) == set(os.listdir(csrc))
    assert len({bench.kernel_source_hash(p) for p in bench.KERNEL_SOURCES}) == len(bench.KERNEL_SOURCES)
