"""fa_decode_noalloc (the allocation-free decode entry point, scratch in a static device
buffer) against fa_decode with a caller workspace, through the C ABI: the same kernels on
the same inputs, so the outputs must be bit-identical.  Two calls in a row, the second
smaller (the buffer keeps the first call's contents), then a configuration beyond the
static buffer, which must be refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import workloads as wl
from harness import say

pytestmark = pytest.mark.gpu


def _inputs(c):
    cfg = fa.DecodeConfig(c.batch, c.max_seq_len, c.num_heads, c.num_kv_heads, c.head_dim, c.dtype, c.scale,
                          c.layout, c.lens)
    return cfg, c.q.cuda(), c.padded_cache("k", "cuda"), c.padded_cache("v", "cuda")


def test_noalloc_decode_matches_workspace_decode():
    # a split-heavy call (long sequences over several items, partial results in the scratch)
    # and then a smaller one that splits differently
    big = wl.make_decode_case("noalloc big", [16384, 3000, 1, 0, 9000], 16384, num_heads=64, num_kv_heads=8,
                              head_dim=128, dtype=torch.bfloat16, layout="BSND", seed=31)
    small = wl.make_decode_case("noalloc small", [700, 33], 1024, num_heads=16, num_kv_heads=2, head_dim=64,
                                dtype=torch.float16, layout="BNSD", seed=32)
    for c in (big, small):
        cfg, q, k, v = _inputs(c)
        need = fa.fa_decode_workspace_size(cfg)
        say(f"{c.name}: lens={list(c.lens)} scratch need {need} of {fa.FA_DECODE_NOALLOC_SCRATCH_BYTES}")
        assert need <= fa.FA_DECODE_NOALLOC_SCRATCH_BYTES
        ref = fa.fa_decode(cfg, q, k, v)
        out = torch.full_like(q, float("nan"))
        fa.fa_decode_noalloc(cfg, q, k, v, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), c.name
        # the same call again on the kept scratch contents
        out2 = torch.full_like(q, float("nan"))
        fa.fa_decode_noalloc(cfg, q, k, v, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref), c.name


def test_noalloc_decode_refuses_oversized_scratch():
    # 8192 sequences of 2048 keys over 8 kv heads: far more split partials than the buffer holds
    n = 8192
    cfg = fa.DecodeConfig(n, 2048, 64, 8, 128, torch.bfloat16, 0.0883883, "BSND", np.full(n, 2048))
    assert fa.fa_decode_workspace_size(cfg) > fa.FA_DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((n, 64, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device="cuda")
    # the size check runs before the tensors are read: pass views of the right shape over tiny storage
    k = kv.expand(n, 2048, 8, 128)
    out = torch.empty_like(q)
    with pytest.raises(fa.FaError) as e:
        fa.lib()
        st = fa.lib().fa_decode_noalloc(cfg.ref, q.data_ptr(), k.data_ptr(), k.data_ptr(), out.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_decode_noalloc")
    assert e.value.status == fa.FA_ERR_SCRATCH
