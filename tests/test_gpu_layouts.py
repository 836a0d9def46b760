"""GPU checks of the fixed-length input layouts (BSH, BSND, BNSD, SBH): the same
problem in each layout must give bit-identical results to the packed TND run
(deterministic backward), whose parity with the oracle is tested elsewhere; one
layout is also compared with the oracle directly."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import workloads as wl
from harness import TOL, compare, run_oracle, say

pytestmark = pytest.mark.gpu

B, SQ, SKV = 3, 200, 333


def to_layout(x, layout, b, s):
    """[B*S, N, D] (TND, equal lengths) -> the layout's tensor (contiguous)."""
    t, n, d = x.shape
    x4 = x.reshape(b, s, n, d)
    return {"TND": x, "BSND": x4, "BSH": x4.reshape(b, s, n * d), "BNSD": x4.permute(0, 2, 1, 3),
            "SBH": x4.permute(1, 0, 2, 3).reshape(s, b, n * d)}[layout].contiguous()


def from_layout(y, layout, b, s, n, d):
    x4 = {"TND": lambda: y.reshape(b, s, n, d), "BSND": lambda: y, "BSH": lambda: y.reshape(b, s, n, d),
          "BNSD": lambda: y.permute(0, 2, 1, 3), "SBH": lambda: y.reshape(s, b, n, d).permute(1, 0, 2, 3)}[layout]()
    return x4.reshape(b * s, n, d).contiguous()


def _case(dtype, seed, **kw):
    return wl.make_case("layouts", [SQ] * B, [SKV] * B, head_num=4, kv_heads=2, head_dim=128, dtype=dtype, seed=seed,
                        **kw)


def _run(case, layout, deterministic=True):
    dev = torch.device("cuda")
    cfg = fa.Config(case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.head_dim, case.dtype,
                    case.scale, case.keep_prob, case.sparse_mode, case.pre_tokens, case.next_tokens, deterministic,
                    layout=layout, atomic_dq=not deterministic)
    q = to_layout(case.q, layout, B, SQ).to(dev)
    k = to_layout(case.k, layout, B, SKV).to(dev)
    v = to_layout(case.v, layout, B, SKV).to(dev)
    dy = to_layout(case.dy, layout, B, SQ).to(dev)
    drop = torch.from_numpy(case.drop_mask).to(dev) if case.drop_mask is not None else None
    sink = torch.from_numpy(case.sink).to(dev) if case.sink is not None else None
    out, m, l = fa.fa_fwd(cfg, q, k, v, drop, None, sink)
    dq, dk, dv, ds = fa.fa_bwd(cfg, q, k, v, dy, out, m, l, drop, None, sink)
    torch.cuda.synchronize()
    nq, nkv, d = case.head_num, case.kv_heads, case.head_dim
    res = dict(out=from_layout(out, layout, B, SQ, nq, d), m=m, l=l, dq=from_layout(dq, layout, B, SQ, nq, d),
               dk=from_layout(dk, layout, B, SKV, nkv, d), dv=from_layout(dv, layout, B, SKV, nkv, d), dsink=ds)
    return {key: (None if t is None else t.double().cpu().numpy()) for key, t in res.items()}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("layout", ["BSND", "BSH", "BNSD", "SBH"])
def test_layout_is_bitwise_the_tnd_result(layout, dtype):
    case = _case(dtype, 31, sparse_mode=3, keep_prob=0.85, sink=True)
    say(f"layout {layout} dtype={dtype}")
    ref, got = _run(case, "TND"), _run(case, layout)
    for key in ("out", "m", "l", "dq", "dk", "dv", "dsink"):
        assert np.array_equal(got[key], ref[key]), key


def test_layout_against_the_oracle():
    case = _case(torch.bfloat16, 32, sparse_mode=4, pre_tokens=64, next_tokens=16)
    say("layout SBH vs oracle")
    compare(_run(case, "SBH", deterministic=False), run_oracle(case), TOL[torch.bfloat16])


def _views(x, kind):
    """The same values as a strided TND view: padded D rows, every other head of a wider
    tensor, or a head-major (transposed) storage."""
    t, n, d = x.shape
    if kind == "padded":
        buf = torch.full((t, n, d + 8), float("nan"), dtype=x.dtype, device=x.device)
        buf[:, :, :d] = x
        return buf[:, :, :d]
    if kind == "every_other_head":
        buf = torch.full((t, 2 * n, d), float("nan"), dtype=x.dtype, device=x.device)
        buf[:, ::2] = x
        return buf[:, ::2]
    return x.permute(1, 0, 2).contiguous().permute(1, 0, 2)   # head-major storage


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_strided_tnd_views_are_bitwise_the_packed_result(dtype):
    case = wl.make_case("strided", [37, 200, 129], [90, 200, 64], head_num=4, kv_heads=2, head_dim=128,
                        dtype=dtype, seed=33, sparse_mode=0, keep_prob=0.9, sink=True)
    say(f"strided TND views dtype={dtype}")
    dev = torch.device("cuda")
    cfg = fa.Config(case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.head_dim, dtype,
                    case.scale, case.keep_prob, case.sparse_mode, deterministic=True)
    q, k, v, dy = (t.to(dev) for t in (case.q, case.k, case.v, case.dy))
    drop = torch.from_numpy(case.drop_mask).to(dev)
    sink = torch.from_numpy(case.sink).to(dev)
    out, m, l = fa.fa_fwd(cfg, q, k, v, drop, None, sink)
    ref = fa.fa_bwd(cfg, q, k, v, dy, out, m, l, drop, None, sink)
    torch.cuda.synchronize()
    # strided inputs and strided outputs (views into larger buffers)
    qs, ks, vs, dys = _views(q, "padded"), _views(k, "every_other_head"), _views(v, "head_major"), _views(dy, "padded")
    outs = _views(torch.zeros_like(q), "every_other_head")
    outs, ms, ls = fa.fa_fwd(cfg, qs, ks, vs, drop, None, sink, out=outs)
    dqs, dks, dvs = (_views(torch.zeros_like(t), kind) for t, kind in ((q, "head_major"), (k, "padded"),
                                                                      (v, "every_other_head")))
    got = fa.fa_bwd(cfg, qs, ks, vs, dys, outs, ms, ls, drop, None, sink, dq=dqs, dk=dks, dv=dvs)
    torch.cuda.synchronize()
    assert torch.equal(outs, out) and torch.equal(ms, m) and torch.equal(ls, l)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_autograd_binding_matches_the_direct_calls():
    from attention_fa_fwd_amd.autograd import varlen_attention
    case = wl.make_case("autograd", [37, 200], head_num=4, kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                        seed=34, sparse_mode=3, keep_prob=0.9, sink=True, alibi=True)
    say("autograd binding")
    dev = torch.device("cuda")
    cfg = fa.Config(case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.head_dim,
                    case.dtype, case.scale, case.keep_prob, case.sparse_mode, deterministic=True)
    q, k, v, dy = (t.to(dev) for t in (case.q, case.k, case.v, case.dy))
    drop = torch.from_numpy(case.drop_mask).to(dev)
    slopes = torch.from_numpy(case.alibi_slopes).to(dev)
    sink = torch.from_numpy(case.sink).to(dev)
    out, m, l = fa.fa_fwd(cfg, q, k, v, drop, slopes, sink)
    ref = fa.fa_bwd(cfg, q, k, v, dy, out, m, l, drop, slopes, sink)
    qg, kg, vg, sg = (t.clone().requires_grad_(True) for t in (q, k, v, sink))
    o2 = varlen_attention(qg, kg, vg, cfg, sink=sg, alibi_slopes=slopes, drop_mask=drop)
    o2.backward(dy)
    torch.cuda.synchronize()
    assert torch.equal(o2.detach(), out)
    for got, want in ((qg.grad, ref[0]), (kg.grad, ref[1]), (vg.grad, ref[2]), (sg.grad, ref[3])):
        assert torch.equal(got, want)
