"""Shared helpers for the GPU parity tests: run the HIP library and the fp64
oracle on the same seeded inputs and compare them tensor by tensor."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import attention_fa_fwd_amd as fa
import oracle
import workloads as wl

# Max relative L2 error per output tensor.  16-bit runs round P and dS (and the
# outputs) to the input type; the bound scales with that type's unit roundoff:
# bf16 u = 2^-8 -> 2e-2 (about 5u), fp16 u = 2^-11 -> 5e-3 (the same 5u, x2 margin).
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 5e-3}


def say(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def config_of(case: wl.Case, deterministic: bool = True, mask=None, pse=None) -> fa.Config:
    """mask, pse: the case's attenMask and external pse as device tensors (required when the case has them).
    deterministic=False selects the fp32-atomic dQ scheme, so the tests cover both backward variants."""
    return fa.Config(case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.head_dim,
                     case.dtype, case.scale, case.keep_prob, case.sparse_mode, case.pre_tokens,
                     case.next_tokens, deterministic, prefix=case.prefix, atten_mask=mask, pse_type=case.pse_type,
                     slopes_per_batch=case.alibi_slopes is not None and case.alibi_slopes.ndim == 2, pse=pse,
                     atomic_dq=not deterministic)


def device_inputs(case: wl.Case, device="cuda"):
    dev = torch.device(device)
    d = dict(q=case.q.to(dev), k=case.k.to(dev), v=case.v.to(dev), dy=case.dy.to(dev))
    d["drop"] = torch.from_numpy(case.drop_mask).to(dev) if case.drop_mask is not None else None
    d["slopes"] = torch.from_numpy(case.alibi_slopes).to(dev) if case.alibi_slopes is not None else None
    d["sink"] = torch.from_numpy(case.sink).to(dev) if case.sink is not None else None
    d["mask"] = torch.from_numpy(case.atten_mask).to(dev) if case.atten_mask is not None else None
    d["pse"] = case.pse.to(dev) if case.pse is not None else None
    return d


def run_gpu(case: wl.Case, deterministic: bool = True, backward: bool = True, inputs=None):
    """fa_fwd (+ fa_bwd) on cuda:0; returns numpy fp64 copies of every output."""
    x = inputs if inputs is not None else device_inputs(case)
    cfg = config_of(case, deterministic, x.get("mask"), x.get("pse"))
    out, m, l = fa.fa_fwd(cfg, x["q"], x["k"], x["v"], x["drop"], x["slopes"], x["sink"])
    res = dict(out=out, m=m, l=l)
    if backward:
        dq, dk, dv, ds = fa.fa_bwd(cfg, x["q"], x["k"], x["v"], x["dy"], out, m, l, x["drop"], x["slopes"],
                                   x["sink"])
        res.update(dq=dq, dk=dk, dv=dv, dsink=ds)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.detach().double().cpu().numpy()) for k, v in res.items()}


def host_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of a bf16 / fp16 / fp32 host tensor."""
    return t.float().numpy()


def run_oracle(case: wl.Case, batches=None, heads=None, backward: bool = True):
    q, k, v = host_f32(case.q), host_f32(case.k), host_f32(case.v)
    kw = dict(keep_prob=case.keep_prob, sparse_mode=case.sparse_mode, pre_tokens=case.pre_tokens,
              next_tokens=case.next_tokens, drop_mask=case.drop_mask, alibi_slopes=case.alibi_slopes,
              sink=case.sink, batches=batches, heads=heads, prefix=case.prefix, atten_mask=case.atten_mask,
              pse_type=case.pse_type, pse=None if case.pse is None else host_f32(case.pse))
    o, m, l = oracle.forward(q, k, v, case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads,
                             case.scale, **kw)
    res = dict(out=o, m=m, l=l)
    if backward:
        dq, dk, dv, ds = oracle.backward(q, k, v, host_f32(case.dy), case.cu_seqlens_q, case.cu_seqlens_kv,
                                         case.head_num, case.kv_heads, case.scale, **kw)
        res.update(dq=dq, dk=dk, dv=dv, dsink=ds)
    return res


def rel_l2(got: np.ndarray, ref: np.ndarray, select=None) -> float:
    """||got - ref|| / ||ref|| over the entries the oracle computed (non-NaN);
    -inf reference entries must be matched exactly and are left out of the norm."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    sel = ~np.isnan(ref) if select is None else select & ~np.isnan(ref)
    r, g = ref[sel], got[sel]
    inf = np.isinf(r)
    if np.any(inf):
        assert np.array_equal(g[inf], r[inf]), "infinite reference entries not reproduced"
    r, g = r[~inf], g[~inf]
    assert np.all(np.isfinite(g)), "non-finite output where the reference is finite"
    den = np.linalg.norm(r)
    num = np.linalg.norm(g - r)
    return float(num / den) if den > 0 else float(num)


def compare(gpu: dict, ref: dict, tol: float, keys=("out", "m", "l", "dq", "dk", "dv", "dsink"), kv_select=None):
    """Max relL2 over the compared tensors; raises AssertionError with a report when above tol."""
    report = {}
    for key in keys:
        if key not in ref or ref[key] is None:
            continue
        sel = kv_select if key in ("dk", "dv") else None
        report[key] = rel_l2(gpu[key], ref[key], sel)
    worst = max(report.values()) if report else 0.0
    say("relL2 " + " ".join(f"{k}={v:.2e}" for k, v in report.items()))
    assert worst <= tol, f"relL2 above {tol}: {report}"
    return report


def kv_heads_complete(case: wl.Case, heads):
    """Mask over [T_kv, Nkv, D] selecting kv heads whose every query head is in `heads`."""
    g = case.head_num // case.kv_heads
    hs = set(range(case.head_num)) if heads is None else set(heads)
    ok = np.array([all((kv * g + j) in hs for j in range(g)) for kv in range(case.kv_heads)])
    sel = np.zeros((int(case.cu_seqlens_kv[-1]), case.kv_heads, case.head_dim), dtype=bool)
    sel[:, ok, :] = True
    return sel
