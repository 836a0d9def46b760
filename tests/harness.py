"""Shared helpers for the GPU parity tests: run the HIP library and the fp64
oracle on the same seeded inputs and compare them tensor by tensor."""
from __future__ import annotations

import os
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
                     atomic_dq=not deterministic, q_start_idx=case.q_start_idx, kv_start_idx=case.kv_start_idx,
                     v_head_dim=case.v.shape[2] if case.v.shape[2] != case.head_dim else None)


def device_inputs(case: wl.Case, device="cuda"):
    dev = torch.device(device)
    d = dict(q=case.q.to(dev), k=case.k.to(dev), v=case.v.to(dev), dy=case.dy.to(dev))
    d["drop"] = torch.from_numpy(case.drop_mask).to(dev) if case.drop_mask is not None else None
    d["slopes"] = torch.from_numpy(case.alibi_slopes).to(dev) if case.alibi_slopes is not None else None
    d["sink"] = torch.from_numpy(case.sink).to(dev) if case.sink is not None else None
    d["mask"] = torch.from_numpy(case.atten_mask).to(dev) if case.atten_mask is not None else None
    d["pse"] = case.pse.to(dev) if case.pse is not None else None
    return d


def run_gpu(case: wl.Case, deterministic: bool = True, backward: bool = True, inputs=None, heads=None,
            kv_heads=None):
    """fa_fwd (+ fa_bwd) on cuda:0; returns numpy fp64 copies of every output (of the
    query heads `heads` and kv heads `kv_heads` only, when given: the copies of the
    large workloads stay small)."""
    x = inputs if inputs is not None else device_inputs(case)
    cfg = config_of(case, deterministic, x.get("mask"), x.get("pse"))
    out, m, l = fa.fa_fwd(cfg, x["q"], x["k"], x["v"], x["drop"], x["slopes"], x["sink"])
    res = dict(out=out, m=m, l=l)
    if backward:
        dq, dk, dv, ds = fa.fa_bwd(cfg, x["q"], x["k"], x["v"], x["dy"], out, m, l, x["drop"], x["slopes"],
                                   x["sink"])
        res.update(dq=dq, dk=dk, dv=dv, dsink=ds)
    torch.cuda.synchronize()
    if heads is not None:
        hs = torch.tensor(list(heads), device=out.device)
        for key in ("out", "m", "l", "dq"):
            if key in res:
                res[key] = res[key].index_select(1, hs)
        if res.get("dsink") is not None:
            res["dsink"] = res["dsink"].index_select(0, hs)
    if kv_heads is not None:
        ks = torch.tensor(list(kv_heads), device=out.device)
        for key in ("dk", "dv"):
            if key in res:
                res[key] = res[key].index_select(1, ks)
    return {k: (None if v is None else v.detach().double().cpu().numpy()) for k, v in res.items()}


def host_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of a bf16 / fp16 / fp32 host tensor."""
    return t.float().numpy()


def run_oracle(case: wl.Case, batches=None, heads=None, backward: bool = True):
    q, k, v = host_f32(case.q), host_f32(case.k), host_f32(case.v)
    kw = dict(keep_prob=case.keep_prob, sparse_mode=case.sparse_mode, pre_tokens=case.pre_tokens,
              next_tokens=case.next_tokens, drop_mask=case.drop_mask, alibi_slopes=case.alibi_slopes,
              sink=case.sink, batches=batches, heads=heads, prefix=case.prefix, atten_mask=case.atten_mask,
              pse_type=case.pse_type, pse=None if case.pse is None else host_f32(case.pse),
              q_start_idx=case.q_start_idx, kv_start_idx=case.kv_start_idx)
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


def compare(gpu: dict, ref: dict, tol: float, keys=("out", "m", "l", "dq", "dk", "dv", "dsink"), kv_select=None,
            case=None):
    """Max relL2 over the compared tensors; raises AssertionError with a report when above tol.
    With `case`, every (sequence, head) block is checked as well (compare_blocks)."""
    report = {}
    for key in keys:
        if key not in ref or ref[key] is None:
            continue
        sel = kv_select if key in ("dk", "dv") else None
        report[key] = rel_l2(gpu[key], ref[key], sel)
    worst = max(report.values()) if report else 0.0
    say("relL2 " + " ".join(f"{k}={v:.2e}" for k, v in report.items()))
    assert worst <= tol, f"relL2 above {tol}: {report}"
    if case is not None:
        blk_ref = dict(ref)
        if kv_select is not None:
            for key in ("dk", "dv"):
                if blk_ref.get(key) is not None:
                    blk_ref[key] = np.where(kv_select, blk_ref[key], np.nan)
        compare_blocks(gpu, blk_ref, tol, case, keys=tuple(k for k in keys if k != "dsink"))
    return report


def kv_heads_complete(case: wl.Case, heads):
    """Mask over [T_kv, Nkv, D] selecting kv heads whose every query head is in `heads`."""
    g = case.head_num // case.kv_heads
    hs = set(range(case.head_num)) if heads is None else set(heads)
    ok = np.array([all((kv * g + j) in hs for j in range(g)) for kv in range(case.kv_heads)])
    sel = np.zeros((int(case.cu_seqlens_kv[-1]), case.kv_heads, case.head_dim), dtype=bool)
    sel[:, ok, :] = True
    return sel


# ---------------------------------------------------------------- sliced, parallel oracle runs

def slice_case(case: wl.Case, b: int, g: int) -> wl.Case:
    """Sequence b and kv group g of `case` as a problem of its own (one sequence, the
    group's G query heads, one kv head).  Varlen runs equal per-sequence runs and GQA
    groups are independent (both pinned oracle identities), so the oracle's result for
    the slice is that block of the whole problem's result."""
    if case.drop_mask is not None or case.pse is not None:
        raise ValueError("slice_case: keep-mask and external-pse cases are compared through oracle subsets")
    G = case.head_num // case.kv_heads
    q0, q1 = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
    k0, k1 = int(case.cu_seqlens_kv[b]), int(case.cu_seqlens_kv[b + 1])
    hs = slice(g * G, (g + 1) * G)
    slopes = None
    if case.alibi_slopes is not None:
        slopes = case.alibi_slopes[b:b + 1, hs] if case.alibi_slopes.ndim == 2 else case.alibi_slopes[hs]
    # modes 7 and 8 pick a mask by the sequence's place in the batch: the slice takes that
    # sequence's own mode (and, as mode 8's first sequence, its start indices)
    mode, qs, ks = case.sparse_mode, None, None
    if mode in (7, 8):
        if mode == 8 and b == 0:
            qs, ks = case.q_start_idx, case.kv_start_idx
        else:
            mode = oracle.sequence_mode(mode, b, case.batch)
    return wl.Case(name=f"{case.name} [seq {b}, group {g}]", dtype=case.dtype,
                   cu_seqlens_q=np.array([0, q1 - q0], np.int64), cu_seqlens_kv=np.array([0, k1 - k0], np.int64),
                   head_num=G, kv_heads=1, head_dim=case.head_dim, scale=case.scale,
                   q=case.q[q0:q1, hs], k=case.k[k0:k1, g:g + 1], v=case.v[k0:k1, g:g + 1],
                   dy=case.dy[q0:q1, hs], keep_prob=case.keep_prob, sparse_mode=mode,
                   pre_tokens=case.pre_tokens, next_tokens=case.next_tokens, alibi_slopes=slopes,
                   pse_type=case.pse_type, sink=None if case.sink is None else case.sink[hs],
                   prefix=None if case.prefix is None else case.prefix[b:b + 1], atten_mask=case.atten_mask,
                   q_start_idx=qs, kv_start_idx=ks)


def oracle_groups(case: wl.Case, groups, batches=None, row_block: int = 1024, workers: int = 0):
    """fp64 oracle over every sequence (or `batches`) of the kv groups `groups`, one
    (sequence, query head) per task on a thread pool (numpy releases the GIL in its array
    work; BLAS runs one thread per task).  Returns reference arrays restricted to the
    groups' heads: out, dq [T_q, |groups|*G, D]; m, l [T_q, |groups|*G]; dk, dv
    [T_kv, |groups|, D]; dsink [|groups|*G] (summed over the chosen sequences) -- rows of
    sequences not chosen are NaN."""
    from concurrent.futures import ThreadPoolExecutor, as_completed
    from threadpoolctl import threadpool_limits
    G = case.head_num // case.kv_heads
    groups = list(groups)
    bs = list(range(case.batch)) if batches is None else list(batches)
    tq, tkv, d = int(case.cu_seqlens_q[-1]), int(case.cu_seqlens_kv[-1]), case.head_dim
    nh = len(groups) * G
    ref = dict(out=np.full((tq, nh, d), np.nan), m=np.full((tq, nh), np.nan), l=np.full((tq, nh), np.nan),
               dq=np.full((tq, nh, d), np.nan), dk=np.full((tkv, len(groups), d), np.nan),
               dv=np.full((tkv, len(groups), d), np.nan),
               dsink=None if case.sink is None else np.zeros(nh))
    slices = {(b, g): slice_case(case, b, g) for b in bs for g in groups}
    # longest sequences first, so the pool's tail is short
    tasks = sorted(((b, g, h) for b in bs for g in groups for h in range(G)),
                   key=lambda t: -int(case.lens_q[t[0]]) * int(case.lens_kv[t[0]]))

    def one(task):
        b, g, h = task
        sc = slices[(b, g)]
        args = (host_f32(sc.q), host_f32(sc.k), host_f32(sc.v))
        kw = dict(keep_prob=sc.keep_prob, sparse_mode=sc.sparse_mode, pre_tokens=sc.pre_tokens,
                  next_tokens=sc.next_tokens, alibi_slopes=sc.alibi_slopes, sink=sc.sink, prefix=sc.prefix,
                  atten_mask=sc.atten_mask, pse_type=sc.pse_type, heads=[h], row_block=row_block,
                  q_start_idx=sc.q_start_idx, kv_start_idx=sc.kv_start_idx)
        o, m, l = oracle.forward(*args, sc.cu_seqlens_q, sc.cu_seqlens_kv, G, 1, sc.scale, **kw)
        dq, dk, dv, ds = oracle.backward(*args, host_f32(sc.dy), sc.cu_seqlens_q, sc.cu_seqlens_kv, G, 1,
                                         sc.scale, **kw)
        return task, (o[:, h], m[:, h], l[:, h], dq[:, h], dk[:, 0], dv[:, 0], None if ds is None else ds[h])

    n = workers or min(16, len(os.sched_getaffinity(0)))
    t0 = last = time.time()
    results = {}
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=n) as ex:
        futures = [ex.submit(one, t) for t in tasks]
        for f in as_completed(futures):
            task, res = f.result()
            results[task] = res
            if time.time() - last > 15:
                last = time.time()
                say(f"oracle: {len(results)} of {len(tasks)} tasks done")
    say(f"oracle: {len(tasks)} (sequence, head) tasks on {n} threads in {time.time() - t0:.1f} s")
    for b in bs:
        q0, q1 = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
        k0, k1 = int(case.cu_seqlens_kv[b]), int(case.cu_seqlens_kv[b + 1])
        for gi, g in enumerate(groups):
            dk = np.zeros((k1 - k0, d))
            dv = np.zeros((k1 - k0, d))
            for h in range(G):     # fixed order: query heads of the group
                o, m, l, dq, dkh, dvh, ds = results[(b, g, h)]
                c = gi * G + h
                ref["out"][q0:q1, c] = o
                ref["m"][q0:q1, c] = m
                ref["l"][q0:q1, c] = l
                ref["dq"][q0:q1, c] = dq
                dk += dkh
                dv += dvh
                if ds is not None:
                    ref["dsink"][c] += ds
            ref["dk"][k0:k1, gi] = dk
            ref["dv"][k0:k1, gi] = dv
    return ref


def gpu_groups(gpu: dict, case: wl.Case, groups) -> dict:
    """The GPU outputs restricted to the heads of kv groups `groups` (layout of oracle_groups)."""
    G = case.head_num // case.kv_heads
    heads = [g * G + h for g in groups for h in range(G)]
    res = {k: gpu[k][:, heads] for k in ("out", "m", "l", "dq")}
    res.update(dk=gpu["dk"][:, list(groups)], dv=gpu["dv"][:, list(groups)])
    if gpu.get("dsink") is not None:
        res["dsink"] = gpu["dsink"][heads]
    return res


def block_errors(got: np.ndarray, ref: np.ndarray, cu: np.ndarray):
    """relL2 of every (sequence, head) block of a [T, N, ...] tensor pair, as a list of
    (error, sequence, head, reference norm, block size); blocks the reference leaves NaN are
    skipped and -inf entries (empty rows) must match exactly."""
    out = []
    for b in range(len(cu) - 1):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 == r0:
            continue
        for n in range(ref.shape[1]):
            r = np.asarray(ref[r0:r1, n], np.float64)
            if np.all(np.isnan(r)):
                continue
            g = np.asarray(got[r0:r1, n], np.float64)
            inf = np.isinf(r)
            if np.any(inf):
                assert np.array_equal(g[inf], r[inf]), f"infinite entries of block ({b}, {n}) not reproduced"
            r, g = r[~inf], g[~inf]
            assert np.all(np.isfinite(g)), f"non-finite output in block ({b}, {n})"
            out.append((float(np.linalg.norm(g - r)), b, n, float(np.linalg.norm(r)), int(r.size)))
    return out


def compare_blocks(gpu: dict, ref: dict, tol: float, case: wl.Case, keys=("out", "m", "l", "dq", "dk", "dv"),
                   floor: float = 1.0):
    """Per-(sequence, head) check beside the whole-tensor one: every block's RMS error must be
    within tol of the larger of its own reference RMS and `floor` times the tensor's RMS.  The
    floor keeps blocks whose exact value cancels to (nearly) zero -- dQ and dK of a one-token
    sequence without a sink are exactly 0, while the device's D_i, formed from the rounded O,
    leaves rounding noise there -- from turning that noise into a large relative error.  A
    wrong wave block (32 rows of one head) has an error of the order of its own norm, which
    for any block of typical size is the tensor's RMS, and fails by a factor ~1/tol.  Prints
    the worst block of each tensor; raises AssertionError listing the blocks above the bound."""
    bad, worst = [], {}
    for key in keys:
        if key not in ref or ref[key] is None:
            continue
        cu = case.cu_seqlens_kv if key in ("dk", "dv") else case.cu_seqlens_q
        blocks = block_errors(gpu[key], ref[key], cu)
        if not blocks:
            continue
        r = np.asarray(ref[key], np.float64)
        fin = r[np.isfinite(r)]
        rms = float(np.sqrt(np.mean(fin * fin))) if fin.size else 0.0
        worst_b = None
        for err, b, n, nrm, size in blocks:
            den = max(nrm, floor * rms * np.sqrt(size))
            rel = err / den if den > 0 else err
            if worst_b is None or rel > worst_b[0]:
                worst_b = (rel, b, n)
            if rel > tol:
                bad.append((key, b, n, rel))
        worst[key] = worst_b
    say("worst blocks " + " ".join(f"{k}={v[0]:.2e}@(seq {v[1]}, head {v[2]})" for k, v in worst.items()))
    assert not bad, f"{len(bad)} blocks above {tol}: {bad[:8]}"
    return worst
