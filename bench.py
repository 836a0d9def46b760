"""Throughput benchmark of the varlen FlashAttention forward + backward on one MI355X.

One step = one full pass of the path over the packed workload: host validation
and tile scheduling, the forward kernel, the backward preprocess, the dK/dV
pass, the dQ pass and the dSink reduction.  Inputs are generated once, are
resident in HBM before timing starts, and are synthetic (seeded normal draws of
the workload's shapes; the pages name no dataset).

Prints ONE JSON line (metric, value, roofline of the dominant kernel, CPU
baseline of the fp64 oracle on a bounded sample).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--atomic-dq]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (published)
HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# Device-code sources of each path (csrc files); the shared headers belong to every path, and
# the host API (fa_api.hip) holds no kernel.  Stored counters stay valid while their path's hash does.
KERNEL_SOURCES = {
    "training": ("fa_fwd.hip", "fa_bwd.hip", "fa_bwd_kv.h", "fa_bwd_kv.hip", "fa_bwd_kv_atomic.hip", "fa_layout.hip"),
    "large": ("fa_large.hip",),
    "decode": ("fa_decode.hip",),
}
SHARED_SOURCES = ("fa_device.h", "fa_kernels.h", "fa_sched.h")
HOST_SOURCES = ("fa_api.hip",)


def kernel_source_hash(path: str = "training") -> str:
    """Hash of the device-code sources that the kernels of `path` are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_fa_fwd_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[path] + SHARED_SOURCES):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def alibi_pse(slopes, s_len, rows):
    """Workload 4's ALiBi bias as an external pse tensor [1, N, rows, S] (pseType 0, added after
    scaling): -slope_h * (i - j) for the last `rows` query rows i of an S x S block."""
    import torch
    i = torch.arange(s_len - rows, s_len, device=slopes.device, dtype=torch.float64)[:, None]
    j = torch.arange(s_len, device=slopes.device, dtype=torch.float64)[None, :]
    return (-slopes.double()[:, None, None] * (i - j)).float()[None].contiguous()


def timed_steps(step, steps, stream, cold_cache, dev):
    """Times `steps` calls of step() with HIP events on `stream`: one event between
    consecutive steps, so each step's duration is known.  Returns (mean ms per step
    over the whole bracket, wall seconds, per-step ms).  With cold_cache, a 1 GiB
    buffer is overwritten between steps (outside each step's events) so that no step
    finds its inputs in the 256 MB last-level cache; the mean is then the mean of the
    per-step durations."""
    import torch
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev) if cold_cache else None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps if cold_cache else steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    if cold_cache:
        for i in range(steps):
            scratch.fill_(float(i))
            ev[2 * i].record(stream)
            step()
            ev[2 * i + 1].record(stream)
    else:
        ev[0].record(stream)
        for i in range(steps):
            step()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    if cold_cache:
        per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]
        return float(np.mean(per)), wall, per
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, wall, per


def flops_of(case):
    import workloads as wl
    pairs = wl.allowed_pairs(case.lens_q, case.lens_kv, case.head_num, case.sparse_mode, case.pre_tokens,
                             case.next_tokens)
    d = case.head_dim
    return pairs, 4.0 * d * pairs, 10.0 * d * pairs


def cpu_baseline(case, budget_s: float = 12.0):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload:
    (sequence, kv-group) units taken in a fixed order (sequences nearest the
    median length first) until the time budget is spent."""
    import oracle
    import workloads as wl
    cores = len(os.sched_getaffinity(0))
    g = case.head_num // case.kv_heads
    lens = case.lens_q
    order = np.argsort(np.abs(lens - np.median(lens)), kind="stable")
    q = case.q.float().numpy()
    k = case.k.float().numpy()
    v = case.v.float().numpy()
    dy = case.dy.float().numpy()
    kw = dict(keep_prob=case.keep_prob, sparse_mode=case.sparse_mode, pre_tokens=case.pre_tokens,
              next_tokens=case.next_tokens, drop_mask=case.drop_mask, alibi_slopes=case.alibi_slopes,
              sink=case.sink)
    done_pairs, units, t_total = 0, [], 0.0
    for b in order:
        for grp in range(case.kv_heads):
            heads = list(range(grp * g, grp * g + g))
            t0 = time.perf_counter()
            oracle.forward(q, k, v, case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads,
                           case.scale, batches=[int(b)], heads=heads, **kw)
            oracle.backward(q, k, v, dy, case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads,
                            case.scale, batches=[int(b)], heads=heads, **kw)
            t_total += time.perf_counter() - t0
            L = int(lens[b])
            done_pairs += wl.allowed_pairs([L], [int(case.lens_kv[b])], len(heads), case.sparse_mode,
                                           case.pre_tokens, case.next_tokens)
            units.append((int(b), grp, L))
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    fl = 14.0 * case.head_dim * done_pairs
    return {
        "value": fl / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle fwd+bwd on {len(units)} (sequence, kv-group) units of this workload "
                   f"(lengths {sorted(set(u[2] for u in units))}, {g} query heads each), {done_pairs} allowed "
                   f"pairs in {t_total:.1f} s; mask-aware 14*D FLOP per pair"),
    }


def decode_cpu_baseline(case, budget_s: float = 10.0):
    """The fp64 decode oracle on whole sequences of the decode workload (nearest the
    median length first) until the time budget is spent; rate in K/V bytes read."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    order = np.argsort(np.abs(case.lens - np.median(case.lens)), kind="stable")
    t_total, done, nbytes = 0.0, [], 0
    row_bytes = 2 * case.num_kv_heads * case.head_dim * 2
    for b in order:
        k = case.padded_cache("k", "cpu", [int(b)]).float().numpy()
        v = case.padded_cache("v", "cpu", [int(b)]).float().numpy()
        q = case.q[[int(b)]].float().numpy()
        t0 = time.perf_counter()
        oracle.decode(q, k, v, case.num_heads, case.num_kv_heads, case.scale, case.layout, case.lens[[int(b)]])
        t_total += time.perf_counter() - t0
        done.append(int(case.lens[b]))
        nbytes += int(case.lens[b]) * row_bytes
        if t_total >= budget_s:
            break
    return {
        "value": nbytes / t_total / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"fp64 numpy decode oracle on {len(done)} whole sequences of this workload (key lengths "
                   f"{sorted(done)}), {nbytes} bytes of K/V rows in {t_total:.1f} s"),
    }


def decode_bench(args):
    """Decode attention over the decode workload: one step = one fa_decode call over
    every sequence (host split planning, the decode kernel, the split reduction)."""
    if args.dtype == "fp32":
        sys.exit("decode attention takes bf16 or fp16 inputs")
    import torch
    import attention_fa_fwd_amd as fa
    import workloads as wl

    fa.lib()
    dev = torch.device("cuda:0")
    log("generating the decode workload")
    dt = torch.float16 if args.dtype == "fp16" else torch.bfloat16
    if args.decode_batch > 0:
        case = wl.make_decode_case(f"decode {args.dtype} B={args.decode_batch} L={args.decode_len} Nq=64 Nkv=8 "
                                   f"D=128 {args.decode_layout}", [args.decode_len] * args.decode_batch,
                                   args.decode_len, num_heads=64, num_kv_heads=8, head_dim=128, dtype=dt,
                                   layout=args.decode_layout, seed=22)
    else:
        case = wl.make_decode_workload(dt, args.decode_layout)
    cfg = fa.DecodeConfig(case.batch, case.max_seq_len, case.num_heads, case.num_kv_heads, case.head_dim,
                          case.dtype, case.scale, case.layout, case.lens)
    q = case.q.to(dev)
    k, v = case.padded_cache("k", dev), case.padded_cache("v", dev)
    out = torch.empty_like(q)
    ws = torch.empty(fa.fa_decode_workspace_size(cfg), dtype=torch.uint8, device=dev)

    def step():
        fa.fa_decode(cfg, q, k, v, out, workspace=ws)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = max(args.steps, 1) * 20          # a decode step is short: time 20 calls per requested step
    log(f"timing {steps} calls")
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    fa.fa_profile_read()
    fa.fa_profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern = {n: (ms, c) for n, (ms, c) in fa.fa_profile_read().items() if c > 0}
    fa.fa_profile_enable(False)
    kv = case.kv_bytes
    io = 2 * case.q.numel() * case.q.element_size()       # q in, out written
    dec_ms = kern["fa_decode"][0] / kern["fa_decode"][1]
    achieved = (kv + io) / (dec_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        ent = json.load(open(TRAFFIC_FILE)).get("decode" + ("_fp16" if args.dtype == "fp16" else ""), {})
        ent = ent.get("fa_decode")
        if ent and ent.get("source_hash") == kernel_source_hash("decode"):
            traffic = ent.get("bytes_per_launch")
    dt_name = "fp16" if args.dtype == "fp16" else "bf16"
    res = {
        "metric": f"decode attention K/V read bandwidth {dt_name} D=128 (valid cache rows / time)",
        "value": round((kv + io) / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic",
        "config": {"workload": case.name, "sequences": case.batch, "cache_len": case.max_seq_len,
                   "keys": int(case.lens.sum()), "heads_q": case.num_heads, "heads_kv": case.num_kv_heads,
                   "head_dim": case.head_dim, "layout": case.layout, "kv_bytes": kv},
        "kernels_ms": {n: round(ms / c, 5) for n, (ms, c) in kern.items()},
        "roofline": {"bound": "hbm", "kernel": "fa_decode", "achieved": round(achieved, 1), "peak": HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_GBS, 4), "traffic": traffic},
        "note": "the pages give API constraints but no throughput figures of their own",
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 decode oracle, bounded sample)")
        res["cpu_baseline"] = decode_cpu_baseline(case)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--atomic-dq", action="store_true", help="time the fp32-atomic dQ variant")
    ap.add_argument("--dtype", choices=("bf16", "fp16", "fp32"), default="bf16",
                    help="element type of workloads 2-5 (fp16 / fp32 draw the same samples in that type; "
                         "decode: bf16 or fp16)")
    ap.add_argument("--pse", choices=("alibi", "full", "compressed"), default="alibi",
                    help="workload 4's bias: generated from the ALiBi slopes, or the same values passed as an "
                         "external pse tensor of the input type, full [1, N, S, S] or 1024-row compressed "
                         "[1, N, 1024, S] (16-bit inputs then run the materialised-score path)")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="head dim of workloads 2-5 instead of 128 (above 128 the materialised-score path runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-cache", action="store_true",
                    help="overwrite a 1 GiB buffer between timed steps (no step finds its inputs in the MALL)")
    ap.add_argument("--variant-steps", type=int, default=3,
                    help="steps timed for the atomic-dQ variant reported beside the deterministic headline "
                         "(0: skip it)")
    ap.add_argument("--layout", choices=("TND", "BSND", "BSH", "BNSD", "SBH"), default="TND",
                    help="input layout of the training path (fixed-length workloads 3 and 4 for the non-TND ones)")
    ap.add_argument("--decode", action="store_true",
                    help="time decode attention (fa_decode) over the decode workload instead")
    ap.add_argument("--decode-layout", choices=("BSND", "BSH", "BNSD"), default="BSND",
                    help="KV cache layout of the decode workload")
    ap.add_argument("--decode-batch", type=int, default=0, metavar="B",
                    help="decode over B sequences of --decode-len keys each instead of the decode workload")
    ap.add_argument("--decode-len", type=int, default=16384)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path is a single-GPU kernel library whose multi-GPU "
              f"sharding is a design, not code (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_fa_fwd_amd as fa
    import workloads as wl

    if args.decode:
        return decode_bench(args)

    fa.lib()   # fail loudly if libfa.so was not built
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calibration}), flush=True)
        return
    # workload 4 is the one with a bias
    if args.pse != "alibi" and (args.workload != 4 or args.layout != "TND"):
        sys.exit("--pse full / compressed: workload 4 in TND only")
    log(f"generating workload {args.workload}")
    case = wl.make_workload(args.workload, {"fp16": torch.float16, "fp32": torch.float32}.get(args.dtype),
                            head_dim=args.head_dim)
    pairs, f_fwd, f_bwd = flops_of(case)
    deterministic = not args.atomic_dq
    pse = None
    if args.pse != "alibi":
        s_len = int(case.lens_q[0])
        pse = alibi_pse(torch.from_numpy(case.alibi_slopes).to(dev), s_len, s_len if args.pse == "full" else 1024)
        pse = pse.to(case.dtype)
    cfg = fa.Config(case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.head_dim,
                    case.dtype, case.scale, case.keep_prob, case.sparse_mode, case.pre_tokens, case.next_tokens,
                    deterministic, layout=args.layout, atomic_dq=args.atomic_dq,
                    **({} if pse is None else dict(pse=pse, pse_type=0)))
    q, k, v, dy = (t.to(dev) for t in (case.q, case.k, case.v, case.dy))
    if args.layout != "TND":
        # the same values in the fixed-length layout (workloads with one common length)
        def lay(x):
            b = case.batch
            x4 = x.reshape(b, x.shape[0] // b, x.shape[1], x.shape[2])
            if args.layout == "BNSD":
                return x4.permute(0, 2, 1, 3).contiguous()
            if args.layout == "SBH":
                return x4.permute(1, 0, 2, 3).reshape(x4.shape[1], b, -1).contiguous()
            return x4 if args.layout == "BSND" else x4.reshape(b, x4.shape[1], -1)
        q, k, v, dy = (lay(t) for t in (q, k, v, dy))
    drop = torch.from_numpy(case.drop_mask).to(dev) if case.drop_mask is not None else None
    slopes = torch.from_numpy(case.alibi_slopes).to(dev) if case.alibi_slopes is not None and pse is None else None
    sink = torch.from_numpy(case.sink).to(dev) if case.sink is not None else None
    out = torch.empty_like(q)
    tq = int(case.cu_seqlens_q[-1])
    m = torch.empty((tq, case.head_num), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsink = torch.empty((case.head_num,), dtype=torch.float32, device=dev) if sink is not None else None
    ws_f = torch.empty(fa.fa_fwd_workspace_size(cfg), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(fa.fa_bwd_workspace_size(cfg), dtype=torch.uint8, device=dev)

    def step():
        fa.fa_fwd(cfg, q, k, v, drop, slopes, sink, out, m, l, workspace=ws_f)
        fa.fa_bwd(cfg, q, k, v, dy, out, m, l, drop, slopes, sink, dq, dk, dv, dsink, workspace=ws_b)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ms_step, wall, step_ms = timed_steps(step, args.steps, stream, args.cold_cache, dev)
    log(f"{ms_step:.3f} ms/step (median {np.median(step_ms):.3f}, min {min(step_ms):.3f}; "
        f"wall {1e3 * wall / args.steps:.3f})")

    # per-kernel durations: HIP events the library records around each launch, over the same
    # number of steps, on the stream each kernel is launched on
    fa.fa_profile_read()
    fa.fa_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = fa.fa_profile_read()
    fa.fa_profile_enable(False)
    kern = {name: (ms, n) for name, (ms, n) in kern.items() if n > 0}
    fwd_ms = kern["fa_fwd"][0] / kern["fa_fwd"][1]
    dom = max(kern, key=lambda n: kern[n][0])
    dom_ms = kern[dom][0] / kern[dom][1]
    d = case.head_dim
    # algorithmic FLOP of each kernel per launch (mask-aware pair count x per-pair work)
    per_pair = {"fa_fwd": 4 * d, "fa_bwd_dkdv": (10 if not deterministic else 8) * d, "fa_bwd_dq": 2 * d}
    if d > 128:
        per_pair["fa_bwd_dkdv"] = 10 * d   # above D = 128 one timed region holds the whole backward
    peak = PEAK_BF16_TFLOPS if case.dtype.is_floating_point and case.q.element_size() == 2 else PEAK_FP32_TFLOPS
    if dom in per_pair:
        achieved = per_pair[dom] * pairs / (dom_ms * 1e-3) / 1e12
        bound, unit, pk = "mfma", "TFLOP/s", peak
    else:
        achieved, bound, unit, pk = None, "hbm", "GB/s", HBM_GBS
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tf = json.load(open(TRAFFIC_FILE))
        key = f"workload{args.workload}" + ("" if args.dtype == "bf16" else "_" + args.dtype)
        key += "" if case.head_dim == 128 else f"_d{case.head_dim}"
        ent = tf.get(key + ("" if args.pse == "alibi" else "_pse_" + args.pse), {}).get(dom)
        # head dims above 128 and a 16-bit external pse run the materialised-score path
        path = "large" if case.head_dim > 128 or (pse is not None and case.dtype != torch.float32) else "training"
        if ent and ent.get("source_hash") == kernel_source_hash(path):
            traffic = ent.get("bytes_per_launch")

    total_flops = f_fwd + f_bwd
    dt_name = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[case.dtype]
    value = total_flops / (ms_step * 1e-3) / 1e12
    res = {
        "metric": f"attention fwd+bwd TFLOP/s (mask-aware) {dt_name} D={d}; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_min": round(float(min(step_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic",
        "config": {"workload": case.name, "total_tokens": int(tq),
                   "sequences": int(case.batch), "heads_q": case.head_num, "heads_kv": case.kv_heads,
                   "head_dim": d, "allowed_pairs": int(pairs),
                   "dq_variant": "deterministic" if deterministic else "atomic", "layout": args.layout,
                   "cache": "cold (1 GiB written between steps)" if args.cold_cache else "warm",
                   **({} if args.pse == "alibi" else {"pse": f"external {args.pse} (the ALiBi bias)"})},
        "frac_of_peak": round(value / peak, 4),
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "kernels_ms": {n: round(ms / c, 4) for n, (ms, c) in kern.items()},
        "roofline": {"bound": bound, "kernel": dom,
                     "achieved": None if achieved is None else round(achieved, 2),
                     "peak": pk, "unit": unit,
                     "frac": None if achieved is None else round(achieved / pk, 4),
                     "traffic": traffic},
        "note": "the pages give API constraints but no throughput figures of their own",
    }
    if deterministic and args.variant_steps > 0:
        # the pages' other backward scheme, timed beside the headline: dQ accumulated with fp32
        # atomics inside the dK/dV pass (where that variant exists; otherwise the library runs
        # the deterministic passes and the record says so)
        acfg = fa.Config(case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.head_dim,
                         case.dtype, case.scale, case.keep_prob, case.sparse_mode, case.pre_tokens,
                         case.next_tokens, False, layout=args.layout, atomic_dq=True,
                         **({} if pse is None else dict(pse=pse, pse_type=0)))
        del ws_b
        ws_a = torch.empty(fa.fa_bwd_workspace_size(acfg), dtype=torch.uint8, device=dev)

        def astep():
            fa.fa_fwd(acfg, q, k, v, drop, slopes, sink, out, m, l, workspace=ws_f)
            fa.fa_bwd(acfg, q, k, v, dy, out, m, l, drop, slopes, sink, dq, dk, dv, dsink, workspace=ws_a)

        log(f"atomic-dQ variant: {args.variant_steps} steps")
        astep()
        a_ms, _, a_per = timed_steps(astep, args.variant_steps, stream, args.cold_cache, dev)
        fa.fa_profile_read()
        fa.fa_profile_enable(True)
        astep()
        torch.cuda.synchronize()
        ak = {n: ms / c for n, (ms, c) in fa.fa_profile_read().items() if c > 0}
        fa.fa_profile_enable(False)
        res["variants"] = {"atomic_dq": {
            "value": round(total_flops / (a_ms * 1e-3) / 1e12, 2), "ms_per_step": round(a_ms, 4),
            "ms_per_step_median": round(float(np.median(a_per)), 4), "steps": args.variant_steps,
            "kernels_ms": {n: round(x, 4) for n, x in ak.items()},
            "ran_atomic_kernel": "fa_bwd_dq_convert" in ak}}
        del ws_a
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle, bounded sample)")
        res["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
