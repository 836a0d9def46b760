"""Tile skipping checked on the device: the trace build of the library
(libfa_trace.so, the same sources with per-tile visit counters; include/fa_trace.h)
counts every tile each pass computes.  The sparse modes fix which (row, key) pairs
are allowed (aclnnFlashAttentionUnpaddingScoreGrad, sparseMode list), so every tile
holding an allowed pair must be computed exactly once and every other tile never:
the counters are compared with a brute-force count over the oracle's mask, and the
host scheduler's work list (fa_debug_schedule) must cover the same tiles."""
import ctypes

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
import workloads as wl
from harness import config_of, device_inputs, say

pytestmark = pytest.mark.gpu

# pass: (rows per block, keys per tile)
GRID = {0: (32, 64), 1: (64, 128), 2: (32, 64)}

CASES = {
    "causal_varlen_gqa": dict(lens_q=[300, 0, 129, 1000, 1], head_num=4, kv_heads=2, sparse_mode=3),
    "causal_rectangular": dict(lens_q=[300, 77, 129], lens_kv=[500, 10, 129], head_num=2, kv_heads=1,
                               sparse_mode=3),
    "left_up_rectangular": dict(lens_q=[90, 200, 513], lens_kv=[300, 65, 513], head_num=2, kv_heads=2,
                                sparse_mode=2),
    "band": dict(lens_q=[600, 129, 1], head_num=2, kv_heads=1, sparse_mode=4, pre_tokens=37, next_tokens=11),
    "band_negative_pre": dict(lens_q=[1000, 257], head_num=2, kv_heads=1, sparse_mode=4, pre_tokens=-20,
                              next_tokens=70),
    "prefix": dict(lens_q=[300, 77, 129, 5], lens_kv=[500, 40, 129, 64], head_num=2, kv_heads=1, sparse_mode=6,
                   prefix=[250, 0, 64, 60]),
    "mode7": dict(lens_q=[300, 77, 513], lens_kv=[500, 77, 700], head_num=2, kv_heads=1, sparse_mode=7,
                  pre_tokens=100, next_tokens=3),
    "mode8_split": dict(lens_q=[150, 300, 64], lens_kv=[400, 300, 64], head_num=2, kv_heads=1, sparse_mode=8,
                        pre_tokens=180, next_tokens=0, q_start_idx=250, kv_start_idx=0),
    "no_mask_cross": dict(lens_q=[333, 64], lens_kv=[129, 500], head_num=2, kv_heads=2, sparse_mode=0),
}


def _expected(case, pass_id):
    """Brute-force visit counts: 1 where the (block, tile) of a (sequence, head) holds an allowed pair."""
    rows, keys = GRID[pass_id]
    lq, lkv = case.lens_q, case.lens_kv
    rb, kt = -(-int(lq.max()) // rows), -(-int(lkv.max()) // keys)
    exp = np.zeros((case.batch, case.head_num, rb, kt), np.uint32)
    for b in range(case.batch):
        if lq[b] == 0 or lkv[b] == 0:
            continue
        mode = oracle.sequence_mode(case.sparse_mode, b, case.batch)
        ok = oracle.allowed(int(lq[b]), int(lkv[b]), mode, case.pre_tokens, case.next_tokens,
                            0 if case.prefix is None else int(case.prefix[b]))
        for r in range(-(-int(lq[b]) // rows)):
            for t in range(-(-int(lkv[b]) // keys)):
                if ok[r * rows:(r + 1) * rows, t * keys:(t + 1) * keys].any():
                    exp[b, :, r, t] = 1
    return exp


def _run_traced(case, det=True):
    """fa_fwd and fa_bwd of the trace build on cuda:0; returns the three passes' counters."""
    TL = fa.trace_lib()
    x = device_inputs(case)
    cfg = config_of(case, det)
    dev = x["q"].device
    counters = {}
    for pass_id, (rows, keys) in GRID.items():
        rb, kt = -(-int(case.lens_q.max()) // rows), -(-int(case.lens_kv.max()) // keys)
        counters[pass_id] = torch.zeros(case.batch * case.head_num * rb * kt, dtype=torch.int32, device=dev)
        assert TL.fa_debug_trace(pass_id, counters[pass_id].data_ptr(), counters[pass_id].numel()) == fa.FA_OK
    tq, nq = int(case.cu_seqlens_q[-1]), case.head_num
    out = torch.empty(fa.layout_shape(cfg, True, True), dtype=case.dtype, device=dev)
    m = torch.empty((tq, nq), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    try:
        ws = torch.empty(max(fa.fa_fwd_workspace_size(cfg), fa.fa_bwd_workspace_size(cfg)), dtype=torch.uint8,
                         device=dev)
        st = TL.fa_fwd(cfg.ref, P(x["q"]), P(x["k"]), P(x["v"]), None, None, None, P(out), P(m), P(l), P(ws),
                       ctypes.c_uint64(ws.numel()), stream)
        assert st == fa.FA_OK, st
        st = TL.fa_bwd(cfg.ref, P(x["q"]), P(x["k"]), P(x["v"]), P(x["dy"]), P(out), P(m), P(l), None, None, None,
                       P(dq), P(dk), P(dv), None, P(ws), ctypes.c_uint64(ws.numel()), stream)
        assert st == fa.FA_OK, st
        torch.cuda.synchronize()
    finally:
        for pass_id in GRID:
            TL.fa_debug_trace(pass_id, None, 0)
    return {k: v.cpu().numpy().astype(np.uint32) for k, v in counters.items()}


@pytest.mark.parametrize("name", list(CASES))
def test_visited_tiles_are_exactly_the_tiles_with_allowed_pairs(name):
    kw = dict(CASES[name])
    lq = kw.pop("lens_q")
    lkv = kw.pop("lens_kv", None)
    case = wl.make_case(name, lq, lkv, head_dim=128, dtype=torch.bfloat16, seed=300, **kw)
    say(f"trace {name}: lens {list(case.lens_q)}/{list(case.lens_kv)} mode {case.sparse_mode}")
    got = _run_traced(case)
    for pass_id in GRID:
        exp = _expected(case, pass_id)
        g = got[pass_id].reshape(exp.shape)
        bad = np.argwhere(g != exp)
        assert bad.size == 0, f"pass {pass_id}: {len(bad)} tiles differ, first (b, h, block, tile) " \
                              f"{bad[:5].tolist()}: counted {[int(g[tuple(i)]) for i in bad[:5]]}"
        # the host work list covers the same tiles (at the scheduler's granularity)
        items, (bm, bn) = fa.fa_debug_schedule(config_of(case, True), pass_id)
        sched = np.zeros((case.batch, -(-int(case.lens_q.max()) // bm) if pass_id != 1 else exp.shape[3],
                          -(-int(case.lens_kv.max()) // bn) if pass_id != 1 else exp.shape[2]), bool)
        for b, tile, lo, hi in items.tolist():
            for o in range(lo, hi):
                if pass_id == 1:
                    sched[b, tile, o] = True           # key tile, query tiles [lo, hi)
                else:
                    sched[b, tile, o] = True           # query tile, key tiles [lo, hi)
        # every visited block lies inside a scheduled item, and every scheduled item is visited
        rows, keys = GRID[pass_id]
        visited = exp[:, 0] > 0
        if pass_id == 1:
            assert np.array_equal(sched.transpose(0, 2, 1), visited), f"pass 1 schedule"
        else:
            ratio = bm // rows
            merged = visited.reshape(case.batch, -1, ratio, visited.shape[2])[:, :sched.shape[1]].any(axis=2) \
                if visited.shape[1] % ratio == 0 else None
            if merged is None:
                pad = ratio - visited.shape[1] % ratio
                v = np.concatenate([visited, np.zeros((case.batch, pad, visited.shape[2]), bool)], axis=1)
                merged = v.reshape(case.batch, -1, ratio, v.shape[2]).any(axis=2)
            assert np.array_equal(sched, merged[:, :sched.shape[1]]), f"pass {pass_id} schedule"
