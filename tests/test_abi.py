"""CPU-only checks of the C ABI: exported symbols, argument validation (every
rejected call returns before any device work), and the tile scheduler's
work lists against brute-force enumeration of the oracle's mask."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
import workloads as wl
from attention_fa_fwd_amd._lib import FaConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:fa_status|const char\*|int32_t)\s+(fa_\w+)\s*\(", text, re.M))
    assert declared == set(fa.EXPORTED), declared ^ set(fa.EXPORTED)
    L = fa.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    for code in (fa.FA_OK, fa.FA_ERR_PARAM_NULLPTR, fa.FA_ERR_PARAM_INVALID, fa.FA_ERR_WORKSPACE, fa.FA_ERR_HIP):
        assert fa.status_string(code).startswith("FA_")
    assert fa.FA_ERR_PARAM_NULLPTR == 161001 and fa.FA_ERR_PARAM_INVALID == 161002


def _cfg(**over):
    base = dict(cu_seqlens_q=[0, 5, 12], cu_seqlens_kv=[0, 5, 12], head_num=4, kv_heads=2, head_dim=128,
                dtype=fa.FA_DTYPE_BF16, scale=0.1, keep_prob=1.0, sparse_mode=3, pre_tokens=fa.TOKENS_DEFAULT,
                next_tokens=fa.TOKENS_DEFAULT, deterministic=True)
    base.update(over)
    return fa.Config(**base)


FAKE = ctypes.c_void_p(0x10000)   # aligned, never dereferenced: every call below fails validation first


def _fwd(cfg, **ptr):
    p = dict(q=FAKE, k=FAKE, v=FAKE, drop=None, slopes=None, sink=None, out=FAKE, m=FAKE, l=FAKE, ws=FAKE,
             ws_bytes=1 << 40)
    p.update(ptr)
    c = None if cfg is None else cfg.ref
    return fa.lib().fa_fwd(c, p["q"], p["k"], p["v"], p["drop"], p["slopes"], p["sink"], p["out"], p["m"],
                           p["l"], p["ws"], ctypes.c_uint64(p["ws_bytes"]), None)


def _bwd(cfg, **ptr):
    p = dict(q=FAKE, k=FAKE, v=FAKE, dy=FAKE, out=FAKE, m=FAKE, l=FAKE, drop=None, slopes=None, sink=None,
             dq=FAKE, dk=FAKE, dv=FAKE, dsink=None, ws=FAKE, ws_bytes=1 << 40)
    p.update(ptr)
    return fa.lib().fa_bwd(cfg.ref, p["q"], p["k"], p["v"], p["dy"], p["out"], p["m"], p["l"], p["drop"],
                           p["slopes"], p["sink"], p["dq"], p["dk"], p["dv"], p["dsink"], p["ws"],
                           ctypes.c_uint64(p["ws_bytes"]), None)


INVALID_CONFIGS = {
    "head_dim_100": dict(head_dim=100),      # bf16 rows of 200 bytes: not whole 16-byte chunks
    "head_dim_520": dict(head_dim=520),     # above the grad page's D limit of 512
    "head_dim_260": dict(head_dim=260),     # bf16 rows of 520 bytes
    "gqa_not_divisible": dict(head_num=4, kv_heads=3),
    "too_many_heads": dict(head_num=512, kv_heads=512),
    "keep_zero": dict(keep_prob=0.0),
    "keep_above_one": dict(keep_prob=1.5),
    "mode_5": dict(sparse_mode=5),
    "mode_9": dict(sparse_mode=9),
    "mode_7_band_without_intersection": dict(sparse_mode=7, pre_tokens=-3, next_tokens=2),
    # start indices: mode 8 only, non-negative, and Lq_0 - Lkv_0 + qStartIdx - kvStartIdx == 0
    "start_idx_outside_mode_8": dict(sparse_mode=4, q_start_idx=3, kv_start_idx=3),
    "start_idx_off_constraint": dict(sparse_mode=8, q_start_idx=3, kv_start_idx=0),
    "start_idx_negative": dict(sparse_mode=8, q_start_idx=-2, kv_start_idx=-2),
    "band_without_intersection": dict(sparse_mode=4, pre_tokens=-3, next_tokens=2),
    "cu_not_monotone": dict(cu_seqlens_q=[0, 7, 5], cu_seqlens_kv=[0, 7, 5]),
    "cu_not_starting_at_zero": dict(cu_seqlens_q=[1, 5, 12]),
    "too_many_tokens": dict(cu_seqlens_q=[0, 1 << 20, (1 << 20) + 1], cu_seqlens_kv=[0, 5, 12]),
    "empty_batch": dict(cu_seqlens_q=[0, 0, 0], cu_seqlens_kv=[0, 0, 0]),
    "bad_dtype": dict(dtype=7),
    "non_finite_scale": dict(scale=float("inf")),
}


@pytest.mark.parametrize("name", list(INVALID_CONFIGS))
def test_invalid_configs_rejected(name):
    cfg = _cfg(**INVALID_CONFIGS[name])
    assert _fwd(cfg) == fa.FA_ERR_PARAM_INVALID
    assert _bwd(cfg) == fa.FA_ERR_PARAM_INVALID
    n = ctypes.c_uint64(0)
    assert fa.lib().fa_fwd_workspace_size(cfg.ref, ctypes.byref(n)) == fa.FA_ERR_PARAM_INVALID


def test_element_types_accepted():
    # FLOAT32, BFLOAT16 and FLOAT16 inputs (aclnnFlashAttentionUnpaddingScoreGrad, parameter table)
    n = ctypes.c_uint64(0)
    for dt in (fa.FA_DTYPE_FP32, fa.FA_DTYPE_BF16, fa.FA_DTYPE_FP16):
        for d in (64, 128):
            assert fa.lib().fa_bwd_workspace_size(_cfg(dtype=dt, head_dim=d).ref, ctypes.byref(n)) == fa.FA_OK
            assert n.value > 0
    for dt in (-1, 3):
        assert fa.lib().fa_fwd_workspace_size(_cfg(dtype=dt).ref, ctypes.byref(n)) == fa.FA_ERR_PARAM_INVALID
    assert fa.Config([0, 4], [0, 4], 2, 2, 64, torch.float16, 0.125).c.dtype == fa.FA_DTYPE_FP16


def test_bad_flags_and_batch_limits():
    for bad in (8, 1 << 30, -1):
        cfg = _cfg()
        cfg.c.flags = bad
        assert _fwd(cfg) == fa.FA_ERR_PARAM_INVALID, bad
    n = ctypes.c_uint64(0)
    for good in (fa.FA_FLAG_PSE_SQRT, fa.FA_FLAG_SLOPES_PER_BATCH, fa.FA_FLAG_PSE_SQRT | fa.FA_FLAG_SLOPES_PER_BATCH):
        cfg = _cfg()
        cfg.c.flags = good
        assert fa.lib().fa_fwd_workspace_size(cfg.ref, ctypes.byref(n)) == fa.FA_OK, good
    assert _cfg(pse_type=3, slopes_per_batch=True).c.flags == fa.FA_FLAG_PSE_SQRT | fa.FA_FLAG_SLOPES_PER_BATCH
    with pytest.raises(ValueError):
        _cfg(pse_type=1)
    cfg = _cfg()
    cfg.c.deterministic = 2
    assert _bwd(cfg) == fa.FA_ERR_PARAM_INVALID
    cu = np.zeros(20002, np.int64)
    cu[1:] = np.arange(1, 20002)
    assert _fwd(_cfg(cu_seqlens_q=cu, cu_seqlens_kv=cu)) == fa.FA_ERR_PARAM_INVALID


def test_null_pointers():
    assert _fwd(None) == fa.FA_ERR_PARAM_NULLPTR
    cfg = _cfg()
    cfg.c.cu_seqlens_q = None
    assert _fwd(cfg) == fa.FA_ERR_PARAM_NULLPTR
    for key in ("q", "k", "v", "out", "m", "l", "ws"):
        assert _fwd(_cfg(), **{key: None}) == fa.FA_ERR_PARAM_NULLPTR, key
    for key in ("q", "k", "v", "dy", "out", "m", "l", "dq", "dk", "dv", "ws"):
        assert _bwd(_cfg(), **{key: None}) == fa.FA_ERR_PARAM_NULLPTR, key
    # keep_prob < 1 needs the keep mask; a sink needs a dSink output
    assert _fwd(_cfg(keep_prob=0.9)) == fa.FA_ERR_PARAM_NULLPTR
    assert _bwd(_cfg(), sink=FAKE) == fa.FA_ERR_PARAM_NULLPTR
    n = ctypes.c_uint64(0)
    assert fa.lib().fa_fwd_workspace_size(_cfg().ref, None) == fa.FA_ERR_PARAM_NULLPTR
    assert fa.lib().fa_fwd_workspace_size(_cfg().ref, ctypes.byref(n)) == fa.FA_OK and n.value > 0


def test_prefix_mode_validation():
    # sparse mode 6 needs prefixOptional, one N per sequence
    assert _fwd(_cfg(sparse_mode=6)) == fa.FA_ERR_PARAM_NULLPTR
    assert _bwd(_cfg(sparse_mode=6)) == fa.FA_ERR_PARAM_NULLPTR
    n = ctypes.c_uint64(0)

    def size(cfg):
        return fa.lib().fa_fwd_workspace_size(cfg.ref, ctypes.byref(n))

    # N range ("Constraints"): [Lkv - Lq, Lkv] when Lq <= Lkv, [0, Lkv] when Lq > Lkv
    cq, ck = [0, 5, 12], [0, 8, 12]        # (Lq, Lkv) = (5, 8) and (7, 4)
    for good in ([3, 0], [8, 4], [5, 2]):
        assert size(_cfg(sparse_mode=6, cu_seqlens_q=cq, cu_seqlens_kv=ck, prefix=good)) == fa.FA_OK, good
    for bad in ([2, 0], [9, 0], [3, 5], [3, -1]):
        cfg = _cfg(sparse_mode=6, cu_seqlens_q=cq, cu_seqlens_kv=ck, prefix=bad)
        assert size(cfg) == fa.FA_ERR_PARAM_INVALID, bad
        assert _fwd(cfg) == fa.FA_ERR_PARAM_INVALID and _bwd(cfg) == fa.FA_ERR_PARAM_INVALID
    # at most 1024 sequences with a prefix; the prefix is ignored by the other modes
    cu = np.arange(1026, dtype=np.int64)
    assert size(_cfg(sparse_mode=6, cu_seqlens_q=cu[:1025], cu_seqlens_kv=cu[:1025], prefix=np.ones(1024))) == fa.FA_OK
    assert size(_cfg(sparse_mode=6, cu_seqlens_q=cu, cu_seqlens_kv=cu, prefix=np.ones(1025))) == fa.FA_ERR_PARAM_INVALID
    assert size(_cfg(sparse_mode=3, prefix=[100, 100])) == fa.FA_OK


def test_atten_mask_validation():
    n = ctypes.c_uint64(0)

    def size(cfg):
        return fa.lib().fa_fwd_workspace_size(cfg.ref, ctypes.byref(n))

    # mode 1 (allMask) needs the mask
    assert _fwd(_cfg(sparse_mode=1)) == fa.FA_ERR_PARAM_NULLPTR
    assert _bwd(_cfg(sparse_mode=1)) == fa.FA_ERR_PARAM_NULLPTR

    def masked(mode, rows, cols):
        cfg = _cfg(sparse_mode=mode)
        cfg.c.atten_mask = 0x20000          # never dereferenced by the size query
        cfg.c.mask_rows, cfg.c.mask_cols = rows, cols
        return cfg

    # [S1Max, S2Max] must cover every sequence (lengths 5 and 7 here)
    base = fa.fa_fwd_workspace_size(_cfg(sparse_mode=0))
    for mode in (0, 1, 4):
        assert size(masked(mode, 7, 7)) == fa.FA_OK and n.value >= base + 7 * 4, mode
        assert size(masked(mode, 6, 7)) == fa.FA_ERR_PARAM_INVALID
        assert size(masked(mode, 7, 6)) == fa.FA_ERR_PARAM_INVALID
    # modes with their own triangle take no mask workspace
    assert size(masked(3, 2, 2)) == fa.FA_OK and n.value == fa.fa_fwd_workspace_size(_cfg(sparse_mode=3))


def test_alignment_alibi_and_workspace_rules():
    odd = ctypes.c_void_p(0x10008)
    assert _fwd(_cfg(), q=odd) == fa.FA_ERR_PARAM_INVALID
    # the workspace is 16-byte aligned too (the plan and the TND copies are stored in 16-byte pieces)
    assert _fwd(_cfg(), ws=odd) == fa.FA_ERR_PARAM_INVALID
    assert _bwd(_cfg(), ws=odd) == fa.FA_ERR_PARAM_INVALID
    assert _fwd(_cfg(keep_prob=0.5), drop=ctypes.c_void_p(0x10002)) == fa.FA_ERR_PARAM_INVALID
    # ALiBi (pseType 2) needs Lq == Lkv per sequence and no empty sequence
    assert _fwd(_cfg(cu_seqlens_kv=[0, 6, 12]), slopes=FAKE) == fa.FA_ERR_PARAM_INVALID
    assert _fwd(_cfg(cu_seqlens_q=[0, 0, 12], cu_seqlens_kv=[0, 0, 12]), slopes=FAKE) == fa.FA_ERR_PARAM_INVALID
    assert _fwd(_cfg(), ws_bytes=16) == fa.FA_ERR_WORKSPACE
    assert _bwd(_cfg(), ws_bytes=16) == fa.FA_ERR_WORKSPACE
    # the fp32-atomic dQ scheme needs its accumulator on top of the deterministic workspace
    assert _bwd(_cfg(deterministic=False, atomic_dq=True),
                ws_bytes=fa.fa_bwd_workspace_size(_cfg())) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_workspace_size(_cfg(deterministic=False)) == fa.fa_bwd_workspace_size(_cfg())


def test_atomic_variant_needs_a_larger_workspace():
    det = fa.fa_bwd_workspace_size(_cfg(deterministic=True))
    atom = fa.fa_bwd_workspace_size(_cfg(deterministic=False, atomic_dq=True))
    assert atom >= det + 4 * 12 * 4 * 128


# --------------------------------------------------------------------------- scheduler

def _brute_ranges(lq, lkv, mode, pre, nxt, bm, bn, by_kv, prefix=0):
    ok = oracle.allowed(lq, lkv, mode, pre, nxt, prefix)   # one sequence's own mode
    res = []
    if by_kv:
        for t in range((lkv + bn - 1) // bn):
            cols = ok[:, t * bn:(t + 1) * bn].any(axis=1)
            tiles = sorted({i // bm for i in np.nonzero(cols)[0]})
            res.append((t, tiles))
    else:
        for t in range((lq + bm - 1) // bm):
            rows = ok[t * bm:(t + 1) * bm, :].any(axis=0)
            tiles = sorted({j // bn for j in np.nonzero(rows)[0]})
            res.append((t, tiles))
    return res


SCHED_CASES = [
    ([300, 0, 129, 1000], [300, 0, 129, 1000], 3, 0, 0),
    ([300, 77, 129], [500, 10, 129], 3, 0, 0),
    ([90, 200, 513], [300, 65, 513], 2, 0, 0),
    ([600, 129, 1], None, 4, 37, 11),
    ([1000, 257], None, 4, -20, 70),
    ([1000, 257], [700, 300], 4, 100, 0),
    ([333, 64], [129, 500], 0, 0, 0),
    ([2048, 2048], None, 4, 2048, 0),
    # prefix (mode 6) with the N of each sequence last
    ([300, 77, 129, 1000, 5], [500, 10, 129, 1000, 64], 6, 0, 0, [200, 0, 64, 0, 60]),
    ([513, 600, 64], [513, 600, 2000], 6, 0, 0, [513, 300, 1999]),
    ([700, 129], [129, 700], 6, 0, 0, [129, 650]),
    # modes 7 / 8: the band on the last / first sequence, a causal triangle on the others
    ([300, 77, 129, 513], [500, 77, 200, 700], 7, 100, 3),
    ([513, 300, 64], [700, 300, 64], 8, 128, 0),
    ([1000, 257, 5], [1000, 257, 5], 8, -20, 70),
]


@pytest.mark.parametrize("case", SCHED_CASES)
@pytest.mark.parametrize("pass_id", [0, 1, 2])
def test_schedule_matches_brute_force(case, pass_id):
    lq, lkv, mode, pre, nxt = case[:5]
    prefix = case[5] if len(case) > 5 else [0] * len(lq)
    lkv = lq if lkv is None else lkv
    cfg = _cfg(cu_seqlens_q=wl.cu_from_lengths(lq), cu_seqlens_kv=wl.cu_from_lengths(lkv), sparse_mode=mode,
               pre_tokens=pre, next_tokens=nxt, prefix=prefix if mode == 6 else None)
    items, (bm, bn) = fa.fa_debug_schedule(cfg, pass_id)
    costs = items[:, 3] - items[:, 2]
    # items of one sequence are consecutive; sequences heaviest first, and
    # inside a sequence items heaviest first
    seqs = [int(b) for i, b in enumerate(items[:, 0]) if i == 0 or b != items[i - 1, 0]]
    assert len(seqs) == len(set(seqs)), "items of a sequence must be consecutive"
    seq_cost = [int(costs[items[:, 0] == b].sum()) for b in seqs]
    assert all(x >= y for x, y in zip(seq_cost, seq_cost[1:])), "sequences heaviest first"
    for b in seqs:
        c = costs[items[:, 0] == b]
        assert np.all(np.diff(c) <= 0), "items of a sequence heaviest first"
    seen = {}
    for b, tile, lo, hi in items.tolist():
        seen[(b, tile)] = (lo, hi)
    expect_keys = set()
    for b in range(len(lq)):
        for t, tiles in _brute_ranges(lq[b], lkv[b], oracle.sequence_mode(mode, b, len(lq)), pre, nxt, bm, bn,
                                      by_kv=(pass_id == 1), prefix=prefix[b]):
            expect_keys.add((b, t))
            lo, hi = seen[(b, t)]
            got = list(range(lo, hi))
            assert got == tiles, (b, t, got, tiles)
    assert set(seen) == expect_keys and len(items) == len(expect_keys)


def test_schedule_of_workload5_skips_upper_triangle():
    lens = wl.workload_lengths(5)
    cfg = _cfg(cu_seqlens_q=wl.cu_from_lengths(lens), cu_seqlens_kv=wl.cu_from_lengths(lens), head_num=64,
               kv_heads=8)
    items, (bm, bn) = fa.fa_debug_schedule(cfg, 0)
    visited = int((items[:, 3] - items[:, 2]).sum())
    dense = int(sum(((L + bm - 1) // bm) * ((L + bn - 1) // bn) for L in lens))
    # a causal mask keeps a little over half of the tiles
    assert 0.45 * dense < visited < 0.56 * dense


def test_build_rejects_spilling_kernels_with_lds_dma(tmp_path):
    from attention_fa_fwd_amd.build import check_no_spill_with_dma
    body = "_Zk1: ; @_Zk1\n  global_load_lds_dword v[0:1], off\n  s_endpgm\n_Zk2: ; @_Zk2\n  v_mov_b32 v0, 0\n  s_endpgm\n"
    meta = ("amdhsa.kernels:\n  - .agpr_count: 0\n    .name: _Zk1\n    .private_segment_fixed_size: {a}\n"
            "  - .agpr_count: 0\n    .name: _Zk2\n    .private_segment_fixed_size: {b}\n")
    ok = tmp_path / "ok.s"
    ok.write_text(body + meta.format(a=0, b=7))       # spills only where no DMA is issued
    check_no_spill_with_dma(str(ok))
    bad = tmp_path / "bad.s"
    bad.write_text(body + meta.format(a=3, b=0))
    with pytest.raises(RuntimeError, match="_Zk1"):
        check_no_spill_with_dma(str(bad))


def _dcfg(**over):
    base = dict(batch=3, max_seq_len=100, num_heads=8, num_kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                scale=0.1, layout="BSND", actual_seq_lengths=[100, 0, 37])
    base.update(over)
    return fa.DecodeConfig(**base)


def _dec(cfg, **ptr):
    p = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40)
    p.update(ptr)
    return fa.lib().fa_decode(None if cfg is None else cfg.ref, p["q"], p["k"], p["v"], p["out"], p["ws"],
                              ctypes.c_uint64(p["ws_bytes"]), None)


DECODE_INVALID = {
    "fp32": dict(dtype=torch.float32),
    "head_dim_96": dict(head_dim=96),
    "group_over_64": dict(num_heads=130, num_kv_heads=2),
    "gqa_not_divisible": dict(num_heads=8, num_kv_heads=3),
    "too_many_heads": dict(num_heads=512, num_kv_heads=512),
    "bad_layout": dict(layout="SBH"),
    "length_beyond_cache": dict(actual_seq_lengths=[101, 0, 1]),
    "negative_length": dict(actual_seq_lengths=[-1, 0, 1]),
    "zero_cache": dict(max_seq_len=0, actual_seq_lengths=None),
    "batch_over_limit": dict(batch=65537, actual_seq_lengths=None),
    "scale_nan": dict(scale=float("nan")),
}


@pytest.mark.parametrize("name", list(DECODE_INVALID))
def test_decode_invalid_configs_rejected(name):
    cfg = _dcfg(**DECODE_INVALID[name])
    n = ctypes.c_uint64(0)
    assert fa.lib().fa_decode_workspace_size(cfg.ref, ctypes.byref(n)) == fa.FA_ERR_PARAM_INVALID
    assert _dec(cfg) == fa.FA_ERR_PARAM_INVALID


def test_decode_validation_and_workspace():
    n = ctypes.c_uint64(0)
    assert fa.lib().fa_decode_workspace_size(None, ctypes.byref(n)) == fa.FA_ERR_PARAM_NULLPTR
    assert fa.lib().fa_decode_workspace_size(_dcfg().ref, None) == fa.FA_ERR_PARAM_NULLPTR
    for key in ("q", "k", "v", "out", "ws"):
        assert _dec(_dcfg(), **{key: None}) == fa.FA_ERR_PARAM_NULLPTR, key
    assert _dec(_dcfg(), q=ctypes.c_void_p(0x10008)) == fa.FA_ERR_PARAM_INVALID   # 8-byte aligned only
    assert _dec(_dcfg(), ws=ctypes.c_void_p(0x10008)) == fa.FA_ERR_PARAM_INVALID
    cfg = _dcfg()
    cfg.c.flags = 1
    assert _dec(cfg) == fa.FA_ERR_PARAM_INVALID
    assert fa.lib().fa_decode_workspace_size(_dcfg().ref, ctypes.byref(n)) == fa.FA_OK
    assert _dec(_dcfg(), ws_bytes=n.value - 1) == fa.FA_ERR_WORKSPACE
    # the workspace grows with the split: one long sequence over many heads needs partials
    small = ctypes.c_uint64(0)
    big = ctypes.c_uint64(0)
    assert fa.lib().fa_decode_workspace_size(_dcfg(actual_seq_lengths=[1, 1, 1]).ref, ctypes.byref(small)) == 0
    cfg = _dcfg(batch=1, max_seq_len=1 << 20, actual_seq_lengths=[1 << 20])
    assert fa.lib().fa_decode_workspace_size(cfg.ref, ctypes.byref(big)) == 0
    assert big.value > small.value >= 256
    # every layout and both 16-bit types are accepted; MQA with 64 query heads too
    for layout in ("BSH", "BSND", "BNSD"):
        for dt in (torch.bfloat16, torch.float16):
            assert fa.lib().fa_decode_workspace_size(_dcfg(layout=layout, dtype=dt).ref, ctypes.byref(n)) == 0
    assert fa.lib().fa_decode_workspace_size(_dcfg(num_heads=64, num_kv_heads=1).ref, ctypes.byref(n)) == 0


def test_layout_validation():
    n = ctypes.c_uint64(0)
    uniform = dict(cu_seqlens_q=[0, 6, 12], cu_seqlens_kv=[0, 9, 18])
    sizes = {}
    for layout in ("TND", "BSND", "BSH", "BNSD", "SBH"):
        cfg = _cfg(layout=layout, **uniform)
        assert fa.lib().fa_bwd_workspace_size(cfg.ref, ctypes.byref(n)) == fa.FA_OK, layout
        sizes[layout] = n.value
    # BSH / BSND are TND in memory; BNSD / SBH add TND copies of the eight tensors
    assert sizes["BSND"] == sizes["BSH"] == sizes["TND"]
    assert sizes["BNSD"] == sizes["SBH"] > sizes["TND"]
    # the fixed-length layouts need one common length per side
    for layout in ("BSND", "BNSD", "SBH"):
        assert _fwd(_cfg(layout=layout)) == fa.FA_ERR_PARAM_INVALID   # lengths 5 and 7
    cfg = _cfg(**uniform)
    cfg.c.layout = 5
    assert _fwd(cfg) == fa.FA_ERR_PARAM_INVALID
    assert fa.layout_shape(_cfg(layout="SBH", **uniform), True) == (6, 2, 4 * 128)
    assert fa.layout_shape(_cfg(layout="BNSD", **uniform), False) == (2, 2, 9, 128)


def test_external_pse_validation():
    import torch as _t
    n = ctypes.c_uint64(0)

    def cfg(**pse_over):
        c = _cfg(cu_seqlens_q=[0, 6, 12], cu_seqlens_kv=[0, 6, 12], dtype=fa.FA_DTYPE_FP32)
        c.c.pse = 0x10000
        c.c.pse_batch, c.c.pse_rows, c.c.pse_cols, c.c.pse_type = 2, 6, 6, 1
        for key, val in pse_over.items():
            setattr(c.c, key, val)
        return c

    def size(c):
        return fa.lib().fa_fwd_workspace_size(c.ref, ctypes.byref(n))

    assert size(cfg()) == fa.FA_OK
    for good in (dict(pse_batch=1), dict(pse_rows=1), dict(pse_rows=1024), dict(pse_type=0), dict(pse_cols=9)):
        assert size(cfg(**good)) == fa.FA_OK, good
    for bad in (dict(pse_type=2), dict(pse_batch=3), dict(pse_rows=5), dict(pse_cols=5), dict(pse_rows=0)):
        assert size(cfg(**bad)) == fa.FA_ERR_PARAM_INVALID, bad
    # the 1024-row compression needs a lower-triangle mode and square sequences
    c = cfg(pse_rows=1024)
    c.c.sparse_mode = 0
    c.c.cu_seqlens_q = (ctypes.c_int64 * 3)(0, 1100, 1101)
    c.c.cu_seqlens_kv = (ctypes.c_int64 * 3)(0, 1100, 1101)
    c.c.pse_cols = 1100
    assert size(c) == fa.FA_ERR_PARAM_INVALID
    c.c.sparse_mode = 3
    assert size(c) == fa.FA_OK
    c.c.cu_seqlens_kv = (ctypes.c_int64 * 3)(0, 1100, 1102)
    assert size(c) == fa.FA_ERR_PARAM_INVALID
    # not with alibi slopes, not with an attenMask
    assert _fwd(cfg(), slopes=FAKE) == fa.FA_ERR_PARAM_INVALID
    c = cfg()
    c.c.sparse_mode, c.c.atten_mask, c.c.mask_rows, c.c.mask_cols = 1, 0x20000, 6, 6
    assert size(c) == fa.FA_ERR_PARAM_INVALID
    with pytest.raises(ValueError):
        _cfg(pse=_t.zeros(1, 4, 1, 7), pse_type=2)
    # 16-bit inputs with an external pse run the materialised-score path: accepted, and the
    # workspace then holds a chunk of fp32 scores and 16-bit probabilities for every head
    assert size(cfg()) == fa.FA_OK
    fp32_bytes = n.value
    for dt in (fa.FA_DTYPE_BF16, fa.FA_DTYPE_FP16):
        assert size(cfg(dtype=dt)) == fa.FA_OK
        c = cfg(dtype=dt)
        heads, ld = c.c.head_num, 8   # 6 keys, rows of 16 bytes
        assert n.value >= fp32_bytes + heads * 64 * ld * (4 + 2)


def test_strides_validation():
    n = ctypes.c_uint64(0)
    uniform = dict(cu_seqlens_q=[0, 6, 12], cu_seqlens_kv=[0, 9, 18])

    def with_strides(vals, **over):
        c = _cfg(**{**uniform, **over})
        c._arr = (ctypes.c_int64 * 16)(*vals)
        c.c.strides = ctypes.cast(c._arr, ctypes.POINTER(ctypes.c_int64))
        return c

    packed = [4 * 128, 128, 2 * 128, 128, 2 * 128, 128, 4 * 128, 128, 4 * 128, 128, 4 * 128, 128,
              2 * 128, 128, 2 * 128, 128]
    base = ctypes.c_uint64(0)
    assert fa.lib().fa_bwd_workspace_size(_cfg(**uniform).ref, ctypes.byref(base)) == 0
    assert fa.lib().fa_bwd_workspace_size(with_strides(packed).ref, ctypes.byref(n)) == 0
    assert n.value == base.value          # packed strides need no copies
    wide = list(packed)
    wide[0] = 4 * 136                     # q rows padded to 136 elements
    assert fa.lib().fa_bwd_workspace_size(with_strides(wide).ref, ctypes.byref(n)) == 0
    assert n.value > base.value
    for bad_index, bad in ((0, 4 * 128 + 4), (1, 3), (10, 0), (2, -128)):
        vals = list(packed)
        vals[bad_index] = bad              # misaligned, output token stride 0, negative
        assert _fwd(with_strides(vals)) == fa.FA_ERR_PARAM_INVALID, (bad_index, bad)
    assert _fwd(with_strides(packed, layout="BSND")) == fa.FA_ERR_PARAM_INVALID


def test_padded_head_dims_accepted():
    # D <= 128 with 16-byte rows: 64 and 128 run natively, the others through zero-padded copies
    n = ctypes.c_uint64(0)
    sizes = {}
    for d in (8, 32, 64, 80, 96, 120, 128):
        assert fa.lib().fa_bwd_workspace_size(_cfg(head_dim=d).ref, ctypes.byref(n)) == fa.FA_OK, d
        sizes[d] = n.value
    assert sizes[96] > sizes[128] and sizes[32] > sizes[64]   # the padded copies live in the workspace
    for d, dt in ((36, fa.FA_DTYPE_FP32), (12, fa.FA_DTYPE_FP32)):
        assert fa.lib().fa_fwd_workspace_size(_cfg(head_dim=d, dtype=dt).ref, ctypes.byref(n)) == fa.FA_OK, d
    for d, dt in ((36, fa.FA_DTYPE_BF16), (6, fa.FA_DTYPE_FP32), (0, fa.FA_DTYPE_BF16)):
        assert fa.lib().fa_fwd_workspace_size(_cfg(head_dim=d, dtype=dt).ref, ctypes.byref(n)) == fa.FA_ERR_PARAM_INVALID, d


def test_large_head_dims_accepted():
    # D in (128, 512] with 16-byte rows runs the materialised-score path: its workspace holds one
    # chunk of scores per call and grows with the head dim only through the dK / dV accumulators
    n = ctypes.c_uint64(0)
    sizes = {}
    for d in (136, 192, 256, 512):
        for dt in (fa.FA_DTYPE_BF16, fa.FA_DTYPE_FP16, fa.FA_DTYPE_FP32):
            assert fa.lib().fa_bwd_workspace_size(_cfg(head_dim=d, dtype=dt).ref, ctypes.byref(n)) == fa.FA_OK, (d, dt)
            assert fa.lib().fa_fwd_workspace_size(_cfg(head_dim=d, dtype=dt).ref, ctypes.byref(n)) == fa.FA_OK, (d, dt)
        assert fa.lib().fa_bwd_workspace_size(_cfg(head_dim=d).ref, ctypes.byref(n)) == fa.FA_OK
        sizes[d] = n.value
    assert sizes[512] > sizes[256] > sizes[192]
    # a narrower value head dim is accepted above 128 too (qD == kD >= vD)
    assert fa.lib().fa_bwd_workspace_size(_cfg(head_dim=256, v_head_dim=128).ref, ctypes.byref(n)) == fa.FA_OK
    assert fa.lib().fa_bwd_workspace_size(_cfg(head_dim=256, v_head_dim=264).ref, ctypes.byref(n)) == \
        fa.FA_ERR_PARAM_INVALID


def test_modes_7_8_pse_rules():
    # mode 7 takes no pse at all, mode 8 no pse tensor (the grad pages' sparse_mode=7/8 notes);
    # mode 8's slopes need equal lengths except on a first sequence placed by start indices
    cq, ck = [0, 5, 12], [0, 9, 16]
    assert _fwd(_cfg(sparse_mode=7), slopes=FAKE) == fa.FA_ERR_PARAM_INVALID
    assert _bwd(_cfg(sparse_mode=7), slopes=FAKE) == fa.FA_ERR_PARAM_INVALID
    assert _fwd(_cfg(sparse_mode=8, cu_seqlens_q=cq, cu_seqlens_kv=ck), slopes=FAKE) == fa.FA_ERR_PARAM_INVALID
    ok = _cfg(sparse_mode=8, cu_seqlens_q=cq, cu_seqlens_kv=ck, q_start_idx=4, kv_start_idx=0)
    n = ctypes.c_uint64(0)
    assert fa.lib().fa_fwd_workspace_size(ok.ref, ctypes.byref(n)) == fa.FA_OK
    # ... but only the first sequence: a later one with Lq != Lkv still fails
    bad = _cfg(sparse_mode=8, cu_seqlens_q=[0, 5, 12], cu_seqlens_kv=[0, 9, 17], q_start_idx=4, kv_start_idx=0)
    assert _fwd(bad, slopes=FAKE) == fa.FA_ERR_PARAM_INVALID
    pse = torch.zeros((1, 4, 7, 7))
    for mode in (7, 8):
        cfg = _cfg(sparse_mode=mode, dtype=fa.FA_DTYPE_FP32, pse=pse, pse_type=0)
        assert fa.lib().fa_fwd_workspace_size(cfg.ref, ctypes.byref(n)) == fa.FA_ERR_PARAM_INVALID


def test_trace_build_exports_its_debug_call_only():
    # include/fa_trace.h declares the visit-counter hook of the trace build (libfa_trace.so);
    # the product library does not have it
    text = open(os.path.join(ROOT, "include", "fa_trace.h")).read()
    declared = set(re.findall(r"^\s*fa_status\s+(fa_\w+)\s*\(", text, re.M))
    assert declared == {"fa_debug_trace"}
    TL = fa.trace_lib()
    assert hasattr(TL, "fa_debug_trace") and not hasattr(fa.lib(), "fa_debug_trace")
    for name in fa.EXPORTED:
        assert hasattr(TL, name), name
    assert TL.fa_debug_trace(3, None, 0) == fa.FA_ERR_PARAM_INVALID
    assert TL.fa_debug_trace(0, None, 0) == fa.FA_OK
