"""Pins for the fp64 oracle against things other than itself: the worked example
on the pages (closed form), closed forms for Q = 0, torch's SDPA library
routine, an independently written autograd expression, finite differences and
structural identities (GQA, varlen, mode equivalences)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _cu(lens):
    return wl.cu_from_lengths(lens)


# --------------------------------------------------------------------------- worked example

def test_page_example_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "p4_example_closed_form.json")))
    inp, exp = g["inputs"], g["expected"]
    s, n, d = inp["seq_len"], inp["head_num"], inp["head_dim"]
    ones = np.ones((s, n, d))
    cu = np.array([0, s])
    o, m, l = oracle.forward(ones, ones, ones, cu, cu, n, n, inp["scale"])
    np.testing.assert_allclose(o, exp["out"], rtol=1e-13)
    np.testing.assert_allclose(m, exp["softmax_max"], rtol=1e-13)
    np.testing.assert_allclose(l, exp["softmax_sum"], rtol=1e-13)
    dq, dk, dv, ds = oracle.backward(ones, ones, ones, ones, cu, cu, n, n, inp["scale"])
    np.testing.assert_allclose(dv, exp["dv"], rtol=1e-13)
    np.testing.assert_allclose(dq, exp["dq"], atol=1e-12)
    np.testing.assert_allclose(dk, exp["dk"], atol=1e-12)
    assert ds is None


# --------------------------------------------------------------------------- normalisation

@pytest.mark.parametrize("mode,pre,nxt", [(0, 0, 0), (2, 0, 0), (3, 0, 0), (4, 5, 2)])
@pytest.mark.parametrize("with_sink", [False, True])
def test_rows_sum_to_one(mode, pre, nxt, with_sink):
    lq, lkv, nq, d = 13, 17, 2, 8
    q, k, v = _rand(1, lq, nq, d), _rand(2, lkv, 1, d), _rand(3, lkv, 1, d)
    sink = np.array([0.3, -1.2], np.float32) if with_sink else None
    for h in range(nq):
        st = oracle.probabilities(q, k, v, [0, lq], [0, lkv], nq, 1, 0.3, 0, h, sparse_mode=mode,
                                  pre_tokens=pre, next_tokens=nxt, sink=sink)
        tot = st["p"].sum(axis=1) + st["p_sink"]
        has = st["l"] > 0
        np.testing.assert_allclose(tot[has], 1.0, rtol=0, atol=1e-14)
        assert np.all(st["p"][~has] == 0)


# --------------------------------------------------------------------------- Q = 0 closed forms

def test_q_zero_causal_is_prefix_mean():
    lens = [7, 12]
    cu = _cu(lens)
    t, d = cu[-1], 5
    q = np.zeros((t, 1, d))
    k, v = _rand(4, t, 1, d), _rand(5, t, 1, d)
    o, m, l = oracle.forward(q, k, v, cu, cu, 1, 1, 0.7, sparse_mode=3)
    for b in range(2):
        vb = v[cu[b]:cu[b + 1], 0]
        csum = np.cumsum(vb, axis=0)
        ref = csum / np.arange(1, lens[b] + 1)[:, None]
        np.testing.assert_allclose(o[cu[b]:cu[b + 1], 0], ref, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(l[cu[b]:cu[b + 1], 0], np.arange(1, lens[b] + 1), rtol=1e-14)
        np.testing.assert_allclose(m[cu[b]:cu[b + 1], 0], 0.0, atol=0)


def test_q_zero_band_is_window_mean():
    lq, pre, nxt, d = 20, 3, 2, 4
    q = np.zeros((lq, 1, d))
    k, v = _rand(6, lq, 1, d), _rand(7, lq, 1, d)
    o, _, l = oracle.forward(q, k, v, [0, lq], [0, lq], 1, 1, 1.0, sparse_mode=4, pre_tokens=pre,
                             next_tokens=nxt)
    csum = np.vstack([np.zeros((1, d)), np.cumsum(v[:, 0], axis=0)])
    for i in range(lq):
        lo, hi = max(0, i - pre), min(lq - 1, i + nxt)
        ref = (csum[hi + 1] - csum[lo]) / (hi - lo + 1)
        np.testing.assert_allclose(o[i, 0], ref, rtol=1e-13, atol=1e-14)
        assert l[i, 0] == hi - lo + 1


def test_q_zero_sink_denominator():
    lq, d = 9, 3
    sink = np.array([0.75], np.float32)
    q = np.zeros((lq, 1, d))
    k, v = _rand(8, lq, 1, d), _rand(9, lq, 1, d)
    o, m, l = oracle.forward(q, k, v, [0, lq], [0, lq], 1, 1, 1.0, sparse_mode=3, sink=sink)
    es = math.exp(float(sink[0]))
    csum = np.cumsum(v[:, 0], axis=0)
    n = np.arange(1, lq + 1)
    # all logits are 0 and the sink is 0.75 > 0, so the max is the sink:
    # O_i = sum_{j<=i} v_j e^0 / (n_i e^0 + e^sink), with both scaled by e^-sink
    ref = csum / (n + es)[:, None]
    np.testing.assert_allclose(o[:, 0], ref, rtol=1e-13)
    np.testing.assert_allclose(m[:, 0], float(sink[0]), rtol=0)
    np.testing.assert_allclose(l[:, 0], (n + es) / es, rtol=1e-14)


def test_q_zero_alibi_geometric_weights():
    lq, d = 11, 2
    slope = np.array([0.37], np.float32)
    q = np.zeros((lq, 1, d))
    k, v = _rand(10, lq, 1, d), _rand(11, lq, 1, d)
    o, m, l = oracle.forward(q, k, v, [0, lq], [0, lq], 1, 1, 1.0, sparse_mode=3, alibi_slopes=slope)
    r = math.exp(float(slope[0]))   # weights on key j proportional to r**j
    for i in range(lq):
        w = r ** np.arange(i + 1)
        ref = (w[:, None] * v[:i + 1, 0]).sum(0) / w.sum()
        np.testing.assert_allclose(o[i, 0], ref, rtol=1e-12)
        # the largest logit is at j = i with value 0, so m = 0 and l = sum r^(j-i)
        assert abs(m[i, 0]) < 1e-15
        np.testing.assert_allclose(l[i, 0], w.sum() / r ** i, rtol=1e-12)


def test_pse_sqrt_on_square_distances_equals_linear():
    # pseType 3 turns distance d into sqrt(d); keys at distances 0, 1, 4, 9 of row 9
    # (all others masked out) then carry the pseType 2 biases of distances 0, 1, 2, 3,
    # i.e. of every key of row 3 in a causal sequence of length 4 holding those keys
    d, slope = 3, np.array([0.61], np.float32)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((10, 1, d))
    k, v = rng.standard_normal((10, 1, d)), rng.standard_normal((10, 1, d))
    dy = rng.standard_normal((10, 1, d))
    mask = np.ones((10, 10), np.uint8)
    mask[:, 9] = 0                                   # every row keeps its diagonal-free key 9 ...
    mask[9, :] = 1
    mask[9, [9, 8, 5, 0]] = 0                        # ... and row 9 keeps exactly distances 0, 1, 4, 9
    for r in range(9):
        mask[r, :] = 1
        mask[r, 0] = 0
    kw3 = dict(sparse_mode=1, atten_mask=mask, alibi_slopes=slope, pse_type=3)
    o3, m3, l3 = oracle.forward(q, k, v, [0, 10], [0, 10], 1, 1, 0.7, **kw3)
    sel = [0, 5, 8, 9]                               # key j' of the short sequence = key sel[j']
    q4 = np.concatenate([q[[0, 1, 2]], q[[9]]])      # row 3 of the short sequence is row 9
    dy4 = np.concatenate([np.zeros((3, 1, d)), dy[[9]]])
    kw2 = dict(sparse_mode=3, alibi_slopes=slope, pse_type=2)
    o2, m2, l2 = oracle.forward(q4, k[sel], v[sel], [0, 4], [0, 4], 1, 1, 0.7, **kw2)
    np.testing.assert_allclose(o3[9], o2[3], rtol=1e-13)
    np.testing.assert_allclose([m3[9, 0], l3[9, 0]], [m2[3, 0], l2[3, 0]], rtol=1e-13)
    # the gradient reaching row 9's query and the four keys agrees too
    dy3 = np.zeros_like(dy)
    dy3[9] = dy[9]
    dq3, dk3, dv3, _ = oracle.backward(q, k, v, dy3, [0, 10], [0, 10], 1, 1, 0.7, **kw3)
    dq2, dk2, dv2, _ = oracle.backward(q4, k[sel], v[sel], dy4, [0, 4], [0, 4], 1, 1, 0.7, **kw2)
    np.testing.assert_allclose(dq3[9], dq2[3], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk3[sel], dk2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv3[sel], dv2, rtol=1e-12, atol=1e-14)


def _alibi_tensor(slopes, rows, cols, first_row=0):
    """[1, N, rows, cols] holding -slope_h * (i - j) for full rows first_row .. first_row + rows - 1."""
    i = np.arange(first_row, first_row + rows, dtype=np.float64)[:, None]
    j = np.arange(cols, dtype=np.float64)[None, :]
    return np.stack([-float(s) * (i - j) for s in slopes])[None]


def test_external_pse_reproduces_the_generated_alibi():
    # pseType 0 (add after scaling) with the ALiBi bias written out as a full [S1, S2]
    # tensor gives the pseType 2 result; pseType 1 (add before scaling) needs the bias / scale;
    # a pse shared by the batch equals per-sequence copies
    lens = [9, 14, 5]
    cu = _cu(lens)
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((cu[-1], 2, 4)) for _ in range(3))
    dy = rng.standard_normal((cu[-1], 2, 4))
    slopes = wl.alibi_slopes(2)
    scale = 0.6
    kw = dict(sparse_mode=3)
    ref = oracle.forward(q, k, v, cu, cu, 2, 2, scale, alibi_slopes=slopes, **kw)
    gref = oracle.backward(q, k, v, dy, cu, cu, 2, 2, scale, alibi_slopes=slopes, **kw)
    full = _alibi_tensor(slopes.astype(np.float64), 14, 14)
    for pse, ptype in ((full, 0), (full / scale, 1), (np.repeat(full, 3, axis=0), 0)):
        got = oracle.forward(q, k, v, cu, cu, 2, 2, scale, pse=pse, pse_type=ptype, **kw)
        ggot = oracle.backward(q, k, v, dy, cu, cu, 2, 2, scale, pse=pse, pse_type=ptype, **kw)
        for a, r in zip(got + ggot[:3], ref + gref[:3]):
            np.testing.assert_allclose(a, r, rtol=1e-12, atol=1e-14)


def test_external_pse_row_broadcast_and_compression():
    # a single row is every query row's bias; the 1024-row alibi compression of a
    # Toeplitz bias (lower triangle, Lq = Lkv > 1024) equals the full bias
    rng = np.random.default_rng(13)
    row = rng.standard_normal((1, 1, 1, 6))
    assert np.array_equal(oracle.pse_block(row, 0, 0, 4, 6), np.repeat(row[0, 0], 4, axis=0))
    lq = 1030
    full = _alibi_tensor([0.013], lq, lq)
    comp = full[:, :, -1024:, :]
    got = oracle.pse_block(comp, 0, 0, lq, lq)
    lower = np.tril(np.ones((lq, lq), bool))
    np.testing.assert_array_equal(got[lower], full[0, 0][lower])
    # shorter sequences read the stored rows from the top
    np.testing.assert_array_equal(oracle.pse_block(comp, 0, 0, 700, 700), comp[0, 0, :700, :700])
    # through the whole pass: 6 rows of a 1030-token causal sequence, D = 2
    q = rng.standard_normal((lq, 1, 2))
    k, v = rng.standard_normal((lq, 1, 2)), rng.standard_normal((lq, 1, 2))
    sel = [0, 3, 5, 6, 700, 1029]
    kw = dict(sparse_mode=3, pse_type=0)
    a = oracle.forward(q, k, v, [0, lq], [0, lq], 1, 1, 0.5, pse=full, **kw)
    c = oracle.forward(q, k, v, [0, lq], [0, lq], 1, 1, 0.5, pse=comp, **kw)
    for x, y in zip(a, c):
        np.testing.assert_array_equal(x[sel], y[sel])


def test_backward_matches_autograd_external_pse():
    # pseType 1 with a random full pse, dropout and sink, rectangular sequences in mode 0
    c = _feature_case(63)
    scale = 0.45
    pse = np.random.default_rng(64).standard_normal((2, c["nq"], 9, 9)) * 0.5
    tq = torch.tensor(c["q"], requires_grad=True)
    tk = torch.tensor(c["k"], requires_grad=True)
    tv = torch.tensor(c["v"], requires_grad=True)
    ts = torch.tensor(c["sink"].astype(np.float64), requires_grad=True)
    bits = np.unpackbits(c["mask"], bitorder="little")
    out = _torch_attention(tq, tk, tv, ts, c["cq"], c["ck"], c["nq"], c["nkv"], scale, 0, 0, 0, c["keep"], bits,
                           None, ext_pse=pse)
    (out * torch.from_numpy(c["dy"])).sum().backward()
    kw = dict(sparse_mode=0, keep_prob=c["keep"], drop_mask=c["mask"], sink=c["sink"], pse=pse, pse_type=1)
    o, _, _ = oracle.forward(c["q"], c["k"], c["v"], c["cq"], c["ck"], c["nq"], c["nkv"], scale, **kw)
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-12, atol=1e-13)
    dq, dk, dv, ds = oracle.backward(c["q"], c["k"], c["v"], c["dy"], c["cq"], c["ck"], c["nq"], c["nkv"],
                                     scale, **kw)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (ds, ts.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_batch_slopes_equal_per_sequence_calls():
    # [B, N] slopes: sequence b uses row b, as a call on that sequence alone with [N] slopes
    lens = [7, 12, 5]
    cu = _cu(lens)
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((cu[-1], 2, 4)) for _ in range(3))
    dy = rng.standard_normal((cu[-1], 2, 4))
    slopes = wl.batch_alibi_slopes(3, 3, 2)
    assert not np.allclose(slopes[0], slopes[1])
    for pt in (2, 3):
        o, m, l = oracle.forward(q, k, v, cu, cu, 2, 2, 0.5, sparse_mode=3, alibi_slopes=slopes, pse_type=pt)
        dq, dk, dv, _ = oracle.backward(q, k, v, dy, cu, cu, 2, 2, 0.5, sparse_mode=3, alibi_slopes=slopes,
                                        pse_type=pt)
        for b, L in enumerate(lens):
            s = slice(cu[b], cu[b + 1])
            kw = dict(sparse_mode=3, alibi_slopes=slopes[b], pse_type=pt)
            ob, mb, lb = oracle.forward(q[s], k[s], v[s], [0, L], [0, L], 2, 2, 0.5, **kw)
            dqb, dkb, dvb, _ = oracle.backward(q[s], k[s], v[s], dy[s], [0, L], [0, L], 2, 2, 0.5, **kw)
            for got, ref in ((o[s], ob), (m[s], mb), (l[s], lb), (dq[s], dqb), (dk[s], dkb), (dv[s], dvb)):
                np.testing.assert_array_equal(got, ref)


# --------------------------------------------------------------------------- library routine (SDPA)

def _sdpa(q, k, v, scale, attn_mask=None, is_causal=False, gqa=False):
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]     # [1, N, L, D]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn_mask, is_causal=is_causal,
                                                           scale=scale, enable_gqa=gqa)
    return out[0].permute(1, 0, 2).numpy()


def test_sdpa_no_mask_and_left_up_causal():
    lq, d = 19, 8
    q, k, v = _rand(12, lq, 4, d), _rand(13, lq, 4, d), _rand(14, lq, 4, d)
    o, _, _ = oracle.forward(q, k, v, [0, lq], [0, lq], 4, 4, 0.21)
    np.testing.assert_allclose(o, _sdpa(q, k, v, 0.21), rtol=1e-12, atol=1e-13)
    o, _, _ = oracle.forward(q, k, v, [0, lq], [0, lq], 4, 4, 0.21, sparse_mode=2)
    np.testing.assert_allclose(o, _sdpa(q, k, v, 0.21, is_causal=True), rtol=1e-12, atol=1e-13)


def test_sdpa_right_down_causal_rectangular():
    from torch.nn.attention.bias import causal_lower_right
    lq, lkv, d = 7, 15, 8
    q, k, v = _rand(15, lq, 2, d), _rand(16, lkv, 2, d), _rand(17, lkv, 2, d)
    o, _, _ = oracle.forward(q, k, v, [0, lq], [0, lkv], 2, 2, 0.3, sparse_mode=3)
    bias = causal_lower_right(lq, lkv)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=bias, scale=0.3)[0].permute(1, 0, 2)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("lq,lkv,n", [(9, 14, 8), (14, 9, 3), (11, 11, 0), (11, 11, 11)])
def test_sdpa_prefix_mask(lq, lkv, n):
    # prefix (mode 6): the bottom-right causal triangle, plus a block of the first N
    # keys kept for every row (the left part of the page's compressed mask)
    d = 8
    q, k, v = _rand(40 + n, lq, 2, d), _rand(41 + n, lkv, 2, d), _rand(42 + n, lkv, 2, d)
    o, _, _ = oracle.forward(q, k, v, [0, lq], [0, lkv], 2, 2, 0.35, sparse_mode=6, prefix=[n])
    keep = torch.ones(lq, lkv, dtype=torch.bool).tril(lkv - lq)
    keep[:, :n] = True
    ref = _sdpa(q, k, v, 0.35, attn_mask=keep)
    rows = keep.any(dim=1).numpy()          # SDPA leaves rows without keys undefined
    np.testing.assert_allclose(o[rows], ref[rows], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("lq,lkv", [(13, 13), (9, 20), (20, 9)])
def test_sdpa_atten_mask(lq, lkv):
    # mode 1 (allMask): the attenMask alone decides; 1 = masked out
    d = 8
    q, k, v = _rand(60 + lq, lq, 2, d), _rand(61 + lq, lkv, 2, d), _rand(62 + lq, lkv, 2, d)
    mask = wl.random_atten_mask(lq + lkv, 24, 24, 0.4, full_rows=[3])
    o, _, _ = oracle.forward(q, k, v, [0, lq], [0, lkv], 2, 2, 0.3, sparse_mode=1, atten_mask=mask)
    keep = torch.from_numpy(mask[:lq, :lkv] == 0)
    ref = _sdpa(q, k, v, 0.3, attn_mask=keep)
    rows = keep.any(dim=1).numpy()
    np.testing.assert_allclose(o[rows], ref[rows], rtol=1e-12, atol=1e-13)
    assert np.all(o[~rows] == 0)


def test_sdpa_gqa_and_band_mask():
    lq, d = 23, 8
    q, k, v = _rand(18, lq, 6, d), _rand(19, lq, 2, d), _rand(20, lq, 2, d)
    pre, nxt = 4, 1
    o, _, _ = oracle.forward(q, k, v, [0, lq], [0, lq], 6, 2, 0.4, sparse_mode=4, pre_tokens=pre, next_tokens=nxt)
    keep = torch.ones(lq, lq, dtype=torch.bool).tril(nxt) & torch.ones(lq, lq, dtype=torch.bool).triu(-pre)
    np.testing.assert_allclose(o, _sdpa(q, k, v, 0.4, attn_mask=keep, gqa=True), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- structural identities

def test_gqa_equals_mha_with_repeated_kv():
    lens = [9, 14]
    cu = _cu(lens)
    t, nq, nkv, d = cu[-1], 6, 2, 4
    q, k, v, dy = _rand(21, t, nq, d), _rand(22, t, nkv, d), _rand(23, t, nkv, d), _rand(24, t, nq, d)
    kw = dict(sparse_mode=3, sink=np.linspace(-1, 1, nq).astype(np.float32))
    o1, m1, l1 = oracle.forward(q, k, v, cu, cu, nq, nkv, 0.5, **kw)
    kr, vr = np.repeat(k, nq // nkv, axis=1), np.repeat(v, nq // nkv, axis=1)
    o2, m2, l2 = oracle.forward(q, kr, vr, cu, cu, nq, nq, 0.5, **kw)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    dq1, dk1, dv1, s1 = oracle.backward(q, k, v, dy, cu, cu, nq, nkv, 0.5, **kw)
    dq2, dk2, dv2, s2 = oracle.backward(q, kr, vr, dy, cu, cu, nq, nq, 0.5, **kw)
    np.testing.assert_allclose(dq1, dq2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk1, dk2.reshape(t, nkv, nq // nkv, d).sum(2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv1, dv2.reshape(t, nkv, nq // nkv, d).sum(2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s1, s2, rtol=1e-13)


def test_varlen_equals_per_sequence_runs():
    lq, lkv = [5, 0, 11, 8], [7, 3, 11, 2]
    cq, ck = _cu(lq), _cu(lkv)
    nq, d = 2, 4
    q, k, v, dy = _rand(25, cq[-1], nq, d), _rand(26, ck[-1], nq, d), _rand(27, ck[-1], nq, d), _rand(28, cq[-1], nq, d)
    keep = 0.8
    mask = wl.draw_keep_mask(3, wl.dropout_bits_total(lq, lkv, nq), keep)
    kw = dict(sparse_mode=3, keep_prob=keep, drop_mask=mask)
    o, m, l = oracle.forward(q, k, v, cq, ck, nq, nq, 0.6, **kw)
    dq, dk, dv, _ = oracle.backward(q, k, v, dy, cq, ck, nq, nq, 0.6, **kw)
    bits = np.unpackbits(mask, bitorder="little")
    off = 0
    for b in range(4):
        qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        nbits = nq * lq[b] * lkv[b]
        sub = np.packbits(bits[off:off + nbits], bitorder="little")
        off += nbits
        one = dict(sparse_mode=3, keep_prob=keep, drop_mask=sub)
        o1, m1, l1 = oracle.forward(q[qs], k[ks], v[ks], [0, lq[b]], [0, lkv[b]], nq, nq, 0.6, **one)
        np.testing.assert_array_equal(o[qs], o1)
        np.testing.assert_array_equal(m[qs], m1)
        g1 = oracle.backward(q[qs], k[ks], v[ks], dy[qs], [0, lq[b]], [0, lkv[b]], nq, nq, 0.6, **one)
        np.testing.assert_array_equal(dq[qs], g1[0])
        np.testing.assert_array_equal(dk[ks], g1[1])
        np.testing.assert_array_equal(dv[ks], g1[2])


def test_mode_equivalences():
    lq, d = 21, 4
    q, k, v = _rand(29, lq, 2, d), _rand(30, lq, 2, d), _rand(31, lq, 2, d)
    cu = [0, lq]
    base = oracle.forward(q, k, v, cu, cu, 2, 2, 0.5, sparse_mode=3)[0]
    # mode 2 == mode 3 when Lq == Lkv
    np.testing.assert_array_equal(oracle.forward(q, k, v, cu, cu, 2, 2, 0.5, sparse_mode=2)[0], base)
    # band with pre >= L and next = 0 == causal
    np.testing.assert_array_equal(
        oracle.forward(q, k, v, cu, cu, 2, 2, 0.5, sparse_mode=4, pre_tokens=lq, next_tokens=0)[0], base)
    # band with both windows at INT_MAX == no mask
    np.testing.assert_array_equal(oracle.forward(q, k, v, cu, cu, 2, 2, 0.5, sparse_mode=4)[0],
                                  oracle.forward(q, k, v, cu, cu, 2, 2, 0.5, sparse_mode=0)[0])
    # sink -> -huge == no sink; slope 0 == no pse; keep 1 == no mask
    np.testing.assert_allclose(
        oracle.forward(q, k, v, cu, cu, 2, 2, 0.5, sparse_mode=3, sink=np.array([-1e30, -1e30], np.float32))[0],
        base, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(
        oracle.forward(q, k, v, cu, cu, 2, 2, 0.5, sparse_mode=3, alibi_slopes=np.zeros(2, np.float32))[0], base)
    # attenMask: all zeros == no mask (modes 0 and 1); a strict upper triangle in mode 1 ==
    # leftUpCausal for every sequence (the mask is indexed at each sequence's local rows / keys);
    # in mode 4 the band and the mask both apply
    lens = [7, 12]
    cu3 = _cu(lens)
    q3, k3, v3, dy3 = (_rand(70 + t, cu3[-1], 2, d) for t in range(4))
    zeros = np.zeros((12, 12), np.uint8)
    upper = np.triu(np.ones((12, 12), np.uint8), 1)
    ref0 = oracle.forward(q3, k3, v3, cu3, cu3, 2, 2, 0.5)
    for mode in (0, 1):
        for x, y in zip(oracle.forward(q3, k3, v3, cu3, cu3, 2, 2, 0.5, sparse_mode=mode, atten_mask=zeros), ref0):
            np.testing.assert_array_equal(x, y)
    for x, y in zip(oracle.forward(q3, k3, v3, cu3, cu3, 2, 2, 0.5, sparse_mode=1, atten_mask=upper),
                    oracle.forward(q3, k3, v3, cu3, cu3, 2, 2, 0.5, sparse_mode=2)):
        np.testing.assert_array_equal(x, y)
    ga = oracle.backward(q3, k3, v3, dy3, cu3, cu3, 2, 2, 0.5, sparse_mode=1, atten_mask=upper)
    gb = oracle.backward(q3, k3, v3, dy3, cu3, cu3, 2, 2, 0.5, sparse_mode=2)
    for x, y in zip(ga[:3], gb[:3]):
        np.testing.assert_array_equal(x, y)
    band = oracle.allowed(12, 12, 4, 3, 1)
    np.testing.assert_array_equal(oracle.allowed(12, 12, 4, 3, 1, atten_mask=upper), band & (upper == 0))
    # prefix N = Lkv - Lq == rightDownCausal; N = Lkv == no mask (rectangular sequences)
    lq2, lkv2 = 9, 17
    q2, k2, v2, dy2 = _rand(35, lq2, 2, d), _rand(36, lkv2, 2, d), _rand(37, lkv2, 2, d), _rand(38, lq2, 2, d)
    cq2, ck2 = [0, lq2], [0, lkv2]
    for n, mode in ((lkv2 - lq2, 3), (lkv2, 0)):
        a = oracle.forward(q2, k2, v2, cq2, ck2, 2, 2, 0.5, sparse_mode=6, prefix=[n])
        b = oracle.forward(q2, k2, v2, cq2, ck2, 2, 2, 0.5, sparse_mode=mode)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
        ga = oracle.backward(q2, k2, v2, dy2, cq2, ck2, 2, 2, 0.5, sparse_mode=6, prefix=[n])
        gb = oracle.backward(q2, k2, v2, dy2, cq2, ck2, 2, 2, 0.5, sparse_mode=mode)
        for x, y in zip(ga[:3], gb[:3]):
            np.testing.assert_array_equal(x, y)


def test_dropout_all_keep_scales_output_and_keeps_stats():
    lq, d, keep = 10, 4, 0.5
    q, k, v = _rand(32, lq, 1, d), _rand(33, lq, 1, d), _rand(34, lq, 1, d)
    cu = [0, lq]
    ones = np.full((lq * lq + 7) // 8, 0xFF, np.uint8)
    zeros = np.zeros_like(ones)
    o0, m0, l0 = oracle.forward(q, k, v, cu, cu, 1, 1, 0.5, sparse_mode=3)
    o1, m1, l1 = oracle.forward(q, k, v, cu, cu, 1, 1, 0.5, sparse_mode=3, keep_prob=keep, drop_mask=ones)
    np.testing.assert_allclose(o1, o0 / keep, rtol=1e-14)
    np.testing.assert_array_equal(m1, m0)
    np.testing.assert_array_equal(l1, l0)
    o2, m2, l2 = oracle.forward(q, k, v, cu, cu, 1, 1, 0.5, sparse_mode=3, keep_prob=keep, drop_mask=zeros)
    assert np.all(o2 == 0)
    np.testing.assert_array_equal(l2, l0)


def test_keep_bits_order_lsb_first():
    mask = np.array([0b00000101, 0b10000000], np.uint8)
    z = oracle.keep_bits(mask, 0, 4, 4)
    expect = np.zeros(16, bool)
    expect[[0, 2, 15]] = True
    np.testing.assert_array_equal(z.reshape(-1), expect)
    np.testing.assert_array_equal(oracle.keep_bits(mask, 2, 1, 1), [[True]])


def test_fully_masked_rows():
    lq, lkv, d = 8, 5, 4   # rightDownCausal with Lq > Lkv: rows i < Lq - Lkv see nothing
    q, k, v, dy = _rand(35, lq, 1, d), _rand(36, lkv, 1, d), _rand(37, lkv, 1, d), _rand(38, lq, 1, d)
    o, m, l = oracle.forward(q, k, v, [0, lq], [0, lkv], 1, 1, 0.5, sparse_mode=3)
    dead = slice(0, lq - lkv)
    assert np.all(o[dead] == 0) and np.all(np.isneginf(m[dead])) and np.all(l[dead] == 0)
    assert np.all(np.isfinite(o))
    dq, dk, dv, _ = oracle.backward(q, k, v, dy, [0, lq], [0, lkv], 1, 1, 0.5, sparse_mode=3)
    assert np.all(dq[dead] == 0) and np.all(np.isfinite(dq))
    sink = np.array([0.2], np.float32)
    o, m, l = oracle.forward(q, k, v, [0, lq], [0, lkv], 1, 1, 0.5, sparse_mode=3, sink=sink)
    assert np.all(o[dead] == 0) and np.allclose(m[dead], 0.2, rtol=1e-7) and np.all(l[dead] == 1.0)


def test_dv_is_pt_transpose_dy():
    lq, d = 12, 4
    q, k, v, dy = _rand(39, lq, 1, d), _rand(40, lq, 1, d), _rand(41, lq, 1, d), _rand(42, lq, 1, d)
    mask = wl.draw_keep_mask(9, lq * lq, 0.7)
    kw = dict(sparse_mode=3, keep_prob=0.7, drop_mask=mask)
    st = oracle.probabilities(q, k, v, [0, lq], [0, lq], 1, 1, 0.5, 0, 0, **kw)
    _, _, dv, _ = oracle.backward(q, k, v, dy, [0, lq], [0, lq], 1, 1, 0.5, **kw)
    np.testing.assert_array_equal(dv[:, 0], 0.0 + st["pt"].T @ dy[:, 0])


# --------------------------------------------------------------------------- autograd + finite differences

def _torch_attention(q, k, v, sink, cu_q, cu_kv, nq, nkv, scale, mode, pre, nxt, keep, bits, slopes, prefix=None,
                     atten_mask=None, pse_type=2, ext_pse=None):
    """A second, plainly written attention in torch: the sink enters as an extra
    softmax column that is dropped afterwards; masks come from tril/triu."""
    outs = []
    g = nq // nkv
    off = 0
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_kv[b]), int(cu_kv[b + 1])
        lq, lkv = q1 - q0, k1 - k0
        heads = []
        for h in range(nq):
            s = scale * q[q0:q1, h] @ k[k0:k1, h // g].T
            if ext_pse is not None:   # pseType 1, a full [B, N, S1, S2] block: scale * (QK^T + pse)
                s = scale * (q[q0:q1, h] @ k[k0:k1, h // g].T + torch.from_numpy(ext_pse[b, h, :lq, :lkv]))
            if slopes is not None:
                ii = torch.arange(lq, dtype=torch.float64)[:, None]
                jj = torch.arange(lkv, dtype=torch.float64)[None, :]
                slope = float(slopes[b][h] if np.ndim(slopes) == 2 else slopes[h])
                if pse_type == 3:
                    s = s - slope * torch.sqrt(torch.abs(ii - jj))
                else:
                    s = s + slope * (jj - ii)
            ones = torch.ones(lq, lkv, dtype=torch.bool)
            if mode == 0:
                ok = ones
            elif mode == 2:
                ok = ones.tril(0)
            elif mode == 3:
                ok = ones.tril(lkv - lq)
            elif mode == 6:
                ok = ones.tril(lkv - lq)
                ok[:, :int(prefix[b])] = True
            elif mode == 1:
                ok = torch.from_numpy(atten_mask[:lq, :lkv] == 0)
            else:
                ok = ones.tril(lkv - lq + nxt) & ones.triu(lkv - lq - pre)
            s = s.masked_fill(~ok, float("-inf"))
            if sink is not None:
                s = torch.cat([s, sink[h].expand(lq, 1)], dim=1)
            p = torch.softmax(s, dim=1)
            p = torch.nan_to_num(p, nan=0.0)
            if sink is not None:
                p = p[:, :lkv]
            if keep < 1.0:
                z = torch.from_numpy(bits[off:off + lq * lkv].reshape(lq, lkv).astype(np.float64))
                p = p * z / keep
            off += lq * lkv
            heads.append(p @ v[k0:k1, h // g])
        outs.append(torch.stack(heads, dim=1))
    return torch.cat(outs, dim=0)


def _feature_case(seed, d=4):
    lq, lkv = [6, 9], [6, 9]
    nq, nkv = 4, 2
    cq, ck = _cu(lq), _cu(lkv)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((cq[-1], nq, d))
    k = rng.standard_normal((ck[-1], nkv, d))
    v = rng.standard_normal((ck[-1], nkv, d))
    dy = rng.standard_normal((cq[-1], nq, d))
    sink = rng.standard_normal(nq).astype(np.float32)
    slopes = wl.alibi_slopes(nq)
    keep = 0.75
    mask = wl.draw_keep_mask([seed, 6], wl.dropout_bits_total(lq, lkv, nq), keep)
    return dict(q=q, k=k, v=v, dy=dy, cq=cq, ck=ck, nq=nq, nkv=nkv, sink=sink, slopes=slopes, keep=keep,
                mask=mask)


@pytest.mark.parametrize("mode,pre,nxt", [(3, 0, 0), (4, 2, 1), (0, 0, 0), (6, 0, 0), (1, 0, 0)])
def test_backward_matches_autograd(mode, pre, nxt):
    c = _feature_case(50 + mode)
    scale = 0.45
    tq = torch.tensor(c["q"], requires_grad=True)
    tk = torch.tensor(c["k"], requires_grad=True)
    tv = torch.tensor(c["v"], requires_grad=True)
    ts = torch.tensor(c["sink"].astype(np.float64), requires_grad=True)
    bits = np.unpackbits(c["mask"], bitorder="little")
    prefix = [2, 5] if mode == 6 else None   # sequence lengths 6 and 9: N in [0, L]
    amask = wl.random_atten_mask(9, 9, 9, 0.3, full_rows=[4]) if mode == 1 else None
    out = _torch_attention(tq, tk, tv, ts, c["cq"], c["ck"], c["nq"], c["nkv"], scale, mode, pre, nxt,
                           c["keep"], bits, c["slopes"], prefix, amask)
    (out * torch.from_numpy(c["dy"])).sum().backward()
    kw = dict(sparse_mode=mode, pre_tokens=pre, next_tokens=nxt, keep_prob=c["keep"], drop_mask=c["mask"],
              alibi_slopes=c["slopes"], sink=c["sink"], prefix=prefix, atten_mask=amask)
    o, _, _ = oracle.forward(c["q"], c["k"], c["v"], c["cq"], c["ck"], c["nq"], c["nkv"], scale, **kw)
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-12, atol=1e-13)
    dq, dk, dv, ds = oracle.backward(c["q"], c["k"], c["v"], c["dy"], c["cq"], c["ck"], c["nq"], c["nkv"],
                                     scale, **kw)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ds, ts.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_matches_autograd_pse_sqrt_batch_slopes():
    # pseType 3 with [B, N] slopes (aclnnFlashAttentionScoreV2, pseType table), causal, dropout and sink
    c = _feature_case(61)
    scale = 0.45
    slopes = wl.batch_alibi_slopes(61, 2, c["nq"])
    tq = torch.tensor(c["q"], requires_grad=True)
    tk = torch.tensor(c["k"], requires_grad=True)
    tv = torch.tensor(c["v"], requires_grad=True)
    ts = torch.tensor(c["sink"].astype(np.float64), requires_grad=True)
    bits = np.unpackbits(c["mask"], bitorder="little")
    out = _torch_attention(tq, tk, tv, ts, c["cq"], c["ck"], c["nq"], c["nkv"], scale, 3, 0, 0, c["keep"], bits,
                           slopes, pse_type=3)
    (out * torch.from_numpy(c["dy"])).sum().backward()
    kw = dict(sparse_mode=3, keep_prob=c["keep"], drop_mask=c["mask"], alibi_slopes=slopes, sink=c["sink"],
              pse_type=3)
    o, _, _ = oracle.forward(c["q"], c["k"], c["v"], c["cq"], c["ck"], c["nq"], c["nkv"], scale, **kw)
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-12, atol=1e-13)
    dq, dk, dv, ds = oracle.backward(c["q"], c["k"], c["v"], c["dy"], c["cq"], c["ck"], c["nq"], c["nkv"],
                                     scale, **kw)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (ds, ts.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_matches_finite_differences():
    c = _feature_case(77)
    scale = 0.6
    kw = dict(sparse_mode=4, pre_tokens=3, next_tokens=1, keep_prob=c["keep"], drop_mask=c["mask"],
              alibi_slopes=c["slopes"])

    def loss(q, k, v, sink):
        o, _, _ = oracle.forward(q, k, v, c["cq"], c["ck"], c["nq"], c["nkv"], scale, sink=sink, **kw)
        return float(np.sum(o * c["dy"]))

    # the sink is fp32 on the interface; differentiate with respect to a float64
    # copy by going through probabilities of the unrounded value
    dq, dk, dv, ds = oracle.backward(c["q"], c["k"], c["v"], c["dy"], c["cq"], c["ck"], c["nq"], c["nkv"], scale,
                                     sink=c["sink"], **kw)
    eps = 1e-6
    for name, arr, grad in (("q", c["q"], dq), ("k", c["k"], dk), ("v", c["v"], dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            args1 = {"q": c["q"], "k": c["k"], "v": c["v"]}
            args2 = dict(args1)
            args1[name], args2[name] = a1, a2
            num[idx] = (loss(args1["q"], args1["k"], args1["v"], c["sink"]) -
                        loss(args2["q"], args2["k"], args2["v"], c["sink"])) / (2 * eps)
        err = np.abs(num - grad).max() / np.abs(grad).max()
        assert err < 1e-7, (name, err)
    # dSink: perturb by an amount exactly representable in fp32 around a dyadic sink
    sink0 = np.round(c["sink"] * 256) / 256
    _, _, _, ds0 = oracle.backward(c["q"], c["k"], c["v"], c["dy"], c["cq"], c["ck"], c["nq"], c["nkv"], scale,
                                   sink=sink0.astype(np.float32), **kw)
    h_eps = 2.0 ** -12
    for h in range(c["nq"]):
        s1, s2 = sink0.copy(), sink0.copy()
        s1[h] += h_eps
        s2[h] -= h_eps
        num = (loss(c["q"], c["k"], c["v"], s1.astype(np.float32)) -
               loss(c["q"], c["k"], c["v"], s2.astype(np.float32))) / (2 * h_eps)
        assert abs(num - ds0[h]) <= 1e-6 * max(1.0, abs(ds0[h])), (h, num, ds0[h])


# --------------------------------------------------------------------------- workload generator facts

def test_workload_lengths_and_pairs():
    n5 = wl.workload_lengths(5)
    assert (n5.min(), n5.max(), int(np.median(n5)), n5.sum(), len(n5)) == (209, 16384, 1096, 131072, 64)
    assert list(wl.workload_lengths(2)) == [1736, 630, 337, 701, 922, 1692, 994, 304]
    # closed-form pair count equals a brute-force count from the oracle's mask
    for lens, mode, pre, nxt in (([37, 64], 0, 0, 0), ([30, 7, 19], 3, 0, 0), ([40, 33], 4, 5, 0),
                                 ([12, 9], 2, 0, 0)):
        bf = sum(int(oracle.allowed(L, L, mode, pre, nxt).sum()) for L in lens) * 3
        assert wl.allowed_pairs(lens, lens, 3, mode, pre, nxt) == bf
    assert wl.dropout_bits_total(wl.workload_lengths(4), wl.workload_lengths(4), 16) == 2 ** 30


def test_subset_selection_matches_full_run():
    lens = [9, 6, 11]
    cu = _cu(lens)
    t, nq, nkv, d = cu[-1], 4, 2, 4
    q, k, v, dy = _rand(60, t, nq, d), _rand(61, t, nkv, d), _rand(62, t, nkv, d), _rand(63, t, nq, d)
    full = oracle.backward(q, k, v, dy, cu, cu, nq, nkv, 0.5, sparse_mode=3)
    fo = oracle.forward(q, k, v, cu, cu, nq, nkv, 0.5, sparse_mode=3)
    sub = oracle.backward(q, k, v, dy, cu, cu, nq, nkv, 0.5, sparse_mode=3, batches=[2, 0], heads=[2, 3])
    so = oracle.forward(q, k, v, cu, cu, nq, nkv, 0.5, sparse_mode=3, batches=[2, 0], heads=[2, 3])
    rows = np.r_[cu[0]:cu[1], cu[2]:cu[3]]
    for a, b in ((fo[0], so[0]), (full[0], sub[0])):
        np.testing.assert_array_equal(b[rows][:, 2:], a[rows][:, 2:])
        assert np.all(np.isnan(b[rows][:, :2])) and np.all(np.isnan(b[cu[1]:cu[2]]))
    # kv head 1 owns query heads 2 and 3: complete; kv head 0 untouched (NaN)
    for a, b in ((full[1], sub[1]), (full[2], sub[2])):
        np.testing.assert_array_equal(b[rows][:, 1], a[rows][:, 1])
        assert np.all(np.isnan(b[rows][:, 0]))


def test_row_blocks_match_the_whole_block():
    # row-chunked materialisation (used for the long sequences of the parity tests) is the
    # same computation: rows stand alone in the forward and in dQ, and dK, dV, dSink only
    # add the same terms in another order
    c = wl.make_case("rows", [37, 200, 129], head_num=4, kv_heads=2, head_dim=64, dtype=torch.float32,
                     sparse_mode=3, keep_prob=0.8, alibi=True, sink=True, seed=3)
    kw = dict(keep_prob=c.keep_prob, sparse_mode=3, drop_mask=c.drop_mask, alibi_slopes=c.alibi_slopes,
              sink=c.sink)
    a = [x.float().numpy() for x in (c.q, c.k, c.v)]
    args = (c.cu_seqlens_q, c.cu_seqlens_kv, 4, 2, c.scale)
    whole = oracle.forward(*a, *args, **kw) + oracle.backward(*a, c.dy.float().numpy(), *args, **kw)
    parts = (oracle.forward(*a, *args, row_block=50, **kw) +
             oracle.backward(*a, c.dy.float().numpy(), *args, row_block=50, **kw))
    for x, y in zip(whole, parts):
        np.testing.assert_allclose(y, x, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- sparse modes 7 and 8

def _run(q, k, v, dy, lq, lkv, nq, nkv, scale, **kw):
    cq, ck = _cu(lq), _cu(lkv)
    return (oracle.forward(q, k, v, cq, ck, nq, nkv, scale, **kw) +
            oracle.backward(q, k, v, dy, cq, ck, nq, nkv, scale, **kw))


@pytest.mark.parametrize("mode", [7, 8])
def test_modes_7_8_are_band_plus_causal_per_sequence(mode):
    # mode 7: the last sequence takes the band, the others rightDownCausal; mode 8: the first
    # takes the band, the others leftUpCausal -- each compared with a one-sequence run of the
    # already pinned mode (rectangular sequences, so the two causal alignments differ)
    lq, lkv = [13, 9, 17], [16, 9, 21]
    nq, nkv, d, pre, nxt = 4, 2, 8, 5, 2
    tq, tkv = sum(lq), sum(lkv)
    q, k, v, dy = _rand(80, tq, nq, d), _rand(81, tkv, nkv, d), _rand(82, tkv, nkv, d), _rand(83, tq, nq, d)
    sink = np.array([0.2, -0.5, 1.0, 0.0], np.float32)
    got = _run(q, k, v, dy, lq, lkv, nq, nkv, 0.4, sparse_mode=mode, pre_tokens=pre, next_tokens=nxt, sink=sink)
    cq, ck = _cu(lq), _cu(lkv)
    for b in range(3):
        want_mode = {7: 4 if b == 2 else 3, 8: 4 if b == 0 else 2}[mode]
        assert oracle.sequence_mode(mode, b, 3) == want_mode
        sl_q, sl_k = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        one = _run(q[sl_q], k[sl_k], v[sl_k], dy[sl_q], [lq[b]], [lkv[b]], nq, nkv, 0.4, sparse_mode=want_mode,
                   pre_tokens=pre, next_tokens=nxt, sink=sink)
        for x, y in zip(got[:4], one[:4]):      # O, max, sum, dQ
            np.testing.assert_allclose(x[sl_q], y, rtol=1e-13, atol=1e-14)
        for x, y in zip(got[4:6], one[4:6]):    # dK, dV
            np.testing.assert_allclose(x[sl_k], y, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("pse_type", [2, 3])
def test_mode8_split_rows_reproduce_the_unsplit_band(pse_type):
    # A long band sequence split outside the operator in the query direction: chunk A holds rows
    # [0, a) with keys [0, a), chunk B rows [a, L) with every key [0, L) (qStartIdx = a,
    # kvStartIdx = 0, so Lq - Lkv + qStartIdx - kvStartIdx = 0).  Each chunk runs as the first
    # sequence of a mode-8 call (a complete leftUpCausal sequence follows), with the generated
    # pse on global positions.  Rows and row sums must equal the unsplit mode-4 run (itself
    # pinned against SDPA and autograd); the chunks' dK, dV and dSink add up to the unsplit ones.
    L, a, other = 37, 20, 11
    nq, d, pre, nxt = 2, 8, 9, 0
    q, k, v, dy = _rand(90, L, nq, d), _rand(91, L, 1, d), _rand(92, L, 1, d), _rand(93, L, nq, d)
    qo, ko, vo, dyo = _rand(94, other, nq, d), _rand(95, other, 1, d), _rand(96, other, 1, d), _rand(97, other, nq, d)
    slopes = np.array([0.3, 0.05], np.float32)
    sink = np.array([-0.4, 0.7], np.float32)
    kw = dict(pre_tokens=pre, next_tokens=nxt, alibi_slopes=slopes, pse_type=pse_type, sink=sink)
    whole = _run(q, k, v, dy, [L], [L], nq, 1, 0.35, sparse_mode=4, **kw)
    chunks = {}
    for name, rows, keys, qs in (("A", slice(0, a), slice(0, a), 0), ("B", slice(a, L), slice(0, L), a)):
        nr, nk = rows.stop - rows.start, keys.stop - keys.start
        cat = lambda x, y: np.concatenate([x, y])
        chunks[name] = _run(cat(q[rows], qo), cat(k[keys], ko), cat(v[keys], vo), cat(dy[rows], dyo),
                            [nr, other], [nk, other], nq, 1, 0.35, sparse_mode=8, q_start_idx=qs,
                            kv_start_idx=0, **kw)
    A, B = chunks["A"], chunks["B"]
    for i in range(4):                          # O, max, sum, dQ rows
        np.testing.assert_allclose(A[i][:a], whole[i][:a], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(B[i][:L - a], whole[i][a:], rtol=1e-12, atol=1e-13)
    for i in (4, 5):                            # dK, dV of the split sequence's keys
        summed = B[i][:L].copy()
        summed[:a] += A[i][:a]
        np.testing.assert_allclose(summed, whole[i], rtol=1e-12, atol=1e-13)
    # dSink: the chunks' own rows (the sequence after each chunk is identical in both calls)
    ds_other = _run(qo, ko, vo, dyo, [other], [other], nq, 1, 0.35, sparse_mode=2, sink=sink,
                    alibi_slopes=slopes, pse_type=pse_type)[6]
    np.testing.assert_allclose(A[6] + B[6] - 2 * ds_other, whole[6], rtol=1e-12, atol=1e-13)


def test_mode8_start_indices_shift_only_the_pse():
    # with equal start indices the global positions differ from the local ones by the same
    # amount on both sides, so every pseType 2 / 3 bias (a function of i - j) is unchanged
    lq = [24, 10]
    q, k, v, dy = _rand(100, 34, 2, 8), _rand(101, 34, 1, 8), _rand(102, 34, 1, 8), _rand(103, 34, 2, 8)
    kw = dict(sparse_mode=8, pre_tokens=6, next_tokens=3, alibi_slopes=np.array([0.2, 0.1], np.float32))
    base = _run(q, k, v, dy, lq, lq, 2, 1, 0.3, **kw)
    moved = _run(q, k, v, dy, lq, lq, 2, 1, 0.3, q_start_idx=500, kv_start_idx=500, **kw)
    for x, y in zip(base[:6], moved[:6]):
        np.testing.assert_allclose(y, x, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- value head dim below qD

def test_narrow_value_head_dim_against_sdpa_and_autograd():
    # qD == kD >= vD (grad page, Constraints): torch SDPA takes a value head dim of its own
    # (forward), and torch autograd of the plain expression gives the gradients
    lq, lkv, d, dv = 13, 17, 12, 5
    q, k, v = _rand(110, lq, 2, d), _rand(111, lkv, 2, d), _rand(112, lkv, 2, dv)
    dy = _rand(113, lq, 2, dv)
    o, _, _ = oracle.forward(q, k, v, [0, lq], [0, lkv], 2, 2, 0.3, sparse_mode=3)
    from torch.nn.attention.bias import causal_lower_right
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2)[None].requires_grad_(True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(lq, lkv),
                                                           scale=0.3)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).detach().numpy(), rtol=1e-12, atol=1e-13)
    ref.backward(torch.from_numpy(dy).permute(1, 0, 2)[None])
    dq, dk, dvv, _ = oracle.backward(q, k, v, dy, [0, lq], [0, lkv], 2, 2, 0.3, sparse_mode=3)
    for got, t in ((dq, tq), (dk, tk), (dvv, tv)):
        np.testing.assert_allclose(got, t.grad[0].permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
