"""CPU pins of the decode oracle (oracle/decode.py) against what the pages and the
mathematics fix: the training forward with one query token (itself pinned in
test_oracle.py), torch SDPA in fp64 with a key-padding mask, the Q = 0 closed
form, layout invariance and the empty / fully masked cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def _case(seed, lens, s_max, nq, nkv, d, mask_p=0.0, layout="BSND"):
    c = wl.make_decode_case("pin", lens, s_max, num_heads=nq, num_kv_heads=nkv, head_dim=d, dtype=torch.float32,
                            layout=layout, seed=seed, mask_p=mask_p)
    return c, c.padded_cache("k").numpy(), c.padded_cache("v").numpy()


def _run(c, k, v, **kw):
    return oracle.decode(c.q.numpy(), k, v, c.num_heads, c.num_kv_heads, c.scale, c.layout, c.lens,
                         c.atten_mask, **kw)


@pytest.mark.parametrize("mask_p", [0.0, 0.3])
def test_decode_is_the_forward_with_one_query_token(mask_p):
    # aclnnIncreFlashAttentionV2 computes the same softmax attention as the training
    # forward, for one query row per sequence: each sequence alone, sparse mode 0,
    # with its row of the mask as a 1 x L attenMask
    c, k, v = _case(3, [5, 17, 1, 30], 32, 8, 2, 16, mask_p)
    out = _run(c, k, v)
    for b, L in enumerate(c.lens):
        kw = {} if c.atten_mask is None else dict(atten_mask=c.atten_mask[b:b + 1, :L])
        o, _, _ = oracle.forward(c.q.numpy()[b:b + 1], k[b, :L], v[b, :L], [0, 1], [0, L], 8, 2, c.scale,
                                 sparse_mode=0, **kw)
        np.testing.assert_allclose(out[b], np.nan_to_num(o[0]), rtol=1e-13, atol=1e-15)


def test_decode_matches_sdpa_with_key_padding():
    c, k, v = _case(4, [9, 32, 20], 32, 6, 3, 8, mask_p=0.25)
    out = _run(c, k, v)
    tq = torch.from_numpy(c.q.numpy().astype(np.float64))[:, :, None, :]          # [B, Nq, 1, D]
    tk = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3)              # [B, Nkv, S, D]
    tv = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3)
    keep = torch.arange(32)[None, :] < torch.from_numpy(c.lens)[:, None]
    keep = keep & torch.from_numpy(c.atten_mask == 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep[:, None, None, :],
                                                           scale=c.scale, enable_gqa=True)
    np.testing.assert_allclose(out, ref[:, :, 0, :].numpy(), rtol=1e-12, atol=1e-14)


def test_zero_query_gives_the_mean_of_the_valid_values():
    c, k, v = _case(5, [7, 12], 16, 4, 1, 8)
    c.q.zero_()
    out = _run(c, k, v)
    for b, L in enumerate(c.lens):
        np.testing.assert_allclose(out[b], np.broadcast_to(v[b, :L, 0].astype(np.float64).mean(0), (4, 8)), rtol=1e-13)


def test_layouts_agree():
    outs = []
    for layout in ("BSND", "BSH", "BNSD"):
        c, k, v = _case(6, [3, 11, 8], 12, 4, 2, 8, layout=layout)
        outs.append(_run(c, k, v))
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_empty_and_fully_masked_sequences_give_zeros():
    c, k, v = _case(7, [0, 6, 4], 8, 2, 2, 4)
    c.atten_mask = np.zeros((3, 8), np.uint8)
    c.atten_mask[2, :] = 1
    out = _run(c, k, v)
    assert np.array_equal(out[0], np.zeros((2, 4))) and np.array_equal(out[2], np.zeros((2, 4)))
    assert np.all(np.isfinite(out[1])) and np.abs(out[1]).sum() > 0


def test_padding_rows_are_never_read():
    c, k, v = _case(8, [5, 9], 12, 2, 1, 4)
    base = _run(c, k, v)
    k[0, 5:], v[0, 5:], k[1, 9:], v[1, 9:] = 1e30, np.nan, np.nan, 1e30
    np.testing.assert_array_equal(_run(c, k, v), base)
