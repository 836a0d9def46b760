"""Plain fp64 CPU oracle for decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
It shares no code with the HIP library and imports nothing from it.

What it computes follows the Ascend CANN page aclnnIncreFlashAttentionV2:
  * "Function description / formula": Attention(Q, K, V) = Softmax(Q K^T / sqrt(d)) V
    with the query's S axis fixed at 1 (one new token per sequence) and K, V the
    KV cache of that sequence.
  * Parameters: numHeads / numKeyValueHeads (GQA, Nq a multiple of Nkv),
    actualSeqLengths (the real key length of each batch; the cache is padded),
    scaleValue (the Muls scalar), inputLayout BSH / BNSD / BSND, attenMask.

Readings taken where the page is silent (listed with their reasons in the
design notes):
  * scaleValue replaces 1/sqrt(d).
  * Query head h reads kv head h // (Nq / Nkv) (contiguous groups).
  * attenMask is [B, S] over the padded key axis, nonzero = masked out.
  * A sequence whose keys are all absent (actual length 0) or masked gets a
    zero output row.

Everything is fp64 numpy, one (sequence, head) at a time.
"""
from __future__ import annotations

import numpy as np


def cache_as_bsnd(cache, layout: str, num_kv_heads: int) -> np.ndarray:
    """The KV cache as an array indexed [b, s, kv head, d] (a view where possible)."""
    x = np.asarray(cache)
    if layout == "BSND":
        return x
    if layout == "BSH":
        b, s, hsz = x.shape
        return x.reshape(b, s, num_kv_heads, hsz // num_kv_heads)
    if layout == "BNSD":
        return x.transpose(0, 2, 1, 3)
    raise ValueError(f"layout {layout} not covered")


def decode(q, k, v, num_heads: int, num_kv_heads: int, scale: float, layout: str = "BSND",
           actual_seq_lengths=None, atten_mask=None, batches=None) -> np.ndarray:
    """Decode attention.  q: B*Nq*D values read as [B, Nq, D]; k, v: padded caches
    in `layout`.  Returns out [B, Nq, D] fp64; with `batches`, only those
    sequences are computed and the other rows are NaN."""
    kk = cache_as_bsnd(k, layout, num_kv_heads)
    vv = cache_as_bsnd(v, layout, num_kv_heads)
    bsz, s_max, nkv, d = kk.shape
    if nkv != num_kv_heads or num_heads % num_kv_heads != 0:
        raise ValueError("head counts do not match the cache")
    group = num_heads // num_kv_heads
    qq = np.asarray(q).reshape(bsz, num_heads, d)
    lens = np.full(bsz, s_max, dtype=np.int64) if actual_seq_lengths is None else np.asarray(actual_seq_lengths)
    mask = None if atten_mask is None else np.asarray(atten_mask)
    out = np.full((bsz, num_heads, d), np.nan)
    for b in (range(bsz) if batches is None else batches):
        L = int(lens[b])
        keep = np.ones(L, dtype=bool) if mask is None else mask[b, :L] == 0
        for h in range(num_heads):
            g = h // group
            if not keep.any():
                out[b, h] = 0.0
                continue
            kb = kk[b, :L, g, :].astype(np.float64)[keep]
            vb = vv[b, :L, g, :].astype(np.float64)[keep]
            s = float(scale) * (kb @ qq[b, h].astype(np.float64))
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ vb
    return out
