"""Plain fp64 CPU oracle for training-time varlen (TND) FlashAttention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
It shares no code with the HIP library and imports nothing from it.

What it computes follows the Ascend CANN pages:
  * aclnnFlashAttentionUnpaddingScoreGrad, section "Function / Formula":
    forward S = Mask(scaled QK^T + pse), P = Dropout(Softmax(S), keep_prob),
    Y = P V; backward dV = P^T dY, dQ = dS K * scale, dK = dS^T Q * scale.
  * aclnnFlashAttentionScoreV2, section "Formula" (pseType other than 1):
    S = scale * (Q K^T) + pse, i.e. the bias is added after scaling.
  * aclnnFlashAttentionUnpaddingScoreGradV5, sink formulas: the running max
    includes the sink logit, the softmax denominator gains exp(sink - m), and
    dSink is a reduction of -P*dP*SimpleSoftmax(sink, max, sum).
  * aclnnFlashAttentionUnpaddingScoreGrad, sparseMode list: 0 no mask,
    2 leftUpCausal, 3 rightDownCausal, 4 band between preTokens/nextTokens,
    6 prefix (with prefixOptional, one N per sequence); attenMaskOptional
    (nonzero = masked out), used by modes 0, 1 (all mask) and 4.

Readings taken where the pages are silent (each is listed with its reason in
the design notes):
  * dS is the softmax Jacobian applied through dropout:
    dS = P * (dP - rowsum(P * dP)), dP = (dY V^T) * z / keep_prob.
  * Dropout is inverted dropout: P~ = P * z / keep_prob; softmax max/sum are
    taken before dropout.  Keep bits: one flat stream over batch, query head,
    query row, key (the page's size formula), LSB first in each byte.
  * "scale" replaces 1/sqrt(d) everywhere (scaleValue is "the Muls scalar").
  * External pse (grad page "pseShiftOptional", ScoreV2 page "realShiftOptional"
    and pseType table): pseType 1 adds it before scaling, S = scale*(QK^T + pse)
    (the grad page's formula); pseType 0 after, S = scale*QK^T + pse.  The
    tensor is [1 or B, N, rows, cols] indexed by local (row, key): one row for
    every query row, the full block, or the ScoreV2 page's alibi compression
    (only the last 1024 rows of the full bias; a row above them is the first
    stored row shifted along its diagonal, which holds for the Toeplitz alibi
    bias the compression is meant for).
  * Generated pse (aclnnFlashAttentionScoreV2, pseType table: types 2 and 3
    build the bias inside the operator from FLOAT32 slopes of shape [N] or
    [B, N]): pseType 2 is ALiBi, pse = -slope_h * (i - j); pseType 3 passes the
    distance through a square root, pse = -slope_h * sqrt(|i - j|); i, j local
    to the sequence, the slope per query head (and per sequence for [B, N]).
  * The sink logit is compared with the scaled, biased logits and is not
    itself scaled.
  * GQA: query head h uses kv head h // (Nq / Nkv).
  * Rows with no allowed key and no sink: O = 0, m = -inf, l = 0, dQ = 0.
  * Band (mode 4) and rightDownCausal (mode 3) align on the bottom-right
    corner (delta = Lkv - Lq); leftUpCausal (mode 2) on the top-left.
  * Prefix (mode 6): the compressed mask the page describes is a lower
    triangle over a block whose left half is kept; read as: row i keeps
    j <= i + delta (the rightDownCausal triangle) and every key j < N of its
    sequence.
  * Sparse modes 7 (rightDownCausal_Band) and 8 (band_LeftUpCausal), which the
    sparseMode list says come from splitting long sequences outside the
    operator: mode 7 gives the last sequence the band and every other one the
    rightDownCausal triangle; mode 8 gives the first sequence the band and every
    other one the leftUpCausal triangle.  The band keeps mode 4's bottom-right
    alignment.
  * qStartIdx / kvStartIdx (ScoreV2 parameters; the V5 grad page's mode-8
    constraint Lq_0 - Lkv_0 + qStartIdx - kvStartIdx == 0): the first sequence
    is a chunk whose row i and key j sit at qStartIdx + i and kvStartIdx + j of
    the unsplit sequence, and in mode 8 its generated pse is formed on those
    positions (the page: "pse generated globally").  Under the constraint the
    band's bottom-right alignment is the unsplit sequence's own diagonal.
  * softmax max/sum are per (row, head) fp32 in natural-log units; the
    page's trailing x8 replication is dropped.

Everything is fp64 numpy; S and P are materialised per (sequence, head).
"""
from __future__ import annotations

import numpy as np

INT_MAX_TOKENS = 2147483647


def allowed(lq: int, lkv: int, sparse_mode: int, pre_tokens: int = INT_MAX_TOKENS,
            next_tokens: int = INT_MAX_TOKENS, prefix: int = 0, atten_mask=None) -> np.ndarray:
    """Boolean [lq, lkv]: True where query row i may attend key j (sparseMode list;
    `prefix` is the sequence's N for mode 6; `atten_mask` [S1Max, S2Max], nonzero =
    masked out, applies in modes 0, 1 and 4 at the sequence's local indices)."""
    if atten_mask is not None and sparse_mode in (0, 1, 4):
        keep = np.asarray(atten_mask)[:lq, :lkv] == 0
        return keep & allowed(lq, lkv, 0 if sparse_mode == 1 else sparse_mode, pre_tokens, next_tokens)
    if sparse_mode == 1:
        raise ValueError("sparse_mode 1 needs atten_mask")
    i = np.arange(lq, dtype=np.int64)[:, None]
    j = np.arange(lkv, dtype=np.int64)[None, :]
    delta = lkv - lq
    if sparse_mode == 0:
        return np.ones((lq, lkv), dtype=bool)
    if sparse_mode == 2:            # leftUpCausal: lower triangle from the top-left corner
        return j <= i
    if sparse_mode == 3:            # rightDownCausal: lower triangle from the bottom-right corner
        return j <= i + delta
    if sparse_mode == 4:            # band: preTokens to the left, nextTokens to the right
        return (j >= i + delta - pre_tokens) & (j <= i + delta + next_tokens)
    if sparse_mode == 6:            # prefix: rightDownCausal plus the first N keys for every row
        return (j <= i + delta) | (j < prefix)
    raise ValueError(f"sparse_mode {sparse_mode} not covered")


def sequence_mode(sparse_mode: int, b: int, batch: int) -> int:
    """The single-sequence mode sequence b of `batch` takes: modes 7 and 8 give the band
    (mode 4) to the last / first sequence and rightDownCausal (3) / leftUpCausal (2) to
    the others; every other mode applies to all sequences alike."""
    if sparse_mode == 7:
        return 4 if b == batch - 1 else 3
    if sparse_mode == 8:
        return 4 if b == 0 else 2
    return sparse_mode


def alibi_pse(lq: int, lkv: int, slope: float, pse_type: int = 2, row0: int = 0, col0: int = 0) -> np.ndarray:
    """Generated bias for one (sequence, head) on positions i = row0 + local row,
    j = col0 + local key (row0 = col0 = 0: local indices):
    pseType 2: -slope * (i - j);  pseType 3: -slope * sqrt(|i - j|)."""
    i = row0 + np.arange(lq, dtype=np.float64)[:, None]
    j = col0 + np.arange(lkv, dtype=np.float64)[None, :]
    if pse_type == 2:
        return -float(slope) * (i - j)
    if pse_type == 3:
        return -float(slope) * np.sqrt(np.abs(i - j))
    raise ValueError(f"pse_type {pse_type} is not a generated pse")


def pse_block(pse: np.ndarray, b: int, h: int, lq: int, lkv: int) -> np.ndarray:
    """Bias of local rows 0..lq-1, keys 0..lkv-1 of (sequence b, head h) from an
    external pse [1 or B, N, rows, cols]; entries the tensor does not define
    (compressed form, above-diagonal keys of rows before the stored block) are NaN."""
    blk = np.asarray(pse[0 if pse.shape[0] == 1 else b, h], dtype=np.float64)
    rows, cols = blk.shape
    if rows == 1:
        return np.repeat(blk[:1, :lkv], lq, axis=0)
    if rows >= lq:
        return blk[:lq, :lkv].copy()
    # alibi compression: the stored rows are full rows lq - rows .. lq - 1
    first = lq - rows
    out = np.full((lq, lkv), np.nan)
    out[first:] = blk[:, :lkv]
    for i in range(first):
        t = first - i                       # value(i, j) = value(i + t, j + t): stored row 0
        j = np.arange(lkv)
        ok = j + t < cols
        out[i, ok] = blk[0, j[ok] + t]
    return out


def keep_bits(drop_mask: np.ndarray, bit_base: int, lq: int, lkv: int) -> np.ndarray:
    """Keep bits z[i, j] for one (sequence, head) block starting at bit `bit_base`
    of the packed mask; bit n lives in byte n // 8 at position n % 8 (LSB first)."""
    idx = bit_base + np.arange(lq * lkv, dtype=np.int64)
    byte = drop_mask[idx >> 3].astype(np.int64)
    return ((byte >> (idx & 7)) & 1).astype(bool).reshape(lq, lkv)


class _Problem:
    """Inputs of one call, upcast to fp64, with the per-sequence bookkeeping."""

    def __init__(self, q, k, v, cu_q, cu_kv, head_num, kv_heads, scale, keep_prob, sparse_mode,
                 pre_tokens, next_tokens, drop_mask, alibi_slopes, sink, prefix=None, atten_mask=None,
                 pse_type=2, pse=None, q_start_idx=None, kv_start_idx=None):
        # kept in their given precision; each (sequence, head) slice is upcast to fp64 when used
        self.q = np.asarray(q)
        self.k = np.asarray(k)
        self.v = np.asarray(v)
        self.cu_q = np.asarray(cu_q, dtype=np.int64)
        self.cu_kv = np.asarray(cu_kv, dtype=np.int64)
        self.nq = int(head_num)
        self.nkv = int(kv_heads)
        if self.nq % self.nkv != 0:
            raise ValueError("Nq must be a multiple of Nkv")
        self.group = self.nq // self.nkv
        self.scale = float(scale)
        self.keep = float(keep_prob)
        self.mode = int(sparse_mode)
        self.pre = int(pre_tokens)
        self.next = int(next_tokens)
        self.drop_mask = None if drop_mask is None else np.asarray(drop_mask, dtype=np.uint8)
        # slopes [Nq] (shared by the sequences) or [B, Nq]
        self.slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float32).astype(np.float64)
        self.pse_type = int(pse_type)
        self.pse = None if pse is None else np.asarray(pse)
        self.sink = None if sink is None else np.asarray(sink, dtype=np.float32).astype(np.float64)
        self.batch = len(self.cu_q) - 1
        self.prefix = np.zeros(self.batch, dtype=np.int64) if prefix is None else np.asarray(prefix, dtype=np.int64)
        self.atten_mask = None if atten_mask is None else np.asarray(atten_mask)
        # positions of the first sequence in the sequence it was split from (mode 8)
        self.q_start = 0 if q_start_idx is None else int(q_start_idx)
        self.kv_start = 0 if kv_start_idx is None else int(kv_start_idx)
        self.lens_q = np.diff(self.cu_q)
        self.lens_kv = np.diff(self.cu_kv)
        # start bit of each sequence's block in the packed keep mask
        self.bit_base = np.concatenate([[0], np.cumsum(self.nq * self.lens_q * self.lens_kv)]).astype(np.int64)

    def probs(self, b: int, h: int, r0: int = 0, r1=None):
        """S, P (pre-dropout), P~ (post-dropout), m, l, p_sink for sequence b, query
        head h, local query rows [r0, r1) (default: every row).  Rows are
        independent in every formula above, so a row range gives exactly those
        rows of the whole block."""
        q0, q1 = self.cu_q[b], self.cu_q[b + 1]
        k0, k1 = self.cu_kv[b], self.cu_kv[b + 1]
        lq, lkv = int(q1 - q0), int(k1 - k0)
        r1 = lq if r1 is None else min(int(r1), lq)
        r0 = int(r0)
        g = h // self.group
        qb = self.q[q0 + r0:q0 + r1, h, :].astype(np.float64)
        kb = self.k[k0:k1, g, :].astype(np.float64)
        s = self.scale * (qb @ kb.T)
        if self.pse is not None:
            bias = pse_block(self.pse, b, h, lq, lkv)[r0:r1]
            s = self.scale * (qb @ kb.T + bias) if self.pse_type == 1 else s + bias
        elif self.slopes is not None:
            slope = self.slopes[b, h] if self.slopes.ndim == 2 else self.slopes[h]
            first = b == 0 and self.mode == 8
            s = s + alibi_pse(lq, lkv, slope, self.pse_type, self.q_start if first else 0,
                              self.kv_start if first else 0)[r0:r1]
        ok = allowed(lq, lkv, sequence_mode(self.mode, b, self.batch), self.pre, self.next, int(self.prefix[b]),
                     self.atten_mask)[r0:r1]
        s = np.where(ok, s, -np.inf)
        m = s.max(axis=1) if lkv > 0 else np.full(r1 - r0, -np.inf)
        if self.sink is not None:
            m = np.maximum(m, self.sink[h])
        finite = np.isfinite(m)
        e = np.where(ok & finite[:, None], np.exp(s - np.where(finite, m, 0.0)[:, None]), 0.0)
        l = e.sum(axis=1)
        p_sink = np.zeros(r1 - r0)
        if self.sink is not None:
            es = np.exp(self.sink[h] - m)
            l = l + es
        nz = l > 0
        p = np.where(nz[:, None], e / np.where(nz, l, 1.0)[:, None], 0.0)
        if self.sink is not None:
            p_sink = np.where(nz, np.exp(self.sink[h] - m) / np.where(nz, l, 1.0), 0.0)
        if self.keep < 1.0:
            z = keep_bits(self.drop_mask, int(self.bit_base[b] + h * lq * lkv + r0 * lkv), r1 - r0, lkv)
            pt = p * z / self.keep
        else:
            z = None
            pt = p
        return dict(s=s, p=p, pt=pt, z=z, m=m, l=l, p_sink=p_sink, lq=lq, lkv=lkv,
                    q0=q0 + r0, q1=q0 + r1, k0=k0, k1=k1, g=g)

    def row_ranges(self, b: int, row_block):
        """Local row ranges covering sequence b, row_block rows at a time (None: one range)."""
        lq = int(self.cu_q[b + 1] - self.cu_q[b])
        if row_block is None or lq == 0:
            return [(0, lq)]
        return [(r, min(r + int(row_block), lq)) for r in range(0, lq, int(row_block))]


def _problem(q, k, v, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, scale, keep_prob=1.0,
             sparse_mode=0, pre_tokens=INT_MAX_TOKENS, next_tokens=INT_MAX_TOKENS, drop_mask=None,
             alibi_slopes=None, sink=None, prefix=None, atten_mask=None, pse_type=2, pse=None,
             q_start_idx=None, kv_start_idx=None):
    return _Problem(q, k, v, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, scale, keep_prob,
                    sparse_mode, pre_tokens, next_tokens, drop_mask, alibi_slopes, sink, prefix, atten_mask,
                    pse_type, pse, q_start_idx, kv_start_idx)


def _selected(subset, n):
    return range(n) if subset is None else list(subset)


def forward(q, k, v, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, scale, keep_prob=1.0,
            sparse_mode=0, pre_tokens=INT_MAX_TOKENS, next_tokens=INT_MAX_TOKENS, drop_mask=None,
            alibi_slopes=None, sink=None, batches=None, heads=None, prefix=None, atten_mask=None,
            pse_type=2, pse=None, row_block=None, q_start_idx=None, kv_start_idx=None):
    """Attention forward.  Returns O [T_q, Nq, D], softmax max m [T_q, Nq] and
    softmax sum l [T_q, Nq] (fp64).  With `batches` / `heads`, only those
    sequences / query heads are computed and every other entry is NaN.
    `row_block` bounds the rows materialised at once (every row stands alone, so
    the result is the same)."""
    pr = _problem(q, k, v, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, scale, keep_prob,
                  sparse_mode, pre_tokens, next_tokens, drop_mask, alibi_slopes, sink, prefix, atten_mask,
                  pse_type, pse, q_start_idx, kv_start_idx)
    tq, d = pr.q.shape[0], pr.v.shape[2]
    out = np.full((tq, pr.nq, d), np.nan)
    mx = np.full((tq, pr.nq), np.nan)
    sm = np.full((tq, pr.nq), np.nan)
    for b in _selected(batches, pr.batch):
        for h in _selected(heads, pr.nq):
            for r0, r1 in pr.row_ranges(b, row_block):
                st = pr.probs(b, h, r0, r1)
                out[st["q0"]:st["q1"], h, :] = st["pt"] @ pr.v[st["k0"]:st["k1"], st["g"], :].astype(np.float64)
                mx[st["q0"]:st["q1"], h] = st["m"]
                sm[st["q0"]:st["q1"], h] = st["l"]
    return out, mx, sm


def backward(q, k, v, dy, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, scale, keep_prob=1.0,
             sparse_mode=0, pre_tokens=INT_MAX_TOKENS, next_tokens=INT_MAX_TOKENS, drop_mask=None,
             alibi_slopes=None, sink=None, batches=None, heads=None, prefix=None, atten_mask=None,
             pse_type=2, pse=None, row_block=None, q_start_idx=None, kv_start_idx=None):
    """Attention backward.  Returns dQ [T_q, Nq, D], dK, dV [T_kv, Nkv, D] and
    dSink [Nq] (None without a sink).  With `batches` / `heads`, only those
    sequences / query heads contribute: rows and keys of other sequences are NaN,
    dK/dV of a kv head are complete only if all of its query heads are chosen,
    and dSink sums the chosen sequences.  `row_block` bounds the rows materialised
    at once: dQ rows are unchanged, and dK, dV, dSink become sums over row
    ranges (the same terms, added in another order)."""
    pr = _problem(q, k, v, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, scale, keep_prob,
                  sparse_mode, pre_tokens, next_tokens, drop_mask, alibi_slopes, sink, prefix, atten_mask,
                  pse_type, pse, q_start_idx, kv_start_idx)
    dy = np.asarray(dy)
    dq = np.full(pr.q.shape, np.nan)
    dk = np.full(pr.k.shape, np.nan)
    dv = np.full(pr.v.shape, np.nan)
    dsink = np.zeros(pr.nq) if pr.sink is not None else None
    for b in _selected(batches, pr.batch):
        k0, k1 = pr.cu_kv[b], pr.cu_kv[b + 1]
        chosen = list(_selected(heads, pr.nq))
        for g in sorted({h // pr.group for h in chosen}):
            dk[k0:k1, g] = 0.0
            dv[k0:k1, g] = 0.0
        for h in chosen:
            for r0, r1 in pr.row_ranges(b, row_block):
                st = pr.probs(b, h, r0, r1)
                g, q0, q1 = st["g"], st["q0"], st["q1"]
                dyb = dy[q0:q1, h, :].astype(np.float64)
                vb = pr.v[k0:k1, g, :].astype(np.float64)
                kb = pr.k[k0:k1, g, :].astype(np.float64)
                qb = pr.q[q0:q1, h, :].astype(np.float64)
                # dV = P~^T dY
                dv[k0:k1, g, :] += st["pt"].T @ dyb
                # dP = (dY V^T) * z / keep  (gradient w.r.t. the pre-dropout P)
                dp = dyb @ vb.T
                if st["z"] is not None:
                    dp = dp * st["z"] / pr.keep
                p = st["p"]
                # softmax Jacobian: dS = P * (dP - rowsum(P * dP)); the sink column has dP = 0
                row = np.sum(p * dp, axis=1)
                ds = p * (dp - row[:, None])
                dq[q0:q1, h, :] = pr.scale * (ds @ kb)
                dk[k0:k1, g, :] += pr.scale * (ds.T @ qb)
                if dsink is not None:
                    # dSink = sum over rows of -p_sink * rowsum(P * dP)
                    dsink[h] += float(np.sum(-st["p_sink"] * row))
    return dq, dk, dv, dsink


def probabilities(q, k, v, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, scale, b, h, **kw):
    """The materialised S, P, P~, m, l and sink probability of one (sequence, head)."""
    pr = _problem(q, k, v, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, scale, **kw)
    return pr.probs(b, h)
