"""Seeded synthetic inputs for varlen (TND) FlashAttention forward/backward.

This module only draws and lays out inputs: sequence lengths, Q/K/V/dY, the
bit-packed dropout keep-mask, ALiBi slopes and per-head sink logits.  It holds
none of the attention arithmetic, so both the fp64 oracle and the HIP path can
consume the same inputs without sharing any of the method's code.

Layout (TND, as on the Ascend pages' aclnnFlashAttentionUnpaddingScoreGrad,
parameter list and the TND note under "Constraints"): Q, dY are [T_q, Nq, D],
K, V are [T_kv, Nkv, D], row-major and contiguous.  Sequence boundaries are
cumulative offsets cu_seqlens (B+1 entries, leading 0).

Dropout mask (same page, dropMaskOptional): one flat bit stream of
sum_b sum_n Sq_b*Skv_b bits, batch-major, then query head, then query row,
then key; bit 1 = keep.  Bits are packed least-significant-bit first.

Seeds: the lengths of workload k come from numpy.random.default_rng(k); tensor
t (1 Q, 2 K, 3 V, 4 dY, 5 sink, 6 dropout mask) from default_rng([k, t]).
bf16 tensors are the fp32 draws rounded to nearest-even by torch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

INT_MAX_TOKENS = 2147483647

# sparse modes built here (aclnnFlashAttentionUnpaddingScoreGrad, sparseMode list)
MODE_NONE = 0
MODE_LEFT_UP_CAUSAL = 2
MODE_RIGHT_DOWN_CAUSAL = 3
MODE_BAND = 4
MODE_PREFIX = 6
MODE_ALL_MASK = 1
MODE_RIGHT_DOWN_CAUSAL_BAND = 7
MODE_BAND_LEFT_UP_CAUSAL = 8


@dataclass
class Case:
    """One attention problem: host-side inputs plus its attributes."""
    name: str
    dtype: torch.dtype
    cu_seqlens_q: np.ndarray          # int64 [B+1]
    cu_seqlens_kv: np.ndarray         # int64 [B+1]
    head_num: int
    kv_heads: int
    head_dim: int
    scale: float
    q: torch.Tensor                   # [T_q, Nq, D] (cpu)
    k: torch.Tensor                   # [T_kv, Nkv, D]
    v: torch.Tensor
    dy: torch.Tensor                  # [T_q, Nq, D]
    keep_prob: float = 1.0
    sparse_mode: int = MODE_NONE
    pre_tokens: int = INT_MAX_TOKENS
    next_tokens: int = INT_MAX_TOKENS
    drop_mask: Optional[np.ndarray] = None     # uint8 packed bits
    alibi_slopes: Optional[np.ndarray] = None  # float32 [Nq] or [B, Nq]
    pse_type: int = 2                          # 2: -slope*(i-j); 3: -slope*sqrt(|i-j|); 0 / 1 with pse
    pse: Optional[torch.Tensor] = None         # external pse [1 or B, Nq, rows, cols] (cpu, input dtype)
    sink: Optional[np.ndarray] = None          # float32 [Nq]
    prefix: Optional[np.ndarray] = None        # int64 [B]: prefix N per sequence (sparse mode 6)
    atten_mask: Optional[np.ndarray] = None    # uint8 [S1Max, S2Max], nonzero = masked (modes 0/1/4)
    q_start_idx: Optional[int] = None          # mode 8: first sequence's row / key offsets in its unsplit
    kv_start_idx: Optional[int] = None         # sequence (qStartIdx / kvStartIdx)
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.cu_seqlens_q) - 1

    @property
    def lens_q(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q)

    @property
    def lens_kv(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_kv)


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([np.zeros(1, np.int64), np.cumsum(lengths)]).astype(np.int64)


def _normal(seed, shape, dtype: torch.dtype, mult: float = 1.0) -> torch.Tensor:
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if mult != 1.0:
        x = (x * np.float32(mult)).astype(np.float32)
    return torch.from_numpy(x).to(dtype)


def dropout_bits_total(lens_q, lens_kv, head_num) -> int:
    """Bit count of the packed keep-mask: head_num * sum_b Sq_b * Skv_b."""
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_kv = np.asarray(lens_kv, dtype=np.int64)
    return int(head_num * int(np.sum(lens_q * lens_kv)))


def draw_keep_mask(seed, nbits: int, keep_prob: float, chunk: int = 1 << 24) -> np.ndarray:
    """Bernoulli(keep_prob) keep bits, packed LSB-first into ceil(nbits/8) bytes."""
    rng = np.random.default_rng(seed)
    nbytes = (nbits + 7) // 8
    out = np.empty(nbytes, dtype=np.uint8)
    done = 0
    while done < nbits:
        n = min(chunk, nbits - done)           # chunk is a multiple of 8
        bits = rng.random(n) < keep_prob
        packed = np.packbits(bits, bitorder="little")
        out[done // 8: done // 8 + packed.size] = packed
        done += n
    return out


def alibi_slopes(head_num: int) -> np.ndarray:
    """slope_h = 2^(-8(h+1)/N), h = query head, computed in fp64 then rounded to fp32."""
    h = np.arange(head_num, dtype=np.float64)
    return np.power(2.0, -8.0 * (h + 1.0) / head_num).astype(np.float32)


def batch_alibi_slopes(seed, batch: int, head_num: int) -> np.ndarray:
    """[B, Nq] slopes: the geometric slopes of alibi_slopes scaled per sequence by
    a factor drawn uniformly from [0.5, 1.5), rounded to fp32."""
    f = np.random.default_rng([seed, 8]).uniform(0.5, 1.5, (batch, 1))
    return (alibi_slopes(head_num).astype(np.float64)[None, :] * f).astype(np.float32)


def lognormal_lengths(seed, total: int, batch: int, median: float, lo: int, hi: int) -> np.ndarray:
    """Lognormal lengths (median `median`, sigma sqrt(2 ln 2) so the mean is 2*median),
    clipped to [lo, hi], rescaled to sum to `total`, rounded, and the residual
    spread one token at a time over sequences in stable descending-length order."""
    rng = np.random.default_rng(seed)
    x = rng.lognormal(math.log(median), math.sqrt(2.0 * math.log(2.0)), batch)
    x = np.clip(x, lo, hi)
    x = x * (total / x.sum())
    n = np.clip(np.rint(x), lo, hi).astype(np.int64)
    order = np.argsort(-n, kind="stable")
    guard = 0
    while n.sum() != total:
        step = 1 if n.sum() < total else -1
        moved = False
        for idx in order:
            if n.sum() == total:
                break
            if lo <= n[idx] + step <= hi:
                n[idx] += step
                moved = True
        guard += 1
        if not moved or guard > 10 * total:
            raise ValueError("cannot distribute residual within bounds")
    return n


def make_case(name, lens_q, lens_kv=None, *, head_num, kv_heads, head_dim, dtype=torch.bfloat16,
              scale=None, keep_prob=1.0, sparse_mode=MODE_NONE, pre_tokens=INT_MAX_TOKENS,
              next_tokens=INT_MAX_TOKENS, alibi=False, sink=False, seed=0, dy_mult=1.0,
              drop_mask=None, prefix=None, atten_mask=None, pse_type=2, slopes_per_batch=False,
              pse=None, q_start_idx=None, kv_start_idx=None, v_head_dim=None) -> Case:
    """A case built from explicit lengths; every tensor is drawn from default_rng([seed, t]).
    alibi=True adds generated-pse slopes ([Nq], or [B, Nq] with slopes_per_batch) of pseType pse_type.
    pse=(form, shared) adds an external pse of pseType pse_type (0 or 1) drawn from
    default_rng([seed, 9]) (normal, x0.5): form "full" [.., max Lq, max Lkv], "row"
    [.., 1, max Lkv] or "compressed" [.., 1024, max Lkv]; shared -> batch dimension 1."""
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_kv = lens_q.copy() if lens_kv is None else np.asarray(lens_kv, dtype=np.int64)
    cu_q, cu_kv = cu_from_lengths(lens_q), cu_from_lengths(lens_kv)
    tq, tkv = int(cu_q[-1]), int(cu_kv[-1])
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    q = _normal([seed, 1], (tq, head_num, head_dim), dtype)
    k = _normal([seed, 2], (tkv, kv_heads, head_dim), dtype)
    dv_ = head_dim if v_head_dim is None else int(v_head_dim)   # V, O, dY head dim (<= head_dim)
    v = _normal([seed, 3], (tkv, kv_heads, dv_), dtype)
    dy = _normal([seed, 4], (tq, head_num, dv_), dtype, dy_mult)
    sink_v = None
    if sink:
        sink_v = np.random.default_rng([seed, 5]).standard_normal(head_num, dtype=np.float32)
    if keep_prob < 1.0 and drop_mask is None:
        drop_mask = draw_keep_mask([seed, 6], dropout_bits_total(lens_q, lens_kv, head_num), keep_prob)
    pse_t = None
    if pse is not None:
        form, shared = pse
        rows = {"full": int(lens_q.max()), "row": 1, "compressed": 1024}[form]
        pse_t = _normal([seed, 9], (1 if shared else len(lens_q), head_num, rows, int(lens_kv.max())), dtype, 0.5)
    slopes = None
    if alibi:
        slopes = batch_alibi_slopes(seed, len(lens_q), head_num) if slopes_per_batch else alibi_slopes(head_num)
    return Case(name=name, dtype=dtype, cu_seqlens_q=cu_q, cu_seqlens_kv=cu_kv, head_num=head_num,
                kv_heads=kv_heads, head_dim=head_dim, scale=float(scale), q=q, k=k, v=v, dy=dy,
                keep_prob=float(keep_prob), sparse_mode=sparse_mode, pre_tokens=int(pre_tokens),
                next_tokens=int(next_tokens), drop_mask=drop_mask,
                alibi_slopes=slopes, pse_type=int(pse_type), pse=pse_t, sink=sink_v,
                prefix=None if prefix is None else np.asarray(prefix, dtype=np.int64),
                atten_mask=None if atten_mask is None else np.ascontiguousarray(atten_mask, dtype=np.uint8),
                q_start_idx=q_start_idx, kv_start_idx=kv_start_idx)


def random_atten_mask(seed, rows: int, cols: int, p_masked: float, full_rows=()) -> np.ndarray:
    """uint8 [rows, cols] attenMask with each pair masked (1) with probability
    p_masked, and the listed rows masked entirely."""
    m = (np.random.default_rng([seed, 7]).random((rows, cols)) < p_masked).astype(np.uint8)
    for r in full_rows:
        m[r, :] = 1
    return m


WORKLOAD_NAMES = {
    1: "tiny varlen fp32 {37,64} Nq=Nkv=2 D=64 no mask",
    2: "varlen bf16 B=8 U[128,2048] Nq=32 Nkv=8 D=128 causal",
    3: "bf16 B=4 S=8192 Nq=Nkv=32 D=128 window pre=2048 next=0",
    4: "bf16 B=16 S=2048 Nq=Nkv=16 D=128 causal alibi dropout keep=0.9",
    5: "packed varlen bf16 T=131072 B=64 lognormal Nq=64 Nkv=8 D=128 causal sink",
}


def workload_lengths(k: int) -> np.ndarray:
    if k == 1:
        return np.array([37, 64], dtype=np.int64)
    if k == 2:
        return np.random.default_rng(2).integers(128, 2048, 8, endpoint=True).astype(np.int64)
    if k == 3:
        return np.full(4, 8192, dtype=np.int64)
    if k == 4:
        return np.full(16, 2048, dtype=np.int64)
    if k == 5:
        return lognormal_lengths(5, 131072, 64, 1024.0, 64, 16384)
    raise ValueError(f"unknown workload {k}")


def workload_name(k: int, dtype: Optional[torch.dtype] = None) -> str:
    """Name of workload k; dtype float16 / float32 renames the 16-bit workloads."""
    name = WORKLOAD_NAMES[k]
    if dtype == torch.float16:
        return name.replace("bf16", "fp16")
    return name.replace("bf16", "fp32") if dtype == torch.float32 and k != 1 else name


def make_workload(k: int, dtype: Optional[torch.dtype] = None, head_dim: Optional[int] = None) -> Case:
    """The five fixed workloads (sizes, masks and features as listed in WORKLOAD_NAMES).
    dtype=torch.float16 (or torch.float32) draws the 16-bit workloads (2-5) in fp16
    (fp32) instead of bf16: the same normal samples, rounded to the other type.
    head_dim replaces the D = 128 of workloads 2-5 (the same shapes otherwise)."""
    if dtype not in (None, torch.bfloat16, torch.float16, torch.float32) or (dtype == torch.float16 and k == 1):
        raise ValueError(f"workload {k} has no {dtype} variant")
    if head_dim is not None and k == 1:
        raise ValueError("workload 1 has a fixed head dim")
    lens = workload_lengths(k)
    dt = dict(dtype=dtype) if dtype is not None else {}
    D = 128 if head_dim is None else int(head_dim)
    if k == 1:
        c = make_case(WORKLOAD_NAMES[1], lens, head_num=2, kv_heads=2, head_dim=64, dtype=torch.float32,
                      scale=1.0 / 8.0, seed=1)
    elif k == 2:
        c = make_case(workload_name(2, dtype), lens, **dt, head_num=32, kv_heads=8, head_dim=D,
                      sparse_mode=MODE_RIGHT_DOWN_CAUSAL, seed=2)
    elif k == 3:
        c = make_case(workload_name(3, dtype), lens, **dt, head_num=32, kv_heads=32, head_dim=D,
                      sparse_mode=MODE_BAND, pre_tokens=2048, next_tokens=0, seed=3, dy_mult=0.1)
    elif k == 4:
        c = make_case(workload_name(4, dtype), lens, **dt, head_num=16, kv_heads=16, head_dim=D,
                      sparse_mode=MODE_RIGHT_DOWN_CAUSAL, keep_prob=0.9, alibi=True, seed=4)
    elif k == 5:
        c = make_case(workload_name(5, dtype), lens, **dt, head_num=64, kv_heads=8, head_dim=D,
                      sparse_mode=MODE_RIGHT_DOWN_CAUSAL, sink=True, seed=5)
    else:
        raise ValueError(k)
    if D != 128:
        c.name = c.name.replace("D=128", f"D={D}")
    c.meta["workload"] = k
    return c


def allowed_pairs(lens_q, lens_kv, head_num, sparse_mode, pre_tokens=INT_MAX_TOKENS,
                  next_tokens=INT_MAX_TOKENS) -> int:
    """Count of allowed (row, key, query-head) triples, by closed-form interval
    lengths per row (used for the mask-aware FLOP count)."""
    total = 0
    for lq, lkv in zip(np.asarray(lens_q, np.int64), np.asarray(lens_kv, np.int64)):
        lq, lkv = int(lq), int(lkv)
        if lq == 0 or lkv == 0:
            continue
        i = np.arange(lq, dtype=np.int64)
        delta = lkv - lq
        if sparse_mode == MODE_NONE:
            lo = np.zeros(lq, np.int64); hi = np.full(lq, lkv - 1, np.int64)
        elif sparse_mode == MODE_LEFT_UP_CAUSAL:
            lo = np.zeros(lq, np.int64); hi = i
        elif sparse_mode == MODE_RIGHT_DOWN_CAUSAL:
            lo = np.zeros(lq, np.int64); hi = i + delta
        elif sparse_mode == MODE_BAND:
            lo = i + delta - pre_tokens; hi = i + delta + next_tokens
        else:
            raise ValueError(sparse_mode)
        lo = np.maximum(lo, 0); hi = np.minimum(hi, lkv - 1)
        total += int(np.sum(np.maximum(hi - lo + 1, 0)))
    return total * int(head_num)


# ---------------------------------------------------------------------------- decode attention

@dataclass
class DecodeCase:
    """One decode problem: a query token per sequence and the valid rows of its KV
    cache, stored compactly (sequence-major [sum L_b, Nkv, D]); padded_cache()
    lays them out in the cache format of `layout`, zeros beyond each length."""
    name: str
    dtype: torch.dtype
    lens: np.ndarray                  # int64 [B] actual key lengths
    max_seq_len: int                  # S of the padded cache
    num_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    layout: str                       # "BSH", "BSND" or "BNSD"
    q: torch.Tensor                   # [B, Nq, D] (cpu)
    k_rows: torch.Tensor              # [sum L_b, Nkv, D] (cpu)
    v_rows: torch.Tensor
    atten_mask: Optional[np.ndarray] = None   # uint8 [B, S], nonzero = masked
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.lens)

    def padded_cache(self, which: str, device="cpu", batches=None) -> torch.Tensor:
        """K ('k') or V ('v') as the padded cache of `layout` for the listed sequences
        (all by default), built on `device`."""
        rows = self.k_rows if which == "k" else self.v_rows
        bl = list(range(self.batch)) if batches is None else list(batches)
        starts = np.concatenate([[0], np.cumsum(self.lens)])
        cache = torch.zeros((len(bl), self.max_seq_len, self.num_kv_heads, self.head_dim), dtype=self.dtype,
                            device=device)
        for i, b in enumerate(bl):
            L = int(self.lens[b])
            if L:
                cache[i, :L] = rows[int(starts[b]):int(starts[b]) + L].to(device)
        if self.layout == "BSND":
            return cache
        if self.layout == "BSH":
            return cache.reshape(len(bl), self.max_seq_len, self.num_kv_heads * self.head_dim)
        return cache.permute(0, 2, 1, 3).contiguous()   # BNSD

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V the pass must read: the valid rows only."""
        return int(2 * self.lens.sum() * self.num_kv_heads * self.head_dim * torch.finfo(self.dtype).bits // 8)


def make_decode_case(name, lens, max_seq_len=None, *, num_heads, num_kv_heads, head_dim, dtype=torch.bfloat16,
                     layout="BSND", scale=None, seed=0, mask_p=0.0) -> DecodeCase:
    """Decode case from explicit lengths: q, K rows, V rows drawn from default_rng([seed, t])
    (t = 11, 12, 13), the optional [B, S] mask (each key masked with probability mask_p)
    from default_rng([seed, 14])."""
    lens = np.asarray(lens, dtype=np.int64)
    s_max = int(max(1, lens.max())) if max_seq_len is None else int(max_seq_len)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    total = int(lens.sum())
    q = _normal([seed, 11], (len(lens), num_heads, head_dim), dtype)
    k = _normal([seed, 12], (total, num_kv_heads, head_dim), dtype)
    v = _normal([seed, 13], (total, num_kv_heads, head_dim), dtype)
    mask = None
    if mask_p > 0.0:
        mask = (np.random.default_rng([seed, 14]).random((len(lens), s_max)) < mask_p).astype(np.uint8)
    return DecodeCase(name=name, dtype=dtype, lens=lens, max_seq_len=s_max, num_heads=num_heads,
                      num_kv_heads=num_kv_heads, head_dim=head_dim, scale=float(scale), layout=layout, q=q,
                      k_rows=k, v_rows=v, atten_mask=mask)


DECODE_WORKLOAD_NAME = ("decode bf16 B=128 S=16384 lognormal lengths (median 1024, sum 262144) "
                        "Nq=64 Nkv=8 D=128 BSND")


def make_decode_workload(dtype: Optional[torch.dtype] = None, layout: str = "BSND") -> DecodeCase:
    """The decode workload: 128 sequences whose cache lengths follow the packed-varlen
    length law (lognormal, median 1024, in [64, 16384], summing to 262144) over a
    cache padded to 16384, GQA 64/8, D = 128, BSND (or the given layout)."""
    lens = lognormal_lengths(21, 262144, 128, 1024.0, 64, 16384)
    dt = torch.bfloat16 if dtype is None else dtype
    name = DECODE_WORKLOAD_NAME if dt == torch.bfloat16 else DECODE_WORKLOAD_NAME.replace("bf16", "fp16")
    name = name.replace("BSND", layout)
    c = make_decode_case(name, lens, 16384, num_heads=64, num_kv_heads=8, head_dim=128, dtype=dt, layout=layout,
                         seed=21)
    c.meta["workload"] = "decode"
    return c
