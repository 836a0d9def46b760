"""ctypes binding of libfa.so (include/fa.h).  Argument marshalling only: every
step of the computation runs in the library's HIP kernels.  torch supplies
device memory and the stream handle.

The library must have been built (python -m attention_fa_fwd_amd.build); there
is no fallback: loading fails loudly when libfa.so is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
# the trace build (same sources, per-tile visit counters; include/fa_trace.h), for tests only
TRACE_LIB_PATH = os.path.join(_PKG, "libfa_trace.so")

FA_OK = 0
FA_ERR_PARAM_NULLPTR = 161001
FA_ERR_PARAM_INVALID = 161002
FA_ERR_WORKSPACE = 1
FA_ERR_HIP = 2
FA_ERR_SCRATCH = 3
FA_DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20

FA_DTYPE_FP32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_FP16 = 2
FA_FLAG_PSE_SQRT = 1
FA_FLAG_SLOPES_PER_BATCH = 2
FA_FLAG_ATOMIC_DQ = 4
TOKENS_DEFAULT = 2147483647
FA_LAYOUT_TND = 0
FA_LAYOUT_BSH = 1
FA_LAYOUT_BSND = 2
FA_LAYOUT_BNSD = 3
FA_LAYOUT_SBH = 4

EXPORTED = ("fa_fwd_workspace_size", "fa_fwd", "fa_bwd_workspace_size", "fa_bwd", "fa_status_string",
            "fa_debug_schedule", "fa_profile_enable", "fa_profile_read", "fa_profile_kernel_count",
            "fa_decode_workspace_size", "fa_decode", "fa_decode_noalloc")


class FaConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("cu_seqlens_q", ctypes.POINTER(ctypes.c_int64)),
        ("cu_seqlens_kv", ctypes.POINTER(ctypes.c_int64)),
        ("head_num", ctypes.c_int64),
        ("num_kv_heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("sparse_mode", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("keep_prob", ctypes.c_double),
        ("pre_tokens", ctypes.c_int64),
        ("next_tokens", ctypes.c_int64),
        ("deterministic", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("prefix", ctypes.POINTER(ctypes.c_int64)),
        ("atten_mask", ctypes.c_void_p),
        ("mask_rows", ctypes.c_int64),
        ("mask_cols", ctypes.c_int64),
        ("layout", ctypes.c_int32),
        ("pse", ctypes.c_void_p),
        ("pse_batch", ctypes.c_int64),
        ("pse_rows", ctypes.c_int64),
        ("pse_cols", ctypes.c_int64),
        ("pse_type", ctypes.c_int32),
        ("strides", ctypes.POINTER(ctypes.c_int64)),
        ("q_start_idx", ctypes.POINTER(ctypes.c_int64)),
        ("kv_start_idx", ctypes.POINTER(ctypes.c_int64)),
        ("v_head_dim", ctypes.c_int64),
    ]


class FaDecodeConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("max_seq_len", ctypes.c_int64),
        ("actual_seq_lengths", ctypes.POINTER(ctypes.c_int64)),
        ("num_heads", ctypes.c_int64),
        ("num_kv_heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("atten_mask", ctypes.c_void_p),
        ("flags", ctypes.c_int32),
    ]


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None
_trace_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if libfa.so was not built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def trace_lib() -> ctypes.CDLL:
    """The trace build of the library (same C ABI plus fa_debug_trace)."""
    global _trace_lib
    if _trace_lib is None:
        L = _load(TRACE_LIB_PATH)
        L.fa_debug_trace.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64]
        L.fa_debug_trace.restype = ctypes.c_int32
        _trace_lib = L
    return _trace_lib


def _load(path: str) -> ctypes.CDLL:
    """Loads one build of the library and declares its C signatures."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m attention_fa_fwd_amd.build`")
    L = ctypes.CDLL(path)
    vp, u64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint64)
    cfgp = ctypes.POINTER(FaConfig)
    L.fa_fwd_workspace_size.argtypes = [cfgp, u64p]
    L.fa_bwd_workspace_size.argtypes = [cfgp, u64p]
    L.fa_fwd.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
    L.fa_bwd.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
    L.fa_status_string.argtypes = [ctypes.c_int32]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_debug_schedule.argtypes = [cfgp, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                    ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int32)]
    L.fa_profile_enable.argtypes = [ctypes.c_int32]
    L.fa_profile_read.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.fa_profile_kernel_count.restype = ctypes.c_int32
    decp = ctypes.POINTER(FaDecodeConfig)
    L.fa_decode_workspace_size.argtypes = [decp, u64p]
    L.fa_decode.argtypes = [decp, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
    L.fa_decode_noalloc.argtypes = [decp, vp, vp, vp, vp, vp]
    for name in ("fa_fwd_workspace_size", "fa_bwd_workspace_size", "fa_fwd", "fa_bwd", "fa_debug_schedule",
                 "fa_profile_enable", "fa_profile_read", "fa_decode_workspace_size", "fa_decode",
                 "fa_decode_noalloc"):
        getattr(L, name).restype = ctypes.c_int32
    return L


def status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


class Config:
    """Owns the host cu_seqlens arrays for the lifetime of a fa_config."""

    def __init__(self, cu_seqlens_q, cu_seqlens_kv, head_num, kv_heads, head_dim, dtype, scale, keep_prob=1.0,
                 sparse_mode=0, pre_tokens=TOKENS_DEFAULT, next_tokens=TOKENS_DEFAULT, deterministic=True,
                 prefix=None, atten_mask=None, pse_type=2, slopes_per_batch=False, layout="TND", pse=None,
                 atomic_dq=False, q_start_idx=None, kv_start_idx=None, v_head_dim=None):
        self.cu_q = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int64))
        self.cu_kv = np.ascontiguousarray(np.asarray(cu_seqlens_kv, dtype=np.int64))
        # per-sequence prefix N of sparse mode 6 (prefixOptional); NULL when None
        self.prefix = None if prefix is None else np.ascontiguousarray(np.asarray(prefix, dtype=np.int64))
        # qStartIdx / kvStartIdx (sparse mode 8): one host value each, or None
        self.q_start = None if q_start_idx is None else np.array([int(q_start_idx)], dtype=np.int64)
        self.kv_start = None if kv_start_idx is None else np.array([int(kv_start_idx)], dtype=np.int64)
        # attenMask: a device tensor of bool / uint8 [S1Max, S2Max], nonzero = masked out (kept alive here)
        self.atten_mask = atten_mask
        if atten_mask is not None:
            if atten_mask.dim() != 2 or atten_mask.dtype not in (torch.uint8, torch.bool) or not atten_mask.is_contiguous():
                raise ValueError("atten_mask must be a contiguous 2-D bool or uint8 tensor [S1Max, S2Max]")
        # pseType of the slopes passed to fa_fwd / fa_bwd: 2 (linear distance) or 3 (square root)
        # pse: optional device tensor [1 or B, Nq, rows, cols] of the input type (pseType 0 / 1);
        # without it pse_type names how alibi slopes generate the bias (2 / 3)
        self.pse = pse
        if pse is not None:
            if pse.dim() != 4 or not pse.is_contiguous() or pse_type not in (0, 1):
                raise ValueError("pse must be a contiguous [1 or B, Nq, rows, cols] tensor with pse_type 0 or 1")
        elif pse_type not in (2, 3):
            raise ValueError("pse_type must be 2 or 3 (generated from alibi slopes) without a pse tensor")
        self.slopes_per_batch = bool(slopes_per_batch)
        # inputLayout of Q, K, V, dY, O and the gradients; the fixed-length layouts take
        # cu_seqlens with one common length per side
        self.layout_name = layout
        # atomic_dq: with deterministic=False, the fp32-atomic dQ scheme instead of the (faster) separate pass
        flags = ((FA_FLAG_PSE_SQRT if pse_type == 3 and pse is None else 0)
                 | (FA_FLAG_SLOPES_PER_BATCH if slopes_per_batch else 0) | (FA_FLAG_ATOMIC_DQ if atomic_dq else 0))
        if isinstance(dtype, torch.dtype):
            dtype = {torch.float32: FA_DTYPE_FP32, torch.bfloat16: FA_DTYPE_BF16,
                     torch.float16: FA_DTYPE_FP16}.get(dtype, -1)
        self.c = FaConfig(
            batch=len(self.cu_q) - 1,
            cu_seqlens_q=self.cu_q.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            cu_seqlens_kv=self.cu_kv.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            head_num=int(head_num), num_kv_heads=int(kv_heads), head_dim=int(head_dim), dtype=int(dtype),
            sparse_mode=int(sparse_mode), scale=float(scale), keep_prob=float(keep_prob),
            pre_tokens=int(pre_tokens), next_tokens=int(next_tokens), deterministic=1 if deterministic else 0,
            flags=flags,
            prefix=(None if self.prefix is None else self.prefix.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
            atten_mask=(None if atten_mask is None else atten_mask.data_ptr()),
            mask_rows=(0 if atten_mask is None else int(atten_mask.shape[0])),
            mask_cols=(0 if atten_mask is None else int(atten_mask.shape[1])),
            layout=_LAYOUTS.get(layout, -1),
            pse=(None if pse is None else pse.data_ptr()),
            pse_batch=(0 if pse is None else int(pse.shape[0])),
            pse_rows=(0 if pse is None else int(pse.shape[2])),
            pse_cols=(0 if pse is None else int(pse.shape[3])),
            pse_type=(int(pse_type) if pse is not None else 0),
            q_start_idx=(None if self.q_start is None else self.q_start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
            kv_start_idx=(None if self.kv_start is None else
                          self.kv_start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
            v_head_dim=0 if v_head_dim is None else int(v_head_dim))

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int, where: str):
    if status != FA_OK:
        raise FaError(status, where)


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensor(name, t, shape, dtype, device, strided=False):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if strided:
        # TND tensors may be strided views: the D axis contiguous, rows 16-byte aligned
        if t.stride(2) != 1 or any((st * t.element_size()) % 16 for st in t.stride()[:2]):
            raise ValueError(f"{name} needs a contiguous last axis and 16-byte multiples as its other strides")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_SLOTS = ("q", "k", "v", "dy", "out", "dq", "dk", "dv")
_VALUE_SIDE = ("v", "dy", "out", "dv")


def head_dims(cfg: "Config"):
    """(head dim of q, k, dq, dk; head dim of v, out, dy, dv)."""
    return cfg.c.head_dim, cfg.c.v_head_dim or cfg.c.head_dim


def _set_strides(cfg: "Config", tensors: dict):
    """Fills cfg's (token, head) strides of the TND tensors of this call; NULL when all are packed."""
    if cfg.layout_name != "TND":
        cfg.c.strides = None
        return
    vals, packed = [], True
    for name in _SLOTS:
        t = tensors.get(name)
        n = cfg.c.head_num if name in ("q", "dy", "out", "dq") else (cfg.c.num_kv_heads or cfg.c.head_num)
        d = head_dims(cfg)[1 if name in _VALUE_SIDE else 0]
        st = (n * d, d) if t is None else (t.stride(0), t.stride(1))
        packed = packed and st == (n * d, d)
        vals += list(st)
    if packed:
        cfg.c.strides = None
        return
    cfg._strides = np.ascontiguousarray(np.asarray(vals, dtype=np.int64))
    cfg.c.strides = cfg._strides.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def fa_fwd_workspace_size(cfg: Config) -> int:
    n = ctypes.c_uint64(0)
    _check(lib().fa_fwd_workspace_size(cfg.ref, ctypes.byref(n)), "fa_fwd_workspace_size")
    return n.value


def fa_bwd_workspace_size(cfg: Config) -> int:
    n = ctypes.c_uint64(0)
    _check(lib().fa_bwd_workspace_size(cfg.ref, ctypes.byref(n)), "fa_bwd_workspace_size")
    return n.value


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def layout_shape(cfg: Config, q_side: bool, value: bool = False):
    """Shape of a query-side (q, dy, out, dq) or key-side (k, v, dk, dv) tensor in cfg's layout;
    value=True for the value-side tensors (v, out, dy, dv), whose head dim may be smaller."""
    n = cfg.c.head_num if q_side else (cfg.c.num_kv_heads or cfg.c.head_num)
    cu = cfg.cu_q if q_side else cfg.cu_kv
    d, t, b = head_dims(cfg)[1 if value else 0], int(cu[-1]), len(cu) - 1
    s = int(cu[1]) if b > 0 else 0
    return {"TND": (t, n, d), "BSND": (b, s, n, d), "BSH": (b, s, n * d), "BNSD": (b, n, s, d),
            "SBH": (s, b, n * d)}[cfg.layout_name]


def _common_checks(q, k, v, cfg: Config):
    dev = q.device
    tq, tkv = int(cfg.cu_q[-1]), int(cfg.cu_kv[-1])
    nq, nkv, d = cfg.c.head_num, cfg.c.num_kv_heads or cfg.c.head_num, cfg.c.head_dim
    if cfg.layout_name not in _LAYOUTS:
        raise ValueError(f"unknown layout {cfg.layout_name}")
    tnd = cfg.layout_name == "TND"
    _check_tensor("q", q, layout_shape(cfg, True), q.dtype, dev, tnd)
    _check_tensor("k", k, layout_shape(cfg, False), q.dtype, dev, tnd)
    _check_tensor("v", v, layout_shape(cfg, False, True), q.dtype, dev, tnd)
    return dev, tq, tkv, nq, nkv, d


def _check_slopes_sink(cfg: Config, alibi_slopes, sink, nq, dev):
    if alibi_slopes is not None:
        shape = (cfg.c.batch, nq) if cfg.slopes_per_batch else (nq,)
        _check_tensor("alibi_slopes", alibi_slopes, shape, torch.float32, dev)
    if sink is not None:
        _check_tensor("sink", sink, (nq,), torch.float32, dev)


def fa_fwd(cfg: Config, q, k, v, drop_mask=None, alibi_slopes=None, sink=None, out=None, softmax_max=None,
           softmax_sum=None, workspace=None):
    """Forward through libfa.so on the current stream; returns (out, softmax_max, softmax_sum)."""
    dev, tq, tkv, nq, nkv, d = _common_checks(q, k, v, cfg)
    if out is None:
        out = torch.empty(layout_shape(cfg, True, True), dtype=q.dtype, device=dev)
    if softmax_max is None:
        softmax_max = torch.empty((tq, nq), dtype=torch.float32, device=dev)
    if softmax_sum is None:
        softmax_sum = torch.empty((tq, nq), dtype=torch.float32, device=dev)
    _check_tensor("out", out, layout_shape(cfg, True, True), q.dtype, dev, cfg.layout_name == "TND")
    _check_tensor("softmax_max", softmax_max, (tq, nq), torch.float32, dev)
    _check_tensor("softmax_sum", softmax_sum, (tq, nq), torch.float32, dev)
    _check_slopes_sink(cfg, alibi_slopes, sink, nq, dev)
    if drop_mask is not None and (drop_mask.dtype != torch.uint8 or drop_mask.device != dev):
        raise ValueError("drop_mask must be a uint8 tensor on the same device")
    _set_strides(cfg, dict(q=q, k=k, v=v, out=out))
    ws = _workspace(fa_fwd_workspace_size(cfg), dev, workspace)
    st = lib().fa_fwd(cfg.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(drop_mask), _ptr(alibi_slopes), _ptr(sink),
                      _ptr(out), _ptr(softmax_max), _ptr(softmax_sum), _ptr(ws),
                      ctypes.c_uint64(ws.numel()), _stream_handle(dev))
    _check(st, "fa_fwd")
    return out, softmax_max, softmax_sum


def fa_bwd(cfg: Config, q, k, v, dy, out, softmax_max, softmax_sum, drop_mask=None, alibi_slopes=None, sink=None,
           dq=None, dk=None, dv=None, dsink=None, workspace=None):
    """Backward through libfa.so on the current stream; returns (dq, dk, dv, dsink or None)."""
    dev, tq, tkv, nq, nkv, d = _common_checks(q, k, v, cfg)
    _check_tensor("dy", dy, layout_shape(cfg, True, True), q.dtype, dev, cfg.layout_name == "TND")
    _check_tensor("out", out, layout_shape(cfg, True, True), q.dtype, dev, cfg.layout_name == "TND")
    _check_tensor("softmax_max", softmax_max, (tq, nq), torch.float32, dev)
    _check_tensor("softmax_sum", softmax_sum, (tq, nq), torch.float32, dev)
    _check_slopes_sink(cfg, alibi_slopes, sink, nq, dev)
    if dq is None:
        dq = torch.empty(layout_shape(cfg, True), dtype=q.dtype, device=dev)
    if dk is None:
        dk = torch.empty(layout_shape(cfg, False), dtype=q.dtype, device=dev)
    if dv is None:
        dv = torch.empty(layout_shape(cfg, False, True), dtype=q.dtype, device=dev)
    if sink is not None and dsink is None:
        dsink = torch.empty((nq,), dtype=torch.float32, device=dev)
    tnd = cfg.layout_name == "TND"
    _check_tensor("dq", dq, layout_shape(cfg, True), q.dtype, dev, tnd)
    _check_tensor("dk", dk, layout_shape(cfg, False), q.dtype, dev, tnd)
    _check_tensor("dv", dv, layout_shape(cfg, False, True), q.dtype, dev, tnd)
    _set_strides(cfg, dict(q=q, k=k, v=v, dy=dy, out=out, dq=dq, dk=dk, dv=dv))
    ws = _workspace(fa_bwd_workspace_size(cfg), dev, workspace)
    st = lib().fa_bwd(cfg.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(dy), _ptr(out), _ptr(softmax_max),
                      _ptr(softmax_sum), _ptr(drop_mask), _ptr(alibi_slopes), _ptr(sink), _ptr(dq), _ptr(dk),
                      _ptr(dv), _ptr(dsink), _ptr(ws), ctypes.c_uint64(ws.numel()), _stream_handle(dev))
    _check(st, "fa_bwd")
    return dq, dk, dv, dsink


def fa_debug_schedule(cfg: Config, pass_id: int):
    """Host-side work list of a pass: (items [n, 4] int64, (tile_rows, tile_cols))."""
    n = ctypes.c_int64(0)
    br, bc = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().fa_debug_schedule(cfg.ref, int(pass_id), None, 0, ctypes.byref(n), ctypes.byref(br),
                                   ctypes.byref(bc)), "fa_debug_schedule")
    items = np.zeros((n.value, 4), dtype=np.int64)
    _check(lib().fa_debug_schedule(cfg.ref, int(pass_id), items.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   n.value, ctypes.byref(n), None, None), "fa_debug_schedule")
    return items, (br.value, bc.value)


def fa_profile_enable(on: bool):
    _check(lib().fa_profile_enable(1 if on else 0), "fa_profile_enable")


def fa_profile_read() -> dict:
    """{kernel name: (total_ms, launches)} since the last read; synchronises the recorded events."""
    res = {}
    for k in range(lib().fa_profile_kernel_count()):
        name = ctypes.c_char_p()
        ms = ctypes.c_double(0)
        cnt = ctypes.c_int64(0)
        _check(lib().fa_profile_read(k, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(cnt)), "fa_profile_read")
        res[name.value.decode()] = (ms.value, cnt.value)
    return res


_LAYOUTS = {"TND": FA_LAYOUT_TND, "BSH": FA_LAYOUT_BSH, "BSND": FA_LAYOUT_BSND, "BNSD": FA_LAYOUT_BNSD,
            "SBH": FA_LAYOUT_SBH}


class DecodeConfig:
    """Owns the host actual_seq_lengths array for the lifetime of a fa_decode_config.
    layout: "BSH", "BSND" or "BNSD" (inputLayout); atten_mask: device bool / uint8 [B, S] or None."""

    def __init__(self, batch, max_seq_len, num_heads, num_kv_heads, head_dim, dtype, scale, layout="BSND",
                 actual_seq_lengths=None, atten_mask=None):
        self.lens = None if actual_seq_lengths is None else np.ascontiguousarray(
            np.asarray(actual_seq_lengths, dtype=np.int64))
        if self.lens is not None and self.lens.shape != (int(batch),):
            raise ValueError("actual_seq_lengths must hold one length per sequence")
        self.atten_mask = atten_mask
        if atten_mask is not None:
            if (atten_mask.dim() != 2 or tuple(atten_mask.shape) != (int(batch), int(max_seq_len))
                    or atten_mask.dtype not in (torch.uint8, torch.bool) or not atten_mask.is_contiguous()):
                raise ValueError("atten_mask must be a contiguous bool or uint8 tensor [B, S]")
        if isinstance(dtype, torch.dtype):
            dtype = {torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_FP16}.get(dtype, -1)
        self.layout_name = layout
        self.c = FaDecodeConfig(
            batch=int(batch), max_seq_len=int(max_seq_len),
            actual_seq_lengths=(None if self.lens is None else self.lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
            num_heads=int(num_heads), num_kv_heads=int(num_kv_heads), head_dim=int(head_dim), dtype=int(dtype),
            layout=_LAYOUTS.get(layout, -1), scale=float(scale),
            atten_mask=(None if atten_mask is None else atten_mask.data_ptr()), flags=0)

    @property
    def ref(self):
        return ctypes.byref(self.c)

    def kv_shape(self):
        b, s, nkv, d = self.c.batch, self.c.max_seq_len, self.c.num_kv_heads or self.c.num_heads, self.c.head_dim
        return {"BSH": (b, s, nkv * d), "BSND": (b, s, nkv, d), "BNSD": (b, nkv, s, d)}[self.layout_name]


def fa_decode_workspace_size(cfg: DecodeConfig) -> int:
    n = ctypes.c_uint64(0)
    _check(lib().fa_decode_workspace_size(cfg.ref, ctypes.byref(n)), "fa_decode_workspace_size")
    return n.value


def _decode_checks(cfg: DecodeConfig, q, k, v, out):
    dev = q.device
    c = cfg.c
    qshape = (c.batch, c.num_heads, c.head_dim)
    if q.numel() != c.batch * c.num_heads * c.head_dim or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous tensor of {qshape} elements")
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, cfg.kv_shape(), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, tuple(q.shape), q.dtype, dev)
    return dev, out


def fa_decode_noalloc(cfg: DecodeConfig, q, k, v, out):
    """Allocation-free decode through libfa.so on the current stream: the library's static
    scratch replaces the workspace, and `out` must be given (nothing is allocated)."""
    if out is None:
        raise ValueError("fa_decode_noalloc writes into a caller-owned out tensor")
    dev, out = _decode_checks(cfg, q, k, v, out)
    _check(lib().fa_decode_noalloc(cfg.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _stream_handle(dev)),
           "fa_decode_noalloc")
    return out


def fa_decode(cfg: DecodeConfig, q, k, v, out=None, workspace=None):
    """Decode attention through libfa.so on the current stream; q, out [B, Nq, D]
    (any view of those elements, e.g. [B, 1, Nq*D]), k, v in cfg's layout.  Returns out."""
    dev, out = _decode_checks(cfg, q, k, v, out)
    ws = _workspace(fa_decode_workspace_size(cfg), dev, workspace)
    st = lib().fa_decode(cfg.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws), ctypes.c_uint64(ws.numel()),
                         _stream_handle(dev))
    _check(st, "fa_decode")
    return out
