"""MI355X-native (gfx950) varlen FlashAttention forward/backward.

The computation lives in libfa.so (hand-written HIP kernels behind the C ABI of
include/fa.h); this package is its thin Python binding.
"""
from ._lib import (EXPORTED, FA_DTYPE_BF16, FA_DTYPE_FP16, FA_DTYPE_FP32, FA_FLAG_PSE_SQRT,
                   FA_FLAG_SLOPES_PER_BATCH, FA_FLAG_ATOMIC_DQ, FA_ERR_HIP, FA_ERR_PARAM_INVALID,
                   FA_ERR_PARAM_NULLPTR, FA_ERR_WORKSPACE, FA_OK, LIB_PATH, TOKENS_DEFAULT, Config, FaError,
                   fa_bwd, fa_bwd_workspace_size, fa_debug_schedule, fa_fwd, fa_fwd_workspace_size,
                   fa_profile_enable, fa_profile_read, lib, status_string, DecodeConfig, fa_decode,
                   fa_decode_workspace_size, fa_decode_noalloc, FA_ERR_SCRATCH,
                   FA_DECODE_NOALLOC_SCRATCH_BYTES, FA_LAYOUT_TND, FA_LAYOUT_BSH, FA_LAYOUT_BSND,
                   FA_LAYOUT_BNSD, FA_LAYOUT_SBH, layout_shape, trace_lib, TRACE_LIB_PATH)

__all__ = ["Config", "FaError", "fa_fwd", "fa_bwd", "fa_fwd_workspace_size", "fa_bwd_workspace_size",
           "fa_debug_schedule", "fa_profile_enable", "fa_profile_read", "lib", "status_string", "EXPORTED",
           "LIB_PATH", "FA_OK", "FA_ERR_PARAM_NULLPTR", "FA_ERR_PARAM_INVALID", "FA_ERR_WORKSPACE", "FA_ERR_HIP",
           "FA_DTYPE_FP32", "FA_DTYPE_BF16", "FA_DTYPE_FP16", "FA_FLAG_PSE_SQRT", "FA_FLAG_SLOPES_PER_BATCH", "FA_FLAG_ATOMIC_DQ",
           "TOKENS_DEFAULT", "DecodeConfig", "fa_decode", "fa_decode_workspace_size", "fa_decode_noalloc",
           "FA_ERR_SCRATCH", "FA_DECODE_NOALLOC_SCRATCH_BYTES", "FA_LAYOUT_TND", "FA_LAYOUT_BSH",
           "FA_LAYOUT_BSND", "FA_LAYOUT_BNSD", "FA_LAYOUT_SBH", "layout_shape", "trace_lib",
           "TRACE_LIB_PATH"]
