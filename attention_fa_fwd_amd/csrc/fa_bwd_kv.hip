// Deterministic dK/dV kernels (see fa_bwd_kv.h) and the launch dispatcher.
#include "fa_bwd_kv.h"

namespace fa {

template <typename T, int D>
static hipError_t launch_kv_t(const BwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_kv_items * p.nkv;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
  return with_flags(p.use_dropout != 0, pse_kind(p), p.mbits != nullptr, [&](auto dr, auto al, auto mk) {
    hipLaunchKernelGGL((fa_bwd_kv_kernel<T, D, false, decltype(dr)::value, decltype(al)::value, decltype(mk)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

// 16-bit dK/dV: producer / consumer waves
template <typename E, int D>
static hipError_t launch_kv_spec(const BwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_kv_items * p.nkv;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(512);
  return with_flags<false>(p.use_dropout != 0, pse_kind(p), p.mbits != nullptr, [&](auto dr, auto al, auto mk) {
    hipLaunchKernelGGL((fa_bwd_kv_spec_kernel<E, D, decltype(dr)::value, decltype(al)::value, decltype(mk)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

// 16-bit dK/dV without dropout, attenMask or pse: two producers and two consumers per SIMD
template <typename E, int D>
static hipError_t launch_kv_16(const BwdParams& p, hipStream_t s) {
  if (p.use_dropout != 0 || pse_kind(p) != kPseNone || p.mbits != nullptr) return launch_kv_spec<E, D>(p, s);
  const int64_t blocks = (int64_t)p.n_kv_items * p.nkv;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((fa_bwd_kv_quad_kernel<E, D>), dim3((unsigned)blocks), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(int dtype, int d, bool atomic_dq, const BwdParams& p, hipStream_t s) {
  if (atomic_dq) return launch_bwd_kv_atomic(dtype, d, p, s);
  if (dtype == 1 && d == 128) return launch_kv_16<__bf16, 128>(p, s);
  if (dtype == 1 && d == 64) return launch_kv_16<__bf16, 64>(p, s);
  if (dtype == 2 && d == 128) return launch_kv_16<_Float16, 128>(p, s);
  if (dtype == 2 && d == 64) return launch_kv_16<_Float16, 64>(p, s);
  if (dtype == 0 && d == 128) return launch_kv_t<float, 128>(p, s);
  if (dtype == 0 && d == 64) return launch_kv_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
