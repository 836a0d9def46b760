// Deterministic dK/dV kernels (see fa_bwd_kv.h) and the launch dispatcher.
#include "fa_bwd_kv.h"

namespace fa {

template <typename T, int D, bool ATOMIC>
static hipError_t launch_kv_t(const BwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_kv_items * p.nkv;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
  const bool drop = p.use_dropout != 0, alibi = p.slopes != nullptr;
  // no alibi instance of the atomic bf16 D = 128 kernel (see launch_bwd_kv)
  constexpr bool kAlibi = !(ATOMIC && sizeof(T) == 2 && D == 128);
  if (alibi && !kAlibi) return hipErrorInvalidValue;
  if (drop && alibi)
    hipLaunchKernelGGL((fa_bwd_kv_kernel<T, D, ATOMIC, true, kAlibi>), grid, block, 0, s, p);
  else if (drop)
    hipLaunchKernelGGL((fa_bwd_kv_kernel<T, D, ATOMIC, true, false>), grid, block, 0, s, p);
  else if (alibi)
    hipLaunchKernelGGL((fa_bwd_kv_kernel<T, D, ATOMIC, false, kAlibi>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fa_bwd_kv_kernel<T, D, ATOMIC, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_kv_pair(const BwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_kv_items * p.nkv;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(512);
  const bool drop = p.use_dropout != 0, alibi = p.slopes != nullptr;
  if (drop && alibi)
    hipLaunchKernelGGL((fa_bwd_kv_pair_kernel<D, true, true>), grid, block, 0, s, p);
  else if (drop)
    hipLaunchKernelGGL((fa_bwd_kv_pair_kernel<D, true, false>), grid, block, 0, s, p);
  else if (alibi)
    hipLaunchKernelGGL((fa_bwd_kv_pair_kernel<D, false, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fa_bwd_kv_pair_kernel<D, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(int dtype, int d, bool atomic_dq, const BwdParams& p, hipStream_t s) {
  if (atomic_dq) return launch_bwd_kv_atomic(dtype, d, p, s);
  if (dtype == 1 && d == 128) return launch_kv_pair<128>(p, s);
  if (dtype == 1 && d == 64) return launch_kv_pair<64>(p, s);
  if (dtype == 0 && d == 128) return launch_kv_t<float, 128, false>(p, s);
  if (dtype == 0 && d == 64) return launch_kv_t<float, 64, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
