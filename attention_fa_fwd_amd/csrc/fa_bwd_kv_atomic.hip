// dK/dV kernels with atomic dQ accumulation (see fa_bwd_kv.h).
#include "fa_bwd_kv.h"

namespace fa {

template <typename T, int D, bool ATOMIC>
static hipError_t launch_kv_t(const BwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_kv_items * p.nkv;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
  // no alibi instance of the atomic 16-bit D = 128 kernel (see launch_bwd_kv)
  constexpr bool kAlibi = !(ATOMIC && sizeof(T) == 2 && D == 128);
  if (!kAlibi && (p.slopes != nullptr || p.pse != nullptr)) return hipErrorInvalidValue;
  // no attenMask instances: the host routes masked problems to the deterministic passes
  if (p.mbits != nullptr) return hipErrorInvalidValue;
  const int pse = kAlibi ? pse_kind(p) : kPseNone;
  return with_flags<sizeof(T) == 4>(p.use_dropout != 0, pse, false, [&](auto dr, auto al, auto mk) {
    constexpr int AL = kAlibi ? decltype(al)::value : kPseNone;
    hipLaunchKernelGGL((fa_bwd_kv_kernel<T, D, ATOMIC, decltype(dr)::value, AL, false>), grid, block, 0, s, p);
    return hipGetLastError();
  });
}

hipError_t launch_bwd_kv_atomic(int dtype, int d, const BwdParams& p, hipStream_t s) {
  // 16-bit D = 128 with alibi runs the deterministic passes (the host routes it)
  if (dtype == 1 && d == 128 && p.slopes == nullptr) return launch_kv_t<__bf16, 128, true>(p, s);
  if (dtype == 1 && d == 64) return launch_kv_t<__bf16, 64, true>(p, s);
  if (dtype == 2 && d == 128 && p.slopes == nullptr) return launch_kv_t<_Float16, 128, true>(p, s);
  if (dtype == 2 && d == 64) return launch_kv_t<_Float16, 64, true>(p, s);
  // fp32 with D = 128 would need more LDS than a CU has; the host runs the
  // deterministic passes for it instead
  if (dtype == 0 && d == 64) return launch_kv_t<float, 64, true>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
