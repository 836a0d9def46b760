// Head dims above 128 (up to 512): the forward and backward of
// aclnnFlashAttentionScoreV2 / aclnnFlashAttentionUnpaddingScoreGrad ("Formula")
// with the scores of a chunk of query rows materialised in the workspace.
//
// The fused kernels keep a wave's Q (or K, V) rows and its O (or dK, dV, dQ) in
// registers, which stops fitting beyond D = 128.  For larger head dims the path
// runs, per (sequence, kv head, chunk of R query rows) and over the G query heads
// of the group:
//   forward   S = Q K^T (MFMA GEMM, fp32) -> masked softmax (m, l, P~ in the input
//             type) -> O = P~ V (GEMM)
//   backward  S = Q K^T, dP = dY V^T (GEMMs) -> P, P~, dS (kernel, input type)
//             -> dQ = scale dS K (GEMM, whole key range, written once)
//             -> dV += P~^T dY_h, dK += scale dS^T Q_h (GEMMs into fp32 accumulators,
//             head by head and chunk by chunk in a fixed order) -> dK, dV
// D_i, lse2 and the dSink partials come from a row-dot kernel for any head dim.
// Every step is a fixed-order computation: bitwise reproducible.  The rounding
// points match the fused kernels (P~ and dS in the input type, fp32 accumulation).
#include <algorithm>
#include <cstring>
#include <vector>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

// ------------------------------------------------------------------ batched GEMM
// C[z][m][n] = alpha * sum_k A[z][m][k] B[z][k][n] (+ C[z][m][n] when accumulating,
// fp32 C only).  Arbitrary element strides, so transposes and TND rows need no
// copies.  One workgroup (4 waves) per 64 x 64 tile of C, each wave a 32 x 32 block;
// k advances 32 at a time through LDS (operands stored k-contiguous per row of
// A and per column of B, the layout of the MFMA operands).
struct GemmDesc {
  const void* a;
  const void* b;
  void* c;
  int32_t m, n, k, batch;
  int64_t a_sm, a_sk, a_sz;
  int64_t b_sk, b_sn, b_sz;
  int64_t c_sm, c_sn, c_sz;
  float alpha;
  int32_t accumulate;
};

constexpr int kGemmTile = 64, kGemmK = 32;

template <typename T>
__device__ __forceinline__ float load_f32(const T* p) {
  if constexpr (sizeof(T) == 2) return (float)*p;
  else return *p;
}

template <typename T>
__device__ __forceinline__ T from_f32(float v) {
  if constexpr (sizeof(T) == 2) return cvt16<T>(v);
  else return v;
}

template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void fa_gemm_kernel(GemmDesc g) {
  // k-contiguous rows of 32 elements, padded by 16 bytes against bank conflicts
  constexpr int PITCH = kGemmK + 16 / (int)sizeof(Tin);
  __shared__ __attribute__((aligned(16))) Tin as[kGemmTile * PITCH];
  __shared__ __attribute__((aligned(16))) Tin bs[kGemmTile * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * kGemmTile, m0 = blockIdx.y * kGemmTile, z = blockIdx.z;
  const Tin* A = reinterpret_cast<const Tin*>(g.a) + (int64_t)z * g.a_sz;
  const Tin* B = reinterpret_cast<const Tin*>(g.b) + (int64_t)z * g.b_sz;
  const int wm = 32 * (wave & 1), wn = 32 * (wave >> 1);
  // element e of a tile: along k when k is the contiguous dimension, else along m / n
  const bool a_kfast = g.a_sk == 1, b_kfast = g.b_sk == 1;
  f32x16 acc = {};
  for (int k0 = 0; k0 < g.k; k0 += kGemmK) {
    Tin ra[8], rb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      const int am = a_kfast ? e / kGemmK : e % kGemmTile, ak = a_kfast ? e % kGemmK : e / kGemmTile;
      const int bn = b_kfast ? e / kGemmK : e % kGemmTile, bk = b_kfast ? e % kGemmK : e / kGemmTile;
      const bool aok = m0 + am < g.m && k0 + ak < g.k, bok = n0 + bn < g.n && k0 + bk < g.k;
      ra[u] = aok ? A[(int64_t)(m0 + am) * g.a_sm + (int64_t)(k0 + ak) * g.a_sk] : Tin{};
      rb[u] = bok ? B[(int64_t)(k0 + bk) * g.b_sk + (int64_t)(n0 + bn) * g.b_sn] : Tin{};
    }
    __syncthreads();   // the previous step's operands are read
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      const int am = a_kfast ? e / kGemmK : e % kGemmTile, ak = a_kfast ? e % kGemmK : e / kGemmTile;
      const int bn = b_kfast ? e / kGemmK : e % kGemmTile, bk = b_kfast ? e % kGemmK : e / kGemmTile;
      as[am * PITCH + ak] = ra[u];
      bs[bn * PITCH + bk] = rb[u];
    }
    __syncthreads();
    if constexpr (sizeof(Tin) == 2) {
      using V8 = typename Vec16<Tin>::v8;
#pragma unroll
      for (int kc = 0; kc < kGemmK / 16; ++kc) {
        const int kk = 16 * kc + 8 * (lane >> 5);
        const V8 av = *reinterpret_cast<const V8*>(&as[(wm + (lane & 31)) * PITCH + kk]);
        const V8 bv = *reinterpret_cast<const V8*>(&bs[(wn + (lane & 31)) * PITCH + kk]);
        acc = mfma32(av, bv, acc);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < kGemmK / 2; ++kc) {
        const int kk = 2 * kc + (lane >> 5);
        acc = mfma32(as[(wm + (lane & 31)) * PITCH + kk], bs[(wn + (lane & 31)) * PITCH + kk], acc);
      }
    }
  }
  // lane holds column n = lane % 32 and rows 8 (r / 4) + 4 (lane / 32) + r % 4 of its block
  Tout* C = reinterpret_cast<Tout*>(g.c) + (int64_t)z * g.c_sz;
  const int n = n0 + wn + (lane & 31);
  if (n < g.n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m < g.m) {
        Tout* cp = C + (int64_t)m * g.c_sm + (int64_t)n * g.c_sn;
        float v = g.alpha * acc[r];
        if constexpr (sizeof(Tout) == 4) {
          if (g.accumulate) v += *cp;
        }
        *cp = from_f32<Tout>(v);
      }
    }
  }
}

template <typename Tin, typename Tout>
static hipError_t gemm(const GemmDesc& g, hipStream_t s) {
  if (g.m <= 0 || g.n <= 0 || g.batch <= 0) return hipSuccess;
  const dim3 grid((unsigned)((g.n + kGemmTile - 1) / kGemmTile), (unsigned)((g.m + kGemmTile - 1) / kGemmTile),
                  (unsigned)g.batch);
  hipLaunchKernelGGL((fa_gemm_kernel<Tin, Tout>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

// ------------------------------------------------------------------ logits
// Logit of local row i, key j of (sequence b, query head h) in the log2 domain:
// scale * s * log2(e) plus the position bias, or -inf outside the mask.
template <typename T, typename P>
__device__ __forceinline__ float large_logit(const P& p, const FaWindow& win, int pse, int b, int h, int i, int j,
                                            int lq, int lkv, float s, float slope_l2, int poff) {
  if (!fa_allowed(win, i, j, lq, lkv)) return kNegInf;
  if (p.mbits && ((p.mbits[(int64_t)i * p.mwords + (j >> 5)] >> (j & 31)) & 1u)) return kNegInf;
  float x = s * p.scale_log2;
  if (pse == kPseExt) x = __builtin_fmaf(p.pse_coef, pse_value<T>(p, b, h, i, j, lq), x);
  else if (pse == kPseLinear) x = add_pse<kPseLinear>(x, slope_l2, (float)(j - i - poff));
  else if (pse == kPseSqrt) x = add_pse<kPseSqrt>(x, slope_l2, (float)(j - i - poff));
  return x;
}

template <typename P>
__device__ __forceinline__ bool keep_bit(const P& p, int b, int h, int i, int j, int lq, int lkv) {
  if (!p.drop) return true;
  const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + i) * lkv + j;
  return (p.drop[pos >> 3] >> (pos & 7)) & 1u;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Chunk of R query rows of sequence b (rows r0 ..) for the G heads of kv head g.
struct LargeChunk {
  int32_t b, g, r0, rows, lq, lkv, q0, k0;
};

// Forward softmax: one wave per (head of the group, row).  S [G][R][lkv] fp32 ->
// P~ [G][R][lkv] (input type; P / l with dropout applied), softmax max / sum.
template <typename T>
__global__ __launch_bounds__(256) void fa_large_softmax_kernel(FwdParams p, LargeChunk c, const float* S, T* Pt) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= p.group * c.rows) return;
  const int hh = wid / c.rows, r = wid - hh * c.rows;
  const int h = c.g * p.group + hh, i = c.r0 + r, b = c.b;
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, c.lq, c.lkv, p.prefix[b]);
  const int pse = pse_kind(p);
  const float slope_l2 = (pse == kPseLinear || pse == kPseSqrt) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
  const int poff = b == 0 ? p.pse_off0 : 0;
  const float* srow = S + ((int64_t)hh * c.rows + r) * c.lkv;
  T* prow = Pt + ((int64_t)hh * c.rows + r) * c.lkv;
  const float sink2 = p.sink ? p.sink[h] * kLog2e : kNegInf;
  float mx = kNegInf;
  for (int j = lane; j < c.lkv; j += 64)
    mx = fmaxf(mx, large_logit<T>(p, win, pse, b, h, i, j, c.lq, c.lkv, srow[j], slope_l2, poff));
  mx = fmaxf(wave_max(mx), sink2);
  const float mu = mx == kNegInf ? 0.f : mx;
  float l = 0.f;
  for (int j = lane; j < c.lkv; j += 64)
    l += fast_exp2(large_logit<T>(p, win, pse, b, h, i, j, c.lq, c.lkv, srow[j], slope_l2, poff) - mu);
  l = wave_sum(l) + (p.sink ? fast_exp2(sink2 - mu) : 0.f);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int j = lane; j < c.lkv; j += 64) {
    const float e = fast_exp2(large_logit<T>(p, win, pse, b, h, i, j, c.lq, c.lkv, srow[j], slope_l2, poff) - mu);
    const bool keep = keep_bit(p, b, h, i, j, c.lq, c.lkv);
    prow[j] = from_f32<T>(keep ? e * inv * p.inv_keep : 0.f);
  }
  if (lane == 0) {
    const int64_t idx = (int64_t)(c.q0 + i) * p.nq + h;
    p.m_out[idx] = mx * kLn2;
    p.l_out[idx] = l;
  }
}

// Backward: one wave per (head of the group, row).  S, dP [G][R][lkv] fp32 ->
// P~ and dS [G][R][lkv] in the input type:
//   P = 2^(x - lse2), P~ = P z / keep, dS = P (dP z / keep - D_i).
template <typename T>
__global__ __launch_bounds__(256) void fa_large_ds_kernel(BwdParams p, LargeChunk c, const float* S, const float* dP,
                                                         T* Pt, T* dS) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= p.group * c.rows) return;
  const int hh = wid / c.rows, r = wid - hh * c.rows;
  const int h = c.g * p.group + hh, i = c.r0 + r, b = c.b;
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, c.lq, c.lkv, p.prefix[b]);
  const int pse = pse_kind(p);
  const float slope_l2 = (pse == kPseLinear || pse == kPseSqrt) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
  const int poff = b == 0 ? p.pse_off0 : 0;
  const int64_t idx = (int64_t)(c.q0 + i) * p.nq + h;
  const float lse2 = p.lse[idx], di = p.delta[idx];
  const int64_t o = ((int64_t)hh * c.rows + r) * c.lkv;
  for (int j = lane; j < c.lkv; j += 64) {
    const float x = large_logit<T>(p, win, pse, b, h, i, j, c.lq, c.lkv, S[o + j], slope_l2, poff);
    const float pr = fast_exp2(x - lse2);   // 0 for masked keys and for rows without any (lse2 = +inf)
    const bool keep = keep_bit(p, b, h, i, j, c.lq, c.lkv);
    const float dpv = keep ? dP[o + j] * p.inv_keep : 0.f;
    Pt[o + j] = from_f32<T>(keep ? pr * p.inv_keep : 0.f);
    dS[o + j] = from_f32<T>(pr * (dpv - di));
  }
}

// D_i = rowsum(dY * O), lse2 = m log2(e) + log2(l) (+inf for empty rows) and the
// per-block dSink partials, for any head dim: one wave per (row, head) of a block of
// kPreRowsPerBlock rows; the partials are summed over the block's rows in order.
template <typename T>
__global__ __launch_bounds__(256) void fa_large_pre_kernel(BwdParams p, int d) {
  extern __shared__ float contrib[];   // [kPreRowsPerBlock][nq]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * kPreRowsPerBlock;
  const int rows = (int)min((int64_t)kPreRowsPerBlock, (int64_t)p.total_q - row0);
  const int nq = p.nq;
  for (int pi = wave; pi < rows * nq; pi += 4) {
    const int r = pi / nq, h = pi - r * nq;
    const int64_t idx = (row0 + r) * nq + h;
    const T* dy = reinterpret_cast<const T*>(p.dy) + idx * d;
    const T* o = reinterpret_cast<const T*>(p.o) + idx * d;
    float acc = 0.f;
    for (int x = lane; x < d; x += 64) acc += load_f32(dy + x) * load_f32(o + x);
    acc = wave_sum(acc);
    if (lane == 0) {
      const float m = p.m_in[idx], l = p.l_in[idx];
      p.delta[idx] = acc;
      p.lse[idx] = l > 0.f ? m * kLog2e + __log2f(l) : __builtin_inff();
      contrib[r * nq + h] = (p.sink && l > 0.f) ? -fast_exp2((p.sink[h] - m) * kLog2e) / l * acc : 0.f;
    }
  }
  if (p.sink) {
    __syncthreads();
    for (int h = threadIdx.x; h < nq; h += 256) {
      float s = 0.f;
      for (int r = 0; r < rows; ++r) s += contrib[r * nq + h];
      p.dsink_part[(int64_t)blockIdx.x * nq + h] = s;
    }
  }
}

// fp32 accumulator [lkv][d] -> rows k0 .. of kv head g of a [T_kv, Nkv, d] tensor
template <typename T>
__global__ __launch_bounds__(256) void fa_large_store_kernel(const float* acc, T* out, int64_t rows, int d, int nkv,
                                                            int g, int64_t k0) {
  const int64_t n = rows * d;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) {
    const int64_t j = x / d, e = x - j * d;
    out[((k0 + j) * nkv + g) * d + e] = from_f32<T>(acc[x]);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void fa_large_zero_kernel(T* p, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) p[x] = T{};
}

static unsigned blocks_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 8192));
}

// ------------------------------------------------------------------ host drivers
template <typename T>
static hipError_t large_fwd_t(const FwdParams& p, const LargePlan& L, char* ws, hipStream_t s) {
  const int G = p.group, d = L.d;
  float* S = reinterpret_cast<float*>(ws + L.off_s);
  T* Pt = reinterpret_cast<T*>(ws + L.off_p);
  hipError_t e = hipSuccess;
  for (int b = 0; b < L.batch && e == hipSuccess; ++b) {
    const int lq = L.cu_q[b + 1] - L.cu_q[b], lkv = L.cu_kv[b + 1] - L.cu_kv[b];
    for (int g = 0; g < p.nkv && e == hipSuccess; ++g)
      for (int r0 = 0; r0 < lq && e == hipSuccess; r0 += L.rows) {
        const LargeChunk c{b, g, r0, std::min(L.rows, lq - r0), lq, lkv, L.cu_q[b], L.cu_kv[b]};
        const T* q = reinterpret_cast<const T*>(p.q) + ((int64_t)(c.q0 + r0) * p.nq + g * G) * d;
        const T* k = reinterpret_cast<const T*>(p.k) + ((int64_t)c.k0 * p.nkv + g) * d;
        const T* v = reinterpret_cast<const T*>(p.v) + ((int64_t)c.k0 * p.nkv + g) * d;
        T* o = reinterpret_cast<T*>(p.o) + ((int64_t)(c.q0 + r0) * p.nq + g * G) * d;
        const int64_t sz = (int64_t)c.rows * lkv;
        // S[hh][r][j] = Q[r, hh] . K[j]
        GemmDesc gs{q, k, S, c.rows, lkv, d, G, (int64_t)p.nq * d, 1, d, 1, (int64_t)p.nkv * d, 0, lkv, 1, sz, 1.f, 0};
        e = gemm<T, float>(gs, s);
        if (e != hipSuccess) break;
        hipLaunchKernelGGL((fa_large_softmax_kernel<T>), dim3((unsigned)((G * c.rows + 3) / 4)), dim3(256), 0, s, p, c,
                           S, Pt);
        e = hipGetLastError();
        if (e != hipSuccess) break;
        // O[r, hh] = P~[hh][r] V
        GemmDesc go{Pt, v, o, c.rows, d, lkv, G, lkv, 1, sz, (int64_t)p.nkv * d, 1, 0, (int64_t)p.nq * d, 1, d, 1.f, 0};
        e = gemm<T, T>(go, s);
      }
  }
  return e;
}

template <typename T>
static hipError_t large_bwd_t(const BwdParams& p, const LargePlan& L, char* ws, hipStream_t s) {
  const int G = p.group, d = L.d;
  float* S = reinterpret_cast<float*>(ws + L.off_s);
  float* dP = reinterpret_cast<float*>(ws + L.off_dp);
  T* Pt = reinterpret_cast<T*>(ws + L.off_p);
  T* dS = reinterpret_cast<T*>(ws + L.off_ds);
  float* dk_acc = reinterpret_cast<float*>(ws + L.off_dk);
  float* dv_acc = reinterpret_cast<float*>(ws + L.off_dv);
  hipError_t e = hipSuccess;
  if (p.n_pre_blocks > 0) {
    hipLaunchKernelGGL((fa_large_pre_kernel<T>), dim3((unsigned)p.n_pre_blocks), dim3(256),
                       sizeof(float) * kPreRowsPerBlock * p.nq, s, p, d);
    e = hipGetLastError();
  }
  for (int b = 0; b < L.batch && e == hipSuccess; ++b) {
    const int lq = L.cu_q[b + 1] - L.cu_q[b], lkv = L.cu_kv[b + 1] - L.cu_kv[b];
    if (lkv == 0) {
      // no keys: the sequence's dQ rows are zero (and it has no dK / dV rows)
      const int64_t n = (int64_t)lq * p.nq * d;
      if (n > 0) {
        hipLaunchKernelGGL((fa_large_zero_kernel<T>), dim3(blocks_for(n)), dim3(256), 0, s,
                           reinterpret_cast<T*>(p.dq) + (int64_t)L.cu_q[b] * p.nq * d, n);
        e = hipGetLastError();
      }
      continue;
    }
    for (int g = 0; g < p.nkv && e == hipSuccess; ++g) {
      const int64_t kn = (int64_t)lkv * d;
      hipLaunchKernelGGL(fa_large_zero_kernel<float>, dim3(blocks_for(kn)), dim3(256), 0, s, dk_acc, kn);
      hipLaunchKernelGGL(fa_large_zero_kernel<float>, dim3(blocks_for(kn)), dim3(256), 0, s, dv_acc, kn);
      e = hipGetLastError();
      const int q0 = L.cu_q[b], k0 = L.cu_kv[b];
      const T* k = reinterpret_cast<const T*>(p.k) + ((int64_t)k0 * p.nkv + g) * d;
      const T* v = reinterpret_cast<const T*>(p.v) + ((int64_t)k0 * p.nkv + g) * d;
      for (int r0 = 0; r0 < lq && e == hipSuccess; r0 += L.rows) {
        const LargeChunk c{b, g, r0, std::min(L.rows, lq - r0), lq, lkv, q0, k0};
        const int64_t qrow = ((int64_t)(q0 + r0) * p.nq + g * G) * d;
        const T* q = reinterpret_cast<const T*>(p.q) + qrow;
        const T* dy = reinterpret_cast<const T*>(p.dy) + qrow;
        T* dq = reinterpret_cast<T*>(p.dq) + qrow;
        const int64_t sz = (int64_t)c.rows * lkv, qs = (int64_t)p.nq * d, ks = (int64_t)p.nkv * d;
        GemmDesc gs{q, k, S, c.rows, lkv, d, G, qs, 1, d, 1, ks, 0, lkv, 1, sz, 1.f, 0};
        GemmDesc gp{dy, v, dP, c.rows, lkv, d, G, qs, 1, d, 1, ks, 0, lkv, 1, sz, 1.f, 0};
        if ((e = gemm<T, float>(gs, s)) != hipSuccess || (e = gemm<T, float>(gp, s)) != hipSuccess) break;
        hipLaunchKernelGGL((fa_large_ds_kernel<T>), dim3((unsigned)((G * c.rows + 3) / 4)), dim3(256), 0, s, p, c, S,
                           dP, Pt, dS);
        if ((e = hipGetLastError()) != hipSuccess) break;
        // dQ[r, hh] = scale dS[hh][r] K over the whole key range
        GemmDesc gq{dS, k, dq, c.rows, d, lkv, G, lkv, 1, sz, ks, 1, 0, qs, 1, d, p.scale, 0};
        if ((e = gemm<T, T>(gq, s)) != hipSuccess) break;
        // dV += P~[hh]^T dY[., hh], dK += scale dS[hh]^T Q[., hh], heads in order
        for (int hh = 0; hh < G && e == hipSuccess; ++hh) {
          GemmDesc gv{Pt + hh * sz, dy + (int64_t)hh * d, dv_acc, lkv, d, c.rows, 1, 1, lkv, 0, qs, 1, 0, d, 1, 0,
                      1.f, 1};
          GemmDesc gk{dS + hh * sz, q + (int64_t)hh * d, dk_acc, lkv, d, c.rows, 1, 1, lkv, 0, qs, 1, 0, d, 1, 0,
                      p.scale, 1};
          if ((e = gemm<T, float>(gv, s)) == hipSuccess) e = gemm<T, float>(gk, s);
        }
      }
      if (e != hipSuccess) break;
      hipLaunchKernelGGL((fa_large_store_kernel<T>), dim3(blocks_for(kn)), dim3(256), 0, s, dk_acc,
                         reinterpret_cast<T*>(p.dk), (int64_t)lkv, d, p.nkv, g, (int64_t)k0);
      hipLaunchKernelGGL((fa_large_store_kernel<T>), dim3(blocks_for(kn)), dim3(256), 0, s, dv_acc,
                         reinterpret_cast<T*>(p.dv), (int64_t)lkv, d, p.nkv, g, (int64_t)k0);
      e = hipGetLastError();
    }
  }
  return e;
}

hipError_t launch_large_fwd(int dtype, const FwdParams& p, const LargePlan& L, char* ws, hipStream_t s) {
  if (dtype == 1) return large_fwd_t<__bf16>(p, L, ws, s);
  if (dtype == 2) return large_fwd_t<_Float16>(p, L, ws, s);
  if (dtype == 0) return large_fwd_t<float>(p, L, ws, s);
  return hipErrorInvalidValue;
}

hipError_t launch_large_bwd(int dtype, const BwdParams& p, const LargePlan& L, char* ws, hipStream_t s) {
  if (dtype == 1) return large_bwd_t<__bf16>(p, L, ws, s);
  if (dtype == 2) return large_bwd_t<_Float16>(p, L, ws, s);
  if (dtype == 0) return large_bwd_t<float>(p, L, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
