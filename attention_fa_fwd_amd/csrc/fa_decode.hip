// Decode attention for gfx950: aclnnIncreFlashAttentionV2 ("Function
// description / formula"): one query token per sequence attends to the first
// L_b keys of a padded KV cache, O = Softmax(scale * q K^T) V, with GQA (the
// query heads of one kv head share its K and V) and an optional per-sequence
// key mask.
//
// The pass streams K and V from HBM once.  One workgroup (kDecWaves = 3 waves)
// takes a key range of one (sequence, kv head); each wave walks its third of the
// range in 32-key blocks through its own three-stage LDS ring, filled by LDS DMA
// two blocks ahead (no barrier inside the loop):
//   S^T (32 keys x 32 query heads) = K Q^T   A = K rows from LDS, B = Q in registers
//   O^T (D x 32 query heads)      += V^T P^T  A = V via the transposing LDS read,
//                                              B = P taken straight from S^T
// The query heads of the group fill the MFMA's row side (zero rows pad a group
// below 32; groups of 33-64 heads take two row blocks against the same K/V
// operands).  The waves' (max, sum, O) merge through LDS; a sequence split
// over several workgroups leaves fp32 partials that fa_decode_reduce_kernel
// combines in a fixed order.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <typename E, int D>
struct DecShape {
  static constexpr int RB = D * 2;                 // bytes per K/V row
  static constexpr int TILE = kDecBlock * RB;      // one K (or V) block, swizzled, unpadded
  static constexpr int STAGE = 2 * TILE;           // K | V
  static constexpr int WAVE_LDS = kDecStages * STAGE;   // the wave's ring
  static constexpr int NQ = D / 16;                // Q operand registers (16-wide d chunks)
  static constexpr int NDB = D / 32;               // 32-wide d blocks of O
  static constexpr int DMA_PER_TILE = TILE / 1024;  // 1 KB LDS copies per K (or V) block
};

// s_waitcnt vmcnt(PER * n) for n in [0, 2]: wait until at most n blocks' copies
// (PER memory instructions each, issued after the awaited block's) are in flight.
template <int PER>
__device__ __forceinline__ void dma_wait_blocks(int n) {
  static_assert(2 * PER <= 63, "vmcnt range");
  if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
}

template <typename E, int D, int NRB, bool MASK>
__global__ __launch_bounds__(64 * kDecWaves, 1) void fa_decode_kernel(DecParams p) {
  using S = DecShape<E, D>;
  using V8 = typename Vec16<E>::v8;
  static_assert(NRB * 32 * D * 4 <= S::WAVE_LDS, "merge buffer fits the wave's ring");
  static_assert(kDecStages >= 2 && kDecStages <= 4, "ring depth");
  __shared__ __attribute__((aligned(16))) char lds[kDecWaves * S::WAVE_LDS];
  __shared__ float mls[2][kDecWaves][32 * NRB];   // per wave and query head: max (log2 domain), sum

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, lrow = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;

  const DecItem it = p.items[blockIdx.x];
  const int b = it.b, g = it.g;
  const int wlo = min(it.lo + wave * p.keys_per_wave, it.hi);
  const int whi = min(wlo + p.keys_per_wave, it.hi);
  const int nblk = (whi - wlo + kDecBlock - 1) / kDecBlock;

  // ---- Q^T operands: lane row = query head 32*rb + lrow of the group ----
  V8 qf[NRB][S::NQ];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int n = 32 * rb + lrow;
    const bool ok = n < p.group;
    const E* qp = reinterpret_cast<const E*>(p.q) + ((int64_t)b * p.nq + g * p.group + (ok ? n : 0)) * D;
#pragma unroll
    for (int c = 0; c < S::NQ; ++c) {
      const V8 v = *reinterpret_cast<const V8*>(qp + 16 * c + 8 * hh);
      qf[rb][c] = ok ? v : V8{};
    }
  }

  float m_run[NRB], l_run[NRB];
  f32x16 o[NRB][S::NDB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) o[rb][db] = f32x16{};
  }

  char* ring = lds + wave * S::WAVE_LDS;
  const int64_t kvoff = ((int64_t)b * p.kv_bstride + (int64_t)g * p.kv_hstride) * 2;
  const char* kbase = reinterpret_cast<const char*>(p.k) + kvoff;
  const char* vbase = reinterpret_cast<const char*>(p.v) + kvoff;
  const int64_t tstride = p.kv_tstride * 2;   // bytes between consecutive keys

  // swizzled tile reads: K chunk 2c + hh of key row lrow; V^T reads of key rows
  // rv and rv + 8 (+16 per 16-key step), chunk 4db + qv
  int koff[S::NQ], voff[2][S::NDB];
#pragma unroll
  for (int c = 0; c < S::NQ; ++c) koff[c] = lrow * S::RB + 16 * ((2 * c + hh) ^ tile_swz<S::RB>(lrow));
  {
    const int rv = 4 * (grp >> 1) + (sl >> 2), qv = 2 * (grp & 1) + ((sl & 3) >> 1), bv = 8 * (sl & 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
        voff[hf][db] = (rv + 8 * hf) * S::RB + 16 * ((4 * db + qv) ^ tile_swz<S::RB>(rv + 8 * hf)) + bv;
  }

  auto copy_block = [&](int t) {
    char* st = ring + (t % kDecStages) * S::STAGE;
    const int c0 = wlo + kDecBlock * t;
    dma_tile_swz<kDecBlock, S::RB, 1>(st, kbase, tstride, c0, whi, 0, lane);
    dma_tile_swz<kDecBlock, S::RB, 1>(st + S::TILE, vbase, tstride, c0, whi, 0, lane);
  };

  const uint8_t* mrow = MASK ? p.mask + (int64_t)b * p.mask_stride : nullptr;
  // blocks run kDecStages - 1 ahead of the one being computed
#pragma unroll
  for (int t = 0; t < kDecStages - 1; ++t)
    if (t < nblk) copy_block(t);
  for (int t = 0; t < nblk; ++t) {
    // block t has landed once at most the copies of the blocks after it are in flight
    // (only this wave reads its ring)
    dma_wait_blocks<2 * S::DMA_PER_TILE>(min(kDecStages - 2, nblk - 1 - t));
    if (t + kDecStages - 1 < nblk) copy_block(t + kDecStages - 1);
    const char* ks = ring + (t % kDecStages) * S::STAGE;
    const char* vs = ks + S::TILE;
    const int c0 = wlo + kDecBlock * t;

    // S^T = K Q^T
    V8 a[S::NQ];
#pragma unroll
    for (int c = 0; c < S::NQ; ++c) a[c] = lds_read_b128<V8>(ks + koff[c]);
    f32x16 s[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      s[rb] = f32x16{};
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) s[rb] = mfma32(a[c], qf[rb][c], s[rb]);
    }

    // keys of this lane's registers: c0 + 8*(r/4) + 4*hh + r%4; masked: beyond the range or by the mask
    uint32_t dead = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = c0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      bool off = j >= whi;
      if constexpr (MASK) off = off || mrow[off ? 0 : j] != 0;
      dead |= (off ? 1u : 0u) << r;
    }

    // online softmax per query head (lanes l and l + 32 share a head)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float mt = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = ((dead >> r) & 1u) ? kNegInf : s[rb][r] * p.scale_log2;
        s[rb][r] = x;
        mt = fmaxf(mt, x);
      }
      mt = half_max(mt);
      const float m_new = fmaxf(m_run[rb], mt);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[rb] - m_use);   // 0 while m_run = -inf
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(s[rb][r] - m_use);
        s[rb][r] = e;
        lsum += e;
      }
      l_run[rb] = l_run[rb] * alpha + lsum;
      m_run[rb] = m_new;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) o[rb][db] *= alpha;
    }

    // O^T += V^T P^T, two 16-key steps
    V8 pb[NRB][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[rb][c2][j] = cvt16<E>(s[rb][8 * c2 + j]);
    V8 av[2][S::NDB];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const char* vrow = vs + (16 * c2) * S::RB;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) av[c2][db] = lds_read_tr_x2<V8>(vrow + voff[0][db], vrow + voff[1][db]);
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) o[rb][db] = mfma32(av[c2][db], pb[rb][c2], o[rb][db]);
  }

  // ---- merge the waves: each writes (max, sum, O) into its own ring ----
  float* ow = reinterpret_cast<float*>(ring);   // [32*NRB heads][D]
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float l_tot = half_sum(l_run[rb]);
    const int n = 32 * rb + lrow;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) ow[n * D + 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3)] = o[rb][db][r];
    if (hh == 0) {
      mls[0][wave][n] = m_run[rb];
      mls[1][wave][n] = l_tot;
    }
  }
  __syncthreads();
  const int rows = min(p.group, 32 * NRB);
  for (int x = tid; x < rows * D; x += 64 * kDecWaves) {
    const int n = x / D, d = x - n * D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, mls[0][w][n]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = mx == kNegInf ? 0.f : fast_exp2(mls[0][w][n] - mx);
      L += mls[1][w][n] * f;
      O += reinterpret_cast<const float*>(lds + w * S::WAVE_LDS)[n * D + d] * f;
    }
    const int h = g * p.group + n;
    if (it.slot < 0) {
      reinterpret_cast<E*>(p.out)[((int64_t)b * p.nq + h) * D + d] = cvt16<E>(L > 0.f ? O / L : 0.f);
    } else {
      const int64_t row = (int64_t)it.slot * p.group + n;
      p.part_o[row * D + d] = O;
      if (d == 0) {
        p.part_m[row] = mx;
        p.part_l[row] = L;
      }
    }
  }
}

// One workgroup of D threads per (sequence, query head) of a split sequence:
// O = sum_c 2^(m_c - m) O_c / sum_c 2^(m_c - m) l_c over its items.  The threads
// share the items for the maximum and the weighted sum of l (fixed-order tree
// sums, so the result is reproducible); then thread d accumulates column d over
// the items in item order, D items' weights at a time staged in LDS, with the
// loads of several items in flight.
template <int D>
__device__ __forceinline__ float block_tree(float* red, float v, bool is_max) {
  const int d = threadIdx.x;
  red[d] = v;
  __syncthreads();
#pragma unroll
  for (int s = D / 2; s > 0; s >>= 1) {
    if (d < s) red[d] = is_max ? fmaxf(red[d], red[d + s]) : red[d] + red[d + s];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

template <typename E, int D>
__global__ __launch_bounds__(D) void fa_decode_reduce_kernel(DecParams p) {
  __shared__ float red[D];
  __shared__ float wts[D];
  const int b = blockIdx.x / p.nq, h = blockIdx.x - b * p.nq;
  const int g = h / p.group, n = h - g * p.group;
  const int first = p.first_slot[b * p.nkv + g];
  if (first < 0) return;   // written by its only item (uniform over the workgroup)
  const int cnt = p.n_split[b];
  const int d = threadIdx.x;
  const int64_t row0 = (int64_t)first * p.group + n;   // partial row of item c: row0 + c * group
  float mx = kNegInf;
  for (int c = d; c < cnt; c += D) mx = fmaxf(mx, p.part_m[row0 + (int64_t)c * p.group]);
  mx = block_tree<D>(red, mx, true);
  float ls = 0.f;
  if (mx != kNegInf)
    for (int c = d; c < cnt; c += D) {
      const int64_t row = row0 + (int64_t)c * p.group;
      ls += p.part_l[row] * fast_exp2(p.part_m[row] - mx);
    }
  const float L = block_tree<D>(red, ls, false);
  float O = 0.f;
  for (int c0 = 0; c0 < cnt; c0 += D) {
    const int c = c0 + d;
    wts[d] = (c < cnt && mx != kNegInf) ? fast_exp2(p.part_m[row0 + (int64_t)c * p.group] - mx) : 0.f;
    __syncthreads();
    const int nc = min(D, cnt - c0);
    const float* po = p.part_o + (row0 + (int64_t)c0 * p.group) * D + d;
    const int64_t step = (int64_t)p.group * D;
#pragma unroll 8
    for (int k = 0; k < nc; ++k) O += po[k * step] * wts[k];
    __syncthreads();
  }
  reinterpret_cast<E*>(p.out)[((int64_t)b * p.nq + h) * D + d] = cvt16<E>(L > 0.f ? O / L : 0.f);
}

template <typename E, int D>
static hipError_t launch_decode_t(int n_items, const DecParams& p, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid((unsigned)n_items), block(64 * kDecWaves);
  const bool two = p.group > 32, mask = p.mask != nullptr;
  if (two && mask) hipLaunchKernelGGL((fa_decode_kernel<E, D, 2, true>), grid, block, 0, s, p);
  else if (two) hipLaunchKernelGGL((fa_decode_kernel<E, D, 2, false>), grid, block, 0, s, p);
  else if (mask) hipLaunchKernelGGL((fa_decode_kernel<E, D, 1, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((fa_decode_kernel<E, D, 1, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, int d, int n_items, const DecParams& p, hipStream_t s) {
  if (p.group > 64 || p.keys_per_wave % kDecBlock != 0) return hipErrorInvalidValue;
  if (dtype == 1 && d == 128) return launch_decode_t<__bf16, 128>(n_items, p, s);
  if (dtype == 1 && d == 64) return launch_decode_t<__bf16, 64>(n_items, p, s);
  if (dtype == 2 && d == 128) return launch_decode_t<_Float16, 128>(n_items, p, s);
  if (dtype == 2 && d == 64) return launch_decode_t<_Float16, 64>(n_items, p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_reduce(int dtype, int d, const DecParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.batch * p.nq));
  if (dtype == 1 && d == 128) hipLaunchKernelGGL((fa_decode_reduce_kernel<__bf16, 128>), grid, dim3(128), 0, s, p);
  else if (dtype == 1 && d == 64) hipLaunchKernelGGL((fa_decode_reduce_kernel<__bf16, 64>), grid, dim3(64), 0, s, p);
  else if (dtype == 2 && d == 128) hipLaunchKernelGGL((fa_decode_reduce_kernel<_Float16, 128>), grid, dim3(128), 0, s, p);
  else if (dtype == 2 && d == 64) hipLaunchKernelGGL((fa_decode_reduce_kernel<_Float16, 64>), grid, dim3(64), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
