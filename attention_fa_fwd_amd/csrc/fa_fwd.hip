// Forward attention kernel for gfx950.
//
// Computes, per query row i of sequence b and query head h (kv head g = h / G),
// following aclnnFlashAttentionScoreV2 "Formula" (pseType 2: bias added after
// scaling) and the sink formulas of aclnnFlashAttentionUnpaddingScoreGradV5:
//   s_ij = scale * q_i.k_j + pse_h(i, j),  masked to -inf outside the window
//   m_i  = max(sink_h, max_j s_ij),  l_i = sum_j e^(s_ij - m_i) + e^(sink_h - m_i)
//   O_i  = sum_j e^(s_ij - m_i) z_ij v_j / (keep * l_i)
// with the online (running max / running sum) softmax over key tiles.
//
// Work decomposition: one workgroup = 4 waves = one 128-row query tile of one
// (sequence, head); each wave owns 32 rows.  Key/value tiles of 64 keys are
// staged in LDS, double buffered, prefetched through registers one tile ahead.
// Per wave and key tile:
//   S^T (64 keys x 32 rows) = K Q^T      A = K rows from LDS, B = Q in registers
//   O^T (D x 32 rows)      += V^T P^T    A = V via the transposing LDS read,
//                                         B = P taken straight from the S^T accumulator
// Every accumulator keeps one query row per lane (lanes l and l+32 share a row),
// so row max / row sum need only in-lane work plus one cross-half exchange.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

template <typename T, int D>
struct FwdShape {
  static constexpr int EB = sizeof(T);
  static constexpr int RB = D * EB;                 // bytes per K/V row
  static constexpr int KP = RB + 16;                // LDS pitch of K rows
  static constexpr int VP = RB + 64;                // LDS pitch of V rows (transposed reads)
  static constexpr int KBYTES = kFwdBN * KP;
  static constexpr int VBYTES = kFwdBN * VP;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int NCH = kFwdBN * CPR / 256;    // chunks per thread per tensor
  static constexpr int NQ = D / ElemTraits<T>::kChunk;  // Q operand registers
  static constexpr int NDB = D / 32;                // 32-wide d blocks of O
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void fa_fwd_kernel(FwdParams p) {
  using S = FwdShape<T, D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;        // which half of the wave (k-group of MFMA operands)
  const int lrow = lane & 31;

  const int item_idx = blockIdx.x / p.nq;
  const int hl = blockIdx.x - item_idx * p.nq;
  // consecutive workgroups go to different XCDs; give each XCD a contiguous run of heads
  const int h = p.head_swizzle ? (hl & 7) * (p.nq >> 3) + (hl >> 3) : hl;
  const int g = h / p.group;
  const WorkItem it = p.items[item_idx];
  const int b = it.b;
  const int q0 = p.cu_q[b], lq = p.cu_q[b + 1] - q0;
  const int k0 = p.cu_kv[b], lkv = p.cu_kv[b + 1] - k0;
  const FaWindow win = fa_make_window(p.mode, p.pre, p.next, lq, lkv);

  const int wr0 = it.tile * kFwdBM + wave * 32;   // first row of this wave (in sequence)
  const int i = wr0 + lrow;                        // this lane's row
  const bool row_ok = i < lq;
  const int64_t qrow_g = (int64_t)(q0 + (row_ok ? i : 0));

  // ---- Q operand in registers (B of S^T = K Q^T) ----
  using QReg = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
  QReg qf[S::NQ];
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + (qrow_g * p.nq + h) * D;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hh);
        if (!row_ok) v = bf16x8{};
        qf[c] = v;
      }
    } else {
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) qf[c] = row_ok ? qp[2 * c + hh] : 0.f;
    }
  }

  const float slope_l2 = p.slopes ? p.slopes[h] * kLog2e : 0.f;
  const bool has_sink = p.sink != nullptr;
  float m_run = has_sink ? p.sink[h] * kLog2e : kNegInf;
  float l_run = (has_sink && hh == 0) ? 1.f : 0.f;   // the two half-lanes are summed at the end
  f32x16 o[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) o[db] = f32x16{};

  const int64_t drop_row = p.use_dropout ? p.bit_base[b] + ((int64_t)h * lq + i) * lkv : 0;

  // ---- cooperative tile loads (global -> registers -> LDS) ----
  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const int64_t kv_stride = (int64_t)p.nkv * S::RB;
  u32x4 kreg[S::NCH], vreg[S::NCH];

  auto load_tile = [&](int t) {
    const int c0 = t * kFwdBN;
#pragma unroll
    for (int n = 0; n < S::NCH; ++n) {
      const int ci = tid + 256 * n;
      const int r = ci / S::CPR, cc = ci % S::CPR;
      const bool ok = c0 + r < lkv;
      const int64_t off = (int64_t)(ok ? c0 + r : 0) * kv_stride + cc * 16;
      u32x4 kv = *reinterpret_cast<const u32x4*>(kbase + off);
      u32x4 vv = *reinterpret_cast<const u32x4*>(vbase + off);
      kreg[n] = ok ? kv : u32x4{};
      vreg[n] = ok ? vv : u32x4{};
    }
  };
  auto store_tile = [&](int stage) {
    char* ks = smem + stage * S::STAGE;
    char* vs = ks + S::KBYTES;
#pragma unroll
    for (int n = 0; n < S::NCH; ++n) {
      const int ci = tid + 256 * n;
      const int r = ci / S::CPR, cc = ci % S::CPR;
      *reinterpret_cast<u32x4*>(ks + r * S::KP + cc * 16) = kreg[n];
      *reinterpret_cast<u32x4*>(vs + r * S::VP + cc * 16) = vreg[n];
    }
  };

  const int t_lo = it.lo, t_hi = it.hi;
  if (t_lo < t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_lo; t < t_hi; ++t) {
    const int stage = (t - t_lo) & 1;
    const bool more = t + 1 < t_hi;
    if (more) load_tile(t + 1);

    const int c0 = t * kFwdBN;
    const char* ks = smem + stage * S::STAGE;
    const char* vs = ks + S::KBYTES;

    bool wave_empty = wr0 >= lq;
    if (!wave_empty) {
      const int r1 = min(wr0 + 32, lq), c1 = min(c0 + kFwdBN, lkv);
      wave_empty = fa_tile_empty(win, wr0, r1, c0, c1);
    }
    if (!wave_empty) {
      const bool full = fa_tile_full(win, wr0, 32, c0, kFwdBN, lq, lkv);
      // ---- S^T = K Q^T for two 32-key blocks ----
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 acc = f32x16{};
        const char* krow = ks + (32 * kb + lrow) * S::KP;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int c = 0; c < S::NQ; ++c) acc = mfma32(lds_read_b128(krow + (16 * c + 8 * hh) * 2), qf[c], acc);
        } else {
#pragma unroll
          for (int c = 0; c < S::NQ; ++c)
            acc = mfma32(*reinterpret_cast<const float*>(krow + (2 * c + hh) * 4), qf[c], acc);
        }
        s[kb] = acc;
      }
      // ---- scale, bias, mask (log2 domain) ----
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = c0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          float x = s[kb][r] * p.scale_log2;
          if (p.slopes) x = __builtin_fmaf(slope_l2, (float)(j - i), x);
          if (!full && !fa_allowed(win, i, j, lq, lkv)) x = kNegInf;
          s[kb][r] = x;
          mt = fmaxf(mt, x);
        }
      }
      mt = fmaxf(mt, wave_xor32(mt));
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float lsum = 0.f;
      uint64_t bits = ~0ull;
      if (p.use_dropout) bits = load_mask_window(p.drop, p.drop_bytes, drop_row + c0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(s[kb][r] - m_use);
          lsum += e;
          const int bit = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          s[kb][r] = ((bits >> bit) & 1ull) ? e : 0.f;
        }
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) o[db] *= alpha;

      // ---- O^T += V^T P^T ----
      if constexpr (sizeof(T) == 2) {
        const int grp = lane >> 4, sl = lane & 15;
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) {
          const int kb = c2 >> 1, sub = c2 & 1;
          bf16x8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[j] = to_bf16(s[kb][8 * sub + j]);
          const int row0 = 32 * kb + 16 * sub + 4 * (grp >> 1) + (sl >> 2);
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            const int col = 32 * db + 16 * (grp & 1) + 4 * (sl & 3);
            const bf16x8 a = lds_read_tr_x2(vs + row0 * S::VP + col * 2, vs + (row0 + 8) * S::VP + col * 2);
            o[db] = mfma32(a, pb, o[db]);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const float pb = s[kb][r];
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
              const float a = *reinterpret_cast<const float*>(vs + key * S::VP + (32 * db + lrow) * 4);
              o[db] = mfma32(a, pb, o[db]);
            }
          }
        }
      }
    }
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_tot = l_run + wave_xor32(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? p.inv_keep / l_tot : 0.f;
    T* op = reinterpret_cast<T*>(p.o) + (qrow_g * p.nq + h) * D;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 32 * db + 8 * a + 4 * hh;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[db][4 * a + e] * inv);
          *reinterpret_cast<bf16x4*>(op + d) = v;
        } else {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[db][4 * a + e] * inv;
          *reinterpret_cast<f32x4*>(op + d) = v;
        }
      }
    }
    if (hh == 0) {
      p.m_out[qrow_g * p.nq + h] = m_run * kLn2;
      p.l_out[qrow_g * p.nq + h] = l_tot;
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  using S = FwdShape<T, D>;
  static_assert(S::NCH * 256 == kFwdBN * S::CPR, "tile load split");
  const int64_t blocks = (int64_t)p.n_items * p.nq;
  if (blocks == 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)fa_fwd_kernel<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     S::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_fwd_kernel<T, D>), dim3((unsigned)blocks), dim3(256), S::LDS, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int d, const FwdParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return launch_fwd_t<__bf16, 128>(p, s);
  if (dtype == 1 && d == 64) return launch_fwd_t<__bf16, 64>(p, s);
  if (dtype == 0 && d == 128) return launch_fwd_t<float, 128>(p, s);
  if (dtype == 0 && d == 64) return launch_fwd_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
