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
// Work decomposition: one workgroup = 4 waves = one query tile of one
// (sequence, head); each wave owns MB blocks of 32 rows.  Key/value tiles of 64
// keys are copied global -> LDS by global_load_lds into two stage buffers (two
// distinct LDS arrays, so reads of one never wait on the copy into the other),
// one tile ahead of the compute.  Per wave and key tile:
//   S^T (64 keys x 32 rows) = K Q^T      A = K rows from LDS, B = Q in registers
//   O^T (D x 32 rows)      += V^T P^T    A = V via the transposing LDS read,
//                                         B = P taken straight from the S^T accumulator
// Every accumulator keeps one query row per lane (lanes l and l+32 share a row),
// so row max / row sum need only in-lane work plus one cross-half exchange.
// Tiles that are fully inside the mask skip all mask arithmetic.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

template <typename T, int D, int MB>
struct FwdShape {
  static constexpr int EB = sizeof(T);
  static constexpr int RB = D * EB;                     // bytes per K/V row
  static constexpr int KP = RB + 16;                    // LDS pitch of K rows (16-byte row reads)
  static constexpr int VP = RB + (EB == 2 ? 32 : 16);   // LDS pitch of V rows (transposing reads)
  static constexpr int BM = 128 * MB;                   // query rows per workgroup
  static constexpr int KT = kFwdBN * KP;
  static constexpr int VT = kFwdBN * VP;
  static constexpr int STAGE = KT + VT;
  static constexpr int NQ = D / ElemTraits<T>::kChunk;  // Q operand registers per row block
  static constexpr int NDB = D / 32;                    // 32-wide d blocks of O
};

// Two workgroups per CU except where the dropout path would not fit 256 registers.
template <typename T, int D, int MB, bool DROP, bool ALIBI>
__global__ __launch_bounds__(256, (MB == 1 && !DROP) ? 2 : 1) void fa_fwd_kernel(FwdParams p) {
  using S = FwdShape<T, D, MB>;
  __shared__ __attribute__((aligned(16))) char st0[S::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[S::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;        // which half of the wave (k-group of MFMA operands)
  const int lrow = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;

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

  const int wr0 = it.tile * S::BM + wave * 32 * MB;   // first row of this wave (in sequence)

  // ---- Q operand in registers (B of S^T = K Q^T) ----
  using QReg = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
  QReg qf[MB][S::NQ];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = wr0 + 32 * mb + lrow;
    const bool ok = i < lq;
    const T* qp = reinterpret_cast<const T*>(p.q) + ((int64_t)(q0 + (ok ? i : 0)) * p.nq + h) * D;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hh);
        qf[mb][c] = ok ? v : bf16x8{};
      }
    } else {
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) qf[mb][c] = ok ? qp[2 * c + hh] : 0.f;
    }
  }

  const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
  const bool has_sink = p.sink != nullptr;
  float m_run[MB], l_run[MB];
  f32x16 o[MB][S::NDB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_run[mb] = has_sink ? p.sink[h] * kLog2e : kNegInf;
    l_run[mb] = (has_sink && hh == 0) ? 1.f : 0.f;   // the two half-lanes are summed at the end
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) o[mb][db] = f32x16{};
  }

  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const int64_t kv_stride = (int64_t)p.nkv * S::RB;
  // per-lane LDS byte offsets; every other offset below is a compile-time immediate
  const int k_lane = lrow * S::KP + 16 * hh;                                      // K row reads
  const int v_lane = (4 * (grp >> 1) + (sl >> 2)) * S::VP + (16 * (grp & 1) + 4 * (sl & 3)) * 2;  // V^T reads

  auto load = [&](char* st, int t) {
    dma_rows<kFwdBN, S::RB, S::KP>(st, kbase, kv_stride, t * kFwdBN, lkv, wave, lane);
    dma_rows<kFwdBN, S::RB, S::VP>(st + S::KT, vbase, kv_stride, t * kFwdBN, lkv, wave, lane);
  };

  // One key tile: everything a wave does between two barriers.
  auto tile = [&](int t, const char* ks) {
    const char* vs = ks + S::KT;
    const int c0 = t * kFwdBN;
    bool empty[MB], full[MB], any = false;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r0 = wr0 + 32 * mb;
      empty[mb] = r0 >= lq || fa_tile_empty(win, r0, min(r0 + 32, lq), c0, min(c0 + kFwdBN, lkv));
      full[mb] = fa_tile_full(win, r0, 32, c0, kFwdBN, lq, lkv);
      any |= !empty[mb];
    }
    if (!any) return;
    // ---- S^T = K Q^T for two 32-key blocks (each K fragment feeds every row block) ----
    f32x16 s[MB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) s[mb][kb] = f32x16{};
      if constexpr (sizeof(T) == 2) {
        bf16x8 a[S::NQ];
#pragma unroll
        for (int c = 0; c < S::NQ; ++c) a[c] = lds_read_b128(ks + k_lane + kb * 32 * S::KP + 32 * c);
#pragma unroll
        for (int c = 0; c < S::NQ; ++c)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) s[mb][kb] = mfma32(a[c], qf[mb][c], s[mb][kb]);
      } else {
#pragma unroll
        for (int c = 0; c < S::NQ; ++c) {
          const float a = *reinterpret_cast<const float*>(ks + lrow * S::KP + kb * 32 * S::KP + (2 * c + hh) * 4);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) s[mb][kb] = mfma32(a, qf[mb][c], s[mb][kb]);
        }
      }
    }
    // ---- online softmax per row block (log2 domain) ----
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int i = wr0 + 32 * mb + lrow;
      float mt = kNegInf;
      if (!ALIBI && full[mb]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[mb][kb][r] *= p.scale_log2;
            mt = fmaxf(mt, s[mb][kb][r]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = c0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            float x = s[mb][kb][r] * p.scale_log2;
            if (ALIBI) x = __builtin_fmaf(slope_l2, (float)(j - i), x);
            if (!full[mb] && !fa_allowed(win, i, j, lq, lkv)) x = kNegInf;
            s[mb][kb][r] = x;
            mt = fmaxf(mt, x);
          }
        }
      }
      mt = fmaxf(mt, wave_xor32(mt));
      const float m_new = fmaxf(m_run[mb], mt);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[mb] - m_use);
      m_run[mb] = m_new;
      float lsum = 0.f;
      if constexpr (DROP) {
        const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + i) * lkv + c0;
        const uint64_t bits = load_mask_window(p.drop, p.drop_bytes, pos);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(s[mb][kb][r] - m_use);
            lsum += e;
            const int bit = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            s[mb][kb][r] = ((bits >> bit) & 1ull) ? e : 0.f;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(s[mb][kb][r] - m_use);
            lsum += e;
            s[mb][kb][r] = e;
          }
      }
      l_run[mb] = l_run[mb] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) o[mb][db] *= alpha;
    }

    // ---- O^T += V^T P^T ----
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        const int kb = c2 >> 1, sub = c2 & 1;
        bf16x8 pb[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[mb][j] = to_bf16(s[mb][kb][8 * sub + j]);
        bf16x8 a[S::NDB];
        const char* vrow = vs + v_lane + (16 * c2) * S::VP;
        if constexpr (S::NDB == 4)
          lds_read_tr_8<0, 8 * S::VP, 64, 64 + 8 * S::VP, 128, 128 + 8 * S::VP, 192, 192 + 8 * S::VP>(
              vrow, a[0], a[1], a[2], a[3]);
        else
          lds_read_tr_4<0, 8 * S::VP, 64, 64 + 8 * S::VP>(vrow, a[0], a[1]);
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) o[mb][db] = mfma32(a[db], pb[mb], o[mb][db]);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            const float a = *reinterpret_cast<const float*>(vs + key * S::VP + (32 * db + lrow) * 4);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) o[mb][db] = mfma32(a, s[mb][kb][r], o[mb][db]);
          }
        }
      }
    }
  };

  const int t_lo = it.lo, t_hi = it.hi;
  if (t_lo < t_hi) load(st0, t_lo);
  __syncthreads();
  for (int t = t_lo; t < t_hi; t += 2) {
    if (t + 1 < t_hi) load(st1, t + 1);
    tile(t, st0);
    __syncthreads();
    if (t + 1 < t_hi) {
      if (t + 2 < t_hi) load(st0, t + 2);
      tile(t + 1, st1);
      __syncthreads();
    }
  }

  // ---- epilogue ----
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = wr0 + 32 * mb + lrow;
    const float l_tot = l_run[mb] + wave_xor32(l_run[mb]);
    if (i < lq) {
      const int64_t rowg = q0 + i;
      const float inv = l_tot > 0.f ? p.inv_keep / l_tot : 0.f;
      T* op = reinterpret_cast<T*>(p.o) + (rowg * p.nq + h) * D;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 32 * db + 8 * a + 4 * hh;
          if constexpr (sizeof(T) == 2) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = to_bf16(o[mb][db][4 * a + e] * inv);
            *reinterpret_cast<bf16x4*>(op + d) = v;
          } else {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = o[mb][db][4 * a + e] * inv;
            *reinterpret_cast<f32x4*>(op + d) = v;
          }
        }
      }
      if (hh == 0) {
        p.m_out[rowg * p.nq + h] = m_run[mb] * kLn2;
        p.l_out[rowg * p.nq + h] = l_tot;
      }
    }
  }
}

template <typename T, int D, int MB>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_items * p.nq;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
  const bool drop = p.use_dropout != 0, alibi = p.slopes != nullptr;
  if (drop && alibi)
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, MB, true, true>), grid, block, 0, s, p);
  else if (drop)
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, MB, true, false>), grid, block, 0, s, p);
  else if (alibi)
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, MB, false, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, MB, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int d, const FwdParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return launch_fwd_t<__bf16, 128, kFwdMB>(p, s);
  if (dtype == 1 && d == 64) return launch_fwd_t<__bf16, 64, kFwdMB>(p, s);
  if (dtype == 0 && d == 128) return launch_fwd_t<float, 128, kFwdMB>(p, s);
  if (dtype == 0 && d == 64) return launch_fwd_t<float, 64, kFwdMB>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
