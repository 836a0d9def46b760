// Forward attention kernel for gfx950.
//
// Computes, per query row i of sequence b and query head h (kv head g = h / G),
// following aclnnFlashAttentionScoreV2 "Formula" (pseType 2: bias added after
// scaling) and the sink formulas of aclnnFlashAttentionUnpaddingScoreGradV5:
//   s_ij = scale * q_i.k_j + pse_h(i, j),  masked to -inf outside the window
//   m_i  = max(sink_h, max_j s_ij),  l_i = sum_j e^(s_ij - m_i) + e^(sink_h - m_i)
//   O_i  = sum_j e^(s_ij - m_i) z_ij v_j / (keep * l_i)
// with an online softmax over key tiles.
//
// Work decomposition: one workgroup = NW waves = one query tile of 32*NW rows of
// one (sequence, head); each wave owns 32 rows, and all waves share each K/V
// tile.  Key/value tiles of 64 keys are copied global -> LDS by global_load_lds
// into two stage buffers, one tile ahead of the compute; each wave drains its own
// copies just before the barrier that publishes a tile.  Per wave and tile:
//   S^T (64 keys x 32 rows) = K Q^T      A = K rows from LDS, B = Q in registers
//   O^T (D x 32 rows)      += V^T P^T    A = V via the transposing LDS read,
//                                         B = P taken straight from the S^T accumulator
// Every accumulator keeps one query row per lane (lanes l and l+32 share a row),
// so row max / row sum need only in-lane work plus one cross-half exchange.
//
// Softmax bookkeeping (log2 units): the exponent offset m_run only moves when a
// row's maximum exceeds it by more than kLazy, so most tiles skip the rescale of
// O and l (probabilities stay below 2^kLazy); the true maximum is tracked apart
// and l is brought to it in the epilogue.  Tiles fully inside the mask skip all
// mask arithmetic and fold the scale into the exponent's FMA.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

constexpr float kLazy = 8.0f;

template <typename T, int D>
struct FwdShape {
  static constexpr int EB = sizeof(T);
  static constexpr int RB = D * EB;                     // bytes per K/V row
  static constexpr int KP = RB + 16;                    // LDS pitch of K rows (16-byte row reads)
  static constexpr int VP = RB + (EB == 2 ? 64 : 16);   // LDS pitch of V rows (transposing reads)
  static constexpr int KT = kFwdBN * KP;
  static constexpr int VT = kFwdBN * VP;
  static constexpr int STAGE = KT + VT;
  static constexpr int NQ = D / ElemTraits<T>::kChunk;  // Q operand registers
  static constexpr int NDB = D / 32;                    // 32-wide d blocks of O
};

// NW = 8 waves share each K/V tile; the dropout variants need more than 256
// registers and run 4-wave workgroups with one wave per SIMD instead.
template <typename T, int D, bool DROP, bool ALIBI>
__global__ __launch_bounds__(64 * fwd_waves(DROP), 1) void fa_fwd_kernel(FwdParams p) {
  using S = FwdShape<T, D>;
  constexpr int NW = fwd_waves(DROP);
  constexpr int BM = 32 * NW;
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

  const int wr0 = it.tile * BM + wave * 32;       // first row of this wave (in sequence)
  const int i = wr0 + lrow;                        // this lane's row
  const bool row_ok = i < lq;

  // ---- Q operand in registers (B of S^T = K Q^T) ----
  using QReg = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
  QReg qf[S::NQ];
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + ((int64_t)(q0 + (row_ok ? i : 0)) * p.nq + h) * D;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hh);
        qf[c] = row_ok ? v : bf16x8{};
      }
    } else {
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) qf[c] = row_ok ? qp[2 * c + hh] : 0.f;
    }
  }

  const float sc = p.scale_log2;
  const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
  const bool has_sink = p.sink != nullptr;
  float m_run = has_sink ? p.sink[h] * kLog2e : kNegInf;   // exponent offset
  float m_true = m_run;                                     // running maximum
  float l_run = (has_sink && hh == 0) ? 1.f : 0.f;          // the two half-lanes are summed at the end
  f32x16 o[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) o[db] = f32x16{};

  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const int64_t kv_stride = (int64_t)p.nkv * S::RB;
  // per-lane LDS byte offsets; every other offset below is a compile-time immediate
  const int k_lane = lrow * S::KP + 16 * hh;                                      // K row reads
  const int v_lane = (4 * (grp >> 1) + (sl >> 2)) * S::VP + (16 * (grp & 1) + 4 * (sl & 3)) * 2;  // V^T reads

  auto load = [&](char* st, int t) {
    dma_rows<kFwdBN, S::RB, S::KP, NW>(st, kbase, kv_stride, t * kFwdBN, lkv, wave, lane);
    dma_rows<kFwdBN, S::RB, S::VP, NW>(st + S::KT, vbase, kv_stride, t * kFwdBN, lkv, wave, lane);
  };

  // One key tile: everything a wave does between two barriers.
  auto tile = [&](int t, const char* ks) {
    const char* vs = ks + S::KT;
    const int c0 = t * kFwdBN;
    if (wr0 >= lq || fa_tile_empty(win, wr0, min(wr0 + 32, lq), c0, min(c0 + kFwdBN, lkv))) return;
    const bool full = fa_tile_full(win, wr0, 32, c0, kFwdBN, lq, lkv);
    uint32_t bits[2] = {~0u, ~0u};
    if constexpr (DROP) {
      // issued before the MFMAs so the global latency overlaps them
      const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + i) * lkv + c0;
      bits[0] = load_mask_bits32(p.drop, p.drop_bytes, pos);
      bits[1] = load_mask_bits32(p.drop, p.drop_bytes, pos + 32);
    }
    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      if constexpr (sizeof(T) == 2) {
        bf16x8 a[S::NQ];
#pragma unroll
        for (int c = 0; c < S::NQ; ++c) a[c] = lds_read_b128(ks + k_lane + kb * 32 * S::KP + 32 * c);
#pragma unroll
        for (int c = 0; c < S::NQ; ++c) s[kb] = mfma32(a[c], qf[c], s[kb]);
      } else {
#pragma unroll
        for (int c = 0; c < S::NQ; ++c) {
          const float a = *reinterpret_cast<const float*>(ks + lrow * S::KP + kb * 32 * S::KP + (2 * c + hh) * 4);
          s[kb] = mfma32(a, qf[c], s[kb]);
        }
      }
    }
    // ---- row maximum of the scaled (biased, masked) logits ----
    const bool plain = !ALIBI && full;   // logits are just sc * s
    float mt;
    if (plain) {
      // max(sc * s) is sc * max(s) for sc >= 0 and sc * min(s) otherwise
      float ext = sc >= 0.f ? kNegInf : __builtin_inff();
      if (sc >= 0.f) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ext = fmaxf(ext, s[kb][r]);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ext = fminf(ext, s[kb][r]);
      }
      mt = ext * sc;
    } else {
      mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = c0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          float x = s[kb][r] * sc;
          if constexpr (ALIBI) x = __builtin_fmaf(slope_l2, (float)(j - i), x);
          if (!full && !fa_allowed(win, i, j, lq, lkv)) x = kNegInf;
          s[kb][r] = x;
          mt = fmaxf(mt, x);
        }
      }
    }
    mt = fmaxf(mt, wave_xor32(mt));
    m_true = fmaxf(m_true, mt);
    const bool need = mt > m_run + kLazy;      // also true on the first finite maximum
    float alpha = 1.f;
    if (need) {
      alpha = fast_exp2(m_run - mt);           // 0 when m_run = -inf
      m_run = mt;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    // ---- probabilities (pre-dropout sum, post-dropout operand) ----
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = plain ? fast_exp2(__builtin_fmaf(s[kb][r], sc, -m_use)) : fast_exp2(s[kb][r] - m_use);
        lsum += e;
        if constexpr (DROP) {
          const int bit = 8 * (r >> 2) + 4 * hh + (r & 3);
          s[kb][r] = ((bits[kb] >> bit) & 1u) ? e : 0.f;
        } else {
          s[kb][r] = e;
        }
      }
    l_run = l_run * alpha + lsum;
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) o[db] *= alpha;
    }

    // ---- O^T += V^T P^T ----
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        const int kb = c2 >> 1, sub = c2 & 1;
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = to_bf16(s[kb][8 * sub + j]);
        bf16x8 a[S::NDB];
        const char* vrow = vs + v_lane + (16 * c2) * S::VP;
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) a[db] = lds_read_tr_x2(vrow + 64 * db, vrow + 8 * S::VP + 64 * db);
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) o[db] = mfma32(a[db], pb, o[db]);
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
            o[db] = mfma32(a, s[kb][r], o[db]);
          }
        }
      }
    }
  };

  const int t_lo = it.lo, t_hi = it.hi;
  if (t_lo < t_hi) load(st0, t_lo);
  dma_wait();
  __syncthreads();
  for (int t = t_lo; t < t_hi; t += 2) {
    if (t + 1 < t_hi) load(st1, t + 1);
    tile(t, st0);
    dma_wait();
    __syncthreads();
    if (t + 1 < t_hi) {
      if (t + 2 < t_hi) load(st0, t + 2);
      tile(t + 1, st1);
      dma_wait();
      __syncthreads();
    }
  }

  // ---- epilogue: O = o / (keep * l_run); l reported against the true maximum ----
  const float l_tot = l_run + wave_xor32(l_run);
  if (row_ok) {
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
      const float l_out = l_tot > 0.f ? l_tot * fast_exp2(m_run - m_true) : 0.f;
      p.m_out[rowg * p.nq + h] = m_true * kLn2;
      p.l_out[rowg * p.nq + h] = l_out;
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_items * p.nq;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  const bool drop = p.use_dropout != 0, alibi = p.slopes != nullptr;
  const dim3 block(64 * fwd_waves(drop));
  if (drop && alibi)
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, true, true>), grid, block, 0, s, p);
  else if (drop)
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, true, false>), grid, block, 0, s, p);
  else if (alibi)
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, false, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, false, false>), grid, block, 0, s, p);
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
