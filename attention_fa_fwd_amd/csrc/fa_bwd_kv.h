// Backward dK / dV kernel for gfx950 (and its atomic-dQ variant).
//
// Gradients of aclnnFlashAttentionUnpaddingScoreGrad ("Formula"):
//   dV = P~^T dY,  dK = scale * dS^T Q  (and dQ = scale * dS K with atomics),
//   dP = (dY V^T) * z / keep,  dS = P * (dP - D_i),  P = 2^(x - lse2).
// One workgroup per (128-key tile, kv head) loops over the heads of its GQA
// group and every query tile with an allowed pair; dK and dV accumulate in
// registers across the whole group (no atomics).
//   fa_bwd_kv_kernel       one wave per 32-key group; fp32, and the atomic-dQ
//                          variant (fa_bwd_kv_atomic.hip, MFMA results in VGPRs)
//   fa_bwd_kv_spec_kernel  16-bit deterministic: producer waves (S, dP, softmax, dS)
//                          beside consumer waves (dK, dV accumulation)
// The deterministic instances (fa_bwd_kv.hip) are compiled with the compiler's
// own MFMA register placement.
#pragma once
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

// ------------------------------------------------------------------ dK / dV (+ atomic dQ)
template <typename T, int D>
struct KvShape {
  static constexpr int EB = sizeof(T);
  static constexpr int RB = D * EB;
  // 16-bit Q / dY tiles are swizzled and unpadded (see tile_swz); fp32 tiles and
  // the K tile of the atomic variant use padded rows
  static constexpr bool kSwz = EB == 2;
  static constexpr int P = kSwz ? RB : RB + 16;     // LDS pitch of Q / dY rows
  static constexpr int KTP = RB + 16;               // LDS pitch of K rows (atomic dQ)
  static constexpr int QT = kKvBM * P;              // one 64-row Q (or dY) tile
  // stage layout: Q | dY | lse2[64] | D_i[64] | keep bits[64][4] | attenMask bits[64][4]
  static constexpr int OFF_DY = QT;
  static constexpr int OFF_LSE = 2 * QT;
  static constexpr int OFF_DEL = OFF_LSE + 4 * kKvBM;
  static constexpr int OFF_BITS = OFF_DEL + 4 * kKvBM;
  static constexpr int OFF_MBITS = OFF_BITS + 16 * kKvBM;   // attenMask bits, same layout as the keep bits
  static constexpr int STAGE = OFF_MBITS + 16 * kKvBM;
  static constexpr int KT = kKvBN * KTP;            // the 128-key K tile (atomic dQ only)
  static constexpr int DSP = kKvBM * EB + 16;       // pitch of dS^T rows (one row per key)
  static constexpr int DST = kKvBN * DSP;
  static constexpr int NOP = D / ElemTraits<T>::kChunk;
  static constexpr int NDB = D / 32;
};

template <typename T, int D, bool ATOMIC, bool DROP, int ALIBI, bool MASK>
__global__ __launch_bounds__(256, 1) void fa_bwd_kv_kernel(BwdParams p) {
  static_assert(sizeof(T) == 4 || ALIBI != kPseExt, "a 16-bit external pse runs the materialised-score path");
  using S = KvShape<T, D>;
  using E = typename std::conditional<sizeof(T) == 2, T, __bf16>::type;   // 16-bit element type
  using V8 = typename Vec16<E>::v8;
  using V4 = typename Vec16<E>::v4;
  using Op = typename std::conditional<sizeof(T) == 2, V8, float>::type;
  __shared__ __attribute__((aligned(16))) char st0[S::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[S::STAGE];
  __shared__ __attribute__((aligned(16))) char kt[ATOMIC ? S::KT : 16];
  __shared__ __attribute__((aligned(16))) char dst[ATOMIC ? S::DST : 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, lrow = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;

  const int item_idx = blockIdx.x / p.nkv;
  const int gl = blockIdx.x - item_idx * p.nkv;
  const int g = (p.nkv % 8 == 0) ? (gl & 7) * (p.nkv >> 3) + (gl >> 3) : gl;
  const WorkItem it = p.kv_items[item_idx];
  const int b = it.b;
  const int q0 = p.cu_q[b], lq = p.cu_q[b + 1] - q0;
  const int k0 = p.cu_kv[b], lkv = p.cu_kv[b + 1] - k0;
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, lq, lkv, p.prefix[b]);
  const int poff = b == 0 ? p.pse_off0 : 0;   // sequence 0 of mode 8: pse row i + qStartIdx - kvStartIdx
  const int c0 = it.tile * kKvBN;          // first key of the workgroup tile
  const int wc0 = c0 + 32 * wave;          // first key of this wave
  const int j = wc0 + lrow;                // this lane's key
  const bool key_ok = j < lkv;

  // K and V rows of this wave's keys as B operands (lane = key, registers = d)
  Op kf[S::NOP], vf[S::NOP];
  {
    const int64_t kr = (int64_t)(k0 + (key_ok ? j : 0)) * p.nkv + g;
    const T* kp = reinterpret_cast<const T*>(p.k) + kr * D;
    const T* vp = reinterpret_cast<const T*>(p.v) + kr * D;
#pragma unroll
    for (int c = 0; c < S::NOP; ++c) {
      if constexpr (sizeof(T) == 2) {
        V8 a = *reinterpret_cast<const V8*>(kp + 16 * c + 8 * hh);
        V8 v = *reinterpret_cast<const V8*>(vp + 16 * c + 8 * hh);
        kf[c] = key_ok ? a : V8{};
        vf[c] = key_ok ? v : V8{};
      } else {
        kf[c] = key_ok ? kp[2 * c + hh] : 0.f;
        vf[c] = key_ok ? vp[2 * c + hh] : 0.f;
      }
    }
  }
  const int64_t kv_stride = (int64_t)p.nkv * S::RB;
  // fp32 stages tiles through registers (no LDS DMA in flight): its register
  // footprint may need scratch, which must not overlap in-flight DMA
  constexpr bool kDma = sizeof(T) == 2;
  if constexpr (ATOMIC) {
    const char* kb = reinterpret_cast<const char*>(p.k) + ((int64_t)k0 * p.nkv + g) * S::RB;
    if constexpr (kDma)
      dma_rows<kKvBN, S::RB, S::KTP>(kt, kb, kv_stride, c0, lkv, wave, lane);
    else
      copy_rows<kKvBN, S::RB, S::KTP>(kt, kb, kv_stride, c0, lkv, tid);
  }

  f32x16 dk[S::NDB], dv[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) {
    if constexpr (sizeof(T) == 2) {
      // zeros produced by an MFMA, so the accumulators start in the register
      // class of the MFMAs that update them
      dk[db] = mfma32(V8{}, V8{}, f32x16{});
      dv[db] = mfma32(V8{}, V8{}, f32x16{});
    } else {
      dk[db] = f32x16{};
      dv[db] = f32x16{};
    }
  }

  const int nqt = it.hi - it.lo;
  const int nsteps = p.group * nqt;
  const int64_t q_stride = (int64_t)p.nq * S::RB;
  // per-lane LDS offsets: A-operand row reads and transposing B-operand reads
  const int a_lane = lrow * S::P + 16 * hh;
  const int t_lane = (4 * (grp >> 1) + (sl >> 2)) * S::P + (16 * (grp & 1) + 4 * (sl & 3)) * 2;
  // swizzled 16-bit tiles: row reads of chunk 2c + hh of row lrow (+32 per row
  // block), transposing reads of rows rv and rv + 8 (+16 per step), chunk 4db + qv
  int qoff[S::kSwz ? S::NOP : 1], toff[2][S::kSwz ? S::NDB : 1];
  if constexpr (S::kSwz) {
#pragma unroll
    for (int c = 0; c < S::NOP; ++c) qoff[c] = lrow * S::RB + 16 * ((2 * c + hh) ^ tile_swz<S::RB>(lrow));
    const int rv = 4 * (grp >> 1) + (sl >> 2), qv = 2 * (grp & 1) + ((sl & 3) >> 1), bv = 8 * (sl & 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
        toff[hf][db] = (rv + 8 * hf) * S::RB + 16 * ((4 * db + qv) ^ tile_swz<S::RB>(rv + 8 * hf)) + bv;
  }

  // steps walk the query tiles from the last one down, the heads of the group
  // innermost: every key tile of a sequence then starts on the same rows at the
  // same time, and the workgroups running together share those Q/dY rows in L2
  auto step_head = [&](int n) { return g * p.group + n % p.group; };
  auto step_row0 = [&](int n) { return (it.hi - 1 - n / p.group) * kKvBM; };

  auto load = [&](char* st, int n) {
    const int h = step_head(n), r0 = step_row0(n);
    const char* qb = reinterpret_cast<const char*>(p.q) + ((int64_t)q0 * p.nq + h) * S::RB;
    const char* dyb = reinterpret_cast<const char*>(p.dy) + ((int64_t)q0 * p.nq + h) * S::RB;
    if constexpr (!kDma) {
      copy_rows<kKvBM, S::RB, S::P>(st, qb, q_stride, r0, lq, tid);
      copy_rows<kKvBM, S::RB, S::P>(st + S::OFF_DY, dyb, q_stride, r0, lq, tid);
      if (tid < 2 * kKvBM) {
        const int rl = tid & (kKvBM - 1);
        const int rr = (r0 + rl < lq) ? r0 + rl : 0;
        const float v = (tid < kKvBM ? p.lse : p.delta)[(int64_t)(q0 + rr) * p.nq + h];
        reinterpret_cast<float*>(st + (tid < kKvBM ? S::OFF_LSE : S::OFF_DEL))[rl] = v;
      }
    } else {
      dma_tile_swz<kKvBM, S::RB, 4>(st, qb, q_stride, r0, lq, wave, lane);
      dma_tile_swz<kKvBM, S::RB, 4>(st + S::OFF_DY, dyb, q_stride, r0, lq, wave, lane);
      const int w = __builtin_amdgcn_readfirstlane(wave);
      if (w < 2) {
        // lse2 (wave 0) and D_i (wave 1) of the 64 rows, one dword per lane
        const int rr = (r0 + lane < lq) ? r0 + lane : 0;
        dma_dword(st + (w == 0 ? S::OFF_LSE : S::OFF_DEL), w == 0 ? p.lse : p.delta,
                  (uint32_t)(((int64_t)(q0 + rr) * p.nq + h) * 4));
      }
    }
  };
  // keep bits of the next step: 64 rows x 128 keys = 256 words, one per thread;
  // stored per wave (32 keys) and row, so a lane reads 4 consecutive rows at once
  const int bits_slot = (tid & 3) * kKvBM + (tid >> 2);
  auto bits_word = [&](int n) -> uint32_t {
    const int h = step_head(n), r0 = step_row0(n);
    const int r = tid >> 2, w = tid & 3;
    if (r0 + r >= lq) return 0u;
    const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + r0 + r) * lkv + c0 + 32 * w;
    return (uint32_t)load_mask_window(p.drop, p.drop_bytes, pos);
  };
  // attenMask bits (1 = masked) of the next step, same slots (only with a mask)
  auto mask_word = [&](int n) -> uint32_t {
    const int r0 = step_row0(n);
    const int r = tid >> 2, w = (c0 >> 5) + (tid & 3);
    if (r0 + r >= lq || w >= p.mwords) return ~0u;
    return p.mbits[(int64_t)(r0 + r) * p.mwords + w];
  };

  // atomic dQ of one 16-bit step: store_ds() puts each block's dS^T into LDS right
  // after it is formed; atomic_dq() then adds dQ(64 rows x 32-wide d block of this
  // wave) += dS K over the 128 keys to the fp32 accumulator
  auto store_ds = [&](int rb, const auto& d) {
    // register 8c + 4t + e holds row 32rb + 16c + 8t + 4hh + e
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        V4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = d[c][4 * t2 + e];
        *reinterpret_cast<V4*>(dst + (32 * wave + lrow) * S::DSP + (32 * rb + 16 * c + 8 * t2 + 4 * hh) * 2) = v;
      }
  };
  auto atomic_dq = [&](auto n) {
    const int h = step_head(n), r0 = step_row0(n);
    __syncthreads();
    const int dcol = 32 * wave;
    if (r0 < lq && dcol < D) {
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kc = 0; kc < kKvBN / 16; ++kc) {
        const int krow = 16 * kc + 4 * (grp >> 1) + (sl >> 2);
        const int coln = (16 * (grp & 1) + 4 * (sl & 3)) * 2;
        const V8 a0 = lds_read_tr_x2<V8>(dst + krow * S::DSP + coln, dst + (krow + 8) * S::DSP + coln);
        const V8 a1 = lds_read_tr_x2<V8>(dst + krow * S::DSP + coln + 64, dst + (krow + 8) * S::DSP + coln + 64);
        const int colk = (dcol + 16 * (grp & 1) + 4 * (sl & 3)) * 2;
        const V8 bo = lds_read_tr_x2<V8>(kt + krow * S::KTP + colk, kt + (krow + 8) * S::KTP + colk);
        acc[0] = mfma32(a0, bo, acc[0]);
        acc[1] = mfma32(a1, bo, acc[1]);
      }
      // acc[rb]: lane = d (dcol + lrow), registers = rows 32rb + 8(r/4) + 4hh + r%4
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (r0 + rr < lq)
            atomicAdd(p.dq_acc + ((int64_t)(q0 + r0 + rr) * p.nq + h) * D + dcol + lrow, acc[rb][r]);
        }
    }
  };
  // ---- 16-bit steps: per 32-row block [S, dP MFMAs] [P, dS] [dV, dK MFMAs] ----
  // Scheduling-group barriers keep the LDS operand reads of each MFMA group a
  // few MFMAs ahead of their use.  Blocks outside the mask are computed like
  // masked ones (every probability is zero): the waves of a workgroup wait for
  // each other at every step anyway.
  auto sdp = [&](const char* st, int rb, auto& s, auto& dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int c = 0; c < S::NOP; ++c) {
      const V8 qa = lds_read_b128<V8>(st + qoff[c] + 32 * rb * S::RB);
      const V8 ya = lds_read_b128<V8>(st + S::OFF_DY + qoff[c] + 32 * rb * S::RB);
      s = mfma32(qa, kf[c], s);
      dp = mfma32(ya, vf[c], dp);
    }
  };
  // P~ and dS of one block as 16-bit A operands (lane = key, registers = rows)
  auto elem = [&](auto full_c, const char* st, int r0, int rb, const f32x16& s, const f32x16& dp, float slope_l2,
                  int h, V8 (&pa)[2], V8 (&da)[2]) {
    constexpr bool plain = !ALIBI && decltype(full_c)::value;
    const float* lse_s = reinterpret_cast<const float*>(st + S::OFF_LSE);
    const float* del_s = reinterpret_cast<const float*>(st + S::OFF_DEL);
    const uint32_t* bits_s = reinterpret_cast<const uint32_t*>(st + S::OFF_BITS);
    const float sc = p.scale_log2;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int rq = 32 * rb + 8 * a + 4 * hh;   // rows rq .. rq+3 sit in registers 4a .. 4a+3
      const f32x4 lse4 = *reinterpret_cast<const f32x4*>(lse_s + rq);
      const f32x4 del4 = *reinterpret_cast<const f32x4*>(del_s + rq);
      u32x4 bits4, mb4 = {};
      if constexpr (DROP) bits4 = *reinterpret_cast<const u32x4*>(bits_s + wave * kKvBM + rq);
      if constexpr (!decltype(full_c)::value && MASK)
        mb4 = *reinterpret_cast<const u32x4*>(st + S::OFF_MBITS + 4 * (wave * kKvBM + rq));
      const float jmi = (float)(j - r0 - rq - poff);   // j - i of register 4a (pse position); minus e for 4a + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a + e, rr = rq + e, i = r0 + rr;
        float pr;
        if constexpr (plain) {
          pr = fast_exp2(__builtin_fmaf(s[r], sc, -lse4[e]));
        } else {
          float x = s[r] * sc;
          if constexpr (ALIBI != 0) x = add_pse<ALIBI>(x, slope_l2, jmi - (float)e);
          if constexpr (!decltype(full_c)::value) {
            const bool ok = (i < lq) & key_ok & (j >= fa_row_lo(win, i)) & (j <= fa_row_hi(win, i)) &
                            !((mb4[e] >> lrow) & 1u);
            x = ok ? x : kNegInf;
          }
          pr = fast_exp2(x - lse4[e]);
        }
        float dpv = dp[r], ptv = pr;
        if constexpr (DROP) {
          const bool keep = (bits4[e] >> lrow) & 1u;
          dpv = keep ? dpv * p.inv_keep : 0.f;
          ptv = keep ? pr * p.inv_keep : 0.f;
        }
        const float dsv = pr * (dpv - del4[e]);
        pa[r >> 3][r & 7] = cvt16<E>(ptv);
        da[r >> 3][r & 7] = cvt16<E>(dsv);
      }
    }
  };
  // dV += P~^T dY, dK += dS^T Q  (B operands through the transposing read)
  auto grads = [&](const char* st, int rb, const auto& pa, const auto& da) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const char* base = st + (32 * rb + 16 * c) * S::RB;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) {
        const V8 yo = lds_read_tr_x2<V8>(base + S::OFF_DY + toff[0][db], base + S::OFF_DY + toff[1][db]);
        const V8 qo = lds_read_tr_x2<V8>(base + toff[0][db], base + toff[1][db]);
        dv[db] = mfma32(pa[c], yo, dv[db]);
        dk[db] = mfma32(da[c], qo, dk[db]);
      }
    }
  };
  constexpr int kSdpMfma = 2 * S::NOP, kGradMfma = 4 * S::NDB;

  auto compute_16 = [&](const char* st, auto n) {
    const int h = step_head(n), r0 = step_row0(n);
    if (tid == 0)
      FA_TRACE_VISIT(p.trace_kv, (((int64_t)b * p.nq + h) * p.trace_kv_rb + r0 / kKvBM) * p.trace_kv_kt + it.tile);
    const float slope_l2 = pse_slopes(ALIBI) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
    // with an attenMask every block takes the masked path
    const bool full0 = fa_tile_full(win, r0, 32, wc0, 32, lq, lkv) && !MASK;
    const bool full1 = fa_tile_full(win, r0 + 32, 32, wc0, 32, lq, lkv) && !MASK;
    f32x16 s0, dp0, s1, dp1;
    V8 pa0[2], da0[2], pa1[2], da1[2];
    auto block = [&](int rb, bool full, auto& sx, auto& dpx, auto& pax, auto& dax) {
      __builtin_amdgcn_sched_barrier(0);
      sdp(st, rb, sx, dpx);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      sched_alternate<kSdpMfma, 0x008, 0x100>();
      __builtin_amdgcn_sched_barrier(0);
      if (full) elem(std::true_type{}, st, r0, rb, sx, dpx, slope_l2, h, pax, dax);
      else elem(std::false_type{}, st, r0, rb, sx, dpx, slope_l2, h, pax, dax);
      if constexpr (ATOMIC) store_ds(rb, dax);
      __builtin_amdgcn_sched_barrier(0);
      grads(st, rb, pax, dax);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      sched_alternate<kGradMfma, 0x008, 0x100, 2>();
      __builtin_amdgcn_sched_barrier(0);
    };
    block(0, full0, s0, dp0, pa0, da0);
    block(1, full1, s1, dp1, pa1, da1);
    if constexpr (ATOMIC) atomic_dq(n);
  };

  auto compute = [&](const char* st, int n) {
    const int h = step_head(n), r0 = step_row0(n);
    if (tid == 0)
      FA_TRACE_VISIT(p.trace_kv, (((int64_t)b * p.nq + h) * p.trace_kv_rb + r0 / kKvBM) * p.trace_kv_kt + it.tile);
    const float slope_l2 = pse_slopes(ALIBI) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
    const float* lse_s = reinterpret_cast<const float*>(st + S::OFF_LSE);
    const float* del_s = reinterpret_cast<const float*>(st + S::OFF_DEL);
    const uint32_t* bits_s = reinterpret_cast<const uint32_t*>(st + S::OFF_BITS);
    V8 da_keep[2][2];   // dS of both row blocks (atomic dQ)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int rb0 = r0 + 32 * rb;
      bool empty = rb0 >= lq || wc0 >= lkv;
      if (!empty) empty = fa_tile_empty(win, rb0, min(rb0 + 32, lq), wc0, min(wc0 + 32, lkv));
      if constexpr (ATOMIC && sizeof(T) == 2) {
        da_keep[rb][0] = V8{};
        da_keep[rb][1] = V8{};
      }
      if (empty) continue;
      const bool full = fa_tile_full(win, rb0, 32, wc0, 32, lq, lkv) && !MASK;
      // ---- S = Q K^T and dP~ = dY V^T (lane = key, registers = rows) ----
      f32x16 s = f32x16{}, dp = f32x16{};
      if constexpr (sizeof(T) == 2) {
        V8 qa[S::NOP];
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) qa[c] = lds_read_b128<V8>(st + a_lane + 32 * rb * S::P + 32 * c);
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) s = mfma32(qa[c], kf[c], s);
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) qa[c] = lds_read_b128<V8>(st + S::OFF_DY + a_lane + 32 * rb * S::P + 32 * c);
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) dp = mfma32(qa[c], vf[c], dp);
      } else {
        const char* qrow = st + (32 * rb + lrow) * S::P;
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) {
          s = mfma32(*reinterpret_cast<const float*>(qrow + (2 * c + hh) * 4), kf[c], s);
          dp = mfma32(*reinterpret_cast<const float*>(qrow + S::OFF_DY + (2 * c + hh) * 4), vf[c], dp);
        }
      }
      // ---- P, P~, dS ----
      f32x16 pt, ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
        float x = s[r] * p.scale_log2;
        if constexpr (ALIBI == kPseExt)
          x = __builtin_fmaf(p.pse_coef, (r0 + rr < lq && key_ok) ? pse_value<T>(p, b, h, r0 + rr, j, lq) : 0.f, x);
        else if constexpr (ALIBI != 0)
          x = add_pse<ALIBI>(x, slope_l2, (float)(j - (r0 + rr) - poff));
        if (!full && (!fa_allowed(win, r0 + rr, j, lq, lkv) ||
                      (MASK && ((reinterpret_cast<const uint32_t*>(st + S::OFF_MBITS)[wave * kKvBM + rr] >> lrow) & 1u))))
          x = kNegInf;
        const float pr = fast_exp2(x - lse_s[rr]);
        float dpv = dp[r], ptv = pr;
        if constexpr (DROP) {
          const bool keep = (bits_s[wave * kKvBM + rr] >> lrow) & 1u;
          dpv = keep ? dpv * p.inv_keep : 0.f;
          ptv = keep ? pr * p.inv_keep : 0.f;
        }
        pt[r] = ptv;
        ds[r] = pr * (dpv - del_s[rr]);
      }
      // ---- dV += P~^T dY, dK += dS^T Q  (B operands through the transposing read) ----
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          V8 pa, da;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pa[e] = cvt16<E>(pt[8 * c + e]);
            da[e] = cvt16<E>(ds[8 * c + e]);
          }
          if constexpr (ATOMIC) da_keep[rb][c] = da;
          const char* base = st + t_lane + (32 * rb + 16 * c) * S::P;
          V8 dyo[S::NDB], qo[S::NDB];
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            dyo[db] = lds_read_tr_x2<V8>(base + S::OFF_DY + 64 * db, base + S::OFF_DY + 8 * S::P + 64 * db);
            qo[db] = lds_read_tr_x2<V8>(base + 64 * db, base + 8 * S::P + 64 * db);
          }
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            dv[db] = mfma32(pa, dyo[db], dv[db]);
            dk[db] = mfma32(da, qo[db], dk[db]);
          }
          // the dropout variants sit at the register limit: keep the next chunk's
          // LDS reads from being hoisted above these MFMAs
          if constexpr (DROP) __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            const float dyo = *reinterpret_cast<const float*>(st + S::OFF_DY + rr * S::P + (32 * db + lrow) * 4);
            const float qo = *reinterpret_cast<const float*>(st + rr * S::P + (32 * db + lrow) * 4);
            dv[db] = mfma32(pt[r], dyo, dv[db]);
            dk[db] = mfma32(ds[r], qo, dk[db]);
          }
          // keep the scheduler from hoisting every LDS read of the loop (register pressure)
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (ATOMIC) {
          // fp32: dS^T[key][row] written directly from the accumulator layout
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = ds[4 * a + e];
            *reinterpret_cast<f32x4*>(dst + (32 * wave + lrow) * S::DSP + (32 * rb + 8 * a + 4 * hh) * 4) = v;
          }
        }
      }
    }
    if constexpr (ATOMIC) {
      if constexpr (sizeof(T) == 2) {
        // dS^T[key][row] from the kept 16-bit operands: register 8c + 4t + e holds row 16c + 8t + 4hh + e
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              V4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = da_keep[rb][c][4 * t2 + e];
              *reinterpret_cast<V4*>(dst + (32 * wave + lrow) * S::DSP +
                                         (32 * rb + 16 * c + 8 * t2 + 4 * hh) * 2) = v;
            }
      } else {
        // rows of empty blocks were never written: clear them
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int rb0 = r0 + 32 * rb;
          bool empty = rb0 >= lq || wc0 >= lkv;
          if (!empty) empty = fa_tile_empty(win, rb0, min(rb0 + 32, lq), wc0, min(wc0 + 32, lkv));
          if (empty)
#pragma unroll
            for (int a = 0; a < 4; ++a)
              *reinterpret_cast<f32x4*>(dst + (32 * wave + lrow) * S::DSP + (32 * rb + 8 * a + 4 * hh) * 4) =
                  f32x4{};
        }
      }
      __syncthreads();
      // ---- dQ(64 rows x this wave's 32-wide d block) += dS K over the 128 keys ----
      const int dcol = 32 * wave;
      if (r0 < lq && dcol < D) {
        f32x16 acc[2] = {f32x16{}, f32x16{}};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int kc = 0; kc < kKvBN / 16; ++kc) {
            const int krow = 16 * kc + 4 * (grp >> 1) + (sl >> 2);
            const int coln = (16 * (grp & 1) + 4 * (sl & 3)) * 2;
            const V8 a0 = lds_read_tr_x2<V8>(dst + krow * S::DSP + coln, dst + (krow + 8) * S::DSP + coln);
            const V8 a1 = lds_read_tr_x2<V8>(dst + krow * S::DSP + coln + 64, dst + (krow + 8) * S::DSP + coln + 64);
            const int colk = (dcol + 16 * (grp & 1) + 4 * (sl & 3)) * 2;
            const V8 bo = lds_read_tr_x2<V8>(kt + krow * S::KTP + colk, kt + (krow + 8) * S::KTP + colk);
            acc[0] = mfma32(a0, bo, acc[0]);
            acc[1] = mfma32(a1, bo, acc[1]);
          }
        } else {
#pragma unroll 8
          for (int kc = 0; kc < kKvBN / 2; ++kc) {
            const int key = 2 * kc + hh;
            const float bo = *reinterpret_cast<const float*>(kt + key * S::KTP + (dcol + lrow) * 4);
            acc[0] = mfma32(*reinterpret_cast<const float*>(dst + key * S::DSP + lrow * 4), bo, acc[0]);
            acc[1] = mfma32(*reinterpret_cast<const float*>(dst + key * S::DSP + (32 + lrow) * 4), bo, acc[1]);
          }
        }
        // acc[rb]: lane = d (dcol + lrow), registers = rows 32rb + 8(r/4) + 4hh + r%4
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (r0 + rr < lq)
              atomicAdd(p.dq_acc + ((int64_t)(q0 + r0 + rr) * p.nq + h) * D + dcol + lrow, acc[rb][r]);
          }
      }
    }
  };

  if (nsteps > 0) load(st0, 0);
  uint32_t word = 0, mword = 0;
  if constexpr (DROP) {
    if (nsteps > 0) word = bits_word(0);
    reinterpret_cast<uint32_t*>(st0 + S::OFF_BITS)[bits_slot] = word;
  }
  if (MASK && nsteps > 0) reinterpret_cast<uint32_t*>(st0 + S::OFF_MBITS)[bits_slot] = mask_word(0);
  dma_wait();
  __syncthreads();
  for (int n = 0; n < nsteps; n += 2) {
    if (n + 1 < nsteps) {
      load(st1, n + 1);
      if constexpr (DROP) word = bits_word(n + 1);
      if constexpr (MASK) mword = mask_word(n + 1);
    }
    if constexpr (sizeof(T) == 2) compute_16(st0, n);
    else compute(st0, n);
    if constexpr (DROP)
      if (n + 1 < nsteps) reinterpret_cast<uint32_t*>(st1 + S::OFF_BITS)[bits_slot] = word;
    if (MASK && n + 1 < nsteps) reinterpret_cast<uint32_t*>(st1 + S::OFF_MBITS)[bits_slot] = mword;
    dma_wait();
    __syncthreads();
    if (n + 1 < nsteps) {
      if (n + 2 < nsteps) {
        load(st0, n + 2);
        if constexpr (DROP) word = bits_word(n + 2);
        if constexpr (MASK) mword = mask_word(n + 2);
      }
      if constexpr (sizeof(T) == 2) compute_16(st1, n + 1);
      else compute(st1, n + 1);
      if constexpr (DROP)
        if (n + 2 < nsteps) reinterpret_cast<uint32_t*>(st0 + S::OFF_BITS)[bits_slot] = word;
      if (MASK && n + 2 < nsteps) reinterpret_cast<uint32_t*>(st0 + S::OFF_MBITS)[bits_slot] = mword;
      dma_wait();
      __syncthreads();
    }
  }

  // ---- epilogue: dK *= scale; write dK, dV (lane = d, registers = keys) ----
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
      const int jj = wc0 + kk;
      if (jj < lkv) {
        const int64_t off = ((int64_t)(k0 + jj) * p.nkv + g) * D + 32 * db + lrow;
        if constexpr (sizeof(T) == 2) {
          reinterpret_cast<E*>(p.dk)[off] = cvt16<E>(dk[db][r] * p.scale);
          reinterpret_cast<E*>(p.dv)[off] = cvt16<E>(dv[db][r]);
        } else {
          reinterpret_cast<float*>(p.dk)[off] = dk[db][r] * p.scale;
          reinterpret_cast<float*>(p.dv)[off] = dv[db][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- producer / consumer waves
// LDS operand reads issued ahead of the first MFMA of a producer / consumer matrix phase
constexpr int kSpecReadAheadP = 4, kSpecReadAheadC = 16;
// 16-bit deterministic dK/dV with specialised waves (8 per workgroup, one workgroup per CU).
//   waves 0-3, producers (key group kg = wave): hold the group's K and V rows; for step
//     t + 1 they compute S = Q K^T and dP~ = dY V^T for both 32-row blocks, then P~ and dS
//     as 16-bit A operands, which they write to the group's exchange area;
//   waves 4-7, consumers (kg = wave - 4): hold dK and dV of the group's 32 keys over all
//     of D; at the start of tick t they take step t's operands out of the exchange area
//     into registers, then issue the tile copies of step t + 2 and accumulate
//     dV += P~^T dY and dK += dS^T Q.
// Wave w and wave w + 4 share a SIMD (checked on the device), so each SIMD runs one
// producer (matrix work, then softmax / dS on the VALU) beside one consumer (matrix work
// and LDS reads): the VALU work of one overlaps the matrix work of the other (two
// identical waves per SIMD would run the same phase at the same time).
// Per tick: barrier A (step t's operands and tiles are in) -> consumers read the exchange
// area -> barrier B (it may be overwritten) -> producers form step t + 1 while consumers
// run step t.  LDS: three Q/dY stages (step t for the consumers, t + 1 for the producers,
// t + 2 in flight) and one exchange area.  Each role runs its own loop (same barriers), so
// neither role's registers are live in the other's.
template <typename E, int D, bool DROP, int ALIBI, bool MASK>
__global__ __launch_bounds__(512, 1) void fa_bwd_kv_spec_kernel(BwdParams p) {
  static_assert(ALIBI != kPseExt, "a 16-bit external pse runs the materialised-score path");
  using S = KvShape<E, D>;
  using V8 = typename Vec16<E>::v8;
  constexpr int XB = 4 * 1024;   // exchange bytes of one 32-row block of one key group (P~, dS: two operands each)
  __shared__ __attribute__((aligned(16))) char stg[3][S::STAGE];
  __shared__ __attribute__((aligned(16))) char xch[4 * 2 * XB];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, lrow = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;
  const bool producer = wave < 4;
  const int kg = wave & 3;

  const int item_idx = blockIdx.x / p.nkv;
  const int gl = blockIdx.x - item_idx * p.nkv;
  const int g = (p.nkv % 8 == 0) ? (gl & 7) * (p.nkv >> 3) + (gl >> 3) : gl;
  const WorkItem it = p.kv_items[item_idx];
  const int b = it.b;
  const int q0 = p.cu_q[b], lq = p.cu_q[b + 1] - q0;
  const int k0 = p.cu_kv[b], lkv = p.cu_kv[b + 1] - k0;
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, lq, lkv, p.prefix[b]);
  const int poff = b == 0 ? p.pse_off0 : 0;   // sequence 0 of mode 8: pse row i + qStartIdx - kvStartIdx
  const int c0 = it.tile * kKvBN;          // first key of the workgroup tile
  const int wc0 = c0 + 32 * kg;            // first key of this wave's group
  const int j = wc0 + lrow;                // this lane's key
  const bool key_ok = j < lkv;
  const int nqt = it.hi - it.lo;
  const int nsteps = p.group * nqt;
  const int64_t q_stride = (int64_t)p.nq * S::RB;
  char* const xkg = xch + kg * 2 * XB + 16 * lane;   // this lane's slots in its key group's exchange area

  // steps walk the query tiles from the last one down, the heads of the group innermost
  auto step_head = [&](int n) { return g * p.group + n % p.group; };
  auto step_row0 = [&](int n) { return (it.hi - 1 - n / p.group) * kKvBM; };
  auto stage = [&](int n) -> char* { return stg[n % 3]; };

  if (producer) {
    // K and V rows of the group's keys as B operands (lane = key, registers = d)
    V8 kf[S::NOP], vf[S::NOP];
    {
      const int64_t kr = (int64_t)(k0 + (key_ok ? j : 0)) * p.nkv + g;
      const E* kp = reinterpret_cast<const E*>(p.k) + kr * D;
      const E* vp = reinterpret_cast<const E*>(p.v) + kr * D;
#pragma unroll
      for (int c = 0; c < S::NOP; ++c) {
        const V8 a = *reinterpret_cast<const V8*>(kp + 16 * c + 8 * hh);
        V8 v = *reinterpret_cast<const V8*>(vp + 16 * c + 8 * hh);
        // without dropout V is held negated (sign bits flipped, exact) and the dP~ accumulator
        // starts at D_i, so the MFMAs leave D_i - dP in it and dS = -P * acc
        if constexpr (!DROP) {
          auto u = __builtin_bit_cast(u32x4, v);
          u ^= 0x80008000u;
          v = __builtin_bit_cast(V8, u);
        }
        kf[c] = key_ok ? a : V8{};
        vf[c] = key_ok ? v : V8{};
      }
    }
    // row reads of chunk 2c + hh of row lrow of a row block: qrow + 16 * ((2c) ^ qsw)
    const int qrow = lrow * S::RB, qsw = tile_swz<S::RB>(lrow) ^ hh;

    // S, dP~ of both row blocks, then P~ and dS written to the exchange area.  Without
    // keep or mask bits the second block's MFMAs are issued before the first block's VALU
    // work, so they run under it; the instances with bits (more registers per element)
    // do one block after the other.
    constexpr bool kSeq = DROP || MASK;
    auto produce = [&](const char* st, int n) {
      const int h = step_head(n), r0 = step_row0(n);
      if (tid == 0)
        FA_TRACE_VISIT(p.trace_kv, (((int64_t)b * p.nq + h) * p.trace_kv_rb + r0 / kKvBM) * p.trace_kv_kt + it.tile);
      const float slope_l2 = pse_slopes(ALIBI) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
      const float sc = p.scale_log2;
      f32x16 s[2], dp[2];
      const float* lse_s = reinterpret_cast<const float*>(st + S::OFF_LSE);
      const float* del_s = reinterpret_cast<const float*>(st + S::OFF_DEL);
      auto sdp = [&](int rb) {
        s[rb] = f32x16{};
        if constexpr (DROP) {
          dp[rb] = f32x16{};
        } else {
          // registers 4a .. 4a + 3 hold rows 32rb + 8a + 4hh .. + 3
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(del_s + 32 * rb + 8 * a + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[rb][4 * a + e] = d4[e];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) {
          const int qo = qrow + 16 * ((2 * c) ^ qsw) + 32 * rb * S::RB;
          const V8 qa = lds_read_b128<V8>(st + qo);
          const V8 ya = lds_read_b128<V8>(st + S::OFF_DY + qo);
          s[rb] = mfma32(qa, kf[c], s[rb]);
          dp[rb] = mfma32(ya, vf[c], dp[rb]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kSpecReadAheadP, 0);
        sched_alternate<2 * S::NOP, 0x008, 0x100>();
        __builtin_amdgcn_sched_barrier(0);
      };
      const uint32_t* bits_s = reinterpret_cast<const uint32_t*>(st + S::OFF_BITS);
      auto elem = [&](auto full_c, int rb) {
        constexpr bool plain = !ALIBI && decltype(full_c)::value;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          V8 pa, da;
#pragma unroll
          for (int a = 2 * c; a < 2 * c + 2; ++a) {
            const int rq = 32 * rb + 8 * a + 4 * hh;   // rows rq .. rq+3 sit in registers 4a .. 4a+3
            const f32x4 lse4 = *reinterpret_cast<const f32x4*>(lse_s + rq);
            f32x4 del4 = {};
            if constexpr (DROP) del4 = *reinterpret_cast<const f32x4*>(del_s + rq);
            u32x4 bits4, mb4 = {};
            if constexpr (DROP) bits4 = *reinterpret_cast<const u32x4*>(bits_s + kg * kKvBM + rq);
            if constexpr (!decltype(full_c)::value && MASK)
              mb4 = *reinterpret_cast<const u32x4*>(st + S::OFF_MBITS + 4 * (kg * kKvBM + rq));
            const float jmi = (float)(j - r0 - rq - poff);   // j - i of register 4a (pse position); minus e for 4a + e
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * a + e, i = r0 + rq + e;
              float pr;
              if constexpr (plain) {
                pr = fast_exp2(__builtin_fmaf(s[rb][r], sc, -lse4[e]));
              } else {
                float x = s[rb][r] * sc;
                if constexpr (ALIBI != 0) x = add_pse<ALIBI>(x, slope_l2, jmi - (float)e);
                if constexpr (!decltype(full_c)::value) {
                  const bool ok = (i < lq) & key_ok & (j >= fa_row_lo(win, i)) & (j <= fa_row_hi(win, i)) &
                                  !((mb4[e] >> lrow) & 1u);
                  x = ok ? x : kNegInf;
                }
                pr = fast_exp2(x - lse4[e]);
              }
              float ptv = pr, dsv;
              if constexpr (DROP) {
                const bool keep = (bits4[e] >> lrow) & 1u;
                const float dpv = keep ? dp[rb][r] * p.inv_keep : 0.f;
                ptv = keep ? pr * p.inv_keep : 0.f;
                dsv = pr * (dpv - del4[e]);
              } else {
                dsv = -(pr * dp[rb][r]);   // the accumulator holds D_i - dP
              }
              pa[r & 7] = cvt16<E>(ptv);
              da[r & 7] = cvt16<E>(dsv);
            }
          }
          *reinterpret_cast<V8*>(xkg + rb * XB + 1024 * c) = pa;
          *reinterpret_cast<V8*>(xkg + rb * XB + 1024 * (2 + c)) = da;
        }
      };
      // with an attenMask every block takes the masked path
      auto softmax = [&](int rb) {
        if (fa_tile_full(win, r0 + 32 * rb, 32, wc0, 32, lq, lkv) && !MASK) elem(std::true_type{}, rb);
        else elem(std::false_type{}, rb);
      };
      if constexpr (kSeq) {
        sdp(0);
        softmax(0);
        sdp(1);
        softmax(1);
      } else {
        sdp(0);
        sdp(1);
        softmax(0);
        softmax(1);
      }
    };

    __syncthreads();   // A: stages of steps 0 and 1 are in
    if (nsteps > 0) produce(stage(0), 0);
    for (int t = 0; t < nsteps; ++t) {
      __syncthreads();   // A: step t's operands and tiles are in
      __syncthreads();   // B: the consumers have taken step t's operands
      if (t + 1 < nsteps) produce(stage(t + 1), t + 1);
    }
  } else {
    const int cw = wave - 4, ctid = tid - 256;
    // transposing reads of rows rv and rv + 8 (+16 per 16-row step), chunk 4db + qv: the
    // offset (rv + 8hf) * RB + 16 * ((4db + qv) ^ swz) + bv equals tx[hf] ^ 64db, because
    // the chunk index enters only bits that the row and byte parts leave clear
    int tx[2];
    {
      const int rv = 4 * (grp >> 1) + (sl >> 2), qv = 2 * (grp & 1) + ((sl & 3) >> 1), bv = 8 * (sl & 1);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        tx[hf] = (rv + 8 * hf) * S::RB + ((16 * qv) ^ (16 * tile_swz<S::RB>(rv + 8 * hf))) + bv;
    }
    f32x16 dk[S::NDB], dv[S::NDB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
      // zeros produced by an MFMA: the accumulators start in the MFMA register class
      dk[db] = mfma32(V8{}, V8{}, f32x16{});
      dv[db] = mfma32(V8{}, V8{}, f32x16{});
    }
    // the four consumer waves copy each step's Q and dY tiles (one set of lane offsets for
    // both: same geometry and row stride), lse2 and D_i
    SwzLane<kKvBM, S::RB, 4> cp;
    cp.init(q_stride, cw, lane);
    auto load = [&](char* st, int n) {
      const int h = step_head(n), r0 = step_row0(n);
      const char* qb = reinterpret_cast<const char*>(p.q) + ((int64_t)q0 * p.nq + h) * S::RB;
      const char* dyb = reinterpret_cast<const char*>(p.dy) + ((int64_t)q0 * p.nq + h) * S::RB;
      cp.copy(st, qb, q_stride, r0, lq, cw, lane);
      cp.copy(st + S::OFF_DY, dyb, q_stride, r0, lq, cw, lane);
      if (cw < 2) {
        const int rr = (r0 + lane < lq) ? r0 + lane : 0;
        dma_dword(st + (cw == 0 ? S::OFF_LSE : S::OFF_DEL), cw == 0 ? p.lse : p.delta,
                  (uint32_t)(((int64_t)(q0 + rr) * p.nq + h) * 4));
      }
    };
    // keep bits (and attenMask bits) of a step: 64 rows x 128 keys = 256 words, one per consumer thread
    const int bits_slot = (ctid & 3) * kKvBM + ((ctid >> 2) & (kKvBM - 1));
    auto bits_word = [&](int n) -> uint32_t {
      const int h = step_head(n), r0 = step_row0(n);
      const int r = (ctid >> 2) & (kKvBM - 1), w = ctid & 3;
      if (r0 + r >= lq) return 0u;
      const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + r0 + r) * lkv + c0 + 32 * w;
      return (uint32_t)load_mask_window(p.drop, p.drop_bytes, pos);
    };
    auto mask_word = [&](int n) -> uint32_t {
      const int r0 = step_row0(n);
      const int r = (ctid >> 2) & (kKvBM - 1), w = (c0 >> 5) + (ctid & 3);
      if (r0 + r >= lq || w >= p.mwords) return ~0u;
      return p.mbits[(int64_t)(r0 + r) * p.mwords + w];
    };
    auto put_words = [&](char* st, uint32_t word, uint32_t mword) {
      if constexpr (DROP) reinterpret_cast<uint32_t*>(st + S::OFF_BITS)[bits_slot] = word;
      if constexpr (MASK) reinterpret_cast<uint32_t*>(st + S::OFF_MBITS)[bits_slot] = mword;
    };
    // step t's P~ and dS operands, [row block][c], taken out of the exchange area
    V8 pt[2][2], ds[2][2];
    auto take = [&]() {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          pt[blk][c] = *reinterpret_cast<const V8*>(xkg + blk * XB + 1024 * c);
          ds[blk][c] = *reinterpret_cast<const V8*>(xkg + blk * XB + 1024 * (2 + c));
        }
    };
    // dV += P~^T dY, dK += dS^T Q over both row blocks and all of D
    auto consume = [&](const char* st) {
      // fresh copies of the offset bases, so their XORs are formed per use, not hoisted into tables
      int tx0 = tx[0], tx1 = tx[1];
      asm volatile("" : "+v"(tx0), "+v"(tx1));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const char* base = st + (32 * blk + 16 * c) * S::RB;
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            const int o0 = tx0 ^ (64 * db), o1 = tx1 ^ (64 * db);
            const V8 yo = lds_read_tr_x2<V8>(base + S::OFF_DY + o0, base + S::OFF_DY + o1);
            const V8 qo = lds_read_tr_x2<V8>(base + o0, base + o1);
            dv[db] = mfma32(pt[blk][c], yo, dv[db]);
            dk[db] = mfma32(ds[blk][c], qo, dk[db]);
          }
        }
      __builtin_amdgcn_sched_group_barrier(0x100, kSpecReadAheadC, 0);
      sched_alternate<8 * S::NDB, 0x008, 0x100, 2>();
      __builtin_amdgcn_sched_barrier(0);
    };

    uint32_t word = 0, mword = 0;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      if (n < nsteps) {
        load(stage(n), n);
        if constexpr (DROP) word = bits_word(n);
        if constexpr (MASK) mword = mask_word(n);
        put_words(stage(n), word, mword);
      }
    }
    dma_wait();
    __syncthreads();   // A: stages of steps 0 and 1 are in
    for (int t = 0; t < nsteps; ++t) {
      __syncthreads();   // A: step t's operands and tiles are in
      take();
      __syncthreads();   // B: the producers may overwrite the exchange area
      if (t + 2 < nsteps) {
        load(stage(t + 2), t + 2);
        if constexpr (DROP) word = bits_word(t + 2);
        if constexpr (MASK) mword = mask_word(t + 2);
      }
      consume(stage(t));
      if (t + 2 < nsteps) put_words(stage(t + 2), word, mword);
      dma_wait();
    }

    // ---- epilogue: dK *= scale; write dK, dV of the group's keys (lane = d, registers = keys) ----
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jj = wc0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (jj < lkv) {
          const int64_t off = ((int64_t)(k0 + jj) * p.nkv + g) * D + 32 * db + lrow;
          reinterpret_cast<E*>(p.dk)[off] = cvt16<E>(dk[db][r] * p.scale);
          reinterpret_cast<E*>(p.dv)[off] = cvt16<E>(dv[db][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- 16 waves: two producers, two consumers per SIMD
// LDS operand reads issued ahead of the first MFMA of a producer / consumer matrix phase
constexpr int kQuadReadAheadP = 4, kQuadReadAheadC = 8;
// 16-bit deterministic dK/dV without dropout, attenMask or pse: the workgroup and its tiles
// are those of fa_bwd_kv_spec_kernel (one 128-key tile of one kv head, 64-row steps, three
// Q/dY stages, one exchange area), run by 16 waves, four per SIMD (key group kg = wave % 4):
//   wave kg      producer of row block 0 (rows 0-31 of a step),
//   wave kg + 4  producer of row block 1 (rows 32-63),
//     each holding K and V (negated) of the group's 32 keys; it forms S and D_i - dP of its
//     block, then P~ and dS, and writes them to its half of the group's exchange area;
//   wave kg + 8  consumer holding dV of the group's keys over all of D (dV += P~^T dY),
//   wave kg + 12 consumer holding dK (dK += dS^T Q);
//     the eight consumers issue the tile copies two steps ahead.
// Each producer's serial chain (16 MFMAs, then the softmax / dS of 16 elements per lane) is
// half that of a spec-kernel producer, and four waves per SIMD give the issue logic more to
// interleave; each wave has 128 registers.  Same two barriers per tick.
template <typename E, int D>
__global__ __launch_bounds__(1024, 1) void fa_bwd_kv_quad_kernel(BwdParams p) {
  using S = KvShape<E, D>;
  using V8 = typename Vec16<E>::v8;
  constexpr int XB = 4 * 1024;   // exchange bytes of one 32-row block of one key group (P~, dS: two operands each)
  __shared__ __attribute__((aligned(16))) char stg[3][S::STAGE];
  __shared__ __attribute__((aligned(16))) char xch[4 * 2 * XB];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, lrow = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;
  const int role = wave >> 2;   // 0, 1: producer of that row block; 2: dV consumer; 3: dK consumer
  const int kg = wave & 3;

  const int item_idx = blockIdx.x / p.nkv;
  const int gl = blockIdx.x - item_idx * p.nkv;
  const int g = (p.nkv % 8 == 0) ? (gl & 7) * (p.nkv >> 3) + (gl >> 3) : gl;
  const WorkItem it = p.kv_items[item_idx];
  const int b = it.b;
  const int q0 = p.cu_q[b], lq = p.cu_q[b + 1] - q0;
  const int k0 = p.cu_kv[b], lkv = p.cu_kv[b + 1] - k0;
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, lq, lkv, p.prefix[b]);
  const int c0 = it.tile * kKvBN;          // first key of the workgroup tile
  const int wc0 = c0 + 32 * kg;            // first key of this wave's group
  const int j = wc0 + lrow;                // this lane's key
  const bool key_ok = j < lkv;
  const int nqt = it.hi - it.lo;
  const int nsteps = p.group * nqt;
  const int64_t q_stride = (int64_t)p.nq * S::RB;
  char* const xkg = xch + kg * 2 * XB + 16 * lane;   // this lane's slots in its key group's exchange area

  // steps walk the query tiles from the last one down, the heads of the group innermost
  auto step_head = [&](int n) { return g * p.group + n % p.group; };
  auto step_row0 = [&](int n) { return (it.hi - 1 - n / p.group) * kKvBM; };
  auto stage = [&](int n) -> char* { return stg[n % 3]; };

  if (role < 2) {
    const int rb = role;   // wave-uniform
    // K and V rows of the group's keys as B operands (lane = key, registers = d); V negated
    // (sign bits flipped, exact), so that the dP~ accumulator, started at D_i, ends at D_i - dP
    V8 kf[S::NOP], vf[S::NOP];
    {
      const int64_t kr = (int64_t)(k0 + (key_ok ? j : 0)) * p.nkv + g;
      const E* kp = reinterpret_cast<const E*>(p.k) + kr * D;
      const E* vp = reinterpret_cast<const E*>(p.v) + kr * D;
#pragma unroll
      for (int c = 0; c < S::NOP; ++c) {
        const V8 a = *reinterpret_cast<const V8*>(kp + 16 * c + 8 * hh);
        auto u = __builtin_bit_cast(u32x4, *reinterpret_cast<const V8*>(vp + 16 * c + 8 * hh));
        u ^= 0x80008000u;
        kf[c] = key_ok ? a : V8{};
        vf[c] = key_ok ? __builtin_bit_cast(V8, u) : V8{};
      }
    }
    // rows [i_lo, i_hi] of the sequence may see this lane's key j (j <= hi(i) holds for every row
    // when j <= floor, else from row j - delta - next on; j >= lo(i) up to row j - delta + pre); an
    // empty range for a key past the end, so the masked path tests a row with two compares
    const int i_lo = j <= win.floor ? 0 : j - win.delta - win.next;
    const int i_hi = key_ok ? min(j - win.delta + win.pre, lq - 1) : -1;
    // row reads of chunk 2c + hh of row lrow of this row block sit at row * RB + 16 * ((2c) ^ qsw),
    // qsw = swz(row) ^ hh; the chunk index only enters bits the row part leaves clear, so the
    // offset is kx ^ 32c
    const int kx = (32 * rb + lrow) * S::RB + 16 * (tile_swz<S::RB>(lrow) ^ hh);

    auto produce = [&](const char* st, int n) {
      const int h = step_head(n), r0 = step_row0(n);
      if (tid == 0)
        FA_TRACE_VISIT(p.trace_kv, (((int64_t)b * p.nq + h) * p.trace_kv_rb + r0 / kKvBM) * p.trace_kv_kt + it.tile);
      const float sc = p.scale_log2;
      const float* lse_s = reinterpret_cast<const float*>(st + S::OFF_LSE) + 32 * rb;
      const float* del_s = reinterpret_cast<const float*>(st + S::OFF_DEL) + 32 * rb;
      f32x16 sv = f32x16{}, dp;
      // registers 4a .. 4a + 3 hold rows 8a + 4hh .. + 3 of the block
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(del_s + 8 * a + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * a + e] = d4[e];
      }
      // a fresh copy of the offset base per step, so the XORs are formed per use, not kept in a table
      int kxl = kx;
      asm volatile("" : "+v"(kxl));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < S::NOP; ++c) {
        const int qo = kxl ^ (32 * c);
        const V8 qa = lds_read_b128<V8>(st + qo);
        const V8 ya = lds_read_b128<V8>(st + S::OFF_DY + qo);
        sv = mfma32(qa, kf[c], sv);
        dp = mfma32(ya, vf[c], dp);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kQuadReadAheadP, 0);
      sched_alternate<2 * S::NOP, 0x008, 0x100>();
      __builtin_amdgcn_sched_barrier(0);
      const int rr0 = r0 + 32 * rb;   // first row of the block
      auto elem = [&](auto full_c) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          V8 pa, da;
#pragma unroll
          for (int a = 2 * c; a < 2 * c + 2; ++a) {
            const int rq = 8 * a + 4 * hh;   // rows rq .. rq+3 of the block sit in registers 4a .. 4a+3
            const f32x4 lse4 = *reinterpret_cast<const f32x4*>(lse_s + rq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * a + e, i = rr0 + rq + e;
              float pr;
              if constexpr (decltype(full_c)::value) {
                pr = fast_exp2(__builtin_fmaf(sv[r], sc, -lse4[e]));
              } else {
                const bool ok = (i >= i_lo) & (i <= i_hi);
                pr = fast_exp2((ok ? sv[r] * sc : kNegInf) - lse4[e]);
              }
              pa[r & 7] = cvt16<E>(pr);
              da[r & 7] = cvt16<E>(-(pr * dp[r]));   // dS = P (dP - D_i)
            }
          }
          *reinterpret_cast<V8*>(xkg + rb * XB + 1024 * c) = pa;
          *reinterpret_cast<V8*>(xkg + rb * XB + 1024 * (2 + c)) = da;
        }
      };
      if (fa_tile_full(win, rr0, 32, wc0, 32, lq, lkv)) elem(std::true_type{});
      else elem(std::false_type{});
    };

    __syncthreads();   // A: stages of steps 0 and 1 are in
    if (nsteps > 0) produce(stage(0), 0);
    for (int t = 0; t < nsteps; ++t) {
      __syncthreads();   // A: step t's operands and tiles are in
      __syncthreads();   // B: the consumers have taken step t's operands
      if (t + 1 < nsteps) produce(stage(t + 1), t + 1);
    }
  } else {
    const int cw = wave - 8;            // copy slot of this consumer, 0 .. 7
    const bool dv_role = role == 2;     // wave-uniform
    const int y_off = dv_role ? S::OFF_DY : 0;   // B operand: dY (dV) or Q (dK)
    const int x_off = dv_role ? 0 : 2 * 1024;    // A operand: P~ (dV) or dS (dK)
    // transposing reads of rows rv and rv + 8 (+16 per 16-row step), chunk 4db + qv: the
    // offset (rv + 8hf) * RB + 16 * ((4db + qv) ^ swz) + bv equals tx[hf] ^ 64db, because
    // the chunk index enters only bits that the row and byte parts leave clear
    int tx[2];
    {
      const int rv = 4 * (grp >> 1) + (sl >> 2), qv = 2 * (grp & 1) + ((sl & 3) >> 1), bv = 8 * (sl & 1);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        tx[hf] = (rv + 8 * hf) * S::RB + ((16 * qv) ^ (16 * tile_swz<S::RB>(rv + 8 * hf))) + bv;
    }
    f32x16 acc[S::NDB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) acc[db] = mfma32(V8{}, V8{}, f32x16{});   // zeros in the MFMA register class
    // the eight consumer waves copy each step's Q and dY tiles (one set of lane offsets for
    // both: same geometry and row stride), lse2 and D_i
    SwzLane<kKvBM, S::RB, 8> cp;
    cp.init(q_stride, cw, lane);
    auto load = [&](char* st, int n) {
      const int h = step_head(n), r0 = step_row0(n);
      const char* qb = reinterpret_cast<const char*>(p.q) + ((int64_t)q0 * p.nq + h) * S::RB;
      const char* dyb = reinterpret_cast<const char*>(p.dy) + ((int64_t)q0 * p.nq + h) * S::RB;
      cp.copy(st, qb, q_stride, r0, lq, cw, lane);
      cp.copy(st + S::OFF_DY, dyb, q_stride, r0, lq, cw, lane);
      if (cw < 2) {
        const int rr = (r0 + lane < lq) ? r0 + lane : 0;
        dma_dword(st + (cw == 0 ? S::OFF_LSE : S::OFF_DEL), cw == 0 ? p.lse : p.delta,
                  (uint32_t)(((int64_t)(q0 + rr) * p.nq + h) * 4));
      }
    };
    // step t's A operands ([row block][c]), taken out of the exchange area
    V8 op[2][2];
    auto take = [&]() {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int c = 0; c < 2; ++c) op[blk][c] = *reinterpret_cast<const V8*>(xkg + blk * XB + x_off + 1024 * c);
    };
    // acc += op^T B over both row blocks and all of D
    auto consume = [&](const char* st) {
      int tx0 = tx[0], tx1 = tx[1];
      asm volatile("" : "+v"(tx0), "+v"(tx1));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const char* base = st + y_off + (32 * blk + 16 * c) * S::RB;
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            const V8 bo = lds_read_tr_x2<V8>(base + (tx0 ^ (64 * db)), base + (tx1 ^ (64 * db)));
            acc[db] = mfma32(op[blk][c], bo, acc[db]);
          }
        }
      __builtin_amdgcn_sched_group_barrier(0x100, kQuadReadAheadC, 0);
      sched_alternate<4 * S::NDB, 0x008, 0x100, 2>();
      __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int n = 0; n < 2; ++n)
      if (n < nsteps) load(stage(n), n);
    dma_wait();
    __syncthreads();   // A: stages of steps 0 and 1 are in
    for (int t = 0; t < nsteps; ++t) {
      __syncthreads();   // A: step t's operands and tiles are in
      take();
      __syncthreads();   // B: the producers may overwrite the exchange area
      if (t + 2 < nsteps) load(stage(t + 2), t + 2);
      consume(stage(t));
      dma_wait();
    }

    // ---- epilogue: dK = scale * acc or dV = acc for the group's keys (lane = d, registers = keys) ----
    E* out = reinterpret_cast<E*>(dv_role ? p.dv : p.dk);
    const float f = dv_role ? 1.f : p.scale;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jj = wc0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (jj < lkv) out[((int64_t)(k0 + jj) * p.nkv + g) * D + 32 * db + lrow] = cvt16<E>(acc[db][r] * f);
      }
    }
  }
}

}  // namespace fa
