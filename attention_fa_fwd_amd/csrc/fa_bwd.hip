// Backward attention kernels for gfx950.
//
// Gradients of aclnnFlashAttentionUnpaddingScoreGrad ("Formula"):
//   dV = P~^T dY,  dQ = scale * dS K,  dK = scale * dS^T Q,
// with dS the softmax Jacobian applied through dropout,
//   dP = (dY V^T) * z / keep,  dS = P * (dP - D_i),  D_i = rowsum(dY * O),
// and the sink gradient of aclnnFlashAttentionUnpaddingScoreGradV5 (sink formulas),
//   dSink_h = -sum_i e^(sink_h - m_i) / l_i * D_i.
// P is recomputed from the forward's softmax max/sum: P = 2^(x - lse2) with x the
// log2-domain logit and lse2 = m*log2(e) + log2(l).
//
// Kernels, in launch order:
//   fa_bwd_pre_kernel   D_i, lse2 per (row, head) and per-block dSink partials
//   fa_bwd_kv_kernel    one 128-key tile of one kv head per workgroup; loops over
//                       the heads of its GQA group and every query tile with an
//                       allowed pair; dK, dV accumulate in registers (no atomics);
//                       optionally also dQ += dS K with fp32 atomics
//   fa_bwd_dq_kernel    deterministic dQ: one 128-row query tile per workgroup,
//                       recomputes S, dP, dS over its key tiles, dQ in registers
//   fa_dq_convert_kernel, fa_dsink_reduce_kernel, fa_zero_kernel
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

#ifndef FA_KV_OVERLAP
#define FA_KV_OVERLAP 0
#endif

// ------------------------------------------------------------------ preprocess
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(BwdParams p) {
  constexpr int EB = sizeof(T);
  constexpr int CPR = D * EB / 16;        // 16-byte chunks per (row, head)
  constexpr int GROUPS = 256 / CPR;       // (row, head) pairs processed at once
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* part = reinterpret_cast<float*>(smem);   // [GROUPS][nq]
  const int tid = threadIdx.x;
  const int grp = tid / CPR, sub = tid % CPR;
  const int nq = p.nq;
  for (int x = tid; x < GROUPS * nq; x += 256) part[x] = 0.f;
  __syncthreads();
  const int64_t row0 = (int64_t)blockIdx.x * kPreRowsPerBlock;
  const int64_t rows = min((int64_t)kPreRowsPerBlock, (int64_t)p.total_q - row0);
  const int64_t npairs = rows * nq;
  const char* dyb = reinterpret_cast<const char*>(p.dy);
  const char* ob = reinterpret_cast<const char*>(p.o);
  constexpr int U = 4;   // pairs in flight per thread
  for (int64_t pb = grp; pb < npairs; pb += GROUPS * U) {
    u32x4 av[U], cv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t pi = pb + (int64_t)u * GROUPS;
      const int64_t idx = row0 * nq + (pi < npairs ? pi : pb);
      av[u] = *reinterpret_cast<const u32x4*>(dyb + idx * (D * EB) + sub * 16);
      cv[u] = *reinterpret_cast<const u32x4*>(ob + idx * (D * EB) + sub * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
    const int64_t pi = pb + (int64_t)u * GROUPS;
    if (pi >= npairs) break;
    const int64_t idx = row0 * nq + pi;            // (t * nq + h)
    const int h = (int)(pi % nq);
    const u32x4 a = av[u];
    const u32x4 c = cv[u];
    float acc = 0.f;
    if constexpr (EB == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc += bf16_bits_to_f32((uint16_t)(a[w] & 0xffff)) * bf16_bits_to_f32((uint16_t)(c[w] & 0xffff));
        acc += bf16_bits_to_f32((uint16_t)(a[w] >> 16)) * bf16_bits_to_f32((uint16_t)(c[w] >> 16));
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += __uint_as_float(a[w]) * __uint_as_float(c[w]);
    }
    // reduce over the CPR lanes of this pair (contiguous, power of two, inside one wave)
#pragma unroll
    for (int o = CPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (sub == 0) {
      const float m = p.m_in[idx], l = p.l_in[idx];
      p.delta[idx] = acc;
      p.lse[idx] = l > 0.f ? m * kLog2e + __log2f(l) : __builtin_inff();
      if (p.sink && l > 0.f) part[grp * nq + h] -= fast_exp2((p.sink[h] - m) * kLog2e) / l * acc;
    }
    }
  }
  if (p.sink) {
    __syncthreads();
    for (int h = tid; h < nq; h += 256) {
      float s = 0.f;
      for (int gi = 0; gi < GROUPS; ++gi) s += part[gi * nq + h];
      p.dsink_part[(int64_t)blockIdx.x * nq + h] = s;
    }
  }
}

// dSink of head blockIdx.x: thread t sums partial blocks t, t + 256, ... in
// order, then a fixed tree adds the 256 thread sums (bitwise reproducible).
__global__ __launch_bounds__(256) void fa_dsink_reduce_kernel(const float* part, int nblocks, int nq, float* out) {
  __shared__ float red[256];
  const int h = blockIdx.x, t = threadIdx.x;
  float s = 0.f;
  for (int b = t; b < nblocks; b += 256) s += part[(int64_t)b * nq + h];
  red[t] = s;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) out[h] = red[0];
}

__global__ __launch_bounds__(256) void fa_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

template <typename T>
__global__ __launch_bounds__(256) void fa_dq_convert_kernel(const float* acc, T* out, float scale, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    if constexpr (sizeof(T) == 2)
      out[i] = to_bf16(acc[i] * scale);
    else
      out[i] = acc[i] * scale;
  }
}

// ------------------------------------------------------------------ dK / dV (+ atomic dQ)
template <typename T, int D>
struct KvShape {
  static constexpr int EB = sizeof(T);
  static constexpr int RB = D * EB;
  // bf16 Q / dY tiles are swizzled and unpadded (see tile_swz); fp32 tiles and
  // the K tile of the atomic variant use padded rows
  static constexpr bool kSwz = EB == 2;
  static constexpr int P = kSwz ? RB : RB + 16;     // LDS pitch of Q / dY rows
  static constexpr int KTP = RB + 16;               // LDS pitch of K rows (atomic dQ)
  static constexpr int QT = kKvBM * P;              // one 64-row Q (or dY) tile
  // stage layout: Q | dY | lse2[64] | D_i[64] | keep bits[64][4]
  static constexpr int OFF_DY = QT;
  static constexpr int OFF_LSE = 2 * QT;
  static constexpr int OFF_DEL = OFF_LSE + 4 * kKvBM;
  static constexpr int OFF_BITS = OFF_DEL + 4 * kKvBM;
  static constexpr int STAGE = OFF_BITS + 16 * kKvBM;
  static constexpr int KT = kKvBN * KTP;            // the 128-key K tile (atomic dQ only)
  static constexpr int DSP = kKvBM * EB + 16;       // pitch of dS^T rows (one row per key)
  static constexpr int DST = kKvBN * DSP;
  static constexpr int NOP = D / ElemTraits<T>::kChunk;
  static constexpr int NDB = D / 32;
};

template <typename T, int D, bool ATOMIC, bool DROP, bool ALIBI>
__global__ __launch_bounds__(256, 1) void fa_bwd_kv_kernel(BwdParams p) {
  using S = KvShape<T, D>;
  using Op = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
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
  const FaWindow win = fa_make_window(p.mode, p.pre, p.next, lq, lkv);
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
        bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + 16 * c + 8 * hh);
        bf16x8 v = *reinterpret_cast<const bf16x8*>(vp + 16 * c + 8 * hh);
        kf[c] = key_ok ? a : bf16x8{};
        vf[c] = key_ok ? v : bf16x8{};
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
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int nqt = it.hi - it.lo;
  const int nsteps = p.group * nqt;
  const int64_t q_stride = (int64_t)p.nq * S::RB;
  // per-lane LDS offsets: A-operand row reads and transposing B-operand reads
  const int a_lane = lrow * S::P + 16 * hh;
  const int t_lane = (4 * (grp >> 1) + (sl >> 2)) * S::P + (16 * (grp & 1) + 4 * (sl & 3)) * 2;
  // swizzled bf16 tiles: row reads of chunk 2c + hh of row lrow (+32 per row
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

  // atomic dQ of one bf16 step: store_ds() puts each block's dS^T into LDS right
  // after it is formed; atomic_dq() then adds dQ(64 rows x 32-wide d block of this
  // wave) += dS K over the 128 keys to the fp32 accumulator
  auto store_ds = [&](int rb, const auto& d) {
    // register 8c + 4t + e holds row 32rb + 16c + 8t + 4hh + e
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = d[c][4 * t2 + e];
        *reinterpret_cast<bf16x4*>(dst + (32 * wave + lrow) * S::DSP + (32 * rb + 16 * c + 8 * t2 + 4 * hh) * 2) = v;
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
        const bf16x8 a0 = lds_read_tr_x2(dst + krow * S::DSP + coln, dst + (krow + 8) * S::DSP + coln);
        const bf16x8 a1 = lds_read_tr_x2(dst + krow * S::DSP + coln + 64, dst + (krow + 8) * S::DSP + coln + 64);
        const int colk = (dcol + 16 * (grp & 1) + 4 * (sl & 3)) * 2;
        const bf16x8 bo = lds_read_tr_x2(kt + krow * S::KTP + colk, kt + (krow + 8) * S::KTP + colk);
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
  // ---- bf16 steps: software pipeline over the step's two 32-row blocks ----
  //   [S, dP of block 0]  [S, dP of block 1 | P, dS of block 0]
  //   [dV, dK of block 0 | P, dS of block 1]  [dV, dK of block 1]
  // Scheduling-group barriers interleave each region's matrix work with the
  // VALU work beside it and keep the LDS reads a few MFMAs ahead of their use.
  // Blocks outside the mask are computed like masked ones (every probability
  // is zero): the waves of a workgroup wait for each other at every step anyway.
  auto sdp = [&](const char* st, int rb, auto& s, auto& dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int c = 0; c < S::NOP; ++c) {
      const bf16x8 qa = lds_read_b128(st + qoff[c] + 32 * rb * S::RB);
      const bf16x8 ya = lds_read_b128(st + S::OFF_DY + qoff[c] + 32 * rb * S::RB);
      s = mfma32(qa, kf[c], s);
      dp = mfma32(ya, vf[c], dp);
    }
  };
  // P~ and dS of one block as bf16 A operands (lane = key, registers = rows)
  auto elem = [&](auto full_c, const char* st, int r0, int rb, const f32x16& s, const f32x16& dp, float slope_l2,
                  bf16x8 (&pa)[2], bf16x8 (&da)[2]) {
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
      u32x4 bits4;
      if constexpr (DROP) bits4 = *reinterpret_cast<const u32x4*>(bits_s + wave * kKvBM + rq);
      const float jmi = (float)(j - r0 - rq);   // j - i of register 4a; minus e for register 4a + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a + e, rr = rq + e, i = r0 + rr;
        float pr;
        if constexpr (plain) {
          pr = fast_exp2(__builtin_fmaf(s[r], sc, -lse4[e]));
        } else {
          float x = s[r] * sc;
          if constexpr (ALIBI) x = __builtin_fmaf(slope_l2, jmi - (float)e, x);
          if constexpr (!decltype(full_c)::value) {
            const bool ok = (i < lq) & key_ok & (j >= fa_row_lo(win, i)) & (j <= fa_row_hi(win, i));
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
        pa[r >> 3][r & 7] = to_bf16(ptv);
        da[r >> 3][r & 7] = to_bf16(dsv);
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
        const bf16x8 yo = lds_read_tr_x2(base + S::OFF_DY + toff[0][db], base + S::OFF_DY + toff[1][db]);
        const bf16x8 qo = lds_read_tr_x2(base + toff[0][db], base + toff[1][db]);
        dv[db] = mfma32(pa[c], yo, dv[db]);
        dk[db] = mfma32(da[c], qo, dk[db]);
      }
    }
  };
  constexpr int kSdpMfma = 2 * S::NOP, kSdpReads = 2 * S::NOP;
  constexpr int kGradMfma = 4 * S::NDB, kGradReads = 8 * S::NDB;
  constexpr int kElemValu = DROP ? 160 : (ALIBI ? 120 : 90);

  auto compute_bf16 = [&](const char* st, auto n) {
    const int h = step_head(n), r0 = step_row0(n);
    const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
    const bool full0 = fa_tile_full(win, r0, 32, wc0, 32, lq, lkv);
    const bool full1 = fa_tile_full(win, r0 + 32, 32, wc0, 32, lq, lkv);
    f32x16 s0, dp0, s1, dp1;
    bf16x8 pa0[2], da0[2], pa1[2], da1[2];
#if FA_KV_OVERLAP
    __builtin_amdgcn_sched_barrier(0);
    sdp(st, 0, s0, dp0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    sched_alternate<kSdpMfma, 0x008, 0x100>();
    __builtin_amdgcn_sched_barrier(0);
    auto region2 = [&](auto full_c) {
      elem(full_c, st, r0, 0, s0, dp0, slope_l2, pa0, da0);
      if constexpr (ATOMIC) store_ds(0, da0);
      sdp(st, 1, s1, dp1);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      sched_alternate3<kSdpMfma, 0x008, 1, 0x002, kElemValu / kSdpMfma, 0x100, 1>();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (full0) region2(std::true_type{});
    else region2(std::false_type{});
    auto region3 = [&](auto full_c) {
      elem(full_c, st, r0, 1, s1, dp1, slope_l2, pa1, da1);
      if constexpr (ATOMIC) store_ds(1, da1);
      grads(st, 0, pa0, da0);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      sched_alternate3<kGradMfma, 0x008, 1, 0x002, kElemValu / kGradMfma, 0x100, 2>();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (full1) region3(std::true_type{});
    else region3(std::false_type{});
    grads(st, 1, pa1, da1);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    sched_alternate<kGradMfma, 0x008, 0x100, 2>();
    __builtin_amdgcn_sched_barrier(0);
#else
    auto block = [&](int rb, bool full, auto& sx, auto& dpx, auto& pax, auto& dax) {
      __builtin_amdgcn_sched_barrier(0);
      sdp(st, rb, sx, dpx);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      sched_alternate<kSdpMfma, 0x008, 0x100>();
      __builtin_amdgcn_sched_barrier(0);
      if (full) elem(std::true_type{}, st, r0, rb, sx, dpx, slope_l2, pax, dax);
      else elem(std::false_type{}, st, r0, rb, sx, dpx, slope_l2, pax, dax);
      if constexpr (ATOMIC) store_ds(rb, dax);
      __builtin_amdgcn_sched_barrier(0);
      grads(st, rb, pax, dax);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      sched_alternate<kGradMfma, 0x008, 0x100, 2>();
      __builtin_amdgcn_sched_barrier(0);
    };
    block(0, full0, s0, dp0, pa0, da0);
    block(1, full1, s1, dp1, pa1, da1);
#endif
    if constexpr (ATOMIC) atomic_dq(n);
  };

  auto compute = [&](const char* st, int n) {
    const int h = step_head(n), r0 = step_row0(n);
    const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
    const float* lse_s = reinterpret_cast<const float*>(st + S::OFF_LSE);
    const float* del_s = reinterpret_cast<const float*>(st + S::OFF_DEL);
    const uint32_t* bits_s = reinterpret_cast<const uint32_t*>(st + S::OFF_BITS);
    bf16x8 da_keep[2][2];   // dS of both row blocks (atomic dQ)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int rb0 = r0 + 32 * rb;
      bool empty = rb0 >= lq || wc0 >= lkv;
      if (!empty) empty = fa_tile_empty(win, rb0, min(rb0 + 32, lq), wc0, min(wc0 + 32, lkv));
      if constexpr (ATOMIC && sizeof(T) == 2) {
        da_keep[rb][0] = bf16x8{};
        da_keep[rb][1] = bf16x8{};
      }
      if (empty) continue;
      const bool full = fa_tile_full(win, rb0, 32, wc0, 32, lq, lkv);
      // ---- S = Q K^T and dP~ = dY V^T (lane = key, registers = rows) ----
      f32x16 s = f32x16{}, dp = f32x16{};
      if constexpr (sizeof(T) == 2) {
        bf16x8 qa[S::NOP];
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) qa[c] = lds_read_b128(st + a_lane + 32 * rb * S::P + 32 * c);
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) s = mfma32(qa[c], kf[c], s);
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) qa[c] = lds_read_b128(st + S::OFF_DY + a_lane + 32 * rb * S::P + 32 * c);
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
        if constexpr (ALIBI) x = __builtin_fmaf(slope_l2, (float)(j - (r0 + rr)), x);
        if (!full && !fa_allowed(win, r0 + rr, j, lq, lkv)) x = kNegInf;
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
          bf16x8 pa, da;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pa[e] = to_bf16(pt[8 * c + e]);
            da[e] = to_bf16(ds[8 * c + e]);
          }
          if constexpr (ATOMIC) da_keep[rb][c] = da;
          const char* base = st + t_lane + (32 * rb + 16 * c) * S::P;
          bf16x8 dyo[S::NDB], qo[S::NDB];
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            dyo[db] = lds_read_tr_x2(base + S::OFF_DY + 64 * db, base + S::OFF_DY + 8 * S::P + 64 * db);
            qo[db] = lds_read_tr_x2(base + 64 * db, base + 8 * S::P + 64 * db);
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
        // dS^T[key][row] from the kept bf16 operands: register 8c + 4t + e holds row 16c + 8t + 4hh + e
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              bf16x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = da_keep[rb][c][4 * t2 + e];
              *reinterpret_cast<bf16x4*>(dst + (32 * wave + lrow) * S::DSP +
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
            const bf16x8 a0 = lds_read_tr_x2(dst + krow * S::DSP + coln, dst + (krow + 8) * S::DSP + coln);
            const bf16x8 a1 = lds_read_tr_x2(dst + krow * S::DSP + coln + 64, dst + (krow + 8) * S::DSP + coln + 64);
            const int colk = (dcol + 16 * (grp & 1) + 4 * (sl & 3)) * 2;
            const bf16x8 bo = lds_read_tr_x2(kt + krow * S::KTP + colk, kt + (krow + 8) * S::KTP + colk);
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
  uint32_t word = 0;
  if constexpr (DROP) {
    if (nsteps > 0) word = bits_word(0);
    reinterpret_cast<uint32_t*>(st0 + S::OFF_BITS)[bits_slot] = word;
  }
  dma_wait();
  __syncthreads();
  for (int n = 0; n < nsteps; n += 2) {
    if (n + 1 < nsteps) {
      load(st1, n + 1);
      if constexpr (DROP) word = bits_word(n + 1);
    }
    if constexpr (sizeof(T) == 2) compute_bf16(st0, n);
    else compute(st0, n);
    if constexpr (DROP)
      if (n + 1 < nsteps) reinterpret_cast<uint32_t*>(st1 + S::OFF_BITS)[bits_slot] = word;
    dma_wait();
    __syncthreads();
    if (n + 1 < nsteps) {
      if (n + 2 < nsteps) {
        load(st0, n + 2);
        if constexpr (DROP) word = bits_word(n + 2);
      }
      if constexpr (sizeof(T) == 2) compute_bf16(st1, n + 1);
      else compute(st1, n + 1);
      if constexpr (DROP)
        if (n + 2 < nsteps) reinterpret_cast<uint32_t*>(st0 + S::OFF_BITS)[bits_slot] = word;
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
          reinterpret_cast<__bf16*>(p.dk)[off] = to_bf16(dk[db][r] * p.scale);
          reinterpret_cast<__bf16*>(p.dv)[off] = to_bf16(dv[db][r]);
        } else {
          reinterpret_cast<float*>(p.dk)[off] = dk[db][r] * p.scale;
          reinterpret_cast<float*>(p.dv)[off] = dv[db][r];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ deterministic dQ
template <typename T, int D>
struct DqShape {
  static constexpr int EB = sizeof(T);
  static constexpr int RB = D * EB;
  static constexpr bool kSwz = EB == 2;     // bf16 tiles swizzled and unpadded
  static constexpr int P = kSwz ? RB : RB + 16;
  static constexpr int TILE = kDqBN * P;
  static constexpr int STAGE = 2 * TILE;    // K | V
  static constexpr int NOP = D / ElemTraits<T>::kChunk;
  static constexpr int NDB = D / 32;
};

template <typename T, int D, bool DROP, bool ALIBI>
__global__ __launch_bounds__(256, DROP ? 1 : 2) void fa_bwd_dq_kernel(BwdParams p) {
  using S = DqShape<T, D>;
  using Op = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
  __shared__ __attribute__((aligned(16))) char st0[S::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[S::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, lrow = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;

  const int item_idx = blockIdx.x / p.nq;
  const int hl = blockIdx.x - item_idx * p.nq;
  const int h = p.head_swizzle ? (hl & 7) * (p.nq >> 3) + (hl >> 3) : hl;
  const int g = h / p.group;
  const WorkItem it = p.dq_items[item_idx];
  const int b = it.b;
  const int q0 = p.cu_q[b], lq = p.cu_q[b + 1] - q0;
  const int k0 = p.cu_kv[b], lkv = p.cu_kv[b + 1] - k0;
  const FaWindow win = fa_make_window(p.mode, p.pre, p.next, lq, lkv);
  const int wr0 = it.tile * kDqBM + 32 * wave;
  const int i = wr0 + lrow;
  const bool row_ok = i < lq;
  const int64_t rowg = (int64_t)q0 + (row_ok ? i : 0);

  Op qf[S::NOP], df[S::NOP];
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + (rowg * p.nq + h) * D;
    const T* dp = reinterpret_cast<const T*>(p.dy) + (rowg * p.nq + h) * D;
#pragma unroll
    for (int c = 0; c < S::NOP; ++c) {
      if constexpr (sizeof(T) == 2) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hh);
        bf16x8 d = *reinterpret_cast<const bf16x8*>(dp + 16 * c + 8 * hh);
        qf[c] = row_ok ? a : bf16x8{};
        df[c] = row_ok ? d : bf16x8{};
      } else {
        qf[c] = row_ok ? qp[2 * c + hh] : 0.f;
        df[c] = row_ok ? dp[2 * c + hh] : 0.f;
      }
    }
  }
  const float lse2 = row_ok ? p.lse[rowg * p.nq + h] : __builtin_inff();
  const float di = row_ok ? p.delta[rowg * p.nq + h] : 0.f;
  const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
  f32x16 acc[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) acc[db] = f32x16{};

  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const int64_t kv_stride = (int64_t)p.nkv * S::RB;
  const int a_lane = lrow * S::P + 16 * hh;
  const int t_lane = (4 * (grp >> 1) + (sl >> 2)) * S::P + (16 * (grp & 1) + 4 * (sl & 3)) * 2;
  // swizzled bf16 tiles: row reads of chunk 2c + hh of row lrow (+32 per key
  // block), transposing reads of rows rv and rv + 8 (+16 per step), chunk 4db + qv
  int koff[S::kSwz ? S::NOP : 1], toff[2][S::kSwz ? S::NDB : 1];
  if constexpr (S::kSwz) {
#pragma unroll
    for (int c = 0; c < S::NOP; ++c) koff[c] = lrow * S::RB + 16 * ((2 * c + hh) ^ tile_swz<S::RB>(lrow));
    const int rv = 4 * (grp >> 1) + (sl >> 2), qv = 2 * (grp & 1) + ((sl & 3) >> 1), bv = 8 * (sl & 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
        toff[hf][db] = (rv + 8 * hf) * S::RB + 16 * ((4 * db + qv) ^ tile_swz<S::RB>(rv + 8 * hf)) + bv;
  }

  auto load = [&](char* st, int t) {
    if constexpr (S::kSwz) {
      dma_tile_swz<kDqBN, S::RB, 4>(st, kbase, kv_stride, t * kDqBN, lkv, wave, lane);
      dma_tile_swz<kDqBN, S::RB, 4>(st + S::TILE, vbase, kv_stride, t * kDqBN, lkv, wave, lane);
    } else {
      dma_rows<kDqBN, S::RB, S::P>(st, kbase, kv_stride, t * kDqBN, lkv, wave, lane);
      dma_rows<kDqBN, S::RB, S::P>(st + S::TILE, vbase, kv_stride, t * kDqBN, lkv, wave, lane);
    }
  };

  auto tile = [&](int t, const char* ks) {
    const char* vs = ks + S::TILE;
    const int c0 = t * kDqBN;
    if (wr0 >= lq || fa_tile_empty(win, wr0, min(wr0 + 32, lq), c0, min(c0 + kDqBN, lkv))) return;
    const bool full = fa_tile_full(win, wr0, 32, c0, kDqBN, lq, lkv);
    uint64_t bits = ~0ull;
    if constexpr (DROP) {
      const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + i) * lkv + c0;
      bits = load_mask_window(p.drop, p.drop_bytes, pos);
    }
#pragma unroll
    for (int kb = 0; kb < kDqBN / 32; ++kb) {
      // ---- S^T = K Q^T, dP~^T = V dY^T for 32 keys (lane = row, registers = keys) ----
      f32x16 s = f32x16{}, dp = f32x16{};
      if constexpr (sizeof(T) == 2) {
        // K and V reads run a few MFMAs ahead of their use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) {
          const bf16x8 ka = lds_read_b128(ks + koff[c] + 32 * kb * S::RB);
          const bf16x8 va = lds_read_b128(vs + koff[c] + 32 * kb * S::RB);
          s = mfma32(ka, qf[c], s);
          dp = mfma32(va, df[c], dp);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        sched_alternate<2 * S::NOP, 0x008, 0x100>();
        __builtin_amdgcn_sched_barrier(0);
      } else {
        const char* krow = ks + (32 * kb + lrow) * S::P;
        const char* vrow = vs + (32 * kb + lrow) * S::P;
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) {
          s = mfma32(*reinterpret_cast<const float*>(krow + (2 * c + hh) * 4), qf[c], s);
          dp = mfma32(*reinterpret_cast<const float*>(vrow + (2 * c + hh) * 4), df[c], dp);
        }
      }
      f32x16 ds;
      const float jmi = (float)(c0 + 32 * kb + 4 * hh - i);   // j - i of register 0
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int jj = c0 + kk;
        float pr;
        if (full && !ALIBI) {
          pr = fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -lse2));
        } else {
          float x = s[r] * p.scale_log2;
          if constexpr (ALIBI) x = __builtin_fmaf(slope_l2, jmi + (float)(8 * (r >> 2) + (r & 3)), x);
          if (!full) {
            const bool ok = row_ok & (jj < lkv) & (jj >= fa_row_lo(win, i)) & (jj <= fa_row_hi(win, i));
            x = ok ? x : kNegInf;
          }
          pr = fast_exp2(x - lse2);
        }
        float dpv = dp[r];
        if constexpr (DROP) dpv = ((bits >> kk) & 1ull) ? dpv * p.inv_keep : 0.f;
        ds[r] = pr * (dpv - di);
      }
      // ---- dQ^T += K^T dS^T (A = K through the transposing read, B = dS from registers) ----
      if constexpr (sizeof(T) == 2) {
        bf16x8 bs[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) bs[c][e] = to_bf16(ds[8 * c + e]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const char* base = ks + (32 * kb + 16 * c) * S::RB;
#pragma unroll
          for (int db = 0; db < S::NDB; ++db)
            acc[db] = mfma32(lds_read_tr_x2(base + toff[0][db], base + toff[1][db]), bs[c], acc[db]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        sched_alternate<2 * S::NDB, 0x008, 0x100, 2>();
        __builtin_amdgcn_sched_barrier(0);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            const float a = *reinterpret_cast<const float*>(ks + kk * S::P + (32 * db + lrow) * 4);
            acc[db] = mfma32(a, ds[r], acc[db]);
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
  if (row_ok) {
    T* op = reinterpret_cast<T*>(p.dq) + (rowg * p.nq + h) * D;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 32 * db + 8 * a + 4 * hh;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = to_bf16(acc[db][4 * a + e] * p.scale);
          *reinterpret_cast<bf16x4*>(op + d) = v;
        } else {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * a + e] * p.scale;
          *reinterpret_cast<f32x4*>(op + d) = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
namespace {
unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}
}  // namespace

template <typename T, int D>
static hipError_t launch_pre_t(const BwdParams& p, hipStream_t s) {
  constexpr int GROUPS = 256 / (D * (int)sizeof(T) / 16);
  const int lds = GROUPS * p.nq * 4;
  hipLaunchKernelGGL((fa_bwd_pre_kernel<T, D>), dim3(p.n_pre_blocks), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(int dtype, int d, const BwdParams& p, hipStream_t s) {
  if (p.n_pre_blocks == 0) return hipSuccess;
  if (dtype == 1 && d == 128) return launch_pre_t<__bf16, 128>(p, s);
  if (dtype == 1 && d == 64) return launch_pre_t<__bf16, 64>(p, s);
  if (dtype == 0 && d == 128) return launch_pre_t<float, 128>(p, s);
  if (dtype == 0 && d == 64) return launch_pre_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

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

hipError_t launch_bwd_kv(int dtype, int d, bool atomic_dq, const BwdParams& p, hipStream_t s) {
  if (atomic_dq) {
    // bf16 D = 128 with alibi runs the deterministic passes (the host routes it)
    if (dtype == 1 && d == 128 && p.slopes == nullptr) return launch_kv_t<__bf16, 128, true>(p, s);
    if (dtype == 1 && d == 64) return launch_kv_t<__bf16, 64, true>(p, s);
    // fp32 with D = 128 would need more LDS than a CU has; the host runs the
    // deterministic passes for it instead
    if (dtype == 0 && d == 64) return launch_kv_t<float, 64, true>(p, s);
  } else {
    if (dtype == 1 && d == 128) return launch_kv_t<__bf16, 128, false>(p, s);
    if (dtype == 1 && d == 64) return launch_kv_t<__bf16, 64, false>(p, s);
    if (dtype == 0 && d == 128) return launch_kv_t<float, 128, false>(p, s);
    if (dtype == 0 && d == 64) return launch_kv_t<float, 64, false>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_dq_t(const BwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_dq_items * p.nq;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
  const bool drop = p.use_dropout != 0, alibi = p.slopes != nullptr;
  if (drop && alibi)
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, true, true>), grid, block, 0, s, p);
  else if (drop)
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, true, false>), grid, block, 0, s, p);
  else if (alibi)
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, false, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(int dtype, int d, const BwdParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return launch_dq_t<__bf16, 128>(p, s);
  if (dtype == 1 && d == 64) return launch_dq_t<__bf16, 64>(p, s);
  if (dtype == 0 && d == 128) return launch_dq_t<float, 128>(p, s);
  if (dtype == 0 && d == 64) return launch_dq_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_convert(int dtype, int d, const BwdParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.total_q * p.nq * d;
  if (dtype == 1)
    hipLaunchKernelGGL((fa_dq_convert_kernel<__bf16>), dim3(grid_for(n)), dim3(256), 0, s, p.dq_acc,
                       reinterpret_cast<__bf16*>(p.dq), p.scale, n);
  else
    hipLaunchKernelGGL((fa_dq_convert_kernel<float>), dim3(grid_for(n)), dim3(256), 0, s, p.dq_acc,
                       reinterpret_cast<float*>(p.dq), p.scale, n);
  return hipGetLastError();
}

hipError_t launch_bwd_dsink(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL(fa_dsink_reduce_kernel, dim3(p.nq), dim3(256), 0, s, p.dsink_part, p.n_pre_blocks, p.nq, p.dsink);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* ptr, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fa_zero_kernel, dim3(grid_for(n)), dim3(256), 0, s, ptr, n);
  return hipGetLastError();
}

}  // namespace fa
