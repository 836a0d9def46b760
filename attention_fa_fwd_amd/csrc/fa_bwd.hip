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
  for (int64_t pi = grp; pi < npairs; pi += GROUPS) {
    const int64_t idx = row0 * nq + pi;            // (t * nq + h)
    const int h = (int)(pi % nq);
    const u32x4 a = *reinterpret_cast<const u32x4*>(dyb + idx * (D * EB) + sub * 16);
    const u32x4 c = *reinterpret_cast<const u32x4*>(ob + idx * (D * EB) + sub * 16);
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
  if (p.sink) {
    __syncthreads();
    for (int h = tid; h < nq; h += 256) {
      float s = 0.f;
      for (int gi = 0; gi < GROUPS; ++gi) s += part[gi * nq + h];
      p.dsink_part[(int64_t)blockIdx.x * nq + h] = s;
    }
  }
}

__global__ __launch_bounds__(256) void fa_dsink_reduce_kernel(const float* part, int nblocks, int nq, float* out) {
  for (int h = blockIdx.x * 256 + threadIdx.x; h < nq; h += gridDim.x * 256) {
    float s = 0.f;
    for (int b = 0; b < nblocks; ++b) s += part[(int64_t)b * nq + h];
    out[h] = s;
  }
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
  static constexpr int P = RB + 16;                 // LDS pitch of Q / dY / K rows
  static constexpr int QT = kKvBM * P;              // one 32-row tile
  static constexpr int KT = kKvBN * P;              // the 128-key K tile (atomic dQ only)
  static constexpr int DSP = kKvBM * EB + 16;       // pitch of dS^T rows (one row per key)
  static constexpr int DST = kKvBN * DSP;
  static constexpr int CPR = RB / 16;
  static constexpr int NQC = kKvBM * CPR / 256;     // 16-byte chunks per thread for a 32-row tile
  static constexpr int NKC = kKvBN * CPR / 256;     // ... for the 128-key tile
  static constexpr int NOP = D / ElemTraits<T>::kChunk;
  static constexpr int NDB = D / 32;
  // LDS: Q | dY | lse[32] delta[32] | bits[32][4] | K tile | dS^T
  static constexpr int OFF_DY = QT;
  static constexpr int OFF_STAT = 2 * QT;
  static constexpr int OFF_BITS = OFF_STAT + 64 * 4;
  static constexpr int OFF_K = OFF_BITS + 32 * 4 * 4;
  static constexpr int OFF_DS = OFF_K + KT;
  static constexpr int LDS_BASE = OFF_K;
  static constexpr int LDS_ATOMIC = OFF_DS + DST;
};

template <typename T, int D, bool ATOMIC>
__global__ __launch_bounds__(256, 1) void fa_bwd_kv_kernel(BwdParams p) {
  using S = KvShape<T, D>;
  using Op = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  if constexpr (ATOMIC) {
    const char* kb = reinterpret_cast<const char*>(p.k) + ((int64_t)k0 * p.nkv + g) * S::RB;
#pragma unroll
    for (int n = 0; n < S::NKC; ++n) {
      const int ci = tid + 256 * n;
      const int r = ci / S::CPR, cc = ci % S::CPR;
      const bool ok = c0 + r < lkv;
      u32x4 v = *reinterpret_cast<const u32x4*>(kb + (int64_t)(ok ? c0 + r : 0) * kv_stride + cc * 16);
      *reinterpret_cast<u32x4*>(smem + S::OFF_K + r * S::P + cc * 16) = ok ? v : u32x4{};
    }
  }

  f32x16 dk[S::NDB], dv[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  float* lse_s = reinterpret_cast<float*>(smem + S::OFF_STAT);
  float* del_s = lse_s + 32;
  uint32_t* bits_s = reinterpret_cast<uint32_t*>(smem + S::OFF_BITS);

  for (int hq = 0; hq < p.group; ++hq) {
    const int h = g * p.group + hq;
    const float slope_l2 = p.slopes ? p.slopes[h] * kLog2e : 0.f;
    const char* qb = reinterpret_cast<const char*>(p.q) + ((int64_t)q0 * p.nq + h) * S::RB;
    const char* dyb = reinterpret_cast<const char*>(p.dy) + ((int64_t)q0 * p.nq + h) * S::RB;
    const int64_t q_stride = (int64_t)p.nq * S::RB;
    for (int qt = it.lo; qt < it.hi; ++qt) {
      const int r0 = qt * kKvBM;
      __syncthreads();
      // ---- stage the Q / dY tile, row statistics and keep bits ----
#pragma unroll
      for (int n = 0; n < S::NQC; ++n) {
        const int ci = tid + 256 * n;
        const int r = ci / S::CPR, cc = ci % S::CPR;
        const bool ok = r0 + r < lq;
        const int64_t off = (int64_t)(ok ? r0 + r : 0) * q_stride + cc * 16;
        u32x4 a = *reinterpret_cast<const u32x4*>(qb + off);
        u32x4 c = *reinterpret_cast<const u32x4*>(dyb + off);
        *reinterpret_cast<u32x4*>(smem + r * S::P + cc * 16) = ok ? a : u32x4{};
        *reinterpret_cast<u32x4*>(smem + S::OFF_DY + r * S::P + cc * 16) = ok ? c : u32x4{};
      }
      if (tid < 32) {
        const bool ok = r0 + tid < lq;
        const int64_t idx = (int64_t)(q0 + (ok ? r0 + tid : 0)) * p.nq + h;
        lse_s[tid] = ok ? p.lse[idx] : __builtin_inff();
        del_s[tid] = ok ? p.delta[idx] : 0.f;
      }
      if (p.use_dropout && tid < 128) {
        const int r = tid >> 2, w = tid & 3;
        uint32_t word = 0;
        if (r0 + r < lq) {
          const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + r0 + r) * lkv + c0 + 32 * w;
          word = (uint32_t)load_mask_window(p.drop, p.drop_bytes, pos);
        }
        bits_s[r * 4 + w] = word;
      }
      __syncthreads();

      bool wave_empty = wc0 >= lkv || r0 >= lq;
      if (!wave_empty) wave_empty = fa_tile_empty(win, r0, min(r0 + kKvBM, lq), wc0, min(wc0 + 32, lkv));
      f32x16 ds = f32x16{};
      if (!wave_empty) {
        const bool full = fa_tile_full(win, r0, kKvBM, wc0, 32, lq, lkv);
        // ---- S = Q K^T and dP~ = dY V^T (lane = key, registers = rows) ----
        f32x16 s = f32x16{}, dp = f32x16{};
        const char* qrow = smem + lrow * S::P;
        const char* dyrow = smem + S::OFF_DY + lrow * S::P;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int c = 0; c < S::NOP; ++c) {
            s = mfma32(lds_read_b128(qrow + (16 * c + 8 * hh) * 2), kf[c], s);
            dp = mfma32(lds_read_b128(dyrow + (16 * c + 8 * hh) * 2), vf[c], dp);
          }
        } else {
#pragma unroll
          for (int c = 0; c < S::NOP; ++c) {
            s = mfma32(*reinterpret_cast<const float*>(qrow + (2 * c + hh) * 4), kf[c], s);
            dp = mfma32(*reinterpret_cast<const float*>(dyrow + (2 * c + hh) * 4), vf[c], dp);
          }
        }
        // ---- P, P~, dS ----
        f32x16 pt;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
          const int i = r0 + rr;
          float x = s[r] * p.scale_log2;
          if (p.slopes) x = __builtin_fmaf(slope_l2, (float)(j - i), x);
          if (!full && !fa_allowed(win, i, j, lq, lkv)) x = kNegInf;
          const float pr = fast_exp2(x - lse_s[rr]);
          float dpv = dp[r], ptv = pr;
          if (p.use_dropout) {
            const bool keep = (bits_s[rr * 4 + wave] >> lrow) & 1u;
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
            const int row0 = 16 * c + 4 * (grp >> 1) + (sl >> 2);
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
              const int col = (32 * db + 16 * (grp & 1) + 4 * (sl & 3)) * 2;
              const bf16x8 dyo = lds_read_tr_x2(smem + S::OFF_DY + row0 * S::P + col,
                                                smem + S::OFF_DY + (row0 + 8) * S::P + col);
              const bf16x8 qo = lds_read_tr_x2(smem + row0 * S::P + col, smem + (row0 + 8) * S::P + col);
              dv[db] = mfma32(pa, dyo, dv[db]);
              dk[db] = mfma32(da, qo, dk[db]);
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
              const float dyo = *reinterpret_cast<const float*>(smem + S::OFF_DY + rr * S::P + (32 * db + lrow) * 4);
              const float qo = *reinterpret_cast<const float*>(smem + rr * S::P + (32 * db + lrow) * 4);
              dv[db] = mfma32(pt[r], dyo, dv[db]);
              dk[db] = mfma32(ds[r], qo, dk[db]);
            }
          }
        }
      }
      if constexpr (ATOMIC) {
        // ---- dQ(rows x d-block of this wave) += dS K over the 128 keys ----
        char* dst = smem + S::OFF_DS;
        // dS^T[key][row]: lane writes its key's rows 8a + 4hh + 0..3
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int key = 32 * wave + lrow, row = 8 * a + 4 * hh;
          if constexpr (sizeof(T) == 2) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = to_bf16(ds[4 * a + e]);
            *reinterpret_cast<bf16x4*>(dst + key * S::DSP + row * 2) = v;
          } else {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = ds[4 * a + e];
            *reinterpret_cast<f32x4*>(dst + key * S::DSP + row * 4) = v;
          }
        }
        __syncthreads();
        const int dcol = 32 * wave;   // this wave's 32-wide d block
        if (r0 < lq && dcol < D) {
          f32x16 acc = f32x16{};
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int c = 0; c < kKvBN / 16; ++c) {
              const int krow = 16 * c + 4 * (grp >> 1) + (sl >> 2);
              const int coln = (16 * (grp & 1) + 4 * (sl & 3)) * 2;
              const bf16x8 a = lds_read_tr_x2(dst + krow * S::DSP + coln, dst + (krow + 8) * S::DSP + coln);
              const int colk = (dcol + 16 * (grp & 1) + 4 * (sl & 3)) * 2;
              const bf16x8 bo = lds_read_tr_x2(smem + S::OFF_K + krow * S::P + colk,
                                               smem + S::OFF_K + (krow + 8) * S::P + colk);
              acc = mfma32(a, bo, acc);
            }
          } else {
#pragma unroll 8
            for (int c = 0; c < kKvBN / 2; ++c) {
              const int key = 2 * c + hh;
              const float a = *reinterpret_cast<const float*>(dst + key * S::DSP + lrow * 4);
              const float bo = *reinterpret_cast<const float*>(smem + S::OFF_K + key * S::P + (dcol + lrow) * 4);
              acc = mfma32(a, bo, acc);
            }
          }
          // acc: lane = d (dcol + lrow), registers = rows 8(r/4) + 4hh + r%4
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
            if (r0 + rr < lq)
              atomicAdd(p.dq_acc + ((int64_t)(q0 + r0 + rr) * p.nq + h) * D + dcol + lrow, acc[r]);
          }
        }
      }
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
  static constexpr int P = RB + 16;
  static constexpr int TILE = kDqBN * P;
  static constexpr int CPR = RB / 16;
  static constexpr int NCH = kDqBN * CPR / 256;
  static constexpr int NOP = D / ElemTraits<T>::kChunk;
  static constexpr int NDB = D / 32;
  static constexpr int LDS = 2 * TILE;   // K | V
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_kernel(BwdParams p) {
  using S = DqShape<T, D>;
  using Op = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const float slope_l2 = p.slopes ? p.slopes[h] * kLog2e : 0.f;
  const int64_t drop_row = p.use_dropout ? p.bit_base[b] + ((int64_t)h * lq + i) * lkv : 0;
  f32x16 acc[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) acc[db] = f32x16{};

  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const int64_t kv_stride = (int64_t)p.nkv * S::RB;

  for (int t = it.lo; t < it.hi; ++t) {
    const int c0 = t * kDqBN;
    __syncthreads();
#pragma unroll
    for (int n = 0; n < S::NCH; ++n) {
      const int ci = tid + 256 * n;
      const int r = ci / S::CPR, cc = ci % S::CPR;
      const bool ok = c0 + r < lkv;
      const int64_t off = (int64_t)(ok ? c0 + r : 0) * kv_stride + cc * 16;
      u32x4 kv = *reinterpret_cast<const u32x4*>(kbase + off);
      u32x4 vv = *reinterpret_cast<const u32x4*>(vbase + off);
      *reinterpret_cast<u32x4*>(smem + r * S::P + cc * 16) = ok ? kv : u32x4{};
      *reinterpret_cast<u32x4*>(smem + S::TILE + r * S::P + cc * 16) = ok ? vv : u32x4{};
    }
    __syncthreads();
    bool wave_empty = wr0 >= lq;
    if (!wave_empty) wave_empty = fa_tile_empty(win, wr0, min(wr0 + 32, lq), c0, min(c0 + kDqBN, lkv));
    if (wave_empty) continue;
    const bool full = fa_tile_full(win, wr0, 32, c0, kDqBN, lq, lkv);
    // ---- S^T = K Q^T, dP~^T = V dY^T (lane = row, registers = keys) ----
    f32x16 s = f32x16{}, dp = f32x16{};
    const char* krow = smem + lrow * S::P;
    const char* vrow = smem + S::TILE + lrow * S::P;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < S::NOP; ++c) {
        s = mfma32(lds_read_b128(krow + (16 * c + 8 * hh) * 2), qf[c], s);
        dp = mfma32(lds_read_b128(vrow + (16 * c + 8 * hh) * 2), df[c], dp);
      }
    } else {
#pragma unroll
      for (int c = 0; c < S::NOP; ++c) {
        s = mfma32(*reinterpret_cast<const float*>(krow + (2 * c + hh) * 4), qf[c], s);
        dp = mfma32(*reinterpret_cast<const float*>(vrow + (2 * c + hh) * 4), df[c], dp);
      }
    }
    uint64_t bits = ~0ull;
    if (p.use_dropout) bits = load_mask_window(p.drop, p.drop_bytes, drop_row + c0);
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
      const int jj = c0 + kk;
      float x = s[r] * p.scale_log2;
      if (p.slopes) x = __builtin_fmaf(slope_l2, (float)(jj - i), x);
      if (!full && !fa_allowed(win, i, jj, lq, lkv)) x = kNegInf;
      const float pr = fast_exp2(x - lse2);
      float dpv = dp[r];
      if (p.use_dropout) dpv = ((bits >> kk) & 1ull) ? dpv * p.inv_keep : 0.f;
      ds[r] = pr * (dpv - di);
    }
    // ---- dQ^T += K^T dS^T (A = K through the transposing read, B = dS from registers) ----
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 bs;
#pragma unroll
        for (int e = 0; e < 8; ++e) bs[e] = to_bf16(ds[8 * c + e]);
        const int row0 = 16 * c + 4 * (grp >> 1) + (sl >> 2);
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) {
          const int col = (32 * db + 16 * (grp & 1) + 4 * (sl & 3)) * 2;
          const bf16x8 a = lds_read_tr_x2(smem + row0 * S::P + col, smem + (row0 + 8) * S::P + col);
          acc[db] = mfma32(a, bs, acc[db]);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) {
          const float a = *reinterpret_cast<const float*>(smem + kk * S::P + (32 * db + lrow) * 4);
          acc[db] = mfma32(a, ds[r], acc[db]);
        }
      }
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
  using S = KvShape<T, D>;
  const int lds = ATOMIC ? S::LDS_ATOMIC : S::LDS_BASE;
  const int64_t blocks = (int64_t)p.n_kv_items * p.nkv;
  if (blocks == 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)fa_bwd_kv_kernel<T, D, ATOMIC>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_kv_kernel<T, D, ATOMIC>), dim3((unsigned)blocks), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(int dtype, int d, bool atomic_dq, const BwdParams& p, hipStream_t s) {
  if (atomic_dq) {
    if (dtype == 1 && d == 128) return launch_kv_t<__bf16, 128, true>(p, s);
    if (dtype == 1 && d == 64) return launch_kv_t<__bf16, 64, true>(p, s);
    if (dtype == 0 && d == 128) return launch_kv_t<float, 128, true>(p, s);
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
  using S = DqShape<T, D>;
  const int64_t blocks = (int64_t)p.n_dq_items * p.nq;
  if (blocks == 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)fa_bwd_dq_kernel<T, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D>), dim3((unsigned)blocks), dim3(256), S::LDS, s, p);
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
  hipLaunchKernelGGL(fa_dsink_reduce_kernel, dim3(1), dim3(256), 0, s, p.dsink_part, p.n_pre_blocks, p.nq, p.dsink);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* ptr, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fa_zero_kernel, dim3(grid_for(n)), dim3(256), 0, s, ptr, n);
  return hipGetLastError();
}

}  // namespace fa
