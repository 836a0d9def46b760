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
//   fa_bwd_kv_kernel    dK, dV (and optionally atomic dQ): fa_bwd_kv.hip
//   fa_bwd_dq_kernel    deterministic dQ: one 128-row query tile per workgroup,
//                       recomputes S, dP, dS over its key tiles, dQ in registers
//   fa_dq_convert_kernel, fa_dsink_reduce_kernel, fa_zero_kernel, fa_mask_pack_kernel
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
  constexpr int U = 8;   // pairs in flight per thread
  for (int64_t pb = grp; pb < npairs; pb += GROUPS * U) {
    u32x4 av[U], cv[U];
    float mv[U], lv[U];   // the softmax max / sum of the pair, loaded beside its rows
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t pi = pb + (int64_t)u * GROUPS;
      const int64_t idx = row0 * nq + (pi < npairs ? pi : pb);
      av[u] = *reinterpret_cast<const u32x4*>(dyb + idx * (D * EB) + sub * 16);
      cv[u] = *reinterpret_cast<const u32x4*>(ob + idx * (D * EB) + sub * 16);
      if (sub == 0) {
        mv[u] = p.m_in[idx];
        lv[u] = p.l_in[idx];
      }
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
        acc += bits16_to_f32<T>((uint16_t)(a[w] & 0xffff)) * bits16_to_f32<T>((uint16_t)(c[w] & 0xffff));
        acc += bits16_to_f32<T>((uint16_t)(a[w] >> 16)) * bits16_to_f32<T>((uint16_t)(c[w] >> 16));
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += __uint_as_float(a[w]) * __uint_as_float(c[w]);
    }
    // reduce over the CPR lanes of this pair (contiguous, power of two, inside one wave)
#pragma unroll
    for (int o = CPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (sub == 0) {
      const float m = mv[u], l = lv[u];
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

// attenMask [rows, cols] of bytes (nonzero = masked out) -> one 32-bit word per
// row and 32 keys, bit k for key 32w + k; keys at or past `cols` read as masked.
__global__ __launch_bounds__(256) void fa_mask_pack_kernel(const uint8_t* mask, int64_t rows, int64_t cols,
                                                           int64_t words, uint32_t* bits) {
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < rows * words; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / words, w = idx - i * words;
    const uint8_t* row = mask + i * cols;
    uint32_t acc = 0;
    for (int k = 0; k < 32; ++k) {
      const int64_t j = 32 * w + k;
      const uint32_t m = j < cols ? (row[j] != 0) : 1u;
      acc |= m << k;
    }
    bits[idx] = acc;
  }
}

__global__ __launch_bounds__(256) void fa_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

template <typename T>
__global__ __launch_bounds__(256) void fa_dq_convert_kernel(const float* acc, T* out, float scale, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    if constexpr (sizeof(T) == 2)
      out[i] = cvt16<T>(acc[i] * scale);
    else
      out[i] = acc[i] * scale;
  }
}

// ------------------------------------------------------------------ deterministic dQ
template <typename T, int D>
struct DqShape {
  static constexpr int EB = sizeof(T);
  static constexpr int RB = D * EB;
  static constexpr bool kSwz = EB == 2;     // 16-bit tiles swizzled and unpadded
  static constexpr int P = kSwz ? RB : RB + 16;
  static constexpr int TILE = kDqBN * P;
  static constexpr int STAGE = 2 * TILE;    // K | V
  static constexpr int NOP = D / ElemTraits<T>::kChunk;
  static constexpr int NDB = D / 32;
};

// Two workgroups per CU need at most 256 registers per lane.  The 16-bit dropout
// instances fit that with the LDS operand reads of the matrix phases kept two (not
// four) ahead of their MFMAs and the swizzled offsets formed per use (kLean below),
// except D = 128 with an attenMask: those, and fp32 with dropout, run one
// workgroup per CU rather than spill.
template <typename T, int D, bool DROP, int ALIBI, bool MASK>
constexpr int dq_occupancy() {
  return DROP && (sizeof(T) == 4 || (D == 128 && MASK)) ? 1 : 2;
}

template <typename T, int D, bool DROP, int ALIBI, bool MASK>
__global__ __launch_bounds__(256, (dq_occupancy<T, D, DROP, ALIBI, MASK>())) void fa_bwd_dq_kernel(BwdParams p) {
  static_assert(sizeof(T) == 4 || ALIBI != kPseExt, "a 16-bit external pse runs the materialised-score path");
  constexpr int kReadAhead = DROP ? 2 : 4;   // LDS operand reads issued before the first MFMA of a phase
  using S = DqShape<T, D>;
  using E = typename std::conditional<sizeof(T) == 2, T, __bf16>::type;   // 16-bit element type
  using V8 = typename Vec16<E>::v8;
  using V4 = typename Vec16<E>::v4;
  using Op = typename std::conditional<sizeof(T) == 2, V8, float>::type;
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
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, lq, lkv, p.prefix[b]);
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
        V8 a = *reinterpret_cast<const V8*>(qp + 16 * c + 8 * hh);
        V8 d = *reinterpret_cast<const V8*>(dp + 16 * c + 8 * hh);
        qf[c] = row_ok ? a : V8{};
        df[c] = row_ok ? d : V8{};
      } else {
        qf[c] = row_ok ? qp[2 * c + hh] : 0.f;
        df[c] = row_ok ? dp[2 * c + hh] : 0.f;
      }
    }
  }
  const float lse2 = row_ok ? p.lse[rowg * p.nq + h] : __builtin_inff();
  const float di = row_ok ? p.delta[rowg * p.nq + h] : 0.f;
  const float slope_l2 = pse_slopes(ALIBI) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
  const int poff = b == 0 ? p.pse_off0 : 0;   // sequence 0 of mode 8: pse row i + qStartIdx - kvStartIdx
  f32x16 acc[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) acc[db] = f32x16{};

  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)k0 * p.nkv + g) * S::RB;
  const int64_t kv_stride = (int64_t)p.nkv * S::RB;
  const int a_lane = lrow * S::P + 16 * hh;
  const int t_lane = (4 * (grp >> 1) + (sl >> 2)) * S::P + (16 * (grp & 1) + 4 * (sl & 3)) * 2;
  // swizzled 16-bit tiles: row reads of chunk 2c + hh of row lrow (+32 per key
  // block), transposing reads of rows rv and rv + 8 (+16 per step), chunk 4db + qv
  // The chunk index enters an offset only through bits the rest of it leaves
  // clear, so koff[c] == kx ^ 32c and toff[hf][db] == tx[hf] ^ 64db.  The dropout
  // instances, short of registers, form the offsets per use from kx, tx (kLean).
  constexpr bool kLean = DROP;
  int koff[S::kSwz ? S::NOP : 1], toff[2][S::kSwz ? S::NDB : 1];
  int kx = 0, tx[2] = {0, 0};
  if constexpr (S::kSwz) {
#pragma unroll
    for (int c = 0; c < S::NOP; ++c) koff[c] = lrow * S::RB + 16 * ((2 * c + hh) ^ tile_swz<S::RB>(lrow));
    const int rv = 4 * (grp >> 1) + (sl >> 2), qv = 2 * (grp & 1) + ((sl & 3) >> 1), bv = 8 * (sl & 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
        toff[hf][db] = (rv + 8 * hf) * S::RB + 16 * ((4 * db + qv) ^ tile_swz<S::RB>(rv + 8 * hf)) + bv;
    kx = lrow * S::RB + ((16 * hh) ^ (16 * tile_swz<S::RB>(lrow)));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) tx[hf] = (rv + 8 * hf) * S::RB + ((16 * qv) ^ (16 * tile_swz<S::RB>(rv + 8 * hf))) + bv;
  }

  // K and V tiles share their geometry and row stride: one set of lane offsets for both
  SwzLane<kDqBN, S::kSwz ? S::RB : 256, 4> cp;
  if constexpr (S::kSwz) cp.init(kv_stride, wave, lane);
  auto load = [&](char* st, int t) {
    if constexpr (S::kSwz) {
      cp.copy(st, kbase, kv_stride, t * kDqBN, lkv, wave, lane);
      cp.copy(st + S::TILE, vbase, kv_stride, t * kDqBN, lkv, wave, lane);
    } else {
      dma_rows<kDqBN, S::RB, S::P>(st, kbase, kv_stride, t * kDqBN, lkv, wave, lane);
      dma_rows<kDqBN, S::RB, S::P>(st + S::TILE, vbase, kv_stride, t * kDqBN, lkv, wave, lane);
    }
  };

  auto tile = [&](int t, const char* ks) {
    const char* vs = ks + S::TILE;
    const int c0 = t * kDqBN;
    if (wr0 >= lq || fa_tile_empty(win, wr0, min(wr0 + 32, lq), c0, min(c0 + kDqBN, lkv))) return;
    if (lane == 0)
      FA_TRACE_VISIT(p.trace_dq, (((int64_t)b * p.nq + h) * p.trace_dq_rb + (wr0 >> 5)) * p.trace_dq_kt + t);
    // with an attenMask every tile takes the masked path
    const bool full = fa_tile_full(win, wr0, 32, c0, kDqBN, lq, lkv) && !MASK;
    uint64_t bits = ~0ull;
    if constexpr (DROP) {
      const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + i) * lkv + c0;
      bits = load_mask_window(p.drop, p.drop_bytes, pos);
    }
#pragma unroll
    for (int kb = 0; kb < kDqBN / 32; ++kb) {
      // ---- S^T = K Q^T, dP~^T = V dY^T for 32 keys (lane = row, registers = keys) ----
      f32x16 s = f32x16{}, dp = f32x16{};
      // lean offsets: fresh copies per key block, so their XORs are not hoisted
      int kxl = kx, tx0 = tx[0], tx1 = tx[1];
      if constexpr (kLean) asm volatile("" : "+v"(kxl), "+v"(tx0), "+v"(tx1));
      if constexpr (sizeof(T) == 2) {
        // K and V reads run a few MFMAs ahead of their use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < S::NOP; ++c) {
          const int ko = kLean ? (kxl ^ (32 * c)) : koff[c];
          const V8 ka = lds_read_b128<V8>(ks + ko + 32 * kb * S::RB);
          const V8 va = lds_read_b128<V8>(vs + ko + 32 * kb * S::RB);
          s = mfma32(ka, qf[c], s);
          dp = mfma32(va, df[c], dp);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kReadAhead, 0);
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
      // attenMask bits (1 = masked) of the lane's row for these 32 keys
      uint32_t mwk = 0;
      if constexpr (MASK) {
        if (row_ok) {
          const int w = (c0 >> 5) + kb;
          mwk = w < p.mwords ? p.mbits[(int64_t)i * p.mwords + w] : ~0u;
        }
      }
      f32x16 ds;
      const float jmi = (float)(c0 + 32 * kb + 4 * hh - i - poff);   // j - i of register 0 (pse position)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int jj = c0 + kk;
        float pr;
        if (full && !ALIBI) {
          pr = fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -lse2));
        } else {
          float x = s[r] * p.scale_log2;
          if constexpr (ALIBI == kPseExt)
            x = __builtin_fmaf(p.pse_coef, (row_ok && jj < lkv) ? pse_value<T>(p, b, h, i, jj, lq) : 0.f, x);
          else if constexpr (ALIBI != 0)
            x = add_pse<ALIBI>(x, slope_l2, jmi + (float)(8 * (r >> 2) + (r & 3)));
          if (!full) {
            const bool ok = row_ok & (jj < lkv) & (jj >= fa_row_lo(win, i)) & (jj <= fa_row_hi(win, i)) &
                            !((mwk >> (kk - 32 * kb)) & 1u);
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
        V8 bs[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) bs[c][e] = cvt16<E>(ds[8 * c + e]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const char* base = ks + (32 * kb + 16 * c) * S::RB;
#pragma unroll
          for (int db = 0; db < S::NDB; ++db)
            acc[db] = mfma32(kLean ? lds_read_tr_x2<V8>(base + (tx0 ^ (64 * db)), base + (tx1 ^ (64 * db)))
                                   : lds_read_tr_x2<V8>(base + toff[0][db], base + toff[1][db]),
                             bs[c], acc[db]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kReadAhead, 0);
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
          V4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = cvt16<E>(acc[db][4 * a + e] * p.scale);
          *reinterpret_cast<V4*>(op + d) = v;
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
  if (dtype == 2 && d == 128) return launch_pre_t<_Float16, 128>(p, s);
  if (dtype == 2 && d == 64) return launch_pre_t<_Float16, 64>(p, s);
  if (dtype == 0 && d == 128) return launch_pre_t<float, 128>(p, s);
  if (dtype == 0 && d == 64) return launch_pre_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_dq_t(const BwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_dq_items * p.nq;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
  const bool drop = p.use_dropout != 0;
  return with_flags<sizeof(T) == 4>(drop, pse_kind(p), p.mbits != nullptr, [&](auto dr, auto al, auto mk) {
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, decltype(dr)::value, decltype(al)::value, decltype(mk)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

hipError_t launch_bwd_dq(int dtype, int d, const BwdParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return launch_dq_t<__bf16, 128>(p, s);
  if (dtype == 1 && d == 64) return launch_dq_t<__bf16, 64>(p, s);
  if (dtype == 2 && d == 128) return launch_dq_t<_Float16, 128>(p, s);
  if (dtype == 2 && d == 64) return launch_dq_t<_Float16, 64>(p, s);
  if (dtype == 0 && d == 128) return launch_dq_t<float, 128>(p, s);
  if (dtype == 0 && d == 64) return launch_dq_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_convert(int dtype, int d, const BwdParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.total_q * p.nq * d;
  if (dtype == 1)
    hipLaunchKernelGGL((fa_dq_convert_kernel<__bf16>), dim3(grid_for(n)), dim3(256), 0, s, p.dq_acc,
                       reinterpret_cast<__bf16*>(p.dq), p.scale, n);
  else if (dtype == 2)
    hipLaunchKernelGGL((fa_dq_convert_kernel<_Float16>), dim3(grid_for(n)), dim3(256), 0, s, p.dq_acc,
                       reinterpret_cast<_Float16*>(p.dq), p.scale, n);
  else
    hipLaunchKernelGGL((fa_dq_convert_kernel<float>), dim3(grid_for(n)), dim3(256), 0, s, p.dq_acc,
                       reinterpret_cast<float*>(p.dq), p.scale, n);
  return hipGetLastError();
}

hipError_t launch_bwd_dsink(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL(fa_dsink_reduce_kernel, dim3(p.nq), dim3(256), 0, s, p.dsink_part, p.n_pre_blocks, p.nq, p.dsink);
  return hipGetLastError();
}

hipError_t launch_mask_pack(const uint8_t* mask, int64_t rows, int64_t cols, uint32_t* bits, hipStream_t s) {
  const int64_t words = (cols + 31) / 32, n = rows * words;
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
  hipLaunchKernelGGL(fa_mask_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, mask, rows, cols, words, bits);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* ptr, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fa_zero_kernel, dim3(grid_for(n)), dim3(256), 0, s, ptr, n);
  return hipGetLastError();
}

}  // namespace fa
