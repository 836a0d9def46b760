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
// Work decomposition: one workgroup = NW waves = one query tile of 32*NW rows
// of one (sequence, head); each wave owns 32 rows, and all waves share each K/V
// tile of 64 keys.  16-bit (bf16, fp16) tiles sit in LDS unpadded with an XOR swizzle of their
// 16-byte chunks and arrive by 16-byte-per-lane LDS DMA (four rows per
// instruction); fp32 tiles use padded rows and 4-byte DMA.  Per wave and tile:
//   S^T (64 keys x 32 rows) = K Q^T      A = K rows from LDS, B = Q in registers
//   O^T (D x 32 rows)      += V^T P^T    A = V via the transposing LDS read,
//                                         B = P taken straight from the S^T accumulator
// Every accumulator keeps one query row per lane (lanes l and l+32 share a row),
// so row max / row sum need only in-lane work plus one cross-half exchange.
//
// 16-bit runs 4 waves per workgroup at two workgroups per CU, so one workgroup's
// softmax (VALU) overlaps the other's matrix work; fp32 runs one workgroup per
// CU.  K and V tiles have two LDS stages each; global_load_lds fills stage t+1
// while tile t is computed, and each wave drains its own copies just before
// the barrier that ends the tile.  Inside a tile the LDS operand reads of each
// MFMA group are issued a few MFMAs ahead of their use (scheduling-group
// barriers).
//
// Softmax bookkeeping (log2 units): the exponent offset m_run only moves when a
// row's maximum exceeds it by more than kLazy, so most tiles skip the rescale of
// O and l (probabilities stay below 2^kLazy); the true maximum is tracked apart
// and l is brought to it in the epilogue.  Tiles fully inside the mask skip all
// mask arithmetic and fold the scale into the exponent's FMA; a negative scale
// is applied as a positive one to -Q (exact), so the row maximum of the raw
// scores always gives the maximum logit.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

constexpr float kLazy = 8.0f;

template <typename T, int D>
struct FwdShape {
  static constexpr int EB = sizeof(T);
  static constexpr int RB = D * EB;                     // bytes per K/V row
  // 16-bit tiles are swizzled and unpadded; fp32 tiles use padded rows
  static constexpr bool kSwz = EB == 2;
  static constexpr int KP = kSwz ? RB : RB + 16;        // LDS pitch of K rows
  static constexpr int VP = kSwz ? RB : RB + 16;        // LDS pitch of V rows
  static constexpr int KT = kFwdBN * KP;
  static constexpr int VT = kFwdBN * VP;
  static constexpr int NQ = D / ElemTraits<T>::kChunk;  // Q operand registers per row block
  static constexpr int NDB = D / 32;                    // 32-wide d blocks of O
};

// One wave's view of one key tile.
struct RowTile {
  bool live;          // the wave's 32 rows hold at least one allowed pair in the tile
  bool full;          // every (row, key) pair of the wave's rows is inside the mask
  uint32_t bits[2];   // keep bits of the lane's row for keys 0-31 and 32-63 of the tile
  uint32_t mw[2];     // attenMask bits (1 = masked) of the lane's row, same keys
};

template <typename T, int D, int NW, int OCC, bool DROP, int ALIBI, bool MASK>
__global__ __launch_bounds__(64 * NW, OCC) void fa_fwd_kernel(FwdParams p) {
  static_assert(sizeof(T) == 4 || ALIBI != kPseExt, "a 16-bit external pse runs the materialised-score path");
  using S = FwdShape<T, D>;
  constexpr int BM = 32 * NW;
  constexpr bool k16 = sizeof(T) == 2;
  using E = typename std::conditional<sizeof(T) == 2, T, __bf16>::type;   // 16-bit element type
  using V8 = typename Vec16<E>::v8;
  using V4 = typename Vec16<E>::v4;
  __shared__ __attribute__((aligned(16))) char kst[2][S::KT];
  __shared__ __attribute__((aligned(16))) char vst[2][S::VT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
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
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, lq, lkv, p.prefix[b]);

  const int wr0 = it.tile * BM + wave * 32;       // first row of this wave (in sequence)
  const int i = wr0 + lrow;                        // this lane's row
  const bool row_ok = i < lq;

  // ---- Q operand in registers (B of S^T = K Q^T), negated for a negative scale ----
  const bool neg = p.scale_log2 < 0.f;
  const float sc = neg ? -p.scale_log2 : p.scale_log2;
  using QReg = typename std::conditional<k16, V8, float>::type;
  QReg qf[S::NQ];
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + ((int64_t)(q0 + (row_ok ? i : 0)) * p.nq + h) * D;
    if constexpr (k16) {
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) {
        V8 v = *reinterpret_cast<const V8*>(qp + 16 * c + 8 * hh);
        if (neg) v = -v;
        qf[c] = row_ok ? v : V8{};
      }
    } else {
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) {
        const float v = qp[2 * c + hh];
        qf[c] = row_ok ? (neg ? -v : v) : 0.f;
      }
    }
  }

  // keys [j_lo, j_hi] of this lane's row are inside the window and the sequence (an empty
  // range for a row past the end), so the masked path tests a key with two compares
  const int j_lo = fa_row_lo(win, i);
  const int j_hi = row_ok ? min(fa_row_hi(win, i), lkv - 1) : j_lo - 1;
  const float slope_l2 = pse_slopes(ALIBI) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
  // generated pse on positions in the unsplit sequence: sequence 0 of mode 8 starts qStartIdx -
  // kvStartIdx rows after its keys, so its bias uses j - (i + poff)
  const int poff = b == 0 ? p.pse_off0 : 0;
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
  // swizzled 16-bit tiles: K chunk 2c + hh of row lrow (+32 for the second key block),
  // V^T reads of rows rv and rv + 8 (+16 per 16-key step), chunk 4db + qv
  int koff[S::kSwz ? S::NQ : 1], voff[2][S::kSwz ? S::NDB : 1];
  if constexpr (S::kSwz) {
#pragma unroll
    for (int c = 0; c < S::NQ; ++c) koff[c] = lrow * S::RB + 16 * ((2 * c + hh) ^ tile_swz<S::RB>(lrow));
    const int rv = 4 * (grp >> 1) + (sl >> 2), qv = 2 * (grp & 1) + ((sl & 3) >> 1), bv = 8 * (sl & 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
        voff[hf][db] = (rv + 8 * hf) * S::RB + 16 * ((4 * db + qv) ^ tile_swz<S::RB>(rv + 8 * hf)) + bv;
  }

  auto classify = [&](int t) {
    RowTile rt;
    const int c0 = t * kFwdBN;
    rt.live = wr0 < lq && !fa_tile_empty(win, wr0, min(wr0 + 32, lq), c0, min(c0 + kFwdBN, lkv));
    // with an attenMask every tile takes the masked path
    rt.full = fa_tile_full(win, wr0, 32, c0, kFwdBN, lq, lkv) && !MASK;
    rt.bits[0] = rt.bits[1] = ~0u;
    rt.mw[0] = rt.mw[1] = 0u;
    if constexpr (MASK) {
      if (rt.live && row_ok) {
        const uint32_t* mr = p.mbits + (int64_t)i * p.mwords + (c0 >> 5);
        rt.mw[0] = mr[0];
        rt.mw[1] = (c0 >> 5) + 1 < p.mwords ? mr[1] : ~0u;
      }
    }
    if constexpr (DROP) {
      if (rt.live) {
        const int64_t pos = p.bit_base[b] + ((int64_t)h * lq + i) * lkv + c0;
        rt.bits[0] = load_mask_bits32(p.drop, p.drop_bytes, pos);
        rt.bits[1] = load_mask_bits32(p.drop, p.drop_bytes, pos + 32);
      }
    }
    return rt;
  };

  // S^T = K Q^T for the tile's two 32-key blocks.  The LDS reads of block 1 are
  // issued between the MFMAs of block 0, so only the first reads wait on LDS.
  auto scores = [&](const char* ks, f32x16 (&s)[2]) {
    if constexpr (k16) {
      V8 a0[S::NQ], a1[S::NQ];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) a0[c] = lds_read_b128<V8>(ks + koff[c]);
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) a1[c] = lds_read_b128<V8>(ks + koff[c] + 32 * S::RB);
      s[0] = f32x16{};
      s[1] = f32x16{};
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) s[0] = mfma32(a0[c], qf[c], s[0]);
#pragma unroll
      for (int c = 0; c < S::NQ; ++c) s[1] = mfma32(a1[c], qf[c], s[1]);
      // all reads of block 0, then one read of block 1 after each MFMA of block 0
      __builtin_amdgcn_sched_group_barrier(0x100, S::NQ, 0);
      sched_alternate<S::NQ, 0x008, 0x100>();
      __builtin_amdgcn_sched_group_barrier(0x008, S::NQ, 0);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int c = 0; c < S::NQ; ++c) {
          const float a = *reinterpret_cast<const float*>(ks + lrow * S::KP + kb * 32 * S::KP + (2 * c + hh) * 4);
          s[kb] = mfma32(a, qf[c], s[kb]);
        }
      }
    }
  };

  // Online-softmax step on key tile c0..c0+63: turns the scores into
  // probabilities (the post-dropout operand of P V), updates m / l and rescales O
  // when the exponent offset moves.
  auto softmax = [&](auto full_c, f32x16 (&s)[2], int c0, const RowTile& rt) {
    constexpr bool plain = !ALIBI && decltype(full_c)::value;   // logits are just sc * s
    float mt = kNegInf;
    if constexpr (plain) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      mt *= sc;
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = c0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          float x = s[kb][r] * sc;
          if constexpr (ALIBI == kPseExt)
            x = __builtin_fmaf(p.pse_coef, (row_ok && j < lkv) ? pse_value<T>(p, b, h, i, j, lq) : 0.f, x);
          else if constexpr (ALIBI != 0)
            x = add_pse<ALIBI>(x, slope_l2, (float)(j - i - poff));
          if constexpr (DROP) {
            // (the dropout instances keep the short-circuit form: the bounds would cost them registers)
            if (!decltype(full_c)::value &&
                (!fa_allowed(win, i, j, lq, lkv) || (MASK && ((rt.mw[kb] >> (8 * (r >> 2) + 4 * hh + (r & 3))) & 1u))))
              x = kNegInf;
          } else if constexpr (!decltype(full_c)::value) {
            bool ok = (j >= j_lo) & (j <= j_hi);
            if constexpr (MASK) ok &= !((rt.mw[kb] >> (8 * (r >> 2) + 4 * hh + (r & 3))) & 1u);
            x = ok ? x : kNegInf;
          }
          s[kb][r] = x;
          mt = fmaxf(mt, x);
        }
      }
    }
    mt = half_max(mt);
    m_true = fmaxf(m_true, mt);
    const bool need = mt > m_run + kLazy;   // also true on the first finite maximum
    const float alpha = need ? fast_exp2(m_run - mt) : 1.f;   // 0 when m_run = -inf
    m_run = need ? mt : m_run;
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float lsum[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = plain ? fast_exp2(__builtin_fmaf(s[kb][r], sc, -m_use)) : fast_exp2(s[kb][r] - m_use);
        lsum[kb] += e;
        if constexpr (DROP) {
          const int bit = 8 * (r >> 2) + 4 * hh + (r & 3);
          s[kb][r] = ((rt.bits[kb] >> bit) & 1u) ? e : 0.f;
        } else {
          s[kb][r] = e;
        }
      }
    l_run = l_run * alpha + (lsum[0] + lsum[1]);
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) o[db] *= alpha;
    }
  };

  // O^T += V^T P^T.  The transposing reads of each 16-key step are issued
  // between the MFMAs of the previous step.
  auto pv = [&](const char* vs, f32x16 (&s)[2]) {
    if constexpr (k16) {
      V8 pb[4];
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        const int kb = c2 >> 1, sub = c2 & 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[c2][j] = cvt16<E>(s[kb][8 * sub + j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      V8 a[4][S::NDB];
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        const char* vrow = vs + (16 * c2) * S::RB;
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) a[c2][db] = lds_read_tr_x2<V8>(vrow + voff[0][db], vrow + voff[1][db]);
      }
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) o[db] = mfma32(a[c2][db], pb[c2], o[db]);
      // reads of step 0, then two reads (one operand of step c2+1) after each MFMA of step c2
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * S::NDB, 0);
      sched_alternate<3 * S::NDB, 0x008, 0x100, 2>();
      __builtin_amdgcn_sched_group_barrier(0x008, S::NDB, 0);
      __builtin_amdgcn_sched_barrier(0);
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

  // softmax + P V of one tile whose scores are in s
  auto finish = [&](f32x16 (&s)[2], int t, const RowTile& rt, const char* vs) {
    if (rt.full) softmax(std::true_type{}, s, t * kFwdBN, rt);
    else softmax(std::false_type{}, s, t * kFwdBN, rt);
    pv(vs, s);
  };

  // K and V tiles share their geometry and row stride, so one set of lane offsets serves both
  SwzLane<kFwdBN, S::kSwz ? S::RB : 256, NW> cp;
  if constexpr (S::kSwz) cp.init(kv_stride, wave, lane);
  auto load_k = [&](char* dst, int t) {
    if constexpr (S::kSwz) cp.copy(dst, kbase, kv_stride, t * kFwdBN, lkv, wave, lane);
    else dma_rows<kFwdBN, S::RB, S::KP, NW>(dst, kbase, kv_stride, t * kFwdBN, lkv, wave, lane);
  };
  auto load_v = [&](char* dst, int t) {
    if constexpr (S::kSwz) cp.copy(dst, vbase, kv_stride, t * kFwdBN, lkv, wave, lane);
    else dma_rows<kFwdBN, S::RB, S::VP, NW>(dst, vbase, kv_stride, t * kFwdBN, lkv, wave, lane);
  };

  const int t_lo = it.lo, t_hi = it.hi;
  if (t_lo < t_hi) {
    load_k(kst[0], t_lo);
    load_v(vst[0], t_lo);
    dma_wait();
    __syncthreads();
  }
  // two stages: the copies of tile t+1 (into kn, vn) are in flight while tile t
  // (kc, vc) is computed
  char* kc = kst[0];
  char* kn = kst[1];
  char* vc = vst[0];
  char* vn = vst[1];
  // with keep-mask or attenMask words to fetch, a tile is classified one tile
  // ahead, beside its copies, so those loads are in flight during the tile before
  // (without them, classifying in place is the faster schedule)
  constexpr bool kAhead = DROP || MASK;
  RowTile rt_next{};
  if (kAhead && t_lo < t_hi) rt_next = classify(t_lo);
  for (int t = t_lo; t < t_hi; ++t) {
    RowTile rt;
    if constexpr (kAhead) rt = rt_next;
    if (t + 1 < t_hi) {
      load_k(kn, t + 1);
      load_v(vn, t + 1);
      if constexpr (kAhead) rt_next = classify(t + 1);
    }
    if constexpr (!kAhead) rt = classify(t);
    if (rt.live) {
      if (lane == 0) FA_TRACE_VISIT(p.trace, (((int64_t)b * p.nq + h) * p.trace_rb + (wr0 >> 5)) * p.trace_kt + t);
      f32x16 s[2];
      scores(kc, s);
      finish(s, t, rt, vc);
    }
    dma_wait();
    __syncthreads();
    char* tk = kc;
    kc = kn;
    kn = tk;
    char* tv = vc;
    vc = vn;
    vn = tv;
  }

  // ---- epilogue: O = o / (keep * l_run); l reported against the true maximum ----
  const float l_tot = half_sum(l_run);
  if (row_ok) {
    const int64_t rowg = q0 + i;
    const float inv = l_tot > 0.f ? p.inv_keep / l_tot : 0.f;
    T* op = reinterpret_cast<T*>(p.o) + (rowg * p.nq + h) * D;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 32 * db + 8 * a + 4 * hh;
        if constexpr (k16) {
          V4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = cvt16<E>(o[db][4 * a + e] * inv);
          *reinterpret_cast<V4*>(op + d) = v;
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
  const bool drop = p.use_dropout != 0;
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int NWD = fwd_waves(true, F32), NWP = fwd_waves(false, F32);
  constexpr int OCD = fwd_occupancy(true, F32), OCP = fwd_occupancy(false, F32);
  const dim3 grid((unsigned)blocks), block(64 * (drop ? NWD : NWP));
  return with_flags<sizeof(T) == 4>(drop, pse_kind(p), p.mbits != nullptr, [&](auto dr, auto al, auto mk) {
    constexpr bool DR = decltype(dr)::value;
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, DR ? NWD : NWP, DR ? OCD : OCP, DR, decltype(al)::value,
                                      decltype(mk)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

hipError_t launch_fwd(int dtype, int d, const FwdParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return launch_fwd_t<__bf16, 128>(p, s);
  if (dtype == 1 && d == 64) return launch_fwd_t<__bf16, 64>(p, s);
  if (dtype == 2 && d == 128) return launch_fwd_t<_Float16, 128>(p, s);
  if (dtype == 2 && d == 64) return launch_fwd_t<_Float16, 64>(p, s);
  if (dtype == 0 && d == 128) return launch_fwd_t<float, 128>(p, s);
  if (dtype == 0 && d == 64) return launch_fwd_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
