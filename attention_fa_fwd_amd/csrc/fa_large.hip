// Head dims above 128 (up to 512), and 16-bit inputs with an external pse: the
// forward and backward of aclnnFlashAttentionScoreV2 /
// aclnnFlashAttentionUnpaddingScoreGrad ("Formula") with the scores of a chunk of
// query rows materialised in the workspace.
//
// The fused kernels keep a wave's Q (or K, V) rows and its O (or dK, dV, dQ) in
// registers, which stops fitting beyond D = 128; their 16-bit instances have no
// external-pse variant.  This path runs, per (sequence, chunk of R query rows),
// over every query head at once
// (query head h reads kv head h / G):
//   forward   S = Q K^T (MFMA GEMM, fp32) -> masked softmax (m, l, P~ in the input
//             type) -> O = P~ V (GEMM)
//   backward  S = Q K^T, dP = dY V^T (GEMMs) -> P, P~, dS (kernel, input type)
//             -> dQ = scale dS K (GEMM over the whole key window, written once)
//             -> dV += P~^T dY, dK += scale dS^T Q (GEMMs into fp32 accumulators, the
//             G query heads of each kv head one after the other, chunk by chunk)
// The mask window prunes the work: score tiles with no allowed pair are not
// computed (their entries are never read), and the contractions over keys (O, dQ)
// or rows (dK, dV) run over the window of their tile only.  D_i, lse2 and the
// dSink partials come from a row-dot kernel for any head dim.  Every step is a
// fixed-order computation: bitwise reproducible.  The rounding points match the
// fused kernels (P~ and dS in the input type, fp32 accumulation).
#include <algorithm>
#include <cstring>
#include <vector>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

// ------------------------------------------------------------------ batched GEMM
// C[z][m][n] = alpha * sum_k A[z][m][k] B[z / b_zdiv][k][n] (+ C[z][m][n] when
// accumulating, fp32 C only), element strides throughout.  Each operand has a unit
// stride along one of its two dimensions (k or m for A, k or n for B), so it
// arrives in 16-byte pieces (`vec`: the host checked that every row start is
// 16-byte aligned; otherwise element by element).
// window: 0 none; 1 skip the C tiles whose rows (m) and keys (n) share no allowed
// pair; 2 k = keys, limited per tile to those the rows m may see; 3 k = rows,
// limited per tile to those that see the keys m.  Rows are row0 + m (1, 2) or
// row0 + k (3), local to the sequence.
struct GemmDesc {
  const void* a;
  const void* b;
  void* c;
  int32_t m, n, k, batch, b_zdiv;
  int64_t a_sm, a_sk, a_sz;
  int64_t b_sk, b_sn, b_sz;
  int64_t c_sm, c_sn, c_sz;
  float alpha;
  int32_t accumulate, vec, window;
  FaWindow win;
  int32_t row0, lq, lkv;
};

constexpr int kGemmM = 128, kGemmN = 128, kGemmK = 32;

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

// 16-byte piece number `c` of a 128 x 32 operand tile (rows r of the M or N side,
// k columns), stored into LDS rows of PITCH elements with k contiguous.
template <typename T, int PITCH>
struct TileLoad {
  static constexpr int CH = 16 / sizeof(T);            // elements per piece
  static constexpr int PER = kGemmM * kGemmK / CH / 256;   // pieces per thread
  // kfast: k is the unit-stride dimension (pieces run along k); else the row dimension is
  __device__ static void load(const T* base, int64_t s_r, int64_t s_k, bool kfast, bool vec, int r0, int rmax,
                              int k0, int klo, int khi, int tid, T (&reg)[PER][CH]) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + 256 * u;
      int r, k;
      if (kfast) {
        r = c / (kGemmK / CH);
        k = (c % (kGemmK / CH)) * CH;
      } else {
        k = c / (kGemmM / CH);
        r = (c % (kGemmM / CH)) * CH;
      }
      const int gr = r0 + r, gk = k0 + k;
      const bool full = kfast ? (gr < rmax && gk >= klo && gk + CH <= khi) : (gk >= klo && gk < khi && gr + CH <= rmax);
      if (vec && full) {
        const T* src = base + (int64_t)gr * s_r + (int64_t)gk * s_k;
        *reinterpret_cast<u32x4*>(&reg[u][0]) = *reinterpret_cast<const u32x4*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          const int rr = kfast ? gr : gr + e, kk = kfast ? gk + e : gk;
          reg[u][e] = (rr < rmax && kk >= klo && kk < khi) ? base[(int64_t)rr * s_r + (int64_t)kk * s_k] : T{};
        }
      }
    }
  }
  // kfast: rows of PITCH elements, k contiguous.  Otherwise 16-bit tiles are stored as
  // they arrive, k rows of 128 elements (256 bytes) with the XOR swizzle of the fused
  // kernels (16-byte chunk q of row k at k * 256 + 16 * (q ^ tile_swz(k))), and read
  // through the transposing LDS read; fp32 tiles are transposed element by element.
  __device__ static void store(T* lds, bool kfast, int tid, const T (&reg)[PER][CH]) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + 256 * u;
      if (kfast) {
        const int r = c / (kGemmK / CH), k = (c % (kGemmK / CH)) * CH;
        *reinterpret_cast<u32x4*>(&lds[r * PITCH + k]) = *reinterpret_cast<const u32x4*>(&reg[u][0]);
      } else if constexpr (sizeof(T) == 2) {
        const int k = c / (kGemmM / CH), q = c % (kGemmM / CH);
        char* row = reinterpret_cast<char*>(lds) + k * 256;
        *reinterpret_cast<u32x4*>(row + 16 * (q ^ tile_swz<256>(k))) = *reinterpret_cast<const u32x4*>(&reg[u][0]);
      } else {
        const int k = c / (kGemmM / CH), r = (c % (kGemmM / CH)) * CH;
#pragma unroll
        for (int e = 0; e < CH; ++e) lds[(r + e) * PITCH + k] = reg[u][e];
      }
    }
  }
};

// AK / BK: the A / B operand has unit stride along k (otherwise along m / n).
template <typename Tin, typename Tout, bool AK, bool BK>
__global__ __launch_bounds__(256) void fa_gemm_kernel(GemmDesc g) {
  constexpr int PITCH = kGemmK + 16 / (int)sizeof(Tin);   // padded k-contiguous rows
  constexpr int TILE = kGemmM * PITCH;                    // >= kGemmK * kGemmM (the [k][row] layout)
  static_assert(kGemmM == kGemmN && kGemmK * kGemmM <= TILE, "one tile size for both layouts");
  using L = TileLoad<Tin, PITCH>;
  __shared__ __attribute__((aligned(16))) Tin as[2][TILE];
  __shared__ __attribute__((aligned(16))) Tin bs[2][TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * kGemmN, m0 = blockIdx.y * kGemmM, z = blockIdx.z;
  // mask-window pruning of this tile
  int klo = 0, khi = g.k;
  if (g.window == 1) {
    const int i0 = g.row0 + m0, i1 = min(g.row0 + m0 + kGemmM, g.row0 + g.m);
    if (fa_tile_empty(g.win, i0, i1, n0, min(n0 + kGemmN, g.n))) return;
  } else if (g.window == 2) {
    const int i0 = g.row0 + m0, i1 = min(g.row0 + m0 + kGemmM, g.row0 + g.m);
    klo = max(0, fa_row_lo(g.win, i0));
    khi = min(g.k, fa_row_hi(g.win, i1 - 1) + 1);
  } else if (g.window == 3) {
    const int j0 = m0, j1 = min(m0 + kGemmM, g.m);   // keys of the tile
    const int ilo = g.win.floor >= j0 ? 0 : j0 - g.win.delta - g.win.next;
    const int ihi = j1 - 1 - g.win.delta + g.win.pre;
    klo = max(0, ilo - g.row0);
    khi = min(g.k, ihi - g.row0 + 1);
  }
  const int kstart = klo > 0 ? klo / kGemmK * kGemmK : 0;
  const Tin* A = reinterpret_cast<const Tin*>(g.a) + (int64_t)z * g.a_sz;
  const Tin* B = reinterpret_cast<const Tin*>(g.b) + (int64_t)(z / g.b_zdiv) * g.b_sz;
  constexpr bool a_kfast = AK, b_kfast = BK;
  const int64_t a_sr = g.a_sm, b_sr = g.b_sn;   // strides of the row (m / n) dimension
  const bool vec = g.vec != 0;
  const int wm = 64 * (wave & 1), wn = 64 * (wave >> 1);
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
  Tin ra[L::PER][L::CH], rb[L::PER][L::CH];
  int buf = 0;
  if (kstart < khi) {
    L::load(A, a_sr, g.a_sk, a_kfast, vec, m0, g.m, kstart, klo, khi, tid, ra);
    L::load(B, b_sr, g.b_sk, b_kfast, vec, n0, g.n, kstart, klo, khi, tid, rb);
    L::store(as[0], a_kfast, tid, ra);
    L::store(bs[0], b_kfast, tid, rb);
    __syncthreads();
  }
  for (int k0 = kstart; k0 < khi; k0 += kGemmK) {
    const bool more = k0 + kGemmK < khi;
    if (more) {
      L::load(A, a_sr, g.a_sk, a_kfast, vec, m0, g.m, k0 + kGemmK, klo, khi, tid, ra);
      L::load(B, b_sr, g.b_sk, b_kfast, vec, n0, g.n, k0 + kGemmK, klo, khi, tid, rb);
    }
    const Tin* at = as[buf];
    const Tin* bt = bs[buf];
    if constexpr (sizeof(Tin) == 2) {
      using V8 = typename Vec16<Tin>::v8;
      // an operand of 32 rows (block rb of the 128) and 16 k, lane l holding row l % 32 and
      // k = 8 (l / 32) .. + 7 in order: 16-byte row reads of the k-contiguous layout, or two
      // transposing reads of the [k][row] layout.  In each 16-lane group, element e of a
      // transposing read comes from the 8-byte piece addressed by lane 4e + i / 4 (element
      // i % 4), so lane a addresses row k0 + a / 4 at rows 4 (a % 4) of its 16: k0 = 8 (l / 32)
      // for the first read and k0 + 4 for the second.  (The fused kernels pair rows rv and
      // rv + 8 instead, to match the k order of an accumulator turned operand.)
      const int grp = lane >> 4, sl = lane & 15;
      const int rv = 8 * (grp >> 1) + (sl >> 2), qv = 2 * (grp & 1) + ((sl & 3) >> 1), bv8 = 8 * (sl & 1);
      auto opnd = [&](const Tin* t, bool kf, int rb, int kc) -> V8 {
        if (kf) return *reinterpret_cast<const V8*>(&t[(32 * rb + (lane & 31)) * PITCH + 16 * kc + 8 * (lane >> 5)]);
        const char* base = reinterpret_cast<const char*>(t) + 16 * kc * 256;
        const int o0 = rv * 256 + 16 * ((4 * rb + qv) ^ tile_swz<256>(rv)) + bv8;
        const int o1 = (rv + 4) * 256 + 16 * ((4 * rb + qv) ^ tile_swz<256>(rv + 4)) + bv8;
        return lds_read_tr_x2<V8>(base + o0, base + o1);
      };
#pragma unroll
      for (int kc = 0; kc < kGemmK / 16; ++kc) {
        V8 av[2], bv[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          av[x] = opnd(at, AK, wm / 32 + x, kc);
          bv[x] = opnd(bt, BK, wn / 32 + x, kc);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[x][y] = mfma32(av[x], bv[y], acc[x][y]);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < kGemmK / 2; ++kc) {
        const int kk = 2 * kc + (lane >> 5);
        float av[2], bv[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          av[x] = at[(wm + 32 * x + (lane & 31)) * PITCH + kk];
          bv[x] = bt[(wn + 32 * x + (lane & 31)) * PITCH + kk];
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[x][y] = mfma32(av[x], bv[y], acc[x][y]);
      }
    }
    if (more) {
      // the other buffer was last read before the previous barrier
      L::store(as[buf ^ 1], a_kfast, tid, ra);
      L::store(bs[buf ^ 1], b_kfast, tid, rb);
    }
    __syncthreads();
    buf ^= 1;
  }
  // lane holds column n = lane % 32 and rows 8 (r / 4) + 4 (lane / 32) + r % 4 of each 32 x 32 block
  Tout* C = reinterpret_cast<Tout*>(g.c) + (int64_t)z * g.c_sz;
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int n = n0 + wn + 32 * y + (lane & 31);
    if (n >= g.n) continue;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm + 32 * x + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < g.m) {
          Tout* cp = C + (int64_t)m * g.c_sm + (int64_t)n * g.c_sn;
          float v = g.alpha * acc[x][y][r];
          if constexpr (sizeof(Tout) == 4) {
            if (g.accumulate) v += *cp;
          }
          *cp = from_f32<Tout>(v);
        }
      }
  }
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename Tin, typename Tout>
static hipError_t gemm(GemmDesc g, hipStream_t s) {
  if (g.m <= 0 || g.n <= 0 || g.batch <= 0) return hipSuccess;
  if ((g.a_sk != 1 && g.a_sm != 1) || (g.b_sk != 1 && g.b_sn != 1) || g.b_zdiv < 1) return hipErrorInvalidValue;
  // 16-byte pieces need every non-unit stride (rows and batches) to keep 16-byte alignment
  const int64_t eb = sizeof(Tin);
  const int64_t an = g.a_sk == 1 ? g.a_sm : g.a_sk, bn = g.b_sk == 1 ? g.b_sn : g.b_sk;
  g.vec = aligned16(g.a) && aligned16(g.b) && (an * eb) % 16 == 0 && (bn * eb) % 16 == 0 &&
          (g.a_sz * eb) % 16 == 0 && (g.b_sz * eb) % 16 == 0;
  const dim3 grid((unsigned)((g.n + kGemmN - 1) / kGemmN), (unsigned)((g.m + kGemmM - 1) / kGemmM), (unsigned)g.batch);
  const bool ak = g.a_sk == 1, bk = g.b_sk == 1;
  if (ak && bk) hipLaunchKernelGGL((fa_gemm_kernel<Tin, Tout, true, true>), grid, dim3(256), 0, s, g);
  else if (ak) hipLaunchKernelGGL((fa_gemm_kernel<Tin, Tout, true, false>), grid, dim3(256), 0, s, g);
  else if (bk) hipLaunchKernelGGL((fa_gemm_kernel<Tin, Tout, false, true>), grid, dim3(256), 0, s, g);
  else hipLaunchKernelGGL((fa_gemm_kernel<Tin, Tout, false, false>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

// ------------------------------------------------------------------ logits
// Logit of local row i, key j of (sequence b, query head h) in the log2 domain:
// scale * s * log2(e) plus the position bias.  The caller has checked the window.
template <typename T, typename P>
__device__ __forceinline__ float large_logit(const P& p, int pse, int b, int h, int i, int j, int lq, float s,
                                            float slope_l2, int poff) {
  float x = s * p.scale_log2;
  if (pse == kPseExt) x = __builtin_fmaf(p.pse_coef, pse_value<T>(p, b, h, i, j, lq), x);
  else if (pse == kPseLinear) x = add_pse<kPseLinear>(x, slope_l2, (float)(j - i - poff));
  else if (pse == kPseSqrt) x = add_pse<kPseSqrt>(x, slope_l2, (float)(j - i - poff));
  return x;
}

// inside the window and not removed by the attenMask
template <typename P>
__device__ __forceinline__ bool large_allowed(const P& p, const FaWindow& win, int i, int j, int lq, int lkv) {
  if (!fa_allowed(win, i, j, lq, lkv)) return false;
  return !(p.mbits && ((p.mbits[(int64_t)i * p.mwords + (j >> 5)] >> (j & 31)) & 1u));
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

// Chunk of `rows` query rows of sequence b (local rows r0 ..), all query heads; the
// scores of head h, row r, key j sit at (h * rows + r) * ld + j.
struct LargeChunk {
  int32_t b, r0, rows, lq, lkv, q0, k0, ld;
};

// Keys [*lo, *hi) of chunk row r whose P~ / dS the contractions read: the key window of
// its 128-row GEMM tile (O, dQ), and the 128-key tiles its own window touches (dK, dV).
// Entries outside the row's own window in this range are written as zeros; entries
// outside it are never read.
__device__ __forceinline__ void large_read_range(const FaWindow& win, const LargeChunk& c, int r, int* lo, int* hi) {
  const int t0 = c.r0 + r / kGemmM * kGemmM, t1 = min(t0 + kGemmM, c.r0 + c.rows) - 1;
  int zlo = max(0, fa_row_lo(win, t0)), zhi = min(c.lkv, fa_row_hi(win, t1) + 1);
  const int i = c.r0 + r;
  const int rlo = max(0, fa_row_lo(win, i)), rhi = min(c.lkv, fa_row_hi(win, i) + 1);
  if (rlo < rhi) {
    zlo = min(zlo, rlo / kGemmM * kGemmM);
    zhi = max(zhi, min(c.lkv, (rhi + kGemmM - 1) / kGemmM * kGemmM));
  }
  *lo = zlo;
  *hi = zhi;
}

// Four consecutive entries of a score row in the input type (8 bytes for 16-bit types, 16 for fp32).
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    using V4 = typename Vec16<T>::v4;
    V4 v;
    v[0] = cvt16<T>(a);
    v[1] = cvt16<T>(b);
    v[2] = cvt16<T>(c);
    v[3] = cvt16<T>(d);
    *reinterpret_cast<V4*>(dst) = v;
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
  }
}

// Score rows are read and written four entries per lane from key j0 = zlo rounded down
// to 4 (rows are ld = a multiple of 8 entries long, so no access leaves the row); entries
// outside the read range [zlo, zhi) are written as zeros, which nothing reads.
constexpr int kSoftCache = 16;   // four-entry pieces per lane kept in registers: one pass over S up to 4,096 keys

// Forward softmax: one wave per (head, row).  S -> P~ (input type; P / l with dropout
// applied; 0 outside the mask, where S was not computed), softmax max / sum.  Rows whose
// read range fits kSoftCache pieces per lane read S once (the logits stay in registers);
// longer rows take three passes.
template <typename T>
__global__ __launch_bounds__(256) void fa_large_softmax_kernel(FwdParams p, LargeChunk c, const float* S, T* Pt) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= p.nq * c.rows) return;
  const int h = wid / c.rows, r = wid - h * c.rows;
  const int i = c.r0 + r, b = c.b;
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, c.lq, c.lkv, p.prefix[b]);
  const int pse = pse_kind(p);
  const float slope_l2 = (pse == kPseLinear || pse == kPseSqrt) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
  const int poff = b == 0 ? p.pse_off0 : 0;
  const float* srow = S + ((int64_t)h * c.rows + r) * c.ld;
  T* prow = Pt + ((int64_t)h * c.rows + r) * c.ld;
  const float sink2 = p.sink ? p.sink[h] * kLog2e : kNegInf;
  const int wlo = max(0, fa_row_lo(win, i)), whi = min(c.lkv, fa_row_hi(win, i) + 1);   // the row's window
  int zlo, zhi;
  large_read_range(win, c, r, &zlo, &zhi);
  const int j0 = zlo & ~3;
  // logit of key j, or -inf where the pair is not allowed (S there was not computed)
  auto logit = [&](int j, float sv) {
    return (j >= wlo && j < whi && large_allowed(p, win, i, j, c.lq, c.lkv))
               ? large_logit<T>(p, pse, b, h, i, j, c.lq, sv, slope_l2, poff)
               : kNegInf;
  };
  float mx, l;
  if (zhi - j0 <= 256 * kSoftCache) {
    f32x4 x[kSoftCache];
    mx = kNegInf;
#pragma unroll
    for (int u = 0; u < kSoftCache; ++u) {
      const int j = j0 + 4 * lane + 256 * u;
      x[u] = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
      if (j < zhi) {
        const f32x4 sv = *reinterpret_cast<const f32x4*>(srow + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[u][e] = logit(j + e, sv[e]);
          mx = fmaxf(mx, x[u][e]);
        }
      }
    }
    mx = fmaxf(wave_max(mx), sink2);
    const float mu = mx == kNegInf ? 0.f : mx;
    l = 0.f;
#pragma unroll
    for (int u = 0; u < kSoftCache; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) l += fast_exp2(x[u][e] - mu);   // 0 for -inf
    l = wave_sum(l) + (p.sink ? fast_exp2(sink2 - mu) : 0.f);
    const float inv = l > 0.f ? p.inv_keep / l : 0.f;
#pragma unroll
    for (int u = 0; u < kSoftCache; ++u) {
      const int j = j0 + 4 * lane + 256 * u;
      if (j < zhi) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (x[u][e] != kNegInf && keep_bit(p, b, h, i, j + e, c.lq, c.lkv)) ? fast_exp2(x[u][e] - mu) * inv : 0.f;
        store4(prow + j, v[0], v[1], v[2], v[3]);
      }
    }
  } else {
    mx = kNegInf;
    for (int j = j0 + 4 * lane; j < zhi; j += 256) {
      const f32x4 sv = *reinterpret_cast<const f32x4*>(srow + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, logit(j + e, sv[e]));
    }
    mx = fmaxf(wave_max(mx), sink2);
    const float mu = mx == kNegInf ? 0.f : mx;
    l = 0.f;
    for (int j = j0 + 4 * lane; j < zhi; j += 256) {
      const f32x4 sv = *reinterpret_cast<const f32x4*>(srow + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) l += fast_exp2(logit(j + e, sv[e]) - mu);
    }
    l = wave_sum(l) + (p.sink ? fast_exp2(sink2 - mu) : 0.f);
    const float inv = l > 0.f ? p.inv_keep / l : 0.f;
    for (int j = j0 + 4 * lane; j < zhi; j += 256) {
      const f32x4 sv = *reinterpret_cast<const f32x4*>(srow + j);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xe = logit(j + e, sv[e]);
        v[e] = (xe != kNegInf && keep_bit(p, b, h, i, j + e, c.lq, c.lkv)) ? fast_exp2(xe - mu) * inv : 0.f;
      }
      store4(prow + j, v[0], v[1], v[2], v[3]);
    }
  }
  if (lane == 0) {
    const int64_t idx = (int64_t)(c.q0 + i) * p.nq + h;
    p.m_out[idx] = mx * kLn2;
    p.l_out[idx] = l;
  }
}

// Backward: one wave per (head, row), four entries per lane.  S, dP (fp32) -> P~ and dS
// (input type): P = 2^(x - lse2), P~ = P z / keep, dS = P (dP z / keep - D_i); both 0
// outside the mask, where S and dP were not computed.
template <typename T>
__global__ __launch_bounds__(256) void fa_large_ds_kernel(BwdParams p, LargeChunk c, const float* S, const float* dP,
                                                         T* Pt, T* dS) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= p.nq * c.rows) return;
  const int h = wid / c.rows, r = wid - h * c.rows;
  const int i = c.r0 + r, b = c.b;
  const FaWindow win = fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, c.lq, c.lkv, p.prefix[b]);
  const int pse = pse_kind(p);
  const float slope_l2 = (pse == kPseLinear || pse == kPseSqrt) ? p.slopes[b * p.slope_bstride + h] * kLog2e : 0.f;
  const int poff = b == 0 ? p.pse_off0 : 0;
  const int64_t idx = (int64_t)(c.q0 + i) * p.nq + h;
  const float lse2 = p.lse[idx], di = p.delta[idx];
  const int64_t o = ((int64_t)h * c.rows + r) * c.ld;
  int zlo, zhi;
  large_read_range(win, c, r, &zlo, &zhi);
#pragma unroll 2
  for (int j = (zlo & ~3) + 4 * lane; j < zhi; j += 256) {
    const f32x4 sv = *reinterpret_cast<const f32x4*>(S + o + j);
    const f32x4 dv = *reinterpret_cast<const f32x4*>(dP + o + j);
    float pt[4], ds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jj = j + e;
      pt[e] = 0.f;
      ds[e] = 0.f;
      if (jj >= zlo && jj < zhi && large_allowed(p, win, i, jj, c.lq, c.lkv)) {
        const float x = large_logit<T>(p, pse, b, h, i, jj, c.lq, sv[e], slope_l2, poff);
        const float pr = fast_exp2(x - lse2);   // 0 for rows without any allowed key (lse2 = +inf)
        const bool keep = keep_bit(p, b, h, i, jj, c.lq, c.lkv);
        const float dpv = keep ? dv[e] * p.inv_keep : 0.f;
        pt[e] = keep ? pr * p.inv_keep : 0.f;
        ds[e] = pr * (dpv - di);
      }
    }
    store4(Pt + o + j, pt[0], pt[1], pt[2], pt[3]);
    store4(dS + o + j, ds[0], ds[1], ds[2], ds[3]);
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

// fp32 accumulators [Nkv][ld_acc rows][d] -> rows k0 .. k0 + rows - 1 of a [T_kv, Nkv, d] tensor
template <typename T>
__global__ __launch_bounds__(256) void fa_large_store_kernel(const float* acc, T* out, int64_t rows, int64_t acc_rows,
                                                            int d, int nkv, int64_t k0) {
  const int64_t n = (int64_t)nkv * rows * d;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) {
    const int64_t e = x % d, j = (x / d) % rows, g = x / (d * rows);
    out[((k0 + j) * nkv + g) * d + e] = from_f32<T>(acc[(g * acc_rows + j) * d + e]);
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

template <typename P>
static FaWindow host_window(const P& p, const LargePlan& L, int b, int lq, int lkv) {
  return fa_make_window(fa_seq_mode(p.mode, b, p.nseq), p.pre, p.next, lq, lkv, L.prefix[b]);
}

// ------------------------------------------------------------------ host drivers
template <typename T>
static hipError_t large_fwd_t(const FwdParams& p, const LargePlan& L, char* ws, hipStream_t s) {
  const int G = p.group, d = L.d, nq = p.nq;
  float* S = reinterpret_cast<float*>(ws + L.off_s);
  T* Pt = reinterpret_cast<T*>(ws + L.off_p);
  hipError_t e = hipSuccess;
  for (int b = 0; b < L.batch && e == hipSuccess; ++b) {
    const int lq = L.cu_q[b + 1] - L.cu_q[b], lkv = L.cu_kv[b + 1] - L.cu_kv[b];
    const FaWindow win = host_window(p, L, b, lq, lkv);
    for (int r0 = 0; r0 < lq && e == hipSuccess; r0 += L.rows) {
      const LargeChunk c{b, r0, std::min(L.rows, lq - r0), lq, lkv, L.cu_q[b], L.cu_kv[b], L.ld};
      const T* q = reinterpret_cast<const T*>(p.q) + (int64_t)(c.q0 + r0) * nq * d;
      const T* k = reinterpret_cast<const T*>(p.k) + (int64_t)c.k0 * p.nkv * d;
      const T* v = reinterpret_cast<const T*>(p.v) + (int64_t)c.k0 * p.nkv * d;
      T* o = reinterpret_cast<T*>(p.o) + (int64_t)(c.q0 + r0) * nq * d;
      const int64_t sz = (int64_t)c.rows * c.ld;
      // S[h][r][j] = Q[r, h] . K[j, h / G]  (tiles outside the window skipped)
      GemmDesc gs{q, k, S, c.rows, lkv, d, nq, G, (int64_t)nq * d, 1, d, 1, (int64_t)p.nkv * d, d, c.ld, 1, sz,
                  1.f, 0, 0, 1, win, r0, lq, lkv};
      if ((e = gemm<T, float>(gs, s)) != hipSuccess) break;
      hipLaunchKernelGGL((fa_large_softmax_kernel<T>), dim3((unsigned)((nq * c.rows + 3) / 4)), dim3(256), 0, s, p, c,
                         S, Pt);
      if ((e = hipGetLastError()) != hipSuccess) break;
      // O[r, h] = P~[h][r] V[., h / G] over the keys the rows may see
      GemmDesc go{Pt, v, o, c.rows, d, lkv, nq, G, c.ld, 1, sz, (int64_t)p.nkv * d, 1, d, (int64_t)nq * d, 1, d,
                  1.f, 0, 0, 2, win, r0, lq, lkv};
      e = gemm<T, T>(go, s);
    }
  }
  return e;
}

template <typename T>
static hipError_t large_bwd_t(const BwdParams& p, const LargePlan& L, char* ws, hipStream_t s) {
  const int G = p.group, d = L.d, nq = p.nq, nkv = p.nkv;
  float* S = reinterpret_cast<float*>(ws + L.off_s);
  float* dP = reinterpret_cast<float*>(ws + L.off_dp);
  T* Pt = reinterpret_cast<T*>(ws + L.off_p);
  T* dS = reinterpret_cast<T*>(ws + L.off_ds);
  float* dk_acc = reinterpret_cast<float*>(ws + L.off_dk);
  float* dv_acc = reinterpret_cast<float*>(ws + L.off_dv);
  hipError_t e = hipSuccess;
  if (p.n_pre_blocks > 0) {
    hipLaunchKernelGGL((fa_large_pre_kernel<T>), dim3((unsigned)p.n_pre_blocks), dim3(256),
                       sizeof(float) * kPreRowsPerBlock * nq, s, p, d);
    e = hipGetLastError();
  }
  const int64_t qs = (int64_t)nq * d, ks = (int64_t)nkv * d;
  for (int b = 0; b < L.batch && e == hipSuccess; ++b) {
    const int lq = L.cu_q[b + 1] - L.cu_q[b], lkv = L.cu_kv[b + 1] - L.cu_kv[b];
    const int q0 = L.cu_q[b], k0 = L.cu_kv[b];
    if (lkv == 0) {
      // no keys: the sequence's dQ rows are zero (and it has no dK / dV rows)
      const int64_t n = (int64_t)lq * qs;
      if (n > 0) {
        hipLaunchKernelGGL((fa_large_zero_kernel<T>), dim3(blocks_for(n)), dim3(256), 0, s,
                           reinterpret_cast<T*>(p.dq) + (int64_t)q0 * qs, n);
        e = hipGetLastError();
      }
      continue;
    }
    const FaWindow win = host_window(p, L, b, lq, lkv);
    const int64_t acc_rows = L.acc_rows, kn = (int64_t)nkv * acc_rows * d;
    hipLaunchKernelGGL(fa_large_zero_kernel<float>, dim3(blocks_for(kn)), dim3(256), 0, s, dk_acc, kn);
    hipLaunchKernelGGL(fa_large_zero_kernel<float>, dim3(blocks_for(kn)), dim3(256), 0, s, dv_acc, kn);
    if ((e = hipGetLastError()) != hipSuccess) break;
    const T* k = reinterpret_cast<const T*>(p.k) + (int64_t)k0 * ks;
    const T* v = reinterpret_cast<const T*>(p.v) + (int64_t)k0 * ks;
    for (int r0 = 0; r0 < lq && e == hipSuccess; r0 += L.rows) {
      const LargeChunk c{b, r0, std::min(L.rows, lq - r0), lq, lkv, q0, k0, L.ld};
      const int64_t qrow = (int64_t)(q0 + r0) * qs;
      const T* q = reinterpret_cast<const T*>(p.q) + qrow;
      const T* dy = reinterpret_cast<const T*>(p.dy) + qrow;
      T* dq = reinterpret_cast<T*>(p.dq) + qrow;
      const int64_t sz = (int64_t)c.rows * c.ld;
      GemmDesc gs{q, k, S, c.rows, lkv, d, nq, G, qs, 1, d, 1, ks, d, c.ld, 1, sz, 1.f, 0, 0, 1, win, r0, lq, lkv};
      GemmDesc gp{dy, v, dP, c.rows, lkv, d, nq, G, qs, 1, d, 1, ks, d, c.ld, 1, sz, 1.f, 0, 0, 1, win, r0, lq, lkv};
      if ((e = gemm<T, float>(gs, s)) != hipSuccess || (e = gemm<T, float>(gp, s)) != hipSuccess) break;
      hipLaunchKernelGGL((fa_large_ds_kernel<T>), dim3((unsigned)((nq * c.rows + 3) / 4)), dim3(256), 0, s, p, c, S,
                         dP, Pt, dS);
      if ((e = hipGetLastError()) != hipSuccess) break;
      // dQ[r, h] = scale dS[h][r] K[., h / G] over the keys the rows may see
      GemmDesc gq{dS, k, dq, c.rows, d, lkv, nq, G, c.ld, 1, sz, ks, 1, d, qs, 1, d, p.scale, 0, 0, 2, win, r0, lq,
                  lkv};
      if ((e = gemm<T, T>(gq, s)) != hipSuccess) break;
      // dV[g] += P~[gG + hh]^T dY[., gG + hh], dK[g] += scale dS[gG + hh]^T Q[., gG + hh]: every kv head at once,
      // the heads of a group one after the other, over the rows that see each key tile
      for (int hh = 0; hh < G && e == hipSuccess; ++hh) {
        GemmDesc gv{Pt + hh * sz, dy + (int64_t)hh * d, dv_acc, lkv, d, c.rows, nkv, 1, 1, c.ld, G * sz, qs, 1,
                    (int64_t)G * d, d, 1, acc_rows * d, 1.f, 1, 0, 3, win, r0, lq, lkv};
        GemmDesc gk{dS + hh * sz, q + (int64_t)hh * d, dk_acc, lkv, d, c.rows, nkv, 1, 1, c.ld, G * sz, qs, 1,
                    (int64_t)G * d, d, 1, acc_rows * d, p.scale, 1, 0, 3, win, r0, lq, lkv};
        if ((e = gemm<T, float>(gv, s)) == hipSuccess) e = gemm<T, float>(gk, s);
      }
    }
    if (e != hipSuccess) break;
    hipLaunchKernelGGL((fa_large_store_kernel<T>), dim3(blocks_for(kn)), dim3(256), 0, s, dk_acc,
                       reinterpret_cast<T*>(p.dk), (int64_t)lkv, acc_rows, d, nkv, (int64_t)k0);
    hipLaunchKernelGGL((fa_large_store_kernel<T>), dim3(blocks_for(kn)), dim3(256), 0, s, dv_acc,
                       reinterpret_cast<T*>(p.dv), (int64_t)lkv, acc_rows, d, nkv, (int64_t)k0);
    e = hipGetLastError();
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
