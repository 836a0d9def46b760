// Device helpers for the gfx950 (CDNA4) attention kernels: MFMA operand types,
// the LDS transpose read, 16-bit rounding and the dropout keep-bit window.
// 16-bit element types: __bf16 and _Float16 share every layout below (their
// MFMAs, v_mfma_f32_32x32x16_bf16 / _f16, take the same operand shapes).
//
// MFMA lane layouts used throughout (checked on the device):
//   v_mfma_f32_32x32x16_bf16  A[m][k]: lane l holds m = l%32, k = 8*(l/32) + 0..7
//                             B[k][n]: lane l holds n = l%32, k = 8*(l/32) + 0..7
//                             C[m][n]: lane l, reg r holds n = l%32,
//                                      m = 8*(r/4) + 4*(l/32) + r%4
//   v_mfma_f32_32x32x2_f32    A: m = l%32, k = l/32;  B: n = l%32, k = l/32; C as above.
// ds_read_b64_tr_b16: inside each group of 16 lanes, element e of lane i's
// result is element i%4 of the 8-byte row addressed by lane 4*e + i/4 of the group.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((address_space(3))) char lds_char;

// MFMA operand vectors of a 16-bit element type E (the fp32 kernels name bf16
// vectors in code they never instantiate)
template <typename E>
struct Vec16 {
  using v8 = bf16x8;
  using v4 = bf16x4;
};
template <>
struct Vec16<_Float16> {
  using v8 = f16x8;
  using v4 = f16x4;
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two transposing LDS reads -> one 8-element 16-bit operand V (see layout note above).
template <typename V = bf16x8>
__device__ __forceinline__ V lds_read_tr_x2(const char* p0, const char* p1) {
  // address-space casts (not integer round trips) keep constant offsets foldable into the instruction
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  V r;
  s16x4* rp = reinterpret_cast<s16x4*>(&r);
  rp[0] = lo;
  rp[1] = hi;
  return r;
}

template <typename V = bf16x8>
__device__ __forceinline__ V lds_read_b128(const char* p) {
  return *reinterpret_cast<const V*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine lane l with lane l^32 (the two halves of a wave hold the two k-groups
// of one MFMA row): one v_permlane32_swap, no LDS round trip.  Both lanes of a
// pair get the same bits (the sum is formed in the same order on both).
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Generated position bias (pseType 2 / 3 of aclnnFlashAttentionScoreV2, pseType
// table), added after scaling, in the log2 domain: slope_l2 = slope * log2(e),
// jmi = j - i (local key minus local row).
//   KIND 1 (pseType 2): -slope * (i - j)
//   KIND 2 (pseType 3): -slope * sqrt(|i - j|)
template <int KIND>
__device__ __forceinline__ float add_pse(float x, float slope_l2, float jmi) {
  if constexpr (KIND == 2) return __builtin_fmaf(-slope_l2, __builtin_amdgcn_sqrtf(__builtin_fabsf(jmi)), x);
  else return __builtin_fmaf(slope_l2, jmi, x);
}

// External pse (pseShiftOptional of the grad page, realShiftOptional of the
// ScoreV2 page) of local row i, key j of (sequence b, query head h), stored as
// [batch or 1, Nq, rows, pse_cols] in the input type.  The stored row of i:
//   mode 0: row i;  mode 1: the single row (shared by every query row);
//   mode 2 (1024-row alibi compression, the last 1024 rows of the full pse):
//     row i - max(0, Lq - 1024); a row above the stored block repeats the first
//     stored row shifted along its diagonal (value(i, j) = value(i + t, j + t)).
// The caller keeps i < Lq and j < Lkv.
template <typename T, typename P>
__device__ __forceinline__ float pse_value(const P& p, int b, int h, int i, int j, int lq) {
  int r = i, c = j;
  if (p.pse_mode == 1) {
    r = 0;
  } else if (p.pse_mode == 2) {
    r = i - (lq > 1024 ? lq - 1024 : 0);
    if (r < 0) {
      c = j - r;
      r = 0;
    }
  }
  const T* base = reinterpret_cast<const T*>(p.pse) + (int64_t)b * p.pse_bstride + (int64_t)h * p.pse_hstride;
  return (float)base[(int64_t)r * p.pse_cols + c];
}

// f32 -> 16-bit element (round to nearest even) and 16-bit element bits -> f32
template <typename E>
__device__ __forceinline__ E cvt16(float f) { return (E)f; }
template <typename E>
__device__ __forceinline__ float bits16_to_f32(uint16_t b) {
  if constexpr (sizeof(E) == 2 && !std::is_same<E, _Float16>::value) return __uint_as_float(((uint32_t)b) << 16);
  else return (float)__builtin_bit_cast(_Float16, b);
}

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<__bf16> {
  static constexpr int kBytes = 2;
  static constexpr int kChunk = 16;  // k per MFMA
};
template <>
struct ElemTraits<_Float16> {
  static constexpr int kBytes = 2;
  static constexpr int kChunk = 16;
};
template <>
struct ElemTraits<float> {
  static constexpr int kBytes = 4;
  static constexpr int kChunk = 2;
};

// Scheduling-group pattern for __builtin_amdgcn_sched_group_barrier (instruction
// classes: 0x002 VALU, 0x008 MFMA, 0x100 LDS read): N times { 1 of A, NB of B }.
template <int N, int A, int B, int NB = 1>
__device__ __forceinline__ void sched_alternate() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(A, 1, 0);
    __builtin_amdgcn_sched_group_barrier(B, NB, 0);
    sched_alternate<N - 1, A, B, NB>();
  }
}
// Load one 32-bit word of the packed keep mask; words that reach past the end
// of the buffer are assembled from the bytes that exist.
__device__ __forceinline__ uint32_t load_mask_word(const uint8_t* mask, int64_t nbytes, int64_t word) {
  int64_t byte = word * 4;
  if (byte + 4 <= nbytes) return *reinterpret_cast<const uint32_t*>(mask + byte);
  uint32_t v = 0;
  for (int i = 0; i < 4; ++i)
    if (byte + i < nbytes && byte + i >= 0) v |= ((uint32_t)mask[byte + i]) << (8 * i);
  return v;
}

// 32 consecutive keep bits starting at bit `pos` (LSB = bit pos).
__device__ __forceinline__ uint32_t load_mask_bits32(const uint8_t* mask, int64_t nbytes, int64_t pos) {
  const int64_t w = pos >> 5;
  const uint32_t sh = (uint32_t)(pos & 31);
  const uint32_t lo = load_mask_word(mask, nbytes, w);
  const uint32_t hi = sh ? load_mask_word(mask, nbytes, w + 1) : 0u;
  return sh ? ((lo >> sh) | (hi << (32 - sh))) : lo;
}

// 64 consecutive keep bits starting at bit `pos` (LSB = bit pos).
__device__ __forceinline__ uint64_t load_mask_window(const uint8_t* mask, int64_t nbytes, int64_t pos) {
  int64_t w = pos >> 5;
  uint32_t sh = (uint32_t)(pos & 31);
  uint64_t lo = (uint64_t)load_mask_word(mask, nbytes, w) | ((uint64_t)load_mask_word(mask, nbytes, w + 1) << 32);
  uint64_t hi = (uint64_t)load_mask_word(mask, nbytes, w + 2);
  return sh ? ((lo >> sh) | (hi << (64 - sh))) : lo;
}

// One global_load_lds_dword issued from asm: 64 lanes copy 4 bytes each from
// gbase + voff (gbase wave-uniform, voff per lane) into LDS at lds + 4*lane.
// The compiler does not see these copies, so it never makes LDS reads wait for
// them; the kernel drains them itself with dma_wait() before the barrier that
// publishes the tile.
__device__ __forceinline__ void dma_dword(const char* lds, const void* gbase, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_char*)(uintptr_t)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %1, %2" ::"{m0}"(m0), "v"(voff), "s"(gbase) : "memory");
}

// Wait until every LDS copy this wave issued has landed.
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The NW waves of a workgroup copy ROWS rows of RB bytes straight from global
// memory into an LDS tile whose rows are P bytes apart, one dword-per-lane copy
// per row (rows of 128 bytes use the first 32 lanes, rows of 512 bytes take two
// copies).  Wave w copies rows [w*ROWS/NW, (w+1)*ROWS/NW); every address is
// wave-uniform apart from the lane offset.  Row r is read from gbase + r' * gstride
// with r' = row0 + r, or r' = 0 when row0 + r is not below `valid` (finite data
// that the caller masks); valid must be >= 1.  When all of a wave's rows are
// valid the source address of full-wave rows just steps by gstride.
template <int ROWS, int RB, int P, int NW = 4>
__device__ __forceinline__ void dma_rows(char* lds, const char* gbase, int64_t gstride, int row0, int valid,
                                         int wave, int lane) {
  static_assert(ROWS % NW == 0, "rows split over the waves");
  static_assert(RB == 128 || RB % 256 == 0, "row size");
  constexpr int RPW = ROWS / NW;
  constexpr int LANES = RB >= 256 ? 64 : RB / 4;  // active lanes per copy
  constexpr int IPR = RB >= 256 ? RB / 256 : 1;   // copies per row
  // the row numbers are wave-uniform; say so, so the copy addresses stay scalar
  const int w = __builtin_amdgcn_readfirstlane(wave);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  valid = __builtin_amdgcn_readfirstlane(valid);
  const int r0 = w * RPW;
  char* dst = lds + r0 * P;
  if constexpr (LANES == 64) {
    if (row0 + r0 + RPW <= valid) {
      const char* src = gbase + (int64_t)(row0 + r0) * gstride;
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
#pragma unroll
        for (int u = 0; u < IPR; ++u) dma_dword(dst + k * P + 256 * u, src + 256 * u, 4 * lane);
        src += gstride;
      }
      return;
    }
  }
  // short rows (a partial wave copies each row: the address must stay scalar
  // inside the lane-masked region) and the sequence tail
  if (LANES == 64 || lane < LANES) {
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int gr = (row0 + r0 + k < valid) ? row0 + r0 + k : 0;
      const char* src = gbase + (int64_t)gr * gstride;
#pragma unroll
      for (int u = 0; u < IPR; ++u) dma_dword(dst + k * P + 256 * u, src + 256 * u, 4 * lane);
    }
  }
}

// ---- swizzled 16-bit tiles ----
// Rows of RB = 128 or 256 bytes are stored back to back (no padding); the
// 16-byte chunk q of row r sits at r*RB + 16*(q ^ tile_swz<RB>(r)).  Under this
// XOR pattern both operand reads of the kernels are free of LDS bank conflicts:
// 16-byte row reads (16 lanes = 16 consecutive rows, one chunk) and the
// transposing 8-byte reads (each half-wave covers 4 consecutive rows x 64 bytes).
template <int RB>
__device__ __forceinline__ int tile_swz(int r) {
  static_assert(RB == 128 || RB == 256, "row size");
  if constexpr (RB == 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// One global_load_lds_dwordx4: lane i copies 16 bytes from gbase + voff into
// LDS at lds + 16*i (1 KB per wave).  Drained like dma_dword.
__device__ __forceinline__ void dma_x4(const char* lds, const void* gbase, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_char*)(uintptr_t)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"{m0}"(m0), "v"(voff), "s"(gbase) : "memory");
}

// The NW waves copy ROWS rows of RB bytes (row r' = row0 + r read from
// gbase + r' * gstride) into a swizzled LDS tile, 1 KB per instruction: lane i
// writes chunk slot i % (RB/16) of tile row r = base + i / (RB/16) and so
// fetches chunk (slot ^ tile_swz(r)) of that row.  Rows at or beyond `valid`
// repeat row valid - 1 (finite data that the caller masks); row0 < valid.
template <int ROWS, int RB, int NW>
__device__ __forceinline__ void dma_tile_swz(char* lds, const char* gbase, int64_t gstride, int row0, int valid,
                                             int wave, int lane) {
  constexpr int RPI = 1024 / RB;   // rows per instruction
  constexpr int CPR = RB / 16;     // chunks per row
  constexpr int NI = ROWS / RPI;   // instructions per tile
  static_assert(NI % NW == 0, "instructions split over the waves");
  constexpr int IPW = NI / NW;
  const int w = __builtin_amdgcn_readfirstlane(wave);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  valid = __builtin_amdgcn_readfirstlane(valid);
  const char* src = gbase + (int64_t)row0 * gstride;
  const int lr = lane / CPR, slot = lane % CPR;
  const int last = valid - 1 - row0;   // last valid tile row (>= 0)
#pragma unroll
  for (int k = 0; k < IPW; ++k) {
    const int r = (w * IPW + k) * RPI + lr;   // this lane's tile row
    const int rc = r < last ? r : last;
    const uint32_t voff = (uint32_t)rc * (uint32_t)gstride + 16u * (uint32_t)(slot ^ tile_swz<RB>(r));
    dma_x4(lds + (w * IPW + k) * 1024, src, voff);
  }
}

// The same copies with the lane offsets of a whole valid tile formed once (SwzLane::init),
// outside the caller's tile loop: a tile whose rows are all below `valid` issues its copies
// with them directly; the sequence's last, partial tile takes the clamped offsets above.
template <int ROWS, int RB, int NW>
struct SwzLane {
  static constexpr int RPI = 1024 / RB, CPR = RB / 16, IPW = ROWS / RPI / NW;
  uint32_t voff[IPW];
  __device__ __forceinline__ void init(int64_t gstride, int wave, int lane) {
    const int w = __builtin_amdgcn_readfirstlane(wave);
    const int lr = lane / CPR, slot = lane % CPR;
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      const int r = (w * IPW + k) * RPI + lr;
      voff[k] = (uint32_t)r * (uint32_t)gstride + 16u * (uint32_t)(slot ^ tile_swz<RB>(r));
    }
  }
  __device__ __forceinline__ void copy(char* lds, const char* gbase, int64_t gstride, int row0, int valid, int wave,
                                       int lane) const {
    const int w = __builtin_amdgcn_readfirstlane(wave);
    const int r0 = __builtin_amdgcn_readfirstlane(row0);
    if (__builtin_amdgcn_readfirstlane(valid) - r0 >= ROWS) {
      const char* src = gbase + (int64_t)r0 * gstride;
#pragma unroll
      for (int k = 0; k < IPW; ++k) dma_x4(lds + (w * IPW + k) * 1024, src, voff[k]);
    } else {
      dma_tile_swz<ROWS, RB, NW>(lds, gbase, gstride, row0, valid, wave, lane);
    }
  }
};

// Same tile layout as dma_rows, copied through registers (global load, then LDS
// store) so that no copy is in flight once it returns.  Used by kernels that may
// keep scratch spills, which must never coexist with in-flight LDS DMA.
template <int ROWS, int RB, int P>
__device__ __forceinline__ void copy_rows(char* lds, const char* gbase, int64_t gstride, int row0, int valid,
                                          int tid) {
  constexpr int CPR = RB / 16;                       // 16-byte chunks per row
  static_assert((ROWS * CPR) % 256 == 0, "chunks split over 256 threads");
#pragma unroll
  for (int n = 0; n < ROWS * CPR / 256; ++n) {
    const int ci = tid + 256 * n;
    const int r = ci / CPR, cc = ci % CPR;
    const int gr = (row0 + r < valid) ? row0 + r : 0;
    const u32x4 v = *reinterpret_cast<const u32x4*>(gbase + (int64_t)gr * gstride + 16 * cc);
    *reinterpret_cast<u32x4*>(lds + r * P + 16 * cc) = v;
  }
}

}  // namespace fa
