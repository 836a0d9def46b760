// Device helpers for the gfx950 (CDNA4) attention kernels: MFMA operand types,
// the LDS transpose read, bf16 rounding and the dropout keep-bit window.
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

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two transposing LDS reads -> one bf16x8 operand (see layout note above).
__device__ __forceinline__ bf16x8 lds_read_tr_x2(const char* p0, const char* p1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
      (lds_char*)(uintptr_t)p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
      (lds_char*)(uintptr_t)p1));
  bf16x8 r;
  s16x4* rp = reinterpret_cast<s16x4*>(&r);
  rp[0] = lo;
  rp[1] = hi;
  return r;
}

// N/2 bf16x8 operands (N transposing 8-byte reads) from one LDS base address and
// compile-time byte offsets; operand k pairs the reads at offsets OFF[2k], OFF[2k+1].
// The reads and their completion wait live in one asm block, so every output is
// complete when the block ends.  Keeping these reads out of the compiler's view
// also keeps it from waiting on global_load_lds copies into other LDS buffers.
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read_tr_4(const char* base, bf16x8& a0, bf16x8& a1) {
  u32x2 r0, r1, r2, r3;
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_char*)(uintptr_t)base;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3)
      : "memory");
  u32x4 x0 = {r0[0], r0[1], r1[0], r1[1]};
  u32x4 x1 = {r2[0], r2[1], r3[0], r3[1]};
  a0 = __builtin_bit_cast(bf16x8, x0);
  a1 = __builtin_bit_cast(bf16x8, x1);
}

template <int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void lds_read_tr_8(const char* base, bf16x8& a0, bf16x8& a1, bf16x8& a2, bf16x8& a3) {
  u32x2 r0, r1, r2, r3, r4, r5, r6, r7;
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_char*)(uintptr_t)base;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%9\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:%15\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3), "i"(O4), "i"(O5), "i"(O6), "i"(O7)
      : "memory");
  a0 = __builtin_bit_cast(bf16x8, (u32x4){r0[0], r0[1], r1[0], r1[1]});
  a1 = __builtin_bit_cast(bf16x8, (u32x4){r2[0], r2[1], r3[0], r3[1]});
  a2 = __builtin_bit_cast(bf16x8, (u32x4){r4[0], r4[1], r5[0], r5[1]});
  a3 = __builtin_bit_cast(bf16x8, (u32x4){r6[0], r6[1], r7[0], r7[1]});
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

// bf16 <-> f32 (round to nearest even)
__device__ __forceinline__ __bf16 to_bf16(float f) { return (__bf16)f; }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<__bf16> {
  static constexpr int kBytes = 2;
  static constexpr int kChunk = 16;  // k per MFMA
};
template <>
struct ElemTraits<float> {
  static constexpr int kBytes = 4;
  static constexpr int kChunk = 2;
};

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

// 64 consecutive keep bits starting at bit `pos` (LSB = bit pos).
__device__ __forceinline__ uint64_t load_mask_window(const uint8_t* mask, int64_t nbytes, int64_t pos) {
  int64_t w = pos >> 5;
  uint32_t sh = (uint32_t)(pos & 31);
  uint64_t lo = (uint64_t)load_mask_word(mask, nbytes, w) | ((uint64_t)load_mask_word(mask, nbytes, w + 1) << 32);
  uint64_t hi = (uint64_t)load_mask_word(mask, nbytes, w + 2);
  return sh ? ((lo >> sh) | (hi << (64 - sh))) : lo;
}

// The four waves of a 256-thread workgroup copy ROWS rows of RB bytes straight
// from global memory into an LDS tile whose rows are P bytes apart, one row per
// global_load_lds_dword instruction (each lane moves 4 bytes into LDS slot
// base + 4*lane; rows of 128 bytes use the first 32 lanes, rows of 512 bytes take
// two instructions).  Wave w copies rows [w*ROWS/4, (w+1)*ROWS/4); every address
// is wave-uniform, so the copy costs scalar arithmetic only.  Row r is read from
// gbase + r' * gstride with r' = row0 + r, or r' = 0 when row0 + r is not below
// `valid` (finite data that the caller masks); valid must be >= 1.
template <int ROWS, int RB, int P>
__device__ __forceinline__ void dma_rows(char* lds, const char* gbase, int64_t gstride, int row0, int valid,
                                         int wave, int lane) {
  static_assert(ROWS % 4 == 0, "rows split over four waves");
  static_assert(RB == 128 || RB % 256 == 0, "row size");
  constexpr int RPW = ROWS / 4;
  constexpr int LANES = RB >= 256 ? 64 : RB / 4;  // active lanes per instruction
  constexpr int IPR = RB >= 256 ? RB / 256 : 1;   // instructions per row
  const int w = __builtin_amdgcn_readfirstlane(wave);
  if (lane < LANES) {
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int r = w * RPW + k;
      const int gr = (row0 + r < valid) ? row0 + r : 0;
      const char* src = gbase + (int64_t)gr * gstride + 4 * lane;
#pragma unroll
      for (int u = 0; u < IPR; ++u)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + 256 * u),
                                         (__attribute__((address_space(3))) void*)(lds_char*)(uintptr_t)(lds + r * P + 256 * u),
                                         4, 0, 0);
    }
  }
}

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
