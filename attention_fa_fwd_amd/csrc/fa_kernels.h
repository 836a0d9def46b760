// Kernel parameter blocks and launch declarations shared by the kernels and
// the host runtime.  All pointers are device pointers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

// Work item of the forward and dQ passes: one query tile of one sequence,
// with the half-open range of key tiles that hold at least one allowed pair.
// For the dK/dV pass `tile` is a key tile and [lo, hi) a range of query tiles.
struct WorkItem {
  int32_t b, tile, lo, hi;
};

// Visited-tile counters of the trace build (FA_TRACE_VISITS): each pass counts every tile
// it computes, indexed ((sequence * Nq + head) * trace_rb + row block) * trace_kt + key
// tile; a pass whose pointer is null is not counted, and the product build compiles the
// counting out.
#if defined(FA_TRACE_VISITS)
#define FA_TRACE_VISIT(ptr, idx) \
  do {                                \
    if (ptr) atomicAdd((ptr) + (idx), 1u); \
  } while (0)
#else
#define FA_TRACE_VISIT(ptr, idx) ((void)0)
#endif

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* m_out;
  float* l_out;
  const uint8_t* drop;
  int64_t drop_bytes;
  const float* slopes;
  int32_t slope_bstride;    // 0: slopes [Nq]; Nq: slopes [B, Nq]
  int32_t pse_sqrt;         // 1: the slopes generate pseType 3 (square-root distance)
  const void* pse;          // external pse [pse batch, Nq, rows, pse_cols] of the input type, or null
  int64_t pse_bstride;      // elements between sequences' blocks (0: one block for every sequence)
  int64_t pse_hstride;      // elements between heads' blocks (rows * pse_cols)
  int32_t pse_cols;
  int32_t pse_mode;         // row of local row i: 0 row i; 1 the only row; 2 1024-row alibi compression
  float pse_coef;           // log2(e) (pseType 0) or scale * log2(e) (pseType 1)
  const float* sink;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int64_t* bit_base;
  const int32_t* prefix;    // per sequence: prefix N of sparse mode 6 (0 otherwise)
  const uint32_t* mbits;    // packed attenMask (1 = masked) [mask rows][mwords], or null
  int32_t mwords;           // 32-key words per packed mask row
  const WorkItem* items;
  int32_t n_items;
  int32_t nq, nkv, group;
  int32_t mode, pre, next;
  int32_t nseq;       // sequences (sparse modes 7 and 8 pick a mask per sequence)
  int32_t pse_off0;   // sequence 0's generated pse uses row i + pse_off0 (qStartIdx - kvStartIdx, mode 8)
  float scale_log2;   // scale * log2(e)
  float inv_keep;     // 1 / keep_prob
  int32_t use_dropout;
  int32_t head_swizzle;
  uint32_t* trace;    // trace build: visits per (sequence, head, 32-row block, 64-key tile)
  int32_t trace_rb, trace_kt;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dy;
  const void* o;
  const float* m_in;
  const float* l_in;
  void* dq;
  void* dk;
  void* dv;
  float* dsink;
  float* dq_acc;       // fp32 [T_q, Nq, D] accumulator (atomic variant)
  float* delta;        // fp32 [T_q, Nq]  rowsum(dY * O)
  float* lse;          // fp32 [T_q, Nq]  log2-domain log-sum-exp (+inf for empty rows)
  float* dsink_part;   // fp32 [n_pre_blocks, Nq]
  const uint8_t* drop;
  int64_t drop_bytes;
  const float* slopes;
  int32_t slope_bstride;    // 0: slopes [Nq]; Nq: slopes [B, Nq]
  int32_t pse_sqrt;         // 1: the slopes generate pseType 3 (square-root distance)
  const void* pse;          // external pse [pse batch, Nq, rows, pse_cols] of the input type, or null
  int64_t pse_bstride;      // elements between sequences' blocks (0: one block for every sequence)
  int64_t pse_hstride;      // elements between heads' blocks (rows * pse_cols)
  int32_t pse_cols;
  int32_t pse_mode;         // row of local row i: 0 row i; 1 the only row; 2 1024-row alibi compression
  float pse_coef;           // log2(e) (pseType 0) or scale * log2(e) (pseType 1)
  const float* sink;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int64_t* bit_base;
  const int32_t* prefix;    // per sequence: prefix N of sparse mode 6 (0 otherwise)
  const uint32_t* mbits;    // packed attenMask (1 = masked) [mask rows][mwords], or null
  int32_t mwords;           // 32-key words per packed mask row
  const int32_t* row_seq;   // sequence index of each query token (preprocess)
  const WorkItem* kv_items;
  const WorkItem* dq_items;
  int32_t n_kv_items, n_dq_items;
  int32_t total_q;
  int32_t nq, nkv, group;
  int32_t mode, pre, next;
  int32_t nseq;       // sequences (sparse modes 7 and 8 pick a mask per sequence)
  int32_t pse_off0;   // sequence 0's generated pse uses row i + pse_off0 (qStartIdx - kvStartIdx, mode 8)
  float scale;
  float scale_log2;
  float inv_keep;
  int32_t use_dropout;
  int32_t head_swizzle;
  int32_t n_pre_blocks;
  uint32_t* trace_kv;   // trace build: dK/dV steps per (sequence, head, 64-row tile, 128-key tile)
  uint32_t* trace_dq;   // trace build: dQ tiles per (sequence, head, 32-row block, 64-key tile)
  int32_t trace_kv_rb, trace_kv_kt, trace_dq_rb, trace_dq_kt;
};

// Decode attention: one work item = a key range [lo, hi) of one (sequence b,
// kv head g); slot >= 0 names its partial-result row when the sequence is split
// over several items, slot < 0 means the item covers the sequence and writes
// the output itself.
struct DecItem {
  int32_t b, g, lo, hi, slot;
};

// Decode workgroup: kDecWaves waves, each streaming its own share of the item's
// keys through a kDecStages-deep LDS ring of 32-key K/V blocks (two blocks in
// flight per wave; at D = 128 the three rings take 144 KB of the CU's 160 KB).
constexpr int kDecWaves = 3;
constexpr int kDecStages = 3;
constexpr int kDecBlock = 32;   // keys per step

struct DecParams {
  const void* q;            // [B, Nq, D]
  const void* k;            // KV cache, element (b, s, g, d) at b*kv_bstride + s*kv_tstride + g*kv_hstride + d
  const void* v;
  void* out;                // [B, Nq, D]
  const uint8_t* mask;      // [B, mask_stride] (nonzero = masked), or null
  int64_t mask_stride;
  const DecItem* items;
  const int32_t* first_slot;   // [B * Nkv]: slot of the first item of (b, g), -1 when not split
  const int32_t* n_split;      // [B]: items per (b, g)
  float* part_o;               // [slots, group, D] unnormalised partial outputs
  float* part_m;               // [slots, group] log2-domain row maxima
  float* part_l;               // [slots, group] row sums
  int64_t kv_bstride, kv_tstride, kv_hstride;   // in elements
  int32_t nq, nkv, group, keys_per_wave, batch;
  float scale_log2;            // scale * log2(e)
};

// Tile shapes (rows x keys) of each pass; the host scheduler uses the same numbers.
// Forward workgroup: 4 waves of 32 query rows each; bf16 runs two workgroups
// per CU, fp32 one (its tiles fill the LDS).
constexpr int fwd_waves(bool dropout, bool fp32) { return 4; }
constexpr int fwd_occupancy(bool dropout, bool fp32) { return fp32 ? 1 : 2; }
constexpr int fwd_rows(bool dropout, bool fp32) { return 32 * fwd_waves(dropout, fp32); }
constexpr int kFwdBN = 64;
constexpr int kKvBN = 128, kKvBM = 64;
constexpr int kDqBM = 128, kDqBN = 64;
constexpr int kPreRowsPerBlock = 16;   // small, so that short batches still spread over every CU

// Kind of the position bias (the ALIBI template argument of the kernels): none,
// generated pseType 2 (linear distance) or 3 (square-root distance), or an
// external pse tensor (pseType 0 / 1).
constexpr int kPseNone = 0, kPseLinear = 1, kPseSqrt = 2, kPseExt = 3;
constexpr bool pse_slopes(int kind) { return kind == kPseLinear || kind == kPseSqrt; }
template <typename P>
__host__ __device__ int pse_kind(const P& p) {
  if (p.pse != nullptr) return kPseExt;
  return p.slopes == nullptr ? kPseNone : (p.pse_sqrt ? kPseSqrt : kPseLinear);
}

// Calls f(drop, pse, mask) with drop and mask as std::integral_constant<bool, .>
// and pse (a kPse* kind) as std::integral_constant<int, .>, so a launcher names
// one kernel instance per combination.  An external pse together with an
// attenMask has no instances (the heaviest of them would not fit the registers);
// the host rejects that combination.  kExtPse = false builds no external-pse
// instance at all (the 16-bit fused kernels: the host sends a 16-bit external pse
// to the materialised-score path).
template <bool kExtPse = true, typename F>
hipError_t with_flags(bool drop, int pse, bool mask, F&& f) {
  auto by_mask = [&](auto d, auto a) -> hipError_t {
    if constexpr (decltype(a)::value == kPseExt) {
      if (mask) return hipErrorInvalidValue;
      return f(d, a, std::false_type{});
    } else {
      return mask ? f(d, a, std::true_type{}) : f(d, a, std::false_type{});
    }
  };
  auto by_pse = [&](auto d) -> hipError_t {
    if (pse == kPseExt) {
      if constexpr (kExtPse) return by_mask(d, std::integral_constant<int, kPseExt>{});
      else return hipErrorInvalidValue;
    }
    if (pse == kPseSqrt) return by_mask(d, std::integral_constant<int, kPseSqrt>{});
    if (pse == kPseLinear) return by_mask(d, std::integral_constant<int, kPseLinear>{});
    return by_mask(d, std::integral_constant<int, kPseNone>{});
  };
  return drop ? by_pse(std::true_type{}) : by_pse(std::false_type{});
}

// Head dims above 128 (fa_large.hip): the work of a call split into chunks of
// `rows` query rows per sequence, every query head at once, with the scores of a
// chunk in the workspace.  cu_q / cu_kv / prefix are HOST copies of the sequence
// offsets and prefix lengths; the off_* are byte offsets into the workspace: fp32 S
// and dP, P~ and dS in the input type, [Nq][rows][ld] each (ld: the longest key
// range rounded up to 8); fp32 dK and dV accumulators [Nkv][acc_rows][d]
// (acc_rows: the longest key range).
struct LargePlan {
  int32_t batch, d, rows, ld, acc_rows;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* prefix;
  uint64_t off_s, off_dp, off_p, off_ds, off_dk, off_dv;
};
hipError_t launch_large_fwd(int dtype, const FwdParams& p, const LargePlan& L, char* ws, hipStream_t s);
hipError_t launch_large_bwd(int dtype, const BwdParams& p, const LargePlan& L, char* ws, hipStream_t s);

hipError_t launch_fwd(int dtype, int d, const FwdParams& p, hipStream_t s);
hipError_t launch_bwd_pre(int dtype, int d, const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_kv(int dtype, int d, bool atomic_dq, const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_kv_atomic(int dtype, int d, const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dq(int dtype, int d, const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dq_convert(int dtype, int d, const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dsink(const BwdParams& p, hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
hipError_t launch_decode(int dtype, int d, int n_items, const DecParams& p, hipStream_t s);
hipError_t launch_decode_reduce(int dtype, int d, const DecParams& p, hipStream_t s);
// layouts the relayout kernel converts to and from TND (values of FA_LAYOUT_BNSD / _SBH;
// kLayoutStrided: a TND tensor with its own token / head strides, B = 1)
constexpr int kLayoutBNSD = 3, kLayoutSBH = 4, kLayoutStrided = 100;
hipError_t launch_relayout(const void* src, void* dst, int64_t B, int64_t S, int64_t N, int64_t D, int64_t DK,
                           int ebytes, int layout, bool to_tnd, hipStream_t s, int64_t ts = 0, int64_t hs = 0);
hipError_t launch_mask_pack(const uint8_t* mask, int64_t rows, int64_t cols, uint32_t* bits, hipStream_t s);
// Copies `bytes` (a multiple of 16) of host memory to dst (16-byte aligned) through
// the arguments of kernel launches of kStageChunkBytes each: no host memory is
// referenced once the call returns, also when the launches are captured in a graph.
constexpr int kStageChunkBytes = 2048;
hipError_t launch_stage(char* dst, const char* src, size_t bytes, hipStream_t s);

}  // namespace fa
