// Host runtime of libfa.so: argument validation, the varlen tile scheduler,
// workspace layout, kernel launch sequences and the C ABI declared in fa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/fa.h"
#include "fa_kernels.h"
#include "fa_sched.h"

// Device scratch of fa_decode_noalloc: a file-scope array, so that entry point
// allocates nothing.  Every GPU the library runs on holds its own copy for the
// life of the process.  In host code `fa_noalloc_scratch` names a host-side
// stand-in, never the device memory: host code uses the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static constexpr uint64_t kNoallocScratchBytes = FA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char fa_noalloc_scratch[kNoallocScratchBytes];

namespace {

using fa::WorkItem;

constexpr int64_t kMaxTokens = int64_t(1) << 20;   // T and S limits of the grad pages ("Constraints")
constexpr int64_t kMaxBatch = 20000;               // B limit of the V5 grad page
constexpr int64_t kMaxHeads = 256;                 // Nq limit ("Nq ranges from 1 to 256")
constexpr int64_t kMaxHeadDim = 512;               // D limit of the grad page ("D 1-512")
constexpr int64_t kMaxPrefixBatch = 1024;          // B limit with prefixOptional (grad page "Constraints")

struct Problem {
  int64_t batch = 0, nq = 0, nkv = 0, d = 0, tq = 0, tkv = 0;
  int64_t du = 0;                  // head dim of Q, K, dQ, dK; d is the kernels' (64 or 128, du <= d; du above 128)
  int64_t dvu = 0;                 // head dim of V, O, dY, dV (<= du)
  int dtype = 0, mode = 0;
  double scale = 0, keep = 1;
  int64_t pre = 0, next = 0;
  bool deterministic = true;
  int layout = FA_LAYOUT_TND;      // fa_config.layout
  // strided TND tensors, index T_Q .. T_DV: (token, head) element strides and whether they
  // differ from the packed ones
  int64_t ts[8] = {}, hs[8] = {};
  bool strided[8] = {};
  const void* pse = nullptr;       // external pse (device) and its shape
  int64_t pse_batch = 0, pse_rows = 0, pse_cols = 0;
  int pse_type = 0, pse_mode = 0;  // mode: 0 row i, 1 single row, 2 1024-row compression
  int64_t sq = 0, skv = 0;         // common sequence lengths of the fixed-length layouts
  bool pse_sqrt = false;           // FA_FLAG_PSE_SQRT: the slopes generate pseType 3
  bool slopes_per_batch = false;   // FA_FLAG_SLOPES_PER_BATCH: slopes are [B, Nq]
  std::vector<int32_t> cu_q, cu_kv;
  std::vector<int64_t> bit_base;   // first keep bit of each sequence
  std::vector<int32_t> prefix;     // prefix N of each sequence (sparse mode 6; zeros otherwise)
  const uint8_t* mask = nullptr;   // attenMask (device) when the mode uses it
  int64_t mask_rows = 0, mask_cols = 0, mask_words = 0;   // words: 32-key words per packed row
  int64_t drop_bits = 0;
  int64_t q_start = 0, kv_start = 0;   // mode 8: positions of sequence 0 in its unsplit sequence
  bool has_start = false;
  bool large = false;   // the materialised-score path (fa_large.hip) runs the problem
};

static_assert(fa::kLayoutBNSD == FA_LAYOUT_BNSD && fa::kLayoutSBH == FA_LAYOUT_SBH, "layout codes");
enum TensorId { T_Q = 0, T_K, T_V, T_DY, T_O, T_DQ, T_DK, T_DV };
bool layout_copies(const Problem& pr) { return pr.layout == FA_LAYOUT_BNSD || pr.layout == FA_LAYOUT_SBH; }
// tensor `id` goes through a packed TND copy in the workspace
// head dim of tensor `id`: the value side (V, O, dY, dV) may be narrower than Q and K
int64_t dim_of(const Problem& pr, int id) {
  return (id == T_V || id == T_O || id == T_DY || id == T_DV) ? pr.dvu : pr.du;
}
bool copied(const Problem& pr, int id) { return layout_copies(pr) || pr.strided[id] || dim_of(pr, id) != pr.d; }
// any tensor does (the workspace then holds copies of all eight)
bool relayout(const Problem& pr) {
  if (layout_copies(pr) || pr.du != pr.d || pr.dvu != pr.d) return true;
  for (bool st : pr.strided)
    if (st) return true;
  return false;
}
int64_t elem_bytes(const Problem& pr) { return pr.dtype == FA_DTYPE_FP32 ? 4 : 2; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fa_status parse(const fa_config* cfg, Problem* pr) {
  if (!cfg || !cfg->cu_seqlens_q || !cfg->cu_seqlens_kv) return FA_ERR_PARAM_NULLPTR;
  if (cfg->batch < 1 || cfg->batch > kMaxBatch) return FA_ERR_PARAM_INVALID;
  if (cfg->head_num < 1 || cfg->head_num > kMaxHeads) return FA_ERR_PARAM_INVALID;
  const int64_t nkv = cfg->num_kv_heads == 0 ? cfg->head_num : cfg->num_kv_heads;
  if (nkv < 1 || cfg->head_num % nkv != 0) return FA_ERR_PARAM_INVALID;
  if (cfg->dtype != FA_DTYPE_FP32 && cfg->dtype != FA_DTYPE_BF16 && cfg->dtype != FA_DTYPE_FP16)
    return FA_ERR_PARAM_INVALID;
  // D <= 128 with rows of whole 16-byte chunks; the kernels run D = 64 and 128, other
  // head dims go through copies zero-padded to the next of them
  const int64_t ebytes = cfg->dtype == FA_DTYPE_FP32 ? 4 : 2;
  if (cfg->head_dim < 1 || cfg->head_dim > kMaxHeadDim || (cfg->head_dim * ebytes) % 16 != 0) return FA_ERR_PARAM_INVALID;
  // the value head dim may be smaller (grad page, Constraints: qD == kD >= vD); 0 = the same
  const int64_t vdim = cfg->v_head_dim == 0 ? cfg->head_dim : cfg->v_head_dim;
  if (vdim < 1 || vdim > cfg->head_dim || (vdim * ebytes) % 16 != 0) return FA_ERR_PARAM_INVALID;
  const int mode = cfg->sparse_mode;
  if (mode != FA_SPARSE_NONE && mode != FA_SPARSE_ALL_MASK && mode != FA_SPARSE_LEFT_UP_CAUSAL &&
      mode != FA_SPARSE_RIGHT_DOWN_CAUSAL && mode != FA_SPARSE_BAND && mode != FA_SPARSE_PREFIX &&
      mode != FA_SPARSE_RIGHT_DOWN_CAUSAL_BAND && mode != FA_SPARSE_BAND_LEFT_UP_CAUSAL)
    return FA_ERR_PARAM_INVALID;
  const bool band_mode = mode == FA_SPARSE_BAND || mode == FA_SPARSE_RIGHT_DOWN_CAUSAL_BAND ||
                         mode == FA_SPARSE_BAND_LEFT_UP_CAUSAL;
  if (mode == FA_SPARSE_ALL_MASK && !cfg->atten_mask) return FA_ERR_PARAM_NULLPTR;
  if (mode == FA_SPARSE_PREFIX && !cfg->prefix) return FA_ERR_PARAM_NULLPTR;
  if (mode == FA_SPARSE_PREFIX && cfg->batch > kMaxPrefixBatch) return FA_ERR_PARAM_INVALID;
  if (!(cfg->keep_prob > 0.0 && cfg->keep_prob <= 1.0)) return FA_ERR_PARAM_INVALID;
  if (!std::isfinite(cfg->scale)) return FA_ERR_PARAM_INVALID;
  if (band_mode && cfg->pre_tokens + cfg->next_tokens < 0) return FA_ERR_PARAM_INVALID;
  // start indices belong to the split of mode 8; modes 7 and 8 take no pse tensor
  if ((cfg->q_start_idx || cfg->kv_start_idx) && mode != FA_SPARSE_BAND_LEFT_UP_CAUSAL) return FA_ERR_PARAM_INVALID;
  if (cfg->pse && (mode == FA_SPARSE_RIGHT_DOWN_CAUSAL_BAND || mode == FA_SPARSE_BAND_LEFT_UP_CAUSAL))
    return FA_ERR_PARAM_INVALID;
  if (cfg->deterministic != 0 && cfg->deterministic != 1) return FA_ERR_PARAM_INVALID;
  if ((cfg->flags & ~(FA_FLAG_PSE_SQRT | FA_FLAG_SLOPES_PER_BATCH | FA_FLAG_ATOMIC_DQ)) != 0)
    return FA_ERR_PARAM_INVALID;

  pr->batch = cfg->batch;
  pr->nq = cfg->head_num;
  pr->nkv = nkv;
  pr->du = cfg->head_dim;
  pr->dvu = vdim;
  // the fused kernels take D = 64 or 128 (smaller head dims zero-padded); above 128 the
  // materialised-score path (fa_large.hip) takes the head dim as it is
  pr->d = cfg->head_dim <= 64 ? 64 : cfg->head_dim <= 128 ? 128 : cfg->head_dim;
  pr->dtype = cfg->dtype;
  pr->mode = mode;
  pr->pse_sqrt = (cfg->flags & FA_FLAG_PSE_SQRT) != 0;
  pr->slopes_per_batch = (cfg->flags & FA_FLAG_SLOPES_PER_BATCH) != 0;
  pr->scale = cfg->scale;
  pr->keep = cfg->keep_prob;
  pr->pre = cfg->pre_tokens;
  pr->next = cfg->next_tokens;
  // The non-deterministic mode allows the deterministic passes' result, and they are the
  // faster scheme here, so they run unless FA_FLAG_ATOMIC_DQ asks for atomic dQ.  That
  // variant is built for bf16, fp16 and for fp32 with D = 64 (head dims above 64 run the
  // D = 128 kernels).
  pr->deterministic = cfg->deterministic != 0 || (cfg->flags & FA_FLAG_ATOMIC_DQ) == 0 ||
                      (cfg->dtype == FA_DTYPE_FP32 && cfg->head_dim > 64) || cfg->head_dim > 128;
  const int64_t* cq = cfg->cu_seqlens_q;
  const int64_t* ck = cfg->cu_seqlens_kv;
  if (cq[0] != 0 || ck[0] != 0) return FA_ERR_PARAM_INVALID;
  pr->cu_q.resize(pr->batch + 1);
  pr->cu_kv.resize(pr->batch + 1);
  pr->bit_base.resize(pr->batch);
  int64_t bits = 0;
  for (int64_t b = 0; b <= pr->batch; ++b) {
    if (cq[b] < 0 || ck[b] < 0 || cq[b] > kMaxTokens || ck[b] > kMaxTokens) return FA_ERR_PARAM_INVALID;
    if (b > 0 && (cq[b] < cq[b - 1] || ck[b] < ck[b - 1])) return FA_ERR_PARAM_INVALID;
    pr->cu_q[b] = (int32_t)cq[b];
    pr->cu_kv[b] = (int32_t)ck[b];
    if (b < pr->batch) {
      pr->bit_base[b] = bits;
      // cq, ck are bounded by 2^20 here, so the products stay far below 2^63
      bits += pr->nq * (cq[b + 1] - cq[b]) * (ck[b + 1] - ck[b]);
    }
  }
  pr->prefix.assign(pr->batch, 0);
  if (mode == FA_SPARSE_PREFIX) {
    for (int64_t b = 0; b < pr->batch; ++b) {
      // prefix N range of the pages: [0, Lkv] when Lq > Lkv, else [Lkv - Lq, Lkv]
      const int64_t lq = cq[b + 1] - cq[b], lkv = ck[b + 1] - ck[b], n = cfg->prefix[b];
      const int64_t lo = lq > lkv ? 0 : lkv - lq;
      if (n < lo || n > lkv) return FA_ERR_PARAM_INVALID;
      pr->prefix[b] = (int32_t)n;
    }
  }
  pr->tq = cq[pr->batch];
  pr->tkv = ck[pr->batch];
  if (cfg->q_start_idx || cfg->kv_start_idx) {
    // the pages' constraint for a split in the query direction:
    // Lq_0 - Lkv_0 + qStartIdx - kvStartIdx == 0 (the chunk's last row meets its last key)
    pr->q_start = cfg->q_start_idx ? *cfg->q_start_idx : 0;
    pr->kv_start = cfg->kv_start_idx ? *cfg->kv_start_idx : 0;
    if (pr->q_start < 0 || pr->kv_start < 0 || pr->q_start > (int64_t(1) << 30) || pr->kv_start > (int64_t(1) << 30))
      return FA_ERR_PARAM_INVALID;
    if ((cq[1] - cq[0]) - (ck[1] - ck[0]) + pr->q_start - pr->kv_start != 0) return FA_ERR_PARAM_INVALID;
    pr->has_start = true;
  }
  if (cfg->pse) {
    int64_t max_q = 0, max_kv = 0;
    for (int64_t b = 0; b < pr->batch; ++b) {
      max_q = std::max<int64_t>(max_q, cq[b + 1] - cq[b]);
      max_kv = std::max<int64_t>(max_kv, ck[b + 1] - ck[b]);
    }
    if (cfg->pse_type != 0 && cfg->pse_type != 1) return FA_ERR_PARAM_INVALID;
    if (cfg->pse_batch != 1 && cfg->pse_batch != pr->batch) return FA_ERR_PARAM_INVALID;
    if (cfg->pse_cols < max_kv || cfg->pse_cols > kMaxTokens || cfg->pse_rows < 1) return FA_ERR_PARAM_INVALID;
    int pmode;
    if (cfg->pse_rows == 1) pmode = 1;
    else if (cfg->pse_rows >= max_q && cfg->pse_rows <= kMaxTokens) pmode = 0;
    else if (cfg->pse_rows == 1024) pmode = 2;
    else return FA_ERR_PARAM_INVALID;
    if (pmode == 2) {
      // the compressed form holds a lower-triangle bias of square sequences
      if (mode != FA_SPARSE_LEFT_UP_CAUSAL && mode != FA_SPARSE_RIGHT_DOWN_CAUSAL) return FA_ERR_PARAM_INVALID;
      for (int64_t b = 0; b < pr->batch; ++b)
        if (cq[b + 1] - cq[b] != ck[b + 1] - ck[b]) return FA_ERR_PARAM_INVALID;
    }
    pr->pse = cfg->pse;
    pr->pse_batch = cfg->pse_batch;
    pr->pse_rows = cfg->pse_rows;
    pr->pse_cols = cfg->pse_cols;
    pr->pse_type = cfg->pse_type;
    pr->pse_mode = pmode;
  }
  if (cfg->layout < FA_LAYOUT_TND || cfg->layout > FA_LAYOUT_SBH) return FA_ERR_PARAM_INVALID;
  for (int id = 0; id < 8; ++id) {   // packed TND strides unless given
    const int64_t n = (id == T_K || id == T_V || id == T_DK || id == T_DV) ? nkv : cfg->head_num;
    pr->ts[id] = n * dim_of(*pr, id);
    pr->hs[id] = dim_of(*pr, id);
  }
  if (cfg->strides) {
    if (cfg->layout != FA_LAYOUT_TND) return FA_ERR_PARAM_INVALID;
    const int64_t eb = cfg->dtype == FA_DTYPE_FP32 ? 4 : 2;
    for (int id = 0; id < 8; ++id) {
      const int64_t n = (id == T_K || id == T_V || id == T_DK || id == T_DV) ? nkv : cfg->head_num;
      const int64_t t = cfg->strides[2 * id], h = cfg->strides[2 * id + 1];
      const bool output = id >= T_DQ || id == T_O;   // O is the forward's output
      // 16-byte rows (the copies move 16-byte chunks); outputs need distinct rows
      if (t < 0 || h < 0 || (t * eb) % 16 != 0 || (h * eb) % 16 != 0) return FA_ERR_PARAM_INVALID;
      if (output && (t == 0 || (h == 0 && n > 1))) return FA_ERR_PARAM_INVALID;
      pr->ts[id] = t;
      pr->hs[id] = h;
      pr->strided[id] = !(t == n * dim_of(*pr, id) && h == dim_of(*pr, id));
    }
  }
  pr->layout = cfg->layout;
  if (pr->layout != FA_LAYOUT_TND) {
    // the fixed-length layouts hold B sequences of one length per side
    pr->sq = cq[1];
    pr->skv = ck[1];
    for (int64_t b = 0; b <= pr->batch; ++b)
      if (cq[b] != b * pr->sq || ck[b] != b * pr->skv) return FA_ERR_PARAM_INVALID;
  }
  if (pr->tq < 1 || pr->tkv < 1) return FA_ERR_PARAM_INVALID;
  const bool uses_mask = mode == FA_SPARSE_NONE || mode == FA_SPARSE_ALL_MASK || mode == FA_SPARSE_BAND;
  if (cfg->atten_mask && uses_mask) {
    int64_t max_q = 0, max_kv = 0;
    for (int64_t b = 0; b < pr->batch; ++b) {
      max_q = std::max<int64_t>(max_q, cq[b + 1] - cq[b]);
      max_kv = std::max<int64_t>(max_kv, ck[b + 1] - ck[b]);
    }
    if (cfg->mask_rows < max_q || cfg->mask_cols < max_kv || cfg->mask_rows > kMaxTokens ||
        cfg->mask_cols > kMaxTokens)
      return FA_ERR_PARAM_INVALID;
    pr->mask = cfg->atten_mask;
    pr->mask_rows = cfg->mask_rows;
    pr->mask_cols = cfg->mask_cols;
    pr->mask_words = (cfg->mask_cols + 31) / 32;
  }
  // the kernels have no instances of an external pse with an attenMask
  if (pr->pse && pr->mask) return FA_ERR_PARAM_INVALID;
  // head dims above 128, and a 16-bit external pse (the fused 16-bit kernels have no
  // instances of it), run the materialised-score path, whose backward is deterministic
  pr->large = pr->d > 128 || (pr->pse && pr->dtype != FA_DTYPE_FP32);
  if (pr->large) pr->deterministic = true;
  pr->drop_bits = bits;
  return FA_OK;
}

fa_status check_alibi(const Problem& pr) {
  // pseType 2 needs Sq == Skv per sequence, and no zero-length sequence carries a pse;
  // mode 7 takes no pse; in mode 8 the first sequence may be a chunk split off a longer
  // one, whose positions the start indices give (checked in parse)
  if (pr.mode == FA_SPARSE_RIGHT_DOWN_CAUSAL_BAND) return FA_ERR_PARAM_INVALID;
  for (int64_t b = 0; b < pr.batch; ++b) {
    const int32_t lq = pr.cu_q[b + 1] - pr.cu_q[b], lkv = pr.cu_kv[b + 1] - pr.cu_kv[b];
    if (lq == 0 || lkv == 0) return FA_ERR_PARAM_INVALID;
    if (lq != lkv && !(b == 0 && pr.has_start)) return FA_ERR_PARAM_INVALID;
  }
  return FA_OK;
}

FaWindow window_of(const Problem& pr, int64_t b) {
  const int32_t lq = pr.cu_q[b + 1] - pr.cu_q[b], lkv = pr.cu_kv[b + 1] - pr.cu_kv[b];
  return fa_make_window(fa_seq_mode(pr.mode, b, pr.batch), pr.pre, pr.next, lq, lkv, pr.prefix[b]);
}

// Work list of one pass.  The items of one sequence are consecutive, so the
// workgroups running at the same time on an XCD (the grid maps each kv head to
// one XCD) share that sequence's K/V (forward, dQ) or Q/dY (dK/dV) in L2;
// sequences come heaviest first and, inside a sequence, items heaviest first,
// so the dispatcher starts long work early and short work fills the tail.
std::vector<WorkItem> schedule(const Problem& pr, int pass, int* bm_out, int* bn_out) {
  std::vector<WorkItem> items;
  int bm, bn;
  if (pass == 0) { bm = fa::fwd_rows(pr.keep < 1.0, pr.dtype == FA_DTYPE_FP32); bn = fa::kFwdBN; }
  else if (pass == 1) { bm = fa::kKvBM; bn = fa::kKvBN; }
  else { bm = fa::kDqBM; bn = fa::kDqBN; }
  if (bm_out) *bm_out = bm;
  if (bn_out) *bn_out = bn;
  for (int64_t b = 0; b < pr.batch; ++b) {
    const int32_t lq = pr.cu_q[b + 1] - pr.cu_q[b], lkv = pr.cu_kv[b + 1] - pr.cu_kv[b];
    const FaWindow w = window_of(pr, b);
    if (pass == 1) {
      const int32_t nt = (lkv + bn - 1) / bn;
      for (int32_t t = 0; t < nt; ++t) {
        int32_t lo, hi;
        fa_q_tile_range(w, t * bn, std::min(t * bn + bn, lkv), lq, bm, &lo, &hi);
        items.push_back({(int32_t)b, t, lo, hi});
      }
    } else {
      const int32_t nt = (lq + bm - 1) / bm;
      for (int32_t t = 0; t < nt; ++t) {
        int32_t lo, hi;
        fa_kv_tile_range(w, t * bm, std::min(t * bm + bm, lq), lkv, bn, &lo, &hi);
        items.push_back({(int32_t)b, t, lo, hi});
      }
    }
  }
  std::vector<int64_t> seq_work(pr.batch, 0);
  for (const WorkItem& x : items) seq_work[x.b] += x.hi - x.lo;
  std::stable_sort(items.begin(), items.end(), [&](const WorkItem& x, const WorkItem& y) {
    if (x.b != y.b) return seq_work[x.b] != seq_work[y.b] ? seq_work[x.b] > seq_work[y.b] : x.b < y.b;
    return (x.hi - x.lo) > (y.hi - y.lo);
  });
  return items;
}

// ---- workspace layout ----
constexpr uint64_t kAlign = 256;
uint64_t align_up(uint64_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
  uint64_t cu_q = 0, cu_kv = 0, bit_base = 0, prefix = 0, items0 = 0, items1 = 0;   // host-staged block
  uint64_t staged_bytes = 0;
  uint64_t delta = 0, lse = 0, dsink_part = 0, dq_acc = 0, mbits = 0;
  // TND copies of the BNSD / SBH tensors
  uint64_t rq = 0, rk = 0, rv = 0, rdy = 0, ro = 0, rdq = 0, rdk = 0, rdv = 0;
  uint64_t total = 0;
  int64_t n_items0 = 0, n_items1 = 0;
  int n_pre_blocks = 0;
  fa::LargePlan large{};          // the materialised-score path
};

// The materialised-score path: chunks of query rows sized so that the scores of one chunk
// (fp32 S, and dP in the backward; P~, and dS, in the input type; every query head)
// take at most about kLargeScoreBytes of the workspace, plus the fp32 dK / dV
// accumulators of every kv head.
constexpr uint64_t kLargeScoreBytes = 4ull << 30;
constexpr int64_t kLargeMinRows = 256;   // fewer rows per chunk make the contractions over rows too short
void large_layout(const Problem& pr, bool bwd, uint64_t* off, fa::LargePlan* P) {
  int64_t mq = 1, mkv = 1;
  for (int64_t b = 0; b < pr.batch; ++b) {
    mq = std::max<int64_t>(mq, pr.cu_q[b + 1] - pr.cu_q[b]);
    mkv = std::max<int64_t>(mkv, pr.cu_kv[b + 1] - pr.cu_kv[b]);
  }
  const int64_t eb = pr.dtype == FA_DTYPE_FP32 ? 4 : 2;
  const int64_t ld = (mkv + 7) / 8 * 8;   // 16-byte rows in both element sizes
  const uint64_t per_row = (uint64_t)(pr.nq * ld * (bwd ? 8 + 2 * eb : 4 + eb));
  int64_t rows = (int64_t)(kLargeScoreBytes / per_row) / 64 * 64;
  rows = std::min<int64_t>(std::max<int64_t>(rows, kLargeMinRows), (mq + 63) / 64 * 64);
  const uint64_t sc = (uint64_t)(pr.nq * rows * ld);
  P->batch = (int32_t)pr.batch;
  P->d = (int32_t)pr.d;
  P->rows = (int32_t)rows;
  P->ld = (int32_t)ld;
  P->acc_rows = (int32_t)mkv;
  P->off_s = *off; *off = align_up(*off + 4 * sc);
  P->off_p = *off; *off = align_up(*off + (uint64_t)eb * sc);
  if (bwd) {
    const uint64_t acc = 4 * (uint64_t)(pr.nkv * mkv * pr.d);
    P->off_dp = *off; *off = align_up(*off + 4 * sc);
    P->off_ds = *off; *off = align_up(*off + (uint64_t)eb * sc);
    P->off_dk = *off; *off = align_up(*off + acc);
    P->off_dv = *off; *off = align_up(*off + acc);
  }
}

Layout layout_fwd(const Problem& pr, int64_t n_items) {
  Layout L;
  uint64_t off = 0;
  L.cu_q = off; off = align_up(off + 4 * (pr.batch + 1));
  L.cu_kv = off; off = align_up(off + 4 * (pr.batch + 1));
  L.bit_base = off; off = align_up(off + 8 * pr.batch);
  L.prefix = off; off = align_up(off + 4 * pr.batch);
  L.items0 = off; off = align_up(off + sizeof(WorkItem) * n_items);
  L.staged_bytes = off;
  L.n_items0 = n_items;
  if (pr.mask) {
    L.mbits = off;
    off = align_up(off + 4 * (uint64_t)pr.mask_rows * pr.mask_words);
  }
  if (pr.large) large_layout(pr, false, &off, &L.large);
  if (relayout(pr)) {
    const uint64_t qb = (uint64_t)(pr.tq * pr.nq * pr.d * elem_bytes(pr));
    const uint64_t kb = (uint64_t)(pr.tkv * pr.nkv * pr.d * elem_bytes(pr));
    L.rq = off; off = align_up(off + qb);
    L.rk = off; off = align_up(off + kb);
    L.rv = off; off = align_up(off + kb);
    L.ro = off; off = align_up(off + qb);
  }
  L.total = std::max<uint64_t>(off, kAlign);
  return L;
}

// sum_b ceil(L_b / tile) <= T / tile + B
int64_t upper_items(const Problem& pr, int tile) { return pr.batch + (std::max(pr.tq, pr.tkv) + tile - 1) / tile; }

Layout layout_bwd(const Problem& pr, int64_t n_kv_items, int64_t n_dq_items) {
  Layout L;
  uint64_t off = 0;
  L.cu_q = off; off = align_up(off + 4 * (pr.batch + 1));
  L.cu_kv = off; off = align_up(off + 4 * (pr.batch + 1));
  L.bit_base = off; off = align_up(off + 8 * pr.batch);
  L.prefix = off; off = align_up(off + 4 * pr.batch);
  L.items0 = off; off = align_up(off + sizeof(WorkItem) * n_kv_items);
  L.items1 = off; off = align_up(off + sizeof(WorkItem) * n_dq_items);
  L.staged_bytes = off;
  L.n_items0 = n_kv_items;
  L.n_items1 = n_dq_items;
  L.delta = off; off = align_up(off + 4 * (uint64_t)pr.tq * pr.nq);
  L.lse = off; off = align_up(off + 4 * (uint64_t)pr.tq * pr.nq);
  L.n_pre_blocks = (int)((pr.tq + fa::kPreRowsPerBlock - 1) / fa::kPreRowsPerBlock);
  L.dsink_part = off; off = align_up(off + 4 * (uint64_t)L.n_pre_blocks * pr.nq);
  if (!pr.deterministic) {
    L.dq_acc = off;
    off = align_up(off + 4 * (uint64_t)pr.tq * pr.nq * pr.d);
  }
  if (pr.mask) {
    L.mbits = off;
    off = align_up(off + 4 * (uint64_t)pr.mask_rows * pr.mask_words);
  }
  if (pr.large) large_layout(pr, true, &off, &L.large);
  if (relayout(pr)) {
    const uint64_t qb = (uint64_t)(pr.tq * pr.nq * pr.d * elem_bytes(pr));
    const uint64_t kb = (uint64_t)(pr.tkv * pr.nkv * pr.d * elem_bytes(pr));
    L.rq = off; off = align_up(off + qb);
    L.rk = off; off = align_up(off + kb);
    L.rv = off; off = align_up(off + kb);
    L.rdy = off; off = align_up(off + qb);
    L.ro = off; off = align_up(off + qb);
    L.rdq = off; off = align_up(off + qb);
    L.rdk = off; off = align_up(off + kb);
    L.rdv = off; off = align_up(off + kb);
  }
  L.total = off;
  return L;
}

// Sizes are computed from upper bounds on the item counts so that the size
// query does not depend on anything but the configuration.
Layout fwd_layout_bound(const Problem& pr) { return layout_fwd(pr, upper_items(pr, fa::fwd_rows(pr.keep < 1.0, pr.dtype == FA_DTYPE_FP32))); }
Layout bwd_layout_bound(const Problem& pr) {
  return layout_bwd(pr, upper_items(pr, fa::kKvBN), upper_items(pr, fa::kDqBM));
}

// ---- kernel timing (measurement hook) ----
enum KernelId { K_FWD = 0, K_PRE, K_KV, K_DQ, K_CONVERT, K_DSINK, K_ZERO, K_MASK, K_DEC, K_DEC_REDUCE, K_RELAYOUT,
                K_COUNT };
const char* kKernelNames[K_COUNT] = {"fa_fwd",         "fa_bwd_preprocess", "fa_bwd_dkdv",  "fa_bwd_dq",
                                     "fa_bwd_dq_convert", "fa_bwd_dsink_reduce", "fa_zero_f32", "fa_mask_pack",
                                     "fa_decode",      "fa_decode_reduce",    "fa_relayout"};
struct ProfState {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[K_COUNT];
  double total_ms[K_COUNT] = {};
  int64_t launches[K_COUNT] = {};
};
ProfState& prof() {
  static ProfState s;
  return s;
}

template <typename F>
hipError_t timed(KernelId id, hipStream_t s, F&& launch) {
  ProfState& P = prof();
  bool on;
  {
    std::lock_guard<std::mutex> g(P.mu);
    on = P.on;
  }
  if (!on) return launch();
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess) return hipErrorUnknown;
  if (hipEventCreate(&b) != hipSuccess) return hipErrorUnknown;
  hipError_t e = hipEventRecord(a, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  std::lock_guard<std::mutex> g(P.mu);
  P.ev[id].push_back({a, b});
  return e;
}

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// FA_LOG=1 in the environment prints one line per call describing the plan (stderr).
bool log_on() {
  static const bool on = [] {
    const char* v = std::getenv("FA_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

void log_plan(const char* what, const Problem& pr, int64_t n0, int64_t n1) {
  if (!log_on()) return;
  std::fprintf(stderr,
               "[fa] %s: B=%lld Tq=%lld Tkv=%lld Nq=%lld Nkv=%lld D=%lld (kernel D=%lld) dtype=%d mode=%d "
               "keep=%.3f layout=%d det=%d items=%lld/%lld\n",
               what, (long long)pr.batch, (long long)pr.tq, (long long)pr.tkv, (long long)pr.nq, (long long)pr.nkv,
               (long long)pr.du, (long long)pr.d, pr.dtype, pr.mode, pr.keep, pr.layout, pr.deterministic ? 1 : 0,
               (long long)n0, (long long)n1);
}

template <typename P>
void fill_pse(const Problem& pr, P& p) {
  p.pse = pr.pse;
  if (!pr.pse) return;
  p.pse_hstride = pr.pse_rows * pr.pse_cols;
  p.pse_bstride = pr.pse_batch == 1 ? 0 : pr.nq * p.pse_hstride;
  p.pse_cols = (int32_t)pr.pse_cols;
  p.pse_mode = pr.pse_mode;
  p.pse_coef = (float)((pr.pse_type == 1 ? pr.scale : 1.0) * 1.4426950408889634);
}

// One BNSD / SBH tensor of the query side (q = true: B sequences of Sq rows, Nq
// heads) or the key side, or one strided TND tensor (id), to or from its packed
// TND copy.
hipError_t relayout_tensor(const Problem& pr, int id, const void* src, void* dst, bool to_tnd, hipStream_t s) {
  const bool q_side = !(id == T_K || id == T_V || id == T_DK || id == T_DV);
  return timed(K_RELAYOUT, s, [&] {
    if (!layout_copies(pr))
      return fa::launch_relayout(src, dst, 1, q_side ? pr.tq : pr.tkv, q_side ? pr.nq : pr.nkv, dim_of(pr, id), pr.d,
                                 (int)elem_bytes(pr), fa::kLayoutStrided, to_tnd, s, pr.ts[id], pr.hs[id]);
    return fa::launch_relayout(src, dst, pr.batch, q_side ? pr.sq : pr.skv, q_side ? pr.nq : pr.nkv, dim_of(pr, id),
                               pr.d,
                               (int)elem_bytes(pr), pr.layout, to_tnd, s);
  });
}

// Gathers the tensor into its workspace copy when it has one; returns the pointer the kernels read.
const void* gather(const Problem& pr, int id, const void* src, char* copy, hipStream_t s, hipError_t* e) {
  if (!copied(pr, id) || *e != hipSuccess) return copied(pr, id) ? copy : src;
  *e = relayout_tensor(pr, id, src, copy, true, s);
  return copy;
}

void fill_common_fwd(const Problem& pr, fa::FwdParams& p) {
  p.nq = (int32_t)pr.nq;
  p.nkv = (int32_t)pr.nkv;
  p.group = (int32_t)(pr.nq / pr.nkv);
  p.mode = pr.mode;
  p.pre = (int32_t)fa_clamp_window(pr.pre);
  p.next = (int32_t)fa_clamp_window(pr.next);
  p.scale_log2 = (float)(pr.scale * 1.4426950408889634);
  p.inv_keep = (float)(1.0 / pr.keep);
  p.use_dropout = pr.keep < 1.0 ? 1 : 0;
  p.head_swizzle = (pr.nq % 8 == 0) ? 1 : 0;
  p.nseq = (int32_t)pr.batch;
  p.pse_off0 = (int32_t)(pr.q_start - pr.kv_start);
}

std::vector<char> stage_block(const Problem& pr, const Layout& L, const std::vector<WorkItem>& i0,
                              const std::vector<WorkItem>* i1) {
  std::vector<char> host(L.staged_bytes, 0);
  std::memcpy(host.data() + L.cu_q, pr.cu_q.data(), 4 * pr.cu_q.size());
  std::memcpy(host.data() + L.cu_kv, pr.cu_kv.data(), 4 * pr.cu_kv.size());
  std::memcpy(host.data() + L.bit_base, pr.bit_base.data(), 8 * pr.bit_base.size());
  std::memcpy(host.data() + L.prefix, pr.prefix.data(), 4 * pr.prefix.size());
  std::memcpy(host.data() + L.items0, i0.data(), sizeof(WorkItem) * i0.size());
  if (i1) std::memcpy(host.data() + L.items1, i1->data(), sizeof(WorkItem) * i1->size());
  return host;
}

// ---- decode attention (aclnnIncreFlashAttentionV2) ----
constexpr int64_t kMaxDecBatch = 65536;            // B limit of the decode page ("B <= 65536")
constexpr int64_t kMaxDecSeq = 1 << 24;            // padded cache length limit (keys index in int32)
constexpr int64_t kMaxDecGroup = 64;               // numHeads / numKeyValueHeads <= 64
constexpr int64_t kDecMinChunk = 32 * fa::kDecWaves * 8;      // keys per work item: whole 32-key steps for
                                                               //   every wave, at least 256 per wave
constexpr int64_t kDecSlots = 256;                             // work items the chip runs at once (one per CU)

struct DecProblem {
  int64_t batch = 0, s = 0, nq = 0, nkv = 0, d = 0;
  int dtype = 0, layout = 0;
  double scale = 0;
  const uint8_t* mask = nullptr;
  std::vector<int32_t> lens;   // actual key length of each sequence
};

fa_status parse_decode(const fa_decode_config* cfg, DecProblem* pr) {
  if (!cfg) return FA_ERR_PARAM_NULLPTR;
  if (cfg->batch < 1 || cfg->batch > kMaxDecBatch) return FA_ERR_PARAM_INVALID;
  if (cfg->max_seq_len < 1 || cfg->max_seq_len > kMaxDecSeq) return FA_ERR_PARAM_INVALID;
  if (cfg->num_heads < 1 || cfg->num_heads > kMaxHeads) return FA_ERR_PARAM_INVALID;
  const int64_t nkv = cfg->num_kv_heads == 0 ? cfg->num_heads : cfg->num_kv_heads;
  if (nkv < 1 || cfg->num_heads % nkv != 0 || cfg->num_heads / nkv > kMaxDecGroup) return FA_ERR_PARAM_INVALID;
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return FA_ERR_PARAM_INVALID;
  if (cfg->dtype != FA_DTYPE_BF16 && cfg->dtype != FA_DTYPE_FP16) return FA_ERR_PARAM_INVALID;
  if (cfg->layout != FA_LAYOUT_BSH && cfg->layout != FA_LAYOUT_BSND && cfg->layout != FA_LAYOUT_BNSD)
    return FA_ERR_PARAM_INVALID;
  if (!std::isfinite(cfg->scale) || cfg->flags != 0) return FA_ERR_PARAM_INVALID;
  pr->batch = cfg->batch;
  pr->s = cfg->max_seq_len;
  pr->nq = cfg->num_heads;
  pr->nkv = nkv;
  pr->d = cfg->head_dim;
  pr->dtype = cfg->dtype;
  pr->layout = cfg->layout;
  pr->scale = cfg->scale;
  pr->mask = cfg->atten_mask;
  pr->lens.assign((size_t)cfg->batch, (int32_t)cfg->max_seq_len);
  if (cfg->actual_seq_lengths) {
    for (int64_t b = 0; b < cfg->batch; ++b) {
      const int64_t L = cfg->actual_seq_lengths[b];
      if (L < 0 || L > cfg->max_seq_len) return FA_ERR_PARAM_INVALID;
      pr->lens[(size_t)b] = (int32_t)L;
    }
  }
  return FA_OK;
}

// Work split: every (sequence, kv head) gets ceil(L_b / chunk) items (at least one,
// so empty sequences still write zeros).  An item costs a pipeline fill of a few
// microseconds on top of its keys, and one item's block takes a CU's LDS, so fewer,
// longer items win while the chip stays busy: the chunk doubles from 768 keys until
// the items number at most one per CU or two per (sequence, kv head), whichever is
// more.  Items stay in (sequence, kv head, chunk) order: neighbouring blocks then
// read neighbouring cache rows.
struct DecPlan {
  int64_t chunk = kDecMinChunk;
  std::vector<fa::DecItem> items;
  std::vector<int32_t> first_slot, n_split;
  int64_t n_slots = 0;
  size_t off_items = 0, off_first = 0, off_nsplit = 0, staged = 0;
  size_t off_o = 0, off_m = 0, off_l = 0, total = 0;
};

DecPlan plan_decode(const DecProblem& pr) {
  DecPlan P;
  int64_t longest = 1;
  for (int32_t L : pr.lens) longest = std::max<int64_t>(longest, L);
  const int64_t limit = std::max<int64_t>(kDecSlots, 2 * pr.batch * pr.nkv);
  auto n_items = [&](int64_t chunk) {
    int64_t n = 0;
    for (int32_t L : pr.lens) n += std::max<int64_t>(1, (L + chunk - 1) / chunk);
    return n * pr.nkv;
  };
  while (P.chunk < longest && n_items(P.chunk) > limit) P.chunk *= 2;
  P.first_slot.assign((size_t)(pr.batch * pr.nkv), -1);
  P.n_split.assign((size_t)pr.batch, 1);
  for (int64_t b = 0; b < pr.batch; ++b) {
    const int64_t L = pr.lens[(size_t)b];
    const int64_t n = std::max<int64_t>(1, (L + P.chunk - 1) / P.chunk);
    P.n_split[(size_t)b] = (int32_t)n;
    // the slots of one (b, g) are consecutive, and so are its items
    const int64_t base = P.n_slots;
    if (n > 1) {
      for (int64_t g = 0; g < pr.nkv; ++g) P.first_slot[(size_t)(b * pr.nkv + g)] = (int32_t)(base + g * n);
      P.n_slots += pr.nkv * n;
    }
    for (int64_t g = 0; g < pr.nkv; ++g)
      for (int64_t c = 0; c < n; ++c) {
        fa::DecItem it;
        it.b = (int32_t)b;
        it.g = (int32_t)g;
        it.lo = (int32_t)(c * P.chunk);
        it.hi = (int32_t)std::min(L, (c + 1) * P.chunk);
        it.slot = n > 1 ? (int32_t)(base + g * n + c) : -1;
        P.items.push_back(it);
      }
  }
  const int64_t group = pr.nq / pr.nkv;
  size_t off = 0;
  P.off_items = off; off = align_up(off + sizeof(fa::DecItem) * P.items.size());
  P.off_first = off; off = align_up(off + 4 * P.first_slot.size());
  P.off_nsplit = off; off = align_up(off + 4 * P.n_split.size());
  P.staged = off;
  P.off_o = off; off = align_up(off + 4 * (size_t)(P.n_slots * group * pr.d));
  P.off_m = off; off = align_up(off + 4 * (size_t)(P.n_slots * group));
  P.off_l = off; off = align_up(off + 4 * (size_t)(P.n_slots * group));
  P.total = std::max<size_t>(off, 256);
  return P;
}

// Copies the host-built plan (work lists, sequence tables) to the workspace.  Outside
// stream capture: one hipMemcpyAsync from pageable memory, which takes the bytes
// before it returns, so the host buffer may go right after.  A captured copy would
// instead keep the host address and read it at every replay, after the buffer is
// gone; under capture the bytes therefore travel as kernel arguments, which the graph
// stores by value (fa::launch_stage).
hipError_t stage_plan(char* ws, const std::vector<char>& host, hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return e;
  if (cs == hipStreamCaptureStatusNone) return hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, s);
  return fa::launch_stage(ws, host.data(), host.size(), s);
}

#if defined(FA_TRACE_VISITS)
// Trace build: device buffers of visit counters for pass 0 (forward), 1 (dK/dV) and
// 2 (dQ), set by fa_debug_trace; null = not traced.
std::mutex g_trace_mu;
uint32_t* g_trace[3] = {};
int64_t g_trace_words[3] = {};
#endif

// Tile grid of a pass's visit counters: rows per block and keys per tile, and the
// block / tile counts of the longest sequences.
void trace_dims(const Problem& pr, int rows, int keys, int32_t* rb, int32_t* kt) {
  int64_t mq = 0, mkv = 0;
  for (int64_t b = 0; b < pr.batch; ++b) {
    mq = std::max<int64_t>(mq, pr.cu_q[b + 1] - pr.cu_q[b]);
    mkv = std::max<int64_t>(mkv, pr.cu_kv[b + 1] - pr.cu_kv[b]);
  }
  *rb = (int32_t)((mq + rows - 1) / rows);
  *kt = (int32_t)((mkv + keys - 1) / keys);
}

// Points the pass's counters at the trace buffer (trace build); false when the buffer
// is set but too small for this problem.
template <typename T>
bool attach_trace(const Problem& pr, int pass, int rows, int keys, T** ptr, int32_t* rb, int32_t* kt) {
  trace_dims(pr, rows, keys, rb, kt);
#if defined(FA_TRACE_VISITS)
  std::lock_guard<std::mutex> g(g_trace_mu);
  if (g_trace[pass]) {
    if (pr.batch * pr.nq * (int64_t)*rb * *kt > g_trace_words[pass]) return false;
    *ptr = g_trace[pass];
  }
#else
  (void)pass;
  *ptr = nullptr;
#endif
  return true;
}

// Address of the current device's copy of fa_noalloc_scratch, looked up once per
// device with that device current (the first fa_decode_noalloc call on it).
hipError_t noalloc_scratch(char** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static char* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(fa_noalloc_scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<char*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_PARAM_NULLPTR: return "FA_ERR_PARAM_NULLPTR: a required pointer argument is NULL";
    case FA_ERR_PARAM_INVALID: return "FA_ERR_PARAM_INVALID: unsupported attribute, shape, dtype or alignment";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace smaller than the size query returned";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the call needs more scratch than the allocation-free entry point's static buffer holds";
    default: return "unknown fa_status";
  }
}

fa_status fa_fwd_workspace_size(const fa_config* cfg, uint64_t* bytes) {
  if (!bytes) return FA_ERR_PARAM_NULLPTR;
  Problem pr;
  fa_status st = parse(cfg, &pr);
  if (st != FA_OK) return st;
  *bytes = fwd_layout_bound(pr).total;
  return FA_OK;
}

fa_status fa_bwd_workspace_size(const fa_config* cfg, uint64_t* bytes) {
  if (!bytes) return FA_ERR_PARAM_NULLPTR;
  Problem pr;
  fa_status st = parse(cfg, &pr);
  if (st != FA_OK) return st;
  *bytes = bwd_layout_bound(pr).total;
  return FA_OK;
}

fa_status fa_fwd(const fa_config* cfg, const void* q, const void* k, const void* v, const uint8_t* drop_mask,
                 const float* alibi_slopes, const float* sink, void* out, float* softmax_max, float* softmax_sum,
                 void* workspace, uint64_t workspace_bytes, void* stream) {
  Problem pr;
  fa_status st = parse(cfg, &pr);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !out || !softmax_max || !softmax_sum) return FA_ERR_PARAM_NULLPTR;
  if (pr.keep < 1.0 && !drop_mask) return FA_ERR_PARAM_NULLPTR;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(softmax_max, 4) ||
      !aligned(softmax_sum, 4) || (drop_mask && !aligned(drop_mask, 4)) || (alibi_slopes && !aligned(alibi_slopes, 4)) ||
      (sink && !aligned(sink, 4)))
    return FA_ERR_PARAM_INVALID;
  if (alibi_slopes && (st = check_alibi(pr)) != FA_OK) return st;
  if (alibi_slopes && pr.pse) return FA_ERR_PARAM_INVALID;
  if (pr.pse && !aligned(pr.pse, 4)) return FA_ERR_PARAM_INVALID;
  const Layout bound = fwd_layout_bound(pr);
  if (!workspace) return FA_ERR_PARAM_NULLPTR;
  if (!aligned(workspace, 16)) return FA_ERR_PARAM_INVALID;
  if (workspace_bytes < bound.total) return FA_ERR_WORKSPACE;

  std::vector<WorkItem> items = schedule(pr, 0, nullptr, nullptr);
  log_plan("fa_fwd", pr, (int64_t)items.size(), 0);
  const Layout L = layout_fwd(pr, (int64_t)items.size());
  std::vector<char> host = stage_block(pr, L, items, nullptr);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  hipError_t e = stage_plan(ws, host, s);
  if (e != hipSuccess) return FA_ERR_HIP;

  fa::FwdParams p{};
  fill_common_fwd(pr, p);
  p.q = q; p.k = k; p.v = v; p.o = out;
  if (relayout(pr)) {
    p.q = gather(pr, T_Q, q, ws + L.rq, s, &e);
    p.k = gather(pr, T_K, k, ws + L.rk, s, &e);
    p.v = gather(pr, T_V, v, ws + L.rv, s, &e);
    if (e != hipSuccess) return FA_ERR_HIP;
    if (copied(pr, T_O)) p.o = ws + L.ro;
  }
  p.m_out = softmax_max; p.l_out = softmax_sum;
  p.drop = pr.keep < 1.0 ? drop_mask : nullptr;
  p.drop_bytes = (pr.drop_bits + 7) / 8;
  p.slopes = alibi_slopes; p.sink = sink;
  p.slope_bstride = pr.slopes_per_batch ? (int32_t)pr.nq : 0;
  p.pse_sqrt = pr.pse_sqrt ? 1 : 0;
  fill_pse(pr, p);
  p.cu_q = reinterpret_cast<const int32_t*>(ws + L.cu_q);
  p.cu_kv = reinterpret_cast<const int32_t*>(ws + L.cu_kv);
  p.bit_base = reinterpret_cast<const int64_t*>(ws + L.bit_base);
  p.prefix = reinterpret_cast<const int32_t*>(ws + L.prefix);
  p.items = reinterpret_cast<const WorkItem*>(ws + L.items0);
  p.n_items = (int32_t)items.size();
  p.mbits = pr.mask ? reinterpret_cast<const uint32_t*>(ws + L.mbits) : nullptr;
  p.mwords = (int32_t)pr.mask_words;
  if (pr.mask) {
    e = timed(K_MASK, s, [&] {
      return fa::launch_mask_pack(pr.mask, pr.mask_rows, pr.mask_cols, reinterpret_cast<uint32_t*>(ws + L.mbits), s);
    });
    if (e != hipSuccess) return FA_ERR_HIP;
  }
  if (!attach_trace(pr, 0, 32, fa::kFwdBN, &p.trace, &p.trace_rb, &p.trace_kt)) return FA_ERR_PARAM_INVALID;
  if (pr.large) {
    fa::LargePlan lp = L.large;
    lp.cu_q = pr.cu_q.data();
    lp.cu_kv = pr.cu_kv.data();
    lp.prefix = pr.prefix.data();
    e = timed(K_FWD, s, [&] { return fa::launch_large_fwd(pr.dtype, p, lp, ws, s); });
  } else {
    e = timed(K_FWD, s, [&] { return fa::launch_fwd(pr.dtype, (int)pr.d, p, s); });
  }
  if (e == hipSuccess && copied(pr, T_O)) e = relayout_tensor(pr, T_O, ws + L.ro, out, false, s);
  return hip_status(e);
}

fa_status fa_bwd(const fa_config* cfg, const void* q, const void* k, const void* v, const void* dy, const void* out,
                 const float* softmax_max, const float* softmax_sum, const uint8_t* drop_mask,
                 const float* alibi_slopes, const float* sink, void* dq, void* dk, void* dv, float* dsink,
                 void* workspace, uint64_t workspace_bytes, void* stream) {
  Problem pr;
  fa_status st = parse(cfg, &pr);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !dy || !out || !softmax_max || !softmax_sum || !dq || !dk || !dv)
    return FA_ERR_PARAM_NULLPTR;
  if (pr.keep < 1.0 && !drop_mask) return FA_ERR_PARAM_NULLPTR;
  if (sink && !dsink) return FA_ERR_PARAM_NULLPTR;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dy, 16) || !aligned(out, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(softmax_max, 4) ||
      !aligned(softmax_sum, 4) || (drop_mask && !aligned(drop_mask, 4)) ||
      (alibi_slopes && !aligned(alibi_slopes, 4)) || (sink && !aligned(sink, 4)) || (dsink && !aligned(dsink, 4)))
    return FA_ERR_PARAM_INVALID;
  if (alibi_slopes && (st = check_alibi(pr)) != FA_OK) return st;
  if (alibi_slopes && pr.pse) return FA_ERR_PARAM_INVALID;
  if (pr.pse && !aligned(pr.pse, 4)) return FA_ERR_PARAM_INVALID;
  const Layout bound = bwd_layout_bound(pr);
  if (!workspace) return FA_ERR_PARAM_NULLPTR;
  if (!aligned(workspace, 16)) return FA_ERR_PARAM_INVALID;
  if (workspace_bytes < bound.total) return FA_ERR_WORKSPACE;

  // the atomic dK/dV kernel for 16-bit D = 128 has no pse variant (its registers
  // do not fit one): run the deterministic passes, which need less workspace
  if ((alibi_slopes || pr.pse) && pr.dtype != FA_DTYPE_FP32 && pr.d == 128) pr.deterministic = true;
  // the attenMask is read by the deterministic passes only (the atomic kernels have no mask instances)
  if (pr.mask) pr.deterministic = true;
  std::vector<WorkItem> kv_items = schedule(pr, 1, nullptr, nullptr);
  std::vector<WorkItem> dq_items = schedule(pr, 2, nullptr, nullptr);
  log_plan("fa_bwd", pr, (int64_t)kv_items.size(), (int64_t)dq_items.size());
  const Layout L = layout_bwd(pr, (int64_t)kv_items.size(), (int64_t)dq_items.size());
  std::vector<char> host = stage_block(pr, L, kv_items, &dq_items);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  hipError_t e = stage_plan(ws, host, s);
  if (e != hipSuccess) return FA_ERR_HIP;

  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.dy = dy; p.o = out;
  p.m_in = softmax_max; p.l_in = softmax_sum;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dsink = sink ? dsink : nullptr;
  if (relayout(pr)) {
    p.q = gather(pr, T_Q, q, ws + L.rq, s, &e);
    p.k = gather(pr, T_K, k, ws + L.rk, s, &e);
    p.v = gather(pr, T_V, v, ws + L.rv, s, &e);
    p.dy = gather(pr, T_DY, dy, ws + L.rdy, s, &e);
    p.o = gather(pr, T_O, out, ws + L.ro, s, &e);
    if (e != hipSuccess) return FA_ERR_HIP;
    if (copied(pr, T_DQ)) p.dq = ws + L.rdq;
    if (copied(pr, T_DK)) p.dk = ws + L.rdk;
    if (copied(pr, T_DV)) p.dv = ws + L.rdv;
  }
  p.delta = reinterpret_cast<float*>(ws + L.delta);
  p.lse = reinterpret_cast<float*>(ws + L.lse);
  p.dsink_part = reinterpret_cast<float*>(ws + L.dsink_part);
  p.dq_acc = pr.deterministic ? nullptr : reinterpret_cast<float*>(ws + L.dq_acc);
  p.drop = pr.keep < 1.0 ? drop_mask : nullptr;
  p.drop_bytes = (pr.drop_bits + 7) / 8;
  p.slopes = alibi_slopes; p.sink = sink;
  p.slope_bstride = pr.slopes_per_batch ? (int32_t)pr.nq : 0;
  p.pse_sqrt = pr.pse_sqrt ? 1 : 0;
  fill_pse(pr, p);
  p.cu_q = reinterpret_cast<const int32_t*>(ws + L.cu_q);
  p.cu_kv = reinterpret_cast<const int32_t*>(ws + L.cu_kv);
  p.bit_base = reinterpret_cast<const int64_t*>(ws + L.bit_base);
  p.prefix = reinterpret_cast<const int32_t*>(ws + L.prefix);
  p.kv_items = reinterpret_cast<const WorkItem*>(ws + L.items0);
  p.dq_items = reinterpret_cast<const WorkItem*>(ws + L.items1);
  p.n_kv_items = (int32_t)kv_items.size();
  p.n_dq_items = (int32_t)dq_items.size();
  p.total_q = (int32_t)pr.tq;
  p.nq = (int32_t)pr.nq;
  p.nkv = (int32_t)pr.nkv;
  p.group = (int32_t)(pr.nq / pr.nkv);
  p.mode = pr.mode;
  p.pre = (int32_t)fa_clamp_window(pr.pre);
  p.next = (int32_t)fa_clamp_window(pr.next);
  p.scale = (float)pr.scale;
  p.scale_log2 = (float)(pr.scale * 1.4426950408889634);
  p.inv_keep = (float)(1.0 / pr.keep);
  p.use_dropout = pr.keep < 1.0 ? 1 : 0;
  p.head_swizzle = (pr.nq % 8 == 0) ? 1 : 0;
  p.nseq = (int32_t)pr.batch;
  p.pse_off0 = (int32_t)(pr.q_start - pr.kv_start);
  p.n_pre_blocks = L.n_pre_blocks;
  p.mbits = pr.mask ? reinterpret_cast<const uint32_t*>(ws + L.mbits) : nullptr;
  p.mwords = (int32_t)pr.mask_words;
  const int dt = pr.dtype, d = (int)pr.d;
  if (!attach_trace(pr, 1, fa::kKvBM, fa::kKvBN, &p.trace_kv, &p.trace_kv_rb, &p.trace_kv_kt) ||
      !attach_trace(pr, 2, 32, fa::kDqBN, &p.trace_dq, &p.trace_dq_rb, &p.trace_dq_kt))
    return FA_ERR_PARAM_INVALID;

  e = hipSuccess;
  if (pr.mask)
    e = timed(K_MASK, s, [&] {
      return fa::launch_mask_pack(pr.mask, pr.mask_rows, pr.mask_cols, reinterpret_cast<uint32_t*>(ws + L.mbits), s);
    });
  if (pr.large) {
    // the materialised-score path: preprocess, dK / dV and dQ
    fa::LargePlan lp = L.large;
    lp.cu_q = pr.cu_q.data();
    lp.cu_kv = pr.cu_kv.data();
    lp.prefix = pr.prefix.data();
    if (e == hipSuccess) e = timed(K_KV, s, [&] { return fa::launch_large_bwd(dt, p, lp, ws, s); });
  } else {
    if (e == hipSuccess) e = timed(K_PRE, s, [&] { return fa::launch_bwd_pre(dt, d, p, s); });
    if (e == hipSuccess && !pr.deterministic)
      e = timed(K_ZERO, s, [&] { return fa::launch_zero_f32(p.dq_acc, pr.tq * pr.nq * pr.d, s); });
    if (e == hipSuccess) e = timed(K_KV, s, [&] { return fa::launch_bwd_kv(dt, d, !pr.deterministic, p, s); });
    if (e == hipSuccess) {
      if (pr.deterministic)
        e = timed(K_DQ, s, [&] { return fa::launch_bwd_dq(dt, d, p, s); });
      else
        e = timed(K_CONVERT, s, [&] { return fa::launch_bwd_dq_convert(dt, d, p, s); });
    }
  }
  if (e == hipSuccess && sink) e = timed(K_DSINK, s, [&] { return fa::launch_bwd_dsink(p, s); });
  if (e == hipSuccess && copied(pr, T_DQ)) e = relayout_tensor(pr, T_DQ, ws + L.rdq, dq, false, s);
  if (e == hipSuccess && copied(pr, T_DK)) e = relayout_tensor(pr, T_DK, ws + L.rdk, dk, false, s);
  if (e == hipSuccess && copied(pr, T_DV)) e = relayout_tensor(pr, T_DV, ws + L.rdv, dv, false, s);
  return hip_status(e);
}

fa_status fa_debug_schedule(const fa_config* cfg, int32_t pass, int64_t* items, int64_t cap, int64_t* n,
                            int32_t* tile_rows, int32_t* tile_cols) {
  if (!n) return FA_ERR_PARAM_NULLPTR;
  if (pass < 0 || pass > 2) return FA_ERR_PARAM_INVALID;
  Problem pr;
  fa_status st = parse(cfg, &pr);
  if (st != FA_OK) return st;
  int bm, bn;
  std::vector<WorkItem> v = schedule(pr, pass, &bm, &bn);
  *n = (int64_t)v.size();
  if (tile_rows) *tile_rows = bm;
  if (tile_cols) *tile_cols = bn;
  if (items) {
    const int64_t m = std::min<int64_t>(cap, (int64_t)v.size());
    for (int64_t i = 0; i < m; ++i) {
      items[4 * i + 0] = v[i].b;
      items[4 * i + 1] = v[i].tile;
      items[4 * i + 2] = v[i].lo;
      items[4 * i + 3] = v[i].hi;
    }
  }
  return FA_OK;
}

fa_status fa_decode_workspace_size(const fa_decode_config* cfg, uint64_t* bytes) {
  if (!bytes) return FA_ERR_PARAM_NULLPTR;
  DecProblem pr;
  fa_status st = parse_decode(cfg, &pr);
  if (st != FA_OK) return st;
  *bytes = plan_decode(pr).total;
  return FA_OK;
}

namespace {

// One decode call on a validated problem and its plan; ws holds at least P.total bytes.
fa_status decode_run(const DecProblem& pr, const DecPlan& P, const void* q, const void* k, const void* v, void* out,
                     char* ws, hipStream_t s) {
  std::vector<char> host(P.staged, 0);
  std::memcpy(host.data() + P.off_items, P.items.data(), sizeof(fa::DecItem) * P.items.size());
  std::memcpy(host.data() + P.off_first, P.first_slot.data(), 4 * P.first_slot.size());
  std::memcpy(host.data() + P.off_nsplit, P.n_split.data(), 4 * P.n_split.size());
  if (stage_plan(ws, host, s) != hipSuccess) return FA_ERR_HIP;

  fa::DecParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out;
  p.mask = pr.mask;
  p.mask_stride = pr.s;
  p.items = reinterpret_cast<const fa::DecItem*>(ws + P.off_items);
  p.first_slot = reinterpret_cast<const int32_t*>(ws + P.off_first);
  p.n_split = reinterpret_cast<const int32_t*>(ws + P.off_nsplit);
  p.part_o = reinterpret_cast<float*>(ws + P.off_o);
  p.part_m = reinterpret_cast<float*>(ws + P.off_m);
  p.part_l = reinterpret_cast<float*>(ws + P.off_l);
  // KV cache strides (elements): BSH and BSND are [B, S, Nkv, D], BNSD is [B, Nkv, S, D]
  p.kv_bstride = pr.s * pr.nkv * pr.d;
  p.kv_tstride = pr.layout == FA_LAYOUT_BNSD ? pr.d : pr.nkv * pr.d;
  p.kv_hstride = pr.layout == FA_LAYOUT_BNSD ? pr.s * pr.d : pr.d;
  p.nq = (int32_t)pr.nq;
  p.nkv = (int32_t)pr.nkv;
  p.group = (int32_t)(pr.nq / pr.nkv);
  p.keys_per_wave = (int32_t)(P.chunk / fa::kDecWaves);
  p.batch = (int32_t)pr.batch;
  p.scale_log2 = (float)(pr.scale * 1.4426950408889634);
  const int n_items = (int)P.items.size();
  if (log_on())
    std::fprintf(stderr, "[fa] fa_decode: B=%lld S=%lld Nq=%lld Nkv=%lld D=%lld layout=%d chunk=%lld items=%d "
                 "split slots=%lld\n", (long long)pr.batch, (long long)pr.s, (long long)pr.nq, (long long)pr.nkv,
                 (long long)pr.d, pr.layout, (long long)P.chunk, n_items, (long long)P.n_slots);
  hipError_t e = timed(K_DEC, s, [&] { return fa::launch_decode(pr.dtype, (int)pr.d, n_items, p, s); });
  if (e == hipSuccess && P.n_slots > 0)
    e = timed(K_DEC_REDUCE, s, [&] { return fa::launch_decode_reduce(pr.dtype, (int)pr.d, p, s); });
  return hip_status(e);
}

}  // namespace

fa_status fa_decode(const fa_decode_config* cfg, const void* q, const void* k, const void* v, void* out,
                    void* workspace, uint64_t workspace_bytes, void* stream) {
  DecProblem pr;
  fa_status st = parse_decode(cfg, &pr);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !out || !workspace) return FA_ERR_PARAM_NULLPTR;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FA_ERR_PARAM_INVALID;
  const DecPlan P = plan_decode(pr);
  if (!aligned(workspace, 16)) return FA_ERR_PARAM_INVALID;
  if (workspace_bytes < P.total) return FA_ERR_WORKSPACE;
  return decode_run(pr, P, q, k, v, out, reinterpret_cast<char*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

fa_status fa_decode_noalloc(const fa_decode_config* cfg, const void* q, const void* k, const void* v, void* out,
                            void* stream) {
  DecProblem pr;
  fa_status st = parse_decode(cfg, &pr);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !out) return FA_ERR_PARAM_NULLPTR;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FA_ERR_PARAM_INVALID;
  const DecPlan P = plan_decode(pr);
  if (P.total > kNoallocScratchBytes) return FA_ERR_SCRATCH;
  char* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  return decode_run(pr, P, q, k, v, out, ws, reinterpret_cast<hipStream_t>(stream));
}

#if defined(FA_TRACE_VISITS)
fa_status fa_debug_trace(int32_t pass, uint32_t* counters, int64_t words) {
  if (pass < 0 || pass > 2 || words < 0) return FA_ERR_PARAM_INVALID;
  std::lock_guard<std::mutex> g(g_trace_mu);
  g_trace[pass] = counters;
  g_trace_words[pass] = counters ? words : 0;
  return FA_OK;
}
#endif

fa_status fa_profile_enable(int32_t on) {
  ProfState& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.on = on != 0;
  return FA_OK;
}

int32_t fa_profile_kernel_count(void) { return K_COUNT; }

fa_status fa_profile_read(int32_t k, const char** name, double* total_ms, int64_t* launches) {
  if (k < 0 || k >= K_COUNT) return FA_ERR_PARAM_INVALID;
  ProfState& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (auto& pr : P.ev[k]) {
    if (hipEventSynchronize(pr.second) != hipSuccess) return FA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return FA_ERR_HIP;
    P.total_ms[k] += ms;
    P.launches[k] += 1;
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  P.ev[k].clear();
  if (name) *name = kKernelNames[k];
  if (total_ms) *total_ms = P.total_ms[k];
  if (launches) *launches = P.launches[k];
  P.total_ms[k] = 0;
  P.launches[k] = 0;
  return FA_OK;
}

}  // extern "C"
