// Mask intervals and tile ranges shared by the host scheduler and the kernels.
//
// The sparse modes of aclnnFlashAttentionUnpaddingScoreGrad ("sparseMode"
// parameter list) and the sliding window of aclnnFlashAttentionScoreV2
// ("preTokens"/"nextTokens" parameters) all reduce to one closed interval of
// allowed keys per query row:
//     allowed(i, j)  <=>  i + delta - pre <= j <= i + delta + next,
//                         0 <= i < Lq, 0 <= j < Lkv
//   mode 0 (no mask)          : pre = next = FA_WINDOW_INF
//   mode 2 (leftUpCausal)     : pre = FA_WINDOW_INF, next = 0, delta = 0
//   mode 3 (rightDownCausal)  : pre = FA_WINDOW_INF, next = 0, delta = Lkv - Lq
//   mode 4 (band)             : pre, next as given,        delta = Lkv - Lq
//   mode 6 (prefix N)         : as mode 3, and hi(i) >= N - 1 ("floor"): the
//                               sequence's first N keys are visible to every row
//   modes 7, 8                : one of the above per sequence (fa_seq_mode)
// Both interval ends are non-decreasing in the row and every non-empty row
// interval meets its neighbours' (they grow by one per row; the prefix floor
// only raises hi where lo is unbounded), so the allowed set of a rectangular
// tile is empty iff hi(last row) < first key or lo(first row) > last key, and
// full iff lo(last row) <= first key and last key <= hi(first row).  Windows
// are clamped to +-2^30, which leaves every allowed set unchanged because
// sequences are at most 2^20 long.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

#define FA_WINDOW_INF (1 << 30)

struct FaWindow {
  int32_t delta;  // diagonal offset (Lkv - Lq for bottom-right aligned modes)
  int32_t pre;    // keys allowed to the left of the diagonal
  int32_t next;   // keys allowed to the right of the diagonal
  int32_t floor;  // every row may also see keys [0, floor] (prefix mode: N - 1; else -1)
};

// Sparse modes 7 and 8 (aclnnFlashAttentionUnpaddingScoreGrad, sparseMode list:
// both arise when long sequences are split outside the operator) combine two of
// the masks above over the batch:
//   mode 7 (rightDownCausal_Band): the last sequence takes the band (mode 4),
//                                  every other one rightDownCausal (mode 3);
//   mode 8 (band_LeftUpCausal):    the first sequence takes the band, every
//                                  other one leftUpCausal (mode 2).
FA_HD int fa_seq_mode(int mode, int64_t b, int64_t nseq) {
  if (mode == 7) return b == nseq - 1 ? 4 : 3;
  if (mode == 8) return b == 0 ? 4 : 2;
  return mode;
}

FA_HD int64_t fa_clamp_window(int64_t w) {
  return w > FA_WINDOW_INF ? FA_WINDOW_INF : (w < -FA_WINDOW_INF ? -FA_WINDOW_INF : w);
}

// Allowed keys of query row i (local indices) form one interval [lo(i), hi(i)],
// both ends non-decreasing in i:
//   mode 0: all keys; mode 2: j <= i; mode 3: j <= i + (Lkv - Lq);
//   mode 4: i + (Lkv - Lq) - pre <= j <= i + (Lkv - Lq) + next;
//   mode 6 (prefix N of the sequence): j <= max(i + (Lkv - Lq), N - 1), i.e. the
//   bottom-right causal triangle plus the first N keys for every row.
FA_HD FaWindow fa_make_window(int mode, int64_t pre, int64_t next, int32_t lq, int32_t lkv, int32_t prefix = 0) {
  FaWindow w;
  w.delta = 0;
  w.pre = FA_WINDOW_INF;
  w.next = FA_WINDOW_INF;
  w.floor = -1;
  if (mode == 6) {
    w.next = 0;
    w.delta = lkv - lq;
    w.floor = prefix - 1;
  } else if (mode == 2) {
    w.next = 0;
  } else if (mode == 3) {
    w.next = 0;
    w.delta = lkv - lq;
  } else if (mode == 4) {
    w.pre = (int32_t)fa_clamp_window(pre);
    w.next = (int32_t)fa_clamp_window(next);
    w.delta = lkv - lq;
  }
  return w;
}

FA_HD int32_t fa_row_lo(const FaWindow& w, int32_t i) { return i + w.delta - w.pre; }
FA_HD int32_t fa_row_hi(const FaWindow& w, int32_t i) {
  const int32_t h = i + w.delta + w.next;
  return h > w.floor ? h : w.floor;
}

FA_HD bool fa_allowed(const FaWindow& w, int32_t i, int32_t j, int32_t lq, int32_t lkv) {
  return i < lq && j < lkv && j >= fa_row_lo(w, i) && j <= fa_row_hi(w, i);
}

// Rows [r0, r1) x keys [c0, c1), already clipped to the sequence; r1 > r0, c1 > c0.
FA_HD bool fa_tile_empty(const FaWindow& w, int32_t r0, int32_t r1, int32_t c0, int32_t c1) {
  return fa_row_hi(w, r1 - 1) < c0 || fa_row_lo(w, r0) > c1 - 1;
}

// Tile of nominal size bm x bn at (r0, c0): full when no row or key falls outside
// the sequence and every pair is allowed (no mask work needed).
FA_HD bool fa_tile_full(const FaWindow& w, int32_t r0, int32_t bm, int32_t c0, int32_t bn,
                        int32_t lq, int32_t lkv) {
  return r0 + bm <= lq && c0 + bn <= lkv && fa_row_lo(w, r0 + bm - 1) <= c0 &&
         c0 + bn - 1 <= fa_row_hi(w, r0);
}

FA_HD int32_t fa_floordiv(int32_t a, int32_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Key tiles [*t_lo, *t_hi) of width bn holding at least one allowed pair for rows [r0, r1).
FA_HD void fa_kv_tile_range(const FaWindow& w, int32_t r0, int32_t r1, int32_t lkv, int32_t bn,
                            int32_t* t_lo, int32_t* t_hi) {
  int32_t ntiles = (lkv + bn - 1) / bn;
  int32_t jlo = fa_row_lo(w, r0);
  int32_t jhi = fa_row_hi(w, r1 - 1);
  if (jlo < 0) jlo = 0;
  if (jhi > lkv - 1) jhi = lkv - 1;
  if (lkv <= 0 || r1 <= r0 || jhi < jlo) {
    *t_lo = 0;
    *t_hi = 0;
    return;
  }
  int32_t a = jlo / bn, b = jhi / bn + 1;
  if (b > ntiles) b = ntiles;
  *t_lo = a;
  *t_hi = b;
}

// Query tiles [*t_lo, *t_hi) of height bm holding at least one allowed pair for keys [c0, c1).
FA_HD void fa_q_tile_range(const FaWindow& w, int32_t c0, int32_t c1, int32_t lq, int32_t bm,
                           int32_t* t_lo, int32_t* t_hi) {
  int32_t ntiles = (lq + bm - 1) / bm;
  // rows i with hi(i) >= c0 and lo(i) <= c1 - 1 (every row reaches c0 when the floor does)
  int32_t ilo = w.floor >= c0 ? 0 : c0 - w.delta - w.next;
  int32_t ihi = c1 - 1 - w.delta + w.pre;
  if (ilo < 0) ilo = 0;
  if (ihi > lq - 1) ihi = lq - 1;
  if (lq <= 0 || c1 <= c0 || ihi < ilo) {
    *t_lo = 0;
    *t_hi = 0;
    return;
  }
  int32_t a = ilo / bm, b = ihi / bm + 1;
  if (b > ntiles) b = ntiles;
  *t_lo = a;
  *t_hi = b;
}
