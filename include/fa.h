/*
 * fa.h -- C ABI of the MI355X (gfx950) varlen FlashAttention library (libfa.so).
 *
 * Operations (semantics from the Ascend CANN pages):
 *   fa_fwd  -- training forward of aclnnFlashAttentionScoreV2 ("Formula",
 *              pseType 2) in TND layout: O = Dropout(Softmax(Mask(scale*QK^T
 *              + pse)), keep_prob) V, plus the per-row softmax max and sum,
 *              with the optional attention sink of
 *              aclnnFlashAttentionUnpaddingScoreGradV5 (sink formulas).
 *   fa_bwd  -- training backward of aclnnFlashAttentionUnpaddingScoreGrad
 *              ("Formula"): dV = P^T dY, dQ = scale * dS K, dK = scale * dS^T Q,
 *              and dSink of aclnnFlashAttentionUnpaddingScoreGradV5.
 *
 * Two phases, as on the pages ("Prototype": GetWorkspaceSize, then execute):
 * call fa_*_workspace_size for the device workspace a call needs, then fa_fwd /
 * fa_bwd with a workspace at least that large.
 *
 * Layout (TND, the only layout of the varlen grad page): Q, O, dY, dQ are
 * [T_q, Nq, D], K, V, dK, dV are [T_kv, Nkv, D], contiguous row-major;
 * element (t, n, d) at (t*N + n)*D + d.  softmax_max / softmax_sum are fp32
 * [T_q, Nq] (the pages' trailing x8 replication is not stored).  The max is in
 * natural-log units of the scaled, biased, masked logits (including the sink);
 * the sum is sum_j exp(s_ij - max) (+ exp(sink - max)), both before dropout.
 * Rows with no allowed key and no sink get max = -inf, sum = 0, O = 0.
 *
 * Ownership: the caller owns every buffer and the stream.  The library
 * allocates no device memory and keeps no per-call state.  Calls enqueue work
 * on `stream` (a hipStream_t; NULL = default stream) and return without
 * synchronising.  cu_seqlens arrays are HOST memory, read during the call and
 * copied into the workspace, so they may be freed when the call returns.
 * Two calls that share a workspace must be ordered on the same stream.  The
 * workspace must be 16-byte aligned (else FA_ERR_PARAM_INVALID).
 *
 * Stream capture: every call may be captured into a HIP graph.  The work plan
 * the call builds on the host reaches the workspace through kernel arguments
 * while the stream is capturing (plain hipMemcpyAsync otherwise), so a graph
 * holds no reference to host memory; each replay recomputes the outputs from
 * the current contents of the input buffers with the captured configuration.
 *
 * Errors: every argument is validated before anything is enqueued; on error
 * nothing is written.  Codes 161001 / 161002 mirror ACLNN_ERR_PARAM_NULLPTR /
 * ACLNN_ERR_PARAM_INVALID of the aclnnFlashAttentionScoreV2 page ("Returns"
 * table).
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fa_status;
#define FA_OK 0
#define FA_ERR_PARAM_NULLPTR 161001 /* a required pointer argument is NULL */
#define FA_ERR_PARAM_INVALID 161002 /* an attribute, shape, dtype or alignment is unsupported */
#define FA_ERR_WORKSPACE 1          /* workspace_bytes smaller than the size query returned */
#define FA_ERR_HIP 2                /* a HIP runtime call or kernel launch failed */
#define FA_ERR_SCRATCH 3            /* fa_decode_noalloc: the call needs more scratch than its
                                       static buffer holds (FA_DECODE_NOALLOC_SCRATCH_BYTES) */

/* element type of Q, K, V, dY, O, dQ, dK, dV (the pages list FLOAT16, BFLOAT16 and
   FLOAT32 for these tensors: aclnnFlashAttentionUnpaddingScoreGrad, parameter table).
   16-bit inputs are multiplied on the matrix cores in their own type with fp32
   accumulation; softmax statistics and dQ partial sums stay fp32. */
#define FA_DTYPE_FP32 0
#define FA_DTYPE_BF16 1
#define FA_DTYPE_FP16 2

/* inputLayout (aclnnFlashAttentionScoreV2, "inputLayout"): TND packs sequences of
   any lengths; the others hold B sequences of one common length S per side
   (H = N*D).  fa_config.layout selects it for Q, K, V, dY, O, dQ, dK, dV. */
#define FA_LAYOUT_TND 0   /* [T, N, D]                                         */
#define FA_LAYOUT_BSH 1   /* [B, S, H]      (same bytes as TND with L_b = S)   */
#define FA_LAYOUT_BSND 2  /* [B, S, N, D]   (same bytes as TND with L_b = S)   */
#define FA_LAYOUT_BNSD 3  /* [B, N, S, D]                                      */
#define FA_LAYOUT_SBH 4   /* [S, B, H]                                         */

/* sparse modes (aclnnFlashAttentionUnpaddingScoreGrad, "sparseMode" parameter) */
#define FA_SPARSE_NONE 0             /* every pair allowed (or those the attenMask keeps)    */
#define FA_SPARSE_ALL_MASK 1         /* the pairs the attenMask keeps (mask required)        */
#define FA_SPARSE_LEFT_UP_CAUSAL 2   /* j <= i                                               */
#define FA_SPARSE_RIGHT_DOWN_CAUSAL 3 /* j <= i + (Lkv - Lq)                                  */
#define FA_SPARSE_BAND 4             /* i+(Lkv-Lq)-pre <= j <= i+(Lkv-Lq)+next (inclusive)    */
#define FA_SPARSE_PREFIX 6           /* j <= i + (Lkv - Lq)  or  j < N_b (prefix, see below)  */
/* modes 7 and 8 (same list: produced when long sequences are split outside the operator)
   give the band to one sequence and a causal triangle to the others; pre/next as in mode 4 */
#define FA_SPARSE_RIGHT_DOWN_CAUSAL_BAND 7  /* last sequence: band; the others: mode 3     */
#define FA_SPARSE_BAND_LEFT_UP_CAUSAL 8     /* first sequence: band; the others: mode 2    */

#define FA_TOKENS_DEFAULT 2147483647 /* preTokens / nextTokens default of the pages */

/* fa_config.flags bits: how alibi_slopes generate the position bias (pse) of
   aclnnFlashAttentionScoreV2 (pseType table: types 2 and 3 generate the pse
   inside the operator from FLOAT32 slopes of shape [B,N] or [N]; the bias is added
   after scaling and needs Lq_b == Lkv_b).  Ignored when alibi_slopes is NULL. */
#define FA_FLAG_PSE_SQRT 1u          /* pseType 3: pse = -slope * sqrt(|i - j|); without
                                        this bit pseType 2: pse = -slope * (i - j)      */
#define FA_FLAG_SLOPES_PER_BATCH 2u  /* alibi_slopes is [B, Nq] (one row per sequence)
                                        instead of [Nq]                                 */
#define FA_FLAG_ATOMIC_DQ 4u         /* with deterministic = 0: accumulate dQ with fp32
                                        atomics inside the dK/dV pass                  */

typedef struct fa_config {
  int64_t batch;                 /* B >= 1 sequences                                          */
  const int64_t* cu_seqlens_q;   /* HOST, B+1 entries: [0] = 0, non-decreasing, [B] = T_q     */
  const int64_t* cu_seqlens_kv;  /* HOST, B+1 entries, same rules, [B] = T_kv               */
  int64_t head_num;              /* Nq in [1, 256] (headNum)                                  */
  int64_t num_kv_heads;          /* Nkv; 0 means Nkv = Nq; Nq % Nkv == 0 (GQA)                */
  int64_t head_dim;              /* D <= 512 (the grad page's limit), D * element size a
                                    multiple of 16 bytes.  64 and 128 run natively, other
                                    D <= 128 on copies zero-padded to 64 or 128; D > 128 runs a
                                    path that materialises one chunk of scores at a time in
                                    the workspace (MFMA GEMMs and softmax kernels; slower,
                                    always deterministic)                                     */
  int32_t dtype;                 /* FA_DTYPE_*                                                */
  int32_t sparse_mode;           /* FA_SPARSE_*; modes 7 and 8 take no pse tensor, and mode 7
                                    no alibi_slopes either (the grad pages' sparse_mode=7/8
                                    constraints)                                              */
  double scale;                  /* scaleValue: multiplies Q K^T (usually D^-0.5)             */
  double keep_prob;              /* keepProb in (0, 1]; < 1 needs drop_mask                   */
  int64_t pre_tokens;            /* band only: keys allowed left of the diagonal              */
  int64_t next_tokens;           /* band only: keys allowed right of the diagonal             */
  int32_t deterministic;         /* bwd: 1 = separate dQ pass (bitwise reproducible); 0 = the
                                    pages' non-deterministic mode, which allows any result of
                                    either scheme: it runs the same passes (faster here than
                                    atomic accumulation), or, with FA_FLAG_ATOMIC_DQ, fp32
                                    atomic dQ in the dK/dV pass where that variant exists
                                    (not fp32 with D > 64, D > 128, a 16-bit external pse,
                                    nor 16-bit D = 128 with alibi_slopes)                    */
  int32_t flags;                 /* FA_FLAG_* bits; any other bit -> FA_ERR_PARAM_INVALID     */
  const int64_t* prefix;         /* HOST, B entries, read in FA_SPARSE_PREFIX only (ignored
                                    otherwise): N_b of the prefix-compressed mask
                                    (aclnnFlashAttentionUnpaddingScoreGrad "prefixOptional";
                                    sparseMode 6).  Row i of sequence b keeps keys
                                    j <= i + (Lkv_b - Lq_b) and every key j < N_b.  Range
                                    ("Constraints"): N_b in [0, Lkv_b] when Lq_b > Lkv_b,
                                    else [Lkv_b - Lq_b, Lkv_b]; B <= 1024 with a prefix.
                                    NULL in mode 6 -> FA_ERR_PARAM_NULLPTR; out of range
                                    -> FA_ERR_PARAM_INVALID.                                 */
  const uint8_t* atten_mask;     /* DEVICE, optional: attenMaskOptional of the grad page, BOOL /
                                    UINT8 [mask_rows, mask_cols] row-major, shared by every
                                    sequence and head and indexed by the sequence's local row
                                    and key; nonzero = the pair is masked out.  Used with
                                    modes 0 (the mask alone), 1 (required) and 4 (and the
                                    band); modes 2, 3 and 6 define their own triangle (the
                                    page's compressed masks for them carry no more) and
                                    ignore it.  NULL = no mask.                               */
  int64_t mask_rows;             /* S1Max >= every Lq_b (with atten_mask)                     */
  int64_t mask_cols;             /* S2Max >= every Lkv_b (with atten_mask)                    */
  int32_t layout;                /* FA_LAYOUT_* of Q, K, V, dY, O and the gradients; 0 = TND.
                                    Other layouts need cu_seqlens with one common length
                                    per side (cu[b] = b*S), else FA_ERR_PARAM_INVALID.  BNSD
                                    and SBH are gathered into TND copies in the workspace
                                    (the size query accounts for them) and the outputs
                                    scattered back.  softmax_max / softmax_sum stay
                                    [T, Nq] with T = B*Sq, row t = b*Sq + s.                 */
  const void* pse;               /* DEVICE, optional external pse of cfg->dtype (grad page
                                    "pseShiftOptional", ScoreV2 page "realShiftOptional"),
                                    row-major [pse_batch, Nq, pse_rows, pse_cols], indexed by
                                    the sequence's local row i and key j.  pse_rows selects
                                    the form: 1 = one row for every query row ([B,N,1,Skv]);
                                    >= every Lq = the full [S1, S2] block; 1024 below some Lq
                                    = alibi compression (the last 1024 rows of the full pse,
                                    Lq == Lkv and sparse mode 2 or 3 required; a row i above
                                    the stored block reads the first stored row shifted along
                                    the diagonal).  Not with alibi_slopes or an attenMask.
                                    With bf16 / fp16 inputs the call runs the materialised-
                                    score path (deterministic backward; its workspace holds
                                    a chunk of scores, up to about 4 GiB).  NULL = none.      */
  int64_t pse_batch;             /* 1 (shared by the sequences) or B                          */
  int64_t pse_rows;              /* see pse                                                   */
  int64_t pse_cols;              /* S2 >= every Lkv                                           */
  int32_t pse_type;              /* with pse: 0 = mul then add, S = scale*QK^T + pse;
                                    1 = add then mul, S = scale*(QK^T + pse) (the grad page's
                                    formula; ScoreV2 pseType table)                           */
  const int64_t* strides;        /* HOST, optional, TND only: 16 element strides, (token, head)
                                    for q, k, v, dy, out, dq, dk, dv in that order; the D
                                    axis stays contiguous.  Each stride times the element size
                                    must be a multiple of 16 bytes; output rows must not
                                    overlap.  Tensors whose strides differ from the packed
                                    ones (N*D, D) are gathered into packed copies in the
                                    workspace (outputs scattered back).  NULL = packed.       */
  const int64_t* q_start_idx;    /* HOST, optional, one value (qStartIdxOptional of
                                    aclnnFlashAttentionScoreV2: where the query rows of a chunk
                                    of a long sequence split outside the operator start in that
                                    sequence).  Sparse mode 8 only: the first sequence's query
                                    row i sits at q_start_idx + i, its key j at kv_start_idx + j,
                                    and its generated pse (alibi_slopes) is formed on those
                                    positions.  Given in mode 8, the pages' constraint
                                    Lq_0 - Lkv_0 + q_start_idx - kv_start_idx == 0 must hold.
                                    Non-NULL in another mode, negative, or off the constraint
                                    -> FA_ERR_PARAM_INVALID.  NULL = 0.                       */
  const int64_t* kv_start_idx;   /* HOST, optional, one value (kvStartIdxOptional): as above
                                    for the first sequence's keys.  NULL = 0.                  */
  int64_t v_head_dim;            /* head dim of V, O, dY and dV when it is smaller than
                                    head_dim (the grad page, Constraints: qD == kD >= vD);
                                    0 = head_dim.  Same 16-byte row rule as head_dim; Q, K,
                                    dQ, dK keep head_dim.  Runs on copies zero-padded to the
                                    kernels' head dim.                                        */
} fa_config;

/* Device workspace bytes needed by fa_fwd for this configuration (>= 256). */
fa_status fa_fwd_workspace_size(const fa_config* cfg, uint64_t* bytes);

/*
 * Forward.  Inputs (device): q [T_q,Nq,D], k, v [T_kv,Nkv,D] of cfg->dtype.
 * drop_mask: device uint8, required iff keep_prob < 1: the keep bits of
 *   aclnnFlashAttentionUnpaddingScoreGrad "dropMaskOptional", one flat stream of
 *   Nq * sum_b Lq_b*Lkv_b bits ordered (sequence, query head, row, key), bit n in
 *   byte n/8 at position n%8 (LSB first), 1 = keep; ceil(bits/8) bytes, 4-byte aligned.
 * alibi_slopes: device fp32 [Nq] (or [B, Nq] with FA_FLAG_SLOPES_PER_BATCH) or NULL:
 *   adds -slope*(i-j) (pseType 2) or, with FA_FLAG_PSE_SQRT, -slope*sqrt(|i-j|)
 *   (pseType 3) after scaling, i and j local to the sequence; requires
 *   Lq_b == Lkv_b > 0 for every sequence (in mode 8 the first sequence may instead
 *   satisfy the start-index constraint, its positions then being global).
 * sink: device fp32 [Nq] or NULL: per-head sink logit in the softmax denominator.
 * Outputs (device): out [T_q,Nq,D] of cfg->dtype; softmax_max, softmax_sum fp32 [T_q,Nq].
 * All tensor pointers must be 16-byte aligned.
 */
fa_status fa_fwd(const fa_config* cfg, const void* q, const void* k, const void* v,
                 const uint8_t* drop_mask, const float* alibi_slopes, const float* sink,
                 void* out, float* softmax_max, float* softmax_sum,
                 void* workspace, uint64_t workspace_bytes, void* stream);

/* Device workspace bytes needed by fa_bwd for this configuration. */
fa_status fa_bwd_workspace_size(const fa_config* cfg, uint64_t* bytes);

/*
 * Backward.  Inputs are the forward's inputs plus dy [T_q,Nq,D] and the
 * forward's out, softmax_max and softmax_sum (attentionIn / softmaxMax / softmaxSum).
 * Outputs (device): dq [T_q,Nq,D], dk, dv [T_kv,Nkv,D] of cfg->dtype, fully
 * overwritten; dsink fp32 [Nq], required iff sink != NULL.
 */
fa_status fa_bwd(const fa_config* cfg, const void* q, const void* k, const void* v, const void* dy,
                 const void* out, const float* softmax_max, const float* softmax_sum,
                 const uint8_t* drop_mask, const float* alibi_slopes, const float* sink,
                 void* dq, void* dk, void* dv, float* dsink,
                 void* workspace, uint64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention: aclnnIncreFlashAttentionV2 (incremental inference).  Each
 * of the B sequences brings one query token (the page fixes the query S axis at
 * 1) and attends to the first L_b keys of a padded KV cache:
 *   out[b, h] = Softmax(scale * q[b, h] K_b^T) V_b      (keys 0 .. L_b - 1)
 * with query head h reading kv head h / (Nq / Nkv) (GQA).  The page's int8
 * quantisation parameters and its reserved pseShift are not part of this call.
 * ------------------------------------------------------------------------ */

/* inputLayout of the decode page: query [B,1,H] / [B,1,N,D] / [B,N,1,D] and
   key, value [B,S,H] / [B,S,N,D] / [B,N,S,D] (H = N*D).  The query and the
   output are [B, Nq, D] in memory under every layout.  (The FA_LAYOUT_* values
   are shared with fa_config.layout.) */
typedef struct fa_decode_config {
  int64_t batch;                      /* B in [1, 65536]                                          */
  int64_t max_seq_len;                /* S: padded key length of the cache, in [1, 2^24]           */
  const int64_t* actual_seq_lengths;  /* HOST, B entries in [0, S] (actualSeqLengths), or NULL
                                         for L_b = S.  A sequence with L_b = 0 (or every key
                                         masked) gets out = 0.                                   */
  int64_t num_heads;                  /* Nq in [1, 256] (numHeads)                                */
  int64_t num_kv_heads;               /* Nkv (numKeyValueHeads); 0 means Nkv = Nq;
                                         Nq % Nkv == 0 and Nq / Nkv <= 64                         */
  int64_t head_dim;                   /* D in {64, 128}                                           */
  int32_t dtype;                      /* FA_DTYPE_BF16 or FA_DTYPE_FP16 (q, k, v, out)            */
  int32_t layout;                     /* FA_LAYOUT_*                                              */
  double scale;                       /* scaleValue, multiplies q K^T                             */
  const uint8_t* atten_mask;          /* DEVICE, optional BOOL / UINT8 [B, S] row-major; nonzero
                                         masks key s out of sequence b.  NULL = no mask.          */
  int32_t flags;                      /* reserved, must be 0                                      */
} fa_decode_config;

/* Device workspace bytes needed by fa_decode for this configuration (depends on
   actual_seq_lengths: query again when they change).  >= 256. */
fa_status fa_decode_workspace_size(const fa_decode_config* cfg, uint64_t* bytes);

/*
 * Decode.  Inputs (device, cfg->dtype): q [B, Nq, D]; k, v: the cache in
 * cfg->layout with S = max_seq_len key rows per sequence (rows at or beyond L_b
 * are never read).  Output (device): out [B, Nq, D] of cfg->dtype, fully
 * overwritten.  q, k, v, out and the workspace 16-byte aligned; the workspace is caller-owned and
 * enqueued work uses it until it completes on `stream`.  Errors as fa_fwd:
 * FA_ERR_PARAM_NULLPTR, FA_ERR_PARAM_INVALID (limits above, misalignment),
 * FA_ERR_WORKSPACE, FA_ERR_HIP; nothing is enqueued on a validation error.
 */
fa_status fa_decode(const fa_decode_config* cfg, const void* q, const void* k, const void* v, void* out,
                    void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory or
 * hand over a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same operation, arguments, kernels and
 * results as fa_decode, but the scratch (the staged work plan and the split
 * partial results) lives in a static device buffer of
 * FA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends; the call allocates nothing.  A configuration whose
 * scratch (fa_decode_workspace_size) exceeds that size returns FA_ERR_SCRATCH
 * before anything is enqueued.  Every call on one GPU shares that GPU's buffer:
 * calls that may overlap on one GPU (different streams, or host threads) race,
 * so order them on one stream.  Errors otherwise as fa_decode.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (32ull << 20)
fa_status fa_decode_noalloc(const fa_decode_config* cfg, const void* q, const void* k, const void* v, void* out,
                            void* stream);

/* Static text for a status code. */
const char* fa_status_string(fa_status status);

/*
 * Host-only view of the tile scheduler (no device calls).  pass 0 = forward,
 * 1 = backward dK/dV pass, 2 = backward dQ pass.  Writes up to `cap` items of
 * 4 int64 each: (sequence, tile, lo, hi) where tile is a query tile (passes 0, 2)
 * or a key tile (pass 1) and [lo, hi) the range of the other axis' tiles that
 * hold at least one allowed pair; *n receives the item count.  Items are in
 * launch order (longest first).  tile_rows / tile_cols receive the pass's tile
 * shape (query rows, keys) when non-NULL.
 */
fa_status fa_debug_schedule(const fa_config* cfg, int32_t pass, int64_t* items, int64_t cap, int64_t* n,
                            int32_t* tile_rows, int32_t* tile_cols);

/*
 * Kernel timing for measurement: while enabled, every kernel the library
 * launches is bracketed by HIP events on its stream.  fa_profile_read
 * synchronises those events and returns, for kernel index k in [0, count),
 * its name, total milliseconds and launch count, then clears the record.
 */
fa_status fa_profile_enable(int32_t on);
fa_status fa_profile_read(int32_t k, const char** name, double* total_ms, int64_t* launches);
int32_t fa_profile_kernel_count(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
