/* Host-only driver of the C ABI for sanitizer runs: every call below returns
 * before any device work (size queries, the host scheduler view, validation
 * failures), so it runs without a GPU.  Exit status 0 when every expectation
 * holds; AddressSanitizer / UBSan abort the run on a memory or UB error. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "expectation failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static uint32_t rng = 12345u;
static uint32_t next_rand(void) {   /* xorshift32 */
  rng ^= rng << 13;
  rng ^= rng >> 17;
  rng ^= rng << 5;
  return rng;
}

static void base_config(fa_config* c, const int64_t* cq, const int64_t* ck, int64_t b) {
  memset(c, 0, sizeof(*c));
  c->batch = b;
  c->cu_seqlens_q = cq;
  c->cu_seqlens_kv = ck;
  c->head_num = 8;
  c->num_kv_heads = 2;
  c->head_dim = 128;
  c->dtype = FA_DTYPE_BF16;
  c->sparse_mode = FA_SPARSE_RIGHT_DOWN_CAUSAL;
  c->scale = 0.088;
  c->keep_prob = 1.0;
  c->pre_tokens = FA_TOKENS_DEFAULT;
  c->next_tokens = FA_TOKENS_DEFAULT;
  c->deterministic = 1;
}

int main(void) {
  int64_t cq[65], ck[65], prefix[64];
  static int64_t items[4 * 200000];
  fa_config c;
  uint64_t bytes = 0;
  for (int trial = 0; trial < 300; ++trial) {
    const int64_t b = 1 + next_rand() % 64;
    cq[0] = ck[0] = 0;
    for (int64_t i = 0; i < b; ++i) {
      cq[i + 1] = cq[i] + next_rand() % 700;
      ck[i + 1] = ck[i] + next_rand() % 700;
    }
    if (cq[b] == 0) cq[b] = 1;
    if (ck[b] == 0) ck[b] = 1;
    base_config(&c, cq, ck, b);
    const int modes[] = {FA_SPARSE_NONE, FA_SPARSE_LEFT_UP_CAUSAL, FA_SPARSE_RIGHT_DOWN_CAUSAL, FA_SPARSE_BAND,
                         FA_SPARSE_PREFIX};
    c.sparse_mode = modes[trial % 5];
    c.pre_tokens = (int64_t)(next_rand() % 300) - 20;
    c.next_tokens = (int64_t)(next_rand() % 300);
    c.head_dim = (trial % 3 == 0) ? 64 : (trial % 3 == 1) ? 128 : 96;
    c.dtype = trial % 2 ? FA_DTYPE_BF16 : FA_DTYPE_FP32;
    c.keep_prob = trial % 4 == 0 ? 0.9 : 1.0;
    if (c.sparse_mode == FA_SPARSE_PREFIX) {
      for (int64_t i = 0; i < b; ++i) {
        const int64_t lq = cq[i + 1] - cq[i], lkv = ck[i + 1] - ck[i];
        prefix[i] = lq > lkv ? lkv / 2 : lkv - lq + (lq ? (int64_t)(next_rand() % (lq + 1)) : 0);
      }
      c.prefix = prefix;
    }
    const fa_status a = fa_fwd_workspace_size(&c, &bytes);
    const fa_status bw = fa_bwd_workspace_size(&c, &bytes);
    EXPECT(a == bw);
    if (a != FA_OK) continue;   /* e.g. an empty band intersection */
    for (int pass = 0; pass < 3; ++pass) {
      int64_t n = 0;
      int32_t rows = 0, cols = 0;
      EXPECT(fa_debug_schedule(&c, pass, items, 200000, &n, &rows, &cols) == FA_OK);
      EXPECT(n >= 0 && rows > 0 && cols > 0);
      for (int64_t i = 0; i < (n < 200000 ? n : 200000); ++i) EXPECT(items[4 * i + 2] <= items[4 * i + 3]);
    }
    /* validation failures return before any device work */
    EXPECT(fa_fwd(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == FA_ERR_PARAM_NULLPTR);
    EXPECT(fa_bwd(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                  NULL) == FA_ERR_PARAM_NULLPTR);
  }
  /* invalid configurations */
  cq[0] = ck[0] = 0;
  cq[1] = ck[1] = 5;
  base_config(&c, cq, ck, 1);
  c.head_dim = 100;
  EXPECT(fa_fwd_workspace_size(&c, &bytes) == FA_ERR_PARAM_INVALID);
  base_config(&c, cq, ck, 1);
  c.flags = 64;
  EXPECT(fa_fwd_workspace_size(&c, &bytes) == FA_ERR_PARAM_INVALID);
  EXPECT(fa_fwd_workspace_size(NULL, &bytes) == FA_ERR_PARAM_NULLPTR);
  for (int s = -2; s < 200000; s += 40000) EXPECT(fa_status_string(s) != NULL);
  /* decode planning */
  int64_t lens[300];
  for (int trial = 0; trial < 100; ++trial) {
    fa_decode_config d;
    memset(&d, 0, sizeof(d));
    d.batch = 1 + next_rand() % 300;
    d.max_seq_len = 1 + next_rand() % 20000;
    for (int64_t i = 0; i < d.batch; ++i) lens[i] = next_rand() % (d.max_seq_len + 1);
    d.actual_seq_lengths = lens;
    d.num_heads = 64;
    d.num_kv_heads = 1 << (next_rand() % 7);
    d.head_dim = trial % 2 ? 128 : 64;
    d.dtype = FA_DTYPE_BF16;
    d.layout = FA_LAYOUT_BSH + trial % 3;
    d.scale = 0.1;
    EXPECT(fa_decode_workspace_size(&d, &bytes) == FA_OK && bytes >= 256);
    EXPECT(fa_decode(&d, NULL, NULL, NULL, NULL, NULL, 0, NULL) == FA_ERR_PARAM_NULLPTR);
  }
  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("host checks passed\n");
  return failures ? 1 : 0;
}
