/* Plain C99 client of duo_attn.h: the header compiles as C and the host-only
 * entry points behave as documented (no GPU is touched). Exit status 0 on
 * success; prints the first failed check otherwise. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "duo_attn.h"

#define CHECK(c) do { if (!(c)) { printf("check failed at line %d: %s (%s)\n", __LINE__, #c, duo_last_error()); return 1; } } while (0)

int main(void) {
  const uint8_t mask[8] = {0, 1, 0, 0, 1, 0, 0, 0};
  duo_layer L;
  memset(&L, 0, sizeof L);
  L.num_q_heads = 48; L.num_kv_heads = 8; L.head_dim = 128; L.kind = DUO_LAYER_FULL;
  L.window = 0; L.sink = 64; L.recent = 256; L.full_attention_heads = mask; L.scale = 0.f;

  CHECK(duo_attn_version() == DUO_ATTN_VERSION);
  CHECK(duo_prefill_tile_rows(&L) == 64);  /* group 6: two heads per workgroup */
  CHECK(duo_prefill_tile_rows(NULL) == DUO_ERR_INVALID_ARG);

  /* head plan: full heads 1 and 4 ranked 0, 1; the rest streaming, ranked in order */
  int32_t cls[8], rank[8], nm = -1, ns = -1;
  CHECK(duo_head_plan(&L, cls, rank, &nm, &ns) == DUO_OK);
  CHECK(nm == 2 && ns == 6);
  CHECK(cls[1] == 0 && rank[1] == 0 && cls[4] == 0 && rank[4] == 1);
  CHECK(cls[0] == 1 && rank[0] == 0 && cls[7] == 1 && rank[7] == 5);

  /* static cache bytes: one of k/v per class */
  int64_t mb = 0, sb = 0;
  CHECK(duo_kv_cache_bytes(&L, 2, 1000, &mb, &sb) == DUO_OK);
  CHECK(mb == (int64_t)2 * 2 * 1000 * 128 * 2);
  CHECK(sb == (int64_t)2 * 6 * (64 + 256) * 128 * 2);

  /* cache report for lengths 10 and 5000 */
  const int32_t lens[2] = {10, 5000};
  duo_cache_report rep;
  CHECK(duo_kv_cache_report(&L, 2, 5000, lens, &rep) == DUO_OK);
  CHECK(rep.main_active == 2 * (10 + 5000));
  CHECK(rep.stream_active == 6 * (10 + 320));
  CHECK(rep.base_active == 8 * (10 + 5000));

  /* rotary frequencies: plain RoPE theta 10000 */
  duo_rope r = {10000.f, 1.f, 0, 0.f, 0.f, 1.f};
  double f[64];
  CHECK(duo_rope_frequencies(&r, f) == DUO_OK);
  CHECK(f[0] == 1.0 && fabs(f[1] - pow(10000.0, -2.0 / 128)) < 1e-15);

  /* validation errors leave nothing launched and set a message */
  duo_layer bad = L;
  bad.head_dim = 64;
  CHECK(duo_head_plan(&bad, cls, rank, &nm, &ns) == DUO_ERR_UNSUPPORTED);
  CHECK(strlen(duo_last_error()) > 0);
  CHECK(duo_attn_decode_workspace_bytes(&bad, 4, 1000) == 0);
  CHECK(duo_attn_decode_workspace_bytes(&L, 4, 1000) > 0);
  CHECK(duo_attn_decode_block_workspace_bytes(&L, 4, 65, 1000) == 0); /* more than 64 tokens */
  r.theta = 1.f;
  CHECK(duo_rope_frequencies(&r, f) == DUO_ERR_INVALID_ARG);

  /* work plans: count, then fill (7 int32 per prefill item, 4 per decode item) */
  {
    int64_t n = 0;
    CHECK(duo_prefill_plan(&L, 2, 300, 0, 0, NULL, &n) == DUO_OK);
    CHECK(n > 0 && n < 100000);
    int32_t* items = (int32_t*)malloc((size_t)n * 7 * sizeof(int32_t));
    CHECK(items != NULL);
    CHECK(duo_prefill_plan(&L, 2, 300, 0, 0, items, &n) == DUO_OK);
    free(items);
    /* a chunk over a long past is cut into pieces when a workspace is given */
    CHECK(duo_attn_prefill_workspace_bytes(&L, 1, 8192, 8192 * 15) > 0);
    CHECK(duo_attn_prefill_workspace_bytes(&L, 4, 8192, 0) == 0);
    CHECK(duo_prefill_plan(&L, 1, 8192, 8192 * 15, 1, NULL, &n) == DUO_OK);
    items = (int32_t*)malloc((size_t)n * 7 * sizeof(int32_t));
    CHECK(items != NULL);
    CHECK(duo_prefill_plan(&L, 1, 8192, 8192 * 15, 1, items, &n) == DUO_OK);
    CHECK(items[5] > 1);
    free(items);
    int32_t split = 0;
    CHECK(duo_decode_plan(&L, 3, 70000, &split, NULL, &n) == DUO_OK);
    CHECK(split > 0 && n > 0);
    items = (int32_t*)malloc((size_t)n * 4 * sizeof(int32_t));
    CHECK(items != NULL);
    CHECK(duo_decode_plan(&L, 3, 70000, &split, items, &n) == DUO_OK);
    free(items);
  }

  /* launching calls refused on the host (bogus but aligned device addresses
   * are never dereferenced on these paths) */
  {
    void* d = (void*)(uintptr_t)0x100000;
    const int32_t* di = (const int32_t*)d;
    duo_kv_cache c;
    memset(&c, 0, sizeof c);
    c.k_main = c.v_main = c.k_stream = c.v_stream = d;
    c.main_capacity = 1000;
    CHECK(duo_attn_prefill(&bad, NULL, 1, d, d, d, 16, 0, d, NULL, NULL, 0, NULL, NULL, NULL) == DUO_ERR_UNSUPPORTED);
    CHECK(duo_attn_prefill(&L, NULL, 1, d, d, d, 16, 5, d, NULL, NULL, 0, NULL, NULL, NULL) == DUO_ERR_INVALID_ARG);
    CHECK(duo_attn_prefill(&L, &c, 1, d, d, d, 16, 2000, d, NULL, NULL, 0, NULL, NULL, NULL) == DUO_ERR_CAPACITY);
    CHECK(duo_kv_append(&L, &c, 1, d, d, 16, di, 3, NULL, NULL) == DUO_ERR_INVALID_ARG);
    CHECK(duo_kv_append(&L, &c, 1, d, d, 16, di, 5000, NULL, NULL) == DUO_ERR_CAPACITY);
    CHECK(duo_attn_decode(&L, &c, 4, d, di, 1000, d, NULL, d, 16, NULL, NULL, NULL) == DUO_ERR_WORKSPACE);
    CHECK(duo_attn_decode_block(&L, &c, 4, d, d, d, 65, di, 900, d, NULL, d, 1 << 20, NULL, NULL, NULL) == DUO_ERR_INVALID_ARG);
    duo_epilogue e = {NULL, d, 7};
    CHECK(duo_attn_prefill(&L, NULL, 1, d, d, d, 16, 0, d, NULL, NULL, 0, NULL, &e, NULL) == DUO_ERR_INVALID_ARG);
    duo_rope yr = {500000.f, 64.f, 4096, 64.f, 1.f, 1.f};
    duo_prologue pro = {NULL, -1.f, &yr};
    CHECK(duo_attn_prefill(&L, NULL, 1, d, d, d, 16, 0, d, NULL, NULL, 0, &pro, NULL, NULL) == DUO_ERR_INVALID_ARG);
    CHECK(strlen(duo_last_error()) > 0);
  }

  /* the device error word: a NULL output is refused before any device call */
  CHECK(duo_device_errors(NULL, 0) == DUO_ERR_INVALID_ARG);
  CHECK(DUO_DEVICE_APPEND_PAST_CAPACITY == 1u && DUO_DEVICE_LENGTH_PAST_CAPACITY == 2u &&
        DUO_DEVICE_LENGTH_PAST_PLAN == 4u);

  /* empty calls are no-ops */
  CHECK(duo_attn_prefill(&L, NULL, 0, NULL, NULL, NULL, 0, 0, NULL, NULL, NULL, 0, NULL, NULL, NULL) == DUO_OK);
  printf("ok\n");
  return 0;
}
