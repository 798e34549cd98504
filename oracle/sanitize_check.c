/*
 * sanitize_check.c -- drives every entry point of the CPU oracle on small
 * inputs, for a build under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitize.py builds it with gcc and runs it).
 *
 * TEST INFRASTRUCTURE ONLY, like the oracle itself.  Inputs come from a small
 * linear congruential generator: integer-valued bf16 index keys and queries in
 * [-8, 8], head weights in [0, 4], int8 latent bytes, fp16 scales near 0.01 and
 * small bf16 RoPE and query values.  The driver checks only what needs no
 * reference: every call returns the status its arguments call for, and the
 * getters fill their buffers.  Parity of the values is pinned elsewhere.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dsa_oracle.h"

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;

static uint32_t lcg(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg_state >> 33);
}

/* bf16 bits of a small integer (exact in bf16). */
static uint16_t bf16_int(int v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static uint16_t bf16_small(void) { /* a value in about [-0.06, 0.06] */
  float f = ((float)(int)(lcg() % 121) - 60.0f) / 1000.0f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      failures++;                                                     \
    }                                                                 \
  } while (0)

static void fill_rows(uint16_t* keys, uint8_t* rows, int64_t n, int D, int64_t rb) {
  for (int64_t i = 0; i < n; ++i) {
    for (int d = 0; d < D; ++d) keys[i * D + d] = bf16_int((int)(lcg() % 17) - 8);
    uint8_t* r = rows + i * rb;
    for (int d = 0; d < 512; ++d) r[d] = (uint8_t)((int)(lcg() % 255) - 127);
    for (int g = 0; g < 8; ++g) { /* fp16 0x2000 + small: about 0.008 .. 0.012 */
      const uint16_t h = (uint16_t)(0x2000 + lcg() % 256);
      r[512 + 2 * g] = (uint8_t)(h & 0xFF);
      r[512 + 2 * g + 1] = (uint8_t)(h >> 8);
    }
    for (int e = 0; e < 64; ++e) {
      const uint16_t b = bf16_small();
      r[528 + 2 * e] = (uint8_t)(b & 0xFF);
      r[528 + 2 * e + 1] = (uint8_t)(b >> 8);
    }
  }
}

static void run(int mode, int replacement) {
  orc_config c;
  memset(&c, 0, sizeof c);
  c.max_positions = 700;
  c.index_heads = 4;
  c.index_dim = 128;
  c.heads = 16;
  c.latent_dim = 512;
  c.rope_dim = 64;
  c.group = 64;
  c.top_k = 32;
  c.hot_slots = 24;
  c.ring_rows = 64;
  c.max_query_rows = 4;
  c.mode = mode;
  c.softmax_scale = 1.0 / 24.0;
  c.replacement = replacement;
  int st = -1;
  orc_unit* u = orc_create(&c, &st);
  EXPECT(u != NULL && st == ORC_OK);
  if (!u) return;
  const int64_t rb = orc_row_bytes(u);
  EXPECT(rb == 656);
  const int R = 4, K = c.top_k, H = c.heads, HI = c.index_heads, D = c.index_dim;

  const int64_t T = 300;
  uint16_t* keys = malloc(sizeof(uint16_t) * 700 * D);
  uint8_t* rows = malloc((size_t)700 * rb);
  fill_rows(keys, rows, 700, D, rb);
  EXPECT(orc_append(u, T, keys, rows) == ORC_OK);
  EXPECT(orc_flush(u) == ORC_OK);
  EXPECT(orc_warm(u) == ORC_OK);

  uint16_t* iq = malloc(sizeof(uint16_t) * R * HI * D);
  float* iw = malloc(sizeof(float) * R * HI);
  uint16_t* ql = malloc(sizeof(uint16_t) * R * H * 512);
  uint16_t* qr = malloc(sizeof(uint16_t) * R * H * 64);
  float* out = malloc(sizeof(float) * R * H * 512);
  int32_t* sel = malloc(sizeof(int32_t) * R * K);
  int32_t* sel_n = malloc(sizeof(int32_t) * R);
  int32_t* uni = malloc(sizeof(int32_t) * R * K);
  int32_t* kind = malloc(sizeof(int32_t) * R * K);
  int32_t* src = malloc(sizeof(int32_t) * R * K);
  int32_t* map = malloc(sizeof(int32_t) * R * K);
  uint8_t* compact = malloc((size_t)R * K * rb);
  int32_t* sp = malloc(sizeof(int32_t) * c.hot_slots * 3);
  uint8_t* ref = malloc((size_t)c.hot_slots);
  uint8_t* slot_bytes = malloc((size_t)c.hot_slots * rb);
  int32_t* pos_slot = malloc(sizeof(int32_t) * 700);
  float* scores = malloc(sizeof(float) * R * 700);
  uint8_t* mirror = malloc((size_t)700 * rb);
  int64_t state[7], cnt[ORC_CNT__N];

  int64_t L = T;
  for (int step = 0; step < 40; ++step) {
    EXPECT(orc_append(u, R, keys + L * D, rows + L * rb) == ORC_OK);
    L += R;
    for (int i = 0; i < R * HI * D; ++i) iq[i] = bf16_int((int)(lcg() % 17) - 8);
    for (int i = 0; i < R * HI; ++i) iw[i] = (float)(lcg() % 5);
    for (int i = 0; i < R * H * 512; ++i) ql[i] = bf16_small();
    for (int i = 0; i < R * H * 64; ++i) qr[i] = bf16_small();
    EXPECT(orc_decode_step(u, R, iq, iw, ql, qr, out) == ORC_OK);
    orc_get_state(u, state);
    EXPECT(state[0] == L);
    orc_get_scores(u, scores);
    orc_get_selection(u, sel, sel_n);
    orc_get_union(u, uni, kind, src);
    orc_get_map(u, map);
    orc_get_compact(u, compact);
    orc_get_counters(u, cnt);
    EXPECT(cnt[ORC_CNT_UNION] == state[5] && cnt[ORC_CNT_UNION] <= R * K);
    orc_get_slots(u, sp, sp + c.hot_slots, sp + 2 * c.hot_slots);
    orc_get_pos_slot(u, pos_slot);
    orc_get_ref(u, ref);
    orc_get_slot_bytes(u, slot_bytes);
    /* a round on the step's own selection, with and without attention */
    if (step % 5 == 1) EXPECT(orc_decode_step_sel(u, R, sel, sel_n, ql, qr, out) == ORC_OK);
    if (step % 5 == 3) EXPECT(orc_prefetch_sel(u, R, sel, sel_n) == ORC_OK);
    /* verify rollback of the step's rows (within the bound), then re-append them */
    if (step % 7 == 6) {
      EXPECT(orc_rollback(u, 2) == ORC_OK);
      L -= 2;
      EXPECT(orc_append(u, 2, keys + L * D, rows + L * rb) == ORC_OK);
      L += 2;
    }
  }
  /* refusals leave the unit unchanged */
  EXPECT(orc_rollback(u, -1) == ORC_E_INVALID);
  EXPECT(orc_rollback(u, L + 1) == ORC_E_STATE);
  EXPECT(orc_append(u, 700 - L + 1, keys, rows) == ORC_E_CAPACITY);
  EXPECT(orc_decode_step(u, R + 1, iq, iw, ql, qr, out) == ORC_E_INVALID);
  orc_get_state(u, state);
  EXPECT(state[0] == L);
  EXPECT(orc_flush(u) == ORC_OK);
  orc_get_state(u, state);
  EXPECT(orc_get_mirror(u, 0, state[1], mirror) == ORC_OK);
  EXPECT(memcmp(mirror, rows, (size_t)state[1] * rb) == 0);
  orc_destroy(u);
  free(keys); free(rows); free(iq); free(iw); free(ql); free(qr); free(out);
  free(sel); free(sel_n); free(uni); free(kind); free(src); free(map); free(compact);
  free(sp); free(ref); free(slot_bytes); free(pos_slot); free(scores); free(mirror);
}

int main(void) {
  run(ORC_MODE_OFFLOAD, ORC_REPL_RING);
  run(ORC_MODE_OFFLOAD, ORC_REPL_CLOCK);
  run(ORC_MODE_RESIDENT, ORC_REPL_RING);
  orc_destroy(NULL);
  int st = 0;
  orc_config bad;
  memset(&bad, 0, sizeof bad);
  EXPECT(orc_create(&bad, &st) == NULL && st != ORC_OK);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle entry points ran clean\n");
  return 0;
}
