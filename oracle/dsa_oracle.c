/*
 * dsa_oracle.c -- plain, slow CPU oracle (float64) for one DSA decode unit.
 *
 * TEST INFRASTRUCTURE ONLY (see dsa_oracle.h).  Written for readability: every
 * step is a direct loop over its definition, in the order the method takes it.
 * OpenMP only splits independent outer loops (positions, heads); it changes no
 * arithmetic.
 *
 * Page cited throughout: "From 1M total to 15+ streams x 1M: the capacity
 * breakthrough of GLM-5.3 KV cache offload" (zhuai.tech), referred to below as
 * "the offload page", with its section headings translated.
 */
#include "dsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

struct orc_unit {
  orc_config c;
  int64_t row_bytes;
  int64_t ring_cap;       /* ring_rows + max_query_rows */
  /* logical state */
  int64_t L;              /* rows appended */
  int64_t M;              /* rows in the mirror; [M, L) live in the ring */
  int64_t round;          /* decode steps done */
  int64_t hand;           /* replacement ring hand */
  int64_t rb_floor;       /* lowest row count a rollback may return to */
  /* storage */
  float* keys;            /* [max_positions][index_dim], exact bf16 values */
  uint8_t* mirror;        /* offload: host mirror; resident: the row store */
  uint8_t* ring;          /* [ring_cap][row_bytes] */
  uint8_t* slots;         /* [S][row_bytes] */
  int32_t* slot_pos;      /* [S], -1 = empty */
  int32_t* fill_round;    /* [S] */
  int32_t* pin_round;     /* [S] */
  uint8_t* ref;           /* [S] reference bits (CLOCK) */
  int32_t* pos_slot;      /* [max_positions], -1 = not cached */
  /* last step */
  int32_t last_R;
  float* scores;          /* [R_max][max_positions] */
  int32_t* sel;           /* [R_max][K] */
  int32_t* sel_n;         /* [R_max] */
  int32_t* uni;           /* [R_max*K] */
  int32_t* kind;          /* [R_max*K] */
  int32_t* src;           /* [R_max*K] */
  int32_t n_union;
  int32_t* map;           /* [R_max][K] */
  uint8_t* compact;       /* [R_max*K][row_bytes] */
  int64_t cnt[ORC_CNT__N];
};

/* ---------------------------------------------------------------- numbers */

/* bf16 is the upper half of an IEEE binary32. */
static double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);                 /* subnormal: m * 2^-14 * 2^-10 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return sign ? -v : v;
}

static float canon_f32(double s) {
  float f = (float)s;
  return f == 0.0f ? 0.0f : f;                 /* -0 and +0 are one score */
}

/* ---------------------------------------------------------------- lifecycle */

int64_t orc_row_bytes(const orc_unit* u) { return u->row_bytes; }

orc_unit* orc_create(const orc_config* cfg, int* status) {
  const orc_config* c = cfg;
  *status = ORC_E_INVALID;
  if (!c || c->max_positions <= 0 || c->index_heads <= 0 || c->index_dim <= 0 || c->heads <= 0 ||
      c->latent_dim <= 0 || c->rope_dim < 0 || c->group <= 0 || c->latent_dim % c->group ||
      c->top_k <= 0 || c->ring_rows <= 0 || c->max_query_rows <= 0 ||
      (c->mode != ORC_MODE_OFFLOAD && c->mode != ORC_MODE_RESIDENT) ||
      (c->mode == ORC_MODE_OFFLOAD && c->hot_slots <= 0) ||
      (c->replacement != ORC_REPL_RING && c->replacement != ORC_REPL_CLOCK))
    return NULL;
  orc_unit* u = (orc_unit*)calloc(1, sizeof(orc_unit));
  if (!u) { *status = ORC_E_NOMEM; return NULL; }
  u->c = *c;
  /* Q8G64 row: int8 latent, one fp16 scale per group, bf16 RoPE (offload page,
   * "Starting point": 512 B + 16 B + 128 B = 656 B). */
  u->row_bytes = (int64_t)c->latent_dim + 2 * (c->latent_dim / c->group) + 2 * (int64_t)c->rope_dim;
  u->ring_cap = (int64_t)c->ring_rows + c->max_query_rows;
  int64_t P = c->max_positions, S = c->mode == ORC_MODE_OFFLOAD ? c->hot_slots : 0;
  int64_t RK = (int64_t)c->max_query_rows * c->top_k;
  u->keys = (float*)malloc((size_t)(P * c->index_dim) * sizeof(float));
  u->mirror = (uint8_t*)malloc((size_t)(P * u->row_bytes));
  u->ring = (uint8_t*)malloc((size_t)(u->ring_cap * u->row_bytes));
  u->slots = (uint8_t*)malloc((size_t)((S ? S : 1) * u->row_bytes));
  u->slot_pos = (int32_t*)malloc((size_t)(S ? S : 1) * sizeof(int32_t));
  u->fill_round = (int32_t*)malloc((size_t)(S ? S : 1) * sizeof(int32_t));
  u->pin_round = (int32_t*)malloc((size_t)(S ? S : 1) * sizeof(int32_t));
  u->ref = (uint8_t*)calloc((size_t)(S ? S : 1), 1);
  u->pos_slot = (int32_t*)malloc((size_t)P * sizeof(int32_t));
  u->scores = (float*)calloc((size_t)(c->max_query_rows * P), sizeof(float));
  u->sel = (int32_t*)malloc((size_t)RK * sizeof(int32_t));
  u->sel_n = (int32_t*)calloc((size_t)c->max_query_rows, sizeof(int32_t));
  u->uni = (int32_t*)malloc((size_t)RK * sizeof(int32_t));
  u->kind = (int32_t*)malloc((size_t)RK * sizeof(int32_t));
  u->src = (int32_t*)malloc((size_t)RK * sizeof(int32_t));
  u->map = (int32_t*)malloc((size_t)RK * sizeof(int32_t));
  u->compact = (uint8_t*)malloc((size_t)(RK * u->row_bytes));
  if (!u->keys || !u->mirror || !u->ring || !u->slots || !u->slot_pos || !u->fill_round ||
      !u->pin_round || !u->ref || !u->pos_slot || !u->scores || !u->sel || !u->sel_n || !u->uni ||
      !u->kind || !u->src || !u->map || !u->compact) {
    orc_destroy(u);
    *status = ORC_E_NOMEM;
    return NULL;
  }
  for (int64_t p = 0; p < P; p++) u->pos_slot[p] = -1;
  for (int64_t v = 0; v < S; v++) { u->slot_pos[v] = -1; u->fill_round[v] = -1; u->pin_round[v] = -1; }
  for (int64_t i = 0; i < RK; i++) { u->sel[i] = -1; u->map[i] = -1; }
  *status = ORC_OK;
  return u;
}

void orc_destroy(orc_unit* u) {
  if (!u) return;
  free(u->keys); free(u->mirror); free(u->ring); free(u->slots); free(u->slot_pos);
  free(u->fill_round); free(u->pin_round); free(u->ref); free(u->pos_slot); free(u->scores); free(u->sel);
  free(u->sel_n); free(u->uni); free(u->kind); free(u->src); free(u->map); free(u->compact);
  free(u);
}

/* ---------------------------------------------------------------- append / writeback */

static uint8_t* ring_row(orc_unit* u, int64_t pos) { return u->ring + (pos % u->ring_cap) * u->row_bytes; }

/* Append: new index keys go to the key store; new MLA rows enter the recent
 * ring (offload page, "Decision 3" data-flow figure).  The ring holds at most
 * ring_cap rows; when an append would overflow it, whole 64-row batches of the
 * oldest rows are written to the mirror first ("Decision 2": batched
 * writeback every 64 rows).  Resident mode stores rows directly. */
int orc_append(orc_unit* u, int64_t n, const uint16_t* keys, const uint8_t* rows) {
  const orc_config* c = &u->c;
  if (n < 0 || (n > 0 && (!keys || !rows))) return ORC_E_INVALID;
  if (u->L + n > c->max_positions) return ORC_E_CAPACITY;
  for (int64_t i = 0; i < n; i++)
    for (int d = 0; d < c->index_dim; d++)
      u->keys[(u->L + i) * c->index_dim + d] = (float)bf16_to_f64(keys[i * c->index_dim + d]);
  if (c->mode == ORC_MODE_RESIDENT) {
    memcpy(u->mirror + u->L * u->row_bytes, rows, (size_t)(n * u->row_bytes));
    u->L += n;
    u->M = u->L;
    return ORC_OK;
  }
  int64_t newM = u->M;
  while (u->L + n - newM > u->ring_cap) newM += c->ring_rows;
  for (int64_t p = u->M; p < newM; p++) {
    const uint8_t* from = p < u->L ? ring_row(u, p) : rows + (p - u->L) * u->row_bytes;
    memcpy(u->mirror + p * u->row_bytes, from, (size_t)u->row_bytes);
  }
  for (int64_t p = (newM > u->L ? newM : u->L); p < u->L + n; p++)
    memcpy(ring_row(u, p), rows + (p - u->L) * u->row_bytes, (size_t)u->row_bytes);
  u->M = newM;
  u->L += n;
  return ORC_OK;
}

/* Before the full history is exported or restored, every pending ring row is
 * written back so the host row count equals the logical row count (offload
 * page, "Capacity must survive the session lifecycle"). */
int orc_flush(orc_unit* u) {
  if (u->c.mode == ORC_MODE_RESIDENT) return ORC_OK;
  for (int64_t p = u->M; p < u->L; p++)
    memcpy(u->mirror + p * u->row_bytes, ring_row(u, p), (size_t)u->row_bytes);
  u->M = u->L;
  return ORC_OK;
}

/* Rollback after a rejected verify (offload page, "Capacity must survive the
 * session lifecycle": rejected drafts are rolled back, and the KV rows and the
 * DSA selection state have to return to the accepted prefix).  The last n rows
 * stop being part of the history: L becomes L-n and the mirror count M is cut
 * to at most L-n; rows still in the ring simply become free ring entries.
 * Offload mode allows this only down to `floor`, the mirror count when the
 * latest decode round started (or L at the latest warm): rows at or above it
 * were classified RING in every round that saw them, so no hot slot holds
 * one and the slot table needs no change.  The round count, the hand and the
 * slots are left as they are; fills made by the rejected round hold rows below
 * the floor and stay valid. */
int orc_rollback(orc_unit* u, int64_t n) {
  if (n < 0) return ORC_E_INVALID;
  if (n > u->L) return ORC_E_STATE;
  const int64_t L2 = u->L - n;
  if (u->c.mode == ORC_MODE_OFFLOAD && L2 < u->rb_floor) return ORC_E_STATE;
  u->L = L2;
  if (u->M > L2) u->M = L2;
  return ORC_OK;
}

/* Warm start: the hot cache holds the most recent min(S, L) positions, slot v
 * holding the v-th of them in ascending order; no slot counts as filled or
 * pinned in any round >= 0; the hand points past the last filled slot.  Under
 * CLOCK every filled slot starts with its reference bit set (a freshly loaded
 * entry counts as referenced), which is the full-cache, all-bits-set state of
 * the page's replacement probe. */
int orc_warm(orc_unit* u) {
  const orc_config* c = &u->c;
  if (c->mode == ORC_MODE_RESIDENT) return ORC_OK;
  if (u->M != u->L) return ORC_E_STATE;
  int64_t S = c->hot_slots;
  for (int64_t v = 0; v < S; v++) {
    if (u->slot_pos[v] >= 0) u->pos_slot[u->slot_pos[v]] = -1;
    u->slot_pos[v] = -1;
    u->fill_round[v] = -1;
    u->pin_round[v] = -1;
    u->ref[v] = 0;
  }
  int64_t n = u->L < S ? u->L : S;
  for (int64_t v = 0; v < n; v++) {
    int64_t pos = u->L - n + v;
    u->slot_pos[v] = (int32_t)pos;
    u->ref[v] = c->replacement == ORC_REPL_CLOCK;
    u->pos_slot[pos] = (int32_t)v;
    memcpy(u->slots + v * u->row_bytes, u->mirror + pos * u->row_bytes, (size_t)u->row_bytes);
  }
  u->hand = n % S;
  u->rb_floor = u->L;
  return ORC_OK;
}

/* End of a step: once a full batch of ring_rows rows is pending, it is written
 * back to the mirror in one batch (offload page, "Decision 2"). */
static void writeback_batch(orc_unit* u) {
  if (u->c.mode == ORC_MODE_RESIDENT) return;
  if (u->L - u->M < u->c.ring_rows) return;
  for (int64_t p = u->M; p < u->M + u->c.ring_rows; p++)
    memcpy(u->mirror + p * u->row_bytes, ring_row(u, p), (size_t)u->row_bytes);
  u->M += u->c.ring_rows;
}

/* ---------------------------------------------------------------- decode step */

typedef struct { float s; int32_t t; } scored;

/* Total order used for selection: higher score first, then lower position. */
static int by_score_then_position(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->t > y->t) - (x->t < y->t);
}

static int ascending_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Indexer score of every visible position for one query row:
 *   score(t) = sum_h w_h * max(0, q_h . k_t),
 * a learned indexer that scans the whole history so that only the top
 * positions reach attention (offload page, "Starting point"). */
static void index_scores(const orc_unit* u, const uint16_t* q, const float* w, int64_t n_vis, float* out) {
  const orc_config* c = &u->c;
  const int HI = c->index_heads, D = c->index_dim;
  double* qd = (double*)malloc((size_t)HI * D * sizeof(double));
  for (int i = 0; i < HI * D; i++) qd[i] = bf16_to_f64(q[i]);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_vis; t++) {
    const float* k = u->keys + t * D;
    double s = 0.0;
    for (int h = 0; h < HI; h++) {
      double dot = 0.0;
      for (int d = 0; d < D; d++) dot += qd[h * D + d] * (double)k[d];
      s += (double)w[h] * (dot > 0.0 ? dot : 0.0);
    }
    out[t] = canon_f32(s);
  }
  free(qd);
}

/* Exact Top-K by (score desc, position asc); the kept positions are returned
 * in ascending position order.  Fewer than K visible: all of them. */
static int32_t select_top_k(const float* s, int64_t n_vis, int32_t K, int32_t* sel) {
  scored* all = (scored*)malloc((size_t)n_vis * sizeof(scored));
  for (int64_t t = 0; t < n_vis; t++) { all[t].s = s[t]; all[t].t = (int32_t)t; }
  qsort(all, (size_t)n_vis, sizeof(scored), by_score_then_position);
  int32_t n = n_vis < K ? (int32_t)n_vis : K;
  for (int32_t j = 0; j < n; j++) sel[j] = all[j].t;
  qsort(sel, (size_t)n, sizeof(int32_t), ascending_i32);
  free(all);
  return n;
}

/* Absorbed-MLA attention of one query row over its selected rows:
 *   c_j[d]  = int8_j[d] * scale_j[d / group]           (symmetric dequantisation)
 *   l_j     = softmax_scale * (q_lat . c_j + q_rope . rho_j)
 *   out[d]  = sum_j softmax(l)_j * c_j[d]
 * Values are the dequantised latent itself (absorbed form). */
static void attend(const orc_unit* u, const uint16_t* q_lat, const uint16_t* q_rope,
                   const int32_t* rows_idx, int32_t n, float* out) {
  const orc_config* c = &u->c;
  const int H = c->heads, DL = c->latent_dim, DR = c->rope_dim, G = c->group;
  const int NG = DL / G;
  double* cj = (double*)malloc((size_t)n * DL * sizeof(double));
  double* rho = (double*)malloc((size_t)n * (DR ? DR : 1) * sizeof(double));
  for (int32_t j = 0; j < n; j++) {
    const uint8_t* b = u->compact + (int64_t)rows_idx[j] * u->row_bytes;
    for (int d = 0; d < DL; d++) {
      int g = d / G;
      uint16_t sc = (uint16_t)(b[DL + 2 * g] | (b[DL + 2 * g + 1] << 8));
      cj[(int64_t)j * DL + d] = (double)(int8_t)b[d] * f16_to_f64(sc);
    }
    for (int e = 0; e < DR; e++) {
      const uint8_t* r = b + DL + 2 * NG + 2 * e;
      rho[(int64_t)j * DR + e] = bf16_to_f64((uint16_t)(r[0] | (r[1] << 8)));
    }
  }
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H; h++) {
    double* logit = (double*)malloc((size_t)(n ? n : 1) * sizeof(double));
    double mx = -INFINITY;
    for (int32_t j = 0; j < n; j++) {
      double a = 0.0;
      for (int d = 0; d < DL; d++) a += bf16_to_f64(q_lat[h * DL + d]) * cj[(int64_t)j * DL + d];
      for (int e = 0; e < DR; e++) a += bf16_to_f64(q_rope[h * DR + e]) * rho[(int64_t)j * DR + e];
      logit[j] = c->softmax_scale * a;
      if (logit[j] > mx) mx = logit[j];
    }
    double z = 0.0;
    for (int32_t j = 0; j < n; j++) { logit[j] = exp(logit[j] - mx); z += logit[j]; }
    for (int d = 0; d < DL; d++) {
      double o = 0.0;
      for (int32_t j = 0; j < n; j++) o += logit[j] * cj[(int64_t)j * DL + d];
      out[h * DL + d] = (float)(n ? o / z : 0.0);
    }
    free(logit);
  }
  free(cj);
  free(rho);
}

/* Steps 4-10 of a round, on the selections in u->sel / u->sel_n: union,
 * classification, pins, replacement, compact rows, attention (skipped when
 * out is NULL) and the batched writeback; the round counter advances. */
static int run_round(orc_unit* u, int32_t R, const uint16_t* q_lat, const uint16_t* q_rope, float* out) {
  const orc_config* c = &u->c;
  const int32_t K = c->top_k;
  const int64_t rb = u->row_bytes;
  const int32_t r = (int32_t)u->round;
  if (c->mode == ORC_MODE_OFFLOAD) u->rb_floor = u->M;
  u->last_R = R;
  memset(u->cnt, 0, sizeof(u->cnt));

  /* 4. Union of the rows' selections, ascending; one entry per distinct
   *    position, so a position several rows select is read once. */
  int32_t total = 0;
  for (int32_t i = 0; i < R; i++)
    for (int32_t j = 0; j < u->sel_n[i]; j++) u->uni[total++] = u->sel[(int64_t)i * K + j];
  qsort(u->uni, (size_t)total, sizeof(int32_t), ascending_i32);
  int32_t U = 0;
  for (int32_t x = 0; x < total; x++)
    if (U == 0 || u->uni[U - 1] != u->uni[x]) u->uni[U++] = u->uni[x];
  u->n_union = U;
  for (int32_t i = 0; i < R; i++)
    for (int32_t j = 0; j < K; j++) {
      int32_t pos = u->sel[(int64_t)i * K + j];
      int32_t* hit = pos < 0 ? NULL : (int32_t*)bsearch(&pos, u->uni, (size_t)U, sizeof(int32_t), ascending_i32);
      u->map[(int64_t)i * K + j] = hit ? (int32_t)(hit - u->uni) : -1;
    }
  u->cnt[ORC_CNT_UNION] = U;

  if (c->mode == ORC_MODE_RESIDENT) {
    for (int32_t x = 0; x < U; x++) {
      u->kind[x] = ORC_SRC_RES;
      u->src[x] = u->uni[x];
      memcpy(u->compact + x * rb, u->mirror + (int64_t)u->uni[x] * rb, (size_t)rb);
    }
    u->cnt[ORC_CNT_RES] = U;
  } else {
    const int64_t S = c->hot_slots;
    /* 5. Classify every union entry against the state at the start of the
     *    round: rows not yet written back are served by the recent ring; a
     *    slot counts as a hit only if it was filled in an earlier round
     *    (offload page, "GPU cache management errs too"). */
    for (int32_t x = 0; x < U; x++) {
      int32_t pos = u->uni[x];
      int32_t v = u->pos_slot[pos];
      if (pos >= u->M) { u->kind[x] = ORC_SRC_RING; u->src[x] = (int32_t)(pos % u->ring_cap); }
      else if (v >= 0 && u->fill_round[v] < r) { u->kind[x] = ORC_SRC_HIT; u->src[x] = v; }
      else { u->kind[x] = ORC_SRC_MISS; u->src[x] = pos; }
    }
    /* 6. Pin every slot this round reads (CLOCK: and mark it referenced). */
    const int clock = c->replacement == ORC_REPL_CLOCK;
    for (int32_t x = 0; x < U; x++)
      if (u->kind[x] == ORC_SRC_HIT) {
        u->pin_round[u->src[x]] = r;
        if (clock) u->ref[u->src[x]] = 1;
      }
    /* 7. Replacement: misses, in ascending position order, take slots found by
     *    a hand that walks the slots in ring order and never takes a slot
     *    pinned this round.  A miss that finds no slot is read from host memory
     *    without being cached.  Every miss's bytes come from the host mirror in
     *    this round, never from the slot just filled.
     *    Ring policy: the next unpinned slot; the walk visits each slot at most
     *    once per round.
     *    CLOCK policy (second chance): an unpinned slot whose reference bit is
     *    set loses the bit and is passed over; one whose bit is clear is taken
     *    (and, being filled, is marked referenced); the walk visits each slot at
     *    most twice per round.  With every bit set and few misses, the hand
     *    clears a whole lap before it takes anything: the long sweep the page
     *    measured. */
    const int64_t max_visits = clock ? 2 * S : S;
    int64_t walk = u->hand, visited = 0, last = -1;
    for (int32_t x = 0; x < U; x++) {
      if (u->kind[x] != ORC_SRC_MISS) continue;
      int found = 0;
      while (visited < max_visits) {
        if (u->pin_round[walk] == r) { walk = (walk + 1) % S; visited++; continue; }
        if (clock && u->ref[walk]) { u->ref[walk] = 0; walk = (walk + 1) % S; visited++; continue; }
        found = 1;
        break;
      }
      if (!found) { u->kind[x] = ORC_SRC_MISS_NOSLOT; continue; }
      int32_t v = (int32_t)walk, pos = u->uni[x];
      if (u->slot_pos[v] >= 0) { u->pos_slot[u->slot_pos[v]] = -1; u->cnt[ORC_CNT_EVICT]++; }
      u->slot_pos[v] = pos;
      u->pos_slot[pos] = v;
      u->fill_round[v] = r;
      u->pin_round[v] = r;
      if (clock) u->ref[v] = 1;
      memcpy(u->slots + (int64_t)v * rb, u->mirror + (int64_t)pos * rb, (size_t)rb);
      last = v;
      walk = (walk + 1) % S;
      visited++;
    }
    if (last >= 0) u->hand = (last + 1) % S;
    /* 8. Compact selection: the bytes of every union entry from its source. */
    for (int32_t x = 0; x < U; x++) {
      const uint8_t* from;
      switch (u->kind[x]) {
        case ORC_SRC_HIT: from = u->slots + (int64_t)u->src[x] * rb; u->cnt[ORC_CNT_HIT]++; break;
        case ORC_SRC_RING: from = ring_row(u, u->uni[x]); u->cnt[ORC_CNT_RING]++; break;
        case ORC_SRC_MISS: from = u->mirror + (int64_t)u->uni[x] * rb; u->cnt[ORC_CNT_MISS]++; break;
        default: from = u->mirror + (int64_t)u->uni[x] * rb; u->cnt[ORC_CNT_MISS_NOSLOT]++; break;
      }
      memcpy(u->compact + x * rb, from, (size_t)rb);
    }
    u->cnt[ORC_CNT_HOST_BYTES] = (u->cnt[ORC_CNT_MISS] + u->cnt[ORC_CNT_MISS_NOSLOT]) * rb;
    /* Rows read from host memory: with attention, each query row reads every
     * selected position of its own that missed; a prefetch round (no attention)
     * reads each miss that took a slot once, to fill the slot. */
    if (out) {
      for (int32_t i = 0; i < R; i++)
        for (int32_t j = 0; j < u->sel_n[i]; j++) {
          const int32_t x = u->map[(int64_t)i * K + j];
          if (x >= 0 && (u->kind[x] == ORC_SRC_MISS || u->kind[x] == ORC_SRC_MISS_NOSLOT)) u->cnt[ORC_CNT_HOST_READS]++;
        }
    } else {
      u->cnt[ORC_CNT_HOST_READS] = u->cnt[ORC_CNT_MISS];
    }
  }

  /* 9. Attention of each query row over its own selection. */
  for (int32_t i = 0; out && i < R; i++)
    attend(u, q_lat + (int64_t)i * c->heads * c->latent_dim,
           q_rope ? q_rope + (int64_t)i * c->heads * c->rope_dim : NULL,
           u->map + (int64_t)i * K, u->sel_n[i], out + (int64_t)i * c->heads * c->latent_dim);

  /* 10. Batched writeback of the recent ring. */
  writeback_batch(u);
  u->round++;
  return ORC_OK;
}

int orc_decode_step(orc_unit* u, int32_t R, const uint16_t* index_q, const float* index_w,
                    const uint16_t* q_lat, const uint16_t* q_rope, float* out) {
  const orc_config* c = &u->c;
  const int32_t K = c->top_k;
  if (R <= 0 || R > c->max_query_rows || !index_q || !index_w || !q_lat || !out ||
      (c->rope_dim > 0 && !q_rope))
    return ORC_E_INVALID;
  if (u->L < R) return ORC_E_STATE;

  /* 1. Visibility: the i-th query row sits at position L-R+i and sees every
   *    position up to and including its own. */
  for (int32_t i = 0; i < R; i++) {
    int64_t n_vis = u->L - R + i + 1;
    float* s = u->scores + (int64_t)i * c->max_positions;
    memset(s, 0, (size_t)u->L * sizeof(float));
    /* 2. Score every visible position. */
    index_scores(u, index_q + (int64_t)i * c->index_heads * c->index_dim,
                 index_w + (int64_t)i * c->index_heads, n_vis, s);
    /* 3. Exact Top-K. */
    for (int32_t j = 0; j < K; j++) u->sel[(int64_t)i * K + j] = -1;
    u->sel_n[i] = select_top_k(s, n_vis, K, u->sel + (int64_t)i * K);
  }

  return run_round(u, R, q_lat, q_rope, out);
}

/* Selection reuse (offload page, "Starting point": some later layers reuse the
 * selection, while each layer keeps its own KV rows).  The given selection of
 * R query rows replaces scoring and Top-K: row i lists sel_n[i] <= K positions,
 * strictly ascending, each visible to it (at most L-R+i).  Nothing changes on
 * an error. */
static int set_selection(orc_unit* u, int32_t R, const int32_t* sel, const int32_t* sel_n) {
  const orc_config* c = &u->c;
  const int32_t K = c->top_k;
  if (R <= 0 || R > c->max_query_rows || !sel || !sel_n) return ORC_E_INVALID;
  if (u->L < R) return ORC_E_STATE;
  for (int32_t i = 0; i < R; i++) {
    if (sel_n[i] < 0 || sel_n[i] > K) return ORC_E_INVALID;
    for (int32_t j = 0; j < sel_n[i]; j++) {
      int32_t p = sel[(int64_t)i * K + j];
      if (p < 0 || p > u->L - R + i || (j > 0 && p <= sel[(int64_t)i * K + j - 1])) return ORC_E_INVALID;
    }
  }
  for (int32_t i = 0; i < R; i++) {
    u->sel_n[i] = sel_n[i];
    for (int32_t j = 0; j < K; j++) u->sel[(int64_t)i * K + j] = j < sel_n[i] ? sel[(int64_t)i * K + j] : -1;
  }
  return ORC_OK;
}

int orc_decode_step_sel(orc_unit* u, int32_t R, const int32_t* sel, const int32_t* sel_n,
                        const uint16_t* q_lat, const uint16_t* q_rope, float* out) {
  if (!q_lat || !out || (u->c.rope_dim > 0 && !q_rope)) return ORC_E_INVALID;
  int st = set_selection(u, R, sel, sel_n);
  if (st != ORC_OK) return st;
  return run_round(u, R, q_lat, q_rope, out);
}

/* Prefetch with a known selection (offload page, first decision: once the
 * selection is known, the rows of layers that reuse it could be moved early,
 * overlapping other work, though not for free).  Read here as one round of the
 * unit's cache without attention: the selection is classified and its misses
 * take slots and are filled from the host mirror exactly as in a decode round,
 * so the unit's next round finds them as hits.  Resident mode: nothing to do. */
int orc_prefetch_sel(orc_unit* u, int32_t R, const int32_t* sel, const int32_t* sel_n) {
  if (u->c.mode == ORC_MODE_RESIDENT) return ORC_OK;
  int st = set_selection(u, R, sel, sel_n);
  if (st != ORC_OK) return st;
  return run_round(u, R, NULL, NULL, NULL);
}

/* ---------------------------------------------------------------- getters */

void orc_get_state(const orc_unit* u, int64_t state[7]) {
  state[0] = u->L; state[1] = u->M; state[2] = u->round; state[3] = u->hand;
  state[4] = u->last_R; state[5] = u->n_union; state[6] = u->rb_floor;
}

void orc_get_scores(const orc_unit* u, float* dst) {
  for (int32_t i = 0; i < u->last_R; i++)
    memcpy(dst + (int64_t)i * u->L, u->scores + (int64_t)i * u->c.max_positions, (size_t)u->L * sizeof(float));
}

void orc_get_selection(const orc_unit* u, int32_t* sel, int32_t* counts) {
  memcpy(sel, u->sel, (size_t)u->last_R * u->c.top_k * sizeof(int32_t));
  memcpy(counts, u->sel_n, (size_t)u->last_R * sizeof(int32_t));
}

void orc_get_union(const orc_unit* u, int32_t* uni, int32_t* kind, int32_t* src) {
  memcpy(uni, u->uni, (size_t)u->n_union * sizeof(int32_t));
  memcpy(kind, u->kind, (size_t)u->n_union * sizeof(int32_t));
  memcpy(src, u->src, (size_t)u->n_union * sizeof(int32_t));
}

void orc_get_map(const orc_unit* u, int32_t* map) {
  memcpy(map, u->map, (size_t)u->last_R * u->c.top_k * sizeof(int32_t));
}

void orc_get_compact(const orc_unit* u, uint8_t* dst) {
  memcpy(dst, u->compact, (size_t)(u->n_union * u->row_bytes));
}

void orc_get_counters(const orc_unit* u, int64_t cnt[ORC_CNT__N]) { memcpy(cnt, u->cnt, sizeof(u->cnt)); }

void orc_get_slots(const orc_unit* u, int32_t* slot_pos, int32_t* fill_round, int32_t* pin_round) {
  int64_t S = u->c.mode == ORC_MODE_OFFLOAD ? u->c.hot_slots : 0;
  memcpy(slot_pos, u->slot_pos, (size_t)S * sizeof(int32_t));
  memcpy(fill_round, u->fill_round, (size_t)S * sizeof(int32_t));
  memcpy(pin_round, u->pin_round, (size_t)S * sizeof(int32_t));
}

void orc_get_ref(const orc_unit* u, uint8_t* ref) {
  if (u->c.mode == ORC_MODE_OFFLOAD) memcpy(ref, u->ref, (size_t)u->c.hot_slots);
}

void orc_get_pos_slot(const orc_unit* u, int32_t* pos_slot) {
  memcpy(pos_slot, u->pos_slot, (size_t)u->L * sizeof(int32_t));
}

void orc_get_slot_bytes(const orc_unit* u, uint8_t* dst) {
  int64_t S = u->c.mode == ORC_MODE_OFFLOAD ? u->c.hot_slots : 0;
  memcpy(dst, u->slots, (size_t)(S * u->row_bytes));
}

int orc_get_mirror(const orc_unit* u, int64_t first, int64_t n, uint8_t* dst) {
  if (first < 0 || n < 0 || first + n > u->M) return ORC_E_INVALID;
  memcpy(dst, u->mirror + first * u->row_bytes, (size_t)(n * u->row_bytes));
  return ORC_OK;
}
