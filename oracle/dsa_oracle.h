/*
 * dsa_oracle.h -- plain, slow CPU oracle for one DSA sparse-attention decode unit.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this; only the tests, the smoke check and the bench's CPU-baseline leg
 * use it.  It shares no code, header, table or constant with the HIP library.
 *
 * What it models (source: the page "From 1M total to 15+ streams x 1M: the
 * capacity breakthrough of GLM-5.3 KV cache offload", zhuai.tech):
 *   - one "unit" = one (layer, sequence) pair with its own index-key store,
 *     pinned-host mirror of Q8G64 MLA rows, recent ring and HBM hot cache
 *     (section "Starting point: separate capacity from the working set");
 *   - new rows enter a recent ring and are written back in 64-row batches
 *     (section "Decision 2: let the CPU manage the GPU hot cache first");
 *   - a decode step scores every visible position, takes the exact Top-K,
 *     resolves each selected position to a hot slot, the ring or the host
 *     mirror, pins the slots in use, fills free slots by a ring walk that skips
 *     pinned slots, and never serves a hit from a slot filled in the same round
 *     (sections "Decision 3: let the GPU manage the hot cache directly" and
 *     "GPU cache management errs too: cross-block visibility and long
 *     replacement sweeps");
 *   - absorbed-MLA attention over the selected rows only;
 *   - around the step: rollback of rejected verify rows (section "Capacity must
 *     survive the session lifecycle"), the CLOCK replacement variant with
 *     reference bits (the policy the ring walk replaced, in "GPU cache management
 *     errs too"), and rounds on a selection made by another layer, with or
 *     without attention -- selection reuse and prefetch (sections "Starting
 *     point" and the first decision).  Quantise-on-append lives in quantize.py.
 *
 * Arithmetic is float64 throughout; scores are reported as float32 with -0
 * canonicalised to +0, and the Top-K decision is taken on those float32 values.
 *
 * Parity pins (what this oracle is checked against, independent of itself)
 * are listed in the tests under tests/test_oracle_*.py.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_E_INVALID = 1, ORC_E_NOMEM = 2, ORC_E_CAPACITY = 3, ORC_E_STATE = 4 };
enum { ORC_MODE_OFFLOAD = 0, ORC_MODE_RESIDENT = 1 };
/* Replacement policy of the hot cache: the ring walk that skips pinned slots,
 * or CLOCK with reference bits (offload page, "GPU cache management errs too",
 * replacement paragraph: the earlier policy, kept as a variant). */
enum { ORC_REPL_RING = 0, ORC_REPL_CLOCK = 1 };
/* Where a selected row's bytes come from in one round. */
enum { ORC_SRC_HIT = 0, ORC_SRC_RING = 1, ORC_SRC_MISS = 2, ORC_SRC_MISS_NOSLOT = 3, ORC_SRC_RES = 4 };
/* Per-step counters, in this order. */
/* HOST_BYTES: bytes of the distinct missed positions (each once).  HOST_READS:
 * rows actually read from the host mirror -- in a round with attention every
 * query row reads each of its own selected misses, so a miss several rows
 * select is read once per row (offload page, "GPU cache management errs too":
 * repeated misses of one round read host memory); in a prefetch round, one read
 * per miss that took a slot. */
enum {
  ORC_CNT_UNION = 0, ORC_CNT_HIT, ORC_CNT_RING, ORC_CNT_MISS, ORC_CNT_MISS_NOSLOT,
  ORC_CNT_EVICT, ORC_CNT_HOST_BYTES, ORC_CNT_RES, ORC_CNT_HOST_READS, ORC_CNT__N
};

typedef struct {
  int64_t max_positions;   /* history rows plus every later append */
  int32_t index_heads;     /* H_I */
  int32_t index_dim;       /* 128 */
  int32_t heads;           /* H (MLA query heads) */
  int32_t latent_dim;      /* 512 */
  int32_t rope_dim;        /* 64 */
  int32_t group;           /* 64: one fp16 scale per group of latent values */
  int32_t top_k;           /* K */
  int32_t hot_slots;       /* S */
  int32_t ring_rows;       /* 64: writeback batch */
  int32_t max_query_rows;  /* R_max */
  int32_t mode;            /* ORC_MODE_* */
  double softmax_scale;    /* 1/sqrt(latent_dim + rope_dim) */
  int32_t replacement;     /* ORC_REPL_* (offload mode) */
} orc_config;

typedef struct orc_unit orc_unit;

orc_unit* orc_create(const orc_config* cfg, int* status);
void orc_destroy(orc_unit* u);
int64_t orc_row_bytes(const orc_unit* u);

/* Append n rows at positions L..L+n-1.  keys: bf16 bits [n][index_dim];
 * rows: packed Q8G64 rows [n][row_bytes]. */
int orc_append(orc_unit* u, int64_t n, const uint16_t* keys, const uint8_t* rows);
/* Write every pending ring row to the mirror (M = L). */
int orc_flush(orc_unit* u);
/* Offload mode: fill the hot cache with the most recent min(S, L) positions. */
int orc_warm(orc_unit* u);
/* Drop the last n rows (L -= n, M = min(M, L)).  Offload mode: ORC_E_STATE if
 * L-n is below the mirror count at the start of the latest decode round (or L
 * at the latest warm); ORC_E_STATE if n > L; ORC_E_INVALID if n < 0. */
int orc_rollback(orc_unit* u, int64_t n);

/* One decode step over the last R appended positions.
 * index_q: bf16 [R][index_heads][index_dim]; index_w: f32 [R][index_heads];
 * q_lat: bf16 [R][heads][latent_dim]; q_rope: bf16 [R][heads][rope_dim];
 * out: f32 [R][heads][latent_dim]. */
int orc_decode_step(orc_unit* u, int32_t R, const uint16_t* index_q, const float* index_w,
                    const uint16_t* q_lat, const uint16_t* q_rope, float* out);

/* A decode round on a given selection (a layer that reuses another layer's
 * selection): sel i32 [R][top_k] ascending, -1 padded; sel_n i32 [R].  No
 * scoring (the scores getter keeps the previous step's values). */
int orc_decode_step_sel(orc_unit* u, int32_t R, const int32_t* sel, const int32_t* sel_n,
                        const uint16_t* q_lat, const uint16_t* q_rope, float* out);
/* A round without attention on a given selection: classification, pins,
 * replacement and slot fills, writeback; the next round finds the filled rows
 * as hits.  Resident mode: no-op. */
int orc_prefetch_sel(orc_unit* u, int32_t R, const int32_t* sel, const int32_t* sel_n);

/* ---- state and last-step getters (host buffers owned by the caller) ---- */
/* state: L, M, round (steps done), hand, last R, union size, rollback floor */
void orc_get_state(const orc_unit* u, int64_t state[7]);
/* scores of the last step, [R][L] f32 (positions a row cannot see hold 0) */
void orc_get_scores(const orc_unit* u, float* dst);
/* selections [R][K] i32 ascending (-1 padded); counts [R] */
void orc_get_selection(const orc_unit* u, int32_t* sel, int32_t* counts);
/* union [U] ascending, source kind [U], source index [U] (slot / ring slot / position) */
void orc_get_union(const orc_unit* u, int32_t* uni, int32_t* kind, int32_t* src);
/* map [R][K]: index into the union of every selected position (-1 padded) */
void orc_get_map(const orc_unit* u, int32_t* map);
/* compact rows [U][row_bytes] */
void orc_get_compact(const orc_unit* u, uint8_t* dst);
void orc_get_counters(const orc_unit* u, int64_t cnt[ORC_CNT__N]);
/* slot table: slot_pos, fill_round, pin_round [S]; pos_slot [L] */
void orc_get_slots(const orc_unit* u, int32_t* slot_pos, int32_t* fill_round, int32_t* pin_round);
void orc_get_pos_slot(const orc_unit* u, int32_t* pos_slot);
/* reference bits [S] (0 or 1; CLOCK only, all 0 for the ring policy) */
void orc_get_ref(const orc_unit* u, uint8_t* ref);
/* hot slot bytes [S][row_bytes] */
void orc_get_slot_bytes(const orc_unit* u, uint8_t* dst);
/* mirror rows [first, first+n) (offload) or row store (resident) */
int orc_get_mirror(const orc_unit* u, int64_t first, int64_t n, uint8_t* dst);

#ifdef __cplusplus
}
#endif
#endif
