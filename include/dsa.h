/*
 * dsa.h -- C ABI of libdsa: DSA sparse-attention decode over an MLA history
 * offloaded to pinned host memory behind an HBM hot cache, for MI355X (gfx950).
 *
 * Method (page "From 1M total to 15+ streams x 1M: the capacity breakthrough of
 * GLM-5.3 KV cache offload", zhuai.tech; the "offload page" below):
 *   - The full MLA history lives in host RAM; the GPU keeps a hot cache of
 *     S slots that is not a sliding window: any position may be cached, and
 *     an old position selected by the indexer is read on a miss (section
 *     "Starting point: separate capacity from the working set").
 *   - A decode step scores every history position with the DSA indexer,
 *     takes the exact Top-K, and the GPU itself resolves each selected
 *     position: a hit reads its HBM slot, a miss reads the registered host
 *     mirror, producing a compact selection consumed by MLA attention; new
 *     rows enter a GPU recent ring and are written back in batches; the CPU
 *     performs no per-selection lookup or copy (section "Decision 3: let the
 *     GPU manage the hot cache directly", data-flow figure).
 *   - Slots filled in a round count as hits only from the next round; a
 *     position missed by several query rows in one round is read from host
 *     memory; slots in use are pinned; replacement walks the slots as a ring
 *     and skips the pinned ones (section "GPU cache management errs too:
 *     cross-block visibility and long replacement sweeps").
 *   - Before the full history is exported, pending rows are flushed and the
 *     host row count must reach the logical row count (section "Capacity must
 *     survive the session lifecycle").
 *
 * Data formats
 *   Q8G64 MLA row (656 bytes for latent_dim=512, group=64, rope_dim=64):
 *     bytes [0, 512)     int8 latent, two's complement
 *     bytes [512, 528)   8 fp16 scales, little endian; latent d uses scale d/64
 *     bytes [528, 656)   64 bf16 RoPE values, little endian
 *   (offload page, section "Starting point": 512 B latent + 16 B scale +
 *   128 B RoPE = 656 B.)  Dequantised latent: c[d] = int8[d] * scale[d/64].
 *   Index keys: bf16 [index_dim] per position, kept in HBM for every position.
 *
 * Units.  A unit is one (layer, sequence) pair with its own key store, host
 * mirror, recent ring, hot cache and slot table.  All sequences of one layer
 * are stepped together by one dsa_decode_step call.
 *
 * Step semantics (per unit, round r = number of decode steps done so far):
 *   1. Query row i of R sits at position L-R+i (the caller appended the R new
 *      rows first) and sees positions [0, L-R+i].
 *   2. score[i][t] = sum_h w[i][h] * max(0, q[i][h] . key[t]), fp32, -0 -> +0.
 *   3. Selection: the K positions with the largest scores, ties broken by the
 *      lower position (all visible positions if fewer than K), reported in
 *      ascending position order.
 *   4. Union U of the R selections, ascending; map[i][j] = index in U.
 *   5. Each union entry is classified on the round-start state: RING if the
 *      row is not yet written back (position >= M), else HIT if cached in a
 *      slot filled in an earlier round, else MISS.
 *   6. HIT slots are pinned for round r.  MISSes, in ascending position order,
 *      take the next slots in ring order from the hand that are not pinned in
 *      round r (each slot visited at most once); a MISS left without a slot is
 *      read from host memory and not cached.  hand = last assigned slot + 1.
 *   7. compact[u] = the 656 bytes of U[u] from its source (slot, ring, or host
 *      mirror; a freshly filled slot is never the source in the same round).
 *   8. out[i][h][:] = sum_j softmax_j(scale * (q_lat[i][h] . c_j +
 *      q_rope[i][h] . rope_j)) * c_j  over row i's selection (absorbed MLA:
 *      the values are the dequantised latent itself).
 *   9. If 64 (ring_rows) rows are pending in the ring, they are written back
 *      to the host mirror as one batch.
 *
 * Ownership.  The session owns every persistent buffer: key stores, hot
 * slots, rings, slot tables and scratch in HBM (allocated once, at exact
 * sizes, at create), and the host mirrors in pinned, device-mapped host memory
 * (hipHostMalloc, touched once at create).  append and decode never allocate.
 * All pointer arguments are borrowed from the caller and must stay valid until
 * the work enqueued on `stream` completes.
 *
 * Asynchrony.  Every call except create, destroy, dsa_unit_state,
 * dsa_mirror_rows and dsa_last_error only enqueues work on the caller's stream;
 * results are valid after the caller synchronises that stream.  All calls on
 * one session must use the same stream, or streams the caller orders; calls on
 * one session from several host threads must be serialised by the caller.
 *
 * Errors.  Arguments are validated before anything is enqueued, so a call that
 * returns an error other than DSA_E_HIP has no effect.  A failing HIP call
 * returns DSA_E_HIP and makes the session sticky-failed: every later call
 * except destroy returns DSA_E_STATE.  dsa_last_error gives the text.
 * The kernels also check every position, slot and union index they follow
 * against what the round's plan allows.  An entry that fails a check is skipped
 * (its row is masked out of attention, its slot-table update is not made) and
 * sets a flag in a small pinned host block that the session reads, without
 * blocking, at the start of every call: the first call made after such a step
 * has run returns DSA_E_STATE, and so does every later one, with the kinds of
 * failed check in dsa_last_error.  A consistent plan never sets a flag.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 3u

typedef enum {
  DSA_OK = 0,
  DSA_E_INVALID = 1,      /* bad argument (NULL, out of range, mismatched size) */
  DSA_E_NOMEM = 2,        /* allocation failed at create */
  DSA_E_CAPACITY = 3,     /* append past max_positions */
  DSA_E_UNSUPPORTED = 4,  /* shape outside what the kernels implement */
  DSA_E_STATE = 5,        /* wrong order of calls, or the session has failed */
  DSA_E_HIP = 6           /* a HIP runtime call failed */
} dsa_status;

typedef enum {
  DSA_KV_OFFLOAD = 0,       /* rows in a pinned host mirror behind an HBM hot cache */
  DSA_KV_HBM_RESIDENT = 1   /* every row in HBM; same scoring, selection and attention */
} dsa_kv_mode;

/* Replacement policy of the hot cache (offload mode).  Both never take a slot
 * pinned this round; they differ in which unpinned slot a miss takes.
 *   DSA_REPL_RING:  the next unpinned slot in ring order from the hand; the
 *                   hand visits each slot at most once per round (offload
 *                   page, section "GPU cache management errs too", the policy
 *                   the page settled on).
 *   DSA_REPL_CLOCK: second chance with one reference bit per slot (the
 *                   policy it replaced): in ring order from the hand, an
 *                   unpinned slot with its bit set loses the bit and is passed
 *                   over, one with the bit clear is taken; hits, fills and warm
 *                   fills set the bit; at most two laps per round.  With a full
 *                   cache, every bit set and few misses the hand clears a whole
 *                   lap before it takes a slot (the page's replacement probe). */
typedef enum {
  DSA_REPL_RING = 0,
  DSA_REPL_CLOCK = 1
} dsa_replacement;

typedef struct {
  uint32_t abi_version;    /* DSA_ABI_VERSION */
  int32_t device;          /* HIP device ordinal */
  int32_t n_layers;        /* >= 1 */
  int32_t n_seqs;          /* sequences per layer, 1..64 */
  int64_t max_positions;   /* per unit: history plus every later append, <= 4,194,304 */
  int32_t index_heads;     /* H_I in {4, 8, 16, 32} */
  int32_t index_dim;       /* 128 */
  int32_t heads;           /* H, multiple of 16, <= 128 */
  int32_t latent_dim;      /* 512 */
  int32_t rope_dim;        /* 64 */
  int32_t group;           /* 64 */
  int32_t top_k;           /* K, 1..4096 */
  int32_t hot_slots;       /* S in [1, 2^20] (offload mode) */
  int32_t ring_rows;       /* writeback batch, 64 */
  int32_t max_query_rows;  /* R_max; R_max * K <= 16384 */
  float softmax_scale;     /* 1/sqrt(latent_dim + rope_dim) */
  int32_t mode;            /* dsa_kv_mode */
  int32_t replacement;     /* dsa_replacement (offload mode; ignored when resident) */
} dsa_config;

typedef struct dsa_session dsa_session;

/* Validate the configuration and allocate every buffer the session will use:
 * the HBM key stores, hot caches, rings and slot tables, the step scratch, and
 * the pinned host mirrors (offload page, section "Starting point: separate
 * capacity from the working set": the capacity lives in host RAM and the GPU
 * keeps only a hot cache; section "The ten-way experiment": long-lived buffers
 * are allocated once, at their exact sizes).  On failure *out is NULL and
 * nothing is left allocated.  DSA_E_INVALID for a NULL pointer, an
 * abi_version mismatch, a bad device or an out-of-range field;
 * DSA_E_UNSUPPORTED for shapes the kernels do not implement; DSA_E_NOMEM if
 * the device or pinned host allocation fails (nothing is kept, and a later
 * create with a smaller shape may succeed); DSA_E_HIP for another HIP failure. */
dsa_status dsa_session_create(const dsa_config* cfg, dsa_session** out);

/* Synchronise the device, then free everything the session owns.  NULL is
 * accepted.  Always DSA_OK (zhuai.tech feed article "用 Rust 统一管理内存与显存
 * 所有权：从 Arc 到 GPU Completion", its closing list of limits: waiting for
 * the GPU is an explicit call, and a destructor is only a last safety net that
 * reports no error); synchronise and check the last call's status first. */
dsa_status dsa_session_destroy(dsa_session* s);

/* Append n rows at positions L..L+n-1 of unit (layer, seq) (offload page,
 * section "Decision 3": new rows go to a GPU recent ring and are written back
 * to host memory in batches; section "Decision 2": the owner quantises a row
 * once and moves the packed 656 bytes).
 *   index_keys: device, bf16 [n][index_dim], row-major, 16-byte aligned.
 *   rows:       device, uint8 [n][row_bytes] packed Q8G64 rows, 16-byte aligned.
 * Keys go to the HBM key store.  Offload mode: rows enter the recent ring;
 * if the ring (ring_rows + max_query_rows rows) would overflow, whole batches
 * of ring_rows oldest rows are written to the host mirror first.  Resident
 * mode: rows go to the HBM row store.  Both buffers are read in stream order
 * and may be reused once the stream has passed this call.  Errors (nothing is
 * appended): DSA_E_INVALID for n < 0, a bad unit or a NULL / misaligned
 * pointer; DSA_E_CAPACITY if L+n > max_positions.  n == 0 is a no-op. */
dsa_status dsa_append_rows(dsa_session* s, int32_t layer, int32_t seq, int64_t n,
                           const void* index_keys, const void* rows, hipStream_t stream);

/* Quantise n MLA rows to packed Q8G64 rows (offload page, section "Decision 2",
 * first problem: the owner quantises a row once and moves the packed 656 B;
 * section "Starting point" for the layout).  The pages give no scale rule;
 * per group of 64 latent values x:
 *   scale = max|x| / 127 in fp32, rounded to fp16 (nearest even; the largest
 *           finite fp16 if it overflows);
 *   code  = 0 if scale == 0, else clamp(rint(x / scale), -127, 127), with an
 *           IEEE fp32 division and rint rounding half to even.
 * RoPE values are stored unchanged.  Inputs must be finite.
 *   latent: device, bf16 [n][latent_dim]  (latent_dim = 512)
 *   rope:   device, bf16 [n][rope_dim]    (rope_dim = 64)
 *   rows:   device (or pinned host), uint8 [n][row_bytes]  (written)
 * All 16-byte aligned.  Stream-ordered; touches no unit.  DSA_E_INVALID on
 * n < 0 or a NULL / misaligned pointer; n == 0 is a no-op. */
dsa_status dsa_quantize_rows(dsa_session* s, int64_t n, const void* latent, const void* rope, void* rows,
                             hipStream_t stream);

/* dsa_append_rows with the rows given unquantised: the rows are quantised as
 * dsa_quantize_rows does, straight into their place (ring, host mirror or
 * row store), in one pass.  Same state changes and errors as dsa_append_rows.
 *   index_keys: device bf16 [n][index_dim]; latent: device bf16 [n][512];
 *   rope: device bf16 [n][64]; all 16-byte aligned. */
dsa_status dsa_append_latent(dsa_session* s, int32_t layer, int32_t seq, int64_t n, const void* index_keys,
                             const void* latent, const void* rope, hipStream_t stream);

/* Write every pending ring row of the unit to the host mirror (M = L), in
 * stream order (offload page, section "Capacity must survive the session
 * lifecycle": before the full history is exported, pending rows are flushed
 * and the host row count must reach the logical row count; dsa_mirror_rows
 * reports that count).  Resident mode: no-op.  DSA_E_INVALID for a bad unit. */
dsa_status dsa_flush(dsa_session* s, int32_t layer, int32_t seq, hipStream_t stream);

/* Offload mode: refill the unit's hot cache with its most recent min(S, L)
 * positions (slot v holds position L-min(S,L)+v), clear all round marks and
 * set the hand past the last filled slot (offload page, section "Starting
 * point": the hot cache is not a sliding window, but a session starts from
 * its most recent rows; the page's end-to-end runs keep a 32,768-row hot
 * cache).  Requires a flushed unit (M == L), else DSA_E_STATE.  Resident
 * mode: no-op. */
dsa_status dsa_warm_hot(dsa_session* s, int32_t layer, int32_t seq, hipStream_t stream);

/* Drop the last n rows of unit (layer, seq): L becomes L-n and the mirror
 * count M becomes min(M, L-n).  For a verify step whose drafts were rejected
 * (offload page, section "Capacity must survive the session lifecycle": a
 * rejected draft rolls back the KV rows and the DSA selection state).  Keys
 * and rows past the new L are left in place and are overwritten by the next
 * appends; the round count, the hand and the hot slots are unchanged.
 * Offload mode: allowed only while L-n is at least the mirror count at the
 * start of the unit's latest decode round (L at the latest dsa_warm_hot, 0
 * before either), so that no hot slot can hold a dropped position; rows
 * appended since the latest round started can always be dropped.
 * Stream-ordered: one tiny kernel publishes the new L and M on `stream`.
 * Errors (nothing changes): DSA_E_INVALID if n < 0; DSA_E_STATE if n > L or,
 * offloaded, if L-n is below that bound.  n == 0 is a no-op. */
dsa_status dsa_rollback_rows(dsa_session* s, int32_t layer, int32_t seq, int64_t n, hipStream_t stream);

/* One decode step of every sequence of `layer`, R = rows_per_seq query rows
 * each: steps 1-9 of the step semantics above (offload page, section
 * "Starting point": the DSA indexer scores the whole history and attention
 * reads only the Top-2048 rows; section "Decision 3": selection, slot lookup
 * and gather stay on the GPU, with no per-selection CPU work; section "GPU
 * cache management errs too": round-scoped visibility, pins, and the ring walk
 * that skips pinned slots).  1 <= R <= max_query_rows; every sequence must
 * already hold at least R rows (its last R rows are the query positions).
 *   index_q:  device bf16 [n_seqs][R][index_heads][index_dim], 16-byte aligned
 *   index_w:  device f32  [n_seqs][R][index_heads]
 *   q_latent: device bf16 [n_seqs][R][heads][latent_dim], 16-byte aligned
 *   q_rope:   device bf16 [n_seqs][R][heads][rope_dim], 16-byte aligned
 *   out:      device f32  [n_seqs][R][heads][latent_dim]  (written)
 * Errors (nothing enqueued): DSA_E_INVALID for a bad layer, R or buffer;
 * DSA_E_STATE if a sequence holds fewer than R rows. */
dsa_status dsa_decode_step(dsa_session* s, int32_t layer, int32_t rows_per_seq,
                           const void* index_q, const float* index_w, const void* q_latent,
                           const void* q_rope, float* out, hipStream_t stream);

/* Append R = rows_per_seq rows to every sequence of `layer`, then one decode
 * step of those sequences: the same result, state and errors as
 * dsa_append_rows(layer, q, R, index_keys + q R index_dim, rows + q R
 * row_bytes) for every sequence q followed by dsa_decode_step(layer, R, ...),
 * in one call (offload page, section "Starting point": each decode step appends
 * the step's new KV rows and then attends over the history; section "Decision
 * 3": new rows enter the GPU's recent ring).  The score launch writes the new
 * keys and rows itself (its scoring workgroups read the new keys straight from
 * index_keys), so the step has no launch of its own for the append.
 *   index_keys: device bf16 [n_seqs][R][index_dim], 16-byte aligned
 *   rows:       device uint8 [n_seqs][R][row_bytes] packed Q8G64 rows, 16-byte aligned
 *   index_q, index_w, q_latent, q_rope, out: as for dsa_decode_step.
 * Both append buffers are read in stream order and may be reused once the
 * stream has passed this call.  Errors (nothing enqueued): DSA_E_INVALID for a
 * bad layer, R or buffer; DSA_E_CAPACITY if a sequence would pass
 * max_positions. */
dsa_status dsa_append_decode_step(dsa_session* s, int32_t layer, int32_t rows_per_seq,
                                  const void* index_keys, const void* rows,
                                  const void* index_q, const float* index_w, const void* q_latent,
                                  const void* q_rope, float* out, hipStream_t stream);

/* dsa_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks, state changes and results as dsa_decode_step; the
 * step's scratch (scores, Top-K histograms and candidates, union and plan
 * words, compact rows, split partials) lives in a static device array of the
 * library, 64 MiB per GPU (each GPU that loads the library holds its copy until
 * the process ends), instead of the session's scratch.  The call allocates
 * nothing; its first kernel zeroes the parts of the array a step expects
 * zeroed, because the array keeps the previous call's contents.
 *   - Every such call on one GPU shares that GPU's array: calls that may
 *     overlap on one GPU (other streams, other sessions, other threads) race
 *     and must be ordered by the caller (one stream, or events).
 *   - DSA_E_UNSUPPORTED (nothing enqueued) if the layer's step scratch, which
 *     grows with n_seqs, max_query_rows, top_k, heads and max_positions, is
 *     larger than the array (the 50,023-row single stream with 4 query rows
 *     needs about 27 MB).
 *   - The step items of dsa_debug_get are not kept for such a step (they
 *     return DSA_E_STATE until the next dsa_decode_step), and its selection
 *     cannot be reused by dsa_decode_step_reuse or dsa_prefetch_reuse. */
dsa_status dsa_decode_step_static(dsa_session* s, int32_t layer, int32_t rows_per_seq,
                                  const void* index_q, const float* index_w, const void* q_latent,
                                  const void* q_rope, float* out, hipStream_t stream);

/* Selection reuse (offload page, section "Starting point": some later layers
 * reuse the indexer's selection while each layer keeps its own KV rows).  A
 * decode step of `layer` on the selection made by the most recent
 * dsa_decode_step, which must have been src_layer's (layer != src_layer), with
 * the same rows_per_seq, and every sequence of `layer` must hold exactly as
 * many rows as the same sequence of src_layer held at that step (append the
 * layer's own new rows first).  Steps 4-9 of the step semantics then run on
 * the unit of `layer` -- union, classification against its own cache, pins,
 * replacement, compact rows from its own sources, attention over its own rows,
 * batched writeback -- without scoring or Top-K.  Buffers as for
 * dsa_decode_step.  The selection stays valid until the next dsa_decode_step,
 * so several layers can reuse it.  Errors (nothing enqueued): DSA_E_INVALID for
 * bad layers, rows or buffers; DSA_E_STATE if the conditions above fail.
 * The step items of dsa_debug_get then describe this step (the selection and
 * scores items are the source step's). */
dsa_status dsa_decode_step_reuse(dsa_session* s, int32_t layer, int32_t src_layer, int32_t rows_per_seq,
                                 const void* q_latent, const void* q_rope, float* out, hipStream_t stream);

/* Prefetch for a reusing layer (offload page, first decision: once the
 * selection is known, the rows of layers that reuse it can be moved early,
 * overlapping other work, though not for free).  A round of `layer`'s cache on
 * the same selection and under the same conditions as dsa_decode_step_reuse,
 * without attention: hits are pinned, misses take slots as in any round and
 * their rows are copied from the host mirror into those slots, the batched
 * writeback runs, and the round count advances; the layer's next round (its
 * dsa_decode_step_reuse) then finds those rows as hits.  It uses a scratch set
 * of its own, so it may run on a second stream beside the source step.  The
 * library orders it with events of its own: `stream` first waits for an event
 * recorded right after the source step's Top-K (once per selection and
 * stream), so the prefetch may be enqueued as soon as dsa_decode_step has
 * returned and overlaps that step's gather, attention and merge.  A session
 * records that event in its steps only once it has prefetched (an event
 * between two launches delays the next one by a few µs): the session's first
 * prefetch waits instead for everything the source step's stream had enqueued
 * when the prefetch was called (that stream must still exist then).  The layer's
 * dsa_decode_step_reuse waits for the prefetch's completion event when it runs
 * on another stream; the next dsa_decode_step waits for every prefetch still
 * pending on another stream, since it replaces the selection they read.
 * Between the prefetch and the layer's reuse step the caller enqueues no other
 * work of `layer`.  Resident mode: nothing to do (DSA_OK).
 * On MI355X each of the two cross-stream waits costs more than the host-link
 * time the prefetch saves a reusing layer, so the default is no prefetch:
 * dsa_decode_step_reuse reads the misses itself. */
dsa_status dsa_prefetch_reuse(dsa_session* s, int32_t layer, int32_t src_layer, int32_t rows_per_seq,
                              hipStream_t stream);

/* Host-side logical state of a unit, without blocking:
 * out[0] = L (rows appended), out[1] = M (rows whose writeback has been
 * enqueued), out[2] = decode rounds done, out[3] = row bytes. */
dsa_status dsa_unit_state(const dsa_session* s, int32_t layer, int32_t seq, int64_t out[4]);

/* Rows of the unit known to be in the host mirror: the count of the most
 * recent writeback whose completion has been observed (non-blocking query;
 * offload page, section "Capacity must survive the session lifecycle": the
 * host row count must reach the logical row count before the history is
 * exported).  Until the unit is flushed and that flush has completed it may be
 * below L; after dsa_flush and a synchronisation of its stream it equals L.
 * Resident mode: 0 (there is no mirror). */
dsa_status dsa_mirror_rows(dsa_session* s, int32_t layer, int32_t seq, int64_t* rows);

/* Text of the most recent error on this session ("" if none).  The pointer
 * stays valid until the next call on the session. */
const char* dsa_last_error(const dsa_session* s);

/* ---- Inspection, for parity tests and measurement ------------------------
 * Copy internal state of unit (layer, seq) into the caller's device buffer
 * `dst` of `bytes` bytes, stream-ordered.  Step items describe the most recent
 * dsa_decode_step of that layer.  DSA_E_INVALID if `bytes` is smaller than
 * the item (dsa_debug_size gives the size). */
typedef enum {
  DSA_DBG_SCORES = 0,      /* f32 [R][L]          scores (only t <= L-R+i meaningful for row i) */
  DSA_DBG_SELECTION = 1,   /* i32 [R][K]          selected positions, ascending, -1 padded */
  DSA_DBG_SEL_COUNT = 2,   /* i32 [R]             selected count per row */
  DSA_DBG_UNION = 3,       /* i32 [R*K]           union positions (first U valid) */
  DSA_DBG_UNION_KIND = 4,  /* i32 [R*K]           0 HIT, 1 RING, 2 MISS, 3 MISS_NOSLOT, 4 RESIDENT */
  DSA_DBG_UNION_SRC = 5,   /* i32 [R*K]           slot / ring index / position */
  DSA_DBG_MAP = 6,         /* i32 [R][K]          union index per selected position, -1 padded */
  DSA_DBG_COMPACT = 7,     /* u8  [R*K][row_bytes] compact selection (first U rows valid) */
  DSA_DBG_COUNTERS = 8,    /* i64 [9]  union, hit, ring, miss, miss_noslot, evict, host_bytes (distinct missed
                              rows x row_bytes), resident, host_reads (rows read from the host mirror: in a
                              step every query row reads its own selected misses, so a miss several rows
                              select counts once per row; in a prefetch round one read per filled slot) */
  DSA_DBG_SLOT_POS = 9,    /* i32 [S] */
  DSA_DBG_FILL_ROUND = 10, /* i32 [S] */
  DSA_DBG_PIN_ROUND = 11,  /* i32 [S] */
  DSA_DBG_POS_SLOT = 12,   /* i32 [L] */
  DSA_DBG_HAND = 13,       /* i32 [1] */
  DSA_DBG_SLOT_BYTES = 14, /* u8  [S][row_bytes] */
  DSA_DBG_MIRROR = 15,     /* u8  [M][row_bytes] host mirror (resident: row store [L]) */
  DSA_DBG_KEYS = 16,       /* bf16 [L][index_dim] (dst 16-byte aligned; stored in another order, rebuilt by a kernel) */
  DSA_DBG_TOTALS = 17,     /* i64 [9]  the counters above summed over every round of the unit */
  DSA_DBG_REF_BITS = 18    /* u32 [ceil(S/32)] reference bits, slot v = bit v%32 of word v/32 (CLOCK; 0 otherwise) */
} dsa_debug_item;

dsa_status dsa_debug_size(const dsa_session* s, int32_t layer, int32_t seq, int32_t item,
                          size_t* bytes);
dsa_status dsa_debug_get(dsa_session* s, int32_t layer, int32_t seq, int32_t item, void* dst,
                         size_t bytes, hipStream_t stream);

/* ---- Per-kernel timing -----------------------------------------------------
 * When enabled, each group of kernels below carries HIP events on its first
 * and last dispatch (hipExtLaunchKernel), so the interval is the kernels' own
 * execution time, as a kernel trace reports it.  dsa_kernel_times
 * synchronises those events and returns, per kind, the number of timed groups
 * and their total milliseconds since the last call, then resets.  Kinds:
 *   0 index score (with the first Top-K digit histogram)
 *   1 Top-K collect (candidate lists per 4096-position chunk; with a refine
 *     pass before it for histories longer than 65,536 positions)
 *   2 Top-K resolve (selection, union marks, cache classification, then the
 *     gather plan of each sequence)
 *   3 gather (unused in decode steps, count 0: the slot work runs in the
 *     launch of kind 5, the row copies in kind 4)
 *   4 attention (row copies from their sources into the compact buffer and
 *     the filled slots, then attention)
 *   5 attention merge and the gather's assign pass in one launch (slot table
 *     update, union entries, histogram clears, ring writeback); the merge
 *     part is absent when one split covers the selection
 *   6 append (dsa_append_rows)
 * dsa_set_kernel_timing: enable <= 0 turns timing off; enable > 0 turns it on
 * and pre-creates the events of `enable` decode steps (at most 2^18), so that
 * the timed calls themselves create none. */
#define DSA_KERNEL_KINDS 7
dsa_status dsa_set_kernel_timing(dsa_session* s, int32_t enable);
dsa_status dsa_kernel_times(dsa_session* s, int64_t counts[DSA_KERNEL_KINDS],
                            double total_ms[DSA_KERNEL_KINDS]);

/* ---- Fault injection, for tests of the error model -------------------------
 * Forces an error condition from the host, so that every kernel still runs to
 * its normal end (offload page, section "Capacity must survive the session
 * lifecycle": integrity is checked, not assumed).
 *   DSA_INJECT_HIP_FAILURE: the next HIP call the session checks is not made
 *     and reports a failure: that call returns DSA_E_HIP, later calls
 *     DSA_E_STATE (layer and seq are checked but otherwise unused).
 *   DSA_INJECT_BAD_SLOT: offload mode; enqueues on `stream` a kernel that gives
 *     every cached position of unit (layer, seq) an out-of-range slot index,
 *     so the next decode step's hits fail the device-side checks: they are
 *     skipped, and the first call after that step has run returns DSA_E_STATE.
 * DSA_E_INVALID for an unknown `what` or a bad unit; DSA_E_UNSUPPORTED for
 * DSA_INJECT_BAD_SLOT on a resident session. */
typedef enum {
  DSA_INJECT_HIP_FAILURE = 0,
  DSA_INJECT_BAD_SLOT = 1
} dsa_injection;
dsa_status dsa_debug_inject(dsa_session* s, int32_t layer, int32_t seq, int32_t what, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
