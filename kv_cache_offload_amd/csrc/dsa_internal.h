// dsa_internal.h -- device-visible descriptors and kernel launchers of libdsa.
// Internal to the library; the public interface is include/dsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Kernel kinds for the optional per-kernel timing (order matches dsa.h).
// (KK_GATHER is unused by decode steps -- their assign pass runs in the KK_MERGE
// launch -- and keeps its number for the timing ABI.)
enum KernelKind { KK_SCORE = 0, KK_TOPK_PARTIAL, KK_TOPK_SELECT, KK_GATHER, KK_ATTN, KK_MERGE, KK_APPEND, KK__N };

// Source kinds of a compact row (same numbering as the inspection interface).
enum SrcKind { SRC_HIT = 0, SRC_RING = 1, SRC_MISS = 2, SRC_MISS_NOSLOT = 3, SRC_RES = 4 };

constexpr int kTopkChunk = 4096;      // positions per top-k workgroup
constexpr int kRadixBins = 2048;      // digits 11 + 11 + 10 bits
constexpr int kMaxTopkChunks = 1024;  // chunks per row (positions <= 4M)
constexpr int kHistReps = 8;          // replicas of the first-digit histogram (spreads atomics)
constexpr int kAttnSubRows = 32;      // selected rows per attention sub-chunk
constexpr int kMaxUnion = 16384;      // R_max * K limit
constexpr int kCopyChunks16 = 41;     // 656 / 16

// Pointer flavours of the descriptors below.  The host fills them with plain
// pointers; device code reads the same bytes as pointers into the global
// address space, so every access through them compiles to global_*
// instructions (a flat access also counts against the LDS counter, and LDS
// work in the same wave would wait for it).
#define DSA_GLOBAL __attribute__((address_space(1)))
template <class T> using HostPtr = T*;
// Plain vector types for 8- and 16-byte moves (they load and store through any
// address space, unlike the HIP vector classes).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
template <class T> using GlobalPtr = DSA_GLOBAL T*;

// Index keys are stored in the score kernel's MFMA operand order.  Positions
// form tiles of 32; within a tile, 16-byte piece c (dims 8c .. 8c+7) of the key
// at position t sits at piece index 64 (c % 8) + 32 (c / 8) + t % 32, so that
// load k (c % 8 == k) of a wave reads 1 KiB contiguous and lane (n, half)
// receives exactly its B fragment (key n, dims 64 half + 8 k .. +7).
// Returns the index, in 16-byte pieces from the store's start (index_dim 128).
__host__ __device__ inline int64_t key_piece(int64_t t, int c) {
  return (t >> 5) * 512 + (c & 7) * 64 + (c >> 3) * 32 + (t & 31);
}

// Per-unit persistent state, device-visible.
template <template <class> class P>
struct UnitT {
  P<uint16_t> keys;        // [P_pad / 32][8][64][8] bf16, HBM, in key_piece order
  P<uint8_t> rows;         // offload: device address of the pinned host mirror; resident: HBM row store
  P<uint8_t> slots;        // [S][row_bytes] hot slots (offload)
  P<uint8_t> ring;         // [ring_cap][row_bytes] recent ring (offload)
  P<i32x2> pos_slot;       // [P_pad] (slot, round the slot was filled) of a cached position; slot -1 = not cached
  P<uint32_t> hot;         // [P_pad/32] bit set iff the position is cached (as of the current round's start)
  P<int32_t> slot_pos;     // [S]      -1 = empty
  P<int32_t> fill_round;   // [S]
  P<int32_t> pin_round;    // [S]
  P<uint32_t> ref;         // [ceil(S/32)] reference bits (CLOCK replacement)
  P<int32_t> hand;         // [1]
  P<int64_t> dyn;          // [4] L, M, round, reserved -- updated only by kernels, in stream order
  P<int64_t> totals;       // [16] step counters summed over every round of the unit (first 9 used)
};

// Per-sequence step scratch, shared by the layers (layers run in stream order).
template <template <class> class P>
struct ScratchT {
  P<float> scores;          // [R_max][P_pad]
  P<int32_t> sel;           // [R_max][K]
  P<int32_t> sel_n;         // [R_max]
  P<int32_t> uni;           // [R_max*K]
  P<int32_t> kind;          // [R_max*K]
  P<int32_t> src;           // [R_max*K]
  P<int32_t> map;           // [R_max][K]
  P<uint8_t> compact;       // [R_max*K][row_bytes]
  P<uint16_t> part_o;       // fp16 [R_max][nsplit_max][H/16][32][16][16]: split partials (attention)
  P<float> part_ml;         // [R_max][nsplit_max][H][4]: max, sum, scale of the split partial, 0
  P<int64_t> counters;      // [16] union, hit, ring, miss, miss_noslot, evict, host_bytes, resident,
                            //      host_reads (rows read from the host mirror, per reading query row)
  P<int64_t> info;          // [16] see kInfo* below
  P<uint32_t> selmask;      // [P_pad/32] positions selected by any row this step (cleared by the assign)
  P<uint32_t> hitmask;      // [P_pad/32] selected positions that hit a slot (written by the plan each step)
  P<i32x4> pdesc;           // [P_pad] per selected position: union index, kind, source, slot to fill (this step)
  P<uint32_t> base_u;       // [P_pad/32] union entries before each 32-position word
  P<uint32_t> base_m;       // [P_pad/32] misses before each word
  P<i32x2> victim;          // [S_pad] (slot, position it held or -1) given to the k-th miss of the step
  P<uint32_t> hist0;        // [kHistReps][R_max][2048] first-digit histogram replicas (zeroed after use)
  P<uint32_t> hist1;        // [R_max][2048] second-digit histogram within the first-digit bin
  P<i32x2> cand;            // [R_max][P_pad] top-k candidates (key, position), by chunk, in position order
  P<uint32_t> cand_n;       // [R_max][n_chunks] candidates per chunk
  P<int32_t> rowdig;        // [R_max][4] b0, b1, keys still needed: the row's threshold digits so far
  P<uint32_t> done;         // [1 + R_max] rows of the step that finished their selection, then per row
                            // the chunks that finished their lists (each reset by the last to arrive)
};

using UnitDev = UnitT<HostPtr>;
using SeqScratch = ScratchT<HostPtr>;
using UnitG = UnitT<GlobalPtr>;
using ScratchG = ScratchT<GlobalPtr>;
static_assert(sizeof(UnitDev) == sizeof(UnitG) && sizeof(SeqScratch) == sizeof(ScratchG), "same layout");

// SeqScratch::info fields, written by the gather plan for the rest of the step:
// the counts phase writes the round-start state and the union's counts, the
// walk the writeback position and the number of misses that took a slot.
enum {
  kInfoUnion = 0, kInfoWriteback = 1, kInfoAssigned = 2, kInfoRound = 3, kInfoM = 4, kInfoHand = 5,
  kInfoMiss = 6, kInfoRing = 7, kInfoHit = 8, kInfoNewHand = 9, kInfoL = 10, kInfoWords = 16
};

// Attention counts the union itself (and its extra workgroup runs the whole
// gather plan) when the history's selection words fit this many.
constexpr int64_t kAttnScanWords = 4608;

struct Geometry {
  int index_heads, index_dim, heads, latent, rope, group, top_k, hot_slots;
  int ring_rows, ring_cap, r_max, row_bytes, mode;
  bool clock;             // CLOCK replacement (offload mode)
  int64_t max_positions, p_pad;
  int s_words;            // ceil(hot_slots / 32)
  int n_chunks;           // top-k chunks per row at max_positions
  int nsplit_max;         // attention splits per row at K with the smallest split (64 rows)
  float softmax_scale;
  int n_cu;               // compute units of the device
};

// Every unit's arena buffers, and every sequence's scratch, repeat one layout
// at a constant stride (the session checks this at create).  A kernel gets the
// descriptors of sequence 0 by value in its arguments and forms those of
// sequence q by moving each pointer q strides on: no descriptor table in device
// memory, so no dependent load stands between a kernel's start and its buffers.
struct StepArgs;
// Where a decode step's gather plan runs: 0 in the attention launch (attention
// counts the union itself), 1 counts at the end of the Top-K and the walk in
// the attention launch, 2 all of it at the end of the Top-K (CLOCK).  0 needs
// a history whose selection words fit kAttnScanWords and an attention grid that
// leaves a CU free for the plan's workgroup (attention holds one workgroup per
// CU: a workgroup waiting for a CU would wait for the whole plan).
int topk_plan_mode(const Geometry& g, const StepArgs& a);

struct StepArgs {
  UnitDev u0;             // unit (layer, sequence 0)
  SeqScratch s0;          // scratch of sequence 0 (the main set or the prefetch set)
  int64_t u_stride;       // bytes between consecutive units' arena buffers
  int64_t rows_stride;    // bytes between consecutive units' row stores (offload: host mirrors)
  int64_t s_stride;       // bytes between consecutive sequences' scratch
  int n_seqs;
  int R;
  int64_t l_max;          // max L over the layer's sequences (grid sizing; the appended rows included)
  uint32_t* err;          // device address of the session's error flags (kDevErrWords words)
  int add;                // rows the step's first launch appends to every sequence (an append-and-decode
                          // step; 0 otherwise): until the round ends the unit's L lags by this many
};

// Device-side consistency checks.  A kernel that finds a position, slot or
// union index outside what the step's plan allows skips that access (so it
// stays in bounds) and raises one of these flags in the session's error block:
// pinned host memory mapped into the device, one word per kind, written with a
// plain system-scope store (no read-modify-write over the host link).  The
// session reads the block at the entry of every call and fails the session
// (DSA_E_STATE, with the kinds in the error text) once any flag is set.
enum DevErr {
  kErrSelection = 0,      // a selected position out of range, unmarked in the round's bitmap, or past the union
  kErrHitSlot = 1,        // a hit's slot index outside [0, S)
  kErrVictim = 2,         // a victim slot outside [0, S), or the position it evicts out of range
  kErrWriteback = 3,      // a ring writeback position out of range
  kDevErrWords = 8
};
__device__ inline void raise_err(uint32_t* err, int kind) {
  __hip_atomic_store(err + kind, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Optional timing of the next launches: `start` goes with the first kernel
// launched after it is set (then cleared), `stop` with every kernel, so a
// group of launches is timed from the first kernel's start to the last one's
// end.  The events take the dispatch's own begin/end timestamps.
struct LaunchTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
extern thread_local LaunchTimer t_launch_timer;

template <typename... Args, typename F = void (*)(Args...)>
inline hipError_t launch_k(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st, Args... args) {
  LaunchTimer& t = t_launch_timer;
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, t.start, t.stop, 0u, args...);
  t.start = nullptr;
  return hipGetLastError();
}

__device__ inline UnitG as_global(const UnitDev& u) {
  UnitG g;
  __builtin_memcpy(&g, &u, sizeof(g));
  return g;
}
// A descriptor (a struct of pointers) moved `delta` bytes on, word `alt` by
// `alt_delta` instead; NULL fields stay NULL.
template <class G, class D>
__device__ inline G moved_desc(const D& d, int64_t delta, int alt, int64_t alt_delta) {
  constexpr int kWords = sizeof(D) / 8;
  static_assert(sizeof(D) == kWords * 8 && sizeof(G) == sizeof(D), "descriptors are arrays of pointers");
  uint64_t v[kWords];
  __builtin_memcpy(v, &d, sizeof(D));
#pragma unroll
  for (int i = 0; i < kWords; ++i) v[i] = v[i] ? v[i] + (uint64_t)(i == alt ? alt_delta : delta) : 0u;
  G g;
  __builtin_memcpy(&g, v, sizeof(g));
  return g;
}
// Device views of the descriptors of sequence `seq`.
__device__ inline UnitG unit_of(const StepArgs& a, int seq) {
  return moved_desc<UnitG>(a.u0, seq * a.u_stride, (int)(offsetof(UnitDev, rows) / 8), seq * a.rows_stride);
}
// The history length a step's kernels work on: the unit's L plus the rows the
// step's first launch appends (the assign pass publishes the sum at round end).
__device__ inline int64_t step_L(const UnitG& u, const StepArgs& a) { return u.dyn[0] + a.add; }
__device__ inline ScratchG scratch_of(const StepArgs& a, int seq) {
  return moved_desc<ScratchG>(a.s0, seq * a.s_stride, -1, 0);
}

// Relaxed device-scope atomics on global memory.
__device__ inline void g_or(DSA_GLOBAL uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void g_add(DSA_GLOBAL uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void g_add(DSA_GLOBAL int64_t* p, int64_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- launchers (each returns the hipError_t of its launch) ----
// app_keys/app_rows: the rows an append-and-decode step appends (a.add per
// sequence; ignored when a.add is 0), written by extra workgroups of the launch.
hipError_t launch_score(const Geometry& g, const StepArgs& a, const uint16_t* q, const float* w,
                        const uint16_t* app_keys, const uint8_t* app_rows, hipStream_t st);
// Top-K: a refine pass over chunks for long histories (partial), then candidate
// lists per chunk and a per-row resolve (select); the resolve ends with the
// gather plan, run by the last row of each sequence.
hipError_t launch_topk_partial(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t launch_topk_select(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t prepare_topk_kernels();
// clear_hist: also zero the Top-K histograms for the next step (not in a
// prefetch round, whose scratch set has none).
hipError_t launch_gather(const Geometry& g, const StepArgs& a, hipStream_t st, bool clear_hist = true);
// plan: what of the gather plan the launch runs (an extra workgroup per
// sequence): 0 nothing (the plan ran before), 1 the walk (the counts ran
// before), 2 the whole plan, each attention workgroup counting the union itself.
hipError_t launch_attn(const Geometry& g, const StepArgs& a, const uint16_t* q_lat,
                       const uint16_t* q_rope, float* out, hipStream_t st, int plan);
// The split merge (skipped when one split covers the selection) and, in the
// same launch, the gather's assign pass, which also copies each filled miss's
// row from the compact rows into its slot.
hipError_t launch_attn_merge(const Geometry& g, const StepArgs& a, float* out, hipStream_t st);

// Unit maintenance (one unit per launch).
hipError_t launch_append(const Geometry& g, const UnitDev& unit, int64_t L, int64_t M, int64_t newM,
                         int64_t n, const uint16_t* keys, const uint8_t* rows, hipStream_t st);
hipError_t launch_flush(const Geometry& g, const UnitDev& unit, int64_t M, int64_t L, hipStream_t st);
hipError_t launch_warm(const Geometry& g, const UnitDev& unit, int64_t L, hipStream_t st);
hipError_t launch_rollback(const UnitDev& unit, int64_t L, int64_t M, hipStream_t st);
// Zero what a step expects zeroed in its scratch set (Top-K histograms, the
// selection bitmap, the arrival counter): the static scratch keeps the
// previous call's contents, possibly of another layout.
hipError_t launch_clear_step_scratch(const Geometry& g, const StepArgs& a, hipStream_t st);
// Test hook: every cached position of [0, L) gets an out-of-range slot index (offload).
hipError_t launch_inject_bad_slot(const Geometry& g, const UnitDev& unit, int64_t L, hipStream_t st);
// Keys of positions [0, L) in plain row order [L][index_dim], for inspection.
hipError_t launch_keys_linear(const UnitDev& unit, int64_t L, uint16_t* dst, hipStream_t st);
// Selection reuse and prefetch (k_reuse.hip).
// sel0, sel_stride: the main scratch set, where the selection lives.
hipError_t launch_reuse_mark(const Geometry& g, const StepArgs& a, const SeqScratch& sel0, int64_t sel_stride,
                             hipStream_t st);
hipError_t launch_prefetch_fill(const Geometry& g, const StepArgs& a, hipStream_t st);
// Quantise-on-append (k_quant.hip).
hipError_t launch_quantize(const Geometry& g, int64_t n, const uint16_t* latent, const uint16_t* rope, uint8_t* out,
                           hipStream_t st);
hipError_t launch_append_latent(const Geometry& g, const UnitDev& unit, int64_t L, int64_t M, int64_t newM, int64_t n,
                                const uint16_t* keys, const uint16_t* latent, const uint16_t* rope, hipStream_t st);

// One-time kernel attributes (dynamic LDS above 64 KiB).
hipError_t prepare_score_kernels();

}  // namespace dsa
