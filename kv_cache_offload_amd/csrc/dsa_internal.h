// dsa_internal.h -- device-visible descriptors and kernel launchers of libdsa.
// Internal to the library; the public interface is include/dsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Kernel kinds for the optional per-kernel timing (order matches dsa.h).
enum KernelKind { KK_SCORE = 0, KK_TOPK_COLLECT, KK_TOPK_RESOLVE, KK_SCAN, KK_ASSIGN, KK_COPY, KK_ATTN, KK_MERGE, KK__N };
// (the top-k refine pass is timed with the collect kind)

// Source kinds of a compact row (same numbering as the inspection interface).
enum SrcKind { SRC_HIT = 0, SRC_RING = 1, SRC_MISS = 2, SRC_MISS_NOSLOT = 3, SRC_RES = 4 };

constexpr int kTopkChunk = 4096;      // positions per top-k workgroup
constexpr int kRadixBins = 2048;      // digits 11 + 11 + 10 bits
constexpr int kMaxTopkChunks = 1024;  // chunks per row (positions <= 4M)
constexpr int kHistReps = 8;          // replicas of the first-digit histogram (spreads atomics)
constexpr int kAttnSubRows = 32;      // selected rows per attention sub-chunk
constexpr int kMaxUnion = 16384;      // R_max * K limit
constexpr int kCopyChunks16 = 41;     // 656 / 16

// Per-unit persistent state, device-visible.
struct UnitDev {
  uint16_t* keys;        // [P_pad][index_dim] bf16, HBM
  uint8_t* rows;         // offload: device address of the pinned host mirror; resident: HBM row store
  uint8_t* slots;        // [S][row_bytes] hot slots (offload)
  uint8_t* ring;         // [ring_cap][row_bytes] recent ring (offload)
  int32_t* pos_slot;     // [P_pad]  -1 = not cached
  int32_t* slot_pos;     // [S]      -1 = empty
  int32_t* fill_round;   // [S]
  int32_t* pin_round;    // [S]
  int32_t* hand;         // [1]
  int64_t* dyn;          // [4] L, M, round, reserved -- updated only by kernels, in stream order
  int64_t* totals;       // [8] step counters summed over every decode step of the unit
};

// Per-sequence step scratch, shared by the layers (layers run in stream order).
struct SeqScratch {
  float* scores;          // [R_max][P_pad]
  int32_t* sel;           // [R_max][K]
  int32_t* sel_n;         // [R_max]
  int32_t* uni;           // [R_max*K]
  int32_t* kind;          // [R_max*K]
  int32_t* src;           // [R_max*K]
  int32_t* fill;          // [R_max*K]
  int32_t* map;           // [R_max][K]
  uint8_t* compact;       // [R_max*K][row_bytes]
  float* part_o;          // [R_max][nsplit_max][H][latent]
  float* part_ml;         // [R_max][nsplit_max][H][2]
  int64_t* counters;      // [8] union, hit, ring, miss, miss_noslot, evict, host_bytes, resident
  int64_t* info;          // [8] see kInfo* below
  uint32_t* selmask;      // [P_pad/32] positions selected by any row this step (cleared by the assign)
  uint32_t* hitmask;      // [P_pad/32] selected positions that hit a slot (cleared by the assign)
  int32_t* upos;          // [P_pad] union index of each selected position (valid for this step's selection)
  uint32_t* base_u;       // [P_pad/32] union entries before each 32-position word
  uint32_t* base_m;       // [P_pad/32] misses before each word
  uint32_t* pinmask;      // [S_pad/32] slots pinned this round (cleared by the scan)
  uint32_t* upw;          // [S_pad/32] unpinned slots, in ring order from the hand
  int32_t* victim;        // [S_pad] slot given to the k-th miss of the step
  uint32_t* hist0;        // [kHistReps][R_max][2048] first-digit histogram replicas (zeroed after use)
  uint32_t* hist1;        // [R_max][2048] second-digit histogram within the first-digit bin
  int2* cand;             // [R_max][P_pad] top-k candidates (key, position), by chunk, in position order
  uint32_t* cand_n;       // [R_max][n_chunks] candidates per chunk
  int32_t* victim_old;    // [S_pad] position held by victim[k] before the step (-1: empty)
};

// SeqScratch::info fields, written by the gather scan for the rest of the step.
enum { kInfoUnion = 0, kInfoWriteback = 1, kInfoAssigned = 2, kInfoRound = 3, kInfoM = 4, kInfoHand = 5 };

struct Geometry {
  int index_heads, index_dim, heads, latent, rope, group, top_k, hot_slots;
  int ring_rows, ring_cap, r_max, row_bytes, mode;
  int64_t max_positions, p_pad;
  int s_words;            // ceil(hot_slots / 32)
  int n_chunks;           // top-k chunks per row at max_positions
  int nsplit_max;         // attention splits per row at K with the smallest split (64 rows)
  float softmax_scale;
};

struct StepArgs {
  const UnitDev* units;   // device array, indexed by unit_base + seq
  const SeqScratch* scr;  // device array, indexed by seq
  int unit_base;
  int n_seqs;
  int R;
  int64_t l_max;          // max L over the layer's sequences (grid sizing)
};

// ---- launchers (each returns the hipError_t of its launch) ----
hipError_t launch_score(const Geometry& g, const StepArgs& a, const uint16_t* q, const float* w,
                        hipStream_t st);
hipError_t launch_topk_refine(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t launch_topk_collect(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t launch_topk_resolve(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t prepare_topk_kernels();
hipError_t launch_gather_scan(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t launch_gather_assign(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t launch_copy(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t launch_attn(const Geometry& g, const StepArgs& a, const uint16_t* q_lat,
                       const uint16_t* q_rope, float* out, hipStream_t st);
hipError_t launch_attn_merge(const Geometry& g, const StepArgs& a, float* out, hipStream_t st);

// Unit maintenance (one unit per launch).
hipError_t launch_append(const Geometry& g, const UnitDev& unit, int64_t L, int64_t M, int64_t newM,
                         int64_t n, const uint16_t* keys, const uint8_t* rows, hipStream_t st);
hipError_t launch_flush(const Geometry& g, const UnitDev& unit, int64_t M, int64_t L, hipStream_t st);
hipError_t launch_warm(const Geometry& g, const UnitDev& unit, int64_t L, hipStream_t st);

// One-time kernel attributes (dynamic LDS above 64 KiB).
hipError_t prepare_score_kernels();

}  // namespace dsa
