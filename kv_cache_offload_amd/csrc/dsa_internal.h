// dsa_internal.h -- device-visible descriptors and kernel launchers of libdsa.
// Internal to the library; the public interface is include/dsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Kernel kinds for the optional per-kernel timing (order matches dsa.h).
enum KernelKind { KK_SCORE = 0, KK_TOPK_HIST, KK_TOPK_EMIT, KK_PLAN, KK_COPY, KK_ATTN, KK_MERGE, KK__N };

// Source kinds of a compact row (same numbering as the inspection interface).
enum SrcKind { SRC_HIT = 0, SRC_RING = 1, SRC_MISS = 2, SRC_MISS_NOSLOT = 3, SRC_RES = 4 };

constexpr int kTopkChunk = 4096;      // positions per top-k workgroup
constexpr int kRadixBins = 2048;      // digits 11 + 11 + 10 bits
constexpr int kSuffixLen = 1025;      // last-digit suffix sums per chunk
constexpr int kAttnSubRows = 32;      // selected rows per attention sub-chunk
constexpr int kMaxUnion = 16384;      // R_max * K limit (gather-plan LDS)
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
};

// Per-sequence step scratch, shared by the layers (layers run in stream order).
struct SeqScratch {
  float* scores;          // [R_max][P_pad]
  uint32_t* hist;         // [2 parity][R_max][3 passes][2048]
  uint32_t* suffix;       // [R_max][n_chunks][1025]
  uint32_t* gt22;         // [R_max][n_chunks]
  int32_t* sel;           // [R_max][K]
  int32_t* sel_n;         // [R_max]
  int32_t* uni;           // [R_max*K]
  int32_t* kind;          // [R_max*K]
  int32_t* src;           // [R_max*K]
  int32_t* fill;          // [R_max*K]
  int32_t* map;           // [R_max][K]
  uint8_t* compact;       // [R_max*K][row_bytes]
  float* part_o;          // [R_max][nsplit][H][latent]
  float* part_ml;         // [R_max][nsplit][H][2]
  int64_t* counters;      // [8] union, hit, ring, miss, miss_noslot, evict, host_bytes, resident
  int64_t* info;          // [4] union size, writeback first position (-1: none), reserved
};

struct Geometry {
  int index_heads, index_dim, heads, latent, rope, group, top_k, hot_slots;
  int ring_rows, ring_cap, r_max, row_bytes, mode;
  int64_t max_positions, p_pad;
  int n_chunks;           // top-k chunks per row at max_positions
  int attn_split_rows;    // selected rows per attention workgroup
  int nsplit;             // attention splits per row at K
  float softmax_scale;
};

struct StepArgs {
  const UnitDev* units;   // device array, indexed by unit_base + seq
  const SeqScratch* scr;  // device array, indexed by seq
  int unit_base;
  int n_seqs;
  int R;
  int parity;             // histogram buffer used by this step
  int64_t l_max;          // max L over the layer's sequences (grid sizing)
};

// ---- launchers (each returns the hipError_t of its launch) ----
hipError_t launch_score(const Geometry& g, const StepArgs& a, const uint16_t* q, const float* w,
                        hipStream_t st);
hipError_t launch_topk_hist(const Geometry& g, const StepArgs& a, int pass, hipStream_t st);
hipError_t launch_topk_emit(const Geometry& g, const StepArgs& a, hipStream_t st);
hipError_t launch_plan(const Geometry& g, const StepArgs& a, hipStream_t st);
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
hipError_t prepare_gather_kernels();

}  // namespace dsa
