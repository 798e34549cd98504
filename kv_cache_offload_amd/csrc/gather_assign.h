// gather_assign.h -- the assign pass of the hot gather, after the plan.
//
// Page "From 1M total to 15+ streams x 1M: the capacity breakthrough of
// GLM-5.3 KV cache offload", section "GPU cache management errs too": a hit's
// slot is pinned for the round; the k-th miss in ascending position order takes
// the plan's k-th victim, evicting the position that slot held; section
// "Decision 2": the recent ring goes back to the mirror in 64-row batches.
// One wave per 64 positions, one lane per position: each selected lane writes
// its union entry (position, kind, source) and descriptor and does its slot
// work; in a decode step the wave then copies its filled misses' rows from the
// compact rows into their slots.  Further blocks clear the step's Top-K
// histograms and write a due ring batch back.  It runs as its own kernel
// (prefetch rounds, whose fill kernel copies the rows from the host mirror) or
// as extra workgroups of the attention merge (decode steps), after attention:
// the attention kernel derives its rows' sources from the plan's outputs, and
// no reader of this round consults what this pass writes.
#pragma once

#include "gather_plan.h"

namespace dsa {

constexpr int kGatherThreads = 256;
// Filled misses' rows a wave copies per round trip.  The misses bunch where the
// ring hand has just evicted, so a wave may fill 16 or more; eight in flight
// keeps such a wave to two or three round trips.
constexpr int kFillBatch = 8;

struct GatherKArgs {
  StepArgs a;
  int S, ring_cap, ring_rows, mode, row_bytes, K;
  int max_union;                        // R_max * K: compact rows in the scratch
  int word_blocks;                      // blocks of the union/slot-table part
  int clear_blocks;                     // then blocks clearing the Top-K histograms; the rest write back the ring
  int r_max;
  int clock;                            // CLOCK replacement: hits and fills set their slot's reference bit
  int copy_fills;                       // copy each filled miss's row from the compact rows (attention wrote them)
  int64_t max_positions;
};

// Union entries and slot table: one wave per 64 positions, one lane per position.
// The last blocks write the 64 oldest pending ring rows back to the host mirror
// when a batch is due (positions the step reads from the ring, never from the
// mirror).
__device__ inline void assign_block(const GatherKArgs& ka, int block, int seq) {
  const StepArgs& a = ka.a;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  if (block == 0 && threadIdx.x == 0) {               // the round-end state the plan's walk computed
    const int64_t wb = s.info[kInfoWriteback];
    const int64_t Lr = s.info[kInfoL];                 // with the rows the step appended
    if (ka.mode == 0) {
      *u.hand = (int32_t)s.info[kInfoNewHand];
      if (wb >= 0) u.dyn[1] = wb + ka.ring_rows;
    } else {
      u.dyn[1] = Lr;
    }
    u.dyn[0] = Lr;
    u.dyn[2] = s.info[kInfoRound] + 1;
  }
  if ((int)block >= ka.word_blocks && (int)block < ka.word_blocks + ka.clear_blocks) {
    // the Top-K histograms of this step's rows, consumed: zero for the next step
    const int64_t t = (int64_t)(block - ka.word_blocks) * kGatherThreads + threadIdx.x;
    const int64_t n0 = (int64_t)kHistReps * a.R * (kRadixBins / 4), n1 = (int64_t)a.R * (kRadixBins / 4);
    if (t < n0) {
      const int64_t q = t / (a.R * (kRadixBins / 4)), rest = t % (a.R * (kRadixBins / 4));
      reinterpret_cast<DSA_GLOBAL u32x4*>(s.hist0 + q * ka.r_max * kRadixBins)[rest] = (u32x4){0u, 0u, 0u, 0u};
    } else if (t < n0 + n1) {
      reinterpret_cast<DSA_GLOBAL u32x4*>(s.hist1)[t - n0] = (u32x4){0u, 0u, 0u, 0u};
    }
    return;
  }
  if ((int)block >= ka.word_blocks) {
    const int64_t wb = s.info[kInfoWriteback];
    if (wb < 0) return;
    const int64_t t = (int64_t)(block - ka.word_blocks - ka.clear_blocks) * kGatherThreads + threadIdx.x;
    if (t >= (int64_t)ka.ring_rows * kCopyChunks16) return;
    const int64_t rb = ka.row_bytes;
    const int64_t p = wb + t / kCopyChunks16, c = t % kCopyChunks16;
    if (p >= ka.max_positions) {                       // never, for a consistent round state
      raise_err(a.err, kErrWriteback);
      return;
    }
    const u32x4 v = *reinterpret_cast<const DSA_GLOBAL u32x4*>(u.ring + (p % ka.ring_cap) * rb + c * 16);
    *reinterpret_cast<DSA_GLOBAL u32x4*>(u.rows + p * rb + c * 16) = v;
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = ((int64_t)block * kGatherThreads + threadIdx.x) >> 6;
  const int64_t L = s.info[kInfoL];                   // (block 0 publishes it as the unit's L)
  const int64_t nw = (L + 31) / 32;
  if (2 * wave_id >= nw) return;
  const int64_t w = 2 * wave_id + (lane >> 5);        // this lane's 32-position word
  const int64_t M = s.info[kInfoM];
  const int32_t round = (int32_t)s.info[kInfoRound];
  const uint32_t n_assigned = (uint32_t)s.info[kInfoAssigned];
  const bool off = ka.mode == 0;
  const int bitpos = lane & 31;
  const uint32_t bit = 1u << bitpos;
  const int64_t p = w * 32 + bitpos;

  const int64_t wc = w < nw ? w : nw - 1;
  uint32_t sw = s.selmask[wc], hw = s.hitmask[wc];    // both loads in flight together
  const uint32_t bu = s.base_u[wc], bm = s.base_m[wc];
  if (w >= nw) sw = 0;
  if (!off) hw = 0;
  const bool mine = (sw & bit) != 0;
  const uint64_t selb = __ballot(mine);
  if (!selb) return;
  if (bitpos == 0 && sw) s.selmask[w] = 0;             // read by every lane above: clear for the next step
  const uint32_t below = bit - 1u;
  const uint32_t ux = bu + __popc(sw & below);         // this lane's union entry (if selected)
  const uint32_t rw = off ? (sw & ring_bits(w, M)) : 0u;
  const uint32_t k = bm + __popc(sw & ~hw & ~rw & below);   // this lane's miss index (if a miss)
  const bool fills = off && mine && !((rw | hw) & bit) && k < n_assigned;
  // Decode steps: the compact rows of the wave's first kFillBatch misses that
  // take a slot are requested now, beside the slot-table loads below; lane c
  // holds 16-byte piece c of each.
  const int64_t rb = ka.row_bytes;
  uint64_t pre = ka.copy_fills ? __ballot(fills && ux < (uint32_t)ka.max_union) : 0ull;
  int pl[kFillBatch];
  u32x4 pv[kFillBatch];
#pragma unroll
  for (int q = 0; q < kFillBatch; ++q) {
    pl[q] = -1;
    if (pre) {                                         // (uniform)
      pl[q] = __builtin_ctzll(pre);
      pre &= pre - 1;
      const uint32_t x = __shfl(ux, pl[q]);
      if (lane < kCopyChunks16)
        pv[q] = *reinterpret_cast<const DSA_GLOBAL u32x4*>(s.compact + (int64_t)x * rb + 16 * lane);
    }
  }
  int32_t fill = -1;                                   // the slot this lane's miss fills
  if (mine) {
    int32_t kind, src;
    if (!off) {
      kind = SRC_RES;
      src = (int32_t)p;
    } else {
      if (rw & bit) {
        kind = SRC_RING;
        src = (int32_t)(p % ka.ring_cap);
      } else if (hw & bit) {
        kind = SRC_HIT;                                // the hit's slot is pinned for this round
        src = u.pos_slot[p].x;
        if (src >= 0 && src < ka.S) {
          u.pin_round[src] = round;
          if (ka.clock) g_or(&u.ref[src >> 5], 1u << (src & 31));
        } else {
          raise_err(a.err, kErrHitSlot);
        }
      } else {
        src = (int32_t)p;
        if (k < n_assigned) {
          kind = SRC_MISS;
          const i32x2 vo = s.victim[k];                // (slot, position it held), from the plan
          const int32_t v = vo.x, old = vo.y;
          if (v < 0 || v >= ka.S || old >= ka.max_positions) raise_err(a.err, kErrVictim);
          if (v >= 0 && v < ka.S) {
            if (old >= 0 && old < ka.max_positions) {
              u.pos_slot[old] = (i32x2){-1, -1};
              __hip_atomic_fetch_and(&u.hot[old >> 5], ~(1u << (old & 31)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            u.slot_pos[v] = (int32_t)p;
            u.pos_slot[p] = (i32x2){v, round};
            g_or(&u.hot[p >> 5], bit);
            u.fill_round[v] = round;
            u.pin_round[v] = round;
            if (ka.clock) g_or(&u.ref[v >> 5], 1u << (v & 31));
            fill = v;
          }
        } else {
          kind = SRC_MISS_NOSLOT;
        }
      }
    }
    if (ux < (uint32_t)ka.max_union) {                 // always true for a consistent plan
      s.uni[ux] = (int32_t)p;
      s.kind[ux] = kind;
      s.src[ux] = src;
      s.pdesc[p] = (i32x4){(int32_t)ux, kind, src, fill};
    } else {
      raise_err(a.err, kErrSelection);
      fill = -1;
    }
  }
  if (!ka.copy_fills) return;
  // The filled misses' rows, from the compact rows attention wrote (the bytes it
  // read from the host mirror) into their slots: the ones requested above, then
  // any others of the wave kFillBatch at a time.
  uint64_t fb = __ballot(fill >= 0);
#pragma unroll
  for (int q = 0; q < kFillBatch; ++q) {
    if (pl[q] < 0) continue;                           // (uniform)
    const int32_t f = __shfl(fill, pl[q]);
    fb &= ~(1ull << pl[q]);
    if (f >= 0 && lane < kCopyChunks16)
      *reinterpret_cast<DSA_GLOBAL u32x4*>(u.slots + (int64_t)f * rb + 16 * lane) = pv[q];
  }
  while (fb) {                                         // (uniform)
    int32_t f4[kFillBatch];
    u32x4 v4[kFillBatch];
#pragma unroll
    for (int q = 0; q < kFillBatch; ++q) {
      f4[q] = -1;
      if (fb) {
        const int l = __builtin_ctzll(fb);
        fb &= fb - 1;
        f4[q] = __shfl(fill, l);
        const uint32_t x = __shfl(ux, l);
        if (lane < kCopyChunks16)
          v4[q] = *reinterpret_cast<const DSA_GLOBAL u32x4*>(s.compact + (int64_t)x * rb + 16 * lane);
      }
    }
#pragma unroll
    for (int q = 0; q < kFillBatch; ++q)
      if (f4[q] >= 0 && lane < kCopyChunks16)
        *reinterpret_cast<DSA_GLOBAL u32x4*>(u.slots + (int64_t)f4[q] * rb + 16 * lane) = v4[q];
  }
}

// Arguments and the number of blocks per sequence of the assign pass.
inline GatherKArgs gather_args(const Geometry& g, const StepArgs& a, bool clear_hist, bool copy_fills,
                               int64_t* blocks_per_seq) {
  const int64_t words = (a.l_max + 31) / 32;
  const int64_t waves = (words + 1) / 2;
  const int64_t blocks = (waves + 3) / 4;
  const int64_t wb_blocks = ((int64_t)g.ring_rows * kCopyChunks16 + kGatherThreads - 1) / kGatherThreads;
  const int64_t clear_blocks =
      clear_hist ? ((int64_t)(kHistReps + 1) * a.R * (kRadixBins / 4) + kGatherThreads - 1) / kGatherThreads : 0;
  *blocks_per_seq = blocks + clear_blocks + (g.mode == 0 ? wb_blocks : 0);
  return GatherKArgs{a, g.hot_slots, g.ring_cap, g.ring_rows, g.mode, g.row_bytes, g.top_k, g.r_max * g.top_k,
                     (int)blocks, (int)clear_blocks, g.r_max, g.clock ? 1 : 0, copy_fills ? 1 : 0, g.max_positions};
}

}  // namespace dsa
