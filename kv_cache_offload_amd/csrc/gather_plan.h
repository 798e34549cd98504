// gather_plan.h -- the per-sequence plan of the hot gather, run by one
// 1024-thread workgroup once every query row of the sequence has marked its
// selection in the step's bitmaps.
//
// Page "From 1M total to 15+ streams x 1M: the capacity breakthrough of
// GLM-5.3 KV cache offload", section "GPU cache management errs too": misses
// are served after the hits are pinned, and replacement walks the slots as a
// ring, skipping the pinned ones.  The plan turns the position bitmaps into
// per-32-position-word prefix counts of union entries and of misses, lists the
// unpinned slots in ring order from the hand (the victim of the k-th miss in
// ascending position order is victim[k]), and publishes the step's counters,
// the new hand and the round-end state (M after writeback, round + 1).
#pragma once

#include "dev_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

struct PlanParams {
  int S, s_words, ring_rows, mode;
};

// Bits of word w (positions 32w..32w+31) that lie at or above M.
__device__ inline uint32_t ring_bits(int64_t w, int64_t M) {
  const int64_t first = w * 32;
  if (first >= M) return 0xFFFFFFFFu;
  if (first + 32 <= M) return 0u;
  return ~((1u << (uint32_t)(M - first)) - 1u);
}

// The round-start state the plan works from, read by the caller at its start.
struct PlanState {
  int64_t L, M;
  int32_t round;
  int32_t hand;
};

constexpr int kPlanRegWords = 4;   // union/hit words a thread keeps in registers (histories <= 131,072)
constexpr int kPlanRegSlots = 2;   // pinned-slot words a thread keeps in registers (slots <= 65,536)

// Unpinned slots among the 32 ring offsets 32 j .. 32 j + 31 from the hand.
__device__ inline uint32_t unpinned_word(const ScratchG& s, int S, int nsw, int hand, int j) {
  uint32_t bits = 0;
  if ((S & 31) == 0) {
    // 32 offsets from a word-aligned ring: two pinned words, funnel-shifted
    const int v0 = (hand + 32 * j) % S;
    const int wa = v0 >> 5, sa = v0 & 31;
    const uint32_t lo = s.pinmask[wa];
    const uint32_t hi = sa ? s.pinmask[(wa + 1) % nsw] : 0u;
    bits = ~(sa ? ((lo >> sa) | (hi << (32 - sa))) : lo);
  } else {
    int last = -1;
    uint32_t pw = 0;
    for (int i = 0; i < 32; ++i) {
      const int o = 32 * j + i;
      if (o >= S) break;
      const int v = (hand + o) % S;
      if ((v >> 5) != last) { last = v >> 5; pw = s.pinmask[last]; }
      if (!((pw >> (v & 31)) & 1u)) bits |= 1u << i;
    }
  }
  return bits;
}

// lds: 2 * kPlanThreads words of LDS the caller no longer uses.
__device__ inline void gather_plan_block(const UnitG& u, const ScratchG& s, const PlanParams& pp,
                                         const PlanState& ps, uint32_t* lds) {
  __shared__ uint32_t sh[4 * kPlanWaves];
  __shared__ int s_hand;
  __shared__ uint32_t s_evict;
  const int tid = threadIdx.x;
  const int64_t L = ps.L, M = ps.M;
  const int32_t round = ps.round;
  const bool off = pp.mode == 0;
  const int hand = off ? ps.hand : 0;
  const int64_t nw = (L + 31) / 32;
  const auto sel = s.selmask;
  const auto hit = s.hitmask;
  const int64_t per = (nw + kPlanThreads - 1) / kPlanThreads;
  const int64_t w0 = min(nw, (int64_t)tid * per), w1 = min(nw, w0 + per);
  const int S = pp.S, nsw = off ? pp.s_words : 0;
  const int sper = (nsw + kPlanThreads - 1) / kPlanThreads;
  const int j0 = min(nsw, tid * sper), j1 = min(nsw, j0 + sper);
  const bool words_in_regs = per <= kPlanRegWords;
  const bool slots_in_regs = sper <= kPlanRegSlots;

  // Every independent load at once: this thread's union and hit words, its
  // unpinned-slot words and the running totals.
  uint32_t swr[kPlanRegWords], hwr[kPlanRegWords], upr[kPlanRegSlots];
  if (words_in_regs) {
#pragma unroll
    for (int e = 0; e < kPlanRegWords; ++e) {
      const int64_t w = w0 + e;
      swr[e] = w < w1 ? sel[w] : 0u;
      hwr[e] = (off && w < w1) ? hit[w] : 0u;
    }
  }
  if (slots_in_regs) {
#pragma unroll
    for (int e = 0; e < kPlanRegSlots; ++e) upr[e] = j0 + e < j1 ? unpinned_word(s, S, nsw, hand, j0 + e) : 0u;
  }
  const int64_t total_prev = tid < 8 ? u.totals[tid] : 0;

  // Union, miss, ring and hit counts per word, scanned in word (= position) order.
  // (Register arrays are indexed only by unrolled constants.)
  uint4 c = make_uint4(0u, 0u, 0u, 0u);        // union, miss, ring, hit
  auto count = [&](int64_t w, uint32_t sw, uint32_t hw) {
    if (!sw) return;
    const uint32_t rw = off ? (sw & ring_bits(w, M)) : 0u;
    c.x += __popc(sw);
    if (off) {
      c.y += __popc(sw & ~hw & ~rw);
      c.z += __popc(rw);
      c.w += __popc(hw);
    }
  };
  if (words_in_regs) {
#pragma unroll
    for (int e = 0; e < kPlanRegWords; ++e)
      if (w0 + e < w1) count(w0 + e, swr[e], hwr[e]);
  } else {
    for (int64_t w = w0; w < w1; ++w) count(w, sel[w], off ? hit[w] : 0u);
  }
  uint4 tot;
  const uint4 base = block_scan4<kPlanWaves>(c, &tot, sh);
  const uint32_t U = tot.x, n_miss = tot.y, n_ring = tot.z, n_hit = tot.w;
  uint32_t bu = base.x, bm = base.y;
  auto bases = [&](int64_t w, uint32_t sw, uint32_t hw) {
    s.base_u[w] = bu;
    s.base_m[w] = bm;
    if (!sw) return;
    const uint32_t rw = off ? (sw & ring_bits(w, M)) : 0u;
    bu += __popc(sw);
    if (off) bm += __popc(sw & ~hw & ~rw);
  };
  if (words_in_regs) {
#pragma unroll
    for (int e = 0; e < kPlanRegWords; ++e)
      if (w0 + e < w1) bases(w0 + e, swr[e], hwr[e]);
  } else {
    for (int64_t w = w0; w < w1; ++w) bases(w, sel[w], off ? hit[w] : 0u);
  }

  // Unpinned slots in ring order from the hand; victim[k] for the misses that get one.
  uint32_t n_assigned = 0;
  if (tid == 0) {
    s_hand = hand;
    s_evict = 0;
  }
  if (off) {
    uint32_t cnt = 0;
    if (slots_in_regs) {
#pragma unroll
      for (int e = 0; e < kPlanRegSlots; ++e) cnt += __popc(upr[e]);
    } else {
      for (int j = j0; j < j1; ++j) cnt += __popc(unpinned_word(s, S, nsw, hand, j));
    }
    uint32_t n_unpinned;
    uint32_t k = block_scan<kPlanWaves>(cnt, &n_unpinned, sh);
    n_assigned = min(n_miss, n_unpinned);
    if (sper == 1) {
      // one slot word per thread: expand the words in parallel, 32 lanes (one per
      // bit) per word; word j's unpinned slots take victim indices k_j, k_j + 1, ...
      uint32_t* s_bits = lds;
      uint32_t* s_k = lds + kPlanThreads;
      s_bits[tid] = j0 < j1 ? upr[0] : 0u;
      s_k[tid] = k;
      __syncthreads();
      const int bit = tid & 31;
      for (int j = tid >> 5; j < nsw; j += kPlanThreads / 32) {
        const uint32_t kj = s_k[j];
        if (kj >= n_assigned) break;                   // k_j never decreases with j
        const uint32_t bits = s_bits[j];
        bool evicts = false;
        if ((bits >> bit) & 1u) {
          const uint32_t kk = kj + __popc(bits & ((1u << bit) - 1u));
          if (kk < n_assigned) {
            const int v = (hand + 32 * j + bit) % S;
            const int32_t old = u.slot_pos[v];         // the position the slot gives up
            s.victim[kk] = (i32x2){v, old};
            evicts = old >= 0;
            if (kk + 1 == n_assigned) s_hand = (v + 1) % S;
          }
        }
        // the two half-waves may leave the loop at different j: each counts its own half
        const uint32_t eb = (uint32_t)(__ballot(evicts) >> (tid & 32));
        if (bit == 0 && eb) atomicAdd(&s_evict, (uint32_t)__popc(eb));
      }
    } else {
      for (int j = j0, e = 0; j < j1 && k < n_assigned; ++j, ++e) {
        uint32_t bits = (slots_in_regs && e == 0) ? upr[0] : (slots_in_regs && e == 1) ? upr[1]
                                                                                        : unpinned_word(s, S, nsw, hand, j);
        while (bits && k < n_assigned) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1;
          const int v = (hand + 32 * j + b) % S;
          const int32_t old = u.slot_pos[v];
          s.victim[k] = (i32x2){v, old};
          if (old >= 0) atomicAdd(&s_evict, 1u);
          if (k + 1 == n_assigned) s_hand = (v + 1) % S;
          ++k;
        }
      }
    }
    __syncthreads();                                   // every pinned word has been read
    for (int j = tid; j < nsw; j += kPlanThreads) s.pinmask[j] = 0;
  }
  __syncthreads();
  const int64_t rb = 656;
  const int64_t noslot = off ? (int64_t)n_miss - n_assigned : 0;
  if (tid < 8) {
    int64_t cn = 0;
    switch (tid) {
      case 0: cn = U; break;
      case 1: cn = off ? n_hit : 0; break;
      case 2: cn = off ? n_ring : 0; break;
      case 3: cn = n_assigned; break;
      case 4: cn = noslot; break;
      case 5: cn = off ? s_evict : 0; break;
      case 6: cn = off ? ((int64_t)n_assigned + noslot) * rb : 0; break;
      default: cn = off ? 0 : U; break;
    }
    s.counters[tid] = cn;
    u.totals[tid] = total_prev + cn;
  }
  if (tid == 0) {
    int64_t wb = -1;
    if (off && L - M >= pp.ring_rows) wb = M;
    s.info[kInfoUnion] = U;
    s.info[kInfoWriteback] = wb;
    s.info[kInfoAssigned] = n_assigned;
    s.info[kInfoRound] = round;
    s.info[kInfoM] = M;
    s.info[kInfoHand] = hand;
    if (off) {
      *u.hand = s_hand;
      if (wb >= 0) u.dyn[1] = M + pp.ring_rows;
    }
    u.dyn[2] = round + 1;
  }
}

// Called by every workgroup (one per query row) of a sequence at the end of its
// selection; the last of the n_rows workgroups to arrive runs the plan.  The
// workgroup barrier (a workgroup-scope release and acquire) orders every wave's
// marks before thread 0's arrival, an acquire-release atomic at device scope;
// by transitivity the marks of every earlier arrival are visible to every wave
// of the last workgroup after its barrier.  Only one wave per workgroup carries
// the device-scope cache maintenance.  No workgroup waits for another.
__device__ inline void plan_if_last(const UnitG& u, const ScratchG& s, const PlanParams& pp, uint32_t n_rows,
                                    const PlanState& ps, uint32_t* lds) {
  __shared__ uint32_t s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(s.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == n_rows;
    s_last = last ? 1u : 0u;
    if (last) __hip_atomic_store(s.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  gather_plan_block(u, s, pp, ps, lds);
}

}  // namespace dsa
