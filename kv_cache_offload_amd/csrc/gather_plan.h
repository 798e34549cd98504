// gather_plan.h -- the per-sequence plan of the hot gather, once every query
// row of the sequence has marked its selection in the step's bitmaps.
//
// Page "From 1M total to 15+ streams x 1M: the capacity breakthrough of
// GLM-5.3 KV cache offload", section "GPU cache management errs too": slots in
// use this round are pinned, a slot filled this round is a hit source only from
// the next round, and replacement walks the slots as a ring, skipping the
// pinned ones.  The plan has two phases:
//   * counts (one 1024-thread workgroup): classifies the round's union against
//     the positions cached at round start (a per-position bitmap: every cached
//     slot was filled in an earlier round) and turns the bitmaps into
//     per-32-position-word prefix counts of union entries and of misses -- what
//     attention needs to find each selected row's source and compact place;
//   * walk (one workgroup of any size): lists the unpinned slots in ring order
//     from the hand (the victim of the k-th miss in ascending position order is
//     victim[k]) and publishes the step's counters, the new hand and the
//     round-end state (M after writeback, round + 1).  Only the assign pass,
//     which fills the slots, uses the victims: in a decode step the walk runs in
//     one workgroup of the attention launch, beside attention.
#pragma once

#include "dev_util.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

struct PlanParams {
  int S, s_words, ring_rows, mode;
  int clock;          // CLOCK replacement (second chance with reference bits)
  int add;            // rows appended by the step's first launch, not yet in the unit's L
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

constexpr int kPlanRegWords = 4;   // union words a thread keeps in registers (histories <= 131,072)
constexpr int kPlanChunk = 8;      // 64-word rows of a wave per batch of loads (longer histories)
constexpr int kWalkPer = 4;        // ring offsets a thread examines per pass of the victim walk
// 32-offset words per pass of a T-thread walk
template <int T>
constexpr int walk_words() { return T / 32 * kWalkPer; }
constexpr int kWalkWords = walk_words<kPlanThreads>();

// The union's size and its split by source, from the counts phase.
struct PlanCounts {
  uint32_t U, n_miss, n_ring, n_hit;
};

// Counts phase, by one T-thread workgroup: the hit words, the per-word prefix
// counts of union entries and of misses, and the totals, published with the
// round-start state in the step's info for the rest of the round.
template <int T>
__device__ inline PlanCounts plan_counts_block(const UnitG& u, const ScratchG& s, const PlanParams& pp,
                                               const PlanState& ps) {
  constexpr int kWaves = T / 64;
  __shared__ uint32_t sh[4 * kWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t L = ps.L, M = ps.M;
  const int32_t round = ps.round;
  const bool off = pp.mode == 0;
  const int64_t nw = (L + 31) / 32;
  const auto sel = s.selmask;
  const int64_t per = (nw + T - 1) / T;
  const int64_t w0 = min(nw, (int64_t)tid * per), w1 = min(nw, w0 + per);
  const bool words_in_regs = per <= kPlanRegWords;

  // Every independent load at once: this thread's union words and cached-position
  // words, and the running totals.  A selected position is a hit iff it was
  // cached when the round started (every cached slot was filled in an earlier
  // round); the hit words are published for the assign kernel.
  // The loads are unconditional (a word past the thread's range reads word 0;
  // resident sessions, which cache nothing, read the union words in place of the
  // cached ones) and masked once all are issued: a load in a branch of its own
  // is waited for inside it.
  const auto hot = off ? u.hot : sel;
  uint32_t swr[kPlanRegWords], hwr[kPlanRegWords];
  if (words_in_regs) {
#pragma unroll
    for (int e = 0; e < kPlanRegWords; ++e) {
      const int64_t w = w0 + e < w1 ? w0 + e : 0;
      swr[e] = sel[w];
      hwr[e] = hot[w];
    }
#pragma unroll
    for (int e = 0; e < kPlanRegWords; ++e) {
      const bool in = w0 + e < w1;
      swr[e] = in ? swr[e] : 0u;
      hwr[e] = in && off ? hwr[e] : 0u;
    }
  }

  // Union, miss, ring and hit counts per word, scanned in word (= position) order.
  // (Register arrays are indexed only by unrolled constants.)
  uint4 c = make_uint4(0u, 0u, 0u, 0u);        // union, miss, ring, hit
  auto count = [&](int64_t w, uint32_t sw, uint32_t hw) {
    if (off) s.hitmask[w] = hw;
    if (!sw) return;
    const uint32_t rw = off ? (sw & ring_bits(w, M)) : 0u;
    c.x += __popc(sw);
    if (off) {
      c.y += __popc(sw & ~hw & ~rw);
      c.z += __popc(rw);
      c.w += __popc(hw);
    }
  };
  // Longer histories: wave v owns the words [v seg, (v+1) seg), 64 consecutive
  // words per load instruction (coalesced), kPlanChunk rows of loads in flight.
  const int wave = tid >> 6;
  const int64_t seg = ((nw + kWaves * 64 - 1) / (kWaves * 64)) * 64;
  const int64_t sw0 = min(nw, (int64_t)wave * seg), sw1 = min(nw, sw0 + seg);
  auto wave_rows = [&](auto&& fn) {                    // fn(w, sel word, hit word, valid) per row, all lanes
    for (int64_t r0 = sw0; r0 < sw1; r0 += 64 * kPlanChunk) {
      uint32_t cs[kPlanChunk], ch[kPlanChunk];
#pragma unroll
      for (int e = 0; e < kPlanChunk; ++e) {
        const int64_t w = min(r0 + 64 * e + lane, sw1 - 1);
        cs[e] = sel[w];
        ch[e] = hot[w];
      }
#pragma unroll
      for (int e = 0; e < kPlanChunk; ++e) {
        const int64_t w = r0 + 64 * e + lane;
        const uint32_t sw = w < sw1 ? cs[e] : 0u;
        if (r0 + 64 * e < sw1) fn(w, sw, off ? sw & ch[e] : 0u, w < sw1);   // (uniform in the wave)
      }
    }
  };
  if (words_in_regs) {
#pragma unroll
    for (int e = 0; e < kPlanRegWords; ++e) {
      hwr[e] &= swr[e];
      if (w0 + e < w1) count(w0 + e, swr[e], hwr[e]);
    }
  } else {
    wave_rows([&](int64_t w, uint32_t sw, uint32_t hw, bool valid) {
      if (valid) count(w, sw, hw);
    });
  }
  uint4 tot;
  uint4 base;
  if (words_in_regs) {
    base = block_scan4<kWaves>(c, &tot, sh);
  } else {
    // each wave's counts, then the waves' scan (a wave's words are contiguous)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      c.x += __shfl_xor(c.x, o);
      c.y += __shfl_xor(c.y, o);
      c.z += __shfl_xor(c.z, o);
      c.w += __shfl_xor(c.w, o);
    }
    if (lane == 0) {
      sh[4 * wave] = c.x;
      sh[4 * wave + 1] = c.y;
      sh[4 * wave + 2] = c.z;
      sh[4 * wave + 3] = c.w;
    }
    __syncthreads();
    base = make_uint4(0u, 0u, 0u, 0u);
    tot = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const uint4 x = make_uint4(sh[4 * v], sh[4 * v + 1], sh[4 * v + 2], sh[4 * v + 3]);
      if (v < wave) { base.x += x.x; base.y += x.y; }
      tot.x += x.x; tot.y += x.y; tot.z += x.z; tot.w += x.w;
    }
    __syncthreads();                                   // sh is reused below
  }
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
    // per row of 64 words: the lanes' exclusive scan of (union, miss) counts
    wave_rows([&](int64_t w, uint32_t sw, uint32_t hw, bool valid) {
      uint32_t nu = 0, nm = 0;
      if (valid && sw) {
        const uint32_t rw = off ? (sw & ring_bits(w, M)) : 0u;
        nu = __popc(sw);
        nm = off ? __popc(sw & ~hw & ~rw) : 0u;
      }
      const uint32_t iu = wave_incl_scan(nu, lane), im = wave_incl_scan(nm, lane);
      if (valid) {
        s.base_u[w] = bu + iu - nu;
        s.base_m[w] = bm + im - nm;
      }
      bu += __shfl(iu, 63);
      bm += __shfl(im, 63);
    });
  }

  if (tid == 0) {
    s.info[kInfoUnion] = U;
    s.info[kInfoMiss] = n_miss;
    s.info[kInfoRing] = n_ring;
    s.info[kInfoHit] = n_hit;
    s.info[kInfoRound] = round;
    s.info[kInfoM] = M;
    s.info[kInfoHand] = off ? ps.hand : 0;
    s.info[kInfoL] = ps.L;
  }
  return PlanCounts{U, n_miss, n_ring, n_hit};
}

// Walk phase, by one T-thread workgroup, after the counts phase (the selection
// bitmap still holds the round's marks).  lds: at least walk_words<T>() + 32
// words of LDS the caller no longer uses.
template <int T>
__device__ inline void plan_walk_block(const UnitG& u, const ScratchG& s, const PlanParams& pp,
                                       const PlanState& ps, const PlanCounts& pc, uint32_t* lds) {
  constexpr int NH = T / 32;                           // half-waves
  constexpr int kWords = walk_words<T>();
  constexpr int kEpl = (kWords + 63) / 64;             // pass words per lane in the pass scan
  __shared__ int s_last_v, s_assigned_last_v;
  __shared__ int64_t s_end_o;                          // offset (lap * S + o) of the last victim
  __shared__ uint32_t s_evict;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t L = ps.L, M = ps.M;
  const bool off = pp.mode == 0;
  const int hand = off ? ps.hand : 0;
  const int S = pp.S;
  const auto sel = s.selmask;
  const uint32_t U = pc.U, n_miss = pc.n_miss, n_ring = pc.n_ring, n_hit = pc.n_hit;
  const int64_t total_prev = tid < 8 ? u.totals[tid] : 0;

  // Victims: slots in ring order from the hand, never a pinned one -- a slot is
  // pinned this round iff the position it holds is selected (it is then a hit).
  // Ring policy: every unpinned slot is a candidate; one lap.  CLOCK (second
  // chance): on the first lap the unpinned slots whose reference bit was clear
  // at round start, on the second lap the unpinned slots whose bit was set (the
  // first lap cleared them and took every other unpinned slot).  Passes of
  // walk_words<T>() * 32 ring offsets until every miss has a slot or the laps are
  // done; the k-th miss in ascending position order takes the k-th candidate.
  // victim[k] = (slot, the position it gives up).
  uint32_t n_assigned = 0;
  if (tid == 0) {
    s_last_v = -1;
    s_assigned_last_v = -1;
    s_end_o = 2 * (int64_t)S;
    s_evict = 0;
  }
  if (off && n_miss > 0) {
    uint32_t* cnt_w = lds;                             // [kWords] candidates per word, then their scan
    uint32_t cum = 0;                                  // candidates found in earlier passes
    const int half = tid >> 5, bit = tid & 31;
    const int laps = pp.clock ? 2 : 1;
    for (int lap = 0; lap < laps && cum < n_miss; ++lap) {
      for (int64_t o0 = 0; o0 < S && cum < n_miss; o0 += (int64_t)kWords * 32) {
        int32_t held[kWalkPer], slot[kWalkPer];
        uint32_t refw[kWalkPer];
#pragma unroll
        for (int e = 0; e < kWalkPer; ++e) {           // offset o0 + 32 (half + NH e) + bit within the lap
          const int64_t o = o0 + 32 * (half + NH * e) + bit;
          slot[e] = o < S ? (int32_t)((hand + o) % S) : -1;
          held[e] = u.slot_pos[slot[e] >= 0 ? slot[e] : 0];
          refw[e] = pp.clock && slot[e] >= 0 ? u.ref[slot[e] >> 5] : 0u;
        }
        uint32_t pin_word[kWalkPer];
#pragma unroll
        for (int e = 0; e < kWalkPer; ++e) {
          const int32_t p = held[e];
          pin_word[e] = (slot[e] >= 0 && p >= 0 && p < L) ? sel[p >> 5] : 0u;
        }
        uint32_t ub[kWalkPer];
#pragma unroll
        for (int e = 0; e < kWalkPer; ++e) {
          const int32_t p = held[e];
          const bool pinned = slot[e] >= 0 && p >= 0 && p < L && ((pin_word[e] >> (p & 31)) & 1u);
          const bool referenced = slot[e] >= 0 && ((refw[e] >> (slot[e] & 31)) & 1u);
          const bool cand = slot[e] >= 0 && !pinned && (!pp.clock || referenced == (lap == 1));
          ub[e] = (uint32_t)(__ballot(cand) >> (tid & 32));   // this half-wave's word
          if (bit == 0) cnt_w[half + NH * e] = __popc(ub[e]);
        }
        __syncthreads();
        if (tid < 64) {                                // exclusive scan of the pass's word counts, in offset order
          uint32_t a[kEpl], sum = 0;
#pragma unroll
          for (int i = 0; i < kEpl; ++i) {
            const int w = kEpl * tid + i;
            a[i] = w < kWords ? cnt_w[w] : 0u;
            sum += a[i];
          }
          uint32_t run = wave_incl_scan(sum, lane) - sum;
#pragma unroll
          for (int i = 0; i < kEpl; ++i) {
            const int w = kEpl * tid + i;
            if (w < kWords) cnt_w[w] = run;
            run += a[i];
          }
          if (tid == 63) cnt_w[kWords] = run;
        }
        __syncthreads();
        const uint32_t pass_total = cnt_w[kWords];
#pragma unroll
        for (int e = 0; e < kWalkPer; ++e) {
          if (!((ub[e] >> bit) & 1u)) continue;
          const uint32_t k = cum + cnt_w[half + NH * e] + __popc(ub[e] & ((1u << bit) - 1u));
          if (k + 1 == cum + pass_total) s_last_v = slot[e];
          if (k < n_miss) {
            s.victim[k] = (i32x2){slot[e], held[e]};
            if (held[e] >= 0) atomicAdd(&s_evict, 1u);
            if (k + 1 == n_miss) {
              s_assigned_last_v = slot[e];
              s_end_o = (int64_t)lap * S + o0 + 32 * (half + NH * e) + bit;
            }
          }
        }
        cum += pass_total;
        __syncthreads();                               // cnt_w reused by the next pass
      }
    }
    n_assigned = min(n_miss, cum);
  }
  __syncthreads();
  // CLOCK: the hand cleared the reference bit of every unpinned slot it passed
  // on the first lap before its last victim (all of them if it went further).
  // Clear every bit of that offset range here: the assign kernel then sets the
  // bits of the hits (the only pinned slots) and of the filled victims.
  if (off && pp.clock && n_miss > 0) {
    const int64_t lim = min(s_end_o, (int64_t)S);
    for (int w = tid; w < pp.s_words; w += T) {
      uint32_t m = 0;
      for (int b = 0; b < 32; ++b) {
        const int64_t v = 32 * (int64_t)w + b;
        const int64_t o = v >= hand ? v - hand : v - hand + S;   // ring offset of slot v from the hand
        if (v < S && o < lim) m |= 1u << b;
      }
      if (m) u.ref[w] &= ~m;
    }
  }
  const int last_v = n_assigned == n_miss ? s_assigned_last_v : s_last_v;
  const int new_hand = (off && n_assigned > 0 && last_v >= 0) ? (last_v + 1) % S : hand;
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
  // The round-end state (new hand, M after a due writeback, round + 1) goes to
  // the unit with the assign pass: attention, which may run beside this walk,
  // reads the round-start state.
  if (tid == 0) {
    int64_t wb = -1;
    if (off && L - M >= pp.ring_rows) wb = M;
    s.info[kInfoWriteback] = wb;
    s.info[kInfoAssigned] = n_assigned;
    s.info[kInfoNewHand] = off ? new_hand : 0;
  }
}

// Called by every workgroup (one per query row) of a sequence at the end of its
// selection; the last of the n_rows workgroups to arrive runs the counts phase
// of the plan (full: then the walk too, with all kPlanThreads threads).  Used
// where attention needs the counts before it starts (histories too long for
// attention to count the union itself) or the walk runs here (CLOCK, whose
// first lap can sweep the whole ring; prefetch and reuse rounds).  What the plan reads from the other
// workgroups is only their marks in the selection bitmap, and every mark is a
// device-scope atomic OR: such an atomic is performed where all XCDs see it
// once it has completed.  So before the arrival every wave waits until its own
// marks have completed (a workgroup barrier alone does not wait for another
// wave's outstanding memory operations); thread 0's arrival is a relaxed
// device-scope atomic, and the last workgroup then drops its cached copies
// (an acquire fence at device scope, whose cache invalidation covers the whole
// workgroup: its waves share the CU's and the XCD's caches) before reading the
// bitmap.  Nothing needs releasing -- the selections themselves are read by
// later kernels -- so no L2 is written back here.  No workgroup waits for
// another.
__device__ inline void plan_if_last(const UnitG& u, const ScratchG& s, const PlanParams& pp, uint32_t n_rows,
                                    const PlanState& ps, uint32_t* lds, bool full) {
  __shared__ uint32_t s_last;
  __builtin_amdgcn_s_waitcnt(0);                       // this wave's marks (and every other access) completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(s.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == n_rows;
    s_last = last ? 1u : 0u;
    if (last) {
      __hip_atomic_store(s.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
  }
  __syncthreads();
  if (!s_last) return;
  const PlanCounts pc = plan_counts_block<kPlanThreads>(u, s, pp, ps);
  if (full) {                                          // (uniform)
    __syncthreads();
    plan_walk_block<kPlanThreads>(u, s, pp, ps, pc, lds);
  }
}

// The walk of a decode step, by one T-thread workgroup of the attention
// launch: the round-start state and the counts from the step's info.
template <int T>
__device__ inline void plan_walk_from_info(const UnitG& u, const ScratchG& s, const PlanParams& pp, uint32_t* lds) {
  const PlanState ps{s.info[kInfoL], s.info[kInfoM], (int32_t)s.info[kInfoRound], (int32_t)s.info[kInfoHand]};
  const PlanCounts pc{(uint32_t)s.info[kInfoUnion], (uint32_t)s.info[kInfoMiss], (uint32_t)s.info[kInfoRing],
                      (uint32_t)s.info[kInfoHit]};
  plan_walk_block<T>(u, s, pp, ps, pc, lds);
}

// The whole plan of a decode step, by one T-thread workgroup of the attention
// launch, from the unit's round-start state (nothing updates it before the
// assign pass).
template <int T>
__device__ inline void plan_counts_and_walk(const UnitG& u, const ScratchG& s, const PlanParams& pp, uint32_t* lds) {
  const PlanState ps{u.dyn[0] + pp.add, u.dyn[1], (int32_t)u.dyn[2], pp.mode == 0 ? *u.hand : 0};
  const PlanCounts pc = plan_counts_block<T>(u, s, pp, ps);
  __syncthreads();
  plan_walk_block<T>(u, s, pp, ps, pc, lds);
}

}  // namespace dsa
