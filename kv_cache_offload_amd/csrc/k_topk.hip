// k_topk.hip -- exact Top-K per query row, ties broken by the lower position.
//
// The GPU computes the exact Top-K (page "From 1M total to 15+ streams x 1M:
// the capacity breakthrough of GLM-5.3 KV cache offload", section "Decision 1":
// an approximate CPU selection moved the cutoff and was rejected).
//
// Radix select over order-preserving 32-bit keys of the fp32 scores, digits of
// 11, 11 and 10 bits.  The first digit's histogram is built by the score kernel
// while the scores are still in registers (in kHistReps replicas, so that the
// few bins integer-valued scores crowd into do not serialise the atomics).
// Then, per query row:
//   * chunk (one 1024-thread workgroup per 4096-position chunk): finds the
//     first-digit bin b0 that holds the K-th largest key and writes, in
//     position order, the (key, position) of every key of the chunk whose first
//     digit is at or above b0 -- every position that can be selected -- and
//     adds the second-digit histogram of its keys in b0; for histories longer
//     than 65,536 positions that list would be long, so a refine pass first
//     builds the second-digit histogram and the lists keep only keys whose
//     first two digits are at or above (b0, b1): barely more than K;
//   * final (one 1024-thread workgroup per row: for short histories the last
//     of the row's chunk workgroups to finish, in the same launch; for long
//     ones a launch of its own): loads the row's candidates into LDS, finds the
//     remaining digits -- the threshold key tau and the number E of keys equal
//     to tau that are taken -- and emits the selection in ascending position
//     order: every key above tau plus the E lowest-position keys equal to tau.
//     If the candidates do not fit in LDS (nearly all scores equal), the same
//     passes read the candidate lists from global memory.
// Each selected position is marked in the step's union bitmap, and the last
// row of each sequence to finish runs the counts phase of the gather plan
// (gather_plan.h; its walk runs in the attention launch).  All per-position
// work is spread over the chunks; only the candidates, a few thousand per row,
// reach the final step.
//
// Memory-level parallelism: gathers whose addresses are known are issued
// together, unconditionally (indices clamped into the buffer), and pinned with
// keep() before any of them is used, so a batch costs one memory round trip.
#include "gather_plan.h"

namespace dsa {
namespace {

constexpr int kPartThreads = 256;
constexpr int kPerThread = kTopkChunk / kPartThreads;     // 16 consecutive positions per thread
constexpr int kSelThreads = 1024;                         // select workgroup (also runs the plan)
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelPer = kTopkChunk / kSelThreads;          // 4 consecutive positions per thread
constexpr int kCandCap = 16384;                            // candidates of a row held in LDS
constexpr int kMaxChunks = kMaxTopkChunks;                 // chunk offsets kept in LDS
constexpr int kMaxK = 4096;
constexpr int kShortMax = 65536;                           // candidates by the first digit up to this length
constexpr int kEmitIters = kCandCap / kSelThreads;         // emit iterations of a lane, candidates in LDS
static_assert(kSelThreads == kPlanThreads, "the plan runs on a select workgroup");
static_assert(kSelPer == 4, "one 16-byte score load per thread");
static_assert(kMaxChunks <= kSelThreads, "one chunk count per thread");
static_assert(2 * kCandCap >= 2 * kPlanThreads, "the plan reuses the candidate LDS");

// Keeps x live at this point: a load feeding it cannot be moved into a later
// branch.  Issue a batch of loads first, then keep() each: the loads stay
// together and the batch costs one memory round trip.
template <class T>
__device__ inline void keep(T& x) {
  asm volatile("" : "+v"(x));
}

struct TopkKArgs {
  StepArgs a;
  int64_t p_pad;
  int n_chunks;
  int K;
  int mode;
  int r_max;
  int long_mode;       // 0: candidates by the first digit; 1: by the first two (refine pass first)
  int plan_mode;       // the gather plan here: 0 none (attention counts the union itself and its extra
                       // workgroup runs the whole plan), 1 the counts phase, 2 counts and walk (CLOCK)
  PlanParams plan;
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

// 16 consecutive scores from t0 (in bounds: rows are P_pad long, P_pad a
// multiple of the chunk).
__device__ inline void load_chunk(const DSA_GLOBAL float* sc, int64_t t0, float* v) {
  f32x4v f[kPerThread / 4];
#pragma unroll
  for (int q = 0; q < kPerThread / 4; ++q) f[q] = *reinterpret_cast<const DSA_GLOBAL f32x4v*>(sc + t0 + 4 * q);
#pragma unroll
  for (int q = 0; q < kPerThread / 4; ++q) {
    v[4 * q] = f[q].x;
    v[4 * q + 1] = f[q].y;
    v[4 * q + 2] = f[q].z;
    v[4 * q + 3] = f[q].w;
  }
}

// Marks the row's first n selected positions (in LDS) in the step's union
// bitmap -- a position several rows select is one union entry.  Every thread
// of the workgroup calls it.
__device__ inline void mark_selection(const ScratchG& s, const int32_t* s_sel, int n) {
  constexpr int kPer = kMaxK / kSelThreads;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int j = threadIdx.x + e * kSelThreads;
    const int32_t pos = j < n ? s_sel[j] : -1;
    if (pos >= 0) g_or(&s.selmask[pos >> 5], 1u << (pos & 31));
  }
}

// Fewer visible positions than K: every visible position is selected.
__device__ inline void select_all_visible(const ScratchG& s, int r, int K, int64_t n_vis) {
  const int tid = threadIdx.x;
  const auto sel = s.sel + (int64_t)r * K;
  for (int t = tid; t < K; t += kSelThreads) {
    sel[t] = t < n_vis ? t : -1;
    if (t < n_vis) g_or(&s.selmask[t >> 5], 1u << (t & 31));
  }
  if (tid == 0) s.sel_n[r] = (int32_t)n_vis;
}

// Long histories: the row's threshold digits, once per row (instead of in every
// chunk's workgroup).  Stage 0: the first-digit bin b0 of the K-th largest key
// and the keys still needed from it; stage 1 (after the refine pass): the
// second digit b1 within b0.
__global__ __launch_bounds__(kSelThreads) void topk_digits_kernel(TopkKArgs ka, int stage) {
  __shared__ uint32_t sh[kSelWaves];
  const StepArgs& a = ka.a;
  const int r = blockIdx.x, seq = blockIdx.y;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  const int64_t n_vis = step_L(u, a) - a.R + r + 1;
  if (n_vis <= ka.K) return;
  const auto dig = reinterpret_cast<DSA_GLOBAL i32x4*>(s.rowdig + 4 * r);
  int b;
  uint32_t need;
  if (stage == 0) {
    find_bin<kSelWaves, kRadixBins, kHistReps>(s.hist0 + (int64_t)r * kRadixBins, (uint32_t)ka.K, sh, &b, &need,
                                               (int64_t)ka.r_max * kRadixBins);
    if (threadIdx.x == 0) *dig = (i32x4){b, 0, (int32_t)need, 0};
  } else {
    const i32x4 d = *dig;
    find_bin<kSelWaves, kRadixBins, 1>(s.hist1 + (int64_t)r * kRadixBins, (uint32_t)d.z, sh, &b, &need);
    if (threadIdx.x == 0) *dig = (i32x4){d.x, b, (int32_t)need, 0};
  }
}

// Second-digit histogram of the keys in the first-digit bin b0 (long histories).
__global__ __launch_bounds__(kPartThreads) void topk_refine_kernel(TopkKArgs ka) {
  __shared__ uint32_t lh[kRadixBins];
  const StepArgs& a = ka.a;
  const int chunk = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  const int64_t L = step_L(u, a);
  const int64_t n_vis = L - a.R + r + 1;
  const int64_t start = (int64_t)chunk * kTopkChunk;
  if (n_vis <= ka.K || start >= n_vis) return;
  const int64_t t0 = start + threadIdx.x * kPerThread;
  float v[kPerThread];
  load_chunk(s.scores + (int64_t)r * ka.p_pad, t0, v);
  const int b0 = s.rowdig[4 * r];                      // from the digits pass
  for (int b = threadIdx.x; b < kRadixBins; b += kPartThreads) lh[b] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t key = order_key(v[e]);
    if (t0 + e < n_vis && (key >> 21) == (uint32_t)b0) atomicAdd(&lh[(key >> 10) & 2047u], 1u);
  }
  __syncthreads();
  const auto gh = s.hist1 + (int64_t)r * kRadixBins;
  for (int b = threadIdx.x; b < kRadixBins; b += kPartThreads)
    if (lh[b]) g_add(&gh[b], lh[b]);
}

// The candidates of one row, in position order: LDS copies when they fit, else
// the global per-chunk lists (chunk c's list starts at c * kTopkChunk).
struct CandSrc {
  const uint32_t* lkey;              // LDS keys (or null)
  const int32_t* lpos;               // LDS positions (or null)
  const DSA_GLOBAL i32x2* gcand;     // global candidate lists of the row
  const uint32_t* off;               // LDS: first candidate index of each chunk, [n_chunks + 1]
  int n_chunks;
  __device__ inline int chunk_of(uint32_t i) const {   // the chunk with off[c] <= i < off[c + 1]
    int lo = 0, hi = n_chunks;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= i) lo = mid;
      else hi = mid;
    }
    return lo;
  }
  __device__ inline i32x2 global(uint32_t i) const {
    const int c = chunk_of(i);
    return gcand[(int64_t)c * kTopkChunk + (i - off[c])];
  }
  __device__ inline void get(uint32_t i, uint32_t* key, int32_t* pos) const {
    if (lkey) {
      *key = lkey[i];
      *pos = lpos[i];
      return;
    }
    const i32x2 kp = global(i);
    *key = (uint32_t)kp.x;
    *pos = kp.y;
  }
};

// LDS of the select workgroup.
struct SelectLds {
  uint32_t sh[4 * kSelWaves];
  uint32_t hist[kRadixBins];
  uint32_t off[kMaxChunks + 1];
  uint32_t wcnt[2 * kSelWaves];
  int32_t sel[kMaxK];
  uint32_t last;
  int b1;
  uint32_t need;
};

// The row's final step: the remaining digits over the candidates -- the
// threshold key tau and the number E of keys equal to tau that are taken --
// then the selection in position order (every key above tau, and the E
// lowest-position keys equal to tau) and its marks in the step's union bitmap.
__device__ void resolve_row(const TopkKArgs& ka, const ScratchG& s, int r, int64_t n_vis, int b0, int b1,
                            uint32_t need, uint32_t cnt, const uint32_t* h1c, SelectLds& sm, uint32_t* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = ka.K;
  const int n_chunks = (int)((n_vis + kTopkChunk - 1) / kTopkChunk);

  // (the histograms are cleared for the next step by the gather's assign kernel)
  // One scan for both: the second-digit histogram (short histories; its bins
  // from the highest down, PER to a thread) and the chunk list sizes.
  constexpr int kPer = kRadixBins / kSelThreads;
  uint32_t hl = 0;
  if (!ka.long_mode)
#pragma unroll
    for (int e = 0; e < kPer; ++e) hl += h1c[e];
  {
    uint4 tot;
    const uint4 pre = block_scan4<kSelWaves>(make_uint4(hl, cnt, 0u, 0u), &tot, sm.sh);
    if (tid < n_chunks) sm.off[tid] = pre.y;
    if (tid == 0) sm.off[n_chunks] = tot.y;
    if (!ka.long_mode && pre.x < need && pre.x + hl >= need) {   // the bin holding the need-th key
      uint32_t acc = pre.x;
      bool found = false;
#pragma unroll
      for (int e = kPer - 1; e >= 0; --e) {
        if (!found && acc + h1c[e] >= need) {
          sm.b1 = kRadixBins - (tid + 1) * kPer + e;
          sm.need = need - acc;
          found = true;
        }
        acc += h1c[e];
      }
    }
  }
  for (int b = tid; b < 1024; b += kSelThreads) sm.hist[b] = 0;
  for (int j = tid; j < K; j += kSelThreads) sm.sel[j] = -1;   // every entry is written below
  __syncthreads();
  if (!ka.long_mode) {
    b1 = sm.b1;
    need = sm.need;
  }
  const uint32_t C = sm.off[n_chunks];                 // >= K: every key of tau's first digits or above
  const uint32_t p22 = ((uint32_t)b0 << 11) | (uint32_t)b1;
  uint32_t* lkey = lds;
  int32_t* lpos = reinterpret_cast<int32_t*>(lds + kCandCap);
  CandSrc src{nullptr, nullptr, s.cand + (int64_t)r * ka.p_pad, sm.off, n_chunks};
  // The candidates into LDS, and the last digit counted of the keys whose first
  // two digits are (b0, b1) as they pass.  At most one chunk per wave (short
  // histories): wave w copies chunk w's list (contiguous at both ends).  More
  // chunks (long histories, short lists): candidate i of the row is found by
  // its chunk's offset, and every load of the row is issued at once.
  auto put = [&](uint32_t at, i32x2 kp) {
    const uint32_t key = (uint32_t)kp.x;
    lkey[at] = key;
    lpos[at] = kp.y;
    if ((key >> 10) == p22) atomicAdd(&sm.hist[key & 1023u], 1u);
  };
  if (C <= (uint32_t)kCandCap && n_chunks <= kSelWaves) {
    constexpr int kBatch = 8;
    if (wave < n_chunks) {
      const uint32_t base = sm.off[wave], n = sm.off[wave + 1] - base;
      const DSA_GLOBAL i32x2* lst = src.gcand + (int64_t)wave * kTopkChunk;
      for (uint32_t i0 = 0; i0 < n; i0 += 64 * kBatch) {
        i32x2 kp[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          const uint32_t i = i0 + q * 64 + lane;
          kp[q] = lst[i < n ? i : n - 1];
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) keep(kp[q]);
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          const uint32_t i = i0 + q * 64 + lane;
          if (i < n) put(base + i, kp[q]);
        }
      }
    }
    src.lkey = lkey;
    src.lpos = lpos;
  } else if (C <= (uint32_t)kCandCap) {
    constexpr int kLoads = kCandCap / kSelThreads;
    i32x2 kp[kLoads];
#pragma unroll
    for (int e = 0; e < kLoads; ++e) {
      const uint32_t i = e * kSelThreads + tid;
      if (e * kSelThreads < (int)C) kp[e] = src.global(i < C ? i : C - 1);   // uniform branch
    }
#pragma unroll
    for (int e = 0; e < kLoads; ++e)
      if (e * kSelThreads < (int)C) keep(kp[e]);
#pragma unroll
    for (int e = 0; e < kLoads; ++e) {
      const uint32_t i = e * kSelThreads + tid;
      if (i < C) put(i, kp[e]);
    }
    src.lkey = lkey;
    src.lpos = lpos;
  } else {
    for (uint32_t i = tid; i < C; i += kSelThreads) {
      uint32_t key;
      int32_t pos;
      src.get(i, &key, &pos);
      if ((key >> 10) == p22) atomicAdd(&sm.hist[key & 1023u], 1u);
    }
  }
  __syncthreads();

  // Ordered emit layout: wave w owns candidates [w seg, (w+1) seg), 64
  // consecutive at a time (with the candidates in LDS, at most kEmitIters per lane).
  const uint32_t seg = ((C + kSelWaves * 64 - 1) / (kSelWaves * 64)) * 64;
  const uint32_t w0 = min(C, wave * seg), w1 = min(C, w0 + seg);
  const bool fused = src.lkey != nullptr;              // seg <= 64 kEmitIters

  int b2;
  find_bin<kSelWaves, 1024, 1>(sm.hist, need, sm.sh, &b2, &need);
  const uint32_t tau = (p22 << 10) | (uint32_t)b2;
  const uint32_t E = need;                             // keys equal to tau that are taken

  // A first pass counts each wave's keys above and equal to tau, a scan over the
  // waves gives each wave its starting ranks, a second pass writes.
  const uint64_t below = lanes_below(lane);
  uint32_t n_gt = 0, n_eq = 0;
  for (uint32_t i0 = w0; i0 < w1; i0 += 64) {
    const uint32_t i = i0 + lane;
    uint32_t key = 0;
    int32_t pos;
    if (i < w1) src.get(i, &key, &pos);
    n_gt += (uint32_t)__popcll(__ballot(i < w1 && key > tau));
    n_eq += (uint32_t)__popcll(__ballot(i < w1 && key == tau));
  }
  if (lane == 0) {
    sm.wcnt[wave] = n_gt;
    sm.wcnt[kSelWaves + wave] = n_eq;
  }
  __syncthreads();
  uint32_t gt_run = 0, eq_run = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    gt_run += w < wave ? sm.wcnt[w] : 0u;
    eq_run += w < wave ? sm.wcnt[kSelWaves + w] : 0u;
  }
  const auto sel = s.sel + (int64_t)r * K;
  // the write position of candidate i, or 0xFFFFFFFF if it is not taken
  auto place = [&](uint32_t i, uint32_t key, uint32_t* at) {
    const bool gt = i < w1 && key > tau, eq = i < w1 && key == tau;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const uint32_t gr = gt_run + (uint32_t)__popcll(bg & below);
    const uint32_t er = eq_run + (uint32_t)__popcll(be & below);
    *at = 0xFFFFFFFFu;
    if (gt) *at = gr + min(er, E);
    else if (eq && er < E) *at = gr + er;
    gt_run += (uint32_t)__popcll(bg);
    eq_run += (uint32_t)__popcll(be);
  };
  if (fused) {
    // each taken position is written and marked in the union bitmap at once
#pragma unroll
    for (int it = 0; it < kEmitIters; ++it) {
      const uint32_t i0 = w0 + 64 * it;
      if (i0 >= w1) break;                              // (uniform in the wave)
      const uint32_t i = i0 + lane;
      const uint32_t key = i < w1 ? lkey[i] : 0u;
      const int32_t pos = i < w1 ? lpos[i] : -1;
      uint32_t at;
      place(i, key, &at);
      if (at < (uint32_t)K && pos >= 0) {              // always, when the histograms match the keys
        sel[at] = pos;
        g_or(&s.selmask[pos >> 5], 1u << (pos & 31));
      }
    }
  } else {
    for (uint32_t i0 = w0; i0 < w1; i0 += 64) {
      const uint32_t i = i0 + lane;
      uint32_t key = 0;
      int32_t pos = -1;
      if (i < w1) src.get(i, &key, &pos);
      uint32_t at;
      place(i, key, &at);
      if (at < (uint32_t)K) {                          // always, when the histograms match the keys
        sel[at] = pos;
        sm.sel[at] = pos;
      }
    }
    __syncthreads();
    mark_selection(s, sm.sel, K);
  }
  if (tid == 0) s.sel_n[r] = K;
}

// The row's final step, by one workgroup: resolves the row from its candidate
// lists (or selects every visible position), then, if the gather plan runs
// here, the last row of the sequence to finish runs its counts phase.
__device__ void final_row(const TopkKArgs& ka, const UnitG& u, const ScratchG& s, int r, SelectLds& sm,
                          uint32_t* lds) {
  const StepArgs& a = ka.a;
  const int tid = threadIdx.x;
  // Everything this pass reads first, issued together: the round-start state
  // (the plan needs it too), the row's digits from the chunk pass, the chunk
  // list sizes (one chunk per thread at most) and this thread's bins of the
  // second-digit histogram.
  const PlanState ps{step_L(u, a), u.dyn[1], (int32_t)u.dyn[2], ka.mode == 0 ? *u.hand : 0};
  const i32x4 dig = *reinterpret_cast<const DSA_GLOBAL i32x4*>(s.rowdig + 4 * r);
  const uint32_t cnt_all = tid < ka.n_chunks ? s.cand_n[(int64_t)r * ka.n_chunks + tid] : 0u;
  uint32_t h1c[kRadixBins / kSelThreads];
  load_bins<kSelWaves, kRadixBins, 1>(s.hist1 + (int64_t)r * kRadixBins, h1c);
  const int64_t n_vis = ps.L - a.R + r + 1;
  const int K = ka.K;
  if (r == 0 && tid == 0) s.counters[8] = 0;          // host reads: the round's attention adds them
  if (n_vis <= K) {
    select_all_visible(s, r, K, n_vis);
  } else {
    const int n_chunks = (int)((n_vis + kTopkChunk - 1) / kTopkChunk);
    const uint32_t cnt = tid < n_chunks ? cnt_all : 0u;  // lists of this step's chunks only
    resolve_row(ka, s, r, n_vis, dig.x, dig.y, (uint32_t)dig.z, cnt, h1c, sm, lds);
  }
  // The ring policy's plan runs in the attention launch, beside attention (the
  // counts too, where attention can count the union itself); CLOCK's walk, whose
  // first lap can sweep the whole ring, keeps all 1,024 threads here.
  if (ka.plan_mode > 0) plan_if_last(u, s, ka.plan, (uint32_t)a.R, ps, lds, ka.plan_mode == 2);
}

// The chunk's candidate list (and, for short histories, its part of the
// second-digit histogram).
__device__ inline void chunk_lists(const TopkKArgs& ka, const ScratchG& s, int chunk, int r, int64_t n_vis,
                                   SelectLds& sm) {
  const int tid = threadIdx.x;
  const int64_t start = (int64_t)chunk * kTopkChunk;

  const int64_t t0 = start + tid * kSelPer;
  const f32x4v f = *reinterpret_cast<const DSA_GLOBAL f32x4v*>(s.scores + (int64_t)r * ka.p_pad + t0);
  int b0, b1 = 0;
  uint32_t need;
  if (ka.long_mode) {                                  // both digits from the digits passes
    const i32x4 d = *reinterpret_cast<const DSA_GLOBAL i32x4*>(s.rowdig + 4 * r);
    b0 = d.x;
    b1 = d.y;
    need = (uint32_t)d.z;
  } else {
    find_bin<kSelWaves, kRadixBins, kHistReps>(s.hist0 + (int64_t)r * kRadixBins, (uint32_t)ka.K, sm.sh, &b0,
                                               &need, (int64_t)ka.r_max * kRadixBins);
  }
  uint32_t key[kSelPer];
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) key[e] = t0 + e < n_vis ? order_key(f[e]) : 0u;   // 0: not visible
  const int shift = ka.long_mode ? 10 : 21;
  const uint32_t thr = ka.long_mode ? (((uint32_t)b0 << 11) | (uint32_t)b1) : (uint32_t)b0;
  if (!ka.long_mode && chunk == 0 && tid == 0)         // the row's digits so far, for the final pass
    *reinterpret_cast<DSA_GLOBAL i32x4*>(s.rowdig + 4 * r) = (i32x4){b0, b1, (int32_t)need, 0};

  if (!ka.long_mode) {
    for (int b = tid; b < kRadixBins; b += kSelThreads) sm.hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kSelPer; ++e)
      if (t0 + e < n_vis && (key[e] >> 21) == (uint32_t)b0) atomicAdd(&sm.hist[(key[e] >> 10) & 2047u], 1u);
    __syncthreads();
    const auto gh = s.hist1 + (int64_t)r * kRadixBins;
    for (int b = tid; b < kRadixBins; b += kSelThreads)
      if (sm.hist[b]) g_add(&gh[b], sm.hist[b]);
  }
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) mine += (t0 + e < n_vis && (key[e] >> shift) >= thr) ? 1u : 0u;
  uint32_t tot;
  uint32_t at = block_scan<kSelWaves>(mine, &tot, sm.sh);
  const auto out = s.cand + (int64_t)r * ka.p_pad + start;
#pragma unroll
  for (int e = 0; e < kSelPer; ++e)
    if (t0 + e < n_vis && (key[e] >> shift) >= thr) out[at++] = (i32x2){(int)key[e], (int)(t0 + e)};
  if (tid == 0) s.cand_n[(int64_t)r * ka.n_chunks + chunk] = tot;
}

// Candidate lists.  One workgroup per (4096-position chunk, row, sequence)
// keeps the chunk's candidates -- every key whose first digit is at or above
// the bin b0 of the K-th key (whose first two digits are at or above (b0, b1)
// for long histories, b1 from the refine pass) -- in position order, and, for
// short histories, adds the second-digit histogram of its keys in bin b0.
// FUSED (short histories): the last of a row's chunk workgroups to finish then
// resolves the row itself (final_row), so no launch separates the two passes.
// Each workgroup publishes its lists before it arrives: every wave waits until
// its own stores have completed, then thread 0's arrival is a device-scope
// release (the XCD's L2 is written back, so a workgroup on another XCD reads
// the lists from memory; the histogram adds are device-scope atomics).  The
// last to arrive drops its cached copies (device-scope acquire) before it reads
// the other chunks' lists.  No workgroup waits for another.
template <bool FUSED>
__global__ __launch_bounds__(kSelThreads) void topk_chunk_kernel(TopkKArgs ka) {
  extern __shared__ __align__(16) uint32_t lds[];      // FUSED: keys[kCandCap], positions[kCandCap]
  __shared__ SelectLds sm;
  const StepArgs& a = ka.a;
  const int chunk = blockIdx.x, r = blockIdx.y, seq = blockIdx.z, tid = threadIdx.x;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  const int64_t L = step_L(u, a);
  const int64_t n_vis = L - a.R + r + 1;
  const int64_t start = (int64_t)chunk * kTopkChunk;
  if (n_vis > ka.K) {
    if (start >= n_vis) return;
    chunk_lists(ka, s, chunk, r, n_vis, sm);
    if (!FUSED) return;
    __builtin_amdgcn_s_waitcnt(0);                     // this wave's stores and adds completed
    __syncthreads();
    if (tid == 0) {
      const uint32_t n_ch = (uint32_t)((n_vis + kTopkChunk - 1) / kTopkChunk);
      // release: the L2 written back, and the write-back waited for (explicitly:
      // nothing else is outstanding, so no wait would otherwise be placed here)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t prev = __hip_atomic_fetch_add(s.done + 1 + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = prev + 1 == n_ch;
      sm.last = last ? 1u : 0u;
      if (last) {
        __hip_atomic_store(s.done + 1 + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
    }
    __syncthreads();
    if (!sm.last) return;
  } else if (!FUSED || chunk != 0) {                   // every visible position is selected: chunk 0's work
    return;
  }
  if constexpr (FUSED) final_row(ka, u, s, r, sm, lds);
}

// Long histories: one workgroup per (row, sequence) resolves the row from its
// candidate lists after the chunk pass.
__global__ __launch_bounds__(kSelThreads) void topk_final_kernel(TopkKArgs ka) {
  extern __shared__ __align__(16) uint32_t lds[];   // keys[kCandCap], positions[kCandCap]
  __shared__ SelectLds sm;
  const int r = blockIdx.x, seq = blockIdx.y;
  final_row(ka, unit_of(ka.a, seq), scratch_of(ka.a, seq), r, sm, lds);
}

TopkKArgs topk_args(const Geometry& g, const StepArgs& a) {
  return TopkKArgs{a, g.p_pad, g.n_chunks, g.top_k, g.mode, g.r_max, a.l_max > kShortMax ? 1 : 0,
                   topk_plan_mode(g, a),
                   PlanParams{g.hot_slots, g.s_words, g.ring_rows, g.mode, g.clock ? 1 : 0, a.add}};
}

}  // namespace

int topk_plan_mode(const Geometry& g, const StepArgs& a) {
  if (g.clock) return 2;
  const int64_t attn_wgs = (int64_t)a.n_seqs * (a.R * (int64_t)((g.top_k + 63) / 64) + 1);
  return (a.l_max + 31) / 32 <= kAttnScanWords && attn_wgs <= g.n_cu ? 0 : 1;
}

hipError_t prepare_topk_kernels() {
  const hipError_t e = hipFuncSetAttribute((const void*)topk_final_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           2 * kCandCap * (int)sizeof(uint32_t));
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)topk_chunk_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             2 * kCandCap * (int)sizeof(uint32_t));
}

hipError_t launch_topk_partial(const Geometry& g, const StepArgs& a, hipStream_t st) {
  const TopkKArgs ka = topk_args(g, a);
  if (!ka.long_mode) return hipSuccess;
  const int chunks = (int)((a.l_max + kTopkChunk - 1) / kTopkChunk);
  const dim3 rows((unsigned)a.R, (unsigned)a.n_seqs);
  hipError_t e = launch_k(topk_digits_kernel, rows, dim3(kSelThreads), 0, st, ka, 0);
  if (e != hipSuccess) return e;
  e = launch_k(topk_refine_kernel, dim3((unsigned)chunks, (unsigned)a.R, (unsigned)a.n_seqs), dim3(kPartThreads), 0,
               st, ka);
  if (e != hipSuccess) return e;
  return launch_k(topk_digits_kernel, rows, dim3(kSelThreads), 0, st, ka, 1);
}

hipError_t launch_topk_select(const Geometry& g, const StepArgs& a, hipStream_t st) {
  const TopkKArgs ka = topk_args(g, a);
  const int chunks = (int)((a.l_max + kTopkChunk - 1) / kTopkChunk);
  const dim3 grid((unsigned)chunks, (unsigned)a.R, (unsigned)a.n_seqs);
  if (!ka.long_mode)
    return launch_k(topk_chunk_kernel<true>, grid, dim3(kSelThreads), 2 * kCandCap * (uint32_t)sizeof(uint32_t), st,
                    ka);
  const hipError_t e = launch_k(topk_chunk_kernel<false>, grid, dim3(kSelThreads), 0, st, ka);
  if (e != hipSuccess) return e;
  return launch_k(topk_final_kernel, dim3((unsigned)a.R, (unsigned)a.n_seqs), dim3(kSelThreads),
                  2 * kCandCap * (uint32_t)sizeof(uint32_t), st, ka);
}

}  // namespace dsa
