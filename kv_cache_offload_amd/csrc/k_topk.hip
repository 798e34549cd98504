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
//   * collect (one 256-thread workgroup per 4096-position chunk): finds the
//     first-digit bin b0 that holds the K-th largest key and writes, in
//     position order, the (key, position) of every key whose first digit is at
//     or above b0 -- every position that can be selected;
//     for histories longer than 65,536 positions that list would be long, so a
//     refine pass (same grid) first histograms the second digit of the keys in
//     bin b0, and collect keeps only keys whose first two digits are at or
//     above (b0, b1): barely more than K;
//   * resolve (one 1024-thread workgroup per row): loads the candidates into
//     LDS, finds the remaining digits with LDS histograms -- the threshold key
//     tau and the number E of keys equal to tau that are taken -- and writes
//     the selection in ascending position order with an ordered block scan:
//     every key above tau plus the E lowest-position keys equal to tau.  Each
//     selected position is marked in the step's union bitmap and classified
//     against the hot cache.  If the candidates do not fit in LDS (nearly all
//     scores equal), the same passes stream the candidate lists from global
//     memory instead.  The last row of each sequence to finish runs the
//     gather plan (gather_plan.h).
//
// Memory-level parallelism: gathers whose addresses are known are issued
// together, unconditionally (indices clamped into the buffer), and pinned with
// keep() before any of them is used, so a batch costs one memory round trip.
#include "gather_plan.h"

namespace dsa {
namespace {

constexpr int kPartThreads = 256;
constexpr int kPerThread = kTopkChunk / kPartThreads;     // 16 consecutive positions per thread
constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / 64;
constexpr int kCandCap = 12288;                            // candidates held in LDS
constexpr int kTile = kResolveThreads * 16;                // emit tile (16 per thread)
constexpr int kMaxChunks = 1024;                           // chunk offsets kept in LDS
constexpr int kMaxK = 4096;
constexpr int kOneDigitMax = 65536;                        // collect on the first digit up to this length
static_assert(kResolveThreads == kPlanThreads, "the plan runs on a resolve workgroup");

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
  int digits;          // 11: candidates by the first digit; 22: by the first two
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

// In offload mode a selected position is classified on the round-start state
// -- a hit needs a slot filled in an earlier round -- and the hit's slot is
// pinned for this round.  N positions per thread (-1: none), their lookups
// issued together (two dependent round trips).
template <int N>
__device__ inline void classify_and_pin(const UnitG& u, const ScratchG& s, const int32_t* pos, int64_t M,
                                        int32_t round) {
  int32_t v[N];
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = u.pos_slot[(pos[e] >= 0 && pos[e] < M) ? pos[e] : 0];
#pragma unroll
  for (int e = 0; e < N; ++e) keep(v[e]);
#pragma unroll
  for (int e = 0; e < N; ++e)
    if (!(pos[e] >= 0 && pos[e] < M)) v[e] = -1;
  int32_t fr[N];
#pragma unroll
  for (int e = 0; e < N; ++e) fr[e] = u.fill_round[v[e] >= 0 ? v[e] : 0];
#pragma unroll
  for (int e = 0; e < N; ++e) keep(fr[e]);
#pragma unroll
  for (int e = 0; e < N; ++e)
    if (v[e] >= 0 && fr[e] < round) {
      g_or(&s.hitmask[pos[e] >> 5], 1u << (pos[e] & 31));
      u.pin_round[v[e]] = round;
      g_or(&s.pinmask[v[e] >> 5], 1u << (v[e] & 31));
    }
}

// Marks the row's first n selected positions (in LDS) in the union bitmap -- a
// position several rows select is one union entry -- and, in offload mode,
// classifies and pins them.  Every thread of the workgroup calls it.
__device__ inline void mark_selection(const UnitG& u, const ScratchG& s, const int32_t* s_sel, int n, bool offl,
                                      int64_t M, int32_t round) {
  constexpr int kPer = kMaxK / kResolveThreads;
  int32_t pos[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int j = threadIdx.x + e * kResolveThreads;
    pos[e] = j < n ? s_sel[j] : -1;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    if (pos[e] >= 0) g_or(&s.selmask[pos[e] >> 5], 1u << (pos[e] & 31));
  if (offl) classify_and_pin<kPer>(u, s, pos, M, round);
}

// Second-digit histogram of the keys in the first-digit bin b0 (long histories).
__global__ __launch_bounds__(kPartThreads) void topk_refine_kernel(TopkKArgs ka) {
  __shared__ uint32_t sh[kPartThreads / 64];
  __shared__ uint32_t lh[kRadixBins];
  const StepArgs& a = ka.a;
  const int chunk = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  const int64_t L = u.dyn[0];
  const int64_t n_vis = L - a.R + r + 1;
  const int64_t start = (int64_t)chunk * kTopkChunk;
  if (n_vis <= ka.K || start >= n_vis) return;
  const int64_t t0 = start + threadIdx.x * kPerThread;
  float v[kPerThread];
  load_chunk(s.scores + (int64_t)r * ka.p_pad, t0, v);
  int b0;
  uint32_t need;
  find_bin<kPartThreads / 64, kRadixBins, kHistReps>(s.hist0 + (int64_t)r * kRadixBins, (uint32_t)ka.K, sh, &b0,
                                                     &need, (int64_t)ka.r_max * kRadixBins);
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

// Every (key, position) of the chunk whose leading `digits` bits are at or above
// the threshold digits, in position order.
__global__ __launch_bounds__(kPartThreads) void topk_collect_kernel(TopkKArgs ka) {
  __shared__ uint32_t sh[kPartThreads / 64];
  const StepArgs& a = ka.a;
  const int chunk = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  const int64_t L = u.dyn[0];
  const int64_t n_vis = L - a.R + r + 1;
  const int64_t start = (int64_t)chunk * kTopkChunk;
  if (n_vis <= ka.K || start >= n_vis) return;
  const int64_t t0 = start + threadIdx.x * kPerThread;
  float v[kPerThread];
  load_chunk(s.scores + (int64_t)r * ka.p_pad, t0, v);
  int b0;
  uint32_t need;
  find_bin<kPartThreads / 64, kRadixBins, kHistReps>(s.hist0 + (int64_t)r * kRadixBins, (uint32_t)ka.K, sh, &b0,
                                                     &need, (int64_t)ka.r_max * kRadixBins);
  uint32_t thr = (uint32_t)b0;
  int shift = 21;
  if (ka.digits == 22) {
    int b1;
    find_bin<kPartThreads / 64, kRadixBins, 1>(s.hist1 + (int64_t)r * kRadixBins, need, sh, &b1, &need);
    thr = ((uint32_t)b0 << 11) | (uint32_t)b1;
    shift = 10;
  }
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    mine += (t0 + e < n_vis && (order_key(v[e]) >> shift) >= thr) ? 1u : 0u;
  uint32_t tot;
  uint32_t at = block_scan<kPartThreads / 64>(mine, &tot, sh);
  const auto out = s.cand + (int64_t)r * ka.p_pad + start;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t key = order_key(v[e]);
    if (t0 + e < n_vis && (key >> shift) >= thr) out[at++] = (i32x2){(int)key, (int)(t0 + e)};
  }
  if (threadIdx.x == 0) s.cand_n[(int64_t)r * ka.n_chunks + chunk] = tot;
}

// Candidate source for the resolve passes: LDS when the candidates fit, else the
// global per-chunk lists.
struct CandSrc {
  const uint32_t* lkey;              // LDS keys (or null)
  const int32_t* lpos;               // LDS positions (or null)
  const DSA_GLOBAL i32x2* gcand;     // global candidate lists of the row (by chunk)
  const uint32_t* off;               // LDS: first candidate index of each chunk
  int n_chunks;
  __device__ inline int chunk_of(uint32_t i) const {   // last chunk with off <= i
    int lo = 0, hi = n_chunks;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= i) lo = mid;
      else hi = mid;
    }
    return lo;
  }
  __device__ inline void get(uint32_t i, uint32_t* key, int32_t* pos) const {
    if (lkey) {
      *key = lkey[i];
      *pos = lpos[i];
      return;
    }
    const int c = chunk_of(i);
    const i32x2 kp = gcand[(int64_t)c * kTopkChunk + (i - off[c])];
    *key = (uint32_t)kp.x;
    *pos = kp.y;
  }
};

__global__ __launch_bounds__(kResolveThreads) void topk_resolve_kernel(TopkKArgs ka) {
  extern __shared__ __align__(16) uint32_t lds[];   // keys[kCandCap], pos[kCandCap]
  __shared__ uint32_t sh[4 * kResolveWaves];
  __shared__ uint32_t hist[kRadixBins];
  __shared__ uint32_t off[kMaxChunks + 1];
  __shared__ int32_t s_sel[kMaxK];
  __shared__ uint32_t s_run[2];
  const StepArgs& a = ka.a;
  const int r = blockIdx.x, seq = blockIdx.y, tid = threadIdx.x;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  const int64_t L = u.dyn[0];
  const int64_t M = u.dyn[1];
  const int32_t round = (int32_t)u.dyn[2];
  const bool offl = ka.mode == 0;
  const int K = ka.K;
  const int64_t n_vis = L - a.R + r + 1;
  const auto h0 = s.hist0 + (int64_t)r * kRadixBins;
  const auto h1 = s.hist1 + (int64_t)r * kRadixBins;
  const int64_t rep_stride = (int64_t)ka.r_max * kRadixBins;
  const auto sel = s.sel + (int64_t)r * K;

  if (n_vis <= K) {
    // every visible position is selected
    for (int b = tid; b < kRadixBins; b += kResolveThreads)
      for (int q = 0; q < kHistReps; ++q) h0[q * rep_stride + b] = 0;
    for (int t = tid; t < K; t += kResolveThreads) {
      sel[t] = t < n_vis ? t : -1;
      s_sel[t] = t < n_vis ? t : -1;
    }
    __syncthreads();
    mark_selection(u, s, s_sel, (int)n_vis, offl, M, round);
    if (tid == 0) s.sel_n[r] = (int32_t)n_vis;
    plan_if_last(u, s, ka.plan, (uint32_t)a.R);
    return;
  }

  // chunk counts of the candidate lists (loads issued before the histograms are read)
  const int n_chunks = (int)((n_vis + kTopkChunk - 1) / kTopkChunk);
  const int per = (n_chunks + kResolveThreads - 1) / kResolveThreads;
  const int c0 = min(n_chunks, tid * per), c1 = min(n_chunks, c0 + per);
  uint32_t cnt = 0;
  for (int c = c0; c < c1; ++c) cnt += s.cand_n[(int64_t)r * ka.n_chunks + c];

  int b0, b1 = 0, b2;
  uint32_t need;
  find_bin<kResolveWaves, kRadixBins, kHistReps>(h0, (uint32_t)K, sh, &b0, &need, rep_stride);
  if (ka.digits == 22) find_bin<kResolveWaves, kRadixBins, 1>(h1, need, sh, &b1, &need);
  for (int b = tid; b < kRadixBins; b += kResolveThreads) {   // consumed: clear for the next step
    for (int q = 0; q < kHistReps; ++q) h0[q * rep_stride + b] = 0;
    if (ka.digits == 22) h1[b] = 0;
  }
  {
    uint32_t tot;
    uint32_t base = block_scan<kResolveWaves>(cnt, &tot, sh);
    for (int c = c0; c < c1; ++c) {
      off[c] = base;
      base += s.cand_n[(int64_t)r * ka.n_chunks + c];
    }
    if (tid == 0) off[n_chunks] = tot;
  }
  __syncthreads();
  const uint32_t C = off[n_chunks];
  uint32_t* lkey = lds;
  int32_t* lpos = reinterpret_cast<int32_t*>(lds + kCandCap);
  const DSA_GLOBAL i32x2* gcand = s.cand + (int64_t)r * ka.p_pad;
  CandSrc src{nullptr, nullptr, gcand, off, n_chunks};
  if (C <= (uint32_t)kCandCap) {
    // candidate i = k * 1024 + tid, four at a time: loads issued together
    const uint32_t nk = (C + kResolveThreads - 1) / kResolveThreads;
    for (uint32_t k0 = 0; k0 < nk; k0 += 4) {
      i32x2 kp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t i = (k0 + e) * kResolveThreads + tid;
        const uint32_t ic = i < C ? i : C - 1;
        const int c = src.chunk_of(ic);
        kp[e] = gcand[(int64_t)c * kTopkChunk + (ic - off[c])];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) keep(kp[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t i = (k0 + e) * kResolveThreads + tid;
        if (i < C) {
          lkey[i] = (uint32_t)kp[e].x;
          lpos[i] = kp[e].y;
        }
      }
    }
    src.lkey = lkey;
    src.lpos = lpos;
  }
  __syncthreads();

  if (ka.digits == 11) {
    // second digit of the candidates in bin b0
    for (int b = tid; b < kRadixBins; b += kResolveThreads) hist[b] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < C; i += kResolveThreads) {
      uint32_t key;
      int32_t pos;
      src.get(i, &key, &pos);
      if ((key >> 21) == (uint32_t)b0) atomicAdd(&hist[(key >> 10) & 2047u], 1u);
    }
    __syncthreads();
    find_bin<kResolveWaves, kRadixBins, 1>(hist, need, sh, &b1, &need);
  }
  const uint32_t p22 = ((uint32_t)b0 << 11) | (uint32_t)b1;
  for (int b = tid; b < 1024; b += kResolveThreads) hist[b] = 0;
  __syncthreads();
  for (uint32_t i = tid; i < C; i += kResolveThreads) {
    uint32_t key;
    int32_t pos;
    src.get(i, &key, &pos);
    if ((key >> 10) == p22) atomicAdd(&hist[key & 1023u], 1u);
  }
  __syncthreads();
  find_bin<kResolveWaves, 1024, 1>(hist, need, sh, &b2, &need);
  const uint32_t tau = (p22 << 10) | (uint32_t)b2;
  const uint32_t E = need;                             // keys equal to tau that are taken

  // ordered emit, 16 consecutive candidates per thread per tile
  if (tid == 0) { s_run[0] = 0; s_run[1] = 0; }
  __syncthreads();
  for (uint32_t t0 = 0; t0 < C; t0 += kTile) {
    const uint32_t i0 = t0 + tid * 16;
    uint32_t keys[16];
    int32_t poss[16];
    uint32_t my_gt = 0, my_eq = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      keys[e] = 0;
      poss[e] = -1;
      if (i0 + e < C) {
        src.get(i0 + e, &keys[e], &poss[e]);
        my_gt += keys[e] > tau;
        my_eq += keys[e] == tau;
      }
    }
    const uint32_t run_gt = s_run[0], run_eq = s_run[1];
    uint4 tot;
    const uint4 ex = block_scan4<kResolveWaves>(make_uint4(my_gt, my_eq, 0u, 0u), &tot, sh);
    uint32_t gt = run_gt + ex.x, eq = run_eq + ex.y;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t k = keys[e];
      uint32_t at = 0xFFFFFFFFu;
      if (k > tau) {
        at = gt + (eq < E ? eq : E);
        ++gt;
      } else if (k == tau) {
        if (eq < E) at = gt + eq;
        ++eq;
      }
      if (at < (uint32_t)K) {                          // always, when the histograms match the keys
        sel[at] = poss[e];
        s_sel[at] = poss[e];
      }
    }
    __syncthreads();
    if (tid == 0) { s_run[0] = run_gt + tot.x; s_run[1] = run_eq + tot.y; }
    __syncthreads();
  }
  mark_selection(u, s, s_sel, K, offl, M, round);
  if (tid == 0) s.sel_n[r] = K;
  plan_if_last(u, s, ka.plan, (uint32_t)a.R);
}

TopkKArgs topk_args(const Geometry& g, const StepArgs& a) {
  return TopkKArgs{a, g.p_pad, g.n_chunks, g.top_k, g.mode, g.r_max, a.l_max <= kOneDigitMax ? 11 : 22,
                   PlanParams{g.hot_slots, g.s_words, g.ring_rows, g.mode}};
}

}  // namespace

hipError_t prepare_topk_kernels() {
  return hipFuncSetAttribute((const void*)topk_resolve_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             2 * kCandCap * (int)sizeof(uint32_t));
}

hipError_t launch_topk_partial(const Geometry& g, const StepArgs& a, hipStream_t st) {
  const TopkKArgs ka = topk_args(g, a);
  const int chunks = (int)((a.l_max + kTopkChunk - 1) / kTopkChunk);
  const dim3 grid((unsigned)chunks, (unsigned)a.R, (unsigned)a.n_seqs);
  if (ka.digits == 22) {
    const hipError_t e = launch_k(topk_refine_kernel, grid, dim3(kPartThreads), 0, st, ka);
    if (e != hipSuccess) return e;
  }
  return launch_k(topk_collect_kernel, grid, dim3(kPartThreads), 0, st, ka);
}

hipError_t launch_topk_select(const Geometry& g, const StepArgs& a, hipStream_t st) {
  const TopkKArgs ka = topk_args(g, a);
  const dim3 grid((unsigned)a.R, (unsigned)a.n_seqs);
  return launch_k(topk_resolve_kernel, grid, dim3(kResolveThreads), 2 * kCandCap * (uint32_t)sizeof(uint32_t), st,
                  ka);
}

}  // namespace dsa
