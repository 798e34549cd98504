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
//   * refine (one workgroup per 4096-position chunk): finds the first-digit bin
//     b0 that holds the K-th largest key and histograms the second digit of the
//     keys in that bin;
//   * collect (same grid): finds b1 likewise and writes, in position order, the
//     (key, position) of every key whose first two digits are at or above
//     (b0, b1) -- every position that can be selected, barely more than K;
//   * resolve (one 1024-thread workgroup per row): loads the candidates into LDS,
//     histograms the last digit to get the threshold key tau and the number E of
//     keys equal to tau that are taken, and writes the selection in ascending
//     position order with an ordered block scan: every key above tau plus the
//     lowest-position keys equal to tau.  Each selected position is marked in the
//     step's union bitmap and classified against the hot cache on the spot.  If
//     the candidates do not fit in LDS (e.g. nearly all scores equal), the same
//     passes stream the candidate list from global memory instead.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kCollectThreads = 256;
constexpr int kPerThread = kTopkChunk / kCollectThreads;   // 16 consecutive positions per thread
constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / 64;
constexpr int kCandCap = 16384;                            // candidates held in LDS
constexpr int kTile = kResolveThreads * 16;                 // emit tile (16 per thread)
constexpr int kMaxChunks = 1024;                           // chunk offsets kept in LDS

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive block scan (thread order) for NW waves; total in *tot.
template <int NW>
__device__ inline uint32_t block_scan(uint32_t v, uint32_t* tot, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  uint32_t base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t x = sh[w];
    base += (w < wave) ? x : 0u;
    all += x;
  }
  __syncthreads();
  *tot = all;
  return base + inc - v;
}

// The bin holding the k-th largest key among those counted in hist[NBINS] (summed
// over REPS replicas `stride` apart): the largest b with suffix(b) >= k, and the
// number of keys still needed from it.  Each thread owns NBINS/(64 NW)
// contiguous bins, loaded together; thread 0 owns the highest.
template <int NW, int NBINS, int REPS>
__device__ inline void find_bin(const uint32_t* hist, uint32_t k, uint32_t* sh, int* out_bin,
                                uint32_t* out_need, int64_t stride = 0) {
  constexpr int PER = NBINS / (NW * 64);
  static_assert(PER >= 1 && NBINS % (NW * 64) == 0, "bins per thread");
  __shared__ int s_bin;
  __shared__ uint32_t s_need;
  const int lo = NBINS - ((int)threadIdx.x + 1) * PER;
  uint32_t c[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) c[e] = 0;
#pragma unroll
  for (int q = 0; q < REPS; ++q)
#pragma unroll
    for (int e = 0; e < PER; ++e) c[e] += hist[q * stride + lo + e];
  uint32_t local = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) local += c[e];
  uint32_t tot;
  const uint32_t before = block_scan<NW>(local, &tot, sh);   // keys in higher bins
  if (before < k && before + local >= k) {
    uint32_t acc = before;
    bool done = false;
#pragma unroll
    for (int e = PER - 1; e >= 0; --e) {
      if (!done && acc + c[e] >= k) {
        s_bin = lo + e;
        s_need = k - acc;
        done = true;
      }
      acc += c[e];
    }
  }
  __syncthreads();
  *out_bin = s_bin;
  *out_need = s_need;
  __syncthreads();
}

// A selected position joins this step's union (one bit per position), and is
// classified on the round-start state: a hit needs a slot filled in an earlier
// round; the hit's slot is pinned for this round.  Rows selecting the same
// position repeat identical writes.  Up to 16 positions of one thread are marked
// together, their cache lookups issued at once (two dependent rounds of loads).
__device__ inline void mark_batch(const UnitDev& u, const SeqScratch& s, const int32_t* pos, const bool* taken,
                                  bool off, int64_t M, int32_t round) {
  int32_t v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    v[e] = -1;
    if (taken[e]) {
      atomicOr(&s.selmask[pos[e] >> 5], 1u << (pos[e] & 31));
      if (off && pos[e] < M) v[e] = u.pos_slot[pos[e]];
    }
  }
  int32_t fr[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) fr[e] = v[e] >= 0 ? u.fill_round[v[e]] : round;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (v[e] >= 0 && fr[e] < round) {
      atomicOr(&s.hitmask[pos[e] >> 5], 1u << (pos[e] & 31));
      u.pin_round[v[e]] = round;
      atomicOr(&s.pinmask[v[e] >> 5], 1u << (v[e] & 31));
    }
}

struct TopkKArgs {
  StepArgs a;
  int64_t p_pad;
  int n_chunks;
  int K;
  int mode;
  int r_max;
};

__device__ inline void load_chunk(const float* sc, int64_t t0, float* v) {
#pragma unroll
  for (int q = 0; q < kPerThread / 4; ++q) {
    const float4 f = *reinterpret_cast<const float4*>(sc + t0 + 4 * q);   // in bounds: rows are P_pad long
    v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
  }
}

// Second-digit histogram of the keys in the first-digit bin b0.
__global__ __launch_bounds__(kCollectThreads) void topk_refine_kernel(TopkKArgs ka) {
  __shared__ uint32_t sh[kCollectThreads / 64];
  __shared__ uint32_t lh[kRadixBins];
  const StepArgs& a = ka.a;
  const int chunk = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int64_t L = u.dyn[0];
  const int64_t n_vis = L - a.R + r + 1;
  const int64_t start = (int64_t)chunk * kTopkChunk;
  if (n_vis <= ka.K || start >= n_vis) return;
  int b0;
  uint32_t need;
  find_bin<kCollectThreads / 64, kRadixBins, kHistReps>(s.hist0 + (int64_t)r * kRadixBins, (uint32_t)ka.K, sh, &b0,
                                                        &need, (int64_t)ka.r_max * kRadixBins);
  for (int b = threadIdx.x; b < kRadixBins; b += kCollectThreads) lh[b] = 0;
  __syncthreads();
  const int64_t t0 = start + threadIdx.x * kPerThread;
  float v[kPerThread];
  load_chunk(s.scores + (int64_t)r * ka.p_pad, t0, v);
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t key = order_key(v[e]);
    if (t0 + e < n_vis && (key >> 21) == (uint32_t)b0) atomicAdd(&lh[(key >> 10) & 2047u], 1u);
  }
  __syncthreads();
  uint32_t* gh = s.hist1 + (int64_t)r * kRadixBins;
  for (int b = threadIdx.x; b < kRadixBins; b += kCollectThreads)
    if (lh[b]) atomicAdd(&gh[b], lh[b]);
}

// Every (key, position) whose first two digits are at or above (b0, b1), in order.
__global__ __launch_bounds__(kCollectThreads) void topk_collect_kernel(TopkKArgs ka) {
  __shared__ uint32_t sh[kCollectThreads / 64];
  const StepArgs& a = ka.a;
  const int chunk = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int64_t L = u.dyn[0];
  const int64_t n_vis = L - a.R + r + 1;
  const int64_t start = (int64_t)chunk * kTopkChunk;
  if (n_vis <= ka.K || start >= n_vis) return;
  int b0, b1;
  uint32_t need;
  find_bin<kCollectThreads / 64, kRadixBins, kHistReps>(s.hist0 + (int64_t)r * kRadixBins, (uint32_t)ka.K, sh, &b0,
                                                        &need, (int64_t)ka.r_max * kRadixBins);
  find_bin<kCollectThreads / 64, kRadixBins, 1>(s.hist1 + (int64_t)r * kRadixBins, need, sh, &b1, &need);
  const uint32_t p22 = ((uint32_t)b0 << 11) | (uint32_t)b1;

  const int64_t t0 = start + threadIdx.x * kPerThread;
  float v[kPerThread];
  load_chunk(s.scores + (int64_t)r * ka.p_pad, t0, v);
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    mine += (t0 + e < n_vis && (order_key(v[e]) >> 10) >= p22) ? 1u : 0u;
  uint32_t tot;
  uint32_t at = block_scan<kCollectThreads / 64>(mine, &tot, sh);
  int2* out = s.cand + (int64_t)r * ka.p_pad + start;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t key = order_key(v[e]);
    if (t0 + e < n_vis && (key >> 10) >= p22) out[at++] = make_int2((int)key, (int)(t0 + e));
  }
  if (threadIdx.x == 0) s.cand_n[(int64_t)r * ka.n_chunks + chunk] = tot;
}

// Candidate source for the resolve passes: LDS when the candidates fit, else global.
struct CandSrc {
  const uint32_t* lkey;     // LDS keys (or null)
  const int32_t* lpos;      // LDS positions (or null)
  const int2* gcand;        // global candidate lists of the row (by chunk)
  const uint32_t* off;      // LDS: first candidate index of each chunk
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
    const int2 kp = gcand[(int64_t)c * kTopkChunk + (i - off[c])];
    *key = (uint32_t)kp.x;
    *pos = kp.y;
  }
};

__global__ __launch_bounds__(kResolveThreads) void topk_resolve_kernel(TopkKArgs ka) {
  extern __shared__ __align__(16) uint32_t lds[];   // keys[kCandCap], pos[kCandCap]
  __shared__ uint32_t sh[kResolveWaves];
  __shared__ uint32_t hist[kRadixBins];
  __shared__ uint32_t off[kMaxChunks + 1];
  __shared__ uint32_t s_run[2];
  const StepArgs& a = ka.a;
  const int r = blockIdx.x, seq = blockIdx.y, tid = threadIdx.x;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int64_t L = u.dyn[0];
  const int64_t M = u.dyn[1];
  const int32_t round = (int32_t)u.dyn[2];
  const bool offl = ka.mode == 0;
  const int K = ka.K;
  const int64_t n_vis = L - a.R + r + 1;
  int32_t* sel = s.sel + (int64_t)r * K;
  uint32_t* h0 = s.hist0 + (int64_t)r * kRadixBins;

  if (n_vis <= K) {                                  // every visible position is selected
    for (int64_t t0 = (int64_t)tid * 16; t0 < K; t0 += (int64_t)kResolveThreads * 16) {
      int32_t poss[16];
      bool taken[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = t0 + e;
        taken[e] = t < n_vis;
        poss[e] = (int32_t)t;
        if (t < K) sel[t] = taken[e] ? (int32_t)t : -1;
      }
      mark_batch(u, s, poss, taken, offl, M, round);
    }
    for (int b = tid; b < kRadixBins; b += kResolveThreads)
      for (int q = 0; q < kHistReps; ++q) h0[(int64_t)q * ka.r_max * kRadixBins + b] = 0;
    if (tid == 0) s.sel_n[r] = (int32_t)n_vis;
    return;
  }

  int b0, b1, b2;
  uint32_t need;
  const int64_t rep_stride = (int64_t)ka.r_max * kRadixBins;
  uint32_t* h1 = s.hist1 + (int64_t)r * kRadixBins;
  find_bin<kResolveWaves, kRadixBins, kHistReps>(h0, (uint32_t)K, sh, &b0, &need, rep_stride);
  find_bin<kResolveWaves, kRadixBins, 1>(h1, need, sh, &b1, &need);
  for (int b = tid; b < kRadixBins; b += kResolveThreads) {   // consumed
    for (int q = 0; q < kHistReps; ++q) h0[q * rep_stride + b] = 0;
    h1[b] = 0;
  }

  // chunk offsets of the candidate lists
  const int n_chunks = (int)((n_vis + kTopkChunk - 1) / kTopkChunk);
  {
    const int per = (n_chunks + kResolveThreads - 1) / kResolveThreads;
    const int c0 = min(n_chunks, tid * per), c1 = min(n_chunks, c0 + per);
    uint32_t cnt = 0;
    for (int c = c0; c < c1; ++c) cnt += s.cand_n[(int64_t)r * ka.n_chunks + c];
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
  const int2* gcand = s.cand + (int64_t)r * ka.p_pad;
  CandSrc src{nullptr, nullptr, gcand, off, n_chunks};
  if (C <= (uint32_t)kCandCap) {
    // 16 consecutive candidates per thread, loads issued together
    for (uint32_t i0 = tid * 16; i0 < C; i0 += kResolveThreads * 16) {
      int c = src.chunk_of(i0);
      int2 kp[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t i = i0 + e;
        while (c + 1 < n_chunks && off[c + 1] <= i) ++c;
        kp[e] = i < C ? gcand[(int64_t)c * kTopkChunk + (i - off[c])] : make_int2(0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (i0 + e < C) {
          lkey[i0 + e] = (uint32_t)kp[e].x;
          lpos[i0 + e] = kp[e].y;
        }
    }
    src.lkey = lkey;
    src.lpos = lpos;
  }
  __syncthreads();

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
  const uint32_t E = need;

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
    uint32_t tg, te;
    uint32_t gt = run_gt + block_scan<kResolveWaves>(my_gt, &tg, sh);
    uint32_t eq = run_eq + block_scan<kResolveWaves>(my_eq, &te, sh);
    bool taken[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      taken[e] = false;
      if (i0 + e < C) {
        const uint32_t k = keys[e];
        if (k > tau) {
          sel[gt + (eq < E ? eq : E)] = poss[e];
          taken[e] = true;
          ++gt;
        } else if (k == tau) {
          if (eq < E) {
            sel[gt + eq] = poss[e];
            taken[e] = true;
          }
          ++eq;
        }
      }
    }
    mark_batch(u, s, poss, taken, offl, M, round);
    __syncthreads();
    if (tid == 0) { s_run[0] = run_gt + tg; s_run[1] = run_eq + te; }
    __syncthreads();
  }
  if (tid == 0) s.sel_n[r] = K;
}

}  // namespace

hipError_t prepare_topk_kernels() {
  return hipFuncSetAttribute((const void*)topk_resolve_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             2 * kCandCap * (int)sizeof(uint32_t));
}

hipError_t launch_topk_refine(const Geometry& g, const StepArgs& a, hipStream_t st) {
  TopkKArgs ka{a, g.p_pad, g.n_chunks, g.top_k, g.mode, g.r_max};
  const int chunks = (int)((a.l_max + kTopkChunk - 1) / kTopkChunk);
  dim3 grid((unsigned)chunks, (unsigned)a.R, (unsigned)a.n_seqs);
  hipLaunchKernelGGL(topk_refine_kernel, grid, dim3(kCollectThreads), 0, st, ka);
  return hipGetLastError();
}

hipError_t launch_topk_collect(const Geometry& g, const StepArgs& a, hipStream_t st) {
  TopkKArgs ka{a, g.p_pad, g.n_chunks, g.top_k, g.mode, g.r_max};
  const int chunks = (int)((a.l_max + kTopkChunk - 1) / kTopkChunk);
  dim3 grid((unsigned)chunks, (unsigned)a.R, (unsigned)a.n_seqs);
  hipLaunchKernelGGL(topk_collect_kernel, grid, dim3(kCollectThreads), 0, st, ka);
  return hipGetLastError();
}

hipError_t launch_topk_resolve(const Geometry& g, const StepArgs& a, hipStream_t st) {
  TopkKArgs ka{a, g.p_pad, g.n_chunks, g.top_k, g.mode, g.r_max};
  dim3 grid((unsigned)a.R, (unsigned)a.n_seqs);
  hipLaunchKernelGGL(topk_resolve_kernel, grid, dim3(kResolveThreads), 2 * kCandCap * sizeof(uint32_t), st, ka);
  return hipGetLastError();
}

}  // namespace dsa
