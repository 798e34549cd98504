// k_topk.hip -- exact Top-K per query row, ties broken by the lower position.
//
// The GPU computes the exact Top-K (page "From 1M total to 15+ streams x 1M:
// the capacity breakthrough of GLM-5.3 KV cache offload", section "Decision 1":
// an approximate CPU selection moved the cutoff and was rejected).
//
// Radix select over order-preserving 32-bit keys of the fp32 scores, in three
// digit passes (bits 31..21, 20..10, 9..0).  Every workgroup owns a chunk of
// 4096 positions of one row, builds an LDS histogram of the current digit for
// the keys that match the prefix found so far, and adds it to the row's global
// histogram.  Each workgroup of the next pass re-derives the prefix from the
// finished histograms itself (a 2048-bin suffix scan), so no serial pass runs
// between them.  The last pass also stores each chunk's suffix sums of the
// last digit; the emit kernel turns them into per-chunk counts of keys above
// the threshold and equal to it, and writes the selection in ascending
// position order with an ordered block scan: every key above the threshold,
// plus the lowest-position keys equal to it until K are taken.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kTopkChunk / kThreads;  // 16 consecutive positions per thread

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide inclusive scan helpers over 256 threads (4 waves).
__device__ inline uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Returns the exclusive prefix of v over the block (thread order); total in *tot.
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* tot, uint32_t* sh /*[8]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  uint32_t base = 0, all = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    uint32_t x = sh[w];
    if (w < wave) base += x;
    all += x;
  }
  __syncthreads();
  *tot = all;
  return base + inc - v;
}

// Find the digit bin that holds the k-th largest key among those counted in
// hist[nbins]: the largest b with suffix(b) >= k.  Returns b and the number of
// keys still needed from bin b (k - suffix(b+1)).  Every thread gets the result.
__device__ inline void find_bin(const uint32_t* __restrict__ hist, int nbins, uint32_t k,
                                uint32_t* sh_scan, int* out_bin, uint32_t* out_need) {
  __shared__ int s_bin;
  __shared__ uint32_t s_need;
  // each thread owns a contiguous block of bins, scanned from the top
  const int per = nbins / kThreads;            // 8 or 4
  const int hi = nbins - 1 - threadIdx.x * per;  // thread 0 owns the highest bins
  uint32_t local = 0;
  for (int e = 0; e < per; ++e) local += hist[hi - e];
  uint32_t tot;
  uint32_t before = block_excl_scan(local, &tot, sh_scan);   // keys in higher bins
  if (before < k && before + local >= k) {
    uint32_t acc = before;
    for (int e = 0; e < per; ++e) {
      uint32_t c = hist[hi - e];
      if (acc + c >= k) {
        s_bin = hi - e;
        s_need = k - acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  *out_bin = s_bin;
  *out_need = s_need;
  __syncthreads();
}

struct TopkKArgs {
  StepArgs a;
  int64_t p_pad;
  int n_chunks;
  int K;
  int pass;
};

__device__ inline const uint32_t* row_hist(const SeqScratch& s, int parity, int r_max, int r, int pass) {
  return s.hist + (((int64_t)parity * r_max + r) * 3 + pass) * kRadixBins;
}

__global__ __launch_bounds__(kThreads) void topk_hist_kernel(TopkKArgs ka, int r_max) {
  __shared__ uint32_t lh[kRadixBins];
  __shared__ uint32_t sh_scan[8];
  const StepArgs& a = ka.a;
  const int chunk = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int64_t L = u.dyn[0];
  const int64_t n_vis = L - a.R + r + 1;
  const int64_t start = (int64_t)chunk * kTopkChunk;
  if (n_vis <= ka.K) return;                     // everything visible is selected
  const int pass = ka.pass;

  // Prefix of the threshold found by the earlier passes.
  uint32_t need = (uint32_t)ka.K;
  uint32_t prefix = 0;
  if (pass >= 1) {
    int b0;
    find_bin(row_hist(s, a.parity, r_max, r, 0), kRadixBins, need, sh_scan, &b0, &need);
    prefix = (uint32_t)b0;
  }
  if (pass >= 2) {
    int b1;
    find_bin(row_hist(s, a.parity, r_max, r, 1), kRadixBins, need, sh_scan, &b1, &need);
    prefix = (prefix << 11) | (uint32_t)b1;
  }
  const int nbins = pass == 2 ? 1024 : kRadixBins;
  for (int b = threadIdx.x; b < nbins; b += kThreads) lh[b] = 0;
  __syncthreads();

  const float* sc = s.scores + (int64_t)r * ka.p_pad;
  uint32_t gt22 = 0;
  if (start < n_vis) {
    const int64_t t_begin = start + threadIdx.x * kPerThread;
    for (int e = 0; e < kPerThread; ++e) {
      const int64_t t = t_begin + e;
      if (t >= n_vis) break;
      const uint32_t key = order_key(sc[t]);
      if (pass == 0) {
        atomicAdd(&lh[key >> 21], 1u);
      } else if (pass == 1) {
        if ((key >> 21) == prefix) atomicAdd(&lh[(key >> 10) & 2047u], 1u);
      } else {
        const uint32_t p22 = key >> 10;
        if (p22 == prefix) atomicAdd(&lh[key & 1023u], 1u);
        else if (p22 > prefix) ++gt22;
      }
    }
  }
  __syncthreads();
  uint32_t* gh = const_cast<uint32_t*>(row_hist(s, a.parity, r_max, r, pass));
  for (int b = threadIdx.x; b < nbins; b += kThreads)
    if (lh[b]) atomicAdd(&gh[b], lh[b]);
  if (pass == 2) {
    // Chunk suffix sums of the last digit: suf[b] = sum of lh[b..1023], suf[1024] = 0.
    uint32_t* suf = s.suffix + ((int64_t)r * ka.n_chunks + chunk) * kSuffixLen;
    const int per = 1024 / kThreads;                 // 4 bins per thread, from the top
    const int hi = 1023 - threadIdx.x * per;
    uint32_t local = 0;
    for (int e = 0; e < per; ++e) local += lh[hi - e];
    uint32_t tot;
    uint32_t above = block_excl_scan(local, &tot, sh_scan);
    uint32_t acc = above;
    for (int e = 0; e < per; ++e) {
      acc += lh[hi - e];
      suf[hi - e] = acc;
    }
    if (threadIdx.x == 0) suf[1024] = 0;
    uint32_t tot_gt;
    block_excl_scan(gt22, &tot_gt, sh_scan);
    if (threadIdx.x == 0) s.gt22[(int64_t)r * ka.n_chunks + chunk] = tot_gt;
  }
}

__global__ __launch_bounds__(kThreads) void topk_emit_kernel(TopkKArgs ka, int r_max) {
  __shared__ uint32_t sh_scan[8];
  __shared__ uint32_t s_base[2];
  const StepArgs& a = ka.a;
  const int chunk = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int64_t L = u.dyn[0];
  const int K = ka.K;
  const int64_t n_vis = L - a.R + r + 1;
  const int64_t start = (int64_t)chunk * kTopkChunk;
  int32_t* sel = s.sel + (int64_t)r * K;

  // Clear the other parity's histograms for the next step: this row, and (from
  // row 0) the rows this step does not use, which an earlier step may have left.
  if (chunk == 0) {
    uint32_t* nxt = s.hist + (((int64_t)(a.parity ^ 1) * r_max + r) * 3) * kRadixBins;
    for (int b = threadIdx.x; b < 3 * kRadixBins; b += kThreads) nxt[b] = 0;
    if (r == 0) {
      uint32_t* rest = s.hist + (((int64_t)(a.parity ^ 1) * r_max + a.R) * 3) * kRadixBins;
      for (int64_t b = threadIdx.x; b < (int64_t)(r_max - a.R) * 3 * kRadixBins; b += kThreads) rest[b] = 0;
    }
  }

  if (n_vis <= K) {
    // every visible position is selected, in order
    for (int64_t t = start + threadIdx.x; t < start + kTopkChunk && t < n_vis; t += kThreads)
      sel[t] = (int32_t)t;
    if (chunk == 0) {
      for (int64_t j = n_vis + threadIdx.x; j < K; j += kThreads) sel[j] = -1;
      if (threadIdx.x == 0) s.sel_n[r] = (int32_t)n_vis;
    }
    return;
  }
  if (start >= n_vis) return;

  // Threshold key tau and the number E of keys equal to tau that are taken.
  uint32_t need = (uint32_t)K;
  int b0, b1, b2;
  find_bin(row_hist(s, a.parity, r_max, r, 0), kRadixBins, need, sh_scan, &b0, &need);
  find_bin(row_hist(s, a.parity, r_max, r, 1), kRadixBins, need, sh_scan, &b1, &need);
  find_bin(row_hist(s, a.parity, r_max, r, 2), 1024, need, sh_scan, &b2, &need);
  const uint32_t tau = ((uint32_t)b0 << 21) | ((uint32_t)b1 << 10) | (uint32_t)b2;
  const uint32_t E = need;

  // Counts of earlier chunks: above tau and equal to tau.
  uint32_t gt_before = 0, eq_before = 0;
  for (int c = threadIdx.x; c < chunk; c += kThreads) {
    const uint32_t* suf = s.suffix + ((int64_t)r * ka.n_chunks + c) * kSuffixLen;
    const uint32_t above = suf[b2 + 1];
    gt_before += s.gt22[(int64_t)r * ka.n_chunks + c] + above;
    eq_before += suf[b2] - above;
  }
  uint32_t tot;
  block_excl_scan(gt_before, &tot, sh_scan);
  if (threadIdx.x == 0) s_base[0] = tot;
  block_excl_scan(eq_before, &tot, sh_scan);
  if (threadIdx.x == 0) s_base[1] = tot;
  __syncthreads();
  const uint32_t base_gt = s_base[0], base_eq = s_base[1];

  // This thread's 16 consecutive positions.
  const float* sc = s.scores + (int64_t)r * ka.p_pad;
  const int64_t t_begin = start + threadIdx.x * kPerThread;
  uint32_t keys[kPerThread];
  uint32_t my_gt = 0, my_eq = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int64_t t = t_begin + e;
    keys[e] = t < n_vis ? order_key(sc[t]) : 0u;
    if (t < n_vis) {
      my_gt += keys[e] > tau;
      my_eq += keys[e] == tau;
    }
  }
  uint32_t gt_pre = block_excl_scan(my_gt, &tot, sh_scan);
  uint32_t eq_pre = block_excl_scan(my_eq, &tot, sh_scan);
  uint32_t gt_run = base_gt + gt_pre, eq_run = base_eq + eq_pre;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int64_t t = t_begin + e;
    if (t >= n_vis) break;
    const uint32_t k = keys[e];
    if (k > tau) {
      sel[gt_run + (eq_run < E ? eq_run : E)] = (int32_t)t;
      ++gt_run;
    } else if (k == tau) {
      if (eq_run < E) sel[gt_run + eq_run] = (int32_t)t;
      ++eq_run;
    }
  }
  if (chunk == 0 && threadIdx.x == 0) s.sel_n[r] = K;
}

}  // namespace

hipError_t launch_topk_hist(const Geometry& g, const StepArgs& a, int pass, hipStream_t st) {
  TopkKArgs ka{a, g.p_pad, g.n_chunks, g.top_k, pass};
  const int chunks = (int)((a.l_max + kTopkChunk - 1) / kTopkChunk);
  dim3 grid((unsigned)chunks, (unsigned)a.R, (unsigned)a.n_seqs);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, st, ka, g.r_max);
  return hipGetLastError();
}

hipError_t launch_topk_emit(const Geometry& g, const StepArgs& a, hipStream_t st) {
  TopkKArgs ka{a, g.p_pad, g.n_chunks, g.top_k, 3};
  const int chunks = (int)((a.l_max + kTopkChunk - 1) / kTopkChunk);
  dim3 grid((unsigned)chunks, (unsigned)a.R, (unsigned)a.n_seqs);
  hipLaunchKernelGGL(topk_emit_kernel, grid, dim3(kThreads), 0, st, ka, g.r_max);
  return hipGetLastError();
}

}  // namespace dsa
