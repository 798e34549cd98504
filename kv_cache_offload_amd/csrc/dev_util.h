// dev_util.h -- small device helpers shared by the libdsa kernels: wave and
// workgroup scans, the order-preserving key of an fp32 score, and the radix
// bin search of the Top-K.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Order-preserving 32-bit key of an fp32 value (larger float -> larger key).
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// v plus the same register of another lane chosen by a DPP control: lanes
// whose source is outside the row (row_shr) or whose row is masked off
// (row_bcast) add 0.
template <int CTRL, int ROW_MASK>
__device__ inline uint32_t dpp_add(uint32_t v) {
  return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive scan over the 64 lanes of a wave, on DPP (no LDS traffic): shifts
// by 1, 2, 4, 8 within each 16-lane row, then lane 15 of each row into the next
// (rows 1 and 3) and lane 31 into rows 2 and 3.  Every lane of the wave must be
// active.  (lane: unused, kept for the callers.)
__device__ inline uint32_t wave_incl_scan(uint32_t v, int lane) {
  (void)lane;
  v = dpp_add<0x111, 0xf>(v);   // row_shr:1
  v = dpp_add<0x112, 0xf>(v);   // row_shr:2
  v = dpp_add<0x114, 0xf>(v);   // row_shr:4
  v = dpp_add<0x118, 0xf>(v);   // row_shr:8
  v = dpp_add<0x142, 0xa>(v);   // row_bcast:15
  v = dpp_add<0x143, 0xc>(v);   // row_bcast:31
  return v;
}

// Exclusive scan in thread order over a workgroup of NW waves; total in *tot.
// sh: NW words of LDS.  Contains two barriers; every thread must call it.
template <int NW>
__device__ inline uint32_t block_scan(uint32_t v, uint32_t* tot, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  uint32_t base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = sh[w];
    base += (w < wave) ? x : 0u;
    all += x;
  }
  __syncthreads();
  *tot = all;
  return base + inc - v;
}

// Four independent exclusive scans with one pair of barriers.  sh: 4*NW words.
template <int NW>
__device__ inline uint4 block_scan4(uint4 v, uint4* tot, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint4 inc;
  inc.x = wave_incl_scan(v.x, lane);
  inc.y = wave_incl_scan(v.y, lane);
  inc.z = wave_incl_scan(v.z, lane);
  inc.w = wave_incl_scan(v.w, lane);
  if (lane == 63) {
    sh[4 * wave + 0] = inc.x;
    sh[4 * wave + 1] = inc.y;
    sh[4 * wave + 2] = inc.z;
    sh[4 * wave + 3] = inc.w;
  }
  __syncthreads();
  uint4 base = make_uint4(0u, 0u, 0u, 0u), all = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t a = sh[4 * w], b = sh[4 * w + 1], c = sh[4 * w + 2], d = sh[4 * w + 3];
    if (w < wave) { base.x += a; base.y += b; base.z += c; base.w += d; }
    all.x += a; all.y += b; all.z += c; all.w += d;
  }
  __syncthreads();
  *tot = all;
  return make_uint4(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z, base.w + inc.w - v.w);
}

// The bin holding the k-th largest key, from counts already in registers: each
// thread holds the PER contiguous bins lo(tid) .. lo(tid) + PER - 1 with
// lo(tid) = NBINS - (tid + 1) PER (thread 0 owns the highest).  Returns the
// largest b with suffix(b) >= k and the number of keys still needed from it.
// Every thread of the workgroup must call it.
template <int NW, int NBINS, int PER>
__device__ inline void find_bin_regs(const uint32_t* c, uint32_t k, uint32_t* sh, int* out_bin,
                                     uint32_t* out_need) {
  static_assert(PER >= 1 && NBINS == NW * 64 * PER, "bins per thread");
  __shared__ int s_bin;
  __shared__ uint32_t s_need;
  const int lo = NBINS - ((int)threadIdx.x + 1) * PER;
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

// This thread's bins of hist[NBINS] (summed over REPS replicas `stride` apart),
// in the layout find_bin_regs expects.  hist may be in global memory or LDS.
template <int NW, int NBINS, int REPS, class HistPtr>
__device__ inline void load_bins(HistPtr hist, uint32_t* c, int64_t stride = 0) {
  constexpr int PER = NBINS / (NW * 64);
  const int lo = NBINS - ((int)threadIdx.x + 1) * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) c[e] = 0;
#pragma unroll
  for (int q = 0; q < REPS; ++q)
#pragma unroll
    for (int e = 0; e < PER; ++e) c[e] += hist[q * stride + lo + e];
}

// The bin holding the k-th largest key among those counted in hist[NBINS] (summed
// over REPS replicas `stride` apart): the largest b with suffix(b) >= k, and the
// number of keys still needed from it.  Every thread of the workgroup must call it.
template <int NW, int NBINS, int REPS, class HistPtr>
__device__ inline void find_bin(HistPtr hist, uint32_t k, uint32_t* sh, int* out_bin,
                                uint32_t* out_need, int64_t stride = 0) {
  constexpr int PER = NBINS / (NW * 64);
  static_assert(PER >= 1 && NBINS % (NW * 64) == 0, "bins per thread");
  uint32_t c[PER];
  load_bins<NW, NBINS, REPS>(hist, c, stride);
  find_bin_regs<NW, NBINS, PER>(c, k, sh, out_bin, out_need);
}

// Lanes below this one, as a 64-bit mask.
__device__ inline uint64_t lanes_below(int lane) {
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

}  // namespace dsa
