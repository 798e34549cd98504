// k_gather.hip -- GPU-managed hot gather, recent ring, append, flush and warm.
//
// Page "From 1M total to 15+ streams x 1M: the capacity breakthrough of
// GLM-5.3 KV cache offload" (zhuai.tech):
//   * section "Decision 3: let the GPU manage the hot cache directly": the
//     selection stays on the GPU, the GPU looks up hot slots, a hit reads HBM,
//     a miss reads the registered host mirror, and the result is a compact
//     selection for attention; new rows go to a GPU recent ring and are written
//     back to host memory in batches;
//   * section "GPU cache management errs too": a slot filled in this round is
//     a hit source only from the next round, repeated misses of one round read
//     host memory, slots in use are pinned first, and replacement is a ring
//     walk that skips the currently pinned slots;
//   * section "Decision 2": 64-row batched writeback instead of per-row copies;
//   * section "Capacity must survive the session lifecycle": flush before the
//     full history is exported.
//
// gfx950 design.  The plan is one 1024-thread workgroup per sequence working
// in LDS: the R sorted selections are merged pairwise with merge-path
// partitioning, duplicates are dropped with a block scan (a position several
// rows select is read once, which is how "repeated misses read host memory"
// holds structurally), each union entry is classified on the round-start
// state, hits are pinned, and the k-th miss in ascending position order takes
// the k-th unpinned slot after the hand, found from a bitmap of pinned slots
// over the window the walk can reach and a prefix count of unpinned slots per
// 32-slot word.  The copy is a separate wide kernel: one thread per 16-byte
// piece of a row, loading from the hot slot, the ring, or the host mirror
// (zero-copy reads of pinned host memory over the host link), storing to the
// compact buffer and, for a miss that got a slot, to the slot as well.  No
// workgroup ever reads a slot filled in the same round.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kMaxPer = kMaxUnion / kPlanThreads;   // 16 elements per thread at most

__device__ inline uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive block scan over 1024 threads (thread order); total in *tot.
__device__ inline uint32_t block_scan(uint32_t v, uint32_t* tot, uint32_t* sh /*[16]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  uint32_t base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    uint32_t x = sh[w];
    base += (w < wave) ? x : 0u;
    all += x;
  }
  __syncthreads();
  *tot = all;
  return base + inc - v;
}

// Stable merge of sorted A[na] and B[nb] into dst by all threads (merge path).
__device__ inline void merge_pair(const uint32_t* A, int na, const uint32_t* B, int nb, uint32_t* dst) {
  const int total = na + nb;
  const int per = (total + kPlanThreads - 1) / kPlanThreads;
  const int d0 = threadIdx.x * per;
  if (d0 >= total) return;
  const int d1 = min(total, d0 + per);
  int lo = max(0, d0 - nb), hi = min(d0, na);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (A[mid] <= B[d0 - 1 - mid]) lo = mid + 1;
    else hi = mid;
  }
  int i = lo, j = d0 - lo;
  for (int d = d0; d < d1; ++d) {
    if (j >= nb || (i < na && A[i] <= B[j])) dst[d] = A[i++];
    else dst[d] = B[j++];
  }
}

__device__ inline int nth_set_bit(uint32_t x, int n) {
  for (int i = 0; i < n; ++i) x &= x - 1;
  return __ffs(x) - 1;
}

struct PlanKArgs {
  StepArgs a;
  int K, S, ring_cap, ring_rows, mode;
};

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanKArgs ka) {
  extern __shared__ __align__(16) uint32_t lds[];   // two buffers of R*K entries
  __shared__ uint32_t sh_scan[kPlanWaves];
  __shared__ int s_off[9], s_n[9];
  __shared__ uint32_t bm[kMaxUnion / 32];            // pinned bitmap, then unpinned words
  __shared__ uint32_t wpre[kMaxUnion / 32];          // exclusive prefix of unpinned counts
  __shared__ int s_new_hand;

  const StepArgs& a = ka.a;
  const int seq = blockIdx.x;
  const int tid = threadIdx.x;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int R = a.R, K = ka.K, S = ka.S;
  const int64_t L = u.dyn[0], M = u.dyn[1];
  const int32_t round = (int32_t)u.dyn[2];
  const int hand = ka.mode == 0 ? *u.hand : 0;
  uint32_t* X = lds;
  uint32_t* Y = lds + R * K;

  // 1. the R selections, concatenated
  if (tid < R) s_n[tid] = s.sel_n[tid];
  __syncthreads();
  if (tid == 0) {
    int o = 0;
    for (int i = 0; i < R; ++i) { s_off[i] = o; o += s_n[i]; }
    s_off[R] = o;
  }
  __syncthreads();
  const int total = s_off[R];
  for (int i = 0; i < R; ++i)
    for (int j = tid; j < s_n[i]; j += kPlanThreads) X[s_off[i] + j] = (uint32_t)s.sel[i * K + j];
  __syncthreads();

  // 2. pairwise merge rounds
  uint32_t* cur = X;
  uint32_t* nxt = Y;
  int nl = R;
  while (nl > 1) {
    for (int p = 0; p + 1 < nl; p += 2) {
      merge_pair(cur + s_off[p], s_n[p], cur + s_off[p + 1], s_n[p + 1], nxt + s_off[p]);
      __syncthreads();
    }
    if (nl & 1)
      for (int j = tid; j < s_n[nl - 1]; j += kPlanThreads) nxt[s_off[nl - 1] + j] = cur[s_off[nl - 1] + j];
    __syncthreads();
    if (tid == 0) {
      int q = 0;
      for (int p = 0; p < nl; p += 2) {
        s_off[q] = s_off[p];
        s_n[q] = s_n[p] + (p + 1 < nl ? s_n[p + 1] : 0);
        ++q;
      }
    }
    __syncthreads();
    uint32_t* t = cur; cur = nxt; nxt = t;
    nl = (nl + 1) >> 1;
  }

  // 3. drop duplicates: union U in ascending order, into nxt
  uint32_t U;
  {
    const int per = (total + kPlanThreads - 1) / kPlanThreads;
    const int x0 = min(total, tid * per), x1 = min(total, x0 + per);
    uint32_t cnt = 0;
    for (int x = x0; x < x1; ++x) cnt += (x == 0 || cur[x] != cur[x - 1]);
    uint32_t base = block_scan(cnt, &U, sh_scan);
    for (int x = x0; x < x1; ++x)
      if (x == 0 || cur[x] != cur[x - 1]) nxt[base++] = cur[x];
  }
  __syncthreads();
  const uint32_t* uni = nxt;
  for (uint32_t x = tid; x < U; x += kPlanThreads) s.uni[x] = (int32_t)uni[x];

  // 4. map every selected position to its union index
  for (int i = 0; i < R; ++i) {
    for (int j = tid; j < K; j += kPlanThreads) {
      int32_t m = -1;
      if (j < s.sel_n[i]) {
        const uint32_t pos = (uint32_t)s.sel[i * K + j];
        uint32_t lo = 0, hi = U;
        while (lo < hi) {
          const uint32_t mid = (lo + hi) >> 1;
          if (uni[mid] < pos) lo = mid + 1;
          else hi = mid;
        }
        m = (int32_t)lo;
      }
      s.map[i * K + j] = m;
    }
  }

  // 5. classify on the round-start state; pin hits
  const int per = ((int)U + kPlanThreads - 1) / kPlanThreads;   // <= kMaxPer
  const int x0 = min((int)U, tid * per), x1 = min((int)U, x0 + per);
  int32_t kind[kMaxPer], src[kMaxPer];
  uint32_t my_hit = 0, my_ring = 0, my_miss = 0;
  if (ka.mode == 1) {
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e) {
      const int x = x0 + e;
      kind[e] = SRC_RES;
      src[e] = x < x1 ? (int32_t)uni[x] : -1;
    }
  } else {
    int32_t v[kMaxPer];
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e) {
      const int x = x0 + e;
      v[e] = -1;
      if (x < x1) {
        const int64_t pos = uni[x];
        if (pos < M) v[e] = u.pos_slot[pos];
      }
    }
    int32_t fr[kMaxPer];
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e) fr[e] = (x0 + e < x1 && v[e] >= 0) ? u.fill_round[v[e]] : 0;
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e) {
      const int x = x0 + e;
      kind[e] = SRC_RES;
      src[e] = -1;
      if (x >= x1) continue;
      const int64_t pos = uni[x];
      if (pos >= M) {
        kind[e] = SRC_RING; src[e] = (int32_t)(pos % ka.ring_cap); ++my_ring;
      } else if (v[e] >= 0 && fr[e] < round) {
        kind[e] = SRC_HIT; src[e] = v[e]; ++my_hit;
        u.pin_round[v[e]] = round;
      } else {
        kind[e] = SRC_MISS; src[e] = (int32_t)pos; ++my_miss;
      }
    }
  }
  uint32_t n_hit, n_ring, n_miss;
  const uint32_t miss_base = block_scan(my_miss, &n_miss, sh_scan);
  block_scan(my_hit, &n_hit, sh_scan);
  block_scan(my_ring, &n_ring, sh_scan);

  // 6. replacement window: the walk from the hand reaches at most n_miss + n_hit slots
  uint32_t n_assigned = 0, evicted = 0;
  if (ka.mode == 0) {
    const uint32_t W = min((uint32_t)S, n_miss + n_hit);
    const uint32_t nw = (W + 31) / 32;
    for (uint32_t w = tid; w < nw; w += kPlanThreads) bm[w] = 0;
    if (tid == 0) s_new_hand = hand;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e)
      if (x0 + e < x1 && kind[e] == SRC_HIT) {
        const uint32_t off = (uint32_t)((src[e] - hand + S) % S);
        if (off < W) atomicOr(&bm[off >> 5], 1u << (off & 31));
      }
    __syncthreads();
    uint32_t uw = 0;
    if ((uint32_t)tid < nw) {
      const uint32_t valid = ((uint32_t)tid + 1) * 32 <= W ? 0xFFFFFFFFu : ((1u << (W & 31)) - 1u);
      uw = ~bm[tid] & valid;
    }
    uint32_t n_unpinned;
    const uint32_t wbase = block_scan(__popc(uw), &n_unpinned, sh_scan);
    if ((uint32_t)tid < nw) { bm[tid] = uw; wpre[tid] = wbase; }
    __syncthreads();
    n_assigned = min(n_miss, n_unpinned);

    // 7. misses in ascending position order take the unpinned slots in ring order
    uint32_t k = miss_base;
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e) {
      if (x0 + e >= x1 || kind[e] != SRC_MISS) continue;
      if (k < n_assigned) {
        uint32_t lo = 0, hi = nw;            // last word with wpre <= k
        while (hi - lo > 1) {
          const uint32_t mid = (lo + hi) >> 1;
          if (wpre[mid] <= k) lo = mid;
          else hi = mid;
        }
        const uint32_t off = lo * 32 + nth_set_bit(bm[lo], (int)(k - wpre[lo]));
        const int32_t vslot = (int32_t)((hand + off) % (uint32_t)S);
        const int32_t pos = src[e];
        const int32_t old = u.slot_pos[vslot];
        if (old >= 0) { u.pos_slot[old] = -1; ++evicted; }
        u.slot_pos[vslot] = pos;
        u.pos_slot[pos] = vslot;
        u.fill_round[vslot] = round;
        u.pin_round[vslot] = round;
        s.fill[x0 + e] = vslot;
        if (k + 1 == n_assigned) s_new_hand = (vslot + 1) % S;
      } else {
        kind[e] = SRC_MISS_NOSLOT;
        s.fill[x0 + e] = -1;
      }
      ++k;
    }
  }
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) {
    if (x0 + e >= x1) continue;
    s.kind[x0 + e] = kind[e];
    s.src[x0 + e] = src[e];
    if (kind[e] != SRC_MISS) s.fill[x0 + e] = -1;
  }
  uint32_t n_evict;
  block_scan(evicted, &n_evict, sh_scan);

  // 8. counters, writeback decision, state for the next round
  if (tid == 0) {
    const int64_t rb = 656;
    const int64_t noslot = (int64_t)n_miss - n_assigned;
    s.counters[0] = U;
    s.counters[1] = ka.mode == 0 ? n_hit : 0;
    s.counters[2] = ka.mode == 0 ? n_ring : 0;
    s.counters[3] = ka.mode == 0 ? n_assigned : 0;
    s.counters[4] = ka.mode == 0 ? noslot : 0;
    s.counters[5] = n_evict;
    s.counters[6] = ka.mode == 0 ? ((int64_t)n_assigned + noslot) * rb : 0;
    s.counters[7] = ka.mode == 1 ? U : 0;
    s.info[0] = U;
    int64_t wb = -1;
    if (ka.mode == 0 && L - M >= ka.ring_rows) wb = M;
    s.info[1] = wb;
    if (ka.mode == 0) {
      *u.hand = s_new_hand;
      if (wb >= 0) u.dyn[1] = M + ka.ring_rows;
    }
    u.dyn[2] = round + 1;
  }
}

struct CopyKArgs {
  StepArgs a;
  int row_bytes, ring_cap, ring_rows;
};

__global__ __launch_bounds__(256) void copy_kernel(CopyKArgs ka) {
  const StepArgs& a = ka.a;
  const int seq = blockIdx.y;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int64_t U = s.info[0];
  const int64_t wb = s.info[1];
  const int64_t rb = ka.row_bytes;
  const int64_t n_gather = U * kCopyChunks16;
  const int64_t total = n_gather + (wb >= 0 ? (int64_t)ka.ring_rows * kCopyChunks16 : 0);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    if (t < n_gather) {
      const int64_t x = t / kCopyChunks16, c = t % kCopyChunks16;
      const int32_t kind = s.kind[x];
      const int64_t src = s.src[x];
      const uint8_t* from = kind == SRC_HIT ? u.slots + src * rb
                          : kind == SRC_RING ? u.ring + src * rb
                          : u.rows + src * rb;
      const uint4 v = *reinterpret_cast<const uint4*>(from + c * 16);
      *reinterpret_cast<uint4*>(s.compact + x * rb + c * 16) = v;
      if (kind == SRC_MISS) {
        const int32_t f = s.fill[x];
        if (f >= 0) *reinterpret_cast<uint4*>(u.slots + (int64_t)f * rb + c * 16) = v;
      }
    } else {
      const int64_t w = t - n_gather;
      const int64_t p = wb + w / kCopyChunks16, c = w % kCopyChunks16;
      const uint4 v = *reinterpret_cast<const uint4*>(u.ring + (p % ka.ring_cap) * rb + c * 16);
      *reinterpret_cast<uint4*>(u.rows + p * rb + c * 16) = v;
    }
  }
}

// ---- unit maintenance ----

struct AppendKArgs {
  UnitDev u;
  int64_t L, newM, n;
  const uint16_t* keys;
  const uint8_t* rows;
  int row_bytes, ring_cap, index_dim, mode;
};

// Keys to the key store; rows to the mirror (positions below newM), the ring
// (offload) or the HBM row store (resident).  Block 0 publishes the new L, M.
__global__ __launch_bounds__(256) void append_kernel(AppendKArgs ka) {
  const int64_t key_chunks = ka.n * ka.index_dim / 8;      // 16-byte pieces
  const int64_t row_chunks = ka.n * kCopyChunks16;
  const int64_t rb = ka.row_bytes;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < key_chunks + row_chunks;
       t += (int64_t)gridDim.x * blockDim.x) {
    if (t < key_chunks) {
      reinterpret_cast<uint4*>(ka.u.keys + ka.L * ka.index_dim)[t] = reinterpret_cast<const uint4*>(ka.keys)[t];
    } else {
      const int64_t w = t - key_chunks;
      const int64_t i = w / kCopyChunks16, c = w % kCopyChunks16;
      const int64_t p = ka.L + i;
      const uint4 v = *reinterpret_cast<const uint4*>(ka.rows + i * rb + c * 16);
      uint8_t* dst = (ka.mode == 1 || p < ka.newM) ? ka.u.rows + p * rb : ka.u.ring + (p % ka.ring_cap) * rb;
      *reinterpret_cast<uint4*>(dst + c * 16) = v;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ka.u.dyn[0] = ka.L + ka.n;
    ka.u.dyn[1] = ka.mode == 1 ? ka.L + ka.n : ka.newM;
  }
}

// Ring rows [from, to) to the mirror; then M = to.
__global__ __launch_bounds__(256) void ring_to_mirror_kernel(UnitDev u, int64_t from, int64_t to,
                                                             int row_bytes, int ring_cap) {
  const int64_t total = (to - from) * kCopyChunks16;
  const int64_t rb = row_bytes;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = from + t / kCopyChunks16, c = t % kCopyChunks16;
    const uint4 v = *reinterpret_cast<const uint4*>(u.ring + (p % ring_cap) * rb + c * 16);
    *reinterpret_cast<uint4*>(u.rows + p * rb + c * 16) = v;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) u.dyn[1] = to;
}

// Warm, phase 1: forget the positions currently cached.
__global__ __launch_bounds__(256) void warm_clear_kernel(UnitDev u, int S) {
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < S; v += gridDim.x * blockDim.x) {
    const int32_t old = u.slot_pos[v];
    if (old >= 0) u.pos_slot[old] = -1;
  }
}

// Warm, phase 2: slot v <- position L-n+v for v < n; other slots empty; no round marks.
__global__ __launch_bounds__(256) void warm_fill_kernel(UnitDev u, int S, int64_t L, int64_t n, int row_bytes) {
  const int64_t rb = row_bytes;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < S; v += (int64_t)gridDim.x * blockDim.x) {
    const int32_t pos = v < n ? (int32_t)(L - n + v) : -1;
    u.slot_pos[v] = pos;
    u.fill_round[v] = -1;
    u.pin_round[v] = -1;
    if (pos >= 0) u.pos_slot[pos] = (int32_t)v;
  }
  const int64_t total = n * kCopyChunks16;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = t / kCopyChunks16, c = t % kCopyChunks16;
    const uint4 x = *reinterpret_cast<const uint4*>(u.rows + (L - n + v) * rb + c * 16);
    *reinterpret_cast<uint4*>(u.slots + v * rb + c * 16) = x;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *u.hand = (int32_t)(n % S);
}

unsigned grid_for(int64_t work, int64_t cap = 4096) {
  int64_t b = (work + 255) / 256;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (unsigned)b;
}

}  // namespace

hipError_t prepare_gather_kernels() {
  return hipFuncSetAttribute((const void*)plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             2 * kMaxUnion * (int)sizeof(uint32_t));
}

hipError_t launch_plan(const Geometry& g, const StepArgs& a, hipStream_t st) {
  PlanKArgs ka{a, g.top_k, g.hot_slots, g.ring_cap, g.ring_rows, g.mode};
  const size_t lds = 2 * (size_t)a.R * g.top_k * sizeof(uint32_t);
  hipLaunchKernelGGL(plan_kernel, dim3((unsigned)a.n_seqs), dim3(kPlanThreads), lds, st, ka);
  return hipGetLastError();
}

hipError_t launch_copy(const Geometry& g, const StepArgs& a, hipStream_t st) {
  CopyKArgs ka{a, g.row_bytes, g.ring_cap, g.ring_rows};
  const int64_t work = (int64_t)a.R * g.top_k * kCopyChunks16 + (int64_t)g.ring_rows * kCopyChunks16;
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(work, 2048), (unsigned)a.n_seqs), dim3(256), 0, st, ka);
  return hipGetLastError();
}

hipError_t launch_append(const Geometry& g, const UnitDev& unit, int64_t L, int64_t M, int64_t newM,
                         int64_t n, const uint16_t* keys, const uint8_t* rows, hipStream_t st) {
  if (g.mode == 0 && newM > M && M < L) {
    const int64_t to = newM < L ? newM : L;
    hipLaunchKernelGGL(ring_to_mirror_kernel, dim3(grid_for((to - M) * kCopyChunks16)), dim3(256), 0, st,
                       unit, M, to, g.row_bytes, g.ring_cap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  AppendKArgs ka{unit, L, newM, n, keys, rows, g.row_bytes, g.ring_cap, g.index_dim, g.mode};
  const int64_t work = n * g.index_dim / 8 + n * kCopyChunks16;
  hipLaunchKernelGGL(append_kernel, dim3(grid_for(work)), dim3(256), 0, st, ka);
  return hipGetLastError();
}

hipError_t launch_flush(const Geometry& g, const UnitDev& unit, int64_t M, int64_t L, hipStream_t st) {
  hipLaunchKernelGGL(ring_to_mirror_kernel, dim3(grid_for((L - M) * kCopyChunks16)), dim3(256), 0, st,
                     unit, M, L, g.row_bytes, g.ring_cap);
  return hipGetLastError();
}

hipError_t launch_warm(const Geometry& g, const UnitDev& unit, int64_t L, hipStream_t st) {
  const int64_t n = L < g.hot_slots ? L : g.hot_slots;
  hipLaunchKernelGGL(warm_clear_kernel, dim3(grid_for(g.hot_slots)), dim3(256), 0, st, unit, g.hot_slots);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(warm_fill_kernel, dim3(grid_for(n * kCopyChunks16 > g.hot_slots ? n * kCopyChunks16 : g.hot_slots)),
                     dim3(256), 0, st, unit, g.hot_slots, L, n, g.row_bytes);
  return hipGetLastError();
}

}  // namespace dsa
