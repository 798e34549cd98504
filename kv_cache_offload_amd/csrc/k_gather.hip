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
// gfx950 design.  Selection, classification and pinning happen where the
// selection is produced: the top-k emit kernel sets, for every selected
// position, a bit in a per-position selection bitmap (so a position several
// rows select is one union entry -- "repeated misses read host memory" holds
// structurally: one host read per distinct position), classifies it against
// the round-start state (a hit needs a slot filled in an earlier round) and
// pins the hit's slot.  The gather scan is one workgroup per sequence: it turns
// the bitmaps into per-32-position-word prefix counts of union entries and of
// misses, and the pinned-slot bitmap into a per-word prefix of unpinned slots in
// ring order from the hand, and lists the victim slot of the k-th miss.  The
// gather assign kernel is wide: one wave per 32-position word, one lane per
// position; the k-th miss in ascending position order takes victim[k], evicts
// its old position and fills the slot table.  The copy is a separate
// wide kernel: one thread per 16-byte piece of a row, loading from the hot
// slot, the ring, or the host mirror (zero-copy reads of pinned host memory
// over the host link), storing to the compact buffer and, for a miss that got
// a slot, to the slot as well.  No thread ever reads a slot filled in the same
// round.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;

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
  for (int w = 0; w < kScanWaves; ++w) {
    uint32_t x = sh[w];
    base += (w < wave) ? x : 0u;
    all += x;
  }
  __syncthreads();
  *tot = all;
  return base + inc - v;
}

// Bits of word w (positions 32w..32w+31) that lie at or above M.
__device__ inline uint32_t ring_bits(int64_t w, int64_t M) {
  const int64_t first = w * 32;
  if (first >= M) return 0xFFFFFFFFu;
  if (first + 32 <= M) return 0u;
  return ~((1u << (uint32_t)(M - first)) - 1u);
}

struct ScanKArgs {
  StepArgs a;
  int S, s_words, ring_rows, mode;
};

__global__ __launch_bounds__(kScanThreads) void gather_scan_kernel(ScanKArgs ka) {
  __shared__ uint32_t sh[kScanWaves];
  __shared__ int s_hand;
  const StepArgs& a = ka.a;
  const int seq = blockIdx.x, tid = threadIdx.x;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int64_t L = u.dyn[0], M = u.dyn[1];
  const int32_t round = (int32_t)u.dyn[2];
  const bool off = ka.mode == 0;
  const int hand = off ? *u.hand : 0;
  const int64_t nw = (L + 31) / 32;
  const uint32_t* sel = s.selmask;
  const uint32_t* hit = s.hitmask;

  // Union and miss counts per word, scanned in word (= position) order.
  const int64_t per = (nw + kScanThreads - 1) / kScanThreads;
  const int64_t w0 = min(nw, (int64_t)tid * per), w1 = min(nw, w0 + per);
  uint32_t cu = 0, cm = 0, cr = 0, ch = 0;
  for (int64_t w = w0; w < w1; ++w) {
    const uint32_t sw = sel[w];
    if (!sw) continue;
    const uint32_t hw = off ? hit[w] : 0u;
    const uint32_t rw = off ? (sw & ring_bits(w, M)) : 0u;
    cu += __popc(sw);
    cr += __popc(rw);
    ch += __popc(hw);
    if (off) cm += __popc(sw & ~hw & ~rw);
  }
  uint32_t U, n_miss, n_ring, n_hit;
  uint32_t bu = block_scan(cu, &U, sh);
  uint32_t bm = block_scan(cm, &n_miss, sh);
  block_scan(cr, &n_ring, sh);
  block_scan(ch, &n_hit, sh);
  for (int64_t w = w0; w < w1; ++w) {
    const uint32_t sw = sel[w];
    s.base_u[w] = bu;
    s.base_m[w] = bm;
    if (!sw) continue;
    const uint32_t hw = off ? hit[w] : 0u;
    const uint32_t rw = off ? (sw & ring_bits(w, M)) : 0u;
    bu += __popc(sw);
    if (off) bm += __popc(sw & ~hw & ~rw);
  }

  // Unpinned slots in ring order from the hand.
  uint32_t n_unpinned = 0, n_evict = 0;
  if (off) {
    const int S = ka.S, nsw = ka.s_words;
    const int sper = (nsw + kScanThreads - 1) / kScanThreads;
    const int j0 = min(nsw, tid * sper), j1 = min(nsw, j0 + sper);
    uint32_t cnt = 0;
    for (int j = j0; j < j1; ++j) {
      uint32_t bits = 0;
      if ((S & 31) == 0) {
        // 32 offsets from a word-aligned ring: two pinned words, funnel-shifted
        const int v0 = (hand + 32 * j) % S;
        const int w0 = v0 >> 5, sh0 = v0 & 31;
        const uint32_t lo = s.pinmask[w0];
        const uint32_t hi = sh0 ? s.pinmask[(w0 + 1) % nsw] : 0u;
        bits = ~(sh0 ? ((lo >> sh0) | (hi << (32 - sh0))) : lo);
      } else {
        int last = -1;
        uint32_t pw_ = 0;
        for (int i = 0; i < 32; ++i) {
          const int o = 32 * j + i;
          if (o >= S) break;
          const int v = (hand + o) % S;
          if ((v >> 5) != last) { last = v >> 5; pw_ = s.pinmask[last]; }
          if (!((pw_ >> (v & 31)) & 1u)) bits |= 1u << i;
        }
      }
      s.upw[j] = bits;
      cnt += __popc(bits);
    }
    uint32_t base = block_scan(cnt, &n_unpinned, sh);
    const uint32_t n_assigned = min(n_miss, n_unpinned);
    // victim[k] = the k-th unpinned slot after the hand, for the misses that get one,
    // with the position it holds now (to be evicted)
    for (int j = j0; j < j1; ++j) {
      uint32_t bits = s.upw[j];
      while (bits && base < n_assigned) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        s.victim[base++] = (int32_t)((hand + 32 * j + b) % S);
      }
    }
    __syncthreads();                                   // victims written; pinmask no longer read
    uint32_t my_evict = 0;
    for (uint32_t k0 = tid; k0 < n_assigned; k0 += 4 * kScanThreads) {
      int32_t v[4], old[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = k0 + e * kScanThreads;
        v[e] = k < n_assigned ? s.victim[k] : -1;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) old[e] = v[e] >= 0 ? u.slot_pos[v[e]] : -1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = k0 + e * kScanThreads;
        if (k < n_assigned) {
          s.victim_old[k] = old[e];
          my_evict += old[e] >= 0;
        }
      }
    }
    block_scan(my_evict, &n_evict, sh);
    for (int j = tid; j < nsw; j += kScanThreads) s.pinmask[j] = 0;
    if (tid == 0) {
      s_hand = hand;
      if (n_assigned > 0) s_hand = (s.victim[n_assigned - 1] + 1) % S;
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int64_t rb = 656;
    const uint32_t n_assigned = off ? min(n_miss, n_unpinned) : 0u;
    const int64_t noslot = off ? (int64_t)n_miss - n_assigned : 0;
    s.counters[0] = U;
    s.counters[1] = off ? n_hit : 0;
    s.counters[2] = off ? n_ring : 0;
    s.counters[3] = n_assigned;
    s.counters[4] = noslot;
    s.counters[5] = n_evict;
    s.counters[6] = off ? ((int64_t)n_assigned + noslot) * rb : 0;
    s.counters[7] = off ? 0 : U;
    for (int c = 0; c < 8; ++c) u.totals[c] += s.counters[c];
    int64_t wb = -1;
    if (off && L - M >= ka.ring_rows) wb = M;
    s.info[kInfoUnion] = U;
    s.info[kInfoWriteback] = wb;
    s.info[kInfoAssigned] = n_assigned;
    s.info[kInfoRound] = round;
    s.info[kInfoM] = M;
    s.info[kInfoHand] = hand;
    if (off) {
      *u.hand = s_hand;
      if (wb >= 0) u.dyn[1] = M + ka.ring_rows;
    }
    u.dyn[2] = round + 1;
  }
}

struct AssignKArgs {
  StepArgs a;
  int S, s_words, ring_cap, mode;
  int64_t max_positions;
};

// One wave per 32-position word, one lane per position.
__global__ __launch_bounds__(256) void gather_assign_kernel(AssignKArgs ka) {
  const StepArgs& a = ka.a;
  const int seq = blockIdx.y;
  const UnitDev u = a.units[a.unit_base + seq];
  const SeqScratch s = a.scr[seq];
  const int64_t L = u.dyn[0];
  const int64_t M = s.info[kInfoM];
  const int32_t round = (int32_t)s.info[kInfoRound];
  const uint32_t n_assigned = (uint32_t)s.info[kInfoAssigned];
  const bool off = ka.mode == 0;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (L + 31) / 32;
  const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  uint32_t* sel = s.selmask;
  uint32_t* hit = s.hitmask;
  for (int64_t w = wave_id; w < nw; w += n_waves) {
    const uint32_t sw = sel[w];
    if (!sw) continue;
    const uint32_t hw0 = off ? hit[w] : 0u;
    // every lane has read the word; clear it for the next step
    if (lane == 32) {
      sel[w] = 0;
      if (hw0) hit[w] = 0;
    }
    if (lane >= 32) continue;
    const uint32_t bit = 1u << lane;
    if (!(sw & bit)) continue;
    const uint32_t below = bit - 1u;
    const int64_t p = w * 32 + lane;
    const uint32_t ux = s.base_u[w] + __popc(sw & below);
    int32_t kind, src, fill = -1;
    if (!off) {
      kind = SRC_RES;
      src = (int32_t)p;
    } else {
      const uint32_t hw = hw0;
      const uint32_t rw = sw & ring_bits(w, M);
      if (rw & bit) {
        kind = SRC_RING;
        src = (int32_t)(p % ka.ring_cap);
      } else if (hw & bit) {
        kind = SRC_HIT;
        src = u.pos_slot[p];
      } else {
        const uint32_t k = s.base_m[w] + __popc(sw & ~hw & ~rw & below);
        src = (int32_t)p;
        if (k < n_assigned) {
          kind = SRC_MISS;
          const int32_t v = s.victim[k];
          const int32_t old = s.victim_old[k];
          if (old >= 0 && old < ka.max_positions) u.pos_slot[old] = -1;
          u.slot_pos[v] = (int32_t)p;
          u.pos_slot[p] = v;
          u.fill_round[v] = round;
          u.pin_round[v] = round;
          fill = v;
        } else {
          kind = SRC_MISS_NOSLOT;
        }
      }
    }
    s.uni[ux] = (int32_t)p;
    s.upos[p] = (int32_t)ux;
    s.kind[ux] = kind;
    s.src[ux] = src;
    s.fill[ux] = fill;
  }
}

struct CopyKArgs {
  StepArgs a;
  int row_bytes, ring_cap, ring_rows, hot_slots;
  int64_t max_positions;
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
      // every source index is range-checked: an inconsistent plan copies nothing
      const bool ok = kind == SRC_HIT ? (src >= 0 && src < ka.hot_slots)
                    : kind == SRC_RING ? (src >= 0 && src < ka.ring_cap)
                    : (src >= 0 && src < ka.max_positions);
      if (!ok) continue;
      const uint8_t* from = kind == SRC_HIT ? u.slots + src * rb
                          : kind == SRC_RING ? u.ring + src * rb
                          : u.rows + src * rb;
      const uint4 v = *reinterpret_cast<const uint4*>(from + c * 16);
      *reinterpret_cast<uint4*>(s.compact + x * rb + c * 16) = v;
      if (kind == SRC_MISS) {
        const int32_t f = s.fill[x];
        if (f >= 0 && f < ka.hot_slots) *reinterpret_cast<uint4*>(u.slots + (int64_t)f * rb + c * 16) = v;
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

hipError_t launch_gather_scan(const Geometry& g, const StepArgs& a, hipStream_t st) {
  ScanKArgs ka{a, g.hot_slots, g.s_words, g.ring_rows, g.mode};
  hipLaunchKernelGGL(gather_scan_kernel, dim3((unsigned)a.n_seqs), dim3(kScanThreads), 0, st, ka);
  return hipGetLastError();
}

hipError_t launch_gather_assign(const Geometry& g, const StepArgs& a, hipStream_t st) {
  AssignKArgs ka{a, g.hot_slots, g.s_words, g.ring_cap, g.mode, g.max_positions};
  const int64_t words = (a.l_max + 31) / 32;
  int64_t blocks = (words + 3) / 4;                 // 4 waves per block, one word per wave
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gather_assign_kernel, dim3((unsigned)blocks, (unsigned)a.n_seqs), dim3(256), 0, st, ka);
  return hipGetLastError();
}

hipError_t launch_copy(const Geometry& g, const StepArgs& a, hipStream_t st) {
  CopyKArgs ka{a, g.row_bytes, g.ring_cap, g.ring_rows, g.hot_slots, g.max_positions};
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
