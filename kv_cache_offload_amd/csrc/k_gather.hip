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
// selection is produced: the Top-K kernel sets, for every selected position, a
// bit in a per-position selection bitmap (a position several rows select is
// one union entry), classifies it against the round-start state (a hit needs a
// slot filled in an earlier round) and pins the hit's slot.  The last Top-K
// workgroup of the sequence then runs the gather plan (gather_plan.h): prefix
// counts per 32-position word and the victim list.  The assign kernel is wide:
// one wave per 64 positions, one lane per position.  Each selected lane
// computes its union index, kind and source; the k-th miss in ascending
// position order takes victim[k], evicts the position the slot held and
// updates the slot table; the lane leaves a descriptor of the position (union
// index, kind, source, slot to fill).  The row copies themselves are done by
// the attention kernel while it stages the rows (k_attn.hip): one 16-byte
// piece per thread, from the hot slot, the ring, or the host mirror (zero-copy
// reads of pinned host memory over the host link; a miss that several query
// rows select is read from host memory by each of them, as the page's rule for
// repeated misses has it), to LDS, the compact buffer and, for a miss that got
// a slot, to the slot.  No reader consults a slot filled in the same round:
// victims are unpinned, hits are pinned.  When a batch is due, the assign
// kernel's last blocks write the 64 oldest ring rows back to the mirror.
#include "gather_plan.h"

namespace dsa {
namespace {

constexpr int kGatherThreads = 256;

struct GatherKArgs {
  StepArgs a;
  int S, ring_cap, ring_rows, mode, row_bytes, K;
  int max_union;                        // R_max * K: compact rows in the scratch
  int word_blocks;                      // blocks of the union/slot-table part
  int clear_blocks;                     // then blocks clearing the Top-K histograms; the rest write back the ring
  int r_max;
  int clock;                            // CLOCK replacement: hits and fills set their slot's reference bit
  int64_t max_positions;
};

// Union entries and slot table: one wave per 64 positions, one lane per position.
// The last blocks write the 64 oldest pending ring rows back to the host mirror
// when a batch is due (positions the step reads from the ring, never from the
// mirror).
__global__ __launch_bounds__(kGatherThreads) void gather_assign_kernel(GatherKArgs ka) {
  const StepArgs& a = ka.a;
  const int seq = blockIdx.y;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  if ((int)blockIdx.x >= ka.word_blocks && (int)blockIdx.x < ka.word_blocks + ka.clear_blocks) {
    // the Top-K histograms of this step's rows, consumed: zero for the next step
    const int64_t t = (int64_t)(blockIdx.x - ka.word_blocks) * kGatherThreads + threadIdx.x;
    const int64_t n0 = (int64_t)kHistReps * a.R * (kRadixBins / 4), n1 = (int64_t)a.R * (kRadixBins / 4);
    if (t < n0) {
      const int64_t q = t / (a.R * (kRadixBins / 4)), rest = t % (a.R * (kRadixBins / 4));
      reinterpret_cast<DSA_GLOBAL u32x4*>(s.hist0 + q * ka.r_max * kRadixBins)[rest] = (u32x4){0u, 0u, 0u, 0u};
    } else if (t < n0 + n1) {
      reinterpret_cast<DSA_GLOBAL u32x4*>(s.hist1)[t - n0] = (u32x4){0u, 0u, 0u, 0u};
    }
    return;
  }
  if ((int)blockIdx.x >= ka.word_blocks) {
    const int64_t wb = s.info[kInfoWriteback];
    if (wb < 0) return;
    const int64_t t = (int64_t)(blockIdx.x - ka.word_blocks - ka.clear_blocks) * kGatherThreads + threadIdx.x;
    if (t >= (int64_t)ka.ring_rows * kCopyChunks16) return;
    const int64_t rb = ka.row_bytes;
    const int64_t p = wb + t / kCopyChunks16, c = t % kCopyChunks16;
    if (p >= ka.max_positions) return;
    const u32x4 v = *reinterpret_cast<const DSA_GLOBAL u32x4*>(u.ring + (p % ka.ring_cap) * rb + c * 16);
    *reinterpret_cast<DSA_GLOBAL u32x4*>(u.rows + p * rb + c * 16) = v;
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = ((int64_t)blockIdx.x * kGatherThreads + threadIdx.x) >> 6;
  const int64_t L = u.dyn[0];
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
  if (mine) {
    const uint32_t below = bit - 1u;
    const uint32_t ux = bu + __popc(sw & below);
    int32_t kind, src, fill = -1;
    if (!off) {
      kind = SRC_RES;
      src = (int32_t)p;
    } else {
      const uint32_t rw = sw & ring_bits(w, M);
      if (rw & bit) {
        kind = SRC_RING;
        src = (int32_t)(p % ka.ring_cap);
      } else if (hw & bit) {
        kind = SRC_HIT;                                // the hit's slot is pinned for this round
        src = u.pos_slot[p].x;
        if (src >= 0 && src < ka.S) {
          u.pin_round[src] = round;
          if (ka.clock) g_or(&u.ref[src >> 5], 1u << (src & 31));
        }
      } else {
        const uint32_t k = bm + __popc(sw & ~hw & ~rw & below);
        src = (int32_t)p;
        if (k < n_assigned) {
          kind = SRC_MISS;
          const i32x2 vo = s.victim[k];                // (slot, position it held), from the plan
          const int32_t v = vo.x, old = vo.y;
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
  const UnitG u = as_global(ka.u);
  const int64_t key_chunks = ka.n * ka.index_dim / 8;      // 16-byte pieces
  const int64_t row_chunks = ka.n * kCopyChunks16;
  const int64_t rb = ka.row_bytes;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < key_chunks + row_chunks;
       t += (int64_t)gridDim.x * blockDim.x) {
    if (t < key_chunks) {                                // piece c of new key i, to its operand-order place
      const int64_t i = t / (ka.index_dim / 8), c = t % (ka.index_dim / 8);
      reinterpret_cast<DSA_GLOBAL u32x4*>(u.keys)[key_piece(ka.L + i, (int)c)] = reinterpret_cast<const u32x4*>(ka.keys)[t];
    } else {
      const int64_t w = t - key_chunks;
      const int64_t i = w / kCopyChunks16, c = w % kCopyChunks16;
      const int64_t p = ka.L + i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ka.rows + i * rb + c * 16);
      const auto dst = (ka.mode == 1 || p < ka.newM) ? u.rows + p * rb : u.ring + (p % ka.ring_cap) * rb;
      *reinterpret_cast<DSA_GLOBAL u32x4*>(dst + c * 16) = v;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    u.dyn[0] = ka.L + ka.n;
    u.dyn[1] = ka.mode == 1 ? ka.L + ka.n : ka.newM;
  }
}

// Ring rows [from, to) to the mirror; then M = to.
__global__ __launch_bounds__(256) void ring_to_mirror_kernel(UnitDev ud, int64_t from, int64_t to,
                                                             int row_bytes, int ring_cap) {
  const UnitG u = as_global(ud);
  const int64_t total = (to - from) * kCopyChunks16;
  const int64_t rb = row_bytes;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = from + t / kCopyChunks16, c = t % kCopyChunks16;
    const u32x4 v = *reinterpret_cast<const DSA_GLOBAL u32x4*>(u.ring + (p % ring_cap) * rb + c * 16);
    *reinterpret_cast<DSA_GLOBAL u32x4*>(u.rows + p * rb + c * 16) = v;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) u.dyn[1] = to;
}

// Warm, phase 1: forget the positions currently cached.
__global__ __launch_bounds__(256) void warm_clear_kernel(UnitDev ud, int S) {
  const UnitG u = as_global(ud);
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < S; v += gridDim.x * blockDim.x) {
    const int32_t old = u.slot_pos[v];
    if (old >= 0) {
      u.pos_slot[old] = (i32x2){-1, -1};
      __hip_atomic_fetch_and(&u.hot[old >> 5], ~(1u << (old & 31)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Warm, phase 2: slot v <- position L-n+v for v < n; other slots empty; no round
// marks; under CLOCK every filled slot starts referenced.
__global__ __launch_bounds__(256) void warm_fill_kernel(UnitDev ud, int S, int64_t L, int64_t n, int row_bytes,
                                                        int clock) {
  const UnitG u = as_global(ud);
  const int64_t rb = row_bytes;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < (S + 31) / 32; w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lo = 32 * w;                         // slots [lo, lo + 32) filled iff below n
    const uint32_t m = n <= lo ? 0u : (n >= lo + 32 ? 0xFFFFFFFFu : (1u << (uint32_t)(n - lo)) - 1u);
    u.ref[w] = clock ? m : 0u;
  }
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < S; v += (int64_t)gridDim.x * blockDim.x) {
    const int32_t pos = v < n ? (int32_t)(L - n + v) : -1;
    u.slot_pos[v] = pos;
    u.fill_round[v] = -1;
    u.pin_round[v] = -1;
    if (pos >= 0) {
      u.pos_slot[pos] = (i32x2){(int32_t)v, -1};
      g_or(&u.hot[pos >> 5], 1u << (pos & 31));
    }
  }
  const int64_t total = n * kCopyChunks16;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = t / kCopyChunks16, c = t % kCopyChunks16;
    const u32x4 x = *reinterpret_cast<const DSA_GLOBAL u32x4*>(u.rows + (L - n + v) * rb + c * 16);
    *reinterpret_cast<DSA_GLOBAL u32x4*>(u.slots + v * rb + c * 16) = x;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *u.hand = (int32_t)(n % S);
}

// Keys of positions [0, L) back in row order, one 16-byte piece per thread.
__global__ __launch_bounds__(256) void keys_linear_kernel(UnitDev ud, int64_t L, uint16_t* dst) {
  const UnitG u = as_global(ud);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < L * 16; t += (int64_t)gridDim.x * blockDim.x)
    reinterpret_cast<u32x4*>(dst)[t] = reinterpret_cast<const DSA_GLOBAL u32x4*>(u.keys)[key_piece(t / 16, (int)(t % 16))];
}

// Rollback: publish the shortened row count and mirror count in stream order.
__global__ __launch_bounds__(64) void rollback_kernel(UnitDev ud, int64_t L, int64_t M) {
  const UnitG u = as_global(ud);
  if (threadIdx.x == 0) {
    u.dyn[0] = L;
    u.dyn[1] = M;
  }
}

unsigned grid_for(int64_t work, int64_t cap = 4096) {
  int64_t b = (work + 255) / 256;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_gather(const Geometry& g, const StepArgs& a, hipStream_t st, bool clear_hist) {
  const int64_t words = (a.l_max + 31) / 32;
  const int64_t waves = (words + 1) / 2;
  const int64_t blocks = (waves + 3) / 4;
  const int64_t wb_blocks = ((int64_t)g.ring_rows * kCopyChunks16 + kGatherThreads - 1) / kGatherThreads;
  const int64_t clear_blocks =
      clear_hist ? ((int64_t)(kHistReps + 1) * a.R * (kRadixBins / 4) + kGatherThreads - 1) / kGatherThreads : 0;
  GatherKArgs ka{a, g.hot_slots, g.ring_cap, g.ring_rows, g.mode, g.row_bytes, g.top_k, g.r_max * g.top_k,
                 (int)blocks, (int)clear_blocks, g.r_max, g.clock ? 1 : 0, g.max_positions};
  return launch_k(gather_assign_kernel,
                  dim3((unsigned)(blocks + clear_blocks + (g.mode == 0 ? wb_blocks : 0)), (unsigned)a.n_seqs),
                  dim3(kGatherThreads), 0, st, ka);
}

hipError_t launch_append(const Geometry& g, const UnitDev& unit, int64_t L, int64_t M, int64_t newM,
                         int64_t n, const uint16_t* keys, const uint8_t* rows, hipStream_t st) {
  if (g.mode == 0 && newM > M && M < L) {
    const int64_t to = newM < L ? newM : L;
    hipError_t e = launch_k(ring_to_mirror_kernel, dim3(grid_for((to - M) * kCopyChunks16)), dim3(256), 0, st,
                            unit, M, to, g.row_bytes, g.ring_cap);
    if (e != hipSuccess) return e;
  }
  AppendKArgs ka{unit, L, newM, n, keys, rows, g.row_bytes, g.ring_cap, g.index_dim, g.mode};
  const int64_t work = n * g.index_dim / 8 + n * kCopyChunks16;
  return launch_k(append_kernel, dim3(grid_for(work)), dim3(256), 0, st, ka);
}

hipError_t launch_flush(const Geometry& g, const UnitDev& unit, int64_t M, int64_t L, hipStream_t st) {
  return launch_k(ring_to_mirror_kernel, dim3(grid_for((L - M) * kCopyChunks16)), dim3(256), 0, st, unit, M, L,
                  g.row_bytes, g.ring_cap);
}

hipError_t launch_warm(const Geometry& g, const UnitDev& unit, int64_t L, hipStream_t st) {
  const int64_t n = L < g.hot_slots ? L : g.hot_slots;
  hipError_t e = launch_k(warm_clear_kernel, dim3(grid_for(g.hot_slots)), dim3(256), 0, st, unit, g.hot_slots);
  if (e != hipSuccess) return e;
  return launch_k(warm_fill_kernel, dim3(grid_for(n * kCopyChunks16 > g.hot_slots ? n * kCopyChunks16 : g.hot_slots)),
                  dim3(256), 0, st, unit, g.hot_slots, L, n, g.row_bytes, g.clock ? 1 : 0);
}

hipError_t launch_keys_linear(const UnitDev& unit, int64_t L, uint16_t* dst, hipStream_t st) {
  return launch_k(keys_linear_kernel, dim3(grid_for(L * 16)), dim3(256), 0, st, unit, L, dst);
}

hipError_t launch_rollback(const UnitDev& unit, int64_t L, int64_t M, hipStream_t st) {
  return launch_k(rollback_kernel, dim3(1), dim3(64), 0, st, unit, L, M);
}

}  // namespace dsa
