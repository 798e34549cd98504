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
// gfx950 design.  Selection and classification happen where the selection is
// produced: the Top-K kernel sets, for every selected position, a bit in a
// per-position selection bitmap (a position several rows select is one union
// entry), and the last Top-K workgroup of the sequence runs the gather plan
// (gather_plan.h): hits against the cached-position bitmap, prefix counts per
// 32-position word and the victim list.  The attention kernel derives each of
// its rows' union index, kind and source from those outputs and does the row
// copies while it stages the rows (k_attn.hip): one 16-byte piece per thread,
// from the hot slot, the ring, or the host mirror (zero-copy reads of pinned
// host memory over the host link; a miss that several query rows select is
// read from host memory by each of them, as the page's rule for repeated
// misses has it), to LDS, the compact buffer and, for a miss that got a slot,
// to the slot.  The assign pass (gather_assign.h) then pins the hits' slots,
// gives the k-th miss in ascending position order victim[k] (evicting the
// position the slot held and updating the slot table), writes the union
// entries and descriptors, and, when a batch is due, writes the 64 oldest
// ring rows back to the mirror; in a decode step it runs as extra workgroups
// of the merge launch.  No reader consults a slot filled in the same round:
// victims are unpinned, hits are pinned.  This file holds the assign kernel of
// prefetch rounds and the unit maintenance kernels.
#include "gather_assign.h"

namespace dsa {
namespace {

__global__ __launch_bounds__(kGatherThreads) void gather_assign_kernel(GatherKArgs ka) {
  assign_block(ka, (int)blockIdx.x, (int)blockIdx.y);
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

// Test hook (dsa_debug_inject): every cached position of [0, L) is given the
// slot index S + 1, outside the cache, so that the next round's hits fail the
// device-side checks of attention and the assign pass (which then skip them).
__global__ __launch_bounds__(256) void bad_slot_kernel(UnitDev ud, int64_t L, int S) {
  const UnitG u = as_global(ud);
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < L; p += (int64_t)gridDim.x * blockDim.x) {
    const i32x2 ps = u.pos_slot[p];
    if (ps.x >= 0) u.pos_slot[p] = (i32x2){S + 1, ps.y};
  }
}

// Zero the Top-K histograms, the selection bitmap and the arrival counters of
// every sequence's scratch set (blockIdx.y = sequence), one word per thread.
__global__ __launch_bounds__(256) void clear_step_kernel(StepArgs a, int r_max, int64_t sel_words) {
  const ScratchG s = scratch_of(a, (int)blockIdx.y);
  const int64_t n0 = (int64_t)kHistReps * r_max * kRadixBins, n1 = (int64_t)r_max * kRadixBins;
  const int64_t n = n0 + n1 + sel_words + 1 + r_max;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
    if (t < n0) s.hist0[t] = 0u;
    else if (t < n0 + n1) s.hist1[t - n0] = 0u;
    else if (t < n0 + n1 + sel_words) s.selmask[t - n0 - n1] = 0u;
    else s.done[t - n0 - n1 - sel_words] = 0u;
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
  int64_t blocks = 0;
  const GatherKArgs ka = gather_args(g, a, clear_hist, false, &blocks);
  return launch_k(gather_assign_kernel, dim3((unsigned)blocks, (unsigned)a.n_seqs), dim3(kGatherThreads), 0, st, ka);
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

hipError_t launch_clear_step_scratch(const Geometry& g, const StepArgs& a, hipStream_t st) {
  const int64_t words = (int64_t)(kHistReps + 1) * g.r_max * kRadixBins + g.p_pad / 32 + 1 + g.r_max;
  return launch_k(clear_step_kernel, dim3(grid_for(words, 64), (unsigned)a.n_seqs), dim3(256), 0, st, a, g.r_max,
                  g.p_pad / 32);
}

hipError_t launch_inject_bad_slot(const Geometry& g, const UnitDev& unit, int64_t L, hipStream_t st) {
  return launch_k(bad_slot_kernel, dim3(grid_for(L)), dim3(256), 0, st, unit, L, g.hot_slots);
}

}  // namespace dsa
