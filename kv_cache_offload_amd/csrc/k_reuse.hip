// k_reuse.hip -- selection reuse and prefetch.
//
// Page "From 1M total to 15+ streams x 1M: the capacity breakthrough of
// GLM-5.3 KV cache offload" (zhuai.tech):
//   * section "Starting point": some later layers reuse the indexer's
//     selection, while every layer keeps its own KV rows;
//   * first decision ("CPU stores the history and runs the indexer?"): once
//     the selection is known, the history rows of the layers that reuse it can
//     be moved early, overlapping independent work -- a real opportunity, but
//     not a free one.
//
// A reusing layer runs a round of its own cache on the selection of the most
// recent full decode step (left in the per-sequence scratch by the Top-K):
// the mark kernel sets the selection bitmap of the round and its last
// workgroup runs the layer's gather plan; the assign kernel, attention and
// merge follow unchanged.  A prefetch is such a round without attention, run
// on a second scratch set so that it can overlap the source layer's remaining
// kernels on another stream: its misses take slots and the fill kernel copies
// their rows from the host mirror into those slots, so the layer's next round
// (the reuse step) finds them as hits.
#include "gather_plan.h"

namespace dsa {
namespace {

struct MarkKArgs {
  StepArgs a;                 // a.s0: the round's scratch (main, or the prefetch set)
  SeqScratch sel0;            // where the selection lives: the main scratch (sequence 0)
  int64_t sel_stride;         // and its stride between sequences
  int K, mode;
  PlanParams plan;
};

// One workgroup per (query row, sequence): mark the row's selection in the
// round's bitmap; the last row of the sequence runs the gather plan.
__global__ __launch_bounds__(kPlanThreads) void reuse_mark_kernel(MarkKArgs ka) {
  __shared__ uint32_t lds[kWalkWords + 32];
  const StepArgs& a = ka.a;
  const int r = blockIdx.x, seq = blockIdx.y;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  const ScratchG src = moved_desc<ScratchG>(ka.sel0, seq * ka.sel_stride, -1, 0);
  const PlanState ps{u.dyn[0], u.dyn[1], (int32_t)u.dyn[2], ka.mode == 0 ? *u.hand : 0};
  const int n = src.sel_n[r];
  const auto sel = src.sel + (int64_t)r * ka.K;
  if (r == 0 && threadIdx.x == 0) s.counters[8] = 0;  // host reads: the round's readers add them
  for (int j = threadIdx.x; j < n; j += kPlanThreads) {
    const int32_t pos = sel[j];
    if (pos >= 0 && pos < ps.L) g_or(&s.selmask[pos >> 5], 1u << (pos & 31));
    else raise_err(a.err, kErrSelection);
  }
  plan_if_last(u, s, ka.plan, (uint32_t)a.R, ps, lds, true);
}

struct FillKArgs {
  StepArgs a;
  int max_union, row_bytes, S;
  int64_t max_positions;
};

// Prefetch: copy every union entry that took a slot from the host mirror into
// the slot, one 16-byte piece per thread.
__global__ __launch_bounds__(256) void prefetch_fill_kernel(FillKArgs ka) {
  const StepArgs& a = ka.a;
  const int seq = blockIdx.y;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  const int64_t U = s.info[kInfoUnion];
  const int64_t rb = ka.row_bytes;
  if (blockIdx.x == 0 && threadIdx.x == 0) g_add(&u.totals[8], s.info[kInfoAssigned]);   // one host read per fill
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < U * kCopyChunks16;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t ux = t / kCopyChunks16, c = t % kCopyChunks16;
    if (ux >= ka.max_union) {
      raise_err(a.err, kErrSelection);
      break;
    }
    const int32_t p = s.uni[ux];
    if (p < 0 || p >= ka.max_positions) {
      raise_err(a.err, kErrSelection);
      continue;
    }
    const int32_t fill = s.pdesc[p].w;
    if (fill >= ka.S) raise_err(a.err, kErrVictim);
    if (fill < 0 || fill >= ka.S) continue;
    const u32x4 v = *reinterpret_cast<const DSA_GLOBAL u32x4*>(u.rows + (int64_t)p * rb + c * 16);
    *reinterpret_cast<DSA_GLOBAL u32x4*>(u.slots + (int64_t)fill * rb + c * 16) = v;
  }
}

}  // namespace

hipError_t launch_reuse_mark(const Geometry& g, const StepArgs& a, const SeqScratch& sel0, int64_t sel_stride,
                             hipStream_t st) {
  MarkKArgs ka{a, sel0, sel_stride, g.top_k, g.mode, PlanParams{g.hot_slots, g.s_words, g.ring_rows, g.mode, g.clock ? 1 : 0, 0}};
  return launch_k(reuse_mark_kernel, dim3((unsigned)a.R, (unsigned)a.n_seqs), dim3(kPlanThreads), 0, st, ka);
}

hipError_t launch_prefetch_fill(const Geometry& g, const StepArgs& a, hipStream_t st) {
  const int max_union = g.r_max * g.top_k;
  FillKArgs ka{a, max_union, g.row_bytes, g.hot_slots, g.max_positions};
  // host-link bound: 64 blocks keep 256 KiB of reads in flight, more than the
  // link's bandwidth-delay product, and leave the CUs to the kernels it overlaps
  int64_t blocks = ((int64_t)max_union * kCopyChunks16 + 255) / 256;
  if (blocks > 64) blocks = 64;
  return launch_k(prefetch_fill_kernel, dim3((unsigned)blocks, (unsigned)a.n_seqs), dim3(256), 0, st, ka);
}

}  // namespace dsa
