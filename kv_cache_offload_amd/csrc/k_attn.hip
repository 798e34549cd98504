// k_attn.hip -- absorbed-MLA attention over the selected Q8G64 rows only.
//
//   c_j[d] = int8_j[d] * scale_j[d/64]
//   l_j    = softmax_scale * (q_lat . c_j + q_rope . rope_j)
//   out[d] = sum_j softmax(l)_j * c_j[d]
//
// Attention consumes only the rows the DSA indexer selected, from the compact
// selection the hot gather produced (page "From 1M total to 15+ streams x 1M:
// the capacity breakthrough of GLM-5.3 KV cache offload", section "Starting
// point" and the data-flow figure of section "Decision 3").  The row format is
// the page's 656-byte Q8G64 layout: int8 latent, fp16 scale per group of 64,
// bf16 RoPE.
//
// gfx950 mapping.  A workgroup owns one query row and a split of 64 of its
// selected rows (every nsplit-th), all heads: wave w holds heads 16w..16w+15.
// The rows are staged in 32-row blocks through two LDS buffers, once for all
// waves: the int8 latent widened to bf16 (exact,
// |int8| < 2^8) in one row-major layout, the fp16 scales as fp32, the RoPE as
// is.  Both products run on v_mfma_f32_16x16x32_bf16:
//   * logits, transposed: S^T[j][h] = sum_d C[j][d] Q[h][d], the A operand
//     read straight from the row-major latent, the query (B operand) held in
//     registers; each 64-dim group is accumulated separately and scaled by its
//     fp32 scale per row, so the int8 operand stays exact;
//   * softmax online over the 32-row blocks: a block's max is known before
//     any of its weights is formed, and the running output and sum are
//     rescaled when a later block raises the max;
//   * output: O[h][d] += sum_j P'_g[h][j] C[j][d] with P'_g = p * scale_g,
//     carried as a bf16 high part plus a bf16 low part (~16 mantissa bits).
//     In the transposed logits a lane already holds p for one head and 8 rows
//     of each 32-row half, which is exactly its A fragment, so P never goes
//     through LDS; the B fragments (8 rows of one dim) come from the row-major
//     latent with the LDS transpose read ds_read_b64_tr_b16 (4 rows x 1
//     column per lane).
// Each workgroup writes its (max, sum) and its normalised O / sum in fp16 with
// a power-of-two scale per head, and a merge kernel combines the splits with the
// log-sum-exp rule.  The fp16 rounding is at most 2^-11 of the split's largest
// |O / sum| for a head, a weighted mean of dequantised rows, so each output
// element is off by at most 2^-11 of the largest |dequantised latent| it mixes.
#include "gather_assign.h"

namespace dsa {
namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef short bf16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float fx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bfx2 __attribute__((ext_vector_type(2)));
#define DSA_LDS __attribute__((address_space(3)))

constexpr int kSplit = 64;             // selected rows per workgroup
constexpr int kBlk = 32;               // rows per staged block (online softmax over the blocks)
constexpr int kRowPieces = kCopyChunks16;            // 16-byte pieces of a 656-byte row
constexpr int kBlkPieces = kBlk * kRowPieces;
constexpr int kLatStride = 536;        // bf16 per row of the latent in LDS (512 + 24: no bank conflicts
                                       // for the row reads of the logits nor the transpose reads)
constexpr int kRopeStride = 72;        // bf16 per row of RoPE (64 + 8)
constexpr int kMaxSplits = 4096 / kSplit;

struct AttnKArgs {
  StepArgs a;
  const uint16_t* q_lat;     // [n_seqs][R][H][512]
  const uint16_t* q_rope;    // [n_seqs][R][H][64]
  float* out;                // [n_seqs][R][H][512]
  int K, H, nsplit, ns_stride, row_bytes;
  int S, ring_cap, max_union;
  int off;                   // offload mode (hot slots, ring, host mirror)
  int64_t max_positions;
  float scale_log2;          // softmax_scale * log2(e)
  int plan;                  // the extra workgroup of each sequence: 0 nothing (the plan ran before),
                             // 1 the plan's walk (its counts ran before), 2 the whole plan, and every
                             // workgroup counts the union words before its rows itself
  PlanParams pp;
};

// Two fp32 -> packed fp16 (round to nearest even), as one 32-bit word.
__device__ inline uint32_t pack_f16(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &ha, 2);
  __builtin_memcpy(&ub, &hb, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// Two fp32 -> packed bf16 (round to nearest even), as one 32-bit word.
__device__ inline uint32_t pack_bf16(float a, float b) {
  const bfx2 v = __builtin_convertvector((fx2){a, b}, bfx2);
  uint32_t w;
  __builtin_memcpy(&w, &v, 4);
  return w;
}

// 2^x by the hardware instruction alone.  Results below 2^-126 flush to zero:
// such a softmax weight is below 2^-126 of the largest one of its head, far
// under any rounding the output carries.
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline float f16_bits_to_f32(uint32_t h) {
  _Float16 f;
  const uint16_t b = (uint16_t)h;
  __builtin_memcpy(&f, &b, 2);
  return (float)f;                     // exact widening
}

// 16 signed bytes -> 16 bf16 (exact), as 8 words.
__device__ inline void widen16(u32x4 raw, uint32_t* out) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = raw[w];
    const float f0 = (float)(int8_t)(x & 0xFFu), f1 = (float)(int8_t)((x >> 8) & 0xFFu);
    const float f2 = (float)(int8_t)((x >> 16) & 0xFFu), f3 = (float)(int8_t)(x >> 24);
    out[2 * w] = pack_bf16(f0, f1);
    out[2 * w + 1] = pack_bf16(f2, f3);
  }
}

// 4 bf16 of rows r0..r0+3 at column col0 + (lane % 16): lane c of each 16-lane
// group supplies the address of row r0 + c/4, columns col0 + 4 (c % 4) .. +3
// (the lane groups may use different r0).
__device__ inline bf16x4 read_tr(const uint16_t* lat_s, int r0, int col0, int lane) {
  const int c = lane & 15;
  const uint16_t* p = lat_s + (r0 + (c >> 2)) * kLatStride + col0 + 4 * (c & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS bf16x4*)(DSA_LDS void*)p);
}

// One workgroup: one query row, all H = HG*16 heads, NBLK * 32 selected rows
// (a split), staged in 32-row blocks through two LDS buffers.  Split s takes
// the row's selected indices s, s + nsplit, s + 2 nsplit, ...: the host-mirror
// reads of a row's misses (old positions, early in the ascending selection)
// spread over all its workgroups instead of loading its first splits.
// DS waves share each group of 16 heads: every one of them forms the group's
// logits and softmax (the same instructions on the same operands, so the same
// values), and wave (head group hg, part dh) accumulates output dims
// [512 dh / DS, 512 (dh + 1) / DS).  With DS = 2 a wave holds half the output
// accumulators, two waves fit a SIMD, and the staging has twice the threads.
template <int HG, int DS, int NBLK>
__global__ __launch_bounds__(HG * DS * 64) void attn_kernel(AttnKArgs ka) {
  constexpr int NW = HG * DS;
  constexpr int NT = NW * 64;
  constexpr int NTD = 32 / DS;                           // 16-dim output tiles of a wave
  constexpr int GD = 8 / DS;                             // 64-dim scale groups of a wave's output dims
  static_assert(DS == 1 || DS == 2, "one or two waves per head group");
  constexpr int kSplit = NBLK * kBlk;                    // this kernel's split
  static_assert(kSplit <= NT, "one thread per row of the split reads its source");
  constexpr int PPT = (kBlkPieces + NT - 1) / NT;        // row pieces per thread per block
  __shared__ __align__(16) uint16_t lat_s[2][kBlk * kLatStride];
  __shared__ __align__(16) uint16_t rope_s[2][kBlk * kRopeStride];
  __shared__ __align__(16) float scl_s[2][8 * kBlk];
  __shared__ const DSA_GLOBAL uint8_t* s_from[kSplit];   // where each row is read from (null: masked)
  __shared__ int s_ux[kSplit];                            // its compact row, -1 if masked
  __shared__ uint32_t s_scan[NW];
  __shared__ uint32_t s_host;                             // any row of the split read from the host mirror
  __shared__ float s_amax[NW][16];                        // per wave: its heads' largest |O| (DS > 1)

  const StepArgs& a = ka.a;
  const int split = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const UnitG u = unit_of(a, seq);
  const ScratchG s = scratch_of(a, seq);
  if (split == ka.nsplit) {                              // (uniform) past the splits: the sequence's plan
    if (r == 0 && ka.plan == 1) plan_walk_from_info<NT>(u, s, ka.pp, reinterpret_cast<uint32_t*>(lat_s[0]));
    if (r == 0 && ka.plan == 2) plan_counts_and_walk<NT>(u, s, ka.pp, reinterpret_cast<uint32_t*>(lat_s[0]));
    return;
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int H = ka.H;
  const int hg = DS == 1 ? wave : wave % HG;             // head group
  const int dh = DS == 1 ? 0 : wave / HG;                // part of the output dims
  const int h0 = hg * 16;
  const int64_t rb = ka.row_bytes;

  // The split's rows: position (selection), then the row's place in the
  // round, derived from the counts phase of the gather plan exactly as the
  // assign pass derives it -- union index from the word's union count and the
  // selected bits below, kind from the ring boundary M and the hit bits, and
  // the source: a hit from its HBM slot (the position's slot), a ring row from
  // the recent ring, a miss from the host mirror (repeated misses of the same
  // round each read host memory), a resident row from the HBM row store.  The
  // map entry of every selected index of the split is written here.  A hit's
  // slot is read with the words (for every selected position: a non-hit
  // ignores it), so only the row's address is on the path to its data.
  const int n_sel = s.sel_n[r];
  // Whole plan here (ka.plan == 2): this workgroup counts the union entries
  // before each selection word itself (the plan's workgroup runs beside it),
  // from the round's bitmap: every word requested at once with the selection,
  // counted into LDS (the second staging buffer, free until block 1), and
  // scanned once the rows are requested -- only the compact row and the map
  // entry need the union index, not the row's source.  A selected position is
  // a hit iff it was cached at round start.
  const bool own_counts = ka.plan == 2;
  const int64_t L = step_L(u, a);
  const int64_t M = own_counts ? u.dyn[1] : s.info[kInfoM];   // the ring boundary at round start
  const int64_t nw = own_counts ? (L + 31) / 32 : 0;     // within kAttnScanWords (the host's choice)
  uint32_t* cnt = reinterpret_cast<uint32_t*>(lat_s[1]);
  static_assert(kAttnScanWords * 4 <= (int64_t)sizeof(lat_s[1]), "the word counts fit a staging buffer");
  // The split's selected positions are requested first and the union words
  // (own counts) behind them, all unconditionally (indices clamped into the
  // buffers): the words' round trip then overlaps the positions', and the
  // loads of the rows' sources wait for the positions only.
  const int j = split + tid * ka.nsplit;
  int32_t pos = -1;
  if (tid < kSplit) pos = s.sel[(int64_t)r * ka.K + min(j, ka.K - 1)];
  constexpr int kLoads = (int)((kAttnScanWords / 4 + NT - 1) / NT);
  u32x4 wv[kLoads];
  if (own_counts) {                                      // (uniform)
    const int64_t last = max((nw + 3) / 4 - 1, (int64_t)0);   // the last 4-word piece holding a word
#pragma unroll
    for (int e = 0; e < kLoads; ++e)
      wv[e] = reinterpret_cast<const DSA_GLOBAL u32x4*>(s.selmask)[min(tid + (int64_t)e * NT, last)];
  }
  bool host = false;                                     // this row is read from the host mirror
  bool live = false;                                     // this row's source is known (own counts: ux pending)
  int map_v = -2;                                        // its map entry, stored once the rows are requested
                                                         // (-2: none, or own counts: after the scan)
  uint32_t t_sw = 0, t_below = 0;                        // its selection word and the bits below it
  int64_t t_w = 0;
  if (tid < kSplit) {
    if (j >= ka.K) pos = -1;
    const bool ok = j < n_sel && pos >= 0 && pos < ka.max_positions && (!own_counts || pos < L);
    const int64_t w = ok ? pos >> 5 : 0;
    const uint32_t sw = s.selmask[w];
    const uint32_t hraw = !ka.off ? 0u : own_counts ? u.hot[w] : s.hitmask[w];
    const uint32_t bu = own_counts ? 0u : s.base_u[w];
    const i32x2 ps = ka.off ? u.pos_slot[ok ? pos : 0] : (i32x2){-1, -1};
    const uint32_t hw = own_counts ? (hraw & sw) : hraw;   // (after every load is issued)
    const uint32_t bit = 1u << (pos & 31), below = bit - 1u;
    const uint32_t ux = bu + __popc(sw & below);
    const DSA_GLOBAL uint8_t* from = nullptr;
    // A selected index whose position, bitmap bit, union index or hit slot is
    // not what the plan allows is skipped (its row masked) and raises the
    // session's error flag: such a plan is inconsistent.
    if (ok && (sw & bit) && (own_counts || ux < (uint32_t)ka.max_union)) {
      if (!ka.off) {
        from = u.rows + (int64_t)pos * rb;
      } else {
        const uint32_t rw = sw & ring_bits(w, M);
        if (rw & bit) {
          from = u.ring + (int64_t)(pos % ka.ring_cap) * rb;
        } else if (hw & bit) {
          const int32_t slot = ps.x;
          if (slot >= 0 && slot < ka.S) from = u.slots + (int64_t)slot * rb;
          else raise_err(a.err, kErrHitSlot);
        } else {
          from = u.rows + (int64_t)pos * rb;
          host = true;
        }
      }
    } else if (j < n_sel) {
      raise_err(a.err, kErrSelection);
    }
    s_from[tid] = from;
    live = from != nullptr;
    t_sw = sw;
    t_below = below;
    t_w = w;
    if (!own_counts) {
      s_ux[tid] = from ? (int)ux : -1;
      if (j < ka.K) map_v = from ? (int)ux : -1;
    } else if (!from && j < ka.K) {
      map_v = -1;
    }
  }
  if (own_counts) {                                      // (uniform) the union words counted into LDS
#pragma unroll
    for (int e = 0; e < kLoads; ++e) {
      const int64_t q = tid + (int64_t)e * NT;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < nw) cnt[4 * q + i] = __popc(wv[e][i]);
    }
  }
  uint64_t host_bits = 0;
  if (wave == 0) {                                       // the split's host-mirror reads (one wave holds its rows)
    host_bits = __ballot(host);
    if (lane == 0) s_host = host_bits ? 1u : 0u;
  }
  // The map entries and the host-read counts are stored after the rows are
  // requested: a store ahead of the row loads would be waited for first.
  auto store_map_and_counts = [&]() {
    if (map_v != -2) s.map[(int64_t)r * ka.K + j] = map_v;
    if (lane == 0 && host_bits) {
      g_add(&s.counters[8], (int64_t)__popcll(host_bits));
      g_add(&u.totals[8], (int64_t)__popcll(host_bits));
    }
  };
  if (split >= n_sel) {                                  // (uniform) nothing to attend: the map entries only
    store_map_and_counts();
    return;
  }

  // Query fragments (B operand of the logits): lane holds Q[h0 + l16][32 ks + 8 q4 .. +7].
  bf16x8 qa[18];
  {
    const int64_t qrow = ((int64_t)seq * a.R + r) * H + h0 + l16;
    const uint16_t* ql = ka.q_lat + qrow * 512 + 8 * q4;
    const uint16_t* qr = ka.q_rope + qrow * 64 + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qa[ks] = *reinterpret_cast<const bf16x8*>(ql + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qa[16 + ks] = *reinterpret_cast<const bf16x8*>(qr + 32 * ks);
  }
  __syncthreads();                                       // s_from (and the word counts) for every thread

  // Every 16-byte piece of a block is requested at once.  A split with rows on
  // the host requests block b + 1 as soon as block b has arrived, before block
  // b is computed: the host link then serves every workgroup's first block
  // before any second block, and each block is computed while the next one
  // arrives.  A split whose rows are all in HBM requests its second block with
  // the first (both register buffers are free): one memory round trip for both.
  // Piece q of a block: row q / 41, bytes 16 (q % 41) .. ; masked rows read the
  // unit's key store (always mapped) and are zeroed below.
  u32x4 raw[2][PPT];
  auto request = [&](int b) {
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      const int q = min(tid + e * NT, kBlkPieces - 1);
      const int row = b * kBlk + q / kRowPieces, part = q % kRowPieces;
      const DSA_GLOBAL uint8_t* from = s_from[row];
      const DSA_GLOBAL uint8_t* at = from ? from + 16 * part : reinterpret_cast<const DSA_GLOBAL uint8_t*>(u.keys);
      raw[b & 1][e] = *reinterpret_cast<const DSA_GLOBAL u32x4*>(at);
    }
  };
  const bool early = NBLK > 1 && !s_host;                // (uniform)
  request(0);
  if (early) request(1);
  store_map_and_counts();
  if (own_counts) {                                      // (uniform) the union indices, while the rows arrive
    const int64_t per = (nw + NT - 1) / NT;
    const int64_t c0 = min(nw, (int64_t)tid * per), c1 = min(nw, c0 + per);
    uint32_t sum = 0;
    for (int64_t w = c0; w < c1; ++w) sum += cnt[w];
    uint32_t tot;
    uint32_t run = block_scan<NW>(sum, &tot, s_scan);
    for (int64_t w = c0; w < c1; ++w) {
      const uint32_t x = cnt[w];
      cnt[w] = run;
      run += x;
    }
    __syncthreads();
    if (tid < kSplit) {
      const int j = split + tid * ka.nsplit;
      int ux = -1;
      if (live) {
        const uint32_t x = cnt[t_w] + __popc(t_sw & t_below);
        if (x < (uint32_t)ka.max_union) ux = (int)x;
        else raise_err(a.err, kErrSelection);           // (the row's data is then masked)
      }
      s_ux[tid] = ux;
      if (live && j < ka.K) s.map[(int64_t)r * ka.K + j] = ux;
    }
    __syncthreads();                                     // s_ux before block 0 is staged
  }

  f32x4 o[NTD];                                          // o[nt]: output dims 16 (NTD dh + nt) ..
#pragma unroll
  for (int i = 0; i < NTD; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;                  // of head h0 + l16

#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    // buffer b & 1 was last read by block b - 2, which every wave finished
    // before the barrier of block b - 1
    uint16_t* lat = lat_s[b & 1];
    uint16_t* rope = rope_s[b & 1];
    float* scl = scl_s[b & 1];
    // This block's rows, staged in LDS: the int8 latent widened to bf16, the
    // scales as fp32, the RoPE as is; and their compact copy (the gather's
    // output; only the assign pass, which copies a miss's row into its slot,
    // reads it again in this step, so it is streamed past the caches with
    // non-temporal stores).  The copy is stored here, beside the staging, except
    // for a block of a split with host-mirror rows whose next block is still to
    // arrive: that block's copy is stored once it is computed, since a store
    // whose data registers are reused is waited for there, and, behind a
    // branch, together with every later load -- the next block's host rows --
    // so a store issued here would hold the block's products until the next
    // block had arrived.
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      const int q = tid + e * NT;
      if (q >= kBlkPieces) continue;
      const int rl = q / kRowPieces, part = q % kRowPieces, row = b * kBlk + rl;
      const int ux = s_ux[row];
      const u32x4 v = ux >= 0 ? raw[b & 1][e] : (u32x4){0u, 0u, 0u, 0u};
      if ((early || b + 1 == NBLK) && ux >= 0)
        __builtin_nontemporal_store(v, reinterpret_cast<DSA_GLOBAL u32x4*>(s.compact + (int64_t)ux * rb + 16 * part));
      if (part < 32) {
        uint32_t w[8];
        widen16(v, w);
        uint32_t* dst = reinterpret_cast<uint32_t*>(lat + rl * kLatStride + 16 * part);
        *reinterpret_cast<u32x4*>(dst) = (u32x4){w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(dst + 4) = (u32x4){w[4], w[5], w[6], w[7]};
      } else if (part == 32) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const uint32_t word = v[g >> 1];
          scl[g * kBlk + rl] = f16_bits_to_f32((g & 1) ? (word >> 16) : (word & 0xFFFFu));
        }
      } else {
        *reinterpret_cast<u32x4*>(rope + rl * kRopeStride + 8 * (part - 33)) = v;
      }
    }
    if (b + 1 < NBLK && !(b == 0 && early)) request(b + 1);
    __syncthreads();

    // Logits S^T[j][h]: lane holds rows 16 mt + 4 q4 + v of head h0 + l16; each
    // 64-dim group is accumulated separately and scaled by its fp32 scale per row.
    float lg[2][4];
    {
      f32x4 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) sacc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        f32x4 acc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ks = 2 * g + kk;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 av = *reinterpret_cast<const bf16x8*>(lat + (16 * mt + l16) * kLatStride + 32 * ks + 8 * q4);
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qa[ks], acc[mt], 0, 0, 0);
          }
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const f32x4 sc = *reinterpret_cast<const f32x4*>(scl + g * kBlk + 16 * mt + 4 * q4);
#pragma unroll
          for (int v = 0; v < 4; ++v) sacc[mt][v] += sc[v] * acc[mt][v];
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(rope + (16 * mt + l16) * kRopeStride + 32 * kk + 8 * q4);
          sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qa[16 + kk], sacc[mt], 0, 0, 0);
        }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = b * kBlk + 16 * mt + 4 * q4 + v;
          lg[mt][v] = s_ux[j] >= 0 ? sacc[mt][v] * ka.scale_log2 : -INFINITY;
        }
    }

    // Online softmax of head h0 + l16 (the block's 32 rows sit in the 4 lane groups).
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, lg[mt][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : exp2_hw(m_run - m_new);
    float p[2][4];
    float ps = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[mt][v] = none ? 0.f : exp2_hw(lg[mt][v] - m_new);
        ps += p[mt][v];
      }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (b > 0) {
      // O rows are heads h0 + 4 q4 + v: their alphas come from lanes 4 q4 + v
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = __shfl(alpha, 4 * q4 + v);
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt) o[nt][v] *= av;
      }
    }

    // O[h][d] += sum_j (p[h][j] * scale_j[g]) * int8_j[d].  The A fragment of
    // head h0 + l16 holds rows {4 q4 .. 4 q4 + 3, 16 + 4 q4 .. 16 + 4 q4 + 3}, in
    // that order; the B fragments (LDS transpose reads) match it.
#pragma unroll
    for (int gl = 0; gl < GD; ++gl) {
      const int g = GD * dh + gl;                        // the 64-dim group (its scale)
      bf16x8 pa_hi, pa_lo;
      {
        const f32x4 sa = *reinterpret_cast<const f32x4*>(scl + g * kBlk + 4 * q4);
        const f32x4 sb = *reinterpret_cast<const f32x4*>(scl + g * kBlk + 16 + 4 * q4);
        float pv[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pv[v] = p[0][v] * sa[v];
          pv[4 + v] = p[1][v] * sb[v];
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = pack_bf16(pv[2 * e], pv[2 * e + 1]);
          lo[e] = pack_bf16(pv[2 * e] - bf16_lo_to_f32(hi[e]), pv[2 * e + 1] - bf16_hi_to_f32(hi[e]));
        }
        __builtin_memcpy(&pa_hi, hi, 16);
        __builtin_memcpy(&pa_lo, lo, 16);
      }
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int nt = 4 * gl + t4, col = 16 * (4 * g + t4);
        const bf16x4 b0 = read_tr(lat, 4 * q4, col, lane);
        const bf16x4 b1 = read_tr(lat, 16 + 4 * q4, col, lane);
        const bf16x8 bv = (bf16x8){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, bv, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, bv, o[nt], 0, 0, 0);
      }
    }

    // A split with host-mirror rows, not its last block: the block's compact rows, now (above).
#pragma unroll
    for (int e = 0; e < PPT && !early && b + 1 < NBLK; ++e) {
      const int q = tid + e * NT;
      if (q >= kBlkPieces) continue;
      const int rl = q / kRowPieces, part = q % kRowPieces;
      const int ux = s_ux[b * kBlk + rl];
      if (ux >= 0)
        __builtin_nontemporal_store(raw[b & 1][e],
                                    reinterpret_cast<DSA_GLOBAL u32x4*>(s.compact + (int64_t)ux * rb + 16 * part));
    }
  }
  const float mx = m_run, ps = l_run;

  // o[nt][v] = O[h0 + 4 q4 + v][16 (NTD dh + nt) + l16]; (max, sum) of head h0 + l16 in every lane group
  if (ka.nsplit == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float den = __shfl(ps, 4 * q4 + v);
      const float inv = den > 0.f ? 1.f / den : 0.f;
      float* dst = ka.out + (((int64_t)seq * a.R + r) * H + h0 + 4 * q4 + v) * 512 + 16 * NTD * dh;
#pragma unroll
      for (int nt = 0; nt < NTD; ++nt) dst[nt * 16 + l16] = o[nt][v] * inv;
    }
  } else {
    // The split's partial, normalised (y = O / sum, a weighted mean of the
    // split's dequantised rows) and stored as fp16 with a power-of-two scale per
    // head that keeps |y| below 2^15: relative rounding 2^-11 per element, and
    // half the bytes of fp32 for the merge to read.  Layout
    // [r][split][wave][nt][l16][16 heads]: a wave's store covers 512 contiguous
    // bytes per nt (whole lines); the lane's four heads are contiguous.  Only
    // the merge reads them, once: non-temporal stores (measured: the attention
    // launch ends 0.8 us sooner, the merge reads them 0.5 us slower).
    // The DS waves of a head group take the largest |O| over all 512 dims, so
    // they agree on each head's scale.
    f32x4 amax = (f32x4){0.f, 0.f, 0.f, 0.f};        // per head, of the unnormalised O
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) amax[v] = fmaxf(amax[v], fabsf(o[nt][v]));
    if constexpr (DS > 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int sh = 1; sh < 16; sh <<= 1) amax[v] = fmaxf(amax[v], __shfl_xor(amax[v], sh));
      if (l16 == 0)
#pragma unroll
        for (int v = 0; v < 4; ++v) s_amax[wave][4 * q4 + v] = amax[v];
      __syncthreads();
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int d = 0; d < DS; ++d) amax[v] = fmaxf(amax[v], s_amax[hg + HG * d][4 * q4 + v]);
    }
    float scv[4], mul[4];                            // the scale, and 1 / sum times the scale
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float m = amax[v];
      if constexpr (DS == 1)
#pragma unroll
        for (int sh = 1; sh < 16; sh <<= 1) m = fmaxf(m, __shfl_xor(m, sh));
      const float den = __shfl(ps, 4 * q4 + v);      // the sum of head h0 + 4 q4 + v
      const float inv = den > 0.f ? 1.f / den : 0.f;
      int ex = 0;
      (void)frexpf(m * inv, &ex);                    // max |y| < 2^ex
      scv[v] = ex > 15 ? ldexpf(1.f, 15 - ex) : 1.f;
      mul[v] = inv * scv[v];
    }
    const auto dst = s.part_o + ((((int64_t)r * ka.ns_stride + split) * HG + hg) * 32 * 16 + l16) * 16 + 4 * q4 +
                     (int64_t)NTD * dh * 16 * 16;
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt) {
      u32x2 w;
      w.x = pack_f16(o[nt][0] * mul[0], o[nt][1] * mul[1]);
      w.y = pack_f16(o[nt][2] * mul[2], o[nt][3] * mul[3]);
      __builtin_nontemporal_store(w, reinterpret_cast<DSA_GLOBAL u32x2*>(dst + (int64_t)nt * 16 * 16));
    }
    // (max, sum, 1 / scale) of head h0 + l16: its scale sits in lane group l16 / 4, register l16 % 4
    const float s0 = __shfl(scv[0], 16 * (l16 >> 2)), s1 = __shfl(scv[1], 16 * (l16 >> 2));
    const float s2 = __shfl(scv[2], 16 * (l16 >> 2)), s3 = __shfl(scv[3], 16 * (l16 >> 2));
    const float sc = (l16 & 3) == 0 ? s0 : (l16 & 3) == 1 ? s1 : (l16 & 3) == 2 ? s2 : s3;
    if (q4 == 0 && dh == 0) {
      const int64_t base = ((int64_t)r * ka.ns_stride + split) * H + h0 + l16;
      __builtin_nontemporal_store((f32x4){mx, ps, 1.f / sc, 0.f}, reinterpret_cast<DSA_GLOBAL f32x4*>(s.part_ml + base * 4));
    }
  }
}

struct MergeKArgs {
  GatherKArgs ga;            // the assign pass (ga.a: the step's arguments)
  float* out;
  int H, ns_stride;
  int split_rows;            // selected rows per attention split
  int assign_blocks;         // assign workgroups per sequence (first: their chain of loads is the longer);
                             // the rest of a row of the grid merge
};

// Workgroups [0, assign_blocks) of each sequence run the gather's assign pass
// (gather_assign.h), which nothing in the round waits for; the others merge.
// One merge workgroup per (16-dim tile nt, group of HW heads, query row), for
// at most MAXS splits, each split s holding y_s = O_s / l_s times its scale c_s:
// out[h][d] = sum_s w_s[h] y_s[h][d] with w_s = 2^(m_s - M) l_s / sum_s' 2^(m_s' - M) l_s'.
// A split's tile of dims nt is 16 heads x 16 dims per attention wave (512
// contiguous bytes of fp16); the workgroup reads the tiles of its HW heads
// (whole lines), EPT consecutive values per thread.  The sums leave through LDS
// as [h][16] (16 contiguous floats per head).
template <int MAXS, int HW>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeKArgs ka) {
  constexpr int EPT = 16 * HW / 256;          // tile elements per thread
  constexpr int TPH = 256 / HW;               // threads per head in the weight pass
  constexpr int kPer = (MAXS + TPH - 1) / TPH;
  static_assert(EPT >= 1 && 16 * HW == 256 * EPT, "tile of 16 x HW floats over 256 threads");
  __shared__ float wgt[MAXS * HW];            // [split][head]: the max, then the weight
  __shared__ float sl[MAXS * HW];             // [split][head]: the sum
  __shared__ float isc[MAXS * HW];            // [split][head]: 1 / the partial's scale
  __shared__ float tile[HW * 17];
  const StepArgs& a = ka.ga.a;
  const int seq = blockIdx.y;
  if ((int)blockIdx.x < ka.assign_blocks) {             // (uniform) an assign workgroup
    assign_block(ka.ga, (int)blockIdx.x, seq);
    return;
  }
  const int mb = (int)blockIdx.x - ka.assign_blocks;   // this merge workgroup
  const int n_hg = ka.H / HW;
  const int r = mb / (32 * n_hg), rem = mb % (32 * n_hg);
  const int nt = rem / n_hg, hg = rem % n_hg;
  const ScratchG s = scratch_of(a, seq);
  const int H = ka.H;
  const int used = min(MAXS, min((ka.ga.K + ka.split_rows - 1) / ka.split_rows, s.sel_n[r]));
  if (used < 1) return;                                  // (uniform) no selection: nothing to merge
  const int tid = threadIdx.x;
  const int e0 = tid * EPT, l16 = e0 / HW, hl0 = e0 % HW;
  // Every split's (max, sum, 1 / scale) of the workgroup's heads is requested
  // first, then this thread's elements of every split (splits past `used`
  // re-read the last one and get weight 0): loads complete in issue order, so
  // the weights are formed while the elements are still arriving.
  static_assert(EPT <= 2, "a thread's elements lie in one attention wave's tile");
  constexpr int kMl = (MAXS * HW + 255) / 256;          // (max, sum, 1 / scale) loads per thread
  // (every address first: the loads then issue back to back)
  const DSA_GLOBAL f32x4* mlp[kMl];
#pragma unroll
  for (int e = 0; e < kMl; ++e) {
    const int t = tid + 256 * e;
    const int sp = min(t / HW, used - 1), h = t % HW;
    mlp[e] = reinterpret_cast<const DSA_GLOBAL f32x4*>(s.part_ml) + ((int64_t)r * ka.ns_stride + sp) * H + HW * hg + h;
  }
  const int hh = HW * hg + hl0;                          // the thread's first head
  const auto src = s.part_o + (((int64_t)r * ka.ns_stride * (H / 16) + hh / 16) * 32 + nt) * 256 + l16 * 16 + hh % 16;
  const int64_t split_stride = (int64_t)32 * 16 * H;
  f32x4 mlv[kMl];
#pragma unroll
  for (int e = 0; e < kMl; ++e) mlv[e] = *mlp[e];
  uint32_t xr[MAXS];                                     // fp16 bits (two heads per word when EPT == 2)
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp) {
    const auto at = src + (sp < used ? sp : used - 1) * split_stride;
    if constexpr (EPT == 2) xr[sp] = *reinterpret_cast<const DSA_GLOBAL uint32_t*>(at);
    else xr[sp] = *at;
  }
#pragma unroll
  for (int e = 0; e < kMl; ++e) {
    const int t = tid + 256 * e;
    if (t < used * HW) {
      wgt[t] = mlv[e][0];
      sl[t] = mlv[e][1];
      isc[t] = mlv[e][2];
    }
  }
  __syncthreads();
  {
    // the weights of head wh: its TPH threads take the splits c, c + TPH, ...,
    // then reduce the max and the denominator by shuffles
    const int wh = tid / TPH, c = tid % TPH;
    float mloc[kPer];
    float M = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int sp = c + TPH * e;
      mloc[e] = sp < used ? wgt[sp * HW + wh] : -INFINITY;
      M = fmaxf(M, mloc[e]);
    }
#pragma unroll
    for (int o = 1; o < TPH; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    float wloc[kPer];
    float den = 0.f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int sp = c + TPH * e;
      wloc[e] = (sp < used && M != -INFINITY) ? exp2_hw(mloc[e] - M) : 0.f;
      if (sp < used) den += wloc[e] * sl[sp * HW + wh];
    }
#pragma unroll
    for (int o = 1; o < TPH; o <<= 1) den += __shfl_xor(den, o);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    __syncthreads();                                   // every max read before any weight is written
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int sp = c + TPH * e;
      if (sp < used) wgt[sp * HW + wh] = wloc[e] * inv * sl[sp * HW + wh] * isc[sp * HW + wh];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    float acc = 0.f;
#pragma unroll
    for (int sp = 0; sp < MAXS; ++sp)
      acc += (sp < used ? wgt[sp * HW + hl0 + k] : 0.f) * f16_bits_to_f32(k == 0 ? (xr[sp] & 0xFFFFu) : (xr[sp] >> 16));
    tile[(hl0 + k) * 17 + l16] = acc;
  }
  __syncthreads();
  for (int t = tid; t < HW * 16; t += 256) {
    const int h2 = t / 16, d2 = t % 16;
    ka.out[(((int64_t)seq * a.R + r) * H + HW * hg + h2) * 512 + nt * 16 + d2] = tile[h2 * 17 + d2];
  }
}

}  // namespace

// Rows per attention split: 64 (two blocks).  Longer splits halve the partials
// the merge reads, but when most selected rows are hits they halve the
// workgroups of a kernel that is then latency-bound, not link-bound.
inline int split_rows(const Geometry&) { return kSplit; }

hipError_t launch_attn(const Geometry& g, const StepArgs& a, const uint16_t* q_lat, const uint16_t* q_rope,
                       float* out, hipStream_t st, int plan) {
  const int rows = split_rows(g);
  const int nsplit = (g.top_k + rows - 1) / rows;
  AttnKArgs ka{a, q_lat, q_rope, out, g.top_k, g.heads, nsplit, g.nsplit_max, g.row_bytes,
               g.hot_slots, g.ring_cap, g.r_max * g.top_k, g.mode == 0 ? 1 : 0, g.max_positions,
               g.softmax_scale * 1.4426950408889634f, plan,
               PlanParams{g.hot_slots, g.s_words, g.ring_rows, g.mode, g.clock ? 1 : 0, a.add}};
  // one workgroup past the splits of each (row, sequence): row 0's runs the plan's part
  dim3 grid((unsigned)nsplit + 1u, (unsigned)a.R, (unsigned)a.n_seqs);
  // Two waves per head group where that keeps a workgroup within 512 threads.
  switch (g.heads) {
    case 16: return launch_k(attn_kernel<1, 2, 2>, grid, dim3(128), 0, st, ka);
    case 32: return launch_k(attn_kernel<2, 2, 2>, grid, dim3(256), 0, st, ka);
    case 64: return launch_k(attn_kernel<4, 2, 2>, grid, dim3(512), 0, st, ka);
    case 128: return launch_k(attn_kernel<8, 1, 2>, grid, dim3(512), 0, st, ka);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_merge(const Geometry& g, const StepArgs& a, float* out, hipStream_t st) {
  int64_t assign_blocks = 0;
  const GatherKArgs ga = gather_args(g, a, true, true, &assign_blocks);
  const int rows = split_rows(g);
  const int nsplit = (g.top_k + rows - 1) / rows;
  const int HW = g.heads == 16 ? 16 : 32;
  const int merge_blocks = nsplit == 1 ? 0 : 32 * (g.heads / HW) * a.R;   // one split: attention wrote out
  MergeKArgs ka{ga, out, g.heads, g.nsplit_max, rows, (int)assign_blocks};
  const dim3 grid((unsigned)(merge_blocks + assign_blocks), (unsigned)a.n_seqs);
  static_assert(kGatherThreads == 256, "assign and merge workgroups share the launch");
  if (HW == 16) {
    if (nsplit <= 32) return launch_k(attn_merge_kernel<32, 16>, grid, dim3(256), 0, st, ka);
    return launch_k(attn_merge_kernel<kMaxSplits, 16>, grid, dim3(256), 0, st, ka);
  }
  if (nsplit <= 16) return launch_k(attn_merge_kernel<16, 32>, grid, dim3(256), 0, st, ka);
  if (nsplit <= 32) return launch_k(attn_merge_kernel<32, 32>, grid, dim3(256), 0, st, ka);
  return launch_k(attn_merge_kernel<kMaxSplits, 32>, grid, dim3(256), 0, st, ka);
}

}  // namespace dsa
