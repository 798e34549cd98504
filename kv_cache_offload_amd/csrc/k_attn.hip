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
// gfx950 mapping.  A workgroup owns one query row and a split of its selected
// rows, all heads: wave w holds heads 16w..16w+15.  Rows are processed 32 at a
// time.  The int8 latent is widened to bf16 in LDS (exact: |int8| < 2^8) in two
// layouts -- row-major for QK^T (the MFMA K index runs over dims) and
// dim-major for PV (the K index runs over rows) -- and the per-group scale is
// kept in fp32: QK^T accumulates each 64-dim group separately with
// v_mfma_f32_16x16x32_bf16 and scales the 16x16 group result per row before
// adding; PV folds the scale into P (P'_g = p * scale_g per group), carried as
// a bf16 high part plus a bf16 low part so the weights keep ~16 mantissa bits.  The query sits in registers for the whole workgroup (18 A
// fragments).  Softmax is online over the 32-row blocks in the exp2 domain;
// each workgroup writes (max, sum, unnormalised O) and a merge kernel combines
// the splits with the log-sum-exp rule.
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kSub = kAttnSubRows;     // 32 rows per block
constexpr int kLatStride = 520;        // bf16 per row in the row-major latent (512 + 8)
constexpr int kDjStride = 40;          // bf16 per dim in the dim-major latent (32 + 8)
constexpr int kRopeStride = 72;        // bf16 per row of RoPE (64 + 8)
constexpr int kPStride = 33;           // f32 per head row of P (32 + 1)
constexpr int kMaxSplitRows = 256;     // selected rows per workgroup at most
constexpr int kMaxSplits = 4096 / 64;  // K <= 4096, at least 64 rows per split

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float f16_bits_to_f32(uint16_t h) {
  _Float16 f;
  __builtin_memcpy(&f, &h, 2);
  return (float)f;                     // exact widening
}

struct AttnKArgs {
  StepArgs a;
  const uint16_t* q_lat;     // [n_seqs][R][H][512]
  const uint16_t* q_rope;    // [n_seqs][R][H][64]
  float* out;                // [n_seqs][R][H][512]
  int K, H, split_rows, nsplit, ns_stride, row_bytes;
  int64_t max_positions;
  float scale_log2;          // softmax_scale * log2(e)
};

// Raw Q8G64 bytes of one 32-row block, held in registers so the next block's
// loads are in flight while the current block is computed.  Latent task t covers
// 8 rows (group t % 4) x 8 dims (chunk t / 4); side task covers one row's scale
// of one group plus 16 bytes of its RoPE.
template <int NW>
struct RawBlock {
  static constexpr int kLatTasks = (kSub / 8) * 64 / (NW * 64);   // per thread
  static constexpr int kSideTasks = kSub * 8 / (NW * 64);
  u32x2 lat[kLatTasks][8];
  uint16_t scl[kSideTasks];
  u32x4 rope[kSideTasks];

  __device__ inline void load(const DSA_GLOBAL uint8_t* compact, const int* idx, int64_t rb, int tid) {
#pragma unroll
    for (int q = 0; q < kLatTasks; ++q) {
      const int task = tid + q * NW * 64;
      const int jg = task & 3, dc = task >> 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int id = idx[jg * 8 + e];
        // unconditional loads (row 0 always exists); rows past the split's end are
        // masked out of the softmax, so their values never reach the output
        lat[q][e] = *reinterpret_cast<const DSA_GLOBAL u32x2*>(compact + (id >= 0 ? id : 0) * rb + dc * 8);
      }
    }
#pragma unroll
    for (int q = 0; q < kSideTasks; ++q) {
      const int task = tid + q * NW * 64;
      const int j = task >> 3, g = task & 7;
      const int id = idx[j];
      const int64_t row = (id >= 0 ? id : 0) * rb;
      scl[q] = *reinterpret_cast<const DSA_GLOBAL uint16_t*>(compact + row + 512 + 2 * g);
      rope[q] = *reinterpret_cast<const DSA_GLOBAL u32x4*>(compact + row + 528 + 16 * g);
    }
  }

  // int8 -> bf16 (exact) in both layouts; scales to fp32; RoPE copied.
  __device__ inline void store(uint16_t* lat_jd, uint16_t* lat_dj, uint16_t* rope_jd, float* sclf, int tid) const {
#pragma unroll
    for (int q = 0; q < kLatTasks; ++q) {
      const int task = tid + q * NW * 64;
      const int jg = task & 3, dc = task >> 2;        // row group fastest: conflict-free dim-major writes
      uint16_t w[8][8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t word = k < 4 ? lat[q][e].x : lat[q][e].y;
          const int8_t v = (int8_t)((word >> (8 * (k & 3))) & 0xFFu);
          w[e][k] = (uint16_t)(__float_as_uint((float)v) >> 16);
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x8 row;
#pragma unroll
        for (int k = 0; k < 8; ++k) row[k] = (short)w[e][k];
        *reinterpret_cast<bf16x8*>(lat_jd + (jg * 8 + e) * kLatStride + dc * 8) = row;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        bf16x8 col;
#pragma unroll
        for (int e = 0; e < 8; ++e) col[e] = (short)w[e][k];
        *reinterpret_cast<bf16x8*>(lat_dj + (dc * 8 + k) * kDjStride + jg * 8) = col;
      }
    }
#pragma unroll
    for (int q = 0; q < kSideTasks; ++q) {
      const int task = tid + q * NW * 64;
      const int j = task >> 3, g = task & 7;
      sclf[j * 8 + g] = f16_bits_to_f32(scl[q]);
      *reinterpret_cast<u32x4*>(rope_jd + j * kRopeStride + 8 * g) = rope[q];
    }
  }
};

// One workgroup: one query row, NW*16 heads, one split of the row's selection.
template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnKArgs ka) {
  __shared__ __align__(16) uint16_t lat_jd[kSub * kLatStride];   // also the P staging area
  __shared__ __align__(16) uint16_t lat_dj[512 * kDjStride];
  __shared__ __align__(16) uint16_t rope_jd[kSub * kRopeStride];
  __shared__ float scl[kSub * 8];
  __shared__ int s_idx[kMaxSplitRows];

  const StepArgs& a = ka.a;
  const int split = blockIdx.x, seq = blockIdx.z;
  const int n_hg = ka.H / (NW * 16);
  const int r = blockIdx.y / n_hg, hg = blockIdx.y % n_hg;
  const ScratchG s = scratch_of(a, seq);
  const int n_sel = s.sel_n[r];
  const int j_begin = split * ka.split_rows;
  if (j_begin >= n_sel) return;
  const int j_end = min(n_sel, j_begin + ka.split_rows);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int H = ka.H;
  const int h0 = hg * NW * 16 + wave * 16;
  const int64_t rb = ka.row_bytes;

  // Compact-row index of every selected row of this split (the map: union index of
  // the selected position, from the per-position index the gather wrote).
  const auto sel = s.sel + (int64_t)r * ka.K;
  const auto map = s.map + (int64_t)r * ka.K;
  const int64_t U = s.info[kInfoUnion];
  for (int j = tid; j < ka.split_rows; j += NW * 64) {
    int idx = -1;
    if (j_begin + j < j_end) {
      const int32_t p = sel[j_begin + j];
      idx = (p >= 0 && p < ka.max_positions) ? s.upos[p] : -1;
      if (idx >= U) idx = -1;                        // never index past the compact rows
      if (hg == 0) map[j_begin + j] = idx;
    }
    s_idx[j] = idx;
  }
  if (split == 0 && hg == 0)
    for (int j = n_sel + tid; j < ka.K; j += NW * 64) map[j] = -1;
  __syncthreads();

  RawBlock<NW> raw;
  raw.load(s.compact, s_idx, rb, tid);

  // Query fragments: lane holds Q[h0 + l16][32*ks + 8*g4 .. +7].
  bf16x8 qa[18];
  {
    const int64_t qrow = ((int64_t)seq * a.R + r) * H + h0 + l16;
    const uint16_t* ql = ka.q_lat + qrow * 512 + 8 * g4;
    const uint16_t* qr = ka.q_rope + qrow * 64 + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qa[ks] = *reinterpret_cast<const bf16x8*>(ql + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qa[16 + ks] = *reinterpret_cast<const bf16x8*>(qr + 32 * ks);
  }

  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { m_run[v] = -INFINITY; l_run[v] = 0.f; }

  for (int jb = j_begin; jb < j_end; jb += kSub) {
    const int nrows = min(kSub, j_end - jb);
    __syncthreads();                                   // previous block's PV is done with LDS
    raw.store(lat_jd, lat_dj, rope_jd, scl, tid);
    if (jb + kSub < j_end) raw.load(s.compact, s_idx + (jb + kSub - j_begin), rb, tid);
    __syncthreads();
    // QK^T: logits for heads h0+4*g4+v, rows nt*16 + l16.
    f32x4 lg[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int jrow = nt * 16 + l16;
      f32x4 acc_all = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ks = 2 * g + kk;
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(lat_jd + jrow * kLatStride + 32 * ks + 8 * g4);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], b, acc, 0, 0, 0);
        }
        const float sc = scl[jrow * 8 + g];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc_all[v] += sc * acc[v];
      }
      f32x4 ra = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(rope_jd + jrow * kRopeStride + 32 * kk + 8 * g4);
        ra = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[16 + kk], b, ra, 0, 0, 0);
      }
      const bool valid = jrow < nrows && s_idx[jb - j_begin + jrow] >= 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) lg[nt][v] = valid ? (acc_all[v] + ra[v]) * ka.scale_log2 : -INFINITY;
    }

    // Online softmax per head (16 lanes of a group share the head's rows).
    float p[2][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float mx = fmaxf(lg[0][v], lg[1][v]);
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
      const float m_new = fmaxf(m_run[v], mx);
      const bool none = m_new == -INFINITY;
      const float alpha = none ? 1.f : exp2f(m_run[v] - m_new);
      p[0][v] = none ? 0.f : exp2f(lg[0][v] - m_new);
      p[1][v] = none ? 0.f : exp2f(lg[1][v] - m_new);
      float ps = p[0][v] + p[1][v];
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) ps += __shfl_xor(ps, o2);
      l_run[v] = l_run[v] * alpha + ps;
      m_run[v] = m_new;
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i][v] *= alpha;
    }

    // Stage P through LDS to the A-operand layout (lane: head l16, rows 8*g4..+7).
    __syncthreads();                                   // every wave is done reading lat_jd
    float* pbuf = reinterpret_cast<float*>(lat_jd) + wave * 16 * kPStride;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) pbuf[(4 * g4 + v) * kPStride + nt * 16 + l16] = p[nt][v];
    __syncthreads();
    float pr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[e] = pbuf[l16 * kPStride + 8 * g4 + e];

    // PV: O[h][d] += sum_j (p[h][j] * scale_j[g]) * int8_j[d], group g = d / 64.
    // P' is split into bf16 high and low parts (P' = hi + lo to about 2^-16 relative), so
    // the weights keep fp32-like precision while the int8 operand stays exact in bf16.
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      bf16x8 pa_hi, pa_lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = pr[e] * scl[(8 * g4 + e) * 8 + g];
        const uint16_t hi = f32_to_bf16_rne(pv);
        pa_hi[e] = (short)hi;
        pa_lo[e] = (short)f32_to_bf16_rne(pv - __uint_as_float((uint32_t)hi << 16));
      }
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int nt2 = g * 4 + t4;
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(lat_dj + (nt2 * 16 + l16) * kDjStride + 8 * g4);
        o[nt2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, b, o[nt2], 0, 0, 0);
        o[nt2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, b, o[nt2], 0, 0, 0);
      }
    }
  }

  // o[nt2][v] = O[h0 + 4*g4 + v][nt2*16 + l16]
  if (ka.nsplit == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = h0 + 4 * g4 + v;
      const float inv = 1.f / l_run[v];
      float* dst = ka.out + (((int64_t)seq * a.R + r) * H + h) * 512;
#pragma unroll
      for (int nt2 = 0; nt2 < 32; ++nt2) dst[nt2 * 16 + l16] = o[nt2][v] * inv;
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = h0 + 4 * g4 + v;
      const int64_t base = ((int64_t)r * ka.ns_stride + split) * H + h;
      const auto dst = s.part_o + base * 512;
#pragma unroll
      for (int nt2 = 0; nt2 < 32; ++nt2) dst[nt2 * 16 + l16] = o[nt2][v];
      if (l16 == 0) {
        s.part_ml[base * 2 + 0] = m_run[v];
        s.part_ml[base * 2 + 1] = l_run[v];
      }
    }
  }
}

struct MergeKArgs {
  StepArgs a;
  float* out;
  int H, split_rows, ns_stride;
};

// One workgroup per (head, query row): out[d] = sum_s w_s O_s[d] with
// w_s = 2^(m_s - M) / sum_s' 2^(m_s' - M) l_s'.
__global__ __launch_bounds__(128) void attn_merge_kernel(MergeKArgs ka) {
  __shared__ float wgt[kMaxSplits];
  const StepArgs& a = ka.a;
  const int h = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const ScratchG s = scratch_of(a, seq);
  const int used = (s.sel_n[r] + ka.split_rows - 1) / ka.split_rows;
  const int H = ka.H;
  // splits' (max, sum) in the first wave, one split per lane (used <= 64)
  if (threadIdx.x < 64) {
    const int sp = threadIdx.x;
    float m = -INFINITY, l = 0.f;
    if (sp < used) {
      const int64_t base = ((int64_t)r * ka.ns_stride + sp) * H + h;
      m = s.part_ml[base * 2];
      l = s.part_ml[base * 2 + 1];
    }
    float mx = m;
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float w = sp < used ? exp2f(m - mx) : 0.f;
    float den = w * l;
    for (int o = 1; o < 64; o <<= 1) den += __shfl_xor(den, o);
    if (sp < used) wgt[sp] = w / den;
  }
  __syncthreads();
  const int d = threadIdx.x * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int sp = 0; sp < used; ++sp) {
    const f32x4 v = *reinterpret_cast<const DSA_GLOBAL f32x4*>(
        s.part_o + (((int64_t)r * ka.ns_stride + sp) * H + h) * 512 + d);
    const float w = wgt[sp];
    acc.x += w * v[0]; acc.y += w * v[1]; acc.z += w * v[2]; acc.w += w * v[3];
  }
  *reinterpret_cast<float4*>(ka.out + (((int64_t)seq * a.R + r) * H + h) * 512 + d) = acc;
}

// Rows per workgroup: 128, or 64 when that leaves fewer than 256 workgroups.
int attn_split_rows(const Geometry& g, const StepArgs& a) {
  const int nw = g.heads >= 32 ? 2 : 1;
  const int64_t groups = (int64_t)a.R * a.n_seqs * (g.heads / (16 * nw));
  const int64_t wg128 = groups * ((g.top_k + 127) / 128);
  return wg128 >= 256 ? 128 : 64;
}

}  // namespace

hipError_t launch_attn(const Geometry& g, const StepArgs& a, const uint16_t* q_lat, const uint16_t* q_rope,
                       float* out, hipStream_t st) {
  const int split_rows = attn_split_rows(g, a);
  const int nsplit = (g.top_k + split_rows - 1) / split_rows;
  const int nw = g.heads >= 32 ? 2 : 1;
  AttnKArgs ka{a, q_lat, q_rope, out, g.top_k, g.heads, split_rows, nsplit, g.nsplit_max, g.row_bytes,
               g.max_positions, g.softmax_scale * 1.4426950408889634f};
  dim3 grid((unsigned)nsplit, (unsigned)(a.R * (g.heads / (16 * nw))), (unsigned)a.n_seqs);
  if (nw == 1) return launch_k(attn_kernel<1>, grid, dim3(64), 0, st, ka);
  return launch_k(attn_kernel<2>, grid, dim3(128), 0, st, ka);
}

hipError_t launch_attn_merge(const Geometry& g, const StepArgs& a, float* out, hipStream_t st) {
  const int split_rows = attn_split_rows(g, a);
  if ((g.top_k + split_rows - 1) / split_rows == 1) return hipSuccess;
  MergeKArgs ka{a, out, g.heads, split_rows, g.nsplit_max};
  return launch_k(attn_merge_kernel, dim3((unsigned)g.heads, (unsigned)a.R, (unsigned)a.n_seqs), dim3(128), 0, st,
                  ka);
}

}  // namespace dsa
