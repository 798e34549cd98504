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
// rows, all heads: wave w holds heads 16w..16w+15.  Rows go through LDS 32 at
// a time, staged once for all waves: the int8 latent widened to bf16 (exact,
// |int8| < 2^8) in one row-major layout, the fp16 scales as fp32, the RoPE as
// is; the next block's bytes are already in registers while the current one is
// computed.  Both products run on v_mfma_f32_16x16x32_bf16:
//   * logits, transposed: S^T[j][h] = sum_d C[j][d] Q[h][d], the A operand
//     read straight from the row-major latent, the query (B operand) held in
//     registers for the whole workgroup; each 64-dim group is accumulated
//     separately and scaled by its fp32 scale per row, so the int8 operand
//     stays exact;
//   * output: O[h][d] += sum_j P'_g[h][j] C[j][d] with P'_g = p * scale_g,
//     carried as a bf16 high part plus a bf16 low part (~16 mantissa bits).
//     In the transposed logits a lane already holds p for one head and 8 rows,
//     which is exactly its A fragment, so P never goes through LDS; the B
//     fragments (8 rows of one dim) come from the row-major latent with the
//     LDS transpose read ds_read_b64_tr_b16 (4 rows x 1 column per lane).
// Softmax is online over the 32-row blocks in the exp2 domain; each
// workgroup writes (max, sum, unnormalised O) and a merge kernel combines the
// splits with the log-sum-exp rule.
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef short bf16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float fx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bfx2 __attribute__((ext_vector_type(2)));
#define DSA_LDS __attribute__((address_space(3)))

constexpr int kBlk = kAttnSubRows;     // 32 selected rows per block
constexpr int kLatStride = 520;        // bf16 per row of the latent in LDS (512 + 8)
constexpr int kRopeStride = 72;        // bf16 per row of RoPE (64 + 8)
constexpr int kMaxSplitRows = 256;     // selected rows per workgroup at most
constexpr int kMaxSplits = 4096 / 64;  // K <= 4096, at least 64 rows per split
constexpr int kSidePieces = kBlk * 9;  // 16-byte pieces of scales + RoPE per block

struct AttnKArgs {
  StepArgs a;
  const uint16_t* q_lat;     // [n_seqs][R][H][512]
  const uint16_t* q_rope;    // [n_seqs][R][H][64]
  float* out;                // [n_seqs][R][H][512]
  int K, H, split_rows, nsplit, ns_stride, row_bytes;
  int64_t max_positions;
  float scale_log2;          // softmax_scale * log2(e)
};

template <class T>
__device__ inline void keep(T& x) {
  asm volatile("" : "+v"(x));
}

// Two fp32 -> packed bf16 (round to nearest even), as one 32-bit word.
__device__ inline uint32_t pack_bf16(float a, float b) {
  const bfx2 v = __builtin_convertvector((fx2){a, b}, bfx2);
  uint32_t w;
  __builtin_memcpy(&w, &v, 4);
  return w;
}

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

// The bytes of one 32-row block, in registers between the global loads and the
// LDS stores.  Latent piece p (16 bytes) of the block: row p / 32, bytes
// 16 (p % 32).. ; side piece q: row q / 9, part q % 9 (0: the 8 scales, 1..8:
// 16 bytes of RoPE).
template <int NT>
struct RawBlock {
  static constexpr int LP = kBlk * 32 / NT;
  static constexpr int SP = (kSidePieces + NT - 1) / NT;
  u32x4 lat[LP];
  u32x4 side[SP];

  // rows past the split, or with no valid union index, read compact row 0 (it
  // exists whenever a split has work); their logits are masked, so their
  // values never reach the output
  __device__ inline void load(const DSA_GLOBAL uint8_t* compact, const int* idx, int64_t rb, int tid) {
#pragma unroll
    for (int p = 0; p < LP; ++p) {
      const int piece = tid + p * NT;
      const int id = idx[piece >> 5];
      lat[p] = *reinterpret_cast<const DSA_GLOBAL u32x4*>(compact + (id >= 0 ? id : 0) * rb + 16 * (piece & 31));
    }
#pragma unroll
    for (int q = 0; q < SP; ++q) {
      const int piece = min(tid + q * NT, kSidePieces - 1);
      const int row = piece / 9, part = piece % 9;
      const int id = idx[row];
      side[q] = *reinterpret_cast<const DSA_GLOBAL u32x4*>(compact + (id >= 0 ? id : 0) * rb + 512 +
                                                           (part ? 16 + 16 * (part - 1) : 0));
    }
  }

  __device__ inline void store(uint16_t* lat_s, uint16_t* rope_s, float* scl_s, int tid) const {
#pragma unroll
    for (int p = 0; p < LP; ++p) {
      const int piece = tid + p * NT;
      const int row = piece >> 5, c16 = piece & 31;
      uint32_t w[8];
      widen16(lat[p], w);
      uint32_t* dst = reinterpret_cast<uint32_t*>(lat_s + row * kLatStride + 16 * c16);
      *reinterpret_cast<u32x4*>(dst) = (u32x4){w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(dst + 4) = (u32x4){w[4], w[5], w[6], w[7]};
    }
#pragma unroll
    for (int q = 0; q < SP; ++q) {
      const int piece = tid + q * NT;
      if (piece >= kSidePieces) continue;
      const int row = piece / 9, part = piece % 9;
      if (part == 0) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const uint32_t word = side[q][g >> 1];
          scl_s[g * kBlk + row] = f16_bits_to_f32((g & 1) ? (word >> 16) : (word & 0xFFFFu));
        }
      } else {
        *reinterpret_cast<u32x4*>(rope_s + row * kRopeStride + 8 * (part - 1)) = side[q];
      }
    }
  }
};

// 4 bf16 of rows r0..r0+3 at column col0 + (lane % 16) (see the file comment):
// lane c of each 16-lane group supplies the address of row r0 + c/4, columns
// col0 + 4 (c % 4) .. +3, where r0 may differ between the lane groups.
__device__ inline bf16x4 read_tr(const uint16_t* lat_s, int r0, int col0, int lane) {
  const int c = lane & 15;
  const uint16_t* p = lat_s + (r0 + (c >> 2)) * kLatStride + col0 + 4 * (c & 3);
  const DSA_LDS bf16x4* a = (const DSA_LDS bf16x4*)(const DSA_LDS void*)p;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<DSA_LDS bf16x4*>(a));
}

// One workgroup: one query row, all H = NW*16 heads, one split of the row's selection.
template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnKArgs ka) {
  constexpr int NT = NW * 64;
  __shared__ __align__(16) uint16_t lat_s[kBlk * kLatStride];
  __shared__ __align__(16) uint16_t rope_s[kBlk * kRopeStride];
  __shared__ __align__(16) float scl_s[8 * kBlk];
  __shared__ int s_idx[kMaxSplitRows + kBlk];

  const StepArgs& a = ka.a;
  const int split = blockIdx.x, r = blockIdx.y, seq = blockIdx.z;
  const ScratchG s = scratch_of(a, seq);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int H = ka.H;
  const int h0 = wave * 16;
  const int64_t rb = ka.row_bytes;

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

  const int n_sel = s.sel_n[r];
  const int j_begin = split * ka.split_rows;
  if (j_begin >= n_sel) return;
  const int j_end = min(n_sel, j_begin + ka.split_rows);
  const int nrows = j_end - j_begin;

  // Compact-row index of every selected row of the split (the map: union index
  // of the selected position, from the per-position index the gather wrote).
  const auto sel = s.sel + (int64_t)r * ka.K;
  const auto map = s.map + (int64_t)r * ka.K;
  const int64_t U = s.info[kInfoUnion];
  for (int j = tid; j < ka.split_rows + kBlk; j += NT) {
    int idx = -1;
    if (j < nrows) {
      const int32_t p = sel[j_begin + j];
      idx = (p >= 0 && p < ka.max_positions) ? s.upos[p] : -1;
      if (idx >= U) idx = -1;                        // never index past the compact rows
      map[j_begin + j] = idx;
    }
    s_idx[j] = idx;
  }
  if (split == 0)
    for (int j = n_sel + tid; j < ka.K; j += NT) map[j] = -1;
  __syncthreads();

  RawBlock<NT> raw;
  raw.load(s.compact, s_idx, rb, tid);

  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;             // of head h0 + l16

  for (int jb = 0; jb < nrows; jb += kBlk) {
    __syncthreads();                                  // the previous block's LDS reads are done
    raw.store(lat_s, rope_s, scl_s, tid);
    if (jb + kBlk < nrows) raw.load(s.compact, s_idx + jb + kBlk, rb, tid);
    __syncthreads();

    // logits S^T[j][h]: lane holds rows 16 mt + 4 q4 + v of head h0 + l16
    float lg[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ks = 2 * g + kk;
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(lat_s + (16 * mt + l16) * kLatStride + 32 * ks + 8 * q4);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qa[ks], acc, 0, 0, 0);
        }
        const f32x4 sc = *reinterpret_cast<const f32x4*>(scl_s + g * kBlk + 16 * mt + 4 * q4);
#pragma unroll
        for (int v = 0; v < 4; ++v) sacc[v] += sc[v] * acc[v];
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(rope_s + (16 * mt + l16) * kRopeStride + 32 * kk + 8 * q4);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qa[16 + kk], sacc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = jb + 16 * mt + 4 * q4 + v;
        lg[mt][v] = (j < nrows && s_idx[j] >= 0) ? sacc[v] * ka.scale_log2 : -INFINITY;
      }
    }

    // online softmax of head h0 + l16 over the block (its 32 rows sit in the 4 lane groups)
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, lg[mt][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float p[2][4];
    float ps = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[mt][v] = none ? 0.f : exp2f(lg[mt][v] - m_new);
        ps += p[mt][v];
      }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // O rows are heads h0 + 4 q4 + v: their alphas come from lanes 4 q4 + v
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float av = __shfl(alpha, 4 * q4 + v);
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) o[nt][v] *= av;
    }

    // O[h][d] += sum_j (p[h][j] * scale_j[g]) * int8_j[d]; A fragment of head h0 + l16,
    // rows {4 q4 .. 4 q4 + 3, 16 + 4 q4 .. 16 + 4 q4 + 3} in that order
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const f32x4 sa = *reinterpret_cast<const f32x4*>(scl_s + g * kBlk + 4 * q4);
      const f32x4 sb = *reinterpret_cast<const f32x4*>(scl_s + g * kBlk + 16 + 4 * q4);
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
      bf16x8 pa_hi, pa_lo;
      __builtin_memcpy(&pa_hi, hi, 16);
      __builtin_memcpy(&pa_lo, lo, 16);
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int nt = 4 * g + t4;
        const bf16x4 b0 = read_tr(lat_s, 4 * q4, 16 * nt, lane);
        const bf16x4 b1 = read_tr(lat_s, 16 + 4 * q4, 16 * nt, lane);
        const bf16x8 bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, bv, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, bv, o[nt], 0, 0, 0);
      }
    }
  }

  // o[nt][v] = O[h0 + 4 q4 + v][16 nt + l16]; (m, l) of head h0 + l16 in every lane group
  if (ka.nsplit == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float lv = __shfl(l_run, 4 * q4 + v);
      const float inv = 1.f / lv;
      float* dst = ka.out + (((int64_t)seq * a.R + r) * H + h0 + 4 * q4 + v) * 512;
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) dst[nt * 16 + l16] = o[nt][v] * inv;
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = h0 + 4 * q4 + v;
      const int64_t base = ((int64_t)r * ka.ns_stride + split) * H + h;
      const auto dst = s.part_o + base * 512;
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) dst[nt * 16 + l16] = o[nt][v];
    }
    if (q4 == 0) {
      const int64_t base = ((int64_t)r * ka.ns_stride + split) * H + h0 + l16;
      s.part_ml[base * 2 + 0] = m_run;
      s.part_ml[base * 2 + 1] = l_run;
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
  const int64_t wg128 = (int64_t)a.R * a.n_seqs * ((g.top_k + 127) / 128);
  return wg128 >= 256 ? 128 : 64;
}

}  // namespace

hipError_t launch_attn(const Geometry& g, const StepArgs& a, const uint16_t* q_lat, const uint16_t* q_rope,
                       float* out, hipStream_t st) {
  const int split_rows = attn_split_rows(g, a);
  const int nsplit = (g.top_k + split_rows - 1) / split_rows;
  AttnKArgs ka{a, q_lat, q_rope, out, g.top_k, g.heads, split_rows, nsplit, g.nsplit_max, g.row_bytes,
               g.max_positions, g.softmax_scale * 1.4426950408889634f};
  dim3 grid((unsigned)nsplit, (unsigned)a.R, (unsigned)a.n_seqs);
  switch (g.heads) {
    case 16: return launch_k(attn_kernel<1>, grid, dim3(64), 0, st, ka);
    case 32: return launch_k(attn_kernel<2>, grid, dim3(128), 0, st, ka);
    case 64: return launch_k(attn_kernel<4>, grid, dim3(256), 0, st, ka);
    case 128: return launch_k(attn_kernel<8>, grid, dim3(512), 0, st, ka);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_merge(const Geometry& g, const StepArgs& a, float* out, hipStream_t st) {
  const int split_rows = attn_split_rows(g, a);
  if ((g.top_k + split_rows - 1) / split_rows == 1) return hipSuccess;
  MergeKArgs ka{a, out, g.heads, split_rows, g.nsplit_max};
  return launch_k(attn_merge_kernel, dim3((unsigned)g.heads, (unsigned)a.R, (unsigned)a.n_seqs), dim3(128), 0, st,
                  ka);
}

}  // namespace dsa
