// k_score.hip -- DSA indexer score over every visible history position.
//
//   score[i][t] = sum_h w[i][h] * max(0, q[i][h] . key[t])
//
// The indexer scans the whole history so that only the top positions reach
// attention (page "From 1M total to 15+ streams x 1M: the capacity breakthrough
// of GLM-5.3 KV cache offload", section "Starting point").  Index keys stay in
// HBM for every position.
//
// gfx950 mapping.  The (query row, head) pairs of a sequence form the M
// dimension (R*H_I rows, padded to 32), positions form N, the 128 key dims K.
// One v_mfma_f32_32x32x16_bf16 tile covers 32 (row, head) pairs x 32
// positions x 16 dims.  Q lives in LDS (row stride padded to 272 B), keys are
// streamed from HBM straight into B fragments: the key store keeps each
// 32-position tile in operand order, so each of a tile's 8 loads reads 1 KiB
// contiguous (fully coalesced) and lane (n, half) receives 16 bytes of key
// t0+n; every byte of a key is read exactly once per wave.  The K index is
// permuted (half 0 takes dims 0..63, half 1 dims 64..127, 8 per k-step); both
// operands use the same permutation, so the dot products are unchanged.
// The fp32 accumulator is exact for integer-valued bf16 inputs (|q.k| <= 2^13).
// After the tile, each lane applies ReLU and the head weight to its 16
// accumulator rows and the head sum is finished with one cross-half shuffle.
// While the scores are in registers, the workgroup also counts the first
// radix digit (top 11 bits of the order-preserving key) of every visible score
// per query row, in packed 16-bit LDS counters, and adds them to the row's
// global histogram -- the first pass of the exact Top-K.
//
// In an append-and-decode step the launch also appends the step's rows (the
// new rows enter the history before it is scored: page as above, section
// "Decision 3", the recent ring): workgroups past the scoring ones write the
// new keys into the key store and the new rows into the ring or the row store,
// and the scoring workgroups read the new positions' keys from the caller's
// buffer instead of the key store.
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kQStride = 136;           // bf16 per Q row in LDS (128 + 8 pad)
constexpr int kMaxQRows = 256;          // R * H_I

struct ScoreKArgs {
  StepArgs a;
  const uint16_t* q;                    // [n_seqs][R][HI][128]
  const float* w;                       // [n_seqs][R][HI]
  int64_t p_pad;
  int subs_per_wave;                    // 32-position sub-tiles per wave
  int r_max;
  // an append-and-decode step (a.add rows per sequence); null otherwise
  const uint16_t* app_keys;             // [n_seqs][add][128] bf16
  const uint8_t* app_rows;              // [n_seqs][add][row_bytes]
  int score_blocks;                     // workgroups per sequence that score; the rest append
  int row_bytes, ring_cap, mode;
};

__device__ inline float canon0(float s) { return s == 0.0f ? 0.0f : s; }

// The B fragments of 32-position tile `tile` (load k gives lane (n, half) dims
// 64 half + 8 k .. +7 of key tile * 32 + n): from the key store, which holds
// them in operand order, except the positions [Lo, L) the step appends, whose
// keys come from the caller's buffer (row-major, 16 pieces a key).
__device__ inline void load_tile(const DSA_GLOBAL bf16x8* keys16, int64_t tile, int lane, const bf16x8* app16,
                                 int64_t Lo, int64_t L, bf16x8* b) {
  if (app16 && tile * 32 + 32 > Lo) {                  // (uniform) the tile holds appended positions
    const int64_t t = tile * 32 + (lane & 31);
    const bool fresh = t >= Lo && t < L;
    const bf16x8* kp = fresh ? app16 + (t - Lo) * 16 + 8 * (lane >> 5) : (const bf16x8*)(keys16 + tile * 512 + lane);
    const int st = fresh ? 1 : 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) b[ks] = kp[ks * st];
  } else {
    const DSA_GLOBAL bf16x8* kp = keys16 + tile * 512 + lane;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) b[ks] = kp[ks * 64];
  }
}

// An append-and-decode step's appended rows, by the workgroups past the scoring
// ones: each key to its operand-order place in the key store, each row to the
// ring (offload; the spill that makes room ran before) or the HBM row store.
__device__ inline void append_block(const ScoreKArgs& ka, const UnitG& u, int seq, int block, int n_blocks) {
  const int64_t Lo = u.dyn[0], M = u.dyn[1];
  const int64_t n = ka.a.add, rb = ka.row_bytes;
  const int64_t key_pieces = n * 16, total = key_pieces + n * kCopyChunks16;
  const uint16_t* keys = ka.app_keys + (int64_t)seq * n * 128;
  const uint8_t* rows = ka.app_rows + (int64_t)seq * n * rb;
  for (int64_t t = (int64_t)block * blockDim.x + threadIdx.x; t < total; t += (int64_t)n_blocks * blockDim.x) {
    if (t < key_pieces) {
      const int64_t i = t / 16;
      const int c = (int)(t % 16);
      reinterpret_cast<DSA_GLOBAL u32x4*>(u.keys)[key_piece(Lo + i, c)] =
          reinterpret_cast<const u32x4*>(keys)[t];
    } else {
      const int64_t w = t - key_pieces, i = w / kCopyChunks16, c = w % kCopyChunks16;
      const int64_t p = Lo + i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(rows + i * rb + c * 16);
      const auto dst = (ka.mode == 1 || p < M) ? u.rows + p * rb : u.ring + (p % ka.ring_cap) * rb;
      *reinterpret_cast<DSA_GLOBAL u32x4*>(dst + c * 16) = v;
    }
  }
}

// max(0, x) for a finite x as one integer max on its bits: a negative float
// (-0 included) is a negative int32, and positive floats order as their bits.
__device__ inline float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ inline uint32_t first_digit(float f) {
  const uint32_t u = __float_as_uint(f);
  return ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) >> 21;
}

// Count the score in row r's packed LDS histogram (two 16-bit bins per word):
// one LDS atomic per lane; lanes that hit the same word are serialised by the
// LDS unit, which is cheaper than combining them in a loop first.
__device__ inline void count_digit(uint32_t* lh, int r, float score) {
  const uint32_t d = first_digit(score);
  atomicAdd(&lh[r * (kRadixBins / 2) + (d >> 1)], 1u << (16 * (d & 1)));
}

// NW waves share one staged Q.  Eight waves (launch_score picks them for a
// large Q or a short history): a 50,023-row history needs 196 workgroups, one
// tile per wave and every workgroup resident at once, even with 8 query rows,
// whose 69 KiB of Q leave room for one workgroup per CU.  Four waves (long
// histories, Q of at most 128 rows): three workgroups per CU (the LDS allows
// three), and the register budget this implies (at most 168 VGPRs) lets 12 waves
// per CU keep their next key tile in flight (with the compiler's unbounded
// choice, about 228, only 8 could, and the kernel waited on HBM latency).
// H_I = 4 keeps the default: it would spill under the bound.
// G row tiles are multiplied at a time (Q is zero padded to a whole number of
// groups): with G fixed at compile time the A fragments of the next k-step are
// read from LDS while this k-step's G products run, instead of one read and one
// wait per product.
template <int HI, int NW, int G>
__global__ __launch_bounds__(NW * 64, NW == 4 && HI >= 8 ? 3 : 1) void score_kernel(ScoreKArgs ka) {
  constexpr int kWaves = NW;
  constexpr int kThreads = NW * 64;
  constexpr int kMaxQPieces = kMaxQRows * 16 / kThreads;   // 16-byte Q pieces per thread
  extern __shared__ __align__(16) uint16_t sq[];   // [MTP*32][kQStride], weights, digit histograms
  const StepArgs& a = ka.a;
  const int seq = blockIdx.y;
  const UnitG u = unit_of(a, seq);
  if ((int)blockIdx.x >= ka.score_blocks) {            // (uniform) an appending workgroup
    append_block(ka, u, seq, (int)blockIdx.x - ka.score_blocks, (int)gridDim.x - ka.score_blocks);
    return;
  }
  const ScratchG s = scratch_of(a, seq);
  const int64_t L = step_L(u, a);                        // requested first; the key loads wait for it only
  const int R = a.R;
  const int M = R * HI;
  const int MT = (M + 31) / 32;
  const int MTP = (MT + G - 1) / G * G;                  // row tiles padded to whole groups
  float* sw = reinterpret_cast<float*>(sq + MTP * 32 * kQStride);
  uint32_t* lh = reinterpret_cast<uint32_t*>(sw + MTP * 32);   // [R][1024] packed pairs of bins

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int64_t first_sub = ((int64_t)blockIdx.x * kWaves + wave) * ka.subs_per_wave;

  // Q (zero padded to MTP*32 rows) and the head weights, staged in LDS below.
  // They are requested right behind L, and without a branch per load: a
  // padding piece reads row 0 and is zeroed where it is staged, so no load
  // waits for another (M <= 256: at most 16 per thread).
  const uint16_t* qg = ka.q + (int64_t)seq * M * 128;
  const int nq = MTP * 32 * 16;                          // 16-byte pieces of the padded Q
  bf16x8 qv[kMaxQPieces];
#pragma unroll
  for (int e = 0; e < kMaxQPieces; ++e) {
    const int c = threadIdx.x + e * kThreads;
    const int row = c >> 4, col = (c & 15) * 8;
    const bool real = c < nq && row < M;
    qv[e] = *reinterpret_cast<const bf16x8*>(qg + (real ? (int64_t)row * 128 + col : 0));
  }
  const float wv_raw = ka.w[(int64_t)seq * M + min((int)threadIdx.x, M - 1)];
  const int64_t Lo = L - a.add;                          // the appended positions [Lo, L)
  const bf16x8* app16 = ka.app_keys ? reinterpret_cast<const bf16x8*>(ka.app_keys) + (int64_t)seq * a.add * 16 : nullptr;
  // The first key tile's loads, behind the Q loads: loads complete in issue
  // order, so staging Q does not wait for the keys (HBM).
  // Positions past L read (unused) rows of the key store, so the loads need not
  // wait for L.
  // The key store is in operand order (key_piece): load k of a 32-position tile
  // is 1 KiB contiguous and gives lane (n, hf) its B fragment.
  const int64_t last_tile = ka.p_pad / 32 - 1;
  const DSA_GLOBAL bf16x8* keys16 = reinterpret_cast<const DSA_GLOBAL bf16x8*>(u.keys);
  bf16x8 b[8];
  load_tile(keys16, min(first_sub, last_tile), lane, app16, Lo, L, b);

  for (int w = threadIdx.x; w < R * (kRadixBins / 2); w += blockDim.x) lh[w] = 0;
#pragma unroll
  for (int e = 0; e < kMaxQPieces; ++e) {
    const int c = threadIdx.x + e * kThreads;
    const bf16x8 zero = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
    if (c < nq) *reinterpret_cast<bf16x8*>(sq + (c >> 4) * kQStride + (c & 15) * 8) = (c >> 4) < M ? qv[e] : zero;
  }
  if (threadIdx.x < MTP * 32) sw[threadIdx.x] = (int)threadIdx.x < M ? wv_raw : 0.0f;
  __syncthreads();

  const auto scores = s.scores;

  for (int si = 0; si < ka.subs_per_wave; ++si) {
    const int64_t t0 = (first_sub + si) * 32;
    if (t0 >= L) break;
    const int64_t t = t0 + n;
    // The next tile's keys are requested before this tile is computed (loads
    // complete in issue order, so this tile's wait does not include them).
    bf16x8 bn[8];
    if (si + 1 < ka.subs_per_wave) load_tile(keys16, min(first_sub + si + 1, last_tile), lane, app16, Lo, L, bn);
    // G row tiles at a time: independent accumulation chains, so the MFMA
    // pipeline is never waiting on one accumulator; the next k-step's A
    // fragments are read while this k-step's products run.
    for (int mt0 = 0; mt0 < MTP; mt0 += G) {
      f32x16 acc4[G];
      bf16x8 av[2][G];
#pragma unroll
      for (int i4 = 0; i4 < G; ++i4) {
        acc4[i4] = (f32x16){0};
        av[0][i4] = *reinterpret_cast<const bf16x8*>(sq + ((mt0 + i4) * 32 + n) * kQStride + 64 * hf);
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks + 1 < 8) {
#pragma unroll
          for (int i4 = 0; i4 < G; ++i4)
            av[(ks + 1) & 1][i4] =
                *reinterpret_cast<const bf16x8*>(sq + ((mt0 + i4) * 32 + n) * kQStride + 64 * hf + 8 * (ks + 1));
        }
#pragma unroll
        for (int i4 = 0; i4 < G; ++i4)
          acc4[i4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks & 1][i4], b[ks], acc4[i4], 0, 0, 0);
      }
#pragma unroll
      for (int i4 = 0; i4 < G; ++i4) {
        if (mt0 + i4 >= MT) continue;                  // (uniform) a padding tile
        const int mt = mt0 + i4;
        // acc[v] holds C[row = (v/4)*8 + hf*4 + v%4][col = n]
        float part[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            int m = mt * 32 + i * 8 + hf * 4 + j;
            p += sw[m] * relu(acc4[i4][i * 4 + j]);
          }
          part[i] = p;
        }
        if constexpr (HI == 32) {
          float sum = (part[0] + part[1]) + (part[2] + part[3]);
          sum += __shfl_xor(sum, 32);
          const int r = mt;
          if (hf == 0 && r < R && t < L - R + r + 1) {
            scores[(int64_t)r * ka.p_pad + t] = canon0(sum);
            count_digit(lh, r, canon0(sum));
          }
        } else if constexpr (HI == 16) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            float sum = part[2 * k2] + part[2 * k2 + 1];
            sum += __shfl_xor(sum, 32);
            const int r = mt * 2 + k2;
            if (hf == 0 && r < R && t < L - R + r + 1) {
              scores[(int64_t)r * ka.p_pad + t] = canon0(sum);
              count_digit(lh, r, canon0(sum));
            }
          }
        } else if constexpr (HI == 8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float sum = part[i] + __shfl_xor(part[i], 32);
            const int r = mt * 4 + i;
            if (hf == 0 && r < R && t < L - R + r + 1) {
              scores[(int64_t)r * ka.p_pad + t] = canon0(sum);
              count_digit(lh, r, canon0(sum));
            }
          }
        } else {  // HI == 4: rows of one query row sit in one lane half
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mt * 8 + 2 * i + hf;
            if (r < R && t < L - R + r + 1) {
              scores[(int64_t)r * ka.p_pad + t] = canon0(part[i]);
              count_digit(lh, r, canon0(part[i]));
            }
          }
        }
      }
    }
    if (si + 1 < ka.subs_per_wave) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) b[ks] = bn[ks];
    }
  }
  __syncthreads();
  // Four packed words per thread per round, all read before any is added.
  const int rep = blockIdx.x % kHistReps;
  const int n_words = R * (kRadixBins / 2);
  for (int w0 = threadIdx.x; w0 < n_words; w0 += 4 * kThreads) {
    uint32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = w0 + k * kThreads < n_words ? lh[w0 + k * kThreads] : 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!v[k]) continue;
      const int w = w0 + k * kThreads;
      const int r = w / (kRadixBins / 2), d = 2 * (w % (kRadixBins / 2));
      const auto gh = s.hist0 + ((int64_t)rep * ka.r_max + r) * kRadixBins + d;
      if (v[k] & 0xFFFFu) g_add(gh, v[k] & 0xFFFFu);
      if (v[k] >> 16) g_add(gh + 1, v[k] >> 16);
    }
  }
}

}  // namespace

#define DSA_SCORE_KERNELS(HI, NW) \
  (const void*)score_kernel<HI, NW, 1>, (const void*)score_kernel<HI, NW, 2>, (const void*)score_kernel<HI, NW, 4>

hipError_t prepare_score_kernels() {
  const int max_lds = kMaxQRows * kQStride * 2 + kMaxQRows * 4 + 8 * (kRadixBins / 2) * 4;
  const void* kernels[] = {DSA_SCORE_KERNELS(4, 4),  DSA_SCORE_KERNELS(8, 4),  DSA_SCORE_KERNELS(16, 4),
                           DSA_SCORE_KERNELS(32, 4), DSA_SCORE_KERNELS(4, 8),  DSA_SCORE_KERNELS(8, 8),
                           DSA_SCORE_KERNELS(16, 8), DSA_SCORE_KERNELS(32, 8)};
  for (const void* k : kernels) {
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
#undef DSA_SCORE_KERNELS

hipError_t launch_score(const Geometry& g, const StepArgs& a, const uint16_t* q, const float* w,
                        const uint16_t* app_keys, const uint8_t* app_rows, hipStream_t st) {
  ScoreKArgs ka;
  ka.a = a;
  ka.q = q;
  ka.w = w;
  ka.p_pad = g.p_pad;
  ka.r_max = g.r_max;
  ka.app_keys = a.add > 0 ? app_keys : nullptr;
  ka.app_rows = a.add > 0 ? app_rows : nullptr;
  ka.row_bytes = g.row_bytes;
  ka.ring_cap = g.ring_cap;
  ka.mode = g.mode;
  const int64_t subs = (a.l_max + 31) / 32;
  const int M = a.R * g.index_heads;
  // Eight waves for a large Q (more than 128 rows: one workgroup per CU) or a
  // short history (about one tile per wave over the chip); four otherwise.
  const bool wide = M > 128 || subs * a.n_seqs <= 8 * 256 * 2;
  const int nw = wide ? 8 : 4;
  // Enough waves (over all sequences) to cover the chip several times; longer
  // per-wave runs amortise the Q staging and keep the next tile's keys in flight.
  int spw = (int)((subs * a.n_seqs + nw * 256 * 4 - 1) / (nw * 256 * 4));
  if (spw < 1) spw = 1;
  if (spw > 8) spw = 8;
  ka.subs_per_wave = spw;
  const int64_t blocks = (subs + (int64_t)nw * spw - 1) / ((int64_t)nw * spw);
  ka.score_blocks = (int)blocks;
  const int64_t app_work = ka.app_keys ? (int64_t)a.add * (16 + kCopyChunks16) : 0;
  const int64_t app_blocks = (app_work + nw * 64 - 1) / (nw * 64);
  const int MT = (M + 31) / 32;
  const int G = MT >= 4 ? 4 : MT >= 2 ? 2 : 1;         // row tiles per group (Q padded to whole groups)
  const int MTP = (MT + G - 1) / G * G;
  const size_t lds = (size_t)MTP * 32 * kQStride * sizeof(uint16_t) + (size_t)MTP * 32 * sizeof(float) +
                     (size_t)a.R * (kRadixBins / 2) * sizeof(uint32_t);
  dim3 grid((unsigned)(blocks + app_blocks), (unsigned)a.n_seqs), block(nw * 64);
#define DSA_SCORE_G(HI, NW)                                                                  \
  (G == 4 ? launch_k(score_kernel<HI, NW, 4>, grid, block, lds, st, ka)                    \
          : G == 2 ? launch_k(score_kernel<HI, NW, 2>, grid, block, lds, st, ka)           \
                   : launch_k(score_kernel<HI, NW, 1>, grid, block, lds, st, ka))
#define DSA_SCORE_CASE(HI) \
  case HI:                 \
    return wide ? DSA_SCORE_G(HI, 8) : DSA_SCORE_G(HI, 4);
  switch (g.index_heads) {
    DSA_SCORE_CASE(4)
    DSA_SCORE_CASE(8)
    DSA_SCORE_CASE(16)
    DSA_SCORE_CASE(32)
    default: return hipErrorInvalidValue;
  }
#undef DSA_SCORE_CASE
#undef DSA_SCORE_G
}

}  // namespace dsa
