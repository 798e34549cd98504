// k_quant.hip -- quantise-on-append: bf16 MLA latent + RoPE -> packed Q8G64 row.
//
// Page "From 1M total to 15+ streams x 1M: the capacity breakthrough of
// GLM-5.3 KV cache offload" (zhuai.tech):
//   * section "Starting point": a row is 512 B of int8 latent, 16 B of scales
//     (one fp16 per 64 latent values) and 128 B of bf16 RoPE, 656 B in all;
//     the latent is symmetric, value = scale * code;
//   * section "Decision 2", first problem: the owner quantises a row once and
//     then moves the packed 656 B, rather than every holder re-quantising.
// The pages leave the scale rule and the rounding open.  Taken here, per group
// of 64 values x: scale = binary16(RNE) of max|x| / 127 computed in fp32 (the
// largest finite binary16 if that overflows); code = 0 if scale is 0, else
// clamp(rint(x / scale), -127, 127) with x / scale an IEEE fp32 division and
// rint rounding half to even.
//
// gfx950 design.  A wave works on one row at a time.  Lane l loads latent
// values [8l, 8l+8) (16 B; the wave reads the row's 1 KiB in one coalesced
// pass), so a group of 64 values is 8 adjacent lanes and its max is three xor-shuffles.  Each lane
// stores its 8 codes (8 B, the wave writes the 512 B contiguously); lane 0
// stores the 8 scales as one 16-byte piece; lanes 0-7 copy the 128 B of RoPE,
// lanes 0-15 the 256 B index key.  A wave takes 2 consecutive rows per pass and
// issues both rows' loads before quantising the first (measured: 4.5 TB/s over
// 2^20 rows, against 5.3 TB/s for a plain device copy of the same bytes; one
// row per pass or four gave 3.8-4.2 TB/s).  The kernel is bound by HBM (or
// host-link) bytes: 1,024 + 128 (+ 256 key) B read and 656 (+ 256 key) B
// written per row.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kLatent = 512, kGroup = 64, kRope = 64;
constexpr int kScaleOff = kLatent, kRopeOff = kLatent + 2 * (kLatent / kGroup);
static_assert(kRopeOff + 2 * kRope == 656, "Q8G64 row is 656 bytes");
constexpr int kIndexDim = 128;
constexpr int kRopePieces = 2 * kRope / 16, kKeyPieces = 2 * kIndexDim / 16;   // 16-byte pieces
constexpr int kQuantThreads = 256;                 // 4 waves per block
constexpr int kRowsPerWave = 2;

struct QuantKArgs {
  UnitDev u;                 // append target (out == nullptr)
  uint8_t* out;              // plain destination [n][656], or nullptr
  const uint16_t* latent;    // bf16 [n][512]
  const uint16_t* rope;      // bf16 [n][64]
  const uint16_t* keys;      // bf16 [n][index_dim] (append only)
  int64_t L, newM, n;
  int ring_cap, mode;
};

__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// One row: codes, scales and RoPE to dst; the index key to the key store.
__device__ inline void quantize_one(const QuantKArgs& ka, const UnitG& u, int lane, int64_t i, u32x4 raw,
                                    u32x4 rope_raw, u32x4 key_raw) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16_to_f32(raw[k] & 0xffffu);
    x[2 * k + 1] = bf16_to_f32(raw[k] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  _Float16 s16 = (_Float16)(amax / 127.0f);
  if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
  const float s = (float)s16;
  uint32_t packed[2] = {0u, 0u};
  if (s != 0.f) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float q = fminf(fmaxf(rintf(x[k] / s), -127.f), 127.f);
      packed[k >> 2] |= ((uint32_t)(int32_t)q & 0xffu) << (8 * (k & 3));
    }
  }
  const int64_t p = ka.L + i;
  DSA_GLOBAL uint8_t* dst;
  if (ka.out) dst = (DSA_GLOBAL uint8_t*)ka.out + i * 656;   // device memory (or pinned host, mapped)
  else if (ka.mode == 1 || p < ka.newM) dst = u.rows + p * 656;
  else dst = u.ring + (p % ka.ring_cap) * 656;
  reinterpret_cast<DSA_GLOBAL u32x2*>(dst)[lane] = (u32x2){packed[0], packed[1]};
  // scales of groups 0..7 live in lanes 0, 8, ..., 56
  const uint32_t sb = (uint32_t)__builtin_bit_cast(uint16_t, s16);
  uint32_t sc[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) sc[g] = __shfl(sb, 8 * g);
  if (lane == 0)
    *reinterpret_cast<DSA_GLOBAL u32x4*>(dst + kScaleOff) =
        (u32x4){sc[0] | sc[1] << 16, sc[2] | sc[3] << 16, sc[4] | sc[5] << 16, sc[6] | sc[7] << 16};
  if (lane < kRopePieces) reinterpret_cast<DSA_GLOBAL u32x4*>(dst + kRopeOff)[lane] = rope_raw;
  if (!ka.out && lane < kKeyPieces) reinterpret_cast<DSA_GLOBAL u32x4*>(u.keys)[key_piece(p, lane)] = key_raw;
}

// Each wave takes kRowsPerWave consecutive rows per pass and issues all their
// loads before it quantises the first, so that a wave keeps several rows' reads
// in flight.
__global__ __launch_bounds__(kQuantThreads) void quantize_rows_kernel(QuantKArgs ka) {
  const UnitG u = as_global(ka.u);
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * (kQuantThreads / 64) * kRowsPerWave;
  for (int64_t i0 = wave * kRowsPerWave; i0 < ka.n; i0 += stride) {
    u32x4 raw[kRowsPerWave], rope_raw[kRowsPerWave], key_raw[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int64_t i = i0 + r < ka.n ? i0 + r : ka.n - 1;     // the tail re-reads the last row, writes nothing
      raw[r] = reinterpret_cast<const u32x4*>(ka.latent + i * kLatent)[lane];
      rope_raw[r] = lane < kRopePieces ? reinterpret_cast<const u32x4*>(ka.rope + i * kRope)[lane] : (u32x4){};
      key_raw[r] = !ka.out && lane < kKeyPieces ? reinterpret_cast<const u32x4*>(ka.keys + i * kIndexDim)[lane]
                                                  : (u32x4){};
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
      if (i0 + r < ka.n) quantize_one(ka, u, lane, i0 + r, raw[r], rope_raw[r], key_raw[r]);
  }
  if (!ka.out && blockIdx.x == 0 && threadIdx.x == 0) {
    u.dyn[0] = ka.L + ka.n;
    u.dyn[1] = ka.mode == 1 ? ka.L + ka.n : ka.newM;
  }
}

unsigned quant_grid(int64_t n) {
  const int64_t rows_per_block = (kQuantThreads / 64) * kRowsPerWave;
  int64_t b = (n + rows_per_block - 1) / rows_per_block;
  if (b < 1) b = 1;
  if (b > (1 << 22)) b = 1 << 22;            // grid-stride beyond 2^25 rows
  return (unsigned)b;
}

}  // namespace

hipError_t launch_quantize(const Geometry& g, int64_t n, const uint16_t* latent, const uint16_t* rope, uint8_t* out,
                           hipStream_t st) {
  QuantKArgs ka{};
  ka.out = out;
  ka.latent = latent;
  ka.rope = rope;
  ka.n = n;
  ka.ring_cap = g.ring_cap;
  ka.mode = g.mode;
  return launch_k(quantize_rows_kernel, dim3(quant_grid(n)), dim3(kQuantThreads), 0, st, ka);
}

hipError_t launch_append_latent(const Geometry& g, const UnitDev& unit, int64_t L, int64_t M, int64_t newM, int64_t n,
                                const uint16_t* keys, const uint16_t* latent, const uint16_t* rope, hipStream_t st) {
  if (g.mode == 0 && newM > M && M < L) {
    hipError_t e = launch_flush(g, unit, M, newM < L ? newM : L, st);
    if (e != hipSuccess) return e;
  }
  if (g.index_dim != kIndexDim) return hipErrorInvalidValue;
  QuantKArgs ka{unit, nullptr, latent, rope, keys, L, newM, n, g.ring_cap, g.mode};
  return launch_k(quantize_rows_kernel, dim3(quant_grid(n)), dim3(kQuantThreads), 0, st, ka);
}

}  // namespace dsa
