"""CPU oracle for quantise-on-append: bf16 MLA latent + RoPE -> packed Q8G64 row.

TEST INFRASTRUCTURE, like the rest of this package: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import it.

Row layout (page "From 1M total to 15+ streams x 1M: the capacity breakthrough
of GLM-5.3 KV cache offload", section "Starting point": 512 B latent + 16 B scale
+ 128 B RoPE = 656 B; section "Decision 2", first problem: the owner quantises
a row once and then moves the packed 656 B, instead of each side re-quantising).
The pages fix the layout and the symmetric dequantisation value = scale * code,
but not how the scale is chosen or how codes are rounded.
The reading taken here, for each group of 64 latent values x (bf16, exact in
float32):

  a     = max |x| over the group                        (float32, exact)
  s32   = a / 127                                       (float32 division, IEEE RNE)
  s     = s32 rounded to binary16 (RNE); if that overflows, the largest finite
          binary16 (65504)
  code  = 0 for every element if s == 0, else
          clamp(round_half_even(x / s), -127, 127)      (x / s: float32 division)

The RoPE values are stored unchanged (bf16 bits).  Every step that decides an
integer is done in float32, the precision the GPU kernel computes in.
Parity unpinned by the pages (they give no rule); pinned instead by exact
recovery of codes on power-of-two grids, round-half-even ties, and the
|x - code * s| <= s / 2 bound of unclamped elements (tests/test_oracle_quantize.py).
"""
from __future__ import annotations

import numpy as np

LATENT, GROUP, ROPE = 512, 64, 64
ROW_BYTES = LATENT + 2 * (LATENT // GROUP) + 2 * ROPE
F16_MAX = np.float16(65504.0)


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def group_scales(latent_bits: np.ndarray) -> np.ndarray:
    """binary16 scale of every group: [n][LATENT // GROUP] float16."""
    x = _bf16_to_f32(latent_bits).reshape(-1, LATENT // GROUP, GROUP)
    a = np.max(np.abs(x), axis=2)                              # float32
    s32 = a / np.float32(127.0)                                # float32, correctly rounded
    with np.errstate(over="ignore"):
        s = s32.astype(np.float16)                             # RNE
    s[np.isinf(s)] = F16_MAX
    return s


def quantize_rows(latent_bits: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """latent bf16 bits [n][512], RoPE bf16 bits [n][64] -> packed rows uint8 [n][656]."""
    latent_bits = np.ascontiguousarray(latent_bits, dtype=np.uint16)
    rope_bits = np.ascontiguousarray(rope_bits, dtype=np.uint16)
    n = latent_bits.shape[0]
    assert latent_bits.shape == (n, LATENT) and rope_bits.shape == (n, ROPE)
    s = group_scales(latent_bits)                              # [n][8] float16
    x = _bf16_to_f32(latent_bits).reshape(n, LATENT // GROUP, GROUP)
    s32 = s.astype(np.float32)[:, :, None]
    codes = np.zeros(x.shape, dtype=np.int8)
    live = np.broadcast_to(s32 != 0, x.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = x / s32                                        # float32 division
    q = np.clip(np.rint(ratio[live]), -127, 127)               # rint: round half to even
    codes[live] = q.astype(np.int8)
    out = np.empty((n, ROW_BYTES), dtype=np.uint8)
    out[:, :LATENT] = codes.reshape(n, LATENT).view(np.uint8)
    out[:, LATENT:LATENT + 2 * (LATENT // GROUP)] = s.astype("<f2").view(np.uint8).reshape(n, -1)
    out[:, LATENT + 2 * (LATENT // GROUP):] = rope_bits.astype("<u2").view(np.uint8).reshape(n, -1)
    return out
