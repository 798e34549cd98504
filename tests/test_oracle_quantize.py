"""Pins for the quantise-on-append oracle (bf16 latent + RoPE -> packed Q8G64 row).

The pages fix the row layout (page "From 1M total to 15+ streams x 1M", section
"Starting point": int8 latent, one fp16 scale per 64 values, bf16 RoPE, 656 B)
and the symmetric dequantisation value = scale * code; the scale rule
(max |x| / 127 in float32, rounded to binary16) and round-half-even codes are
this implementation's reading.  The pins below hold for that reading whatever
the arithmetic order: exact recovery on power-of-two grids, ties to even, the
half-step error bound, the degenerate groups.
"""
import numpy as np
import pytest

import dsa_synth as S
from oracle.quantize import LATENT, GROUP, ROPE, ROW_BYTES, quantize_rows

G = LATENT // GROUP


def _split(rows):
    codes = rows[:, :LATENT].view(np.int8).reshape(-1, G, GROUP).astype(np.int64)
    scales = rows[:, LATENT:LATENT + 2 * G].copy().view("<f2").astype(np.float64)
    rope = rows[:, LATENT + 2 * G:].copy().view("<u2")
    return codes, scales, rope


def _rope(g, n):
    return S.bf16_bits(g.standard_normal((n, ROPE)))


def test_row_size_matches_the_page():
    assert ROW_BYTES == 656


@pytest.mark.parametrize("e", [-14, -3, 0, 7])
def test_power_of_two_grid_is_recovered_exactly(e):
    # values j * 2^e with one element at +-127 * 2^e: the scale is exactly 2^e and
    # every code is j; the RoPE bits pass through unchanged
    g = np.random.default_rng(100 + e)
    n = 6
    j = g.integers(-127, 128, size=(n, G, GROUP))
    j[:, :, 0] = np.where(g.integers(0, 2, size=(n, G)) == 1, 127, -127)
    lat = S.bf16_bits(j.astype(np.float64) * 2.0 ** e).reshape(n, LATENT)
    rope = _rope(g, n)
    codes, scales, rope_out = _split(quantize_rows(lat, rope))
    assert np.all(scales == 2.0 ** e)
    assert np.array_equal(codes, j)
    assert np.array_equal(rope_out, rope)


def test_halfway_values_round_to_even():
    s = 0.25
    j = np.arange(-127, 127)                       # (j + 0.5) * s for every half step
    vals = np.zeros((4, G, GROUP))
    flat = np.concatenate([(j + 0.5) * s, np.zeros(4 * G * (GROUP - 1) - len(j))])
    vals[:, :, 1:] = flat.reshape(4, G, GROUP - 1)
    vals[:, :, 0] = 127 * s
    lat = S.bf16_bits(vals).reshape(4, LATENT)
    codes, scales, _ = _split(quantize_rows(lat, np.zeros((4, ROPE), np.uint16)))
    assert np.all(scales == s)
    got = codes[:, :, 1:].reshape(-1)[:len(j)]
    lo, hi = j, j + 1
    expect = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("lo,hi", [(-4, 12), (-16, -8)])
def test_half_step_error_bound_and_scale_rule_on_random_rows(lo, hi):
    # groups of widely different magnitudes, so a scale applied to the wrong group
    # or a wrong divisor breaks the bound; the second range gives subnormal scales
    g = np.random.default_rng(7 - lo)
    n = 300
    mag = 2.0 ** g.integers(lo, hi, size=(n, G, 1))
    x = S.bf16_value(S.bf16_bits(g.standard_normal((n, G, GROUP)) * mag))
    lat = S.bf16_bits(x).reshape(n, LATENT)
    codes, scales, _ = _split(quantize_rows(lat, _rope(g, n)))
    a = np.max(np.abs(x), axis=2)
    # the scale is the binary16 value nearest a / 127: half a unit in the last place,
    # relative 2^-11 in the normal range, absolute 2^-25 below it
    half_ulp = np.maximum(2.0 ** -11 * (a / 127), 2.0 ** -25)
    assert np.all(np.abs(scales - a / 127) <= half_ulp)
    live = (scales > 0)[:, :, None].repeat(GROUP, 2)
    s_el = scales[:, :, None].repeat(GROUP, 2)
    err = np.abs(x - codes * scales[:, :, None])
    unclamped = live & (np.abs(x) <= 127 * s_el)
    assert np.all(err[unclamped] <= s_el[unclamped] / 2)
    # a clamped element takes the end code of its sign
    clamped = live & ~unclamped
    assert np.all(codes[clamped] == np.sign(x[clamped]) * 127)
    # with a normal (not subnormal) scale the largest element of a group uses
    # (almost) the full code range
    assert np.all(np.max(np.abs(codes), axis=2)[scales >= 2.0 ** -14] >= 126)
    assert np.all(codes[~live] == 0)


def test_degenerate_groups():
    lat = np.zeros((1, G, GROUP))
    lat[0, 1, 5] = 1e-7            # a / 127 underflows binary16 to zero: every code 0
    lat[0, 2, :] = 1e10            # a / 127 overflows binary16: largest finite scale, codes clamp
    lat[0, 2, 3] = -1e10
    lat[0, 3, 7] = -3.0            # a lone value maps to -127
    codes, scales, _ = _split(quantize_rows(S.bf16_bits(lat).reshape(1, LATENT), np.zeros((1, ROPE), np.uint16)))
    assert scales[0, 0] == 0 and np.all(codes[0, 0] == 0)
    assert scales[0, 1] == 0 and np.all(codes[0, 1] == 0)
    assert scales[0, 2] == 65504.0 and np.all(np.abs(codes[0, 2]) == 127) and codes[0, 2, 3] == -127
    assert codes[0, 3, 7] == -127 and np.count_nonzero(codes[0, 3]) == 1
    assert abs(scales[0, 3] - 3.0 / 127) <= 2.0 ** -11 * 3.0 / 127
