"""Pins for the oracle's absorbed-MLA attention over the selected rows."""
import json
import math
import os

import numpy as np
import pytest
import torch

import dsa_synth as S
from tests.oracle_util import unit, valid_rows

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dequant_row.json")))


def dequant_numpy(rows):
    """Independent decoding: numpy's own float16 and a bit-shift for bf16."""
    lat = rows[:, :512].view(np.int8).astype(np.float64)
    sc = rows[:, 512:528].copy().view("<f2").astype(np.float64)          # [n][8]
    c = lat * np.repeat(sc, 64, axis=1)
    rope = S.bf16_value(rows[:, 528:656].copy().view("<u2"))
    return c, rope


def _run(rows, keys_val, q_idx, w, q_lat, q_rope, K, R=1, scale=None, heads=None):
    n = rows.shape[0]
    D = keys_val.shape[1]
    H = q_lat.shape[1]
    u = unit(max_positions=n, index_heads=q_idx.shape[1], index_dim=D, heads=H, top_k=K,
             hot_slots=max(4, K), max_query_rows=R, softmax_scale=scale)
    u.append(S.bf16_bits(keys_val[:n - R]), rows[:n - R])
    u.flush()
    u.warm()
    u.append(S.bf16_bits(keys_val[n - R:]), rows[n - R:])
    out = u.decode_step(S.bf16_bits(q_idx), np.asarray(w, np.float32), q_lat, q_rope)
    return u, out


def test_dense_case_matches_sdpa_float64():
    # K >= visible rows: the sparse step is dense softmax attention over every position,
    # which torch's scaled_dot_product_attention computes (float64, CPU)
    g = np.random.default_rng(0)
    T, H = 40, 4
    rows = valid_rows(T, 1)
    keys = g.integers(-3, 4, (T, 8)).astype(float)
    ql = S.bf16_bits(0.5 * g.standard_normal((1, H, 512)))
    qr = S.bf16_bits(0.5 * g.standard_normal((1, H, 64)))
    u, out = _run(rows, keys, g.integers(-3, 4, (1, 1, 8)).astype(float), [[1.0]], ql, qr, K=64)
    c, rope = dequant_numpy(rows)
    q = torch.tensor(np.concatenate([S.bf16_value(ql), S.bf16_value(qr)], -1))       # [1][H][576]
    k = torch.tensor(np.concatenate([c, rope], -1))[None, None].expand(1, H, T, 576)
    v = torch.tensor(c)[None, None].expand(1, H, T, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[:, :, None, :], k, v, scale=1.0 / 24.0)[:, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_zero_query_is_the_mean_of_the_selected_rows():
    g = np.random.default_rng(1)
    T, K = 60, 16
    rows = valid_rows(T, 2)
    keys = g.integers(-3, 4, (T, 8)).astype(float)
    u, out = _run(rows, keys, g.integers(-3, 4, (1, 1, 8)).astype(float), [[2.0]],
                  np.zeros((1, 2, 512), np.uint16), np.zeros((1, 2, 64), np.uint16), K=K)
    sel, cnt = u.selection()
    c, _ = dequant_numpy(rows)
    mean = c[sel[0, :K]].mean(axis=0)
    assert np.allclose(out[0, 0], mean, rtol=1e-6, atol=1e-9)
    assert np.allclose(out[0, 1], mean, rtol=1e-6, atol=1e-9)


def test_single_selected_row_is_its_dequantised_latent():
    T = 8
    rows = valid_rows(T, 3)
    row = np.zeros(656, np.uint8)
    row[:512] = np.arange(512) % 256
    for g_, b in enumerate(GOLD["scale_bits"]):
        v = int(b, 16)
        row[512 + 2 * g_] = v & 0xFF
        row[513 + 2 * g_] = v >> 8
    rows[5] = row
    keys = np.zeros((T, 8))
    keys[5, 0] = 1.0
    q_idx = np.zeros((1, 1, 8))
    q_idx[0, 0, 0] = 1.0
    u, out = _run(rows, keys, q_idx, [[1.0]], S.bf16_bits(np.ones((1, 1, 512))),
                  np.zeros((1, 1, 64), np.uint16), K=1)
    assert u.selection()[0][0, 0] == 5
    lat = (np.arange(512) % 256).astype(np.uint8).view(np.int8).astype(np.float64)
    want = lat * np.repeat(np.array(GOLD["scale_values"]), 64)
    assert np.array_equal(out[0, 0], want.astype(np.float32))


def test_two_rows_rope_only_closed_form():
    # q_lat = 0, q_rope = a*e_0: the logits differ by a*(x1-x2)/24, so the first row's
    # weight is the logistic function of that difference
    T = 10
    rows = valid_rows(T, 4)
    x = [1.0, -2.0]
    for j, xv in zip((2, 6), x):
        rows[j, 528:656] = 0
        b = int(S.bf16_bits(np.array([xv]))[0])
        rows[j, 528], rows[j, 529] = b & 0xFF, b >> 8
    keys = np.zeros((T, 8))
    keys[[2, 6], 0] = 1.0
    q_idx = np.zeros((1, 1, 8))
    q_idx[0, 0, 0] = 1.0
    a = 12.0
    qr = np.zeros((1, 1, 64))
    qr[0, 0, 0] = a
    u, out = _run(rows, keys, q_idx, [[1.0]], np.zeros((1, 1, 512), np.uint16), S.bf16_bits(qr), K=2)
    sel, _ = u.selection()
    assert sel[0].tolist() == [2, 6]
    p = 1.0 / (1.0 + math.exp(-a * (x[0] - x[1]) / 24.0))
    c, _ = dequant_numpy(rows)
    want = p * c[2] + (1 - p) * c[6]
    assert np.allclose(out[0, 0], want, rtol=1e-6, atol=1e-9)


def test_softmax_scale_zero_gives_uniform_weights():
    g = np.random.default_rng(6)
    T, K = 30, 8
    rows = valid_rows(T, 7)
    keys = g.integers(-3, 4, (T, 8)).astype(float)
    ql = S.bf16_bits(3.0 * g.standard_normal((1, 1, 512)))
    u, out = _run(rows, keys, g.integers(-3, 4, (1, 1, 8)).astype(float), [[1.0]], ql,
                  np.zeros((1, 1, 64), np.uint16), K=K, scale=0.0)
    sel, _ = u.selection()
    c, _ = dequant_numpy(rows)
    assert np.allclose(out[0, 0], c[sel[0]].mean(0), rtol=1e-6, atol=1e-9)
