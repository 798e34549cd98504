"""Pins for the oracle's indexer score (closed forms, hand-worked values, identities)."""
import json
import os

import numpy as np

import dsa_synth as S
from tests.oracle_util import random_rows, unit


def _one_step(index_dim, index_heads, keys_val, q_val, w, history, R=1, top_k=4):
    """Run one decode step with history keys `keys_val` (float [T+R][D]); return oracle scores."""
    n = keys_val.shape[0]
    u = unit(max_positions=n, index_heads=index_heads, index_dim=index_dim, top_k=top_k,
             hot_slots=4, max_query_rows=R)
    rows = random_rows(n, 7)
    u.append(S.bf16_bits(keys_val[:history]), rows[:history])
    u.flush()
    u.append(S.bf16_bits(keys_val[history:]), rows[history:])
    q = S.bf16_bits(q_val).reshape(R, index_heads, index_dim)
    wq = np.asarray(w, np.float32).reshape(R, index_heads)
    u.decode_step(q, wq, np.zeros((R, 1, 512), np.uint16), np.zeros((R, 1, 64), np.uint16))
    return u


def test_handworked_example():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "scores_handworked.json")))
    keys = np.array(g["keys"], float)
    for K, want in ((1, g["top1"]), (2, g["top2"])):
        u = _one_step(g["index_dim"], 2, keys, np.array(g["q"], float), g["w"], history=2, top_k=K)
        assert u.scores()[0].tolist() == g["scores"]
        sel, cnt = u.selection()
        assert sel[0, :cnt[0]].tolist() == want


def test_closed_form_all_eights():
    # every key and query element = 8: q_h . k_t = 128 * 64 = 8192 for every head
    T, D, HI = 50, 128, 4
    w = [0.0, 1.0, 2.0, 4.0]
    u = _one_step(D, HI, np.full((T, D), 8.0), np.full((HI, D), 8.0), w, history=T - 1)
    assert np.all(u.scores()[0] == 8192.0 * sum(w))


def test_zero_weights_give_zero_scores_and_first_positions():
    T, D, HI = 40, 128, 3
    g = np.random.default_rng(1)
    u = _one_step(D, HI, g.integers(-8, 9, (T, D)).astype(float), g.integers(-8, 9, (HI, D)).astype(float),
                  [0.0] * HI, history=T - 1, top_k=5)
    assert np.all(u.scores()[0] == 0.0)
    sel, cnt = u.selection()
    assert sel[0, :cnt[0]].tolist() == [0, 1, 2, 3, 4]


def test_relu_identities_against_matmul():
    # s(q) - s(-q) = sum_h w_h (q_h . k_t)   and   s(q) + s(-q) = sum_h w_h |q_h . k_t|
    T, D, HI = 300, 128, 4
    g = np.random.default_rng(2)
    keys = g.integers(-8, 9, (T, D)).astype(float)
    q = g.integers(-8, 9, (HI, D)).astype(float)
    w = g.integers(0, 5, HI).astype(float)
    sp = _one_step(D, HI, keys, q, w, history=T - 1).scores()[0].astype(np.int64)
    sm = _one_step(D, HI, keys, -q, w, history=T - 1).scores()[0].astype(np.int64)
    dots = np.matmul(keys.astype(np.int64), q.astype(np.int64).T)      # [T][HI]
    wi = w.astype(np.int64)
    assert np.array_equal(sp - sm, dots @ wi)
    assert np.array_equal(sp + sm, np.abs(dots) @ wi)


def test_visibility_row_sees_only_up_to_its_own_position():
    # R=2 rows at positions T-2 and T-1; a dominant key sits at position T-1.
    T, D, HI = 30, 128, 1
    keys = np.zeros((T, D))
    keys[:, 0] = 1.0
    keys[T - 1, 0] = 8.0
    q = np.zeros((2, HI, D))
    q[:, 0, 0] = 1.0
    u = _one_step(D, HI, keys, q.reshape(2 * HI, D), [1.0, 1.0], history=T - 2, R=2, top_k=1)
    sel, cnt = u.selection()
    assert sel[1, 0] == T - 1          # row 1 sees its own row
    assert sel[0, 0] == 0              # row 0 does not: all visible scores tie at 1 -> lowest position
    s = u.scores()
    assert s[0, T - 1] == 0.0 and s[1, T - 1] == 8.0


def test_negative_zero_is_canonical():
    # negative weights times a zero ReLU give -0 in float64; the score must be +0
    T, D = 10, 128
    keys = np.zeros((T, D))
    q = np.ones((1, D))
    u = _one_step(D, 1, keys, q, [-1.0], history=T - 1)
    s = u.scores()[0]
    assert np.all(s == 0.0) and not np.any(np.signbit(s))
