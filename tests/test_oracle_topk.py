"""Pins for the oracle's exact Top-K: brute force over tiny inputs, ties, and maximality."""
import numpy as np
import pytest

import dsa_synth as S
from tests.oracle_util import random_rows, unit


def _scores_and_selection(keys, q, w, K, R=1):
    n = keys.shape[0]
    D = keys.shape[1]
    HI = q.shape[1]
    u = unit(max_positions=n, index_heads=HI, index_dim=D, top_k=K, hot_slots=8, max_query_rows=R)
    rows = random_rows(n, 3)
    u.append(S.bf16_bits(keys[:n - R]), rows[:n - R])
    u.flush()
    u.append(S.bf16_bits(keys[n - R:]), rows[n - R:])
    u.decode_step(S.bf16_bits(q), np.asarray(w, np.float32), np.zeros((R, 1, 512), np.uint16),
                  np.zeros((R, 1, 64), np.uint16))
    return u.scores(), u.selection()


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    # keys from {-1,0,1} make many equal scores, so the tie rule decides often
    g = np.random.default_rng(seed)
    T, D, HI, K, R = 37, 8, 2, 9, 2
    keys = g.integers(-1, 2, (T, D)).astype(float)
    q = g.integers(-1, 2, (R, HI, D)).astype(float)
    w = g.integers(0, 3, (R, HI)).astype(float)
    s, (sel, cnt) = _scores_and_selection(keys, q, w, K, R)
    for i in range(R):
        n_vis = T - R + i + 1
        order = sorted(range(n_vis), key=lambda t: (-float(s[i, t]), t))   # library sort
        assert sel[i, :cnt[i]].tolist() == sorted(order[:K])
        assert cnt[i] == min(K, n_vis)


def test_maximality_and_tie_rule_invariants():
    g = np.random.default_rng(11)
    T, D, HI, K = 500, 16, 2, 64
    keys = g.integers(-2, 3, (T, D)).astype(float)
    q = g.integers(-2, 3, (1, HI, D)).astype(float)
    w = g.integers(0, 3, (1, HI)).astype(float)
    s, (sel, cnt) = _scores_and_selection(keys, q, w, K)
    s = s[0]
    chosen = np.zeros(T, bool)
    chosen[sel[0, :cnt[0]]] = True
    assert chosen.sum() == K
    assert np.all(np.diff(sel[0, :K]) > 0)                      # ascending, distinct
    lo = s[chosen].min()
    assert np.all(s[~chosen] <= lo)                              # nothing unselected beats the cutoff
    # at the cutoff score, every selected position precedes every unselected one
    tie_sel = np.nonzero(chosen & (s == lo))[0]
    tie_uns = np.nonzero(~chosen & (s == lo))[0]
    if len(tie_sel) and len(tie_uns):
        assert tie_sel.max() < tie_uns.min()


def test_all_equal_scores_select_first_k():
    T, D = 100, 4
    keys = np.ones((T, D))
    q = np.ones((1, 1, D))
    s, (sel, cnt) = _scores_and_selection(keys, q, [[1.0]], 10)
    assert np.all(s[0] == 4.0)
    assert sel[0, :10].tolist() == list(range(10))


def test_fewer_visible_than_k_selects_all():
    T, D = 6, 4
    g = np.random.default_rng(5)
    s, (sel, cnt) = _scores_and_selection(g.integers(-3, 4, (T, D)).astype(float),
                                          g.integers(-3, 4, (1, 1, D)).astype(float), [[1.0]], 10)
    assert cnt[0] == T and sel[0, :T].tolist() == list(range(T))
    assert np.all(sel[0, T:] == -1)
