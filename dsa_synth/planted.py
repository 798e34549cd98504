"""Planted index keys and queries for the 78-layer replacement/visibility stress workload.

Goal: every query row's Top-2048 holds 2,028 positions that sit in the warm hot
cache and 20 positions that do not (about 1% misses per row), and pairs of rows
select the same missing positions, so one step carries duplicate misses.

Recipe (per layer, all values inside the usual ranges: keys/queries in
{-8, 0, 8}, head weights in {0, 1, 4}):
  - hot set: 2,028 positions drawn from the cached range [T-S, T); key has
    k[0] = k[127] = 8;
  - cold range [0, T-S) is coded in pairs: code (a, b), 1 <= a < b <= 126, is
    carried by two positions whose key has k[a] = k[b] = k[127] = 8; positions
    left over, cached non-hot positions and appended rows have only k[127] = 8;
  - query head 0: w = 4, q[0] = 8  -> hot keys score 4*64 = 256;
  - query heads 1..10: w = 1, q[a] = q[b] = 8, q[127] = -8 for ten fresh codes
    -> each exactly matching key scores 64; a partial or no match is <= 0;
  - heads 11.. : q = 0, w = 0.
Rows 2i and 2i+1 use the same ten codes, so a step has 40 fresh codes
(80 missing positions).  Codes are never reused: 128 steps x 40 = 5,120 of the
7,875 codes.
"""
from __future__ import annotations

import numpy as np

from . import HISTORY_CHUNK, Workload, _rng, bf16_bits, make_rows

HOT = 2028
CODES_PER_ROW = 10
_T_PLAN = 11
_T_HIST_ROWS = 2
_T_NEW_ROWS = 4


def _codes(max_b: int = 126):
    return [(a, b) for a in range(1, max_b + 1) for b in range(a + 1, max_b + 1)]


_CODE_LIST = _codes()


def _plan(w: Workload, layer: int):
    """(hot positions, code -> 2 cold positions) for one layer."""
    g = _rng(w, layer, 0, -1, _T_PLAN)
    S, T = w.hot_slots, w.history
    cached0 = max(0, T - S)
    hot = np.sort(g.choice(np.arange(cached0, T), size=HOT, replace=False))
    cold = g.permutation(cached0)
    n_codes = min(len(_CODE_LIST), cached0 // 2)
    code_pos = cold[:2 * n_codes].reshape(n_codes, 2)
    return hot, code_pos


_plan_cache: dict = {}


def plan(w: Workload, layer: int):
    key = (w.wid, w.history, w.hot_slots, layer)
    if key not in _plan_cache:
        if len(_plan_cache) > 8:
            _plan_cache.clear()
        _plan_cache[key] = _plan(w, layer)
    return _plan_cache[key]


def _keys_for(w: Workload, layer: int, first: int, n: int) -> np.ndarray:
    hot, code_pos = plan(w, layer)
    k = np.zeros((n, w.index_dim), dtype=np.float64)
    k[:, 127] = 8.0
    pos = np.arange(first, first + n)
    is_hot = np.isin(pos, hot)
    k[is_hot, 0] = 8.0
    flat = code_pos.reshape(-1)
    code_of = np.full(max(w.history, 1), -1, dtype=np.int64)
    code_of[flat] = np.repeat(np.arange(code_pos.shape[0]), 2)
    in_hist = pos < w.history
    cid = np.where(in_hist, code_of[np.minimum(pos, w.history - 1)], -1)
    for i in np.nonzero(cid >= 0)[0]:
        a, b = _CODE_LIST[cid[i]]
        k[i, a] = 8.0
        k[i, b] = 8.0
    return bf16_bits(k)


def history(w: Workload, layer: int, seq: int, first: int = 0, n: int | None = None):
    if n is None:
        n = w.history - first
    keys = _keys_for(w, layer, first, n)
    rows = np.empty((n, w.row_bytes), dtype=np.uint8)
    pos = first
    while pos < first + n:
        c = pos // HISTORY_CHUNK
        c0 = c * HISTORY_CHUNK
        clen = min(HISTORY_CHUNK, w.history - c0)
        take = min(first + n, c0 + clen) - pos
        cr = make_rows(_rng(w, layer, seq, -1, _T_HIST_ROWS, c), clen, w)
        rows[pos - first:pos - first + take] = cr[pos - c0:pos - c0 + take]
        pos += take
    return keys, rows


def step_rows(w: Workload, layer: int, seq: int, step: int):
    k = np.zeros((w.rows_per_step, w.index_dim), dtype=np.float64)
    k[:, 127] = 8.0
    rows = make_rows(_rng(w, layer, seq, step, _T_NEW_ROWS), w.rows_per_step, w)
    return bf16_bits(k), rows


def max_steps(w: Workload) -> int:
    """Steps whose queries get fresh codes (codes are never reused)."""
    return len(_CODE_LIST) // ((w.rows_per_step + 1) // 2 * CODES_PER_ROW)


def index_queries(w: Workload, layer: int, seq: int, step: int):
    R, HI = w.rows_per_step, w.index_heads
    q = np.zeros((R, HI, w.index_dim), dtype=np.float64)
    wt = np.zeros((R, HI), dtype=np.float32)
    pairs = (R + 1) // 2
    for i in range(R):
        q[i, 0, 0] = 8.0
        wt[i, 0] = 4.0
        for h in range(1, 1 + CODES_PER_ROW):
            code = step * pairs * CODES_PER_ROW + (i // 2) * CODES_PER_ROW + (h - 1)
            if code >= len(_CODE_LIST):
                raise ValueError(f"the planted workload has fresh codes for {max_steps(w)} steps; step {step} asked")
            a, b = _CODE_LIST[code]
            q[i, h, a] = 8.0
            q[i, h, b] = 8.0
            q[i, h, 127] = -8.0
            wt[i, h] = 1.0
    return bf16_bits(q), wt


def expected_overlap(w: Workload, layer: int, step: int):
    """Per-row planted (hot positions, missing positions) for checks."""
    hot, code_pos = plan(w, layer)
    R = w.rows_per_step
    pairs = (R + 1) // 2
    out = []
    for i in range(R):
        codes = [step * pairs * CODES_PER_ROW + (i // 2) * CODES_PER_ROW + j for j in range(CODES_PER_ROW)]
        out.append((hot, np.sort(code_pos[codes].reshape(-1))))
    return out
