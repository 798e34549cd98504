"""Checks on the seeded input generator (determinism, ranges, rounding, planted overlap)."""
import numpy as np
import pytest

import dsa_synth as S
from dsa_synth import planted


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1.0)
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.0, 0.25, 8.0, -8.0])
    assert S.bf16_bits(vals).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x3E80, 0x4100, 0xC100]


def test_fp16_bits():
    assert S.f16_bits(np.array([1.0, 0.5, -1.0, 65504.0])).tolist() == [0x3C00, 0x3800, 0xBC00, 0x7BFF]


def test_deterministic_and_sliceable():
    w = S.WORKLOADS["tiny"]
    k1, r1 = S.history(w, 0, 0)
    k2, r2 = S.history(w, 0, 0, 1000, 50)
    assert np.array_equal(k1[1000:1050], k2) and np.array_equal(r1[1000:1050], r2)
    assert np.array_equal(S.step_queries(w, 0, 0, 3)[0], S.step_queries(w, 0, 0, 3)[0])
    assert not np.array_equal(S.step_queries(w, 0, 0, 3)[0], S.step_queries(w, 0, 0, 2)[0])


def test_value_ranges():
    w = S.WORKLOADS["tiny"]
    keys, rows = S.history(w, 0, 0)
    kv = S.bf16_value(keys)
    assert kv.min() >= -8 and kv.max() <= 8 and np.all(kv == np.round(kv))
    lat = rows[:, :512].view(np.int8)
    assert lat.min() >= -127 and lat.max() <= 127
    sc = rows[:, 512:528].copy().view("<f2").astype(np.float64)
    assert sc.min() >= 0.0019 and sc.max() <= 0.0201
    iq, iw, ql, qr = S.step_queries(w, 0, 0, 0)
    assert iw.min() >= 0 and iw.max() <= 4 and np.all(iw == np.round(iw))
    assert abs(S.bf16_value(ql).std() - 0.05) < 0.005


def test_shapes_of_every_workload():
    for name, w in S.WORKLOADS.items():
        assert w.row_bytes == 656
        iq, iw, ql, qr = S.step_queries(w, 0, 0, 0)
        R = w.rows_per_step
        assert iq.shape == (R, w.index_heads, 128) and iw.shape == (R, w.index_heads)
        assert ql.shape == (R, w.heads, 512) and qr.shape == (R, w.heads, 64)


def test_planted_overlap_selects_2028_hot_and_20_cold():
    # the planted recipe makes Top-2048 exact: hot keys score 256, code matches 64, the rest 0
    w = S.WORKLOADS["stress_78_layers"]
    keys, _ = S.history(w, 5, 0)
    kv = S.bf16_value(keys)
    iq, iw, _, _ = S.step_queries(w, 5, 0, 7)
    q = S.bf16_value(iq)
    for i in range(w.rows_per_step):
        s = np.maximum(kv @ q[i].T, 0.0) @ iw[i].astype(np.float64)
        hot, cold = planted.expected_overlap(w, 5, 7)[i]
        top = np.argsort(-s, kind="stable")[:2048]
        assert set(top.tolist()) == set(hot.tolist()) | set(cold.tolist())
        assert np.all(hot >= w.history - w.hot_slots) and np.all(cold < w.history - w.hot_slots)
        assert len(cold) == 20 and len(hot) == 2028


def test_planted_queries_stop_at_their_fresh_codes():
    # every step's queries use fresh codes; past the last one the generator refuses
    w = S.WORKLOADS["stress_78_layers"]
    last = planted.max_steps(w) - 1
    iq, iw = planted.index_queries(w, 0, 0, last)
    assert iq.shape[0] == w.rows_per_step and np.all(iw[:, 0] == 4.0)
    with pytest.raises(ValueError):
        planted.index_queries(w, 0, 0, last + 1)
