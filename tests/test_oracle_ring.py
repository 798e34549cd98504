"""Pins for the recent ring, batched writeback, flush and warm start."""
import numpy as np
import pytest

import dsa_synth as S
from oracle import E_CAPACITY, E_STATE, MODE_RESIDENT, OracleError
from tests.oracle_util import random_rows, unit, valid_rows, zero_queries


def _keys(n, D=16, seed=0):
    return S.bf16_bits(np.random.default_rng(seed).integers(-3, 4, (n, D)).astype(float))


def test_writeback_fires_on_full_batches_only():
    # R=4 rows per step, 64-row batches: M moves by 64 exactly every 16 steps
    T, R, steps = 100, 4, 40
    u = unit(max_positions=T + R * steps, index_heads=1, index_dim=16, top_k=4, hot_slots=8,
             max_query_rows=R, ring_rows=64)
    rows = random_rows(T + R * steps, 1)
    keys = _keys(T + R * steps)
    u.append(keys[:T], rows[:T])
    u.flush()
    assert u.state()["M"] == T
    for s in range(steps):
        L = T + R * s
        u.append(keys[L:L + R], rows[L:L + R])
        u.decode_step(*zero_queries(R, 1, 16))
        st = u.state()
        pending = st["L"] - st["M"]
        assert 0 <= pending < 64
        assert st["M"] == T + 64 * ((R * (s + 1)) // 64)
    assert np.array_equal(u.mirror(0, u.state()["M"]), rows[:u.state()["M"]])


def test_bulk_append_spills_whole_batches_and_flush_completes():
    n = 1000
    u = unit(max_positions=n, index_dim=16, max_query_rows=4, ring_rows=64)
    rows = random_rows(n, 2)
    u.append(_keys(n), rows)
    st = u.state()
    # the ring keeps at most ring_rows + max_query_rows rows; the rest went out in whole batches
    assert st["L"] == n and (n - st["M"]) <= 68 and st["M"] % 64 == 0
    assert np.array_equal(u.mirror(0, st["M"]), rows[:st["M"]])
    u.flush()
    assert u.state()["M"] == n
    assert np.array_equal(u.mirror(), rows)


def test_capacity_is_checked_before_any_change():
    u = unit(max_positions=10, index_dim=16)
    u.append(_keys(8), random_rows(8, 3))
    with pytest.raises(OracleError) as e:
        u.append(_keys(3), random_rows(3, 4))
    assert e.value.status == E_CAPACITY
    assert u.state()["L"] == 8


def test_warm_needs_flushed_history_and_takes_most_recent():
    u = unit(max_positions=50, index_dim=16, hot_slots=16)
    rows = random_rows(40, 5)
    u.append(_keys(40), rows)
    with pytest.raises(OracleError) as e:
        u.warm()
    assert e.value.status == E_STATE
    u.flush()
    u.warm()
    sp, fr, pr = u.slots()
    assert sp.tolist() == list(range(24, 40))
    assert np.all(fr == -1) and np.all(pr == -1)
    assert u.state()["hand"] == 0
    assert np.array_equal(u.slot_bytes(), rows[24:40])


def test_warm_with_fewer_rows_than_slots():
    u = unit(max_positions=50, index_dim=16, hot_slots=16)
    u.append(_keys(5), random_rows(5, 6))
    u.flush()
    u.warm()
    sp, _, _ = u.slots()
    assert sp.tolist() == [0, 1, 2, 3, 4] + [-1] * 11
    assert u.state()["hand"] == 5


def test_offloaded_and_resident_compact_bytes_and_outputs_are_identical():
    # the cache changes only where bytes come from (offload page, six interleaved pairs:
    # outputs identical between offloaded and resident runs)
    g = np.random.default_rng(8)
    T, R, steps, HI, Dk, H = 300, 2, 10, 2, 16, 2
    n = T + R * steps
    keys = S.bf16_bits(g.integers(-3, 4, (n, Dk)).astype(float))
    rows = valid_rows(n, 9)
    units = [unit(max_positions=n, index_heads=HI, index_dim=Dk, heads=H, top_k=12, hot_slots=16,
                  max_query_rows=R, ring_rows=8, mode=m) for m in (0, MODE_RESIDENT)]
    for u in units:
        u.append(keys[:T], rows[:T])
        u.flush()
    units[0].warm()
    for s in range(steps):
        L = T + R * s
        q = S.bf16_bits(g.integers(-3, 4, (R, HI, Dk)).astype(float))
        w = g.integers(0, 3, (R, HI)).astype(np.float32)
        ql = S.bf16_bits(0.3 * g.standard_normal((R, H, 512)))
        qr = S.bf16_bits(0.3 * g.standard_normal((R, H, 64)))
        outs = []
        for u in units:
            u.append(keys[L:L + R], rows[L:L + R])
            outs.append(u.decode_step(q, w, ql, qr))
        assert np.array_equal(units[0].compact(), units[1].compact())
        assert np.array_equal(outs[0], outs[1])
