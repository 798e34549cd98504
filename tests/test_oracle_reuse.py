"""Pins for selection reuse and prefetch (offload page, "Starting point": some later
layers reuse the selection while keeping their own KV rows; first decision: with
the selection known, those layers' rows could be moved early, not for free)."""
import numpy as np
import pytest

import dsa_synth as S
from oracle import E_INVALID, MODE_RESIDENT, OracleError
from tests.oracle_util import unit, valid_rows

HI, DK, H = 2, 16, 2


def _keys(g, n):
    return S.bf16_bits(g.integers(-3, 4, (n, DK)).astype(float))


def _queries(g, R):
    return (S.bf16_bits(g.integers(-3, 4, (R, HI, DK)).astype(float)),
            g.integers(0, 3, (R, HI)).astype(np.float32),
            S.bf16_bits(0.3 * g.standard_normal((R, H, 512))),
            S.bf16_bits(0.3 * g.standard_normal((R, H, 64))))


def _unit(n, mode=0, R=3, S_=40, K=24):
    return unit(max_positions=n, index_heads=HI, index_dim=DK, heads=H, top_k=K, hot_slots=S_,
                max_query_rows=R, ring_rows=8, mode=mode)


def _pair(T=300, steps=6, R=3, S_=40, K=24, seed=4):
    """Two units with the same history and appended rows."""
    g = np.random.default_rng(seed)
    n = T + R * steps
    keys, rows = _keys(g, n), valid_rows(n, seed + 1)
    us = [_unit(n, R=R, S_=S_, K=K) for _ in range(2)]
    for u in us:
        u.append(keys[:T], rows[:T])
        u.flush()
        u.warm()
    return g, keys, rows, us


def test_round_on_the_own_selection_equals_the_full_step():
    # a unit given exactly the selection its own indexer makes steps exactly like the
    # full step: same union, sources, slot table, compact bytes and outputs
    T, R = 300, 3
    g, keys, rows, (a, b) = _pair(T=T, R=R)
    for s in range(6):
        L = T + R * s
        for u in (a, b):
            u.append(keys[L:L + R], rows[L:L + R])
        q = _queries(g, R)
        out_a = a.decode_step(*q)
        sel, cnt = a.selection()
        out_b = b.decode_step_sel(sel, cnt, q[2], q[3])
        assert np.array_equal(out_a.view(np.uint32), out_b.view(np.uint32))
        for get in ("union", "slots", "selection"):
            for x, y in zip(getattr(a, get)(), getattr(b, get)()):
                assert np.array_equal(x, y), get
        assert np.array_equal(a.compact(), b.compact())
        assert a.counters() == b.counters()
        assert a.state() == b.state()


def test_invalid_selections_are_refused_without_change():
    T, R, K = 50, 2, 24
    u = _unit(T + 10, R=R, K=K)
    g = np.random.default_rng(1)
    u.append(_keys(g, T), valid_rows(T, 2))
    u.flush()
    before = u.state()
    z = np.zeros((R, H, 512), np.uint16), np.zeros((R, H, 64), np.uint16)
    sel = np.full((R, K), -1, np.int32)
    sel[:, :3] = [[1, 5, 9], [2, 3, 4]]
    bad = []
    s1 = sel.copy(); s1[0, :3] = [5, 1, 9]; bad.append((s1, [3, 3]))          # not ascending
    s2 = sel.copy(); s2[0, :3] = [1, 5, 5]; bad.append((s2, [3, 3]))          # repeated
    s3 = sel.copy(); s3[0, 2] = T - 1; bad.append((s3, [3, 3]))               # row 0 sees up to L-2
    bad.append((sel, [K + 1, 3]))                                            # more than K
    s5 = sel.copy(); s5[1, 0] = -2; bad.append((s5, [3, 3]))
    for s_, c_ in bad:
        with pytest.raises(OracleError) as e:
            u.decode_step_sel(s_, np.array(c_), *z)
        assert e.value.status == E_INVALID
        with pytest.raises(OracleError):
            u.prefetch_sel(s_, np.array(c_))
    assert u.state() == before
    u.decode_step_sel(sel, np.array([3, 3]), *z)                             # the valid one runs
    assert u.state()["round"] == 1 and u.selection()[1].tolist() == [3, 3]


def test_prefetch_turns_the_next_rounds_misses_into_hits_without_changing_outputs():
    T, R = 300, 3
    g, keys, rows, (p, n_) = _pair(T=T, R=R, S_=120)
    src = _unit(T + R * 6, R=R, S_=120)                  # the layer whose indexer selects
    src.append(keys[:T], rows[:T])
    src.flush()
    src.warm()
    for s in range(6):
        L = T + R * s
        for u in (src, p, n_):
            u.append(keys[L:L + R], rows[L:L + R])
        q = _queries(g, R)
        src.decode_step(*q)
        sel, cnt = src.selection()
        p.prefetch_sel(sel, cnt)
        pre = p.counters()
        out_p = p.decode_step_sel(sel, cnt, q[2], q[3])
        out_n = n_.decode_step_sel(sel, cnt, q[2], q[3])
        cp, cn = p.counters(), n_.counters()
        # the outputs and compact bytes depend on the rows only, never on where they came from
        assert np.array_equal(out_p.view(np.uint32), out_n.view(np.uint32))
        uni = p.union()[0]
        assert np.array_equal(p.compact(), rows[uni]) and np.array_equal(n_.compact(), rows[n_.union()[0]])
        # every miss of the prefetch round that got a slot is a hit in the round after
        # it; what misses then is what found no slot, plus ring rows the prefetch
        # round's own batched writeback sent to the mirror
        assert cp["miss"] + cp["miss_noslot"] == pre["miss_noslot"] + pre["ring"] - cp["ring"], (s, pre, cp)
        assert cp["union"] == cn["union"] == pre["union"]
        assert p.state()["round"] == 2 * (s + 1) and n_.state()["round"] == s + 1


def test_prefetch_is_a_no_op_when_resident():
    u = _unit(100, mode=MODE_RESIDENT)
    g = np.random.default_rng(3)
    u.append(_keys(g, 60), valid_rows(60, 4))
    before = u.state()
    sel = np.full((3, 24), -1, np.int32)
    sel[:, 0] = [1, 2, 3]
    u.prefetch_sel(sel, np.array([1, 1, 1]))
    assert u.state() == before
