"""Pins for rollback after a rejected verify (offload page, "Capacity must survive
the session lifecycle": rejected drafts roll back the KV rows and the DSA state).

What fixes the oracle here is not the rollback code itself but what a rollback
must preserve: every later step depends on the logical history only, so it has
to give exactly what a unit that never saw the rejected rows gives; the compact
rows must be the logical rows' bytes; the mirror must end up holding exactly the
logical rows; no hot slot may hold a position past the end of the history.
"""
import numpy as np
import pytest

import dsa_synth as S
from oracle import E_INVALID, E_STATE, MODE_RESIDENT, OracleError
from tests.oracle_util import random_rows, unit, valid_rows

HI, DK, H = 2, 16, 2


def _keys(g, n):
    return S.bf16_bits(g.integers(-3, 4, (n, DK)).astype(float))


def _queries(g, R):
    return (S.bf16_bits(g.integers(-3, 4, (R, HI, DK)).astype(float)),
            g.integers(0, 3, (R, HI)).astype(np.float32),
            S.bf16_bits(0.3 * g.standard_normal((R, H, 512))),
            S.bf16_bits(0.3 * g.standard_normal((R, H, 64))))


def _unit(n, mode=0, R=4, S_=32, K=24, ring_rows=8):
    return unit(max_positions=n, index_heads=HI, index_dim=DK, heads=H, top_k=K, hot_slots=S_,
                max_query_rows=R, ring_rows=ring_rows, mode=mode)


def _slot_table_consistent(u):
    L = u.state()["L"]
    sp, _, _ = u.slots()
    ps = u.pos_slot()
    assert np.all(sp < L), "a slot holds a position past the end of the history"
    for v, p in enumerate(sp):
        if p >= 0:
            assert ps[p] == v
    assert np.all((ps[:L] == -1) | (sp[np.maximum(ps[:L], 0)] == np.arange(L)))


@pytest.mark.parametrize("mode", [0, MODE_RESIDENT])
def test_verify_rounds_with_rejections_match_a_unit_that_never_saw_them(mode):
    g = np.random.default_rng(31)
    T, R, steps = 300, 4, 30
    cap = T + R * steps
    keys = _keys(g, T)
    rows = valid_rows(T, 32)
    a = _unit(cap, mode)
    a.append(keys, rows)
    a.flush()
    if mode == 0:
        a.warm()
    log_k, log_r = keys, rows              # the logical history
    cut_mirror = deep = 0
    for s in range(steps):
        dk, dr = _keys(g, R), valid_rows(R, 100 + s)
        q = _queries(g, R)
        a.append(dk, dr)
        out = a.decode_step(*q)
        sel, cnt = a.selection()
        uni, _, _ = a.union()

        # a unit built from the logical history plus this step's rows, never rolled back
        hk, hr = np.concatenate([log_k, dk]), np.concatenate([log_r, dr])
        b = _unit(cap, mode)
        b.append(hk, hr)
        b.flush()
        out_b = b.decode_step(*q)
        sel_b, cnt_b = b.selection()
        assert np.array_equal(out.view(np.uint32), out_b.view(np.uint32)), f"step {s}: outputs"
        assert np.array_equal(sel, sel_b) and np.array_equal(cnt, cnt_b), f"step {s}: selection"
        assert np.array_equal(a.scores().view(np.uint32), b.scores().view(np.uint32)), f"step {s}: scores"
        # every compact row holds the logical row's bytes, whatever its source
        assert np.array_equal(a.compact(), hr[uni]), f"step {s}: compact bytes"
        b.close()

        before = a.state()
        if mode == 0 and s % 6 == 5:
            # as far back as allowed: every row appended since the round's mirror count
            n = before["L"] - before["floor"]
            deep += n > R
        else:
            n = R - int(g.integers(1, R + 1))
        a.rollback(n)
        st = a.state()
        assert st["L"] == before["L"] - n
        assert st["round"] == before["round"] and st["hand"] == before["hand"]
        cut_mirror += before["M"] > st["L"]
        if mode == 0:
            _slot_table_consistent(a)
        log_k, log_r = hk[:st["L"]], hr[:st["L"]]
    if mode == 0:
        assert cut_mirror > 0, "no rollback reached into rows already written back"
        assert deep > 0, "no rollback reached past this round's rows"
    a.flush()
    assert np.array_equal(a.mirror(), log_r)


def test_rollback_is_refused_below_the_round_start_mirror_count():
    g = np.random.default_rng(5)
    T, R = 100, 4
    u = _unit(T + 40, R=R, ring_rows=8)
    u.append(_keys(g, T), random_rows(T, 1))
    u.flush()
    u.warm()                                # rows below L = 100 may now sit in slots
    for n in (1, T + 1):
        with pytest.raises(OracleError) as e:
            u.rollback(n)
        assert e.value.status == E_STATE and u.state()["L"] == T
    with pytest.raises(OracleError) as e:
        u.rollback(-1)
    assert e.value.status == E_INVALID
    u.rollback(0)
    u.append(_keys(g, R), random_rows(R, 2))
    u.rollback(R)                           # rows appended since the warm: allowed
    assert u.state()["L"] == T
    for s in range(2):                      # two rounds: 8 pending rows are written back
        u.append(_keys(g, R), random_rows(R, 3 + s))
        u.decode_step(*_queries(g, R))
    st = u.state()
    assert (st["L"], st["M"]) == (T + 8, T + 8)
    u.append(_keys(g, R), random_rows(R, 9))
    u.decode_step(*_queries(g, R))          # this round started with M = 108
    with pytest.raises(OracleError) as e:
        u.rollback(R + 1)
    assert e.value.status == E_STATE and u.state()["L"] == T + 12
    u.rollback(R)
    assert (u.state()["L"], u.state()["M"]) == (T + 8, T + 8)


def test_resident_rollback_reaches_any_prefix():
    g = np.random.default_rng(6)
    u = _unit(50, MODE_RESIDENT)
    rows = random_rows(40, 7)
    u.append(_keys(g, 40), rows)
    u.decode_step(*_queries(g, 4))
    u.rollback(40)
    assert (u.state()["L"], u.state()["M"]) == (0, 0)
    with pytest.raises(OracleError) as e:
        u.rollback(1)
    assert e.value.status == E_STATE
    u.append(_keys(g, 10), rows[5:15])
    assert np.array_equal(u.mirror(), rows[5:15])
