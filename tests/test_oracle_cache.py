"""Pins for the hot cache: hand-worked scenarios and structural invariants."""
import json
import os

import numpy as np
import pytest

import dsa_synth as S
from oracle import SRC_HIT, SRC_MISS, SRC_MISS_NOSLOT, SRC_RING
from tests.oracle_util import onehot_keys, random_rows, select_query, unit

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_scenarios.json")))
D = 16


@pytest.mark.parametrize("sc", GOLD["scenarios"], ids=lambda s: s["name"][:40])
def test_handworked_scenario(sc):
    R, T = sc["rows"], sc["history"]
    n_total = T + R * len(sc["steps"])
    u = unit(max_positions=n_total, index_dim=D, top_k=sc["top_k"], hot_slots=sc["hot_slots"],
             max_query_rows=R, ring_rows=4)
    rows = random_rows(n_total, 9)
    u.append(onehot_keys(range(T), D), rows[:T])
    u.flush()
    if sc["warm"]:
        u.warm()
    L = T
    for st in sc["steps"]:
        u.append(onehot_keys(range(L, L + R), D), rows[L:L + R])
        L += R
        q, w = select_query(st["select"], D)
        u.decode_step(q, w, np.zeros((R, 1, 512), np.uint16), np.zeros((R, 1, 64), np.uint16))
        uni, kind, src = u.union()
        assert uni.tolist() == st["union"], st["why"]
        assert kind.tolist() == st["kind"], st["why"]
        assert src.tolist() == st["src"], st["why"]
        sp, fr, pr = u.slots()
        assert sp.tolist() == st["slot_pos"], st["why"]
        assert fr.tolist() == st["fill_round"], st["why"]
        assert pr.tolist() == st["pin_round"], st["why"]
        state = u.state()
        assert (state["hand"], state["M"], state["L"]) == (st["hand"], st["M"], st["L"]), st["why"]
        cnt = u.counters()
        for k, v in st["counters"].items():
            assert cnt[k] == v, (k, st["why"])
        assert cnt["host_bytes"] == (cnt["miss"] + cnt["miss_noslot"]) * 656
        # whatever the source, the compact bytes are the appended bytes of each position
        assert np.array_equal(u.compact(), rows[uni])


def _run_random(T, S_, K, R, steps, seed, warm):
    g = np.random.default_rng(seed)
    n_total = T + R * steps
    HI, Dk = 2, 16
    u = unit(max_positions=n_total, index_heads=HI, index_dim=Dk, top_k=K, hot_slots=S_,
             max_query_rows=R, ring_rows=8)
    keys = S.bf16_bits(g.integers(-3, 4, (n_total, Dk)).astype(float))
    rows = random_rows(n_total, seed + 100)
    u.append(keys[:T], rows[:T])
    u.flush()
    if warm:
        u.warm()
    L = T
    for step in range(steps):
        before_sp, before_fr, _ = u.slots()
        before_ps = u.pos_slot()
        before = u.state()
        u.append(keys[L:L + R], rows[L:L + R])
        L += R
        q = S.bf16_bits(g.integers(-3, 4, (R, HI, Dk)).astype(float))
        w = g.integers(0, 3, (R, HI)).astype(np.float32)
        u.decode_step(q, w, np.zeros((R, 1, 512), np.uint16), np.zeros((R, 1, 64), np.uint16))
        yield step, u, rows, (before_sp, before_fr, before_ps, before)


@pytest.mark.parametrize("T,S_,K,R,warm", [(200, 16, 8, 3, False), (300, 64, 16, 4, True),
                                            (120, 8, 6, 2, True), (400, 256, 32, 4, True)])
def test_invariants_random(T, S_, K, R, warm):
    for step, u, rows, (bsp, bfr, bps, bst) in _run_random(T, S_, K, R, 12, T + S_, warm):
        sp, fr, pr = u.slots()
        ps = u.pos_slot()
        r = bst["round"]
        uni, kind, src = u.union()
        # pos_slot and slot_pos are inverse maps
        for v in range(S_):
            if sp[v] >= 0:
                assert ps[sp[v]] == v
        cached = np.nonzero(ps >= 0)[0]
        assert np.array_equal(sp[ps[cached]], cached)
        assert len(cached) <= S_
        # slot bytes are the mirror bytes of the position they hold
        sb = u.slot_bytes()
        for v in range(S_):
            if sp[v] >= 0:
                assert np.array_equal(sb[v], rows[sp[v]])
        # compact bytes are the appended bytes, whatever the source
        assert np.array_equal(u.compact(), rows[uni])
        # a hit was cached before the round started, in a slot filled in an earlier round
        for x in np.nonzero(kind == SRC_HIT)[0]:
            v = src[x]
            assert bps[uni[x]] == v and bsp[v] == uni[x] and bfr[v] < r
            assert pr[v] == r                                   # and it is pinned now
        # ring rows are exactly the ones not yet written back at round start
        assert np.all((kind == SRC_RING) == (uni >= bst["M"]))
        # misses were not cached at round start; slotted misses fill in ascending order
        miss = np.nonzero(kind == SRC_MISS)[0]
        for x in miss:
            assert bps[uni[x]] == -1
            v = ps[uni[x]]
            assert v >= 0 and fr[v] == r and pr[v] == r and sp[v] == uni[x]
        if len(miss):
            slots = ps[uni[miss]]
            offs = (slots - bst["hand"]) % S_
            assert np.all(np.diff(offs) > 0)                   # ring order == ascending position order
        for x in np.nonzero(kind == SRC_MISS_NOSLOT)[0]:
            assert ps[uni[x]] == -1
        # pinned (hit) slots were never evicted
        for x in np.nonzero(kind == SRC_HIT)[0]:
            assert sp[src[x]] == uni[x]
        # map points every selected position at its union entry
        sel, cnt = u.selection()
        m = u.map()
        for i in range(sel.shape[0]):
            assert np.array_equal(uni[m[i, :cnt[i]]], sel[i, :cnt[i]])


def test_noslot_happens_only_when_every_slot_is_taken_or_pinned():
    for step, u, rows, (bsp, bfr, bps, bst) in _run_random(100, 4, 6, 3, 8, 5, False):
        c = u.counters()
        if c["miss_noslot"]:
            sp, fr, pr = u.slots()
            assert np.all(pr == bst["round"])                 # every slot was used this round
            assert c["miss"] + c["hit"] >= 4
