"""Pins for the CLOCK replacement variant (second chance with reference bits) and
for the ring walk on the same hand-worked steps."""
import json
import os

import numpy as np
import pytest

from oracle import REPL_CLOCK, REPL_RING
from tests.oracle_util import onehot_keys, random_rows, select_query, unit

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "clock_scenarios.json")))
D = 16


@pytest.mark.parametrize("policy", [REPL_RING, REPL_CLOCK], ids=["ring", "clock"])
@pytest.mark.parametrize("sc", GOLD["scenarios"], ids=lambda s: s["name"][:40])
def test_handworked_scenario(sc, policy):
    R, T = sc["rows"], sc["history"]
    n_total = T + R * len(sc["steps"])
    u = unit(max_positions=n_total, index_dim=D, top_k=sc["top_k"], hot_slots=sc["hot_slots"],
             max_query_rows=R, ring_rows=4, replacement=policy)
    rows = random_rows(n_total, 9)
    keys = onehot_keys(range(n_total), D)
    u.append(keys[:T], rows[:T])
    u.flush()
    if sc["warm"]:
        u.warm()
    L = T
    for st in sc["steps"]:
        u.append(keys[L:L + R], rows[L:L + R])
        L += R
        q, w = select_query(st["select"], D)
        u.decode_step(q, w, np.zeros((R, 1, 512), np.uint16), np.zeros((R, 1, 64), np.uint16))
        why = st["why"]
        uni, kind, src = u.union()
        assert (uni.tolist(), kind.tolist(), src.tolist()) == (st["union"], st["kind"], st["src"]), why
        want = st["clock"] if policy == REPL_CLOCK else st["ring"]
        sp, fr, pr = u.slots()
        assert (sp.tolist(), fr.tolist(), pr.tolist()) == (want["slot_pos"], want["fill_round"], want["pin_round"]), why
        state = u.state()
        assert (state["hand"], state["L"], state["M"]) == (want["hand"], st["L"], st["M"]), why
        ref = u.ref().tolist()
        assert ref == (want["ref"] if policy == REPL_CLOCK else [0] * sc["hot_slots"]), why
        cnt = u.counters()
        for k, v in st["counters"].items():
            assert cnt[k] == v, (k, why)
        assert np.array_equal(u.compact(), rows[uni])


def _clock_reference(S, hand, ref, pinned, n_miss):
    """Second chance, visit by visit: (victims in order, hand after, ref after)."""
    ref = list(ref)
    taken, visits, v = [], 0, hand
    pinned = set(pinned)
    while len(taken) < n_miss and visits < 2 * S:
        if v in pinned or v in taken:
            pass
        elif ref[v]:
            ref[v] = 0
        else:
            taken.append(v)
            ref[v] = 1
            if len(taken) == n_miss:
                break
        v = (v + 1) % S
        visits += 1
    new_hand = (taken[-1] + 1) % S if taken else hand
    return taken, new_hand, ref


@pytest.mark.parametrize("seed", range(6))
def test_random_rounds_follow_second_chance(seed):
    # many rounds on a small cache with random hits and misses: each round's fills,
    # hand and reference bits equal a visit-by-visit second-chance walk over the
    # round-start state (hits marked referenced and pinned first)
    g = np.random.default_rng(seed)
    S_, T, R, K, steps = 8, 12, 2, 3, 30
    D16 = 16
    n_total = T + R * steps
    u = unit(max_positions=n_total, index_dim=D16, top_k=K, hot_slots=S_, max_query_rows=R, ring_rows=4,
             replacement=REPL_CLOCK)
    rows = random_rows(n_total, seed)
    keys = onehot_keys(range(n_total), D16)
    u.append(keys[:T], rows[:T])
    u.flush()
    u.warm()
    L = T
    for step in range(steps):
        sp0, fr0, _ = u.slots()
        ref0 = u.ref().tolist()
        hand0 = u.state()["hand"]
        u.append(keys[L:L + R], rows[L:L + R])
        L += R
        picks = [sorted(g.choice(min(L - R + i + 1, D16), size=K, replace=False).tolist()) for i in range(R)]
        q, w = select_query(picks, D16)
        u.decode_step(q, w, np.zeros((R, 1, 512), np.uint16), np.zeros((R, 1, 64), np.uint16))
        uni, kind, src = u.union()
        hits = [int(s) for s, k in zip(src, kind) if k == 0]
        misses = [int(p) for p, k in zip(uni, kind) if k in (2, 3)]
        ref_in = list(ref0)
        for v in hits:
            ref_in[v] = 1
        taken, hand1, ref1 = _clock_reference(S_, hand0, ref_in, hits, len(misses))
        sp, fr, _ = u.slots()
        assert [int(sp[v]) for v in taken] == misses[:len(taken)], f"step {step}"
        assert [int(k) for p, k in zip(uni, kind) if k in (2, 3)] == [2] * len(taken) + [3] * (len(misses) - len(taken))
        assert u.state()["hand"] == hand1, f"step {step}"
        assert u.ref().tolist() == ref1, f"step {step}"
