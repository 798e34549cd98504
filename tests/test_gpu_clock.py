"""GPU parity of the CLOCK replacement variant (second chance with reference bits)
against the oracle: the hand-worked scenarios of tests/golden/clock_scenarios.json
under both policies, and whole workloads under CLOCK with the slot table and the
reference bits compared after every step."""
import json
import os

import numpy as np
import pytest

import dsa_synth as S
from oracle import MODE_OFFLOAD, REPL_CLOCK, REPL_RING
from tests.parity_util import compare_unit, dev_tensor, gpu_items, gpu_session, load_history, oracle_units, run_step

pytestmark = pytest.mark.gpu


def _note(*a):
    print("[gpu-clock]", *a, flush=True)


@pytest.mark.parametrize("policy", [REPL_RING, REPL_CLOCK], ids=["ring", "clock"])
def test_handworked_clock_scenarios_on_gpu(policy):
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "clock_scenarios.json")))
    import kv_cache_offload_amd as K
    import torch
    for sc in gold["scenarios"]:
        _note("scenario", sc["name"][:40], "policy", policy)
        R, T = sc["rows"], sc["history"]
        n = T + R * len(sc["steps"])
        cfg = K.make_config(max_positions=n, index_heads=4, heads=16, top_k=sc["top_k"], hot_slots=sc["hot_slots"],
                            max_query_rows=R, ring_rows=4, replacement=policy)
        sess = K.Session(cfg)
        rows = np.random.default_rng(9).integers(0, 256, (n, 656), dtype=np.uint8)
        keys = np.zeros((n, 128))
        for t in range(min(n, 16)):
            keys[t, t] = 1.0
        keys = S.bf16_bits(keys)
        sess.append_rows(0, 0, dev_tensor(keys[:T], sess.device), dev_tensor(rows[:T], sess.device))
        sess.flush(0, 0)
        if sc["warm"]:
            sess.warm_hot(0, 0)
        L = T
        for st in sc["steps"]:
            sess.append_rows(0, 0, dev_tensor(keys[L:L + R], sess.device), dev_tensor(rows[L:L + R], sess.device))
            L += R
            q = np.zeros((1, R, 4, 128))
            for i, ps in enumerate(st["select"]):
                for p in ps:
                    q[0, i, 0, p] = 2.0
            wq = np.zeros((1, R, 4), np.float32)
            wq[:, :, 0] = 1.0
            out = torch.zeros((1, R, 16, 512), dtype=torch.float32, device=sess.device)
            zl = np.zeros((1, R, 16, 512), np.uint16)
            zr = np.zeros((1, R, 16, 64), np.uint16)
            sess.decode_step(0, dev_tensor(S.bf16_bits(q), sess.device), dev_tensor(wq, sess.device),
                             dev_tensor(zl, sess.device), dev_tensor(zr, sess.device), out)
            g = gpu_items(sess, 0, 0, R, sc["top_k"], sc["hot_slots"], L)
            why = st["why"]
            assert (g["union"].tolist(), g["kind"].tolist(), g["src"].tolist()) == \
                (st["union"], st["kind"], st["src"]), why
            want = st["clock"] if policy == REPL_CLOCK else st["ring"]
            assert g["slot_pos"].tolist() == want["slot_pos"], why
            assert g["fill_round"].tolist() == want["fill_round"], why
            assert g["pin_round"].tolist() == want["pin_round"], why
            assert g["hand"] == want["hand"], why
            assert g["ref"].tolist() == (want["ref"] if policy == REPL_CLOCK else [0] * sc["hot_slots"]), why
            us = sess.unit_state(0, 0)
            assert (us["M"], us["L"]) == (st["M"], st["L"]), why
            names = ("union", "hit", "ring", "miss", "miss_noslot", "evict", "host_bytes", "res", "host_reads")
            assert {k: v for k, v in zip(names, [int(x) for x in g["counters"]]) if k in st["counters"]} == st["counters"], why
            assert np.array_equal(g["compact"], rows[g["union"]]), why
        sess.close()


def _clock_run(w, steps, layers=(0,), warm=None):
    seqs = list(range(w.seqs))
    sess = gpu_session(w, MODE_OFFLOAD, n_layers=len(layers), replacement=REPL_CLOCK)
    orcs = oracle_units(w, MODE_OFFLOAD, layers=layers, seqs=seqs, replacement=REPL_CLOCK)
    load_history(w, sess, orcs, layers=layers, seqs=seqs, warm=warm)
    for step in range(steps):
        for gl, l in enumerate(layers):
            gout, oout = run_step(w, l, step, sess, orcs, gpu_layer=gl, seqs=seqs)
            gnp = gout.cpu().numpy()
            for i, q in enumerate(seqs):
                compare_unit(sess, orcs[(l, q)], gl, q, gnp[i], oout[q],
                             what=f"{w.name} clock layer={l} seq={q} step={step}")
        _note(f"{w.name} step {step} matches")
    sess.close()
    return orcs


def test_clock_tiny_cold_cache_every_step():
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=4, steps=12, hot_slots=600)
    _clock_run(w, steps=w.steps)


def test_clock_more_misses_than_slots():
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=4, hot_slots=300, steps=3)
    _clock_run(w, steps=3)


def test_clock_small_cache_many_rounds():
    # a 700-slot cache that misses part of every selection: reference bits are set,
    # cleared and reused over many rounds, and the hand laps the cache
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=2, top_k=128, hot_slots=700, steps=30, warm=True)
    _clock_run(w, steps=w.steps)


def test_clock_full_cache_all_referenced_single_stream():
    # warm 32,768-slot cache, every reference bit set: the first misses make the hand
    # clear a whole lap before it takes a slot
    w = S.WORKLOADS["single_stream_50k"]
    _clock_run(w, steps=3)


def test_clock_planted_stress_probe_shape():
    # the page's probe: full cache, every bit set, about 1% of the 2,048 selected rows miss
    w = S.WORKLOADS["stress_78_layers"]
    orcs = _clock_run(w, steps=2, layers=(0, 41))
    c = orcs[(0, 0)].counters()
    assert c["miss"] == 80 and c["hit"] == 2028
