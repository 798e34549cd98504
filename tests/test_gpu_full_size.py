"""GPU parity at the full workload sizes, through the C ABI, against the CPU oracle.

The first decode steps of each workload at its real shape: the same sessions,
kernels and launch configurations `bench.py` times.  Every item the oracle keeps
is compared (scores, selections, union, map, compact bytes, counters, slot
table, outputs).  The 78-layer stress workload runs every layer on the GPU and
compares a sample of layers against the oracle; the planted miss counts are
checked on every layer.
"""
import functools
import time

import numpy as np
import pytest

import dsa_synth as S
from oracle import MODE_OFFLOAD, MODE_RESIDENT
from tests.parity_util import (HIST_CHUNK, compare_unit, dev_tensor, gpu_items, gpu_session, oracle_units,
                               run_step)

pytestmark = pytest.mark.gpu


def _note(*a):
    print("[gpu-full]", *a, flush=True)


@functools.lru_cache(maxsize=None)
def _history(name, layer, seq):
    return S.history(S.WORKLOADS[name], layer, seq)


def _load(w, sess, orcs, layers, seqs):
    for gl, l in enumerate(layers):
        for q in seqs:
            keys, rows = _history(w.name, l, q)
            if orcs is not None and (l, q) in orcs:
                o = orcs[(l, q)]
                o.append(keys, rows)
                o.flush()
                o.warm()
            for c in range(0, keys.shape[0], HIST_CHUNK):
                sess.append_rows(gl, q, dev_tensor(keys[c:c + HIST_CHUNK], sess.device),
                                 dev_tensor(rows[c:c + HIST_CHUNK], sess.device))
            sess.flush(gl, q)
            sess.warm_hot(gl, q)


def _full_size(name, mode, steps):
    w = S.WORKLOADS[name]
    t0 = time.time()
    seqs = list(range(w.seqs))
    sess = gpu_session(w, mode)
    orcs = oracle_units(w, mode, layers=(0,), seqs=seqs)
    _load(w, sess, orcs, (0,), seqs)
    _note(name, f"mode={mode} loaded in {time.time() - t0:.1f} s")
    for step in range(steps):
        gout, oout = run_step(w, 0, step, sess, orcs, seqs=seqs)
        gnp = gout.cpu().numpy()
        for i, q in enumerate(seqs):
            compare_unit(sess, orcs[(0, q)], 0, q, gnp[i], oout[q], what=f"{name} mode={mode} seq={q} step={step}")
        _note(name, f"step {step} matches ({time.time() - t0:.1f} s)")
    sess.close()
    for o in orcs.values():
        o.close()


def test_million_history_offload():
    _full_size("million", MODE_OFFLOAD, steps=2)


def test_million_history_resident():
    _full_size("million", MODE_RESIDENT, steps=1)


def test_batched_16x131k_offload():
    _full_size("batched_16x131k", MODE_OFFLOAD, steps=2)


def test_stress_all_78_layers_sampled():
    w = S.WORKLOADS["stress_78_layers"]
    t0 = time.time()
    sampled = (0, 41, 77)
    sess = gpu_session(w, MODE_OFFLOAD)
    orcs = oracle_units(w, MODE_OFFLOAD, layers=sampled, seqs=[0])
    layers = list(range(w.layers))
    _load(w, sess, orcs, layers, [0])
    _note(f"stress: 78 layers loaded in {time.time() - t0:.1f} s")
    for step in range(2):
        for l in layers:
            gout, oout = run_step(w, l, step, sess, orcs if l in sampled else None)
            g = gpu_items(sess, l, 0, w.rows_per_step, w.top_k, 0, w.history + w.rows_per_step * (step + 1))
            cnt = [int(x) for x in g["counters"][:6]]
            assert (cnt[1], cnt[3]) == (2028, 80), f"layer {l} step {step}: counters {cnt}"
            if l in sampled:
                compare_unit(sess, orcs[(l, 0)], l, 0, gout.cpu().numpy()[0], oout[0],
                             what=f"stress layer={l} step={step}")
        _note(f"stress step {step}: 78 layers, sampled layers match ({time.time() - t0:.1f} s)")
    sess.close()


def test_maximum_cache_and_union_long_history():
    # the largest hot cache (2^20 slots, empty at first: the first step's ~15,000
    # misses walk several 4,096-offset passes), the largest union (8 rows x
    # Top-2048 = 16,384 entries) and a history above 65,536 positions (the Top-K's
    # long-history path with its digit and refine passes)
    from tests.parity_util import load_history
    w = S.WORKLOADS["stress_78_layers"].scaled(name="max_cache_union", wid=6, layers=1, history=100_003,
                                               hot_slots=1 << 20, planted_overlap=False, steps=3, warm=False)
    t0 = time.time()
    sess = gpu_session(w, MODE_OFFLOAD)
    orcs = oracle_units(w, MODE_OFFLOAD)
    load_history(w, sess, orcs)
    for step in range(w.steps):
        gout, oout = run_step(w, 0, step, sess, orcs)
        compare_unit(sess, orcs[(0, 0)], 0, 0, gout.cpu().numpy()[0], oout[0], what=f"max sizes step={step}")
        _note(f"max sizes step {step} matches ({time.time() - t0:.1f} s)")
    sess.close()


def test_append_past_capacity_is_refused_without_change():
    import kv_cache_offload_amd as K
    w = S.WORKLOADS["tiny"].scaled(history=100, rows_per_step=1, steps=2)
    sess = gpu_session(w, MODE_OFFLOAD)
    keys, rows = S.history(w, 0, 0)
    sess.append_rows(0, 0, dev_tensor(keys, sess.device), dev_tensor(rows, sess.device))
    k3, r3 = S.history(w.scaled(history=103), 0, 0)
    with pytest.raises(K.DsaError) as e:
        sess.append_rows(0, 0, dev_tensor(k3[:3], sess.device), dev_tensor(r3[:3], sess.device))
    assert e.value.status == K.E_CAPACITY
    assert sess.unit_state(0, 0)["L"] == 100
    sess.append_rows(0, 0, dev_tensor(k3[:2], sess.device), dev_tensor(r3[:2], sess.device))   # exactly full
    assert sess.unit_state(0, 0)["L"] == 102
    sess.close()
