"""GPU parity at the full workload sizes, through the C ABI, against the CPU oracle.

The first decode steps of each workload at its real shape: the same sessions,
kernels and launch configurations `bench.py` times (its steps append and decode
in one dsa_append_decode_step call; some cases here take the two-call form).  Every item the oracle keeps
is compared (scores, selections, union, map, compact bytes, counters, slot
table, outputs).  The 78-layer stress workload compares every layer against the oracle
on its first step, in both modes, with the planted hit and miss counts checked
on every layer; offloaded and resident sessions are checked to agree bit for bit
at the 50,023-row shape across a ring writeback.
"""
import time

import numpy as np
import pytest

import dsa_synth as S
from oracle import MODE_OFFLOAD, MODE_RESIDENT
from tests.parity_util import (HIST_CHUNK, compare_unit, dev_tensor, gpu_session, load_history, oracle_units,
                               run_step)

pytestmark = pytest.mark.gpu


def _note(*a):
    print("[gpu-full]", *a, flush=True)


def _load(w, sess, orcs, layers, seqs, gpu_layers=None):
    gpu_layers = range(len(layers)) if gpu_layers is None else gpu_layers
    for gl, l in zip(gpu_layers, layers):
        for q in seqs:
            keys, rows = S.history(w, l, q)
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


def _full_size(name, mode, steps, combined=True):
    w = S.WORKLOADS[name]
    t0 = time.time()
    seqs = list(range(w.seqs))
    sess = gpu_session(w, mode)
    orcs = oracle_units(w, mode, layers=(0,), seqs=seqs)
    _load(w, sess, orcs, (0,), seqs)
    _note(name, f"mode={mode} loaded in {time.time() - t0:.1f} s")
    for step in range(steps):
        gout, oout = run_step(w, 0, step, sess, orcs, seqs=seqs, combined=combined)
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
    _full_size("million", MODE_RESIDENT, steps=1, combined=False)


@pytest.mark.parametrize("mode", [MODE_OFFLOAD, MODE_RESIDENT], ids=["offload", "resident"])
def test_single_stream_50k_append_and_decode_in_one_call(mode):
    _full_size("single_stream_50k", mode, steps=3)


def test_batched_16x131k_offload():
    _full_size("batched_16x131k", MODE_OFFLOAD, steps=2)


def _stress_every_layer(mode):
    # Every layer is loaded and stepped once with the oracle beside it (the oracle unit is
    # dropped after its comparison, except for three layers kept for a second step);
    # then every layer steps again, with the planted hit/miss counts checked on all of
    # them (offload) and the kept layers compared in full.  The first step appends with
    # dsa_append_rows, the second in the dsa_append_decode_step call.
    w = S.WORKLOADS["stress_78_layers"]
    t0 = time.time()
    kept = (0, 41, 77)
    sess = gpu_session(w, mode)
    orcs = {}
    for l in range(w.layers):
        one = oracle_units(w, mode, layers=(l,), seqs=[0])
        _load(w, sess, one, (l,), [0], gpu_layers=(l,))
        gout, oout = run_step(w, l, 0, sess, one)
        compare_unit(sess, one[(l, 0)], l, 0, gout.cpu().numpy()[0], oout[0], what=f"stress mode={mode} layer={l} step=0")
        if mode == MODE_OFFLOAD:
            cnt = sess.debug("counters", l, 0).cpu().numpy().view(np.int64)
            assert (int(cnt[1]), int(cnt[3])) == (2028, 80), f"layer {l} step 0: counters {cnt}"
        if l in kept:
            orcs.update(one)
        else:
            one[(l, 0)].close()
        if l % 13 == 12:
            _note(f"stress mode={mode}: layers 0..{l} match at step 0 ({time.time() - t0:.1f} s)")
    for l in range(w.layers):
        gout, oout = run_step(w, l, 1, sess, orcs if l in kept else None, combined=True)
        if mode == MODE_OFFLOAD:
            cnt = sess.debug("counters", l, 0).cpu().numpy().view(np.int64)
            assert (int(cnt[1]), int(cnt[3])) == (2028, 80), f"layer {l} step 1: counters {cnt}"
        if l in kept:
            compare_unit(sess, orcs[(l, 0)], l, 0, gout.cpu().numpy()[0], oout[0],
                         what=f"stress mode={mode} layer={l} step=1")
    _note(f"stress mode={mode}: step 1 on 78 layers, kept layers match ({time.time() - t0:.1f} s)")
    sess.close()
    for o in orcs.values():
        o.close()


def test_stress_all_78_layers_offload():
    _stress_every_layer(MODE_OFFLOAD)


def test_stress_all_78_layers_resident():
    _stress_every_layer(MODE_RESIDENT)


def test_batched_16x131k_resident():
    _full_size("batched_16x131k", MODE_RESIDENT, steps=2)


def test_offload_and_resident_are_identical_single_stream_50k():
    # The offload page's acceptance check (section "GPU cache management errs too"): with
    # the cache fixed, the offloaded run's output matched the resident run's exactly.  Both
    # sessions take the same inputs for 24 steps: the ring's first 64-row batch goes back
    # to the mirror after step 15, so the later steps read those rows as misses, not ring
    # rows.  Outputs, selections and the compact rows must agree bit for bit.
    import torch
    w = S.WORKLOADS["single_stream_50k"]
    t0 = time.time()
    off = gpu_session(w, MODE_OFFLOAD)
    res = gpu_session(w, MODE_RESIDENT)
    load_history(w, off)
    load_history(w, res)
    kinds_seen = set()
    for step in range(24):
        go, _ = run_step(w, 0, step, off)
        gr, _ = run_step(w, 0, step, res)
        torch.cuda.synchronize()
        assert torch.equal(go.view(torch.int32), gr.view(torch.int32)), f"step {step}: outputs differ"
        co = off.debug("counters").cpu().numpy().view(np.int64)
        cr = res.debug("counters").cpu().numpy().view(np.int64)
        U = int(co[0])
        assert U == int(cr[0]), f"step {step}: union sizes differ"
        for item in ("selection", "sel_count", "union", "map"):
            a, b = off.debug(item).cpu().numpy(), res.debug(item).cpu().numpy()
            if item == "union":
                a, b = a.view(np.int32)[:U], b.view(np.int32)[:U]
            assert np.array_equal(a, b), f"step {step}: {item} differs"
        ca = off.debug("compact").cpu().numpy().reshape(-1, 656)[:U]
        cb = res.debug("compact").cpu().numpy().reshape(-1, 656)[:U]
        assert np.array_equal(ca, cb), f"step {step}: compact rows differ"
        kinds_seen |= set(off.debug("union_kind").cpu().numpy().view(np.int32)[:U].tolist())
    st = off.unit_state(0, 0)
    assert st["M"] == w.history + 64, f"one ring batch written back: {st}"
    assert {0, 1, 2} <= kinds_seen, f"hits, ring rows and misses all seen: {kinds_seen}"
    _note(f"offload == resident for 24 steps ({time.time() - t0:.1f} s)")
    off.close()
    res.close()


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
    # the one-call step refuses rows past max_positions before it enqueues anything
    import torch
    iq, iw, ql, qr = (dev_tensor(x[None], sess.device) for x in S.step_queries(w, 0, 0, 0))
    out = torch.zeros((1, 1, w.heads, w.latent_dim), dtype=torch.float32, device=sess.device)
    with pytest.raises(K.DsaError) as e:
        sess.append_decode_step(0, dev_tensor(k3[None, 2:3], sess.device), dev_tensor(r3[None, 2:3], sess.device),
                                iq, iw, ql, qr, out)
    assert e.value.status == K.E_CAPACITY
    assert sess.unit_state(0, 0)["L"] == 102
    sess.close()
