"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Scores, selections, union/map, compact bytes, counters and slot-table state are
compared bit-exactly (integer-valued inputs make every fp32 sum exact); attention
outputs within |d| <= 2e-3 + 1e-2 |ref|.
"""
import json
import os

import numpy as np
import pytest

import dsa_synth as S
from oracle import MODE_OFFLOAD, MODE_RESIDENT, OracleUnit, UnitShape
from tests.parity_util import (compare_unit, dev_tensor, gpu_items, gpu_session, load_history,
                               oracle_units, run_step)

pytestmark = pytest.mark.gpu

MODES = [pytest.param(MODE_OFFLOAD, id="offload"), pytest.param(MODE_RESIDENT, id="resident")]


def _note(*a):
    print("[gpu-parity]", *a, flush=True)


def _run_and_compare(w, mode, steps, layers=(0,), seqs=None, rows_fn=None, query_fn=None, history_fn=None,
                     warm=None, check_scores=True, replacement=0, combined=False, before_steps=None):
    seqs = list(range(w.seqs) if seqs is None else seqs)
    sess = gpu_session(w, mode, n_layers=len(layers), replacement=replacement)
    orcs = oracle_units(w, mode, layers=layers, seqs=seqs, replacement=replacement)
    load_history(w, sess, orcs, layers=layers, seqs=seqs, warm=warm, history_fn=history_fn)
    if before_steps is not None:
        before_steps(sess, orcs)
    for step in range(steps):
        for gl, l in enumerate(layers):
            gout, oout = run_step(w, l, step, sess, orcs, gpu_layer=gl, seqs=seqs, rows_fn=rows_fn,
                                  query_fn=query_fn, combined=combined)
            gnp = gout.cpu().numpy()
            for i, q in enumerate(seqs):
                compare_unit(sess, orcs[(l, q)], gl, q, gnp[i], oout[q], check_scores=check_scores,
                             what=f"{w.name} mode={mode} layer={l} seq={q} step={step}")
    sess.close()
    return orcs


@pytest.mark.parametrize("mode", MODES)
def test_tiny_workload_every_step(mode):
    w = S.WORKLOADS["tiny"]
    _note("tiny", mode)
    _run_and_compare(w, mode, steps=w.steps)


@pytest.mark.parametrize("mode", MODES)
def test_single_stream_50k_first_steps(mode):
    w = S.WORKLOADS["single_stream_50k"]
    _note("single_stream_50k", mode)
    _run_and_compare(w, mode, steps=3)


def test_history_shorter_than_k():
    # every visible position is selected; rows see different numbers of positions
    w = S.WORKLOADS["tiny"].scaled(history=150, rows_per_step=4, top_k=256, hot_slots=64, steps=3)
    _note("short history")
    _run_and_compare(w, MODE_OFFLOAD, steps=3)


def test_all_scores_equal_select_lowest_positions():
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=2, steps=2)

    def q_zero_weight(w_, layer, seq, step):
        iq, iw, ql, qr = S.step_queries(w_, layer, seq, step)
        return iq, np.zeros_like(iw), ql, qr
    _note("ties")
    orcs = _run_and_compare(w, MODE_OFFLOAD, steps=2, query_fn=q_zero_weight)
    sel, _ = orcs[(0, 0)].selection()
    assert sel[0].tolist() == list(range(w.top_k))


def test_all_equal_scores_long_history():
    # 50,023 equal scores: the Top-K candidates exceed what the resolve keeps in LDS,
    # so the selection runs its streaming path; the lowest 2048 positions are selected
    w = S.WORKLOADS["single_stream_50k"]

    def q_zero_weight(w_, layer, seq, step):
        iq, iw, ql, qr = S.step_queries(w_, layer, seq, step)
        return iq, np.zeros_like(iw), ql, qr
    _note("ties, long history")
    orcs = _run_and_compare(w, MODE_OFFLOAD, steps=1, query_fn=q_zero_weight)
    sel, _ = orcs[(0, 0)].selection()
    assert sel[3].tolist() == list(range(w.top_k))


def test_planted_ties_small_key_alphabet():
    # keys and queries from {-1, 0, 1}: scores collide often, the tie rule decides the cutoff
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=3, steps=3, history=6000)

    def hist(w_, layer, seq):
        keys, rows = S.history(w_, layer, seq)
        g = np.random.default_rng(77)
        return S.bf16_bits(g.integers(-1, 2, keys.shape).astype(float)), rows

    def q_small(w_, layer, seq, step):
        iq, iw, ql, qr = S.step_queries(w_, layer, seq, step)
        g = np.random.default_rng(1000 + step)
        return S.bf16_bits(g.integers(-1, 2, iq.shape).astype(float)), iw, ql, qr
    _note("planted ties")
    _run_and_compare(w, MODE_OFFLOAD, steps=3, history_fn=hist, query_fn=q_small)


def test_one_chunk_holds_every_candidate():
    # positions 8192..12287 (the third 4096-position chunk) carry one key that
    # outscores every other: the Top-K's candidates are that chunk's 4,096 equal
    # keys, one chunk list far longer than the part the final step reads early,
    # and the tie rule takes its lowest 2,048 positions
    w = S.WORKLOADS["tiny"].scaled(history=20000, rows_per_step=2, steps=2, top_k=2048, hot_slots=4096)

    def hist(w_, layer, seq):
        keys, rows = S.history(w_, layer, seq)
        keys = keys.copy()
        keys[8192:12288] = S.bf16_bits(np.full((4096, keys.shape[1]), 8.0))
        return keys, rows

    def q_ones(w_, layer, seq, step):
        iq, iw, ql, qr = S.step_queries(w_, layer, seq, step)
        return S.bf16_bits(np.ones(iq.shape)), np.ones_like(iw), ql, qr
    _note("one chunk of candidates")
    orcs = _run_and_compare(w, MODE_OFFLOAD, steps=2, history_fn=hist, query_fn=q_ones)
    sel, _ = orcs[(0, 0)].selection()
    assert sel[0].tolist() == list(range(8192, 8192 + 2048))


def test_peaked_attention():
    # queries x50 (integer-valued latent/rope queries in [-4, 4] * 50): softmax far from uniform,
    # so a wrong scale, RoPE term or row index moves outputs past the tolerance
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=2, steps=2)

    def q_peaked(w_, layer, seq, step):
        iq, iw, _, _ = S.step_queries(w_, layer, seq, step)
        g = np.random.default_rng(500 + step)
        ql = S.bf16_bits(g.integers(-4, 5, (w_.rows_per_step, w_.heads, 512)) * 50.0 / 64.0)
        qr = S.bf16_bits(g.integers(-4, 5, (w_.rows_per_step, w_.heads, 64)) * 50.0)
        return iq, iw, ql, qr
    _note("peaked")
    _run_and_compare(w, MODE_OFFLOAD, steps=2, query_fn=q_peaked)


def test_more_misses_than_slots():
    # S < R*K: pinned hits plus fills exhaust the cache, the rest read from host without a slot
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=4, hot_slots=300, steps=3)
    _note("noslot")
    _run_and_compare(w, MODE_OFFLOAD, steps=3)


def test_ring_rows_and_writeback_over_many_steps():
    # small history, one row per step: recent rows are selected from the ring and the
    # 64-row batch writeback fires; every step is compared
    w = S.WORKLOADS["tiny"].scaled(history=300, rows_per_step=1, top_k=64, hot_slots=128, steps=70)

    def q_recent(w_, layer, seq, step):
        iq, iw, ql, qr = S.step_queries(w_, layer, seq, step)
        return iq, iw, ql, qr

    def rows_recent(w_, layer, seq, step):
        keys, rows = S.step_rows(w_, layer, seq, step)
        return S.bf16_bits(np.full(keys.shape, 8.0)), rows     # new keys score high for positive queries
    _note("ring + writeback")
    _run_and_compare(w, MODE_OFFLOAD, steps=70, rows_fn=rows_recent, query_fn=q_recent)


@pytest.mark.parametrize("mode", MODES)
def test_append_and_decode_in_one_call(mode):
    # dsa_append_decode_step against the oracle's append then decode, every step of the tiny workload
    w = S.WORKLOADS["tiny"]
    _note("append + decode in one call", mode)
    _run_and_compare(w, mode, steps=w.steps, combined=True)


@pytest.mark.parametrize("mode", MODES)
def test_append_and_decode_in_one_call_batched(mode):
    # five sequences: each gets its own rows from the one call
    w = S.WORKLOADS["batched_16x131k"].scaled(history=9000, seqs=5, hot_slots=1024, steps=3)
    _note("append + decode in one call, batched", mode)
    _run_and_compare(w, mode, steps=3, combined=True)


def test_append_and_decode_in_one_call_ring_and_writeback():
    # the ring and its 64-row writeback over 70 one-row steps, appended by the score launch; the new
    # keys score high, so the rows just appended are selected from the ring in the same step
    w = S.WORKLOADS["tiny"].scaled(history=300, rows_per_step=1, top_k=64, hot_slots=128, steps=70)

    def rows_recent(w_, layer, seq, step):
        keys, rows = S.step_rows(w_, layer, seq, step)
        return S.bf16_bits(np.full(keys.shape, 8.0)), rows
    _note("append + decode in one call, ring + writeback")
    _run_and_compare(w, MODE_OFFLOAD, steps=70, rows_fn=rows_recent, combined=True)


def test_append_and_decode_in_one_call_spills_the_ring_first():
    # 66 rows appended after the warm start leave the ring too full for a step's 4 rows: the call
    # writes the oldest 64 back to the mirror before the score launch appends
    w = S.WORKLOADS["tiny"].scaled(history=2000, rows_per_step=4, hot_slots=512, steps=20)   # room for 66 more

    def extra_rows(sess, orcs):
        g = np.random.default_rng(5)
        keys = S.bf16_bits(g.integers(-8, 8, (66, w.index_dim)).astype(float))
        rows = S.make_rows(g, 66, w)
        sess.append_rows(0, 0, dev_tensor(keys, sess.device), dev_tensor(rows, sess.device))
        orcs[(0, 0)].append(keys, rows)
        st = sess.unit_state(0, 0)
        assert st["L"] - st["M"] == 66, st
    _note("append + decode in one call, ring spill")
    _run_and_compare(w, MODE_OFFLOAD, steps=3, combined=True, before_steps=extra_rows)


@pytest.mark.parametrize("mode", MODES)
def test_batched_sequences(mode):
    w = S.WORKLOADS["batched_16x131k"].scaled(history=9000, seqs=5, hot_slots=1024, steps=2)
    _note("batched", mode)
    _run_and_compare(w, mode, steps=2)


def test_planted_stress_two_layers():
    w = S.WORKLOADS["stress_78_layers"]
    _note("planted stress layers 0 and 41")
    orcs = _run_and_compare(w, MODE_OFFLOAD, steps=2, layers=(0, 41))
    c = orcs[(0, 0)].counters()
    assert c["miss"] == 80 and c["hit"] == 2028


def test_handworked_cache_scenarios_on_gpu():
    # the hand-derived scenarios of tests/golden/cache_scenarios.json, padded to the GPU shapes
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_scenarios.json")))
    import kv_cache_offload_amd as K
    import torch
    for sc in gold["scenarios"]:
        _note("scenario", sc["name"][:40])
        R, T = sc["rows"], sc["history"]
        n = T + R * len(sc["steps"])
        cfg = K.make_config(max_positions=n, index_heads=4, heads=16, top_k=sc["top_k"], hot_slots=sc["hot_slots"],
                            max_query_rows=R, ring_rows=4)
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
            assert g["union"].tolist() == st["union"], st["why"]
            assert g["kind"].tolist() == st["kind"], st["why"]
            assert g["src"].tolist() == st["src"], st["why"]
            assert g["slot_pos"].tolist() == st["slot_pos"], st["why"]
            assert g["fill_round"].tolist() == st["fill_round"], st["why"]
            assert g["pin_round"].tolist() == st["pin_round"], st["why"]
            assert g["hand"] == st["hand"], st["why"]
            us = sess.unit_state(0, 0)
            assert (us["M"], us["L"]) == (st["M"], st["L"]), st["why"]
            names = ("union", "hit", "ring", "miss", "miss_noslot", "evict", "host_bytes", "res", "host_reads")
            assert {k: v for k, v in zip(names, [int(x) for x in g["counters"]]) if k in st["counters"]} == st["counters"], st["why"]
            assert np.array_equal(g["compact"], rows[g["union"]]), st["why"]
        sess.close()


def test_mirror_after_flush_equals_appended_rows():
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=4, steps=20)
    sess = gpu_session(w, MODE_OFFLOAD)
    load_history(w, sess, None)
    appended = [S.history(w, 0, 0)[1]]
    for step in range(20):
        keys, rows = S.step_rows(w, 0, 0, step)
        appended.append(rows)
        sess.append_rows(0, 0, dev_tensor(keys, sess.device), dev_tensor(rows, sess.device))
    sess.flush(0, 0)
    import torch
    torch.cuda.synchronize()
    assert sess.mirror_rows(0, 0) == w.history + 80
    m = sess.debug("mirror", 0, 0).cpu().numpy().reshape(-1, 656)
    assert np.array_equal(m, np.concatenate(appended))
    sess.close()


def test_key_store_round_trip():
    # index keys are kept in the score kernel's operand order; the inspection copy
    # rebuilds row order: both append paths, a ragged tail of a 32-position tile
    w = S.WORKLOADS["tiny"].scaled(history=1000, rows_per_step=3, steps=3)
    sess = gpu_session(w, MODE_OFFLOAD)
    keys, rows = S.history(w, 0, 0)
    sess.append_rows(0, 0, dev_tensor(keys[:700], sess.device), dev_tensor(rows[:700], sess.device))
    g = np.random.default_rng(2)
    lat = S.bf16_bits(g.standard_normal((300, 512)))
    rope = S.bf16_bits(g.standard_normal((300, 64)))
    sess.append_latent(0, 0, dev_tensor(keys[700:], sess.device), dev_tensor(lat, sess.device),
                       dev_tensor(rope, sess.device))
    nk, nr = S.step_rows(w, 0, 0, 0)
    sess.append_rows(0, 0, dev_tensor(nk, sess.device), dev_tensor(nr, sess.device))
    import torch
    torch.cuda.synchronize()
    got = sess.debug("keys", 0, 0).cpu().numpy().view(np.uint16).reshape(-1, 128)
    assert np.array_equal(got, np.concatenate([keys, nk]))
    sess.close()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("heads,index_heads", [(32, 8), (128, 16)], ids=["H32-HI8", "H128-HI16"])
def test_other_head_counts(mode, heads, index_heads):
    # the score kernel's H_I = 8 and 16 variants, the attention kernel's 2- and
    # 8-wave variants and the merge of 32-head groups (one and four per row),
    # over several splits with a ragged last one (K = 320: five 64-row splits)
    w = S.WORKLOADS["tiny"].scaled(heads=heads, index_heads=index_heads, top_k=320, rows_per_step=2,
                                   history=2000, hot_slots=600, steps=4, warm=True)
    _note("heads", heads, "index heads", index_heads, mode)
    _run_and_compare(w, mode, steps=w.steps)


@pytest.mark.parametrize("mode", MODES)
def test_several_layers_and_sequences(mode):
    # kernels form sequence q's buffers from sequence 0's descriptors of the
    # layer and the strides: layers past the first, sequences past the first
    # few, the ring writeback and the hot cache of every (layer, sequence)
    w = S.WORKLOADS["batched_16x131k"].scaled(history=3000, seqs=6, rows_per_step=2, top_k=256,
                                              hot_slots=512, steps=40, warm=True)
    _note("layers x sequences", mode)
    _run_and_compare(w, mode, steps=40, layers=(0, 1, 2))


def test_several_layers_and_sequences_clock():
    # CLOCK's reference bits of every (layer, sequence) unit, through the strided descriptors
    from oracle import REPL_CLOCK
    w = S.WORKLOADS["batched_16x131k"].scaled(history=3000, seqs=5, rows_per_step=2, top_k=256,
                                              hot_slots=400, steps=30, warm=True)
    _note("layers x sequences, CLOCK")
    _run_and_compare(w, MODE_OFFLOAD, steps=30, layers=(0, 1), replacement=REPL_CLOCK)
