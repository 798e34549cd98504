"""GPU parity of selection reuse and prefetch against the oracle.

Layer 0 makes the selection (full decode step); later layers reuse it with
their own rows and caches (dsa_decode_step_reuse), some after a prefetch round
(dsa_prefetch_reuse) enqueued on a second stream while layer 0's step is still
running on the first.  Every step is compared item by item with the oracle's
rounds on the same selection; after a prefetch the unit's slot table and
counters are compared too.
"""
import numpy as np
import pytest

import dsa_synth as S
from oracle import MODE_OFFLOAD, MODE_RESIDENT, REPL_CLOCK, REPL_RING
from tests.parity_util import ATOL, RTOL, compare_unit, dev_tensor, gpu_session, load_history, oracle_units

pytestmark = pytest.mark.gpu


def _note(*a):
    print("[gpu-reuse]", *a, flush=True)


def _unit_state_matches(sess, o, gl, q, S_, what):
    import torch
    torch.cuda.synchronize()
    get = lambda name: sess.debug(name, gl, q).cpu().numpy()
    sp, fr, pr = o.slots()
    assert np.array_equal(get("slot_pos").view(np.int32), sp), what
    assert np.array_equal(get("fill_round").view(np.int32), fr), what
    assert np.array_equal(get("pin_round").view(np.int32), pr), what
    assert np.array_equal(get("pos_slot").view(np.int32), o.pos_slot()), what
    assert int(get("hand").view(np.int32)[0]) == o.state()["hand"], what
    words = get("ref_bits").view(np.uint32)
    ref = ((words[:, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8).reshape(-1)[:S_]
    assert np.array_equal(ref, o.ref()), what
    assert np.array_equal(get("slot_bytes").reshape(S_, -1), o.slot_bytes()), what
    gs, st = sess.unit_state(gl, q), o.state()
    assert (gs["L"], gs["M"], gs["round"]) == (st["L"], st["M"], st["round"]), what


def _reuse_run(w, mode, steps, layers=3, prefetch=(1,), replacement=REPL_RING, side_stream=True):
    import torch
    seqs = list(range(w.seqs))
    R = w.rows_per_step
    sess = gpu_session(w, mode, n_layers=layers, replacement=replacement)
    orcs = oracle_units(w, mode, layers=range(layers), seqs=seqs, replacement=replacement)
    load_history(w, sess, orcs, layers=range(layers), seqs=seqs)
    side = torch.cuda.Stream()
    totals = {(l, q): np.zeros(9, np.int64) for l in range(layers) for q in seqs}
    names = ("union", "hit", "ring", "miss", "miss_noslot", "evict", "host_bytes", "res", "host_reads")
    dev = sess.device
    for step in range(steps):
        for l in range(layers):
            for q in seqs:
                k, r = S.step_rows(w, l, q, step)
                sess.append_rows(l, q, dev_tensor(k, dev), dev_tensor(r, dev))
                orcs[(l, q)].append(k, r)
        # layer 0 selects
        qs = [S.step_queries(w, 0, q, step) for q in seqs]
        st = lambda i: np.stack([x[i] for x in qs])
        out = torch.full((len(seqs), R, w.heads, w.latent_dim), float("nan"), dtype=torch.float32, device=dev)
        sess.decode_step(0, dev_tensor(st(0), dev), dev_tensor(st(1), dev), dev_tensor(st(2), dev),
                         dev_tensor(st(3), dev), out)
        oout = {q: orcs[(0, q)].decode_step(*qs[i]) for i, q in enumerate(seqs)}
        sel = {q: orcs[(0, q)].selection() for q in seqs}
        overlap = step % 2 == 1
        if not overlap:
            # even steps: the source layer's items are compared before any reuse (this
            # synchronises, so here the prefetch below does not overlap layer 0's step)
            g0 = out.cpu().numpy()
            for i, q in enumerate(seqs):
                compare_unit(sess, orcs[(0, q)], 0, q, g0[i], oout[q], what=f"{w.name} source seq={q} step={step}")
        for l in range(1, layers):
            if l in prefetch:
                if side_stream:
                    with torch.cuda.stream(side):             # ordered by the library's own events
                        sess.prefetch_reuse(l, 0, R)
                else:
                    sess.prefetch_reuse(l, 0, R)
                for q in seqs:
                    orcs[(l, q)].prefetch_sel(*sel[q])
                    if mode == MODE_OFFLOAD:                   # resident: no round at all
                        totals[(l, q)] += [orcs[(l, q)].counters()[k] for k in names]
                if mode == MODE_OFFLOAD:
                    for q in seqs:
                        _unit_state_matches(sess, orcs[(l, q)], l, q, w.hot_slots, f"prefetch layer {l} seq {q} step {step}")
            lq = [S.step_queries(w, l, q, step) for q in seqs]
            out_l = torch.full((len(seqs), R, w.heads, w.latent_dim), float("nan"), dtype=torch.float32, device=dev)
            sess.decode_step_reuse(l, 0, dev_tensor(np.stack([x[2] for x in lq]), dev),
                                   dev_tensor(np.stack([x[3] for x in lq]), dev), out_l)
            gl = out_l.cpu().numpy()
            for i, q in enumerate(seqs):
                o = orcs[(l, q)]
                ol = o.decode_step_sel(*sel[q], lq[i][2], lq[i][3])
                totals[(l, q)] += [o.counters()[k] for k in names]
                compare_unit(sess, o, l, q, gl[i], ol, check_scores=False,
                             what=f"{w.name} mode={mode} reuse layer={l} seq={q} step={step}")
                assert np.array_equal(sess.debug("totals", l, q).cpu().numpy().view(np.int64), totals[(l, q)])
        if overlap:
            # odd steps: the prefetch overlapped layer 0's step; its outputs are compared
            # now (its step items belong to the latest step of another layer)
            g0 = out.cpu().numpy()
            for i, q in enumerate(seqs):
                ref = oout[q].astype(np.float64)
                assert np.all(np.abs(g0[i] - ref) <= ATOL + RTOL * np.abs(ref)), f"source outputs seq={q} step={step}"
        _note(f"{w.name} mode={mode} step {step}: source and {layers - 1} reusing layers match")
    return sess, orcs


@pytest.mark.parametrize("mode", [pytest.param(MODE_OFFLOAD, id="offload"), pytest.param(MODE_RESIDENT, id="resident")])
def test_reuse_and_prefetch_small(mode):
    w = S.WORKLOADS["tiny"].scaled(seqs=2, rows_per_step=4, steps=8, hot_slots=700, warm=True, ring_rows=16)
    sess, _ = _reuse_run(w, mode, steps=w.steps)
    sess.close()


def test_reuse_and_prefetch_clock():
    w = S.WORKLOADS["tiny"].scaled(seqs=1, rows_per_step=4, steps=6, hot_slots=500, warm=True)
    sess, _ = _reuse_run(w, MODE_OFFLOAD, steps=w.steps, replacement=REPL_CLOCK)
    sess.close()


def test_reuse_and_prefetch_single_stream_shape():
    w = S.WORKLOADS["single_stream_50k"].scaled(steps=3)
    sess, _ = _reuse_run(w, MODE_OFFLOAD, steps=3, layers=2)
    sess.close()


def test_reuse_conditions_are_checked():
    import kv_cache_offload_amd as K
    import torch
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=2, steps=2, warm=True)
    sess = gpu_session(w, MODE_OFFLOAD, n_layers=3)
    load_history(w, sess, None, layers=range(3))
    dev = sess.device
    z = lambda *shape: torch.zeros(shape, dtype=torch.int16, device=dev)
    out = torch.zeros((1, 2, w.heads, 512), dtype=torch.float32, device=dev)
    ql, qr = z(1, 2, w.heads, 512), z(1, 2, w.heads, 64)

    def expect(status, fn):
        with pytest.raises(K.DsaError) as e:
            fn()
        assert e.value.status == status

    expect(K.E_STATE, lambda: sess.decode_step_reuse(1, 0, ql, qr, out))      # no full step yet
    for l in range(3):
        k, r = S.step_rows(w, l, 0, 0)
        sess.append_rows(l, 0, dev_tensor(k, dev), dev_tensor(r, dev))
    iq, iw, _, _ = S.step_queries(w, 0, 0, 0)
    sess.decode_step(0, dev_tensor(iq[None], dev), dev_tensor(iw[None], dev), ql, qr, out)
    expect(K.E_INVALID, lambda: sess.decode_step_reuse(0, 0, ql, qr, out))    # its own selection
    expect(K.E_STATE, lambda: sess.decode_step_reuse(1, 2, ql, qr, out))      # not the latest full step
    expect(K.E_STATE, lambda: sess.prefetch_reuse(1, 0, 1))                   # other rows per sequence
    k, r = S.step_rows(w, 2, 0, 1)
    sess.append_rows(2, 0, dev_tensor(k, dev), dev_tensor(r, dev))
    expect(K.E_STATE, lambda: sess.decode_step_reuse(2, 0, ql, qr, out))      # row counts differ
    sess.decode_step_reuse(1, 0, ql, qr, out)                                  # the valid one runs
    torch.cuda.synchronize()
    assert sess.unit_state(1, 0)["round"] == 1
    sess.close()
