"""GPU parity of verify rounds with rejected drafts (offload page, "Capacity must
survive the session lifecycle": rejected drafts roll back the KV rows and the DSA
selection state).

Each round appends R draft rows per sequence, runs one decode step over them,
accepts a seeded random prefix of 1..R rows per sequence and rolls the rest back,
on the HIP path (dsa_rollback_rows through the C ABI) and on the oracle.  Every
decode step is compared item by item; after each rollback the host state must
agree, and rollbacks below the allowed bound must be refused on both sides.
"""
import numpy as np
import pytest

import dsa_synth as S
from oracle import E_STATE, MODE_OFFLOAD, MODE_RESIDENT, OracleError
from tests.parity_util import compare_unit, gpu_session, load_history, oracle_units, run_step

pytestmark = pytest.mark.gpu

MODES = [pytest.param(MODE_OFFLOAD, id="offload"), pytest.param(MODE_RESIDENT, id="resident")]


def _note(*a):
    print("[gpu-rollback]", *a, flush=True)


def _verify_rounds(w, mode, seed):
    import kv_cache_offload_amd as K
    seqs = list(range(w.seqs))
    sess = gpu_session(w, mode)
    orcs = oracle_units(w, mode, seqs=seqs)
    load_history(w, sess, orcs, seqs=seqs)
    g = np.random.default_rng(seed)
    cut_mirror = refused = deep = 0
    for step in range(w.steps):
        gout, oout = run_step(w, 0, step, sess, orcs, seqs=seqs)
        gnp = gout.cpu().numpy()
        for i, q in enumerate(seqs):
            compare_unit(sess, orcs[(0, q)], 0, q, gnp[i], oout[q], what=f"{w.name} mode={mode} seq={q} step={step}")
        for q in seqs:
            o = orcs[(0, q)]
            before = o.state()
            if mode == MODE_OFFLOAD and step % 5 == 4:
                # one row past the allowed bound is refused on both sides; the bound
                # itself (every row appended since the round's mirror count) is taken
                n = before["L"] - before["floor"]
                with pytest.raises(OracleError) as e:
                    o.rollback(n + 1)
                assert e.value.status == E_STATE
                with pytest.raises(K.DsaError) as e:
                    sess.rollback_rows(0, q, n + 1)
                assert e.value.status == K.E_STATE
                refused += 1
                deep += n > w.rows_per_step
            else:
                n = w.rows_per_step - int(g.integers(1, w.rows_per_step + 1))
            o.rollback(n)
            sess.rollback_rows(0, q, n)
            st, gs = o.state(), sess.unit_state(0, q)
            assert (gs["L"], gs["M"], gs["round"]) == (st["L"], st["M"], st["round"]), f"seq {q} step {step}"
            cut_mirror += st["M"] < before["M"]
        _note(f"mode={mode} step {step} matches; L={[orcs[(0, q)].state()['L'] for q in seqs]}")
    sess.close()
    return cut_mirror, refused, deep


@pytest.mark.parametrize("mode", MODES)
def test_verify_rounds_with_rejected_drafts(mode):
    w = S.WORKLOADS["tiny"].scaled(seqs=2, rows_per_step=4, steps=40, hot_slots=512, warm=True, ring_rows=16)
    cut, refused, deep = _verify_rounds(w, mode, seed=11)
    if mode == MODE_OFFLOAD:
        assert cut > 0, "no rollback reached into rows already written back"
        assert refused > 0 and deep > 0


def test_verify_rounds_at_the_single_stream_shape():
    w = S.WORKLOADS["single_stream_50k"].scaled(steps=20)
    cut, refused, deep = _verify_rounds(w, MODE_OFFLOAD, seed=12)
    assert refused > 0 and deep > 0
