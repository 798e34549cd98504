"""The error model of the C ABI on the GPU, with every condition forced from the host
(offload page, section "Capacity must survive the session lifecycle": integrity is
checked before the history is trusted).  No test makes a kernel fault or hang: the
injected conditions are either HIP calls that are not made, or slot indices that the
kernels' own bounds checks turn into an error flag."""
import ctypes

import numpy as np
import pytest

import dsa_synth as S
from oracle import MODE_OFFLOAD, MODE_RESIDENT
from tests.parity_util import compare_unit, dev_tensor, gpu_session, load_history, oracle_units, run_step

pytestmark = pytest.mark.gpu


def _note(*a):
    print("[gpu-errors]", *a, flush=True)


def _K():
    import kv_cache_offload_amd as K
    return K


def _small(**kw):
    base = dict(history=4096, rows_per_step=4, steps=8, hot_slots=1024, warm=True)
    base.update(kw)
    return S.WORKLOADS["tiny"].scaled(**base)


def test_create_out_of_memory_leaves_nothing_and_a_smaller_session_works():
    import torch
    K = _K()
    torch.cuda.init()
    free0, total = torch.cuda.mem_get_info()
    # resident rows and keys of 4,194,304 positions are 3.8 GB per unit: 100 units ask
    # for more than the whole HBM, so the session's one device allocation fails
    cfg = K.make_config(max_positions=4_194_304, index_heads=32, heads=64, top_k=2048, hot_slots=1,
                        max_query_rows=8, n_layers=100, mode=K.KV_HBM_RESIDENT)
    _note(f"asking for a session larger than {total / 2**30:.0f} GiB of HBM")
    out = ctypes.c_void_p()
    st = K._lib.dsa_session_create(ctypes.byref(cfg), ctypes.byref(out))
    assert st == K.E_NOMEM and not out.value
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) < 64 << 20, f"free HBM {free0} before, {free1} after the failed create"
    # a session of a workable size is created and steps correctly afterwards
    w = _small()
    sess = gpu_session(w, MODE_OFFLOAD)
    orcs = oracle_units(w, MODE_OFFLOAD)
    load_history(w, sess, orcs)
    gout, oout = run_step(w, 0, 0, sess, orcs)
    compare_unit(sess, orcs[(0, 0)], 0, 0, gout.cpu().numpy()[0], oout[0], what="after a failed create")
    sess.close()


@pytest.mark.parametrize("mode", [MODE_OFFLOAD, MODE_RESIDENT])
def test_decode_before_enough_rows_is_refused_without_change(mode):
    import torch
    K = _K()
    w = _small(history=2)
    sess = gpu_session(w, mode)
    keys, rows = S.history(w, 0, 0)
    sess.append_rows(0, 0, dev_tensor(keys, sess.device), dev_tensor(rows, sess.device))
    iq, iw, ql, qr = (dev_tensor(a[None], sess.device) for a in S.step_queries(w, 0, 0, 0))
    out = torch.zeros((1, w.rows_per_step, w.heads, 512), dtype=torch.float32, device=sess.device)
    with pytest.raises(K.DsaError) as e:
        sess.decode_step(0, iq, iw, ql, qr, out)          # R = 4 query rows, 2 rows held
    assert e.value.status == K.E_STATE
    torch.cuda.synchronize()
    assert sess.unit_state(0, 0) == dict(L=2, M=0 if mode == MODE_OFFLOAD else 2, round=0, row_bytes=656)
    assert torch.count_nonzero(out).item() == 0
    # the refusal is not sticky: with R rows held the step runs
    nk, nr = S.step_rows(w, 0, 0, 0)
    sess.append_rows(0, 0, dev_tensor(nk[:2], sess.device), dev_tensor(nr[:2], sess.device))
    sess.decode_step(0, iq, iw, ql, qr, out)
    torch.cuda.synchronize()
    assert sess.unit_state(0, 0)["round"] == 1 and torch.isfinite(out).all()
    sess.close()


def test_injected_hip_failure_makes_the_session_sticky_failed():
    import torch
    K = _K()
    w = _small()
    sess = gpu_session(w, MODE_OFFLOAD)
    load_history(w, sess)
    keys, rows = S.step_rows(w, 0, 0, 0)
    dk, dr = dev_tensor(keys, sess.device), dev_tensor(rows, sess.device)
    sess.inject("hip_failure")
    with pytest.raises(K.DsaError) as e:
        sess.append_rows(0, 0, dk, dr)                   # its launch is the failing HIP call
    assert e.value.status == K.E_HIP and "injected" in str(e.value)
    assert sess.unit_state(0, 0)["L"] == w.history      # the failed append published nothing
    for call in (lambda: sess.append_rows(0, 0, dk, dr), lambda: sess.flush(0, 0),
                 lambda: sess.mirror_rows(0, 0), lambda: sess.debug("hand")):
        with pytest.raises(K.DsaError) as e:
            call()
        assert e.value.status == K.E_STATE
    torch.cuda.synchronize()
    sess.close()                                         # destroy still frees a failed session


def test_device_side_check_failure_is_reported_and_sticky():
    import torch
    K = _K()
    w = _small()
    sess = gpu_session(w, MODE_OFFLOAD)
    orcs = oracle_units(w, MODE_OFFLOAD)
    load_history(w, sess, orcs)
    # consistent steps raise no flag (the next call would fail otherwise)
    for step in range(2):
        gout, oout = run_step(w, 0, step, sess, orcs)
        compare_unit(sess, orcs[(0, 0)], 0, 0, gout.cpu().numpy()[0], oout[0], what=f"before injection {step}")
    hits = int(sess.debug("counters").cpu().numpy().view(np.int64)[1])
    assert hits > 0, "the warm cache should give hits"
    # every cached position now names slot S + 1: the next step's hits fail the checks
    sess.inject("bad_slot")
    gout, _ = run_step(w, 0, 2, sess)                    # enqueued without error
    torch.cuda.synchronize()
    assert torch.isfinite(gout).all()                    # checked entries were skipped, not read
    with pytest.raises(K.DsaError) as e:
        sess.mirror_rows(0, 0)
    assert e.value.status == K.E_STATE and "hit slot" in str(e.value), str(e.value)
    with pytest.raises(K.DsaError) as e:
        sess.debug("hand")
    assert e.value.status == K.E_STATE
    sess.close()


def test_unknown_injection_and_resident_bad_slot_are_refused():
    K = _K()
    w = _small()
    sess = gpu_session(w, MODE_RESIDENT)
    with pytest.raises(K.DsaError) as e:
        sess.inject(7)
    assert e.value.status == K.E_INVALID
    with pytest.raises(K.DsaError) as e:
        sess.inject("bad_slot")
    assert e.value.status == K.E_UNSUPPORTED
    load_history(w, sess)                                # neither refusal failed the session
    sess.close()


def test_mirror_rows_lag_the_logical_rows_until_flush_and_sync():
    import torch
    w = _small(history=100)
    sess = gpu_session(w, MODE_OFFLOAD)
    keys, rows = S.history(w, 0, 0)
    sess.append_rows(0, 0, dev_tensor(keys, sess.device), dev_tensor(rows, sess.device))
    st = sess.unit_state(0, 0)
    # 100 rows overflow the 68-row ring once: one 64-row batch spilled, 36 rows pending
    assert (st["L"], st["M"]) == (100, 64)
    assert sess.mirror_rows(0, 0) <= 64 < st["L"]
    torch.cuda.synchronize()
    assert sess.mirror_rows(0, 0) == 64
    sess.flush(0, 0)
    assert sess.mirror_rows(0, 0) <= 100
    torch.cuda.synchronize()
    assert sess.mirror_rows(0, 0) == 100
    mirror = sess.debug("mirror").cpu().numpy().reshape(100, 656)
    assert np.array_equal(mirror, rows)
    sess.close()
