"""dsa_decode_step_static (the decode step whose scratch is a static device array, for
callers that cannot allocate) against dsa_decode_step, through the C ABI.

Two sessions take the same inputs; one steps with dsa_decode_step, the other with
dsa_decode_step_static.  The outputs must agree within the attention tolerance (they are
the same kernels, so in practice bit for bit) and the cache state bit for bit.  Two calls
in a row share the static array: first the 50,023-row single stream with 4 query rows,
then a smaller session (4,096 rows, 1 query row, 16 heads), whose step must not see
what the larger call left in the array.
"""
import numpy as np
import pytest

import dsa_synth as S
from oracle import MODE_OFFLOAD
from tests.parity_util import ATOL, RTOL, dev_tensor, gpu_session, load_history, step_inputs

pytestmark = pytest.mark.gpu

STATE_ITEMS = ("slot_pos", "fill_round", "pin_round", "pos_slot", "hand", "slot_bytes", "totals", "mirror")


def _note(*a):
    print("[no-alloc]", *a, flush=True)


def _pair(w):
    reg, sta = gpu_session(w, MODE_OFFLOAD), gpu_session(w, MODE_OFFLOAD)
    load_history(w, reg)
    load_history(w, sta)
    return reg, sta


def _step(w, step, sess, static):
    import torch
    new, (iq, iw, ql, qr) = step_inputs(w, 0, step)
    for q in range(w.seqs):
        sess.append_rows(0, q, dev_tensor(new[q][0], sess.device), dev_tensor(new[q][1], sess.device))
    out = torch.full((w.seqs, w.rows_per_step, w.heads, w.latent_dim), float("nan"), dtype=torch.float32,
                     device=sess.device)
    args = (0, dev_tensor(iq, sess.device), dev_tensor(iw, sess.device), dev_tensor(ql, sess.device),
            dev_tensor(qr, sess.device), out)
    (sess.decode_step_static if static else sess.decode_step)(*args)
    return out


def _compare(w, reg, sta, go, gs, what):
    import torch
    torch.cuda.synchronize()
    a, b = go.cpu().numpy().astype(np.float64), gs.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(b)), f"{what}: non-finite outputs"
    assert np.all(np.abs(a - b) <= ATOL + RTOL * np.abs(a)), f"{what}: outputs differ"
    assert np.array_equal(a, b), f"{what}: outputs differ in bits (same kernels, same inputs)"
    assert reg.unit_state(0, 0) == sta.unit_state(0, 0), what
    for item in STATE_ITEMS:
        x, y = reg.debug(item).cpu().numpy(), sta.debug(item).cpu().numpy()
        assert np.array_equal(x, y), f"{what}: {item} differs"


def test_static_step_matches_the_session_step_twice_then_smaller():
    import kv_cache_offload_amd as K
    big = S.WORKLOADS["single_stream_50k"].scaled(steps=8)
    small = S.WORKLOADS["tiny"].scaled(steps=4)
    reg, sta = _pair(big)
    for step in range(2):
        go, gs = _step(big, step, reg, False), _step(big, step, sta, True)
        _compare(big, reg, sta, go, gs, f"50,023 rows, step {step}")
        _note(f"50,023-row step {step}: static == session scratch")
    with pytest.raises(K.DsaError) as e:                 # step items are not kept for a static step
        sta.debug("selection")
    assert e.value.status == K.E_STATE
    reg.close()
    sta.close()
    # a smaller call on the same static array, after the larger one
    reg, sta = _pair(small)
    for step in range(2):
        go, gs = _step(small, step, reg, False), _step(small, step, sta, True)
        _compare(small, reg, sta, go, gs, f"4,096 rows, step {step}")
        _note(f"4,096-row step {step}: static == session scratch")
    # a session step after a static one keeps its items again
    _step(small, 2, sta, False)
    assert sta.debug("sel_count").numel() == 4
    reg.close()
    sta.close()


def test_static_step_refuses_a_layer_larger_than_the_array():
    import torch
    import kv_cache_offload_amd as K
    # 1,048,576 positions with 8 query rows: the scores and Top-K candidates alone are 96 MiB
    w = S.WORKLOADS["million"].scaled(history=8, rows_per_step=8, steps=131_071)
    sess = gpu_session(w, MODE_OFFLOAD)
    keys, rows = S.history(w.scaled(history=8), 0, 0)
    sess.append_rows(0, 0, dev_tensor(keys, sess.device), dev_tensor(rows, sess.device))
    _, (iq, iw, ql, qr) = step_inputs(w, 0, 0)
    out = torch.zeros((1, 8, w.heads, 512), dtype=torch.float32, device=sess.device)
    with pytest.raises(K.DsaError) as e:
        sess.decode_step_static(0, *(dev_tensor(x, sess.device) for x in (iq, iw, ql, qr)), out)
    assert e.value.status == K.E_UNSUPPORTED and "static scratch" in str(e.value)
    assert sess.unit_state(0, 0)["round"] == 0 and torch.count_nonzero(out).item() == 0
    sess.close()
