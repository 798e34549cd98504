"""GPU parity of quantise-on-append (dsa_quantize_rows, dsa_append_latent) against
the oracle quantiser: packed rows must match byte for byte (the codes are integer
decisions both sides take in fp32), and a unit filled through dsa_append_latent
must step exactly like the oracle unit fed the oracle's packed rows."""
import numpy as np
import pytest

import dsa_synth as S
from oracle import MODE_OFFLOAD, MODE_RESIDENT
from oracle.quantize import quantize_rows
from tests.parity_util import compare_unit, dev_tensor, gpu_session, oracle_units

pytestmark = pytest.mark.gpu


def _note(*a):
    print("[gpu-quantize]", *a, flush=True)


def _latent_inputs(n, seed):
    """bf16 latent [n][512] and RoPE [n][64]: group magnitudes 2^-16..2^11 (normal
    and subnormal scales), with zero, overflowing, lone-value and half-step groups."""
    g = np.random.default_rng(seed)
    mag = 2.0 ** g.integers(-16, 12, size=(n, 8, 1))
    x = g.standard_normal((n, 8, 64)) * mag
    if n >= 8:
        x[0::7, 0, :] = 0.0                                         # zero group
        x[1::7, 1, :] = 3e9 * np.sign(g.standard_normal((len(x[1::7]), 64)))  # scale overflows fp16
        x[2::7, 2, :] = 0.0
        x[2::7, 2, 5] = -2.5                                        # lone value
        j = g.integers(-127, 127, size=(len(x[3::7]), 63))
        x[3::7, 3, 0] = 127 * 0.125                                 # scale 2^-3 exactly
        x[3::7, 3, 1:] = (j + 0.5) * 0.125                          # every other value a tie
    lat = S.bf16_bits(x).reshape(n, 512)
    rope = S.bf16_bits(g.standard_normal((n, 64)))
    return lat, rope


@pytest.mark.parametrize("n", [1, 3, 4099, 40000])
def test_quantize_rows_bytes_match_the_oracle(n):
    import torch
    w = S.WORKLOADS["tiny"]
    sess = gpu_session(w, MODE_OFFLOAD)
    lat, rope = _latent_inputs(n, seed=n)
    out = torch.full((n, 656), 0xAB, dtype=torch.uint8, device=sess.device)
    sess.quantize_rows(dev_tensor(lat, sess.device), dev_tensor(rope, sess.device), out)
    got = out.cpu().numpy()
    want = quantize_rows(lat, rope)
    if not np.array_equal(got, want):
        r, b = np.argwhere(got != want)[0]
        raise AssertionError(f"n={n}: {int(np.sum(np.any(got != want, axis=1)))} rows differ; first row {r} "
                             f"byte {b}: gpu {got[r, b]} oracle {want[r, b]}")
    sess.close()
    _note(f"n={n}: bytes match")


@pytest.mark.parametrize("mode", [pytest.param(MODE_OFFLOAD, id="offload"), pytest.param(MODE_RESIDENT, id="resident")])
def test_append_latent_steps_match_the_oracle(mode):
    import torch
    w = S.WORKLOADS["tiny"].scaled(rows_per_step=4, steps=20, history=3000, warm=True, ring_rows=16)
    sess = gpu_session(w, mode)
    o = oracle_units(w, mode)[(0, 0)]
    # history in two bulk appends (the second spills ring rows to the mirror)
    keys, _ = S.history(w, 0, 0)
    lat, rope = _latent_inputs(w.history, seed=77)
    for a, b in ((0, 1000), (1000, w.history)):
        sess.append_latent(0, 0, dev_tensor(keys[a:b], sess.device), dev_tensor(lat[a:b], sess.device),
                           dev_tensor(rope[a:b], sess.device))
        o.append(keys[a:b], quantize_rows(lat[a:b], rope[a:b]))
    gs, st = sess.unit_state(0, 0), o.state()
    assert (gs["L"], gs["M"]) == (st["L"], st["M"])
    sess.flush(0, 0)
    o.flush()
    sess.warm_hot(0, 0)
    o.warm()
    for step in range(w.steps):
        nk, _ = S.step_rows(w, 0, 0, step)
        nl, nr = _latent_inputs(w.rows_per_step, seed=1000 + step)
        sess.append_latent(0, 0, dev_tensor(nk, sess.device), dev_tensor(nl, sess.device), dev_tensor(nr, sess.device))
        o.append(nk, quantize_rows(nl, nr))
        iq, iw, ql, qr = S.step_queries(w, 0, 0, step)
        out = torch.full((1, w.rows_per_step, w.heads, w.latent_dim), float("nan"), dtype=torch.float32,
                         device=sess.device)
        sess.decode_step(0, dev_tensor(iq[None], sess.device), dev_tensor(iw[None], sess.device),
                         dev_tensor(ql[None], sess.device), dev_tensor(qr[None], sess.device), out)
        oout = o.decode_step(iq, iw, ql, qr)
        compare_unit(sess, o, 0, 0, out.cpu().numpy()[0], oout, what=f"append_latent mode={mode} step={step}")
    sess.flush(0, 0)
    o.flush()
    torch.cuda.synchronize()
    mirror = sess.debug("mirror", 0, 0).cpu().numpy().reshape(-1, 656)
    assert np.array_equal(mirror, o.mirror())
    sess.close()
    _note(f"mode={mode}: {w.steps} steps match")
