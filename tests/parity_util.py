"""Drive the HIP path (through the C ABI binding) and the CPU oracle on the same
seeded inputs, and compare them.  Used by the GPU parity tests and smoke()."""
from __future__ import annotations

import numpy as np

import dsa_synth as S
from oracle import MODE_OFFLOAD, MODE_RESIDENT, OracleUnit, UnitShape

# attention tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle|, element by element
ATOL, RTOL = 2e-3, 1e-2
HIST_CHUNK = 65536          # rows per append call when loading history


def _torch():
    import torch
    return torch


def dev_tensor(a: np.ndarray, device):
    torch = _torch()
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def oracle_units(w: S.Workload, mode: int, layers=None, seqs=None, replacement=0):
    layers = range(w.layers) if layers is None else layers
    seqs = range(w.seqs) if seqs is None else seqs
    shape = UnitShape(max_positions=w.max_positions, index_heads=w.index_heads, index_dim=w.index_dim,
                      heads=w.heads, top_k=w.top_k, hot_slots=w.hot_slots, max_query_rows=w.rows_per_step,
                      latent_dim=w.latent_dim, rope_dim=w.rope_dim, group=w.group, ring_rows=w.ring_rows,
                      mode=mode, softmax_scale=w.softmax_scale, replacement=replacement)
    return {(l, q): OracleUnit(shape) for l in layers for q in seqs}


def gpu_session(w: S.Workload, mode: int, n_layers=None, replacement=0):
    import kv_cache_offload_amd as K
    cfg = K.make_config(max_positions=w.max_positions, index_heads=w.index_heads, heads=w.heads,
                        top_k=w.top_k, hot_slots=w.hot_slots, max_query_rows=w.rows_per_step,
                        n_layers=w.layers if n_layers is None else n_layers, n_seqs=w.seqs,
                        index_dim=w.index_dim, ring_rows=w.ring_rows, softmax_scale=w.softmax_scale,
                        mode=K.KV_OFFLOAD if mode == MODE_OFFLOAD else K.KV_HBM_RESIDENT,
                        replacement=replacement)
    return K.Session(cfg)


def load_history(w, sess=None, orcs=None, layers=(0,), seqs=None, warm=None, history_fn=None):
    """Append the pre-step history of each unit, flush, and warm the caches."""
    seqs = range(w.seqs) if seqs is None else seqs
    warm = w.warm if warm is None else warm
    history_fn = history_fn or S.history
    for gl, l in enumerate(layers):
        for q in seqs:
            keys, rows = history_fn(w, l, q)
            if orcs is not None:
                o = orcs[(l, q)]
                o.append(keys, rows)
                o.flush()
                if warm:
                    o.warm()
            if sess is not None:
                for c in range(0, keys.shape[0], HIST_CHUNK):
                    sess.append_rows(gl, q, dev_tensor(keys[c:c + HIST_CHUNK], sess.device),
                                     dev_tensor(rows[c:c + HIST_CHUNK], sess.device))
                sess.flush(gl, q)
                if warm:
                    sess.warm_hot(gl, q)


def step_inputs(w, layer, step, seqs=None, rows_fn=None, query_fn=None):
    """Per-sequence appended rows and queries of one step, stacked over sequences."""
    seqs = range(w.seqs) if seqs is None else seqs
    rows_fn = rows_fn or S.step_rows
    query_fn = query_fn or S.step_queries
    new = [rows_fn(w, layer, q, step) for q in seqs]
    qs = [query_fn(w, layer, q, step) for q in seqs]
    stack = lambda i: np.stack([x[i] for x in qs])
    return new, (stack(0), stack(1), stack(2), stack(3))


def run_step(w, layer, step, sess=None, orcs=None, gpu_layer=None, seqs=None, rows_fn=None, query_fn=None,
             combined=False):
    """Append the step's rows and run one decode step on both sides (combined: on the GPU side through
    dsa_append_decode_step, one call for every sequence; the oracle still appends, then decodes).
    Returns (gpu_out numpy [n_seqs][R][H][512] or None, {seq: oracle_out})."""
    seqs = list(range(w.seqs) if seqs is None else seqs)
    new, (iq, iw, ql, qr) = step_inputs(w, layer, step, seqs, rows_fn, query_fn)
    gl = layer if gpu_layer is None else gpu_layer
    gout = None
    if sess is not None:
        torch = _torch()
        out = torch.full((len(seqs), w.rows_per_step, w.heads, w.latent_dim), float("nan"),
                         dtype=torch.float32, device=sess.device)
        q_dev = [dev_tensor(x, sess.device) for x in (iq, iw, ql, qr)]
        if combined:
            assert seqs == list(range(w.seqs)), "the combined call appends to every sequence"
            keys = dev_tensor(np.stack([x[0] for x in new]), sess.device)
            rows = dev_tensor(np.stack([x[1] for x in new]), sess.device)
            sess.append_decode_step(gl, keys, rows, *q_dev, out)
        else:
            for i, q in enumerate(seqs):
                sess.append_rows(gl, q, dev_tensor(new[i][0], sess.device), dev_tensor(new[i][1], sess.device))
            sess.decode_step(gl, *q_dev, out)
        gout = out
    oout = {}
    if orcs is not None:
        for i, q in enumerate(seqs):
            o = orcs[(layer, q)]
            o.append(*new[i])
            oout[q] = o.decode_step(iq[i], iw[i], ql[i], qr[i])
    return gout, oout


def gpu_items(sess, layer, seq, R, K, S_, L, row_bytes=656):
    """Fetch the step and state items of one unit as numpy arrays."""
    torch = _torch()
    torch.cuda.synchronize()
    get = lambda name: sess.debug(name, layer, seq).cpu().numpy()
    d = {}
    d["scores"] = get("scores").view(np.float32).reshape(R, L)
    d["selection"] = get("selection").view(np.int32).reshape(R, K)
    d["sel_count"] = get("sel_count").view(np.int32)
    cnt = get("counters").view(np.int64)
    d["counters"] = cnt
    U = int(cnt[0])
    d["union"] = get("union").view(np.int32)[:U]
    d["kind"] = get("union_kind").view(np.int32)[:U]
    d["src"] = get("union_src").view(np.int32)[:U]
    d["map"] = get("map").view(np.int32).reshape(R, K)
    d["compact"] = get("compact").reshape(-1, row_bytes)[:U]
    if S_:
        d["slot_pos"] = get("slot_pos").view(np.int32)
        d["fill_round"] = get("fill_round").view(np.int32)
        d["pin_round"] = get("pin_round").view(np.int32)
        d["pos_slot"] = get("pos_slot").view(np.int32)
        d["hand"] = int(get("hand").view(np.int32)[0])
        words = get("ref_bits").view(np.uint32)
        d["ref"] = ((words[:, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8).reshape(-1)[:S_]
    return d


def compare_unit(sess, o: OracleUnit, gl: int, seq: int, gout, oout, check_scores=True, what=""):
    """Assert bit-exact discrete state and in-tolerance outputs for one unit after a step."""
    st = o.state()
    R, L = st["R"], st["L"]
    K = o.shape.top_k
    S_ = o.shape.hot_slots if o.shape.mode == MODE_OFFLOAD else 0
    g = gpu_items(sess, gl, seq, R, K, S_, L)
    gs = sess.unit_state(gl, seq)
    assert (gs["L"], gs["M"], gs["round"]) == (st["L"], st["M"], st["round"]), what
    if check_scores:
        os_ = o.scores()
        for r in range(R):
            nv = L - R + r + 1
            a, b = g["scores"][r, :nv], os_[r, :nv]
            if not np.array_equal(a.view(np.uint32), b.view(np.uint32)):
                bad = np.nonzero(a.view(np.uint32) != b.view(np.uint32))[0]
                raise AssertionError(f"{what} scores row {r}: {len(bad)} differ, first at t={bad[0]}: "
                                     f"gpu {a[bad[0]]} oracle {b[bad[0]]}")
    osel, ocnt = o.selection()
    assert np.array_equal(g["sel_count"], ocnt), what
    for r in range(R):
        if not np.array_equal(g["selection"][r], osel[r]):
            diff = np.setdiff1d(g["selection"][r], osel[r])
            raise AssertionError(f"{what} selection row {r} differs ({len(diff)} positions)")
    uni, kind, src = o.union()
    assert np.array_equal(g["union"], uni), f"{what} union differs"
    assert np.array_equal(g["kind"], kind), f"{what} union kinds differ"
    assert np.array_equal(g["src"], src), f"{what} union sources differ"
    assert np.array_equal(g["map"], o.map()), f"{what} map differs"
    assert np.array_equal(g["compact"], o.compact()), f"{what} compact bytes differ"
    oc = o.counters()
    names = ("union", "hit", "ring", "miss", "miss_noslot", "evict", "host_bytes", "res", "host_reads")
    assert [int(x) for x in g["counters"]] == [oc[k] for k in names], f"{what} counters differ"
    if S_:
        sp, fr, pr = o.slots()
        assert np.array_equal(g["slot_pos"], sp), f"{what} slot_pos differs"
        assert np.array_equal(g["fill_round"], fr), f"{what} fill_round differs"
        assert np.array_equal(g["pin_round"], pr), f"{what} pin_round differs"
        assert np.array_equal(g["pos_slot"], o.pos_slot()), f"{what} pos_slot differs"
        assert g["hand"] == st["hand"], f"{what} hand differs"
        if not np.array_equal(g["ref"], o.ref()):
            bad = np.nonzero(g["ref"] != o.ref())[0]
            raise AssertionError(f"{what} reference bits differ at {len(bad)} slots, first {bad[0]}")
    if gout is not None:
        ref = oout.astype(np.float64)
        got = gout.astype(np.float64)
        assert np.all(np.isfinite(got)), f"{what} non-finite outputs"
        err = np.abs(got - ref)
        ok = err <= ATOL + RTOL * np.abs(ref)
        if not ok.all():
            i = np.argmax(err - (ATOL + RTOL * np.abs(ref)))
            raise AssertionError(f"{what} attention out of tolerance at {np.unravel_index(i, ref.shape)}: "
                                 f"gpu {got.flat[i]} oracle {ref.flat[i]} (max abs err {err.max():.3g})")
    return g


def attention_error(gout, oout):
    ref = oout.astype(np.float64)
    err = np.abs(gout.astype(np.float64) - ref)
    rel = err[np.abs(ref) > 1e-3] / np.abs(ref[np.abs(ref) > 1e-3])
    return float(err.max()), float(rel.max()) if rel.size else 0.0
