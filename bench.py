#!/usr/bin/env python3
"""Benchmark: DSA sparse-attention decode steps over an offloaded MLA history on one MI355X.

One step = append the step's R new rows (index keys to HBM, Q8G64 rows into the
recent ring) + one decode step (index score over every history position, exact
Top-K, hot-cache gather with host-mirror misses, absorbed-MLA attention over the
selected rows, 64-row batched writeback), for the 50,023-row single-stream
workload (R = 4 query rows, Top-2048, 32,768 hot slots, H_I = 32, H = 64).
All inputs are synthetic, seeded, and resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the timed region's throughput, with no
events in it.  Per-kernel durations come from HIP events that the library
attaches to the kernels' own dispatches (hipExtLaunchKernel start/stop events
on the launch stream) over a second timed pass of the same length that
continues the same workload; they agree with a rocprofv3 kernel trace.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode steps/s at 50,023 history (query rows/s; % HBM roofline)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
HOST_LINK_PEAK_GBPS = 64.0      # PCIe Gen5 x16, one direction, nominal
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1024)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--workload", default="single_stream_50k")
    p.add_argument("--kernel-steps", type=int, default=1024, help="steps of the pass with per-kernel events")
    p.add_argument("--no-resident", action="store_true", help="skip the HBM-resident comparison run")
    p.add_argument("--resident-only", action="store_true",
                   help="run the HBM-resident session alone (counter runs of that mode); the line reports it")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--calib-copy", action="store_true", help="also run a plain 2 GiB device copy (PMC scaling)")
    p.add_argument("--replacement", choices=("ring", "clock"), default="ring",
                   help="hot-cache replacement policy of the offloaded run")
    p.add_argument("--replacement-probe", action="store_true",
                   help="instead of the throughput run: time the first decode step after a warm start (full "
                        "cache, every reference bit set) and the steps after it, under both policies")
    p.add_argument("--reuse-probe", action="store_true",
                   help="instead of the throughput run: layer 0 selects, the other layers reuse its "
                        "selection; steps/s without and with prefetch on a second stream, and resident")
    p.add_argument("--quantize-rows", type=int, default=1 << 20,
                   help="rows of the quantise-on-append measurement (0 skips it)")
    p.add_argument("--separate-append", action="store_true",
                   help="append with dsa_append_rows and decode with dsa_decode_step (an append launch per "
                        "sequence and layer step) instead of one dsa_append_decode_step call")
    p.add_argument("--pairs", type=int, default=3,
                   help="the timed steps of each mode are split into this many segments, offload and resident "
                        "interleaved with the order alternating from pair to pair")
    return p.parse_args()


# Source file of each kernel group (the PMC traffic of a group is reported only
# while its source is the one the counters were taken on).
KERNEL_SOURCES = {"index_score": "k_score.hip", "topk_collect": "k_topk.hip", "topk_resolve": "k_topk.hip",
                  "gather": "k_gather.hip", "attention": "k_attn.hip", "attention_merge": "k_attn.hip",
                  "append": "k_gather.hip"}
# rocprofv3 kernel names of each group
KERNEL_NAMES = {"index_score": ("score_kernel",), "topk_collect": ("topk_refine_kernel", "topk_digits_kernel"),
                "topk_resolve": ("topk_chunk_kernel", "topk_final_kernel"), "gather": ("gather_assign_kernel",),
                "attention": ("attn_kernel",), "attention_merge": ("attn_merge_kernel",), "append": ("append_kernel",)}
# (decode steps run the assign pass inside the merge launch; gather_assign_kernel is the prefetch rounds')
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def source_hash(kind):
    """Hash of a kernel group's source file and of every header the kernels include."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "kv_cache_offload_amd", "csrc")
    h = hashlib.sha256()
    for path in [os.path.join(csrc, KERNEL_SOURCES[kind])] + sorted(glob.glob(os.path.join(csrc, "*.h"))):
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def pmc_traffic(workload, kind):
    """HBM bytes per launch of a kernel group from the committed counter summary, or None."""
    try:
        d = json.load(open(PMC_FILE))[workload][kind]
    except (OSError, KeyError, ValueError):
        return None
    return d["bytes_per_launch"] if d.get("source_sha256_16") == source_hash(kind) else None


def pmc_summary(workload, fetch_csv, write_csv):
    """Write profiles/pmc_traffic.json from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE), each scaled by
    what the counter reads for the 2 GiB device copy of the same run (--calib-copy)."""
    import csv
    import re

    def per_kernel(path, counter):
        # bytes per launch of a group: per kernel, the median dispatch times its dispatches per group
        # launch (the fewest dispatches of any one of the group's kernels: the Top-K collect group runs
        # its digits kernel twice per launch); the median keeps the history load's bulk appends out
        vals, calib = {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0
            if "copyBuffer" in name and int(r["Grid_Size"]) >= 131072:
                calib.append(v)
                continue
            for kind, names in KERNEL_NAMES.items():
                for n in names:
                    if re.search(r"\b" + n + r"\b", name):
                        vals.setdefault(kind, {}).setdefault(n, []).append(v)
        assert calib, f"no calibration copy in {path}"
        factor = (2 << 30) / (sum(calib) / len(calib))
        out = {}
        steps = min(len(v) for v in vals.get("index_score", {"": [0]}).values())
        for k, by_name in vals.items():
            launches = min(len(v) for v in by_name.values())
            if k == "append" and launches < steps:         # only the history load's bulk appends: the steps
                continue                                   # appended inside dsa_append_decode_step
            out[k] = factor * sum(sorted(v)[len(v) // 2] * len(v) / launches for v in by_name.values())
        return out, factor

    f, ff = per_kernel(fetch_csv, "FETCH_SIZE")
    w, wf = per_kernel(write_csv, "WRITE_SIZE")
    try:
        out = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        out = {}
    out[workload] = {k: {"fetch_bytes": f.get(k, 0.0), "write_bytes": w.get(k, 0.0),
                         "bytes_per_launch": f.get(k, 0.0) + w.get(k, 0.0), "fetch_scale": ff, "write_scale": wf,
                         "source_sha256_16": source_hash(k)} for k in sorted(set(f) | set(w))}
    json.dump(out, open(PMC_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps(out[workload], indent=1))


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def dev_tensor(a, device):
    """numpy array -> device tensor with the same bytes (bf16 bit patterns travel as int16)."""
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def make_session(w, mode, n_layers=None, replacement=0):
    import kv_cache_offload_amd as K
    cfg = K.make_config(max_positions=w.max_positions, index_heads=w.index_heads, heads=w.heads,
                        top_k=w.top_k, hot_slots=w.hot_slots, max_query_rows=w.rows_per_step,
                        n_layers=w.layers if n_layers is None else n_layers, n_seqs=w.seqs,
                        softmax_scale=w.softmax_scale, mode=mode, replacement=replacement)
    return K.Session(cfg)


def gen_inputs(w, n_steps):
    """Every step's appended rows and queries, per layer, stacked over sequences."""
    import dsa_synth as S
    R, Q, NL = w.rows_per_step, w.seqs, w.layers
    keys = np.empty((n_steps, NL, Q, R, w.index_dim), np.uint16)
    rows = np.empty((n_steps, NL, Q, R, w.row_bytes), np.uint8)
    iq = np.empty((n_steps, NL, Q, R, w.index_heads, w.index_dim), np.uint16)
    iw = np.empty((n_steps, NL, Q, R, w.index_heads), np.float32)
    ql = np.empty((n_steps, NL, Q, R, w.heads, w.latent_dim), np.uint16)
    qr = np.empty((n_steps, NL, Q, R, w.heads, w.rope_dim), np.uint16)
    for s in range(n_steps):
        for l in range(NL):
            for q in range(Q):
                keys[s, l, q], rows[s, l, q] = S.step_rows(w, l, q, s)
                iq[s, l, q], iw[s, l, q], ql[s, l, q], qr[s, l, q] = S.step_queries(w, l, q, s)
    return keys, rows, iq, iw, ql, qr


class Runner:
    """One session (every layer and sequence of the workload) with every step's
    inputs already in HBM; calls the C ABI directly.  One step = for each layer
    in order: append R rows to each sequence, then one decode step of the layer
    (all sequences together) -- one dsa_append_decode_step call, or, with
    separate_append, dsa_append_rows per sequence and then dsa_decode_step."""

    def __init__(self, w, mode, host_inputs, replacement=0, separate_append=False):
        import torch
        import dsa_synth as S
        import kv_cache_offload_amd as K
        self.K, self.torch, self.w = K, torch, w
        self.combined = not separate_append
        self.sess = make_session(w, mode, replacement=replacement)
        dev = self.sess.device
        for l in range(w.layers):
            for q in range(w.seqs):
                hk, hr = S.history(w, l, q)
                for c in range(0, hk.shape[0], 65536):
                    self.sess.append_rows(l, q, dev_tensor(hk[c:c + 65536], dev), dev_tensor(hr[c:c + 65536], dev))
                self.sess.flush(l, q)
                if mode == K.KV_OFFLOAD and w.warm:
                    self.sess.warm_hot(l, q)
                torch.cuda.synchronize()
        self.d = [dev_tensor(a, dev) for a in host_inputs]
        self.out = torch.empty((w.seqs, w.rows_per_step, w.heads, w.latent_dim), dtype=torch.float32, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        keys, rows, iq, iw, ql, qr = self.d
        self.ptr = [[tuple(int(t[s, l].data_ptr()) for t in self.d) for l in range(w.layers)]
                    for s in range(keys.shape[0])]
        self.h = self.sess.h
        self.next = 0
        torch.cuda.synchronize()

    def steps(self, n):
        K, R, lib, w = self.K, self.w.rows_per_step, self.K._lib, self.w
        out = ctypes.c_void_p(self.out.data_ptr())
        kb, rb = w.index_dim * 2 * R, w.row_bytes * R          # bytes of one sequence's appended keys / rows
        for _ in range(n):
            for l, (pk, pr, piq, piw, pql, pqr) in enumerate(self.ptr[self.next]):
                if self.combined:
                    st = lib.dsa_append_decode_step(self.h, l, R, ctypes.c_void_p(pk), ctypes.c_void_p(pr),
                                                    ctypes.c_void_p(piq), ctypes.c_void_p(piw), ctypes.c_void_p(pql),
                                                    ctypes.c_void_p(pqr), out, self.stream)
                    if st != K.OK:
                        raise K.DsaError("dsa_append_decode_step", st, K.dsa_last_error(self.h))
                    continue
                for q in range(w.seqs):
                    st = lib.dsa_append_rows(self.h, l, q, R, ctypes.c_void_p(pk + q * kb), ctypes.c_void_p(pr + q * rb),
                                             self.stream)
                    if st != K.OK:
                        raise K.DsaError("dsa_append_rows", st, K.dsa_last_error(self.h))
                st = lib.dsa_decode_step(self.h, l, R, ctypes.c_void_p(piq), ctypes.c_void_p(piw),
                                         ctypes.c_void_p(pql), ctypes.c_void_p(pqr), out, self.stream)
                if st != K.OK:
                    raise K.DsaError("dsa_decode_step", st, K.dsa_last_error(self.h))
            self.next += 1

    def totals(self):
        """Step counters summed over every unit."""
        self.torch.cuda.synchronize()
        t = np.zeros(9, np.int64)
        for l in range(self.w.layers):
            for q in range(self.w.seqs):
                t += self.sess.debug("totals", l, q).cpu().numpy().view(np.int64)
        return t

    def L(self):
        return self.sess.unit_state(0, 0)["L"]


def timed(runner, n):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    runner.steps(n)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def algorithmic_bytes(w, kind, n_steps, L0, cnt, long_hist, combined=False):
    """Bytes each kernel group must move per launch (one layer, every sequence),
    averaged over the timed steps.

    Scratch that only the implementation needs (scores, histograms, split-K
    partials) is not counted, except where the kernel's whole job is to move it
    (the partial top-k pass and the attention merge).
    """
    R, K, H, Q = w.rows_per_step, w.top_k, w.heads, w.seqs
    launches = n_steps * w.layers
    Lmean = L0 + R * (n_steps + 1) / 2.0
    rb = w.row_bytes
    U = cnt[0] / launches
    hit, ring, miss, noslot = (cnt[i] / launches for i in (1, 2, 3, 4))
    wb = Q * w.ring_rows * rb * 2 * R / w.ring_rows      # 64-row writeback every 64/R steps, read + write
    if kind == "index_score":                           # every key once (+ the appended rows in one call)
        return Q * Lmean * w.index_dim * 2 + (Q * R * (w.index_dim * 2 + rb) * 2 if combined else 0)
    if kind == "topk_collect":
        return Q * R * Lmean * 4 * (2 if long_hist else 1)
    if kind == "topk_resolve":
        return Q * R * Lmean * 4 + Q * R * K * 4          # the scores once, the selection out
    assign = U * (16 + 12) + miss * (8 + 16) + wb
    if kind == "gather":
        # union bookkeeping: descriptor + union arrays per entry, victim and slot-table entries per miss
        return assign
    if kind == "attention":
        # every distinct selected row read once from its source (slot, ring, host mirror, HBM row store),
        # its compact copy and the misses' slot fills written, the queries read
        return U * rb + U * rb + miss * rb + Q * R * H * (512 + 64) * 2
    if kind == "attention_merge":
        # the merged output, and the assign pass that runs in the same launch
        return Q * R * H * 512 * 4 + assign
    if kind == "append":
        return Q * R * (w.index_dim * 2 + rb) * 2
    return 0.0


def kernel_pass(r, w, args):
    """Per-kernel durations: the same workload continues with the library's
    dispatch events on (their host-side cost would distort the timed region)."""
    kc_before = r.totals()
    kL0 = r.L()
    r.sess.set_kernel_timing(True, reserve_steps=args.kernel_steps * w.layers)
    dt_ev = timed(r, args.kernel_steps)
    kt = r.sess.kernel_times()
    r.sess.set_kernel_timing(False)
    kc = r.totals() - kc_before
    long_hist = r.L() > 65536
    kernels = {k: dict(launches=c, avg_us=(m / c * 1e3) if c else 0.0,
                       bytes_per_launch=algorithmic_bytes(w, k, args.kernel_steps, kL0, kc, long_hist,
                                                          r.combined))
               for k, (c, m) in kt.items() if c}
    for v in kernels.values():
        v["GBps"] = v["bytes_per_launch"] / (v["avg_us"] * 1e-6) / 1e9 if v["avg_us"] > 0 else 0.0
    return dict(steps_per_s_with_kernel_events=args.kernel_steps / dt_ev, kernel_steps=args.kernel_steps,
                kernels=kernels, kernel_counters=kc.tolist())


def run_pairs(w, inputs, args):
    """The offloaded session (and, unless --no-resident, the resident one) over the
    same inputs.  The timed steps of each mode are split into --pairs segments,
    run offload/resident interleaved with the order alternating from pair to pair
    (the offload page, section "Six interleaved pairs": the same binary, the order
    alternated per restart), so a drift of the machine during the run falls on
    both modes alike.  Returns one result per mode."""
    import kv_cache_offload_amd as K
    modes = [("offload", K.KV_OFFLOAD)] + ([] if args.no_resident else [("resident", K.KV_HBM_RESIDENT)])
    if args.resident_only:
        modes = [("resident", K.KV_HBM_RESIDENT)]
    repl = K.REPL_CLOCK if args.replacement == "clock" else K.REPL_RING
    runners, res = {}, {}
    for name, mode in modes:
        runners[name] = Runner(w, mode, inputs, replacement=repl, separate_append=args.separate_append)
        log(f"{name}: history loaded (L={runners[name].L()}), warmup {args.warmup}")
        runners[name].steps(args.warmup)
        res[name] = dict(seconds=0.0, steps=0, L_start=runners[name].L(), counters=np.zeros(9, np.int64),
                         segments=[])
    P = max(1, min(args.pairs, args.steps))
    sizes = [args.steps // P + (1 if i < args.steps % P else 0) for i in range(P)]
    names = [n for n, _ in modes]
    for p, n_seg in enumerate(sizes):
        for name in (names if p % 2 == 0 else names[::-1]):
            r = runners[name]
            c0 = r.totals()
            dt = timed(r, n_seg)
            res[name]["counters"] += r.totals() - c0
            res[name]["seconds"] += dt
            res[name]["steps"] += n_seg
            res[name]["segments"].append(round(n_seg / dt, 2))
    for name in names:
        x = res[name]
        x["steps_per_s"] = x["steps"] / x["seconds"]
        x["counters"] = x["counters"].tolist()
        log(f"{name}: {x['steps']} steps in {x['seconds'] * 1e3:.1f} ms ({x['steps_per_s']:.1f} steps/s; "
            f"segments {x['segments']})")
    for name in names:
        res[name].update(kernel_pass(runners[name], w, args))
        runners[name].sess.close()
    return res


def environment():
    """Read-only record of the host and software the run used."""
    import torch

    def read(path):
        try:
            return open(path).read().strip()
        except OSError:
            return None
    cpu = None
    try:
        cpu = next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")), None)
    except OSError:
        pass
    return {"cpu_model": cpu, "host_threads": len(os.sched_getaffinity(0)),
            "kernel.numa_balancing": read("/proc/sys/kernel/numa_balancing"),
            "vm.compaction_proactiveness": read("/proc/sys/vm/compaction_proactiveness"),
            "rocm": read("/opt/rocm/.info/version"), "torch": torch.__version__, "hip": torch.version.hip,
            "gpu": torch.cuda.get_device_name(0)}


def replacement_probe(w, inputs, args):
    """The replacement A/B of the offload page ("GPU cache management errs too"):
    with a full cache and every reference bit set (a warm start), the first
    decode step of each layer makes CLOCK's hand clear a whole lap before it
    takes a slot; the ring walk takes the next unpinned slot.  Per policy: the
    kernels of that first step (every layer once) and of the steady steps after
    it, from the library's dispatch events."""
    import kv_cache_offload_amd as K
    out = {}
    for name, pol in (("ring", K.REPL_RING), ("clock", K.REPL_CLOCK)):
        r = Runner(w, K.KV_OFFLOAD, inputs, replacement=pol)
        log(f"replacement probe, {name}: history loaded and warmed")
        res = {}
        for phase, n in (("first_step_after_warm", 1), ("steady", args.steps)):
            r.sess.set_kernel_timing(True, reserve_steps=n * w.layers)
            c0 = r.totals()
            dt = timed(r, n)
            kt = r.sess.kernel_times()
            r.sess.set_kernel_timing(False)
            c = (r.totals() - c0).tolist()
            res[phase] = {"steps": n, "layer_steps": n * w.layers, "ms_per_step_with_events": dt * 1e3 / n,
                          "kernels_us": {k: round(m / cnt * 1e3, 2) for k, (cnt, m) in kt.items() if cnt},
                          "misses_per_layer_step": (c[3] + c[4]) / (n * w.layers),
                          "evictions_per_layer_step": c[5] / (n * w.layers)}
        r.sess.close()
        out[name] = res
    return out


def reuse_probe(w, inputs, args):
    """Selection reuse (offload page, "Starting point") and prefetch (first
    decision).  One step: append every layer's rows, a full decode step of layer
    0, then a reuse step of every other layer on layer 0's selection.  With
    prefetch, each reusing layer's prefetch round is enqueued on a second stream
    right after layer 0's step (the library makes it wait for layer 0's Top-K,
    and each reuse step wait for its layer's prefetch); the host-link reads of
    the reusing layers' misses then overlap layer 0's gather and attention and
    the earlier reuse steps."""
    import torch
    import kv_cache_offload_amd as K
    R = w.rows_per_step
    res = {}
    for name, mode, pf in (("offload", K.KV_OFFLOAD, False), ("offload_prefetch", K.KV_OFFLOAD, True),
                           ("resident", K.KV_HBM_RESIDENT, False)):
        r = Runner(w, mode, inputs)
        lib, h, main = K._lib, r.h, r.stream
        side = torch.cuda.Stream(device=r.sess.device)
        side_h = ctypes.c_void_p(side.cuda_stream)
        out = ctypes.c_void_p(r.out.data_ptr())
        kb, rb = w.index_dim * 2 * R, w.row_bytes * R

        def check(st, what):
            if st != K.OK:
                raise K.DsaError(what, st, K.dsa_last_error(h))

        def step():
            ptr = r.ptr[r.next]
            for l, (pk, pr, _, _, _, _) in enumerate(ptr):
                check(lib.dsa_append_rows(h, l, 0, R, ctypes.c_void_p(pk), ctypes.c_void_p(pr), main), "append")
            _, _, piq, piw, pql, pqr = ptr[0]
            check(lib.dsa_decode_step(h, 0, R, ctypes.c_void_p(piq), ctypes.c_void_p(piw), ctypes.c_void_p(pql),
                                      ctypes.c_void_p(pqr), out, main), "decode")
            if pf:                                   # the library orders them with its own events
                for l in range(1, w.layers):
                    check(lib.dsa_prefetch_reuse(h, l, 0, R, side_h), "prefetch")
            for l in range(1, w.layers):
                _, _, _, _, pql, pqr = ptr[l]
                check(lib.dsa_decode_step_reuse(h, l, 0, R, ctypes.c_void_p(pql), ctypes.c_void_p(pqr), out, main),
                      "reuse")
            r.next += 1

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        c0 = r.totals()
        host = 0.0
        t0 = time.perf_counter()
        for _ in range(args.steps):
            th = time.perf_counter()
            step()
            host += time.perf_counter() - th
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        c = (r.totals() - c0).tolist()
        res[name] = {"steps_per_s": args.steps / dt, "ms_per_step": dt * 1e3 / args.steps,
                     "host_enqueue_us_per_step": host * 1e6 / args.steps,
                     "hits_per_step": c[1] / args.steps, "misses_per_step": (c[3] + c[4]) / args.steps,
                     "host_bytes_per_step": c[6] / args.steps}
        log(f"reuse probe, {name}: {res[name]['steps_per_s']:.1f} steps/s")
        r.sess.close()
    return res


def quantize_bench(n_rows, launches=50):
    """dsa_quantize_rows over n_rows bf16 rows already in HBM: average launch time
    from events around back-to-back launches on the launch stream."""
    import torch
    import dsa_synth as S
    import kv_cache_offload_amd as K
    sess = make_session(S.WORKLOADS["tiny"], K.KV_OFFLOAD)
    g = torch.Generator(device="cuda").manual_seed(5)
    lat = torch.randn(n_rows, 512, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    rope = torch.randn(n_rows, 64, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    rows = torch.empty(n_rows, 656, dtype=torch.uint8, device="cuda")
    for _ in range(10):
        sess.quantize_rows(lat, rope, rows)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(launches):
        sess.quantize_rows(lat, rope, rows)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / launches
    sess.close()
    nbytes = n_rows * (512 * 2 + 64 * 2 + 656)        # latent and RoPE read, packed row written
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"rows": n_rows, "us_per_launch": us, "bytes_per_launch": nbytes, "GBps": gbps,
            "hbm_frac": gbps / HBM_PEAK_GBPS, "rows_per_s": n_rows / (us * 1e-6)}


def cpu_baseline(w, inputs, budget_s):
    """The oracle as it stands, on the host cores, on the first decode steps of the same workload
    (its first unit: layer 0, sequence 0)."""
    import dsa_synth as S
    from oracle import MODE_OFFLOAD, OracleUnit, UnitShape
    hist = S.history(w, 0, 0)
    u = OracleUnit(UnitShape(max_positions=w.max_positions, index_heads=w.index_heads, index_dim=w.index_dim,
                             heads=w.heads, top_k=w.top_k, hot_slots=w.hot_slots, max_query_rows=w.rows_per_step,
                             mode=MODE_OFFLOAD, softmax_scale=w.softmax_scale))
    u.append(*hist)
    u.flush()
    if w.warm:
        u.warm()
    keys, rows, iq, iw, ql, qr = inputs
    t0 = time.perf_counter()
    n = 0
    while n < keys.shape[0] and (n < 2 or time.perf_counter() - t0 < budget_s):
        u.append(keys[n, 0, 0], rows[n, 0, 0])
        u.decode_step(iq[n, 0, 0], iw[n, 0, 0], ql[n, 0, 0], qr[n, 0, 0])
        n += 1
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return dict(value=n / dt, unit="decode steps/s", cores=cores, kind="oracle",
                sample=f"first {n} decode steps (append + decode) of {w.name} after loading the "
                       f"{w.history}-row history and warming the cache; {dt:.1f} s of CPU work")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--pmc-summary":
        pmc_summary(*sys.argv[2:5])
        return
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import dsa_synth as S
    import kv_cache_offload_amd as K

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    base = S.WORKLOADS[args.workload]
    n_steps = args.warmup + args.steps + args.kernel_steps
    if base.planted_overlap:
        from dsa_synth import planted
        if n_steps > planted.max_steps(base):
            print(f"{base.name} has planted queries for {planted.max_steps(base)} steps; "
                  f"--warmup + --steps + --kernel-steps asks for {n_steps}", file=sys.stderr)
            sys.exit(2)
    w = base.scaled(steps=max(base.steps, n_steps))
    log(f"generating {n_steps} steps of inputs for {w.name}")
    t0 = time.perf_counter()
    inputs = gen_inputs(w, n_steps)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")

    if args.reuse_probe:
        print(json.dumps({"workload": w.name, "reuse_probe": reuse_probe(w, inputs, args)}), flush=True)
        return
    if args.replacement_probe:
        probe = replacement_probe(w, inputs, args)
        print(json.dumps({"workload": w.name, "replacement_probe": probe}), flush=True)
        return
    both = run_pairs(w, inputs, args)
    primary = "resident" if args.resident_only else "offload"
    off, resd = both[primary], (None if args.resident_only else both.get("resident"))

    R, Q, NL = w.rows_per_step, w.seqs, w.layers
    rb = w.row_bytes
    kern = off["kernels"]
    kc = off["kernel_counters"]
    # dominant kernel of the offloaded step and its roofline: the HBM view (algorithmic bytes), the host-link
    # view (rows actually read from the host mirror, every reading query row counted) and the MFMA view
    # (bf16 flops); the bound is the view the kernel is closest to
    total_ms = {k: v["avg_us"] * v["launches"] for k, v in kern.items()}
    dom = max(total_ms, key=total_ms.get)
    d = kern[dom]
    views = {"hbm": (d["GBps"], HBM_PEAK_GBPS, "GB/s", d["bytes_per_launch"])}
    L_kern = off["L_start"] + R * (args.steps + args.kernel_steps / 2.0)
    if dom == "attention":
        host_b = kc[8] * rb / d["launches"]
        views["host_link"] = (host_b / (d["avg_us"] * 1e-6) / 1e9, HOST_LINK_PEAK_GBPS, "GB/s", host_b)
        flops = Q * R * w.top_k * w.heads * (576 + 512) * 2.0
        views["mfma"] = (flops / (d["avg_us"] * 1e-6) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", flops)
    elif dom == "index_score":
        flops = Q * R * w.index_heads * L_kern * w.index_dim * 2.0
        views["mfma"] = (flops / (d["avg_us"] * 1e-6) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", flops)
    bound = max(views, key=lambda k: views[k][0] / views[k][1])
    a_, p_, u_, per_launch = views[bound]
    roof = dict(kernel=dom, bound=bound, achieved=a_, peak=p_, unit=u_, frac=a_ / p_,
                traffic=pmc_traffic(w.name, dom), avg_us=d["avg_us"],
                algorithmic_per_launch=per_launch,
                views={k: {"achieved": v[0], "peak": v[1], "unit": v[2], "frac": v[0] / v[1], "per_launch": v[3]}
                       for k, v in views.items()})

    c = off["counters"]
    n = off["steps"]
    per_step = lambda k: kern[k]["avg_us"] * kern[k]["launches"] / off["kernel_steps"] if k in kern else 0.0
    L_mean = off["L_start"] + R * (n + 1) / 2.0
    # scoring + selection: every index key once per step (HBM)
    ss_us = per_step("index_score") + per_step("topk_collect") + per_step("topk_resolve")
    ss_bytes = NL * Q * L_mean * w.index_dim * 2
    # gather + attention: each distinct selected row from its source (hits and ring rows from HBM, misses over
    # the host link), compact rows and slot fills written to HBM; host bytes as actually read
    host_distinct = c[6] / n
    host_read = c[8] * rb / n
    ga_us = per_step("gather") + per_step("attention")
    ga_hbm_bytes = ((c[1] + c[2] + c[7]) + c[0] + c[3]) * rb / n
    line = {
        "metric": METRIC,
        "value": off["steps_per_s"],
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * off["seconds"] / off["steps"],
        "steps_per_s_with_kernel_events": off["steps_per_s_with_kernel_events"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": NL, "sequences": Q, "history": w.history, "query_rows": R,
                   "top_k": w.top_k, "hot_slots": w.hot_slots, "index_heads": w.index_heads, "heads": w.heads,
                   "row_bytes": rb, "mode": primary, "replacement": args.replacement,
                   "append": "separate dsa_append_rows" if args.separate_append else "in dsa_append_decode_step",
                   "L_at_timed_start": off["L_start"]},
        "query_rows_per_s": off["steps_per_s"] * R * Q,
        "roofline": roof,
        "score_select": {"us_per_step": ss_us, "hbm_bytes_per_step": ss_bytes,
                         "hbm_frac": ss_bytes / (ss_us * 1e-6) / 1e9 / HBM_PEAK_GBPS if ss_us else 0.0},
        "gather_attention": {"us_per_step": ga_us, "hbm_bytes_per_step": ga_hbm_bytes,
                             "host_bytes_read_per_step": host_read,
                             "hbm_frac": ga_hbm_bytes / (ga_us * 1e-6) / 1e9 / HBM_PEAK_GBPS if ga_us else 0.0,
                             "host_link_GBps": host_read / (ga_us * 1e-6) / 1e9 if ga_us else 0.0,
                             "host_link_frac": host_read / (ga_us * 1e-6) / 1e9 / HOST_LINK_PEAK_GBPS
                             if ga_us else 0.0},
        "host_link": {"bytes_read_per_step": host_read,
                      "rows_read_per_step": c[8] / n,
                      "distinct_miss_bytes_per_step": host_distinct,
                      "distinct_miss_rows_per_step": (c[3] + c[4]) / n,
                      "hit_rate": c[1] / max(1, c[0] - c[2]),
                      "peak_GBps": HOST_LINK_PEAK_GBPS},
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
        "kernels_GBps": {k: round(v["GBps"], 1) for k, v in kern.items()},
        "counters_timed": dict(zip(K.COUNTER_NAMES, c)),
        "segments_steps_per_s": off["segments"],
        "environment": environment(),
    }
    if resd is not None:
        line["resident"] = {"value": resd["steps_per_s"], "ms_per_step": 1e3 * resd["seconds"] / resd["steps"],
                            "segments_steps_per_s": resd["segments"],
                            "kernels_us": {k: round(v["avg_us"], 2) for k, v in resd["kernels"].items()}}
        line["offload_slowdown"] = resd["steps_per_s"] / off["steps_per_s"] - 1.0
        line["offload_slowdown_per_pair"] = [round(b / a - 1.0, 4) for a, b in zip(off["segments"], resd["segments"])]
    if args.quantize_rows > 0:
        log(f"quantise-on-append over {args.quantize_rows} rows")
        line["quantize"] = quantize_bench(args.quantize_rows)
    if not args.no_cpu and NL == 1 and Q == 1:
        log("timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_seconds)
    if args.calib_copy:
        n = 2 << 30                                      # well above the last-level cache
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = n
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
