"""CPU oracle for the DSA sparse-attention decode step (test infrastructure).

This package is TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library and
its Python binding never import, link or call anything here, and nothing here
imports them.

It wraps ``liboracle.so``, built from ``dsa_oracle.c`` (plain C, float64), which
models one unit -- one (layer, sequence) pair -- of the method described on the
page "From 1M total to 15+ streams x 1M: the capacity breakthrough of GLM-5.3 KV
cache offload" (zhuai.tech): index scoring over the whole history, exact Top-K,
a GPU-managed hot cache with a recent ring and a pinned host mirror, and
absorbed-MLA attention over the selected rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_HDR = os.path.join(_HERE, "dsa_oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, E_INVALID, E_NOMEM, E_CAPACITY, E_STATE = 0, 1, 2, 3, 4
MODE_OFFLOAD, MODE_RESIDENT = 0, 1
REPL_RING, REPL_CLOCK = 0, 1
SRC_HIT, SRC_RING, SRC_MISS, SRC_MISS_NOSLOT, SRC_RES = 0, 1, 2, 3, 4
CNT_NAMES = ("union", "hit", "ring", "miss", "miss_noslot", "evict", "host_bytes", "res", "host_reads")


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (C11, OpenMP)."""
    stale = (not os.path.exists(_LIB)) or any(
        os.path.getmtime(p) > os.path.getmtime(_LIB) for p in (_SRC, _HDR))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-fopenmp",
                               "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Config(ctypes.Structure):
    _fields_ = [
        ("max_positions", ctypes.c_int64),
        ("index_heads", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("hot_slots", ctypes.c_int32),
        ("ring_rows", ctypes.c_int32),
        ("max_query_rows", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("softmax_scale", ctypes.c_double),
        ("replacement", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.orc_create.restype = P
        lib.orc_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(ctypes.c_int)]
        lib.orc_destroy.argtypes = [P]
        lib.orc_row_bytes.restype = i64
        lib.orc_row_bytes.argtypes = [P]
        lib.orc_append.argtypes = [P, i64, P, P]
        lib.orc_flush.argtypes = [P]
        lib.orc_warm.argtypes = [P]
        lib.orc_rollback.argtypes = [P, i64]
        lib.orc_decode_step.argtypes = [P, i32, P, P, P, P, P]
        lib.orc_decode_step_sel.argtypes = [P, i32, P, P, P, P, P]
        lib.orc_prefetch_sel.argtypes = [P, i32, P, P]
        for name in ("orc_get_state", "orc_get_scores", "orc_get_map", "orc_get_compact",
                     "orc_get_counters", "orc_get_pos_slot", "orc_get_slot_bytes", "orc_get_ref"):
            getattr(lib, name).argtypes = [P, P]
        lib.orc_get_selection.argtypes = [P, P, P]
        lib.orc_get_union.argtypes = [P, P, P, P]
        lib.orc_get_slots.argtypes = [P, P, P, P]
        lib.orc_get_mirror.argtypes = [P, i64, i64, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    def __init__(self, what: str, status: int):
        super().__init__(f"{what} failed with status {status}")
        self.status = status


@dataclass
class UnitShape:
    max_positions: int
    index_heads: int
    index_dim: int
    heads: int
    top_k: int
    hot_slots: int
    max_query_rows: int
    latent_dim: int = 512
    rope_dim: int = 64
    group: int = 64
    ring_rows: int = 64
    mode: int = MODE_OFFLOAD
    softmax_scale: float | None = None
    replacement: int = REPL_RING

    @property
    def row_bytes(self) -> int:
        return self.latent_dim + 2 * (self.latent_dim // self.group) + 2 * self.rope_dim


class OracleUnit:
    """One (layer, sequence) unit modelled on the CPU."""

    def __init__(self, shape: UnitShape):
        lib = _load()
        scale = shape.softmax_scale
        if scale is None:
            scale = 1.0 / np.sqrt(shape.latent_dim + shape.rope_dim)
        cfg = _Config(shape.max_positions, shape.index_heads, shape.index_dim, shape.heads,
                      shape.latent_dim, shape.rope_dim, shape.group, shape.top_k,
                      shape.hot_slots, shape.ring_rows, shape.max_query_rows, shape.mode,
                      float(scale), shape.replacement)
        st = ctypes.c_int(0)
        h = lib.orc_create(ctypes.byref(cfg), ctypes.byref(st))
        if not h:
            raise OracleError("orc_create", st.value)
        self._h = ctypes.c_void_p(h)
        self._lib = lib
        self.shape = shape
        self.row_bytes = int(lib.orc_row_bytes(self._h))

    def close(self):
        if getattr(self, "_h", None) is not None:
            self._lib.orc_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _check(self, what, st):
        if st != OK:
            raise OracleError(what, st)

    # ---------------------------------------------------------------- calls
    def append(self, keys: np.ndarray, rows: np.ndarray):
        keys = np.ascontiguousarray(keys, dtype=np.uint16)
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        n = keys.shape[0]
        assert keys.shape == (n, self.shape.index_dim) and rows.shape == (n, self.row_bytes)
        self._check("orc_append", self._lib.orc_append(self._h, n, _ptr(keys), _ptr(rows)))

    def flush(self):
        self._check("orc_flush", self._lib.orc_flush(self._h))

    def warm(self):
        self._check("orc_warm", self._lib.orc_warm(self._h))

    def rollback(self, n: int):
        self._check("orc_rollback", self._lib.orc_rollback(self._h, n))

    def decode_step(self, index_q, index_w, q_lat, q_rope) -> np.ndarray:
        s = self.shape
        index_q = np.ascontiguousarray(index_q, dtype=np.uint16)
        index_w = np.ascontiguousarray(index_w, dtype=np.float32)
        q_lat = np.ascontiguousarray(q_lat, dtype=np.uint16)
        q_rope = np.ascontiguousarray(q_rope, dtype=np.uint16)
        R = index_q.shape[0]
        assert index_q.shape == (R, s.index_heads, s.index_dim)
        assert index_w.shape == (R, s.index_heads)
        assert q_lat.shape == (R, s.heads, s.latent_dim) and q_rope.shape == (R, s.heads, s.rope_dim)
        out = np.empty((R, s.heads, s.latent_dim), dtype=np.float32)
        self._check("orc_decode_step", self._lib.orc_decode_step(
            self._h, R, _ptr(index_q), _ptr(index_w), _ptr(q_lat), _ptr(q_rope), _ptr(out)))
        return out

    def _sel_args(self, sel, counts):
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        counts = np.ascontiguousarray(counts, dtype=np.int32)
        assert sel.ndim == 2 and sel.shape[1] == self.shape.top_k and counts.shape == (sel.shape[0],)
        return sel, counts

    def decode_step_sel(self, sel, counts, q_lat, q_rope) -> np.ndarray:
        """A round on a given selection (selection reuse): sel [R][K] ascending, -1 padded."""
        s = self.shape
        sel, counts = self._sel_args(sel, counts)
        R = sel.shape[0]
        q_lat = np.ascontiguousarray(q_lat, dtype=np.uint16)
        q_rope = np.ascontiguousarray(q_rope, dtype=np.uint16)
        assert q_lat.shape == (R, s.heads, s.latent_dim) and q_rope.shape == (R, s.heads, s.rope_dim)
        out = np.empty((R, s.heads, s.latent_dim), dtype=np.float32)
        self._check("orc_decode_step_sel", self._lib.orc_decode_step_sel(
            self._h, R, _ptr(sel), _ptr(counts), _ptr(q_lat), _ptr(q_rope), _ptr(out)))
        return out

    def prefetch_sel(self, sel, counts):
        sel, counts = self._sel_args(sel, counts)
        self._check("orc_prefetch_sel", self._lib.orc_prefetch_sel(self._h, sel.shape[0], _ptr(sel), _ptr(counts)))

    # ---------------------------------------------------------------- getters
    def state(self) -> dict:
        st = np.zeros(7, dtype=np.int64)
        self._lib.orc_get_state(self._h, _ptr(st))
        return dict(L=int(st[0]), M=int(st[1]), round=int(st[2]), hand=int(st[3]),
                    R=int(st[4]), U=int(st[5]), floor=int(st[6]))

    def scores(self) -> np.ndarray:
        st = self.state()
        out = np.zeros((st["R"], st["L"]), dtype=np.float32)
        self._lib.orc_get_scores(self._h, _ptr(out))
        return out

    def selection(self):
        st = self.state()
        sel = np.empty((st["R"], self.shape.top_k), dtype=np.int32)
        cnt = np.empty(st["R"], dtype=np.int32)
        self._lib.orc_get_selection(self._h, _ptr(sel), _ptr(cnt))
        return sel, cnt

    def union(self):
        U = self.state()["U"]
        uni = np.empty(U, dtype=np.int32)
        kind = np.empty(U, dtype=np.int32)
        src = np.empty(U, dtype=np.int32)
        self._lib.orc_get_union(self._h, _ptr(uni), _ptr(kind), _ptr(src))
        return uni, kind, src

    def map(self) -> np.ndarray:
        st = self.state()
        m = np.empty((st["R"], self.shape.top_k), dtype=np.int32)
        self._lib.orc_get_map(self._h, _ptr(m))
        return m

    def compact(self) -> np.ndarray:
        U = self.state()["U"]
        out = np.empty((U, self.row_bytes), dtype=np.uint8)
        self._lib.orc_get_compact(self._h, _ptr(out))
        return out

    def counters(self) -> dict:
        c = np.zeros(len(CNT_NAMES), dtype=np.int64)
        self._lib.orc_get_counters(self._h, _ptr(c))
        return {k: int(v) for k, v in zip(CNT_NAMES, c)}

    def slots(self):
        S = self.shape.hot_slots if self.shape.mode == MODE_OFFLOAD else 0
        sp = np.empty(S, dtype=np.int32)
        fr = np.empty(S, dtype=np.int32)
        pr = np.empty(S, dtype=np.int32)
        self._lib.orc_get_slots(self._h, _ptr(sp), _ptr(fr), _ptr(pr))
        return sp, fr, pr

    def pos_slot(self) -> np.ndarray:
        out = np.empty(self.state()["L"], dtype=np.int32)
        self._lib.orc_get_pos_slot(self._h, _ptr(out))
        return out

    def ref(self) -> np.ndarray:
        out = np.zeros(self.shape.hot_slots if self.shape.mode == MODE_OFFLOAD else 0, dtype=np.uint8)
        self._lib.orc_get_ref(self._h, _ptr(out))
        return out

    def slot_bytes(self) -> np.ndarray:
        S = self.shape.hot_slots if self.shape.mode == MODE_OFFLOAD else 0
        out = np.empty((S, self.row_bytes), dtype=np.uint8)
        self._lib.orc_get_slot_bytes(self._h, _ptr(out))
        return out

    def mirror(self, first: int = 0, n: int | None = None) -> np.ndarray:
        if n is None:
            n = self.state()["M"] - first
        out = np.empty((n, self.row_bytes), dtype=np.uint8)
        self._check("orc_get_mirror", self._lib.orc_get_mirror(self._h, first, n, _ptr(out)))
        return out
