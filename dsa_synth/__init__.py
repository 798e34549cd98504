"""Seeded synthetic inputs for the DSA sparse-attention decode workloads.

This module holds only input generators and workload shapes.  It contains none
of the method's arithmetic (no scoring, selection, caching or attention), so the
CPU oracle and the HIP path can both be fed from it without sharing any of the
computation they are compared on.

Streams are counter-based: every tensor is drawn from its own Philox-4x64
generator keyed by (root seed, workload, layer, sequence, step, tensor tag), so
any slice of any workload can be regenerated without drawing the rest.  Values
are sampled in float64 and rounded to the storage type with round-to-nearest-
even (float64 -> float32 -> bf16 for bf16; float64 -> fp16 for fp16).

Value recipe (same for every workload):
  - indexer keys and queries: bf16 holding integers uniform in [-8, 8];
  - indexer head weights: integers uniform in [0, 4], stored as f32;
  - MLA queries: bf16 latent (512) and RoPE (64) parts ~ N(0, 0.05);
  - Q8G64 rows (656 B): 512 int8 uniform in [-127, 127], then 8 fp16 scales
    uniform in [0.002, 0.02] (one per group of 64), then 64 bf16 RoPE ~ N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

ROOT_SEED = 0
HISTORY_CHUNK = 65536  # rows per history generator substream

# tensor tags of the substream key
_T_HIST_KEYS, _T_HIST_ROWS, _T_NEW_KEYS, _T_NEW_ROWS = 1, 2, 3, 4
_T_INDEX_Q, _T_INDEX_W, _T_Q_LAT, _T_Q_ROPE = 5, 6, 7, 8


@dataclass(frozen=True)
class Workload:
    """Shape of one synthetic decode workload.

    A unit is one (layer, sequence) pair with its own history and hot cache.
    Layers run one after another inside a step; sequences of one layer run
    together in one call.
    """
    name: str
    wid: int                 # workload id in the substream key
    layers: int
    seqs: int
    history: int             # T: rows present before the first step
    rows_per_step: int       # R: query rows (and appended rows) per sequence per step
    steps: int
    index_heads: int         # H_I
    heads: int               # H
    top_k: int
    hot_slots: int
    warm: bool               # hot cache prefilled with the most recent positions
    planted_overlap: bool = False
    index_dim: int = 128
    latent_dim: int = 512
    rope_dim: int = 64
    group: int = 64
    ring_rows: int = 64
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def row_bytes(self) -> int:
        return self.latent_dim + 2 * (self.latent_dim // self.group) + 2 * self.rope_dim

    @property
    def max_positions(self) -> int:
        return self.history + self.rows_per_step * self.steps

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.latent_dim + self.rope_dim))

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny case the oracle finishes in seconds: empty 1024-slot cache.
    "tiny": Workload("tiny", 0, layers=1, seqs=1, history=4096, rows_per_step=1, steps=4,
                     index_heads=4, heads=16, top_k=256, hot_slots=1024, warm=False),
    # Single stream at the pages' acceptance shape: 50,023 history, MTP=3 verify (4 rows).
    "single_stream_50k": Workload("single_stream_50k", 1, layers=1, seqs=1, history=50023,
                                  rows_per_step=4, steps=1024, index_heads=32, heads=64,
                                  top_k=2048, hot_slots=32768, warm=True),
    # 16 independent sequences of 131,072 rows, 8,192-slot cache each.
    "batched_16x131k": Workload("batched_16x131k", 2, layers=1, seqs=16, history=131072,
                                rows_per_step=1, steps=256, index_heads=32, heads=64,
                                top_k=2048, hot_slots=8192, warm=True),
    # One stream with a 1,048,576-row history.
    "million": Workload("million", 3, layers=1, seqs=1, history=1048576, rows_per_step=4,
                        steps=256, index_heads=32, heads=64, top_k=2048, hot_slots=32768,
                        warm=True),
    # Selection reuse: layer 0 makes the selection, layers 1-3 reuse it with their
    # own rows and caches (single stream at the 50,023-row shape).
    "reuse_4_layers": Workload("reuse_4_layers", 5, layers=4, seqs=1, history=50023,
                               rows_per_step=4, steps=256, index_heads=32, heads=64,
                               top_k=2048, hot_slots=32768, warm=True),
    # 78 layers, full caches, 8 query rows with 99% planted overlap with the cache.
    "stress_78_layers": Workload("stress_78_layers", 4, layers=78, seqs=1, history=50023,
                                 rows_per_step=8, steps=128, index_heads=32, heads=64,
                                 top_k=2048, hot_slots=32768, warm=True, planted_overlap=True),
}


# ------------------------------------------------------------------ rounding helpers

def bf16_bits(x) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 bits (RNE), as uint16."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32)
    # finite values are at most 0xFF7FFFFF, so the sum stays below 2^32 in uint32
    rounded = (u >> 16) & 1
    rounded += u
    rounded += 0x7FFF
    rounded >>= 16
    nan = np.isnan(f)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_value(bits) -> np.ndarray:
    """bf16 bits -> float64 value (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _rng(w: Workload, layer: int, seq: int, step: int, tag: int, sub: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, w.wid, layer, seq, step + 1, tag, sub])
    return np.random.Generator(np.random.Philox(ss))


def _int_bf16(g: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    return bf16_bits(g.integers(lo, hi + 1, size=shape).astype(np.float64))


def make_rows(g: np.random.Generator, n: int, w: Workload) -> np.ndarray:
    """n packed Q8G64 rows: int8 latent | fp16 scales (LE) | bf16 RoPE (LE)."""
    lat = g.integers(-127, 128, size=(n, w.latent_dim), dtype=np.int8)
    scales = f16_bits(g.uniform(0.002, 0.02, size=(n, w.latent_dim // w.group)))
    rope = bf16_bits(g.standard_normal(size=(n, w.rope_dim)))
    out = np.empty((n, w.row_bytes), dtype=np.uint8)
    out[:, :w.latent_dim] = lat.view(np.uint8)
    out[:, w.latent_dim:w.latent_dim + 2 * (w.latent_dim // w.group)] = \
        scales.astype("<u2").view(np.uint8).reshape(n, -1)
    out[:, w.latent_dim + 2 * (w.latent_dim // w.group):] = rope.astype("<u2").view(np.uint8).reshape(n, -1)
    return out


# ------------------------------------------------------------------ history and steps

def history(w: Workload, layer: int, seq: int, first: int = 0, n: int | None = None):
    """Rows [first, first+n) of a unit's pre-step history: (keys u16 [n][D_I], rows u8 [n][656])."""
    if w.planted_overlap:
        from . import planted
        return planted.history(w, layer, seq, first, n)
    if n is None:
        n = w.history - first
    keys = np.empty((n, w.index_dim), dtype=np.uint16)
    rows = np.empty((n, w.row_bytes), dtype=np.uint8)
    pos = first
    while pos < first + n:
        c = pos // HISTORY_CHUNK
        c0 = c * HISTORY_CHUNK
        clen = min(HISTORY_CHUNK, w.history - c0)
        take = min(first + n, c0 + clen) - pos
        gk = _rng(w, layer, seq, -1, _T_HIST_KEYS, c)
        gr = _rng(w, layer, seq, -1, _T_HIST_ROWS, c)
        ck = _int_bf16(gk, (clen, w.index_dim), -8, 8)
        cr = make_rows(gr, clen, w)
        keys[pos - first:pos - first + take] = ck[pos - c0:pos - c0 + take]
        rows[pos - first:pos - first + take] = cr[pos - c0:pos - c0 + take]
        pos += take
    return keys, rows


def step_rows(w: Workload, layer: int, seq: int, step: int):
    """The R rows appended before decode step `step`."""
    if w.planted_overlap:
        from . import planted
        return planted.step_rows(w, layer, seq, step)
    keys = _int_bf16(_rng(w, layer, seq, step, _T_NEW_KEYS), (w.rows_per_step, w.index_dim), -8, 8)
    rows = make_rows(_rng(w, layer, seq, step, _T_NEW_ROWS), w.rows_per_step, w)
    return keys, rows


def step_queries(w: Workload, layer: int, seq: int, step: int):
    """(index_q u16 [R][H_I][D_I], index_w f32 [R][H_I], q_lat u16 [R][H][512], q_rope u16 [R][H][64])."""
    R = w.rows_per_step
    if w.planted_overlap:
        from . import planted
        index_q, index_w = planted.index_queries(w, layer, seq, step)
    else:
        index_q = _int_bf16(_rng(w, layer, seq, step, _T_INDEX_Q), (R, w.index_heads, w.index_dim), -8, 8)
        index_w = _rng(w, layer, seq, step, _T_INDEX_W).integers(0, 5, size=(R, w.index_heads)).astype(np.float32)
    q_lat = bf16_bits(0.05 * _rng(w, layer, seq, step, _T_Q_LAT).standard_normal((R, w.heads, w.latent_dim)))
    q_rope = bf16_bits(0.05 * _rng(w, layer, seq, step, _T_Q_ROPE).standard_normal((R, w.heads, w.rope_dim)))
    return index_q, index_w, q_lat, q_rope
