"""Python binding of libdsa (include/dsa.h): DSA sparse-attention decode over an
MLA history offloaded to pinned host memory behind an HBM hot cache, on MI355X.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libdsa.so.  PyTorch supplies device memory and streams.  If the
library is not built, importing this package raises ImportError -- there is no
fallback implementation.

The functions carry the C names (``dsa_session_create``, ``dsa_append_rows``,
``dsa_decode_step``, ...); :class:`Session` wraps them for torch tensors.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

ABI_VERSION = 3
OK, E_INVALID, E_NOMEM, E_CAPACITY, E_UNSUPPORTED, E_STATE, E_HIP = range(7)
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_E_INVALID", 2: "DSA_E_NOMEM", 3: "DSA_E_CAPACITY",
                4: "DSA_E_UNSUPPORTED", 5: "DSA_E_STATE", 6: "DSA_E_HIP"}
KV_OFFLOAD, KV_HBM_RESIDENT = 0, 1
REPL_RING, REPL_CLOCK = 0, 1
KERNEL_KINDS = ("index_score", "topk_collect", "topk_resolve", "gather", "attention", "attention_merge", "append")

# inspection items (dsa_debug_item)
DBG = dict(scores=0, selection=1, sel_count=2, union=3, union_kind=4, union_src=5, map=6,
           compact=7, counters=8, slot_pos=9, fill_round=10, pin_round=11, pos_slot=12, hand=13,
           slot_bytes=14, mirror=15, keys=16, totals=17, ref_bits=18)
COUNTER_NAMES = ("union", "hit", "ring", "miss", "miss_noslot", "evict", "host_bytes", "res", "host_reads")

# every symbol include/dsa.h declares
EXPORTS = ("dsa_session_create", "dsa_session_destroy", "dsa_append_rows", "dsa_flush",
           "dsa_warm_hot", "dsa_rollback_rows", "dsa_quantize_rows", "dsa_append_latent",
           "dsa_decode_step", "dsa_decode_step_reuse", "dsa_prefetch_reuse", "dsa_unit_state",
           "dsa_mirror_rows",
           "dsa_last_error", "dsa_debug_size", "dsa_debug_get", "dsa_set_kernel_timing",
           "dsa_kernel_times", "dsa_debug_inject", "dsa_decode_step_static", "dsa_append_decode_step")
INJECT_HIP_FAILURE, INJECT_BAD_SLOT = 0, 1


class dsa_config(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32),
        ("device", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("n_seqs", ctypes.c_int32),
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
        ("softmax_scale", ctypes.c_float),
        ("mode", ctypes.c_int32),
        ("replacement", ctypes.c_int32),
    ]


def _load_library() -> ctypes.CDLL:
    # One HIP runtime per process: PyTorch ships its own libamdhip64.so.7, so it
    # is loaded first and libdsa's dependency on that soname binds to it.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run: python kv_cache_offload_amd/build.py); "
                          "there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "dsa_session_create": ([ctypes.POINTER(dsa_config), ctypes.POINTER(P)], ctypes.c_int),
        "dsa_session_destroy": ([P], ctypes.c_int),
        "dsa_append_rows": ([P, i32, i32, i64, P, P, P], ctypes.c_int),
        "dsa_flush": ([P, i32, i32, P], ctypes.c_int),
        "dsa_warm_hot": ([P, i32, i32, P], ctypes.c_int),
        "dsa_rollback_rows": ([P, i32, i32, i64, P], ctypes.c_int),
        "dsa_quantize_rows": ([P, i64, P, P, P, P], ctypes.c_int),
        "dsa_append_latent": ([P, i32, i32, i64, P, P, P, P], ctypes.c_int),
        "dsa_decode_step": ([P, i32, i32, P, P, P, P, P, P], ctypes.c_int),
        "dsa_decode_step_reuse": ([P, i32, i32, i32, P, P, P, P], ctypes.c_int),
        "dsa_prefetch_reuse": ([P, i32, i32, i32, P], ctypes.c_int),
        "dsa_unit_state": ([P, i32, i32, ctypes.POINTER(i64)], ctypes.c_int),
        "dsa_mirror_rows": ([P, i32, i32, ctypes.POINTER(i64)], ctypes.c_int),
        "dsa_last_error": ([P], ctypes.c_char_p),
        "dsa_debug_size": ([P, i32, i32, i32, ctypes.POINTER(sz)], ctypes.c_int),
        "dsa_debug_get": ([P, i32, i32, i32, P, sz, P], ctypes.c_int),
        "dsa_set_kernel_timing": ([P, i32], ctypes.c_int),
        "dsa_kernel_times": ([P, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "dsa_debug_inject": ([P, i32, i32, i32, P], ctypes.c_int),
        "dsa_decode_step_static": ([P, i32, i32, P, P, P, P, P, P], ctypes.c_int),
        "dsa_append_decode_step": ([P, i32, i32, P, P, P, P, P, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib = _load_library()


class DsaError(RuntimeError):
    def __init__(self, call: str, status: int, message: str = ""):
        super().__init__(f"{call} -> {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


# ---------------------------------------------------------------- C-named wrappers

def _handle(h):
    return h if isinstance(h, ctypes.c_void_p) else ctypes.c_void_p(h)


def dsa_session_create(cfg: dsa_config) -> ctypes.c_void_p:
    out = ctypes.c_void_p()
    st = _lib.dsa_session_create(ctypes.byref(cfg), ctypes.byref(out))
    if st != OK:
        raise DsaError("dsa_session_create", st)
    return out


def dsa_session_destroy(h) -> int:
    return _lib.dsa_session_destroy(_handle(h) if h is not None else None)


def dsa_append_rows(h, layer, seq, n, index_keys_ptr, rows_ptr, stream) -> int:
    return _lib.dsa_append_rows(_handle(h), layer, seq, n, index_keys_ptr, rows_ptr, stream)


def dsa_flush(h, layer, seq, stream) -> int:
    return _lib.dsa_flush(_handle(h), layer, seq, stream)


def dsa_warm_hot(h, layer, seq, stream) -> int:
    return _lib.dsa_warm_hot(_handle(h), layer, seq, stream)


def dsa_quantize_rows(h, n, latent_ptr, rope_ptr, rows_ptr, stream) -> int:
    return _lib.dsa_quantize_rows(_handle(h), n, latent_ptr, rope_ptr, rows_ptr, stream)


def dsa_append_latent(h, layer, seq, n, index_keys_ptr, latent_ptr, rope_ptr, stream) -> int:
    return _lib.dsa_append_latent(_handle(h), layer, seq, n, index_keys_ptr, latent_ptr, rope_ptr, stream)


def dsa_rollback_rows(h, layer, seq, n, stream) -> int:
    return _lib.dsa_rollback_rows(_handle(h), layer, seq, n, stream)


def dsa_decode_step(h, layer, rows_per_seq, index_q, index_w, q_latent, q_rope, out, stream) -> int:
    return _lib.dsa_decode_step(_handle(h), layer, rows_per_seq, index_q, index_w, q_latent, q_rope,
                                out, stream)


def dsa_append_decode_step(h, layer, rows_per_seq, index_keys, rows, index_q, index_w, q_latent, q_rope, out,
                           stream) -> int:
    return _lib.dsa_append_decode_step(_handle(h), layer, rows_per_seq, index_keys, rows, index_q, index_w,
                                       q_latent, q_rope, out, stream)


def dsa_decode_step_static(h, layer, rows_per_seq, index_q, index_w, q_latent, q_rope, out, stream) -> int:
    return _lib.dsa_decode_step_static(_handle(h), layer, rows_per_seq, index_q, index_w, q_latent, q_rope,
                                       out, stream)


def dsa_decode_step_reuse(h, layer, src_layer, rows_per_seq, q_latent, q_rope, out, stream) -> int:
    return _lib.dsa_decode_step_reuse(_handle(h), layer, src_layer, rows_per_seq, q_latent, q_rope, out, stream)


def dsa_prefetch_reuse(h, layer, src_layer, rows_per_seq, stream) -> int:
    return _lib.dsa_prefetch_reuse(_handle(h), layer, src_layer, rows_per_seq, stream)


def dsa_unit_state(h, layer, seq):
    out = (ctypes.c_int64 * 4)()
    st = _lib.dsa_unit_state(_handle(h), layer, seq, out)
    return st, list(out)


def dsa_mirror_rows(h, layer, seq):
    v = ctypes.c_int64(0)
    st = _lib.dsa_mirror_rows(_handle(h), layer, seq, ctypes.byref(v))
    return st, v.value


def dsa_last_error(h) -> str:
    r = _lib.dsa_last_error(_handle(h) if h is not None else None)
    return r.decode() if r else ""


def dsa_debug_size(h, layer, seq, item):
    v = ctypes.c_size_t(0)
    st = _lib.dsa_debug_size(_handle(h), layer, seq, item, ctypes.byref(v))
    return st, v.value


def dsa_debug_get(h, layer, seq, item, dst_ptr, nbytes, stream) -> int:
    return _lib.dsa_debug_get(_handle(h), layer, seq, item, dst_ptr, nbytes, stream)


def dsa_set_kernel_timing(h, enable: bool) -> int:
    return _lib.dsa_set_kernel_timing(_handle(h), 1 if enable else 0)


def dsa_kernel_times(h):
    counts = (ctypes.c_int64 * len(KERNEL_KINDS))()
    ms = (ctypes.c_double * len(KERNEL_KINDS))()
    st = _lib.dsa_kernel_times(_handle(h), counts, ms)
    return st, list(counts), list(ms)


def dsa_debug_inject(h, layer, seq, what, stream) -> int:
    return _lib.dsa_debug_inject(_handle(h), layer, seq, what, stream)


# ---------------------------------------------------------------- torch convenience

def make_config(*, max_positions, index_heads, heads, top_k, hot_slots, max_query_rows,
                n_layers=1, n_seqs=1, index_dim=128, latent_dim=512, rope_dim=64, group=64,
                ring_rows=64, softmax_scale=None, mode=KV_OFFLOAD, device=0,
                replacement=REPL_RING) -> dsa_config:
    if softmax_scale is None:
        softmax_scale = 1.0 / float((latent_dim + rope_dim) ** 0.5)
    return dsa_config(ABI_VERSION, device, n_layers, n_seqs, max_positions, index_heads, index_dim,
                      heads, latent_dim, rope_dim, group, top_k, hot_slots, ring_rows,
                      max_query_rows, softmax_scale, mode, replacement)


class Session:
    """A libdsa session driven with torch CUDA (HIP) tensors on the current stream."""

    def __init__(self, cfg: dsa_config):
        import torch
        self._torch = torch
        self.cfg = cfg
        self.h = dsa_session_create(cfg)
        self.row_bytes = cfg.latent_dim + 2 * (cfg.latent_dim // cfg.group) + 2 * cfg.rope_dim
        self.device = torch.device("cuda", cfg.device)

    def close(self):
        if getattr(self, "h", None) is not None:
            dsa_session_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _stream(self):
        return ctypes.c_void_p(self._torch.cuda.current_stream(self.device).cuda_stream)

    def _check(self, call, st):
        if st != OK:
            raise DsaError(call, st, dsa_last_error(self.h))

    @staticmethod
    def _ptr(t):
        if t is None:
            return None
        assert t.is_cuda and t.is_contiguous()
        return ctypes.c_void_p(t.data_ptr())

    def append_rows(self, layer, seq, index_keys, rows):
        n = index_keys.shape[0]
        self._check("dsa_append_rows", dsa_append_rows(self.h, layer, seq, n, self._ptr(index_keys),
                                                       self._ptr(rows), self._stream()))

    def flush(self, layer, seq):
        self._check("dsa_flush", dsa_flush(self.h, layer, seq, self._stream()))

    def warm_hot(self, layer, seq):
        self._check("dsa_warm_hot", dsa_warm_hot(self.h, layer, seq, self._stream()))

    def quantize_rows(self, latent, rope, rows):
        n = latent.shape[0]
        self._check("dsa_quantize_rows", dsa_quantize_rows(self.h, n, self._ptr(latent), self._ptr(rope),
                                                           self._ptr(rows), self._stream()))

    def append_latent(self, layer, seq, index_keys, latent, rope):
        n = index_keys.shape[0]
        self._check("dsa_append_latent", dsa_append_latent(self.h, layer, seq, n, self._ptr(index_keys),
                                                           self._ptr(latent), self._ptr(rope), self._stream()))

    def rollback_rows(self, layer, seq, n):
        self._check("dsa_rollback_rows", dsa_rollback_rows(self.h, layer, seq, n, self._stream()))

    def decode_step(self, layer, index_q, index_w, q_latent, q_rope, out):
        R = index_q.shape[1]
        self._check("dsa_decode_step", dsa_decode_step(
            self.h, layer, R, self._ptr(index_q), self._ptr(index_w), self._ptr(q_latent),
            self._ptr(q_rope), self._ptr(out), self._stream()))

    def append_decode_step(self, layer, index_keys, rows, index_q, index_w, q_latent, q_rope, out):
        """index_keys [n_seqs][R][index_dim], rows [n_seqs][R][row_bytes]: appended to every sequence, then
        one decode step."""
        R = index_q.shape[1]
        self._check("dsa_append_decode_step", dsa_append_decode_step(
            self.h, layer, R, self._ptr(index_keys), self._ptr(rows), self._ptr(index_q), self._ptr(index_w),
            self._ptr(q_latent), self._ptr(q_rope), self._ptr(out), self._stream()))

    def decode_step_static(self, layer, index_q, index_w, q_latent, q_rope, out):
        R = index_q.shape[1]
        self._check("dsa_decode_step_static", dsa_decode_step_static(
            self.h, layer, R, self._ptr(index_q), self._ptr(index_w), self._ptr(q_latent),
            self._ptr(q_rope), self._ptr(out), self._stream()))

    def decode_step_reuse(self, layer, src_layer, q_latent, q_rope, out):
        R = q_latent.shape[1]
        self._check("dsa_decode_step_reuse", dsa_decode_step_reuse(
            self.h, layer, src_layer, R, self._ptr(q_latent), self._ptr(q_rope), self._ptr(out), self._stream()))

    def prefetch_reuse(self, layer, src_layer, rows_per_seq):
        self._check("dsa_prefetch_reuse", dsa_prefetch_reuse(self.h, layer, src_layer, rows_per_seq,
                                                             self._stream()))

    def unit_state(self, layer, seq):
        st, v = dsa_unit_state(self.h, layer, seq)
        self._check("dsa_unit_state", st)
        return dict(L=v[0], M=v[1], round=v[2], row_bytes=v[3])

    def mirror_rows(self, layer, seq):
        st, v = dsa_mirror_rows(self.h, layer, seq)
        self._check("dsa_mirror_rows", st)
        return v

    def debug(self, item, layer=0, seq=0):
        """Copy an inspection item into a new uint8 device tensor (caller views/reshapes it)."""
        code = DBG[item] if isinstance(item, str) else item
        st, n = dsa_debug_size(self.h, layer, seq, code)
        self._check("dsa_debug_size", st)
        buf = self._torch.empty(max(n, 16), dtype=self._torch.uint8, device=self.device)
        self._check("dsa_debug_get", dsa_debug_get(self.h, layer, seq, code, self._ptr(buf), buf.numel(),
                                                   self._stream()))
        return buf[:n]

    def set_kernel_timing(self, enable=True, reserve_steps=64):
        """Turn per-kernel timing on (events pre-created for reserve_steps steps) or off."""
        n = max(1, int(reserve_steps)) if enable else 0
        self._check("dsa_set_kernel_timing", dsa_set_kernel_timing(self.h, n))

    def inject(self, what, layer=0, seq=0):
        """Force an error condition from the host (tests of the error model)."""
        code = {"hip_failure": INJECT_HIP_FAILURE, "bad_slot": INJECT_BAD_SLOT}.get(what, what)
        self._check("dsa_debug_inject", dsa_debug_inject(self.h, layer, seq, code, self._stream()))

    def kernel_times(self):
        st, counts, ms = dsa_kernel_times(self.h)
        self._check("dsa_kernel_times", st)
        return {k: (c, m) for k, c, m in zip(KERNEL_KINDS, counts, ms)}
