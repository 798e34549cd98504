"""The C-ABI library loads and exports every symbol include/dsa.h declares; argument
validation that happens before any HIP call is checked here without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ensure_built():
    lib = os.path.join(ROOT, "kv_cache_offload_amd", "libdsa.so")
    if not os.path.exists(lib):
        from __graft_entry__ import _build_module
        _build_module().build()
    return lib


def _declared():
    src = open(os.path.join(ROOT, "include", "dsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:dsa_status|const char\*)\s+(dsa_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary_calls():
    names = _declared()
    for required in ("dsa_session_create", "dsa_append_rows", "dsa_decode_step"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_ensure_built())
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_names_match_header():
    _ensure_built()
    import kv_cache_offload_amd as K
    assert sorted(K.EXPORTS) == _declared()
    for name in _declared():
        assert callable(getattr(K, name))


def _cfg(**kw):
    import kv_cache_offload_amd as K
    base = dict(max_positions=1000, index_heads=32, heads=64, top_k=256, hot_slots=128, max_query_rows=4)
    base.update(kw)
    return K.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), None),
    (dict(index_dim=64), "E_UNSUPPORTED"),
    (dict(index_heads=12), "E_UNSUPPORTED"),
    (dict(heads=48), "E_UNSUPPORTED"),
    (dict(top_k=4096, max_query_rows=8), "E_UNSUPPORTED"),
    (dict(max_positions=0), "E_INVALID"),
    (dict(hot_slots=0), "E_INVALID"),
    (dict(mode=7), "E_INVALID"),
    (dict(softmax_scale=float("inf")), "E_INVALID"),
])
def test_config_validation_before_any_device_call(kw, status):
    _ensure_built()
    import kv_cache_offload_amd as K
    cfg = _cfg(**kw)
    if status is None:
        return                      # a valid config needs a GPU to go further
    out = ctypes.c_void_p()
    st = K._lib.dsa_session_create(ctypes.byref(cfg), ctypes.byref(out))
    assert st == getattr(K, status) and not out.value


def test_abi_version_mismatch_and_nulls():
    _ensure_built()
    import kv_cache_offload_amd as K
    cfg = _cfg()
    cfg.abi_version = 99
    out = ctypes.c_void_p()
    assert K._lib.dsa_session_create(ctypes.byref(cfg), ctypes.byref(out)) == K.E_INVALID
    assert K._lib.dsa_session_create(None, ctypes.byref(out)) == K.E_INVALID
    assert K._lib.dsa_session_create(ctypes.byref(_cfg()), None) == K.E_INVALID
    assert K.dsa_session_destroy(None) == K.OK
    assert K.dsa_last_error(None) == "NULL session"
    assert K._lib.dsa_append_rows(None, 0, 0, 1, None, None, None) == K.E_INVALID
    assert K._lib.dsa_decode_step(None, 0, 1, None, None, None, None, None, None) == K.E_INVALID
    assert K._lib.dsa_rollback_rows(None, 0, 0, 1, None) == K.E_INVALID
    assert K._lib.dsa_quantize_rows(None, 1, None, None, None, None) == K.E_INVALID
    assert K._lib.dsa_append_latent(None, 0, 0, 1, None, None, None, None) == K.E_INVALID
    assert K._lib.dsa_decode_step_reuse(None, 1, 0, 1, None, None, None, None) == K.E_INVALID
    assert K._lib.dsa_prefetch_reuse(None, 1, 0, 1, None) == K.E_INVALID
    assert K._lib.dsa_decode_step_static(None, 0, 1, None, None, None, None, None, None) == K.E_INVALID
    assert K._lib.dsa_append_decode_step(None, 0, 1, None, None, None, None, None, None, None, None) == K.E_INVALID


def test_config_rejects_unknown_replacement_policy():
    _ensure_built()
    import kv_cache_offload_amd as K
    cfg = _cfg(replacement=2)
    out = ctypes.c_void_p()
    assert K._lib.dsa_session_create(ctypes.byref(cfg), ctypes.byref(out)) == K.E_INVALID
    assert not out.value
