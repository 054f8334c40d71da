"""The C ABI: the library loads on a machine without a GPU, exports every
symbol tqkv.h declares, and rejects invalid configurations on the host
(no compute calls here)."""

import ctypes
import os
import re
import subprocess

import pytest

from compressed_kv_decode_amd import tqkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tqkv.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:tq_status|const char\*|uint32_t)\s+(tq_[a-z_]+)\(", txt, re.M)))


def test_header_declares_the_four_method_calls():
    names = _declared()
    for n in ("tq_cache_create", "tq_quantize_append", "tq_decode_attention", "tq_promote"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = tqkv.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", tqkv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (tq_[a-z_]+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(tqkv.EXPORTS) <= exported


def test_version_and_status_strings():
    lib = tqkv.load_library()
    assert lib.tq_version() == 0x00010000
    assert lib.tq_status_string(0) == b"ok"
    assert lib.tq_status_string(3) == b"capacity exceeded"


BASE = dict(n_seq_max=2, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, hot_window=512,
            max_context=4096, formats=[tqkv.F3, tqkv.F4])


def _status(**over):
    lib = tqkv.load_library()
    kw = dict(BASE)
    kw.update(over)
    cfg, _keep = tqkv.make_config(**kw)
    n = ctypes.c_size_t(0)
    return lib.tq_cache_required_bytes(ctypes.byref(cfg), ctypes.byref(n)), n.value


def test_required_bytes_grows_with_context_and_formats():
    s, n1 = _status()
    assert s == 0 and n1 > 0
    s, n2 = _status(max_context=8192)
    assert s == 0 and n2 > n1
    s, n3 = _status(formats=[tqkv.F4, tqkv.F4])
    assert s == 0 and n3 > n1


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=96), 2),
    (dict(n_q_heads=6), 2),
    (dict(n_q_heads=48, n_kv_heads=2), 2),
    (dict(formats=[(5, 3, 32), tqkv.F4]), 2),
    (dict(formats=[tqkv.F3, (3, 4, 48)]), 2),
    (dict(hot_window=0), 1),
    (dict(max_context=-1), 1),
    (dict(n_layers=0, formats=[]), 1),
    (dict(promote_threshold=0.001), 1),
    (dict(promote_threshold=0.15, sticky=0), 1),
])
def test_invalid_configs_rejected_on_host(over, code):
    s, _ = _status(**over)
    assert s == code
    assert tqkv.load_library().tq_last_error()


def test_null_handle_rejected():
    lib = tqkv.load_library()
    assert lib.tq_cache_destroy(None) == 1
    assert lib.tq_promote(None, 0, 0, None, None) == 1
    hc = ctypes.c_int32()
    assert lib.tq_cache_geometry(None, ctypes.byref(hc), None) == 1
