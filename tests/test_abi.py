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
    assert lib.tq_version() == 0x00010500
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
    (dict(rotation_kind=2), 1),
    (dict(rotation_kind=-1), 1),
])
def test_invalid_configs_rejected_on_host(over, code):
    s, _ = _status(**over)
    assert s == code
    assert tqkv.load_library().tq_last_error()


def test_null_handle_rejected():
    lib = tqkv.load_library()
    assert lib.tq_cache_destroy(None) == 1
    assert lib.tq_promote(None, 0, 0, None, None) == 1
    assert lib.tq_decode_step(None, 0, 0, None, None, None, None, None, None, None) == 1
    hc = ctypes.c_int32()
    assert lib.tq_cache_geometry(None, ctypes.byref(hc), None) == 1


class _RecordingLib:
    """Stands in for the library: records calls, returns TQ_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*a):
            self.calls.append(name)
            return 0
        return f


def _shell_cache(hq=8, hkv=2, d=64, stride=320):
    c = object.__new__(tqkv.Cache)
    c.lib, c.h = _RecordingLib(), None
    c.hq, c.hkv, c.d, c.logits_stride = hq, hkv, d, stride
    return c


@pytest.mark.parametrize("bad", ["dtype", "shape", "stride", "device"])
def test_binding_rejects_mismatched_tensors_before_any_library_call(bad, monkeypatch):
    import torch
    monkeypatch.setattr(tqkv, "_stream", lambda: None)
    c = _shell_cache()
    good_kv = torch.zeros((5, 2, 64), dtype=torch.float16)
    good_q = torch.zeros((2, 8, 64), dtype=torch.float16)
    mk = {
        "dtype": lambda t: t.to(torch.bfloat16),
        "shape": lambda t: t[:, :, :32].contiguous(),
        "stride": lambda t: t.transpose(0, 1).contiguous().transpose(0, 1),
        "device": lambda t: t,  # CPU tensors of the right shape fail the device check
    }[bad]
    with pytest.raises(ValueError):
        c.append(0, [0, 1], [2, 3], mk(good_kv), mk(good_kv))
    with pytest.raises(ValueError):
        c.attend(0, [0, 1], mk(good_q), out=torch.zeros((2, 8, 64)))
    with pytest.raises(ValueError):
        c.step(0, [0, 1], [2, 3], mk(good_kv), mk(good_kv), good_q, out=torch.zeros((2, 8, 64)))
    with pytest.raises(ValueError):
        c.step(0, [0, 1], [2, 3], good_kv, good_kv, mk(good_q), out=torch.zeros((2, 8, 64)))
    assert c.lib.calls == []
    # out and logits are checked too (q itself would pass on a GPU)
    with pytest.raises(ValueError):
        tqkv.check_tensor(torch.zeros((2, 8, 64), dtype=torch.float16), "out", torch.float32, (2, 8, 64))
    with pytest.raises(ValueError):
        tqkv.check_tensor(torch.zeros((2, 8, 319)), "logits", torch.float32, (2, 8, 320))
    # an empty append may pass None for k and v
    c.append(0, [0], [0], None, None)
    assert c.lib.calls == ["tq_quantize_append"]
    # token counts must match the sequences
    with pytest.raises(ValueError):
        c.append(0, [0, 1], [2], good_kv, good_kv)


@pytest.mark.parametrize("over", [dict(promote_threshold=0.15), dict(tc_lambda=0.0), dict(tc_lambda=1.5),
                                  dict(tc_eta=float("inf")), dict(tc_gate=float("nan")), dict(cold_tier=2)])
def test_tensor_cache_tier_config_is_validated(over):
    base = dict(n_seq_max=2, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=64, hot_window=64, max_context=512,
                formats=[tqkv.F3], cold_tier=tqkv.COLD_TENSOR_CACHE, tc_lambda=0.99, tc_eta=0.1, tc_gate=0.0)
    n_ok = tqkv.required_bytes(**base)
    codes = tqkv.required_bytes(**dict(base, cold_tier=tqkv.COLD_CODES))
    assert n_ok > 0 and codes > 0
    with pytest.raises(tqkv.TqError) as e:
        tqkv.required_bytes(**dict(base, **over))
    assert e.value.status == 1
