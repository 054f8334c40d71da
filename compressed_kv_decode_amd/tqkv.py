"""Python binding of libtqkv (ctypes): argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module passes
pointers, sizes and the current HIP stream.  PyTorch provides device memory
(the arena and the inputs/outputs) and streams.  If libtqkv.so has not been
built the import fails: there is no fallback.
"""

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtqkv.so")

F3 = (2, 3, 32)
F4 = (3, 4, 64)
F25 = (2, 2, 64)


class TqFormat(ctypes.Structure):
    _fields_ = [("r_bits", ctypes.c_uint8), ("theta_bits", ctypes.c_uint8), ("qjl_m", ctypes.c_uint16)]


class TqConfig(ctypes.Structure):
    _fields_ = [
        ("n_seq_max", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("hot_window", ctypes.c_int32),
        ("max_context", ctypes.c_int32),
        ("layer_formats", ctypes.POINTER(TqFormat)),
        ("seed", ctypes.c_uint64),
        ("promote_threshold", ctypes.c_float),
        ("sticky", ctypes.c_int32),
        ("v_qjl", ctypes.c_int32),
        ("rotation", ctypes.POINTER(ctypes.c_float)),
        ("sketch", ctypes.POINTER(ctypes.c_float)),
        ("cold_tier", ctypes.c_int32),
        ("tc_lambda", ctypes.c_float),
        ("tc_eta", ctypes.c_float),
        ("tc_gate", ctypes.c_float),
        ("rotation_kind", ctypes.c_int32),
    ]


COLD_CODES = 0
COLD_TENSOR_CACHE = 1
ROTATION_HAAR = 0
ROTATION_HADAMARD = 1


class TqStats(ctypes.Structure):
    _fields_ = [
        ("hot_len", ctypes.c_int32),
        ("cold_len", ctypes.c_int32),
        ("live_cold", ctypes.c_int32),
        ("n_promoted", ctypes.c_int32),
        ("n_evicted", ctypes.c_int32),
        ("attn_steps", ctypes.c_int32),
        ("device_error", ctypes.c_int32),
        ("hot_capacity", ctypes.c_int32),
        ("tokens_appended", ctypes.c_int64),
    ]


EXPORTS = [
    "tq_cache_required_bytes", "tq_cache_create", "tq_cache_destroy", "tq_quantize_append",
    "tq_decode_attention", "tq_promote", "tq_evict", "tq_cache_sync_stats", "tq_export_codes", "tq_import_codes",
    "tq_export_hot", "tq_export_paging", "tq_get_rotation", "tq_cache_geometry", "tq_profile_enable",
    "tq_profile_read", "tq_status_string", "tq_last_error", "tq_version", "tq_decode_attention_static",
    "tq_probe_read_bandwidth", "tq_decode_attention_gated", "tq_export_tensor_cache", "tq_mips_workspace_bytes",
    "tq_mips_search", "tq_multi_query_workspace_bytes", "tq_multi_query_attention", "tq_promote_deferred",
    "tq_flush", "tq_decode_step", "tq_multi_query_batch_workspace_bytes", "tq_multi_query_attention_batch",
]

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtqkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m compressed_kv_decode_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_void_p
    sig = {
        "tq_cache_required_bytes": [P(TqConfig), P(ctypes.c_size_t)],
        "tq_cache_create": [P(TqConfig), VP, ctypes.c_size_t, VP, P(VP)],
        "tq_cache_destroy": [VP],
        "tq_quantize_append": [VP, I32, I32, P(I32), P(I32), VP, VP, VP],
        "tq_decode_attention": [VP, I32, I32, P(I32), VP, VP, VP, VP],
        "tq_decode_step": [VP, I32, I32, P(I32), P(I32), VP, VP, VP, VP, VP],
        "tq_decode_attention_static": [VP, I32, I32, P(I32), VP, VP, VP, VP],
        "tq_decode_attention_gated": [VP, I32, I32, P(I32), VP, VP, VP, ctypes.c_float, VP],
        "tq_promote": [VP, I32, I32, P(I32), VP],
        "tq_promote_deferred": [VP, I32, I32, P(I32), VP],
        "tq_flush": [VP],
        "tq_evict": [VP, I32, I32, P(I32), I32, VP],
        "tq_cache_sync_stats": [VP, I32, I32, P(TqStats), VP],
        "tq_export_codes": [VP, I32, I32, I32, I32, I32, I32, VP, VP],
        "tq_import_codes": [VP, I32, I32, I32, I32, I32, I32, VP, VP],
        "tq_export_hot": [VP, I32, I32, P(I32), P(I32), VP, VP, VP],
        "tq_export_paging": [VP, I32, I32, I32, VP, VP, VP],
        "tq_get_rotation": [VP, VP, VP, VP],
        "tq_export_tensor_cache": [VP, I32, I32, I32, VP, VP],
        "tq_mips_workspace_bytes": [VP, I32, I32, P(ctypes.c_size_t)],
        "tq_multi_query_workspace_bytes": [VP, P(ctypes.c_size_t)],
        "tq_multi_query_attention": [VP, I32, I32, I32, VP, VP, VP, ctypes.c_size_t, VP],
        "tq_multi_query_batch_workspace_bytes": [VP, I32, P(ctypes.c_size_t)],
        "tq_multi_query_attention_batch": [VP, I32, I32, P(I32), I32, VP, VP, VP, ctypes.c_size_t, VP],
        "tq_mips_search": [VP, I32, I32, I32, I32, VP, I32, VP, VP, VP, ctypes.c_size_t, VP],
        "tq_cache_geometry": [VP, P(I32), P(I32)],
        "tq_profile_enable": [VP, I32],
        "tq_profile_read": [VP, P(ctypes.c_double), P(I32)],
        "tq_probe_read_bandwidth": [VP, ctypes.c_size_t, VP, I32, VP],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.tq_status_string.argtypes = [ctypes.c_int]
    lib.tq_status_string.restype = ctypes.c_char_p
    lib.tq_last_error.argtypes = []
    lib.tq_last_error.restype = ctypes.c_char_p
    lib.tq_version.argtypes = []
    lib.tq_version.restype = ctypes.c_uint32
    _lib = lib
    return lib


class TqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libtqkv status {status}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise TqError(status, (lib.tq_last_error() or b"").decode())


def _i32(xs: Sequence[int]):
    arr = (ctypes.c_int32 * max(1, len(xs)))(*[int(x) for x in xs])
    return arr


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def check_tensor(t, name: str, dtype, shape) -> None:
    """Raise ValueError unless t is a contiguous tensor of exactly this dtype
    and shape on a GPU.  The library reads and writes the sizes the shape
    implies, so a mismatch would touch memory outside the tensor."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be on a GPU, is on {t.device}")


def probe_read_bandwidth(buf, sink, blocks: int) -> None:
    """One read-only pass over the bytes of device tensor buf (sink: uint32
    device tensor of at least ``blocks`` entries); time it with events."""
    lib = load_library()
    if sink.numel() < blocks or sink.element_size() != 4:
        raise ValueError("sink must hold blocks 32-bit words")
    _check(lib.tq_probe_read_bandwidth(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                       ctypes.c_void_p(sink.data_ptr()), int(blocks), _stream()))


def make_config(*, n_seq_max, n_layers, n_q_heads, n_kv_heads, head_dim, hot_window, max_context, formats,
                seed=0, promote_threshold=2.0, sticky=3, v_qjl=True, rotation=None, sketch=None,
                cold_tier=COLD_CODES, tc_lambda=1.0, tc_eta=1.0, tc_gate=0.0,
                rotation_kind=ROTATION_HAAR):
    """A TqConfig plus the host buffers it points to (keep them alive)."""
    if len(formats) != n_layers:
        raise ValueError(f"{len(formats)} layer formats for {n_layers} layers")
    fm = (TqFormat * n_layers)(*[TqFormat(*f) for f in formats])
    keep = [fm]
    cfg = TqConfig(n_seq_max, n_layers, n_q_heads, n_kv_heads, head_dim, hot_window, max_context,
                   ctypes.cast(fm, ctypes.POINTER(TqFormat)), seed, promote_threshold, sticky, int(bool(v_qjl)),
                   None, None, int(cold_tier), float(tc_lambda), float(tc_eta), float(tc_gate), int(rotation_kind))
    if rotation is not None:
        r = np.ascontiguousarray(rotation, dtype=np.float32)
        keep.append(r)
        cfg.rotation = r.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    if sketch is not None:
        s = np.ascontiguousarray(sketch, dtype=np.float32)
        keep.append(s)
        cfg.sketch = s.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    return cfg, keep


def required_bytes(**kw) -> int:
    lib = load_library()
    cfg, _keep = make_config(**kw)
    n = ctypes.c_size_t(0)
    _check(lib.tq_cache_required_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


class Cache:
    """A compressed KV cache over a torch-allocated device arena."""

    def __init__(self, *, n_seq_max, n_layers, n_q_heads, n_kv_heads, head_dim, hot_window, max_context, formats,
                 seed=0, promote_threshold=2.0, sticky=3, v_qjl=True, rotation=None, sketch=None, device="cuda",
                 cold_tier=COLD_CODES, tc_lambda=1.0, tc_eta=1.0, tc_gate=0.0, rotation_kind=ROTATION_HAAR):
        import torch
        self.lib = load_library()
        self.n_layers, self.hq, self.hkv, self.d = n_layers, n_q_heads, n_kv_heads, head_dim
        self.formats = [tuple(f) for f in formats]
        self.window, self.max_context = hot_window, max_context
        cfg, keep = make_config(n_seq_max=n_seq_max, n_layers=n_layers, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                                head_dim=head_dim, hot_window=hot_window, max_context=max_context, formats=formats,
                                seed=seed, promote_threshold=promote_threshold, sticky=sticky, v_qjl=v_qjl,
                                rotation=rotation, sketch=sketch, cold_tier=cold_tier, tc_lambda=tc_lambda,
                                tc_eta=tc_eta, tc_gate=tc_gate, rotation_kind=rotation_kind)
        n = ctypes.c_size_t(0)
        _check(self.lib.tq_cache_required_bytes(ctypes.byref(cfg), ctypes.byref(n)))
        self.arena_bytes = n.value
        self.arena = torch.empty(n.value, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        _check(self.lib.tq_cache_create(ctypes.byref(cfg), ctypes.c_void_p(self.arena.data_ptr()), n.value, _stream(),
                                        ctypes.byref(h)))
        self._keep = keep
        self.h = h
        hc, ls = ctypes.c_int32(), ctypes.c_int32()
        _check(self.lib.tq_cache_geometry(self.h, ctypes.byref(hc), ctypes.byref(ls)))
        self.hot_capacity, self.logits_stride = hc.value, ls.value

    def close(self):
        if self.h:
            _check(self.lib.tq_cache_destroy(self.h))
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ptr(t):
        return ctypes.c_void_p(0 if t is None else t.data_ptr())

    def append(self, layer: int, seq_ids: Sequence[int], n_new: Sequence[int], k, v) -> None:
        """k, v: fp16 device tensors [sum(n_new), n_kv_heads, head_dim], contiguous
        (None allowed when sum(n_new) == 0)."""
        import torch
        if len(n_new) != len(seq_ids):
            raise ValueError(f"{len(n_new)} token counts for {len(seq_ids)} sequences")
        total = int(sum(int(x) for x in n_new))
        for t, name in ((k, "k"), (v, "v")):
            if t is None and total == 0:
                continue
            check_tensor(t, name, torch.float16, (total, self.hkv, self.d))
        _check(self.lib.tq_quantize_append(self.h, layer, len(seq_ids), _i32(seq_ids), _i32(n_new), self._ptr(k),
                                           self._ptr(v), _stream()))

    def attend(self, layer: int, seq_ids: Sequence[int], q, out=None, logits=None, static_workspace=False,
               gate: Optional[float] = None):
        """q: fp16 [n_seq, n_q_heads, head_dim]; returns fp32 out of the same shape.
        logits: None or fp32 [n_seq, n_q_heads, logits_stride] (debug logits).
        static_workspace: use the entry point that allocates nothing (its
        scratch is the library's static per-GPU array).
        gate: None, or the hot-first threshold (tq_decode_attention_gated)."""
        import torch
        shape = (len(seq_ids), self.hq, self.d)
        check_tensor(q, "q", torch.float16, shape)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=q.device)
        check_tensor(out, "out", torch.float32, shape)
        if logits is not None:
            check_tensor(logits, "logits", torch.float32, (len(seq_ids), self.hq, self.logits_stride))
        if gate is not None:
            if static_workspace:
                raise ValueError("the static-workspace entry point has no gate")
            _check(self.lib.tq_decode_attention_gated(self.h, layer, len(seq_ids), _i32(seq_ids), self._ptr(q),
                                                      self._ptr(out), self._ptr(logits), float(gate), _stream()))
            return out
        fn = self.lib.tq_decode_attention_static if static_workspace else self.lib.tq_decode_attention
        _check(fn(self.h, layer, len(seq_ids), _i32(seq_ids), self._ptr(q), self._ptr(out), self._ptr(logits),
                  _stream()))
        return out

    def step(self, layer: int, seq_ids: Sequence[int], n_new: Sequence[int], k, v, q, out=None):
        """tq_decode_step: append k, v (as append) then attend q (as attend,
        without debug logits), in one call; returns fp32 out."""
        import torch
        if len(n_new) != len(seq_ids):
            raise ValueError(f"{len(n_new)} token counts for {len(seq_ids)} sequences")
        total = int(sum(int(x) for x in n_new))
        for t, name in ((k, "k"), (v, "v")):
            if t is None and total == 0:
                continue
            check_tensor(t, name, torch.float16, (total, self.hkv, self.d))
        shape = (len(seq_ids), self.hq, self.d)
        check_tensor(q, "q", torch.float16, shape)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=q.device)
        check_tensor(out, "out", torch.float32, shape)
        _check(self.lib.tq_decode_step(self.h, layer, len(seq_ids), _i32(seq_ids), _i32(n_new), self._ptr(k),
                                       self._ptr(v), self._ptr(q), self._ptr(out), _stream()))
        return out

    def promote(self, layer: int, seq_ids: Sequence[int], deferred: bool = False) -> None:
        """deferred: tq_promote_deferred (launched by the next call on the
        cache, inside a small append of another layer where it can be)."""
        fn = self.lib.tq_promote_deferred if deferred else self.lib.tq_promote
        _check(fn(self.h, layer, len(seq_ids), _i32(seq_ids), _stream()))

    def flush(self) -> None:
        """Launch a deferred promotion now."""
        _check(self.lib.tq_flush(self.h))

    def evict(self, layer: int, seq_ids: Sequence[int], target_hot: int) -> None:
        _check(self.lib.tq_evict(self.h, layer, len(seq_ids), _i32(seq_ids), int(target_hot), _stream()))

    def stats(self, seq: int, layer: int) -> dict:
        s = TqStats()
        st = self.lib.tq_cache_sync_stats(self.h, seq, layer, ctypes.byref(s), _stream())
        d = {name: getattr(s, name) for name, _ in TqStats._fields_}
        d["status"] = st
        return d

    def record_bytes(self, layer: int) -> int:
        rb, tb, m = self.formats[layer]
        return ((self.d // 2) * (rb + tb) + 7) // 8 + m // 8 + 4

    def export_codes(self, seq, layer, kv_head, kv, first, n) -> np.ndarray:
        out = np.zeros((n, self.record_bytes(layer)), dtype=np.uint8)
        _check(self.lib.tq_export_codes(self.h, seq, layer, kv_head, kv, first, n, out.ctypes.data_as(ctypes.c_void_p),
                                        _stream()))
        return out

    def import_codes(self, seq, layer, kv_head, kv, first, records: np.ndarray) -> None:
        rec = np.ascontiguousarray(records, dtype=np.uint8)
        _check(self.lib.tq_import_codes(self.h, seq, layer, kv_head, kv, first, rec.shape[0],
                                        rec.ctypes.data_as(ctypes.c_void_p), _stream()))

    def export_hot(self, seq, layer):
        n = ctypes.c_int32()
        tags = np.zeros(self.hot_capacity, dtype=np.int32)
        k = np.zeros((self.hkv, self.hot_capacity, self.d), dtype=np.float16)
        v = np.zeros_like(k)
        _check(self.lib.tq_export_hot(self.h, seq, layer, ctypes.byref(n), tags.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      k.ctypes.data_as(ctypes.c_void_p), v.ctypes.data_as(ctypes.c_void_p), _stream()))
        c = n.value
        return tags[:c].tolist(), k[:, :c], v[:, :c]

    def export_paging(self, seq, layer, n):
        live = np.zeros(n, dtype=np.uint8)
        stk = np.zeros(n, dtype=np.int32)
        _check(self.lib.tq_export_paging(self.h, seq, layer, n, live.ctypes.data_as(ctypes.c_void_p),
                                         stk.ctypes.data_as(ctypes.c_void_p), _stream()))
        return live.astype(bool), stk

    def multi_query_workspace_bytes(self) -> int:
        nb = ctypes.c_size_t(0)
        _check(self.lib.tq_multi_query_workspace_bytes(self.h, ctypes.byref(nb)))
        return nb.value

    def multi_query(self, layer: int, seq: int, q, workspace=None):
        """Attention of the newest q.shape[0] tokens' queries q [n_new,
        n_q_heads, head_dim] (fp16) over the cache, causal within the chunk;
        returns fp32 [n_new, n_q_heads, head_dim]."""
        import torch
        n_new = q.shape[0] if hasattr(q, "shape") else 0
        check_tensor(q, "q", torch.float16, (n_new, self.hq, self.d))
        nb = self.multi_query_workspace_bytes()
        if workspace is None or workspace.numel() * workspace.element_size() < nb:
            workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
        out = torch.empty((n_new, self.hq, self.d), dtype=torch.float32, device=q.device)
        _check(self.lib.tq_multi_query_attention(self.h, layer, seq, n_new, self._ptr(q), self._ptr(out),
                                                 self._ptr(workspace), workspace.numel() * workspace.element_size(),
                                                 _stream()))
        return out

    def multi_query_batch_workspace_bytes(self, n_seq: int) -> int:
        nb = ctypes.c_size_t(0)
        _check(self.lib.tq_multi_query_batch_workspace_bytes(self.h, int(n_seq), ctypes.byref(nb)))
        return nb.value

    def multi_query_batch(self, layer: int, seq_ids: Sequence[int], q, workspace=None):
        """tq_multi_query_attention_batch: q [n_seq, n_new, n_q_heads,
        head_dim] (fp16), the queries of each sequence's newest n_new tokens;
        returns fp32 of the same shape."""
        import torch
        n_seq = len(seq_ids)
        n_new = q.shape[1] if hasattr(q, "shape") and len(q.shape) == 4 else 0
        check_tensor(q, "q", torch.float16, (n_seq, n_new, self.hq, self.d))
        nb = self.multi_query_batch_workspace_bytes(n_seq)
        if workspace is None or workspace.numel() * workspace.element_size() < nb:
            workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
        out = torch.empty((n_seq, n_new, self.hq, self.d), dtype=torch.float32, device=q.device)
        _check(self.lib.tq_multi_query_attention_batch(self.h, layer, n_seq, _i32(seq_ids), n_new, self._ptr(q),
                                                       self._ptr(out), self._ptr(workspace),
                                                       workspace.numel() * workspace.element_size(), _stream()))
        return out

    def mips_search(self, seq: int, layer: int, kv_head: int, q, k: int, workspace=None):
        """Top-k compressed inner products of fp16 queries q [n_q, head_dim]
        over the cold slots of (seq, layer, kv_head); returns (idx int32
        [n_q, k], score fp32 [n_q, k]) device tensors."""
        import torch
        n_q = q.shape[0] if hasattr(q, "shape") else 0
        check_tensor(q, "q", torch.float16, (n_q, self.d))
        nb = ctypes.c_size_t(0)
        _check(self.lib.tq_mips_workspace_bytes(self.h, n_q, k, ctypes.byref(nb)))
        if workspace is None or workspace.numel() * workspace.element_size() < nb.value:
            workspace = torch.empty(nb.value, dtype=torch.uint8, device=q.device)
        idx = torch.empty((n_q, k), dtype=torch.int32, device=q.device)
        score = torch.empty((n_q, k), dtype=torch.float32, device=q.device)
        _check(self.lib.tq_mips_search(self.h, seq, layer, kv_head, n_q, self._ptr(q), k, self._ptr(idx),
                                       self._ptr(score), self._ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream()))
        return idx, score

    def export_tensor_cache(self, seq, layer, kv_head) -> np.ndarray:
        a = np.zeros((self.d, self.d), dtype=np.float32)
        _check(self.lib.tq_export_tensor_cache(self.h, seq, layer, kv_head, a.ctypes.data_as(ctypes.c_void_p),
                                               _stream()))
        return a

    def rotation(self):
        pi = np.zeros((self.d, self.d), dtype=np.float32)
        s = np.zeros((64, self.d), dtype=np.float32)
        _check(self.lib.tq_get_rotation(self.h, pi.ctypes.data_as(ctypes.c_void_p), s.ctypes.data_as(ctypes.c_void_p),
                                        _stream()))
        return pi, s

    def profile_enable(self, on: bool = True) -> None:
        _check(self.lib.tq_profile_enable(self.h, int(bool(on))))

    def profile_read(self):
        ms, n = ctypes.c_double(), ctypes.c_int32()
        _check(self.lib.tq_profile_read(self.h, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value
