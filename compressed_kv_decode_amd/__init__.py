"""compressed_kv_decode_amd: decode attention over a compressed KV cache on
AMD Instinct MI355X (gfx950).

The product is the C-ABI library libtqkv (include/tqkv.h, sources in csrc/),
built in-tree by ``python -m compressed_kv_decode_amd.build``.  ``tqkv`` is
its thin Python binding; ``workloads`` draws the seeded synthetic inputs.
The binding is imported lazily so that ``workloads`` needs no GPU build.
"""

__all__ = ["tqkv", "workloads"]


def __getattr__(name):
    if name in ("tqkv", "workloads", "build"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    if name == "Cache":
        from .tqkv import Cache
        return Cache
    raise AttributeError(name)
