"""MI355X-native paged Top-K decode attention.

The compute path is the C-ABI library ``libkvdecode.so`` (hand-written HIP for
gfx950); :mod:`kv_cache_decode_amd.kvdecode` is its thin Python binding and
loads it on first use, failing loudly if it is not built.
:mod:`kv_cache_decode_amd.workload` makes the seeded synthetic inputs.
"""
import importlib

__all__ = ["kvdecode", "workload"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
