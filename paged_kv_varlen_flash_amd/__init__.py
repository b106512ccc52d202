"""Paged-KV varlen flash attention for MI355X (gfx950).

The compute path is ``libpagedattn.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/pagedattn.h``); ``paged_kv_varlen_flash_amd.ops``
is the thin ctypes binding with the same entry-point names.  The binding is
loaded lazily so the input generators in ``workloads`` import without it.
"""
import importlib

__all__ = ["ops", "workloads"]


def __getattr__(name):
    if name in ("ops", "workloads", "build"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
