"""Exact split-KV decode attention for MI355X (gfx950).

The library is ``libkvd.so`` (HIP kernels behind a C ABI declared in
``include/kvd.h``); this package is its Python binding (argument marshalling
only) plus pure-Python roofline arithmetic.  The binding module is loaded on
first use so that ``roofline`` can be imported on hosts without the library.
"""
import importlib

__all__ = ["kvd", "roofline"]


def __getattr__(name):
    if name in ("kvd", "roofline", "build"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
