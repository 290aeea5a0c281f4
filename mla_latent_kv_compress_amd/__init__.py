"""MLA over a compressed latent KV cache on AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI declared in include/mla.h
(libmla.so).  This package holds the thin ctypes binding (`api`), the workload shapes
(`configs`) and the seeded synthetic inputs (`inputs`).  Importing the package loads nothing;
`api` loads libmla.so on first use and raises if it is missing.
"""
import importlib

__all__ = ["api", "configs", "inputs", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
